"""Negative controls: a pin set that never goes red proves nothing.

Each case copies oracle.c, plants one plausible mistake (a dropped term, a
wrong sign, index or operand order), builds it into a temporary library and
checks that at least one pin fails on it.  Runs on the CPU only.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins as P

MUTATIONS = [
    ("nibble_halves_swapped", "(i < 16) ? (blk[2 + i] & 0x0F)", "(i >= 16) ? (blk[2 + i] & 0x0F)"),
    ("q4_bias_off_by_one", ": d * (double)(c - 8);", ": d * (double)(c - 7);"),
    ("nl4_read_as_linear", "? d * (double)orc_cb[c] :", "? d * (double)(c - 8) :"),
    ("nl4_table_index_off_by_one", "d * (double)orc_cb[c]", "d * (double)orc_cb[(c + 1) & 15]"),
    ("nl4_table_entries_as_unsigned", "d * (double)orc_cb[c]", "d * (double)(uint8_t)orc_cb[c]"),
    ("nl4_block_bytes", "if (bits == 4 || bits == ORC_BITS_NL4) return 18;", "if (bits == 4) return 18;"),
    ("q3_high_bit_weight", "int c = lo | (hi << 2);", "int c = lo | (hi << 1);"),
    ("q3_low_field_index", "(blk[2 + (i % 8)] >> (2 * (i / 8))) & 3", "(blk[2 + (i / 4)] >> (2 * (i % 4))) & 3"),
    ("half_exponent_bias", "expo - 15", "expo - 14"),
    ("half_subnormal", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("tie_to_higher_id", "l[e] > l[best]", "l[e] >= l[best]"),
    ("softmax_not_renormalised", "exp((double)l[idx[(int64_t)t * k + j]] - lmax) / sum;",
     "exp((double)l[idx[(int64_t)t * k + j]] - lmax) / (sum + 1.0);"),
    ("group_order_reversed", "pairs[offsets[e] + fill[e]] = (int32_t)p;",
     "pairs[offsets[e + 1] - 1 - fill[e]] = (int32_t)p;"),
    ("swiglu_operands_swapped", "hid[f] = g / (1.0 + exp(-g)) * u;", "hid[f] = u / (1.0 + exp(-u)) * g;"),
    ("down_input_reversed", "acc += dr[f] * hid[f];", "acc += dr[f] * hid[F - 1 - f];"),
    ("shared_expert_dropped", "    if (shared) {\n        orc_expert sx;", "    if (0) {\n        orc_expert sx;"),
    ("combine_drops_last_slot", "for (j = 1; j < k; ++j) acc += w", "for (j = 1; j < k - 1; ++j) acc += w"),
    ("gate_up_swapped", "orc_dequant_matrix(bg, blob, F, H, ex->gate);",
     "orc_dequant_matrix(bg, blob, F, H, ex->up);"),
    ("down_read_in_gate_up_format", "orc_dequant_matrix(bd, blob + 2 * mat, H, F, ex->down);",
     "orc_dequant_matrix(bg, blob + 2 * mat, H, F, ex->down);"),
    ("format_down_width_ignored", "    if (dn == 0) dn = gu;", "    dn = gu;"),
    ("router_row_index", "const uint16_t *we = w + (int64_t)e * H;", "const uint16_t *we = w + (int64_t)t * H;"),
    ("router_bf16_as_half", "acc += xv * orc_bf16_to_double(we[h]);", "acc += xv * orc_half_to_double(we[h]);"),
    ("expert_bytes_uniform", "(2 * orc_block_bytes(bg) + orc_block_bytes(bd))", "(3 * orc_block_bytes(bg))"),
]


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="orc_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmpdir_mod, name, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique for {name}"
    mut = src.replace(old, new)
    if name == "gate_up_swapped":  # load up into gate's slot too, so up reads gate's bytes
        mut = mut.replace("orc_dequant_matrix(bg, blob + mat, F, H, ex->up);",
                          "orc_dequant_matrix(bg, blob + mat, F, H, ex->gate);")
    c_path = os.path.join(tmpdir_mod, f"{name}.c")
    so_path = os.path.join(tmpdir_mod, f"lib{name}.so")
    open(c_path, "w").write(mut)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", so_path, c_path, "-lm"],
                   check=True)
    bad = oracle.Oracle(oracle.load(so_path))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(bad)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
