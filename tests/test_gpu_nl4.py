"""The non-linear 4-bit format through the C ABI against the oracle (GPU).

The thread's §四 names a non-linear 4-bit block (32 values in 18 bytes) and
its §三 decode table pairs it, as the down format, with 3-bit gate/up
formats.  The pages print no table of values, so the table is an input
here: a non-linear test table of our own (127 sign(t)|t|^1.6) and an
unordered one; the identity table c - 8 turns the format into the 4-bit
block, which pins the layout against the linear path bit for bit.

Paths: the column-split decode launch (1-4 rows), the matrix-core decode
launch (5-16 rows), the grouped GEMMs, moe_expert_ffn, and the pairs the
decode launches do not build (served by the grouped GEMMs under
MOE_PATH_AUTO).  Bar: routing bit-exact; max |err| <= 2e-3 * rms(oracle)."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL, DevLayer, oracle_forward, rel_err, x_to_dev
from quantized_routed_expert_amd import moe, synth

pytestmark = pytest.mark.gpu

A, D, P = moe.PATH_AUTO, moe.PATH_DECODE, moe.PATH_PREFILL
NL4 = synth.BITS_NL4
CB = synth.nl4_test_codebook()
CB_SCRAMBLE = tuple(((c * 37 + 11) % 256) - 128 for c in range(16))
CB_IDENTITY = tuple(c - 8 for c in range(16))
PAIRS = [(NL4, NL4), (3, NL4)]  # the pairs the decode launch builds


def _nl(cfg, bg, bd, cb=CB, name=None):
    return dataclasses.replace(cfg, name=name or f"{cfg.name}_nl{bg}_{bd}", bits=bg, down_bits=bd, codebook=cb)


def _check(orc, li, path):
    y, idx, w = DevLayer(li).forward(path)
    yr, ir, wr = oracle_forward(orc, li)
    assert np.array_equal(idx, ir), "routing differs"
    assert np.all(np.isfinite(y))
    e = rel_err(y, yr)
    print(f"    rel err {e:.3e}", flush=True)
    assert e <= TOL, e


@pytest.mark.parametrize("bg,bd", PAIRS)
@pytest.mark.parametrize("name,T,path", [
    ("decode", 1, D), ("e512", 1, D), ("e512", 4, D),  # one to four rows: the column-split launch
    ("mtp16", 16, D), ("e512", 8, D),
    ("e512", 64, P),                                  # grouped GEMMs
])
def test_nl4_full_shapes(orc, bg, bd, name, T, path):
    """The workloads' layer shapes (hidden 2048, 128 or 512 experts)."""
    print(f"[nl4] {name} T={T} path={path} gate/up {bg} down {bd}", flush=True)
    _check(orc, synth.layer_inputs(_nl(synth.CONFIGS[name], bg, bd), T=T), path)


@pytest.mark.parametrize("bg,bd", PAIRS)
def test_nl4_edge_shapes(orc, bg, bd):
    """fp32 activations, a shared expert of another FFN width, no shared
    expert, hidden 256 .. 1024, k = E, an unordered table."""
    cases = [
        (synth.scaled_config(synth.CONFIGS["tiny"], name="nl_tiny"), (1, 3, 5, 16, 40), CB),
        (synth.scaled_config(synth.CONFIGS["decode"], name="nl_h512", n_experts=16, hidden=512, ffn=256,
                             shared_ffn=1024), (1, 2, 9, 33), CB_SCRAMBLE),
        (synth.scaled_config(synth.CONFIGS["e512"], name="nl_h1024", n_experts=40, hidden=1024, ffn=768,
                             shared_ffn=0), (1, 12), CB),
        (synth.scaled_config(synth.CONFIGS["tiny"], name="nl_kE", n_experts=6, top_k=6), (2, 7), CB_SCRAMBLE),
    ]
    for base, Ts, cb in cases:
        cfg = _nl(base, bg, bd, cb)
        for T in Ts:
            for path in ((D, P) if T <= 16 else (P,)):
                print(f"[nl4] {cfg.name} T={T} path={path}", flush=True)
                _check(orc, synth.layer_inputs(cfg, T=T, threads=4), path)


@pytest.mark.parametrize("bg,bd", [(NL4, 3), (4, NL4)])
@pytest.mark.parametrize("T", [2, 40])
def test_nl4_pairs_served_by_gemm(orc, bg, bd, T):
    """Pairs outside the decode launch's set: AUTO serves a decode window
    with the grouped GEMMs, and an explicit decode request is refused."""
    cfg = _nl(synth.scaled_config(synth.CONFIGS["decode"], name="nl_other", n_experts=32, hidden=512, ffn=512,
                                  shared_ffn=256), bg, bd)
    li = synth.layer_inputs(cfg, T=T, threads=4)
    print(f"[nl4] gemm-served pair {bg}/{bd} T={T}", flush=True)
    _check(orc, li, A)
    if T <= 16:
        with pytest.raises(moe.MoeError):
            DevLayer(li).forward(D)


@pytest.mark.parametrize("T,path", [(1, D), (3, D), (8, D), (64, P)])
def test_identity_table_is_the_4bit_format(T, path):
    """The same bytes read as 4-bit and as non-linear 4-bit with the table
    c - 8 give the same bits on the launches that serve both formats."""
    cfg4 = synth.scaled_config(synth.CONFIGS["decode"], name="nl_id", n_experts=32, hidden=1024, ffn=512,
                               shared_ffn=512)
    li4 = synth.layer_inputs(cfg4, T=T, threads=4)
    li20 = dataclasses.replace(li4, cfg=dataclasses.replace(cfg4, bits=NL4, codebook=CB_IDENTITY))
    print(f"[nl4] identity table T={T} path={path}", flush=True)
    y4, i4, w4 = DevLayer(li4).forward(path)
    y20, i20, w20 = DevLayer(li20).forward(path)
    assert np.array_equal(i4, i20) and np.array_equal(w4, w20)
    assert np.array_equal(y4, y20)


@pytest.mark.parametrize("bg,bd", PAIRS)
@pytest.mark.parametrize("T,path", [(2, D), (12, D), (70, P)])
def test_nl4_expert_ffn(orc, bg, bd, T, path):
    """moe_expert_ffn on a given grouping, per-pair rows."""
    cfg = _nl(synth.scaled_config(synth.CONFIGS["e512"], name="nl_ffn", n_experts=24, hidden=512, ffn=512),
              bg, bd, CB_SCRAMBLE)
    li = synth.layer_inputs(cfg, T=T, threads=4)
    ri, rw = orc.route(li.logits, cfg.top_k)
    ro, rp, ra = orc.group(ri, cfg.n_experts)
    ref = orc.expert_ffn(li.x, li.x_code, cfg.top_k, cfg.fmt, cfg.n_experts, cfg.hidden, cfg.ffn, li.routed,
                         ro, rp, ra, rw, codebook=cfg.codebook)
    x = x_to_dev(li.x, cfg.x_dtype)
    _, qw = moe.prepare_qweights(torch.from_numpy(li.routed).to(DEV), bg, cfg.n_experts, cfg.hidden, cfg.ffn,
                                 down_bits=bd, codebook=cfg.codebook)
    out = torch.full((T * cfg.top_k, cfg.hidden), float("nan"), device=DEV)
    ws = moe.workspace(T, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, 0, path)
    moe.expert_ffn(x, qw, torch.from_numpy(ro).to(DEV), torch.from_numpy(np.ascontiguousarray(rp)).to(DEV),
                   torch.from_numpy(ra).to(DEV), cfg.top_k, out, ws,
                   pair_w=torch.from_numpy(rw.astype(np.float32)).to(DEV), path=path)
    torch.cuda.synchronize()
    assert moe.workspace_error(ws) == 0
    e = rel_err(out.cpu().numpy(), ref)
    print(f"[nl4] expert_ffn T={T} path={path} {bg}/{bd}: rel err {e:.3e}", flush=True)
    assert e <= TOL
