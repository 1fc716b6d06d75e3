"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a closed form, a hand-built block, a brute
force or an invariant.  The same functions run against deliberately broken
builds of oracle.c (tests/test_oracle_negative.py): every planted mistake
must trip at least one pin.
"""
import dataclasses

import numpy as np

import npref
from quantized_routed_expert_amd import synth


# ----------------------------------------------------------------------------
# scalar formats
# ----------------------------------------------------------------------------

def pin_half(o):
    """binary16 decode against numpy's float16, all 65536 patterns."""
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([o.half_to_double(h) for h in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # the sign of zero matters for -0.0 patterns
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_bf16(o):
    pats = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        ref = (pats.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([o.bf16_to_double(int(b)) for b in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ----------------------------------------------------------------------------
# hand-built blocks (closed forms from the block statement)
# ----------------------------------------------------------------------------

def _blk4(d_bits, qs):
    return bytes([d_bits & 0xFF, d_bits >> 8]) + bytes(qs)


def _blk3(d_bits, ql, qh):
    return bytes([d_bits & 0xFF, d_bits >> 8]) + bytes(ql) + int(qh).to_bytes(4, "little")


def hand_blocks():
    """(name, bits, bytes, expected float64[32]) built by hand."""
    cases = []
    # 4-bit, d = 1.0 (0x3C00): byte i = i | (15-i) << 4  ->  codes i, then 15-i
    qs = [i | ((15 - i) << 4) for i in range(16)]
    exp = [float(i - 8) for i in range(16)] + [float(7 - i) for i in range(16)]
    cases.append(("q4_ramp_d1", 4, _blk4(0x3C00, qs), exp))
    # 4-bit, d = 2^-10 (0x1400), every byte 0x9F: low nibble 15 -> +7, high nibble 9 -> +1
    cases.append(("q4_const_d2m10", 4, _blk4(0x1400, [0x9F] * 16),
                  [7 * 2.0 ** -10] * 16 + [1 * 2.0 ** -10] * 16))
    # 4-bit, d = -1.0 (0xBC00), byte 0x80: low 0 -> -(0-8) = 8, high 8 -> 0
    cases.append(("q4_negd", 4, _blk4(0xBC00, [0x80] * 16), [8.0] * 16 + [0.0] * 16))
    # 4-bit, smallest subnormal scale 2^-24, byte 0xF0: low 0 -> -8, high 15 -> 7
    cases.append(("q4_subnormal", 4, _blk4(0x0001, [0xF0] * 16),
                  [-8 * 2.0 ** -24] * 16 + [7 * 2.0 ** -24] * 16))
    # 4-bit, largest normal 65504 (0x7BFF), byte 0x98: low 8 -> 0, high 9 -> 65504
    cases.append(("q4_max", 4, _blk4(0x7BFF, [0x98] * 16), [0.0] * 16 + [65504.0] * 16))
    # 4-bit, one code per block position: code of weight i is (i*5) % 16
    codes = [(i * 5) % 16 for i in range(32)]
    qs = [codes[i] | (codes[i + 16] << 4) for i in range(16)]
    cases.append(("q4_scatter_d0.5", 4, _blk4(0x3800, qs), [0.5 * (c - 8) for c in codes]))
    # 3-bit, d = 1.0, code of weight i = i % 8: every 2-bit field of byte j is j & 3,
    # and the third bit is set exactly where i % 8 >= 4
    ql = [(j & 3) * 0x55 for j in range(8)]
    qh = sum(1 << i for i in range(32) if (i % 8) >= 4)
    cases.append(("q3_mod8_d1", 3, _blk3(0x3C00, ql, qh), [float((i % 8) - 4) for i in range(32)]))
    # 3-bit, d = 0.5 (0x3800), code of weight i = 7 - i//4
    codes = [7 - i // 4 for i in range(32)]
    ql = [0] * 8
    for i, c in enumerate(codes):
        ql[i % 8] |= (c & 3) << (2 * (i // 8))
    qh = sum(((c >> 2) & 1) << i for i, c in enumerate(codes))
    cases.append(("q3_desc_d0.5", 3, _blk3(0x3800, ql, qh), [0.5 * (c - 4) for c in codes]))
    # 3-bit, d = -2.0 (0xC000), only weight 31 has code 7, the rest code 0
    ql = [0] * 8
    ql[31 % 8] |= 3 << (2 * (31 // 8))
    cases.append(("q3_single", 3, _blk3(0xC000, ql, 1 << 31),
                  [-2.0 * (0 - 4)] * 31 + [-2.0 * (7 - 4)]))
    return cases


def pin_blocks(o):
    for name, bits, raw, exp in hand_blocks():
        got = o.dequant_block(bits, raw)
        assert np.array_equal(got, np.array(exp, dtype=np.float64)), name


# Non-linear 4-bit: the pages name the block (32 values in 18 bytes, 4-bit
# codes indexing a table) but print no table, so the table is an input.  The
# pins use tables chosen to expose index, sign and layout mistakes.
NL4 = 20
CB_TEST = synth.nl4_test_codebook()                        # monotone, odd-symmetric
CB_SCRAMBLE = tuple(((c * 37 + 11) % 256) - 128 for c in range(16))  # distinct, unordered, signed
CB_EXTREME = (-128, 127, -1, 0, 1, -127, 126, -64, 64, -2, 2, 100, -100, 3, -3, 5)
CB_IDENTITY = tuple(c - 8 for c in range(16))              # reduces to the 4-bit format


def pin_nl4_blocks(o):
    """Hand-built non-linear blocks: value i is d * table[code i] (codes in the
    4-bit block's nibble order), for several tables and scales."""
    qs = [i | ((15 - i) << 4) for i in range(16)]  # codes 0..15, then 15..0
    for cb, d_bits, d in ((CB_TEST, 0x3C00, 1.0), (CB_SCRAMBLE, 0xB800, -0.5), (CB_EXTREME, 0x0001, 2.0 ** -24),
                          (CB_EXTREME, 0x7BFF, 65504.0)):
        exp = [d * cb[i] for i in range(16)] + [d * cb[15 - i] for i in range(16)]
        got = o.dequant_block(NL4, _blk4(d_bits, qs), codebook=cb)
        assert np.array_equal(got, np.array(exp, dtype=np.float64)), (cb, d)
    # one code everywhere: every weight is d * table[that code]
    for c in range(16):
        got = o.dequant_block(NL4, _blk4(0x3400, [c | (c << 4)] * 16), codebook=CB_SCRAMBLE)
        assert np.all(got == 0.25 * CB_SCRAMBLE[c]), c


def pin_nl4_reductions(o, seed=5):
    """With the table c - 8 the non-linear block is the 4-bit block, bitwise,
    on random bytes; with other tables it agrees with the numpy decoder's
    table lookup; random codes packed by the encoder decode to d * table[code]."""
    rg = np.random.default_rng(seed)
    raw = rg.integers(0, 256, size=(300, 18)).astype(np.uint8)
    raw[:, 1] &= 0x7B
    raw = raw.reshape(-1)
    assert np.array_equal(o.dequant_matrix(NL4, raw, 300, 32, codebook=CB_IDENTITY),
                          o.dequant_matrix(4, raw, 300, 32))
    for cb in (CB_TEST, CB_SCRAMBLE, CB_EXTREME):
        assert np.array_equal(o.dequant_matrix(NL4, raw, 300, 32, codebook=cb),
                              npref.dequant_blocks(raw, NL4, cb)), cb
    codes = rg.integers(0, 16, size=(64, 32)).astype(np.uint8)
    d16 = (rg.standard_normal(64) * 0.01).astype(np.float16)
    packed = synth.pack_codes(codes, d16, NL4)
    got = o.dequant_matrix(NL4, packed, 64, 32, codebook=CB_SCRAMBLE)
    exp = d16.astype(np.float64)[:, None] * np.array(CB_SCRAMBLE, dtype=np.float64)[codes]
    assert np.array_equal(got, exp)


def pin_encoder_roundtrip(o, seed=7):
    """Random codes and scales packed by the input encoder, decoded by the
    oracle, equal d * (code - bias) exactly."""
    rg = np.random.default_rng(seed)
    for bits in (4, 3):
        n = 64
        codes = rg.integers(0, 1 << bits, size=(n, 32)).astype(np.uint8)
        d16 = (rg.standard_normal(n) * 0.01).astype(np.float16)
        raw = synth.pack_codes(codes, d16, bits)
        B = o.block_bytes(bits)
        for b in range(n):
            got = o.dequant_block(bits, raw[b * B:(b + 1) * B])
            exp = d16[b].astype(np.float64) * (codes[b].astype(np.float64) - (1 << (bits - 1)))
            assert np.array_equal(got, exp), (bits, b)


def pin_matrix_indexing(o):
    """Per-(row, block) scales 2^r * (b+1) locate each block in a matrix."""
    for bits in (4, 3):
        rows, cols = 5, 96
        nb = cols // 32
        codes = np.full((rows * nb, 32), (1 << (bits - 1)) + 1, dtype=np.uint8)  # value = d * 1
        d = np.array([2.0 ** r * (b + 1) for r in range(rows) for b in range(nb)], dtype=np.float16)
        raw = synth.pack_codes(codes, d, bits)
        got = o.dequant_matrix(bits, raw, rows, cols)
        exp = np.repeat(d.astype(np.float64).reshape(rows, nb), 32, axis=1)
        assert np.array_equal(got, exp), bits
        assert np.array_equal(got, npref.dequant_matrix(raw, bits, rows, cols))


def pin_numpy_dequant_agrees(o, seed=3):
    """Oracle and the independent numpy decoder on random bytes (any byte
    string is a valid block apart from inf/NaN scales)."""
    rg = np.random.default_rng(seed)
    for bits in (4, 3):
        B = o.block_bytes(bits)
        raw = rg.integers(0, 256, size=(200, B)).astype(np.uint8)
        raw[:, 1] &= 0x7B  # keep the exponent below 31 (no inf/NaN scales)
        raw = raw.reshape(-1)
        got = o.dequant_matrix(bits, raw, 200, 32)
        assert np.array_equal(got, npref.dequant_blocks(raw, bits)), bits


def pin_expert_bytes(o):
    # bytes per expert = 3*H*F/32*B for the five workloads' shapes
    assert o.expert_bytes(4, 256, 512) == 221184
    assert o.expert_bytes(4, 2048, 768) == 2654208
    assert o.expert_bytes(3, 2048, 768) == 2064384
    assert o.expert_bytes(3, 2048, 512) == 1376256
    assert o.expert_bytes(5, 256, 512) == -1
    assert o.expert_bytes(4, 250, 512) == -1
    # per-projection widths: H*F/32 * (2*B_gate/up + B_down)
    assert o.expert_bytes(3 | (4 << 8), 2048, 512) == 2048 * 16 * (2 * 14 + 18) == 1507328
    assert o.expert_bytes(4 | (3 << 8), 2048, 768) == 2048 * 24 * (2 * 18 + 14) == 2457600
    assert o.expert_bytes(3 | (3 << 8), 2048, 512) == o.expert_bytes(3, 2048, 512)
    assert o.expert_bytes(3 | (5 << 8), 2048, 512) == -1
    assert o.expert_bytes(3 | (4 << 16), 2048, 512) == -1
    # the non-linear 4-bit block is 18 bytes, alone or beside another width
    assert o.block_bytes(NL4) == 18
    assert o.expert_bytes(NL4, 2048, 768) == 2654208
    assert o.expert_bytes(3 | (NL4 << 8), 2048, 512) == 2048 * 16 * (2 * 14 + 18)
    assert o.expert_bytes(NL4 | (3 << 8), 2048, 512) == 2048 * 16 * (2 * 18 + 14)


def pin_format_bits(o):
    assert (o.format_bits(3, False), o.format_bits(3, True)) == (3, 3)
    assert (o.format_bits(4, False), o.format_bits(4, True)) == (4, 4)
    assert (o.format_bits(3 | (4 << 8), False), o.format_bits(3 | (4 << 8), True)) == (3, 4)
    assert (o.format_bits(4 | (3 << 8), False), o.format_bits(4 | (3 << 8), True)) == (4, 3)
    assert o.format_bits(2, False) == -1 and o.format_bits(4 | (2 << 8), True) == -1
    assert (o.format_bits(3 | (NL4 << 8), False), o.format_bits(3 | (NL4 << 8), True)) == (3, NL4)
    assert (o.format_bits(NL4, False), o.format_bits(NL4, True)) == (NL4, NL4)
    assert o.format_bits(21, False) == -1


def pin_mixed_expert_indexing(o):
    """A blob with gate/up in one width and down in the other: every block's
    scale names its (matrix, row, block) and every code is bias + 1, so each
    dequantized weight is its block's scale; the three matrices must come back
    at their own offsets, in their own widths."""
    H, F = 64, 96
    for bg, bd in ((3, 4), (4, 3)):
        mats, exp = [], []
        for m, (rows, cols, bits) in enumerate(((F, H, bg), (F, H, bg), (H, F, bd))):
            nb = cols // 32
            d = np.array([(m + 1) * 256 + r * 4 + b for r in range(rows) for b in range(nb)], dtype=np.float64)
            d16 = (d / 4096.0).astype(np.float16)  # exact: 11-bit integers over a power of two
            assert np.array_equal(d16.astype(np.float64), d / 4096.0)
            codes = np.full((rows * nb, 32), (1 << (bits - 1)) + 1, dtype=np.uint8)
            mats.append(synth.pack_codes(codes, d16, bits))
            exp.append(np.repeat((d / 4096.0).reshape(rows, nb), 32, axis=1))
        blob = np.concatenate(mats)
        fmt = bg | (bd << 8)
        assert blob.size == o.expert_bytes(fmt, H, F)
        got = o.dequant_expert(fmt, blob, H, F)
        for g, e in zip(got, exp):
            assert np.array_equal(g, e), (bg, bd)
        for g, e in zip(npref.dequant_expert(blob, bg, H, F, bd), exp):
            assert np.array_equal(g, e)


# ----------------------------------------------------------------------------
# router projection
# ----------------------------------------------------------------------------

def pin_router_logits(o, seed=21):
    """x W^T against numpy's float64 matrix product (bf16 and fp32 x), exact
    integers for small integer inputs, and one-hot rows picking W's columns."""
    rg = np.random.default_rng(seed)
    T, H, E = 5, 96, 12
    w = synth.f32_to_bf16_bits((rg.standard_normal((E, H)) * 0.1).astype(np.float32))
    W = npref.bf16_bits_to_f64(w)
    for code in (0, 1):
        xf = rg.standard_normal((T, H)).astype(np.float32)
        x = xf if code == 0 else synth.f32_to_bf16_bits(xf)
        got = o.router_logits(x, code, w)
        ref = npref.x_to_f64(x, code) @ W.T
        assert np.max(np.abs(got - ref)) <= 1e-13 * np.sqrt(np.mean(ref ** 2)), code
    # small integers: every product and partial sum is exact in binary64
    xi = rg.integers(-8, 9, (T, H)).astype(np.float32)
    wi = synth.f32_to_bf16_bits(rg.integers(-8, 9, (E, H)).astype(np.float32))
    exact = xi.astype(np.int64) @ npref.bf16_bits_to_f64(wi).astype(np.int64).T
    assert np.array_equal(o.router_logits(xi, 0, wi), exact.astype(np.float64))
    # one-hot rows: logits[t][e] = W[e][h_t]
    hs = rg.integers(0, H, T)
    oh = np.zeros((T, H), np.float32)
    oh[np.arange(T), hs] = 1.0
    assert np.array_equal(o.router_logits(oh, 0, w), W[:, hs].T)


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

def _brute_route(L, k):
    order = np.argsort(-L.astype(np.float64), axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(L.astype(np.float64), order, axis=1)
    ex = np.exp(sel - sel[:, :1])
    return order.astype(np.int32), ex / ex.sum(axis=1, keepdims=True)


def pin_route_bruteforce(o, seed=11):
    rg = np.random.default_rng(seed)
    for (T, E, k) in [(1, 8, 2), (7, 16, 3), (5, 128, 8), (3, 512, 10), (4, 9, 9)]:
        L = rg.standard_normal((T, E)).astype(np.float32) * 2
        idx, w = o.route(L, k)
        bi, bw = _brute_route(L, k)
        assert np.array_equal(idx, bi), (T, E, k)
        assert np.allclose(w, bw, rtol=1e-14, atol=0)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 4 * k * np.finfo(np.float64).eps)


def pin_route_ties(o, seed=12):
    """Many exact ties: integer logits from a small range; ties go to the lower id."""
    rg = np.random.default_rng(seed)
    L = rg.integers(-2, 3, size=(20, 16)).astype(np.float32)
    idx, w = o.route(L, 5)
    bi, bw = _brute_route(L, 5)
    assert np.array_equal(idx, bi)
    assert np.allclose(w, bw, rtol=1e-14)


def pin_route_special(o):
    # k = 1: weight exactly 1
    L = np.array([[0.5, 3.0, -1.0, 3.0]], dtype=np.float32)
    idx, w = o.route(L, 1)
    assert idx.tolist() == [[1]] and w.tolist() == [[1.0]]
    # all-equal logits: ids 0..k-1, weights 1/k
    L = np.full((3, 12), 0.25, dtype=np.float32)
    idx, w = o.route(L, 4)
    assert idx.tolist() == [[0, 1, 2, 3]] * 3
    assert np.allclose(w, 0.25, rtol=0, atol=1e-16)
    # two selected with a logit gap of ln 3: weights 3/4 and 1/4
    L = np.array([[0.0, np.log(3.0), -5.0]], dtype=np.float32)
    idx, w = o.route(L, 2)
    gap = float(np.float32(np.log(3.0)))
    assert idx.tolist() == [[1, 0]]
    assert abs(w[0, 0] - np.exp(gap) / (1 + np.exp(gap))) < 1e-15
    # selection compares the fp32 logits: adjacent floats are ordered
    a = np.float32(1.0)
    L = np.array([[a, np.nextafter(a, np.float32(2)), a]], dtype=np.float32)
    idx, _ = o.route(L, 2)
    assert idx.tolist() == [[1, 0]]


# ----------------------------------------------------------------------------
# grouping
# ----------------------------------------------------------------------------

def pin_group(o, seed=13):
    rg = np.random.default_rng(seed)
    for (T, E, k) in [(1, 8, 2), (16, 128, 8), (64, 512, 10), (9, 4, 4), (0, 4, 2)]:
        if T:
            L = rg.standard_normal((T, E)).astype(np.float32)
            idx, _ = o.route(L, k)
        else:
            idx = np.zeros((0, k), dtype=np.int32)
        off, pairs, act = o.group(idx, E)
        flat = idx.reshape(-1)
        assert off[0] == 0 and off[E] == T * k
        assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
        assert sorted(pairs.tolist()) == list(range(T * k))
        assert pairs.tolist() == sorted(range(T * k), key=lambda p: (flat[p], p))
        nz = np.nonzero(np.bincount(flat, minlength=E))[0]
        assert act[0] == nz.size and act[1:1 + nz.size].tolist() == nz.tolist()


# ----------------------------------------------------------------------------
# layer
# ----------------------------------------------------------------------------

def small_cfg(bits, x_dtype, E=12, H=64, F=96, k=3, Fs=64, logits=("normal", 1.0)):
    return synth.Config("pin", 90 + bits, H, E, F, k, Fs, (6,), bits, x_dtype, logits, 1)


def pin_layer_dense(o):
    """Oracle layer == dense-with-mask brute force (all experts on all rows),
    uniform, per-projection and non-linear formats."""
    for bits, db, xd, Fs in [(4, 0, "f32", 64), (3, 0, "bf16", 96), (4, 0, "bf16", 0), (3, 0, "f32", 32),
                             (3, 4, "bf16", 64), (4, 3, "f32", 96), (NL4, 0, "bf16", 64), (3, NL4, "f32", 96),
                             (NL4, 3, "bf16", 0)]:
        cb = CB_SCRAMBLE if NL4 in (bits, db) else ()
        cfg = dataclasses.replace(small_cfg(bits, xd, Fs=Fs), down_bits=db, codebook=cb)
        li = synth.layer_inputs(cfg, T=7, threads=1)
        y, idx, w = o.layer_forward(li.x, li.x_code, li.logits, cfg.top_k, cfg.fmt, cfg.ffn,
                                    li.routed, li.shared, s_ffn=Fs or None, codebook=cb or None)
        yr, ir, M = npref.dense_masked_layer(li.x, li.x_code, li.logits, cfg.top_k, bits,
                                             cfg.hidden, cfg.ffn, li.routed, li.shared,
                                             s_F=Fs or None, down_bits=cfg.dbits, codebook=cb or None)
        assert np.array_equal(idx, ir)
        rms = np.sqrt(np.mean(yr ** 2))
        assert np.max(np.abs(y - yr)) <= 1e-12 * rms, (bits, db, xd, np.max(np.abs(y - yr)) / rms)


def pin_layer_single_expert(o):
    """E = 1, k = 1: two SwiGLU MLPs summed (routed weight is exactly 1)."""
    for bits in (4, 3):
        cfg = small_cfg(bits, "f32", E=1, k=1, H=96, F=64, Fs=128)
        li = synth.layer_inputs(cfg, T=5, threads=1)
        y, idx, w = o.layer_forward(li.x, 0, li.logits, 1, bits, 64, li.routed, li.shared, s_ffn=128)
        X = li.x.astype(np.float64)
        ref = npref.swiglu_mlp(X, *npref.dequant_expert(li.routed, bits, 96, 64)) + \
            npref.swiglu_mlp(X, *npref.dequant_expert(li.shared, bits, 96, 128))
        assert np.all(idx == 0) and np.all(w == 1.0)
        assert np.max(np.abs(y - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def pin_layer_zeros(o):
    cfg = small_cfg(4, "f32")
    li = synth.layer_inputs(cfg, T=4, threads=1)
    y, _, _ = o.layer_forward(np.zeros_like(li.x), 0, li.logits, 3, 4, cfg.ffn, li.routed, li.shared,
                              s_ffn=cfg.shared_ffn)
    assert np.all(y == 0.0)
    # every code at the bias: all weights are zero whatever the scale
    for bits in (4, 3):
        cfg = small_cfg(bits, "f32")
        li = synth.layer_inputs(cfg, T=4, threads=1)
        nblk = li.routed.size // cfg.block_bytes
        bias = np.full((nblk, 32), 1 << (bits - 1), dtype=np.uint8)
        routed = synth.pack_codes(bias, np.full(nblk, 0.37, np.float16), bits)
        nsb = li.shared.size // cfg.block_bytes
        shared = synth.pack_codes(np.full((nsb, 32), 1 << (bits - 1), np.uint8),
                                  np.full(nsb, -3.0, np.float16), bits)
        y, _, _ = o.layer_forward(li.x, 0, li.logits, 3, bits, cfg.ffn, routed, shared,
                                  s_ffn=cfg.shared_ffn)
        assert np.all(y == 0.0)


def pin_layer_invariances(o):
    """Token permutation and batch invariance, bitwise: rows are independent."""
    cfg = small_cfg(3, "bf16")
    li = synth.layer_inputs(cfg, T=6, threads=1)
    sf = cfg.shared_ffn
    y, _, _ = o.layer_forward(li.x, 1, li.logits, 3, 3, cfg.ffn, li.routed, li.shared, s_ffn=sf)
    perm = np.array([4, 0, 5, 2, 1, 3])
    yp, _, _ = o.layer_forward(li.x[perm].copy(), 1, li.logits[perm].copy(), 3, 3, cfg.ffn,
                               li.routed, li.shared, s_ffn=sf)
    assert np.array_equal(yp, y[perm])
    for t in range(6):
        y1, _, _ = o.layer_forward(li.x[t:t + 1].copy(), 1, li.logits[t:t + 1].copy(), 3, 3,
                                   cfg.ffn, li.routed, li.shared, s_ffn=sf)
        assert np.array_equal(y1[0], y[t])
    ys, _, _ = o.layer_forward(li.x, 1, li.logits, 3, 3, cfg.ffn, li.routed, li.shared, s_ffn=sf,
                               rows=[5, 1])
    assert np.array_equal(ys, y[[5, 1]])


def pin_expert_ffn_matches_layer(o):
    """Per-pair outputs w*o, summed in slot order plus the shared MLP, give the layer."""
    cfg = small_cfg(4, "bf16")
    li = synth.layer_inputs(cfg, T=5, threads=1)
    y, idx, w = o.layer_forward(li.x, 1, li.logits, 3, 4, cfg.ffn, li.routed, li.shared,
                                s_ffn=cfg.shared_ffn)
    off, pairs, act = o.group(idx, cfg.n_experts)
    po = o.expert_ffn(li.x, 1, 3, 4, cfg.n_experts, cfg.hidden, cfg.ffn, li.routed, off, pairs, act, w)
    X = npref.x_to_f64(li.x, 1)
    s = npref.swiglu_mlp(X, *npref.dequant_expert(li.shared, 4, cfg.hidden, cfg.shared_ffn))
    ref = po.reshape(5, 3, -1).sum(axis=1) + s
    assert np.max(np.abs(ref - y)) <= 1e-12 * np.sqrt(np.mean(y ** 2))
    # weight 1 when pair_w is absent
    po1 = o.expert_ffn(li.x, 1, 3, 4, cfg.n_experts, cfg.hidden, cfg.ffn, li.routed, off, pairs, act)
    nz = w.reshape(-1) > 0
    assert np.allclose(po[nz], po1[nz] * w.reshape(-1)[nz, None], rtol=1e-13, atol=0)


ALL_PINS = [pin_half, pin_bf16, pin_blocks, pin_nl4_blocks, pin_nl4_reductions, pin_encoder_roundtrip, pin_matrix_indexing,
            pin_numpy_dequant_agrees, pin_expert_bytes, pin_format_bits, pin_mixed_expert_indexing,
            pin_router_logits, pin_route_bruteforce, pin_route_ties,
            pin_route_special, pin_group, pin_layer_dense, pin_layer_single_expert,
            pin_layer_zeros, pin_layer_invariances, pin_expert_ffn_matches_layer]
