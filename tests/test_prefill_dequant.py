"""CPU model of the prefill GEMM's in-register dequantization (no GPU).

The gate/up and down tiles turn one k-group (8 weights) of a quant block into
8 bf16 values with byte permutes (v_perm_b32: selector byte k < 4 picks byte k
of the second source, 4..7 byte k-4 of the first) and, for 4-bit, a signed
bit-field extract.  This models those integer steps bit for bit and checks
them against the block format's own definition (the weight = code minus the
bias, as an exact bf16), over random bytes and both blocks of a pair: the
dword realignment of the even block and the aligned odd block."""
import struct

import numpy as np


def perm(s0, s1, sel):
    pool = [(s1 >> (8 * i)) & 255 for i in range(4)] + [(s0 >> (8 * i)) & 255 for i in range(4)]
    out = 0
    for b in range(4):
        k = (sel >> (8 * b)) & 255
        out |= (pool[k] if k < 8 else (0 if k == 12 else 255)) << (8 * b)
    return out


def bf16(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0] >> 16


def alignbit(hi, lo, s):
    return (((hi << 32) | lo) >> s) & 0xFFFFFFFF


def deq3_group(qs0, qs1, qh, g):
    sh = 2 * g
    l0, l1 = (qs0 >> sh) & 0x03030303, (qs1 >> sh) & 0x03030303
    t0, t1 = (qh >> (8 * g)) & 15, (qh >> (8 * g + 4)) & 15
    mul24 = lambda a, b: ((a & 0xFFFFFF) * (b & 0xFFFFFF)) & 0xFFFFFFFF
    c0 = (mul24(t0, 0x810204) & 0x04040404) | l0
    c1 = (mul24(t1, 0x810204) & 0x04040404) | l1
    h0, b0 = perm(0x40403F00, 0xBFC0C0C0, c0), perm(0x40008000, 0x80004080, c0)
    h1, b1 = perm(0x40403F00, 0xBFC0C0C0, c1), perm(0x40008000, 0x80004080, c1)
    words = [perm(h0, b0, 0x05010400), perm(h0, b0, 0x07030602), perm(h1, b1, 0x05010400), perm(h1, b1, 0x07030602)]
    return [(w >> (16 * k)) & 0xFFFF for w in words for k in range(2)]


def sbfe(x, off, w):
    v = (x >> off) & ((1 << w) - 1)
    return v - (1 << w) if v >> (w - 1) else v


def deq4_group(qa, qb, ns):
    qa ^= 0x88888888
    qb ^= 0x88888888
    return [bf16(sbfe(qa, 8 * j + ns, 4)) for j in range(4)] + [bf16(sbfe(qb, 8 * j + ns, 4)) for j in range(4)]


def block_fields(w, odd, o, nq):
    if not odd:
        return w[0] & 0xFFFF, [alignbit(w[i + 1], w[i], 16) for i in range(nq)]
    return w[o] >> 16, [w[o + 1 + i] for i in range(nq)]


def test_dequant_3bit_pairs():
    rng = np.random.default_rng(11)
    for _ in range(500):
        pair = rng.integers(0, 256, 28, dtype=np.uint8).tobytes()
        w = list(struct.unpack("<7I", pair))
        for blk in range(2):
            b = pair[14 * blk:14 * blk + 14]
            qs, qh = b[2:10], int.from_bytes(b[10:14], "little")
            ref = [bf16((((qs[i & 7] >> (2 * (i >> 3))) & 3) | (((qh >> i) & 1) << 2)) - 4) for i in range(32)]
            d, q = block_fields(w, blk == 1, 3, 3)
            assert d == int.from_bytes(b[0:2], "little")
            got = sum((deq3_group(q[0], q[1], q[2], g) for g in range(4)), [])
            assert got == ref


def test_dequant_4bit_pairs():
    rng = np.random.default_rng(12)
    for _ in range(500):
        pair = rng.integers(0, 256, 36, dtype=np.uint8).tobytes()
        w = list(struct.unpack("<9I", pair))
        for blk in range(2):
            b = pair[18 * blk:18 * blk + 18]
            qs = b[2:18]
            ref = [bf16((qs[i] & 15) - 8) for i in range(16)] + [bf16((qs[i] >> 4) - 8) for i in range(16)]
            d, q = block_fields(w, blk == 1, 4, 4)
            assert d == int.from_bytes(b[0:2], "little")
            got = []
            for g in range(4):
                odd = g & 1
                got += deq4_group(q[2] if odd else q[0], q[3] if odd else q[1], 4 * (g >> 1))
            assert got == ref


def test_down_odd_row_run():
    """Down tiles load an odd row's block from the dword holding its scale
    (12 bytes into a 3-bit row pair, 16 into a 4-bit one)."""
    rng = np.random.default_rng(13)
    for bits, bb, off, nq in ((3, 14, 12, 3), (4, 18, 16, 4)):
        for _ in range(200):
            pair = rng.integers(0, 256, 2 * bb, dtype=np.uint8).tobytes()
            run = list(struct.unpack(f"<{(2 * bb - off) // 4}I", pair[off:]))
            d, q = block_fields(run, True, 0, nq)
            assert d == int.from_bytes(pair[bb:bb + 2], "little")
            assert q == list(struct.unpack(f"<{nq}I", pair[bb + 2:bb + 2 + 4 * nq]))
