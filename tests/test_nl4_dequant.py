"""CPU model of the non-linear 4-bit operand paths (no GPU).

The non-linear block has the 4-bit block's bytes; each code indexes a table
of 16 signed 8-bit values.  The kernels hold the table as two byte tables
(the low and the high bytes of a 16-bit float of each entry: fp16 for the
decode launch, bf16 for the grouped GEMM), look four codes up at a time with
v_perm_b32 (entries 0..7 and 8..15 apart, bit 3 of each code choosing by a
byte mask), then interleave low and high bytes into 16-bit values.  This
models those integer steps bit for bit and checks them against the format's
definition (the weight = table[code], as an exact 16-bit float) for random
tables and blocks: the decode lane order (pos_in_block of the 4-bit layout)
and the grouped GEMM's natural order.  The column-split launch instead looks
the codes up in the table's own signed bytes and multiplies them by two
signed radix-256 digits of the integer activations (v_dot4_i32_i8); its
block sums must be the exact integer dot products."""
import struct

import numpy as np

from test_prefill_dequant import alignbit, bf16, perm
from test_split_digits import nibble_k  # the 4-bit layout's nibble -> k map


def fp16(x):
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def tables(cb, conv):
    """The NlTab words: t[0..3] low bytes of entries 0..15, t[4..7] high bytes."""
    t = [0] * 8
    for c in range(16):
        h = conv(cb[c])
        t[c >> 2] |= (h & 0xFF) << (8 * (c & 3))
        t[4 + (c >> 2)] |= (h >> 8) << (8 * (c & 3))
    return t


def nl_lookup(c, t):
    s = c & 0x07070707
    b3 = c & 0x08080808
    m = ((b3 << 5) - (b3 >> 3)) & 0xFFFFFFFF
    l0, l1 = perm(t[1], t[0], s), perm(t[3], t[2], s)
    h0, h1 = perm(t[5], t[4], s), perm(t[7], t[6], s)
    return (l1 & m) | (l0 & ~m & 0xFFFFFFFF), (h1 & m) | (h0 & ~m & 0xFFFFFFFF)


def unpack_nl4(q, t):
    """Decode launch: code bytes 4g..4g+3 -> 8 fp16 patterns in slot order."""
    l0, h0 = nl_lookup(q & 0x0F0F0F0F, t)
    l1, h1 = nl_lookup((q >> 4) & 0x0F0F0F0F, t)
    words = [perm(h0, l0, 0x06020400), perm(h1, l1, 0x06020400), perm(h0, l0, 0x07030501),
             perm(h1, l1, 0x07030501)]
    return [(w >> (16 * k)) & 0xFFFF for w in words for k in range(2)]


def deqnl_group(qa, qb, ns, t):
    """Grouped GEMM: 8 consecutive weights -> 8 bf16 patterns in order."""
    la, ha = nl_lookup((qa >> ns) & 0x0F0F0F0F, t)
    lb, hb = nl_lookup((qb >> ns) & 0x0F0F0F0F, t)
    words = [perm(ha, la, 0x05010400), perm(ha, la, 0x07030602), perm(hb, lb, 0x05010400),
             perm(hb, lb, 0x07030602)]
    return [(w >> (16 * k)) & 0xFFFF for w in words for k in range(2)]


def pos_in_block(g, e):
    r = ((e >> 2) & 1) + ((e & 1) << 1)
    return 4 * g + r + ((e >> 1) & 1) * 16


def block_codes(blk):
    return [(blk[2 + i] & 15) if i < 16 else (blk[2 + i - 16] >> 4) for i in range(32)]


def random_tables(rng, n):
    out = [tuple(int(v) for v in rng.integers(-128, 128, 16)) for _ in range(n)]
    out.append((-128, 127, -1, 0, 1, -127, 126, -64, 64, -2, 2, 100, -100, 3, -3, 5))
    out.append(tuple(c - 8 for c in range(16)))
    return out


def test_mask_spreads_bit3_per_byte():
    for c in range(1 << 16):  # every pair of codes in bytes 0 and 3, bytes 1 and 2 from c too
        codes = [c & 15, (c >> 4) & 15, (c >> 8) & 15, (c >> 12) & 15]
        w = sum(v << (8 * i) for i, v in enumerate(codes))
        b3 = w & 0x08080808
        m = ((b3 << 5) - (b3 >> 3)) & 0xFFFFFFFF
        assert m == sum((0xFF if v >= 8 else 0) << (8 * i) for i, v in enumerate(codes))


def test_decode_lane_values():
    rng = np.random.default_rng(31)
    for cb in random_tables(rng, 20):
        t = tables(cb, fp16)
        for _ in range(40):
            blk = bytes(2) + rng.integers(0, 256, 16, dtype=np.uint8).tobytes()
            codes = block_codes(blk)
            for g in range(4):
                q = int.from_bytes(blk[2 + 4 * g:6 + 4 * g], "little")
                got = unpack_nl4(q, t)
                assert got == [fp16(cb[codes[pos_in_block(g, e)]]) for e in range(8)]


def test_decode_pair_realignment():
    """Block 0 of a pair: code bytes 2+4g.. read as alignbyte(w1, w0, 2)."""
    rng = np.random.default_rng(32)
    cb = random_tables(rng, 1)[0]
    t = tables(cb, fp16)
    for _ in range(200):
        pair = rng.integers(0, 256, 36, dtype=np.uint8).tobytes()
        w = struct.unpack("<9I", pair)
        codes = block_codes(pair[:18])
        for g in range(4):
            q = alignbit(w[g + 1], w[g], 16)
            assert unpack_nl4(q, t) == [fp16(cb[codes[pos_in_block(g, e)]]) for e in range(8)]


def test_gemm_group_values():
    rng = np.random.default_rng(33)
    for cb in random_tables(rng, 20):
        t = tables(cb, bf16)
        for _ in range(40):
            blk = bytes(2) + rng.integers(0, 256, 16, dtype=np.uint8).tobytes()
            codes = block_codes(blk)
            q = [int.from_bytes(blk[2 + 4 * i:6 + 4 * i], "little") for i in range(4)]
            for g in range(4):
                odd = g & 1
                got = deqnl_group(q[2] if odd else q[0], q[3] if odd else q[1], 4 * (g >> 1), t)
                assert got == [bf16(cb[codes[8 * g + e]]) for e in range(8)]


def test_tables_are_exact():
    # every 8-bit integer is exact in fp16 and in bf16
    for v in range(-128, 128):
        assert np.float16(v) == v
        assert struct.unpack("<f", struct.pack("<I", bf16(v) << 16))[0] == v


# ---------------------------------------------------------------------------
# The column-split launch: table bytes times signed radix-256 digits
# ---------------------------------------------------------------------------


def sdot4(a, b, c):
    for i in range(4):
        x, y = (a >> 8 * i) & 255, (b >> 8 * i) & 255
        c += (x - 256 if x >= 128 else x) * (y - 256 if y >= 128 else y)
    return c


def nl8_lookup(c, tb):
    s = c & 0x07070707
    t = c & 0x08080808
    m = ((t << 5) - (t >> 3)) & 0xFFFFFFFF
    lo, hi = perm(tb[1], tb[0], s), perm(tb[3], tb[2], s)
    return (hi & m) | (lo & ~m & 0xFFFFFFFF)


def digit_words8(a, kmask):
    """[digit 2][parity 2][nibble-dword 9] words of signed bytes."""
    out = [0] * 36
    for nd in range(9):
        D = [0] * 4
        for i in range(8):
            kk = nibble_k(4, nd, i)
            v = int(a[kk & kmask]) if kk >= 0 else 0
            a0 = ((v + 128) & 255) - 128
            a1 = (v - a0) >> 8
            assert -128 <= a1 <= 127 and a0 + 256 * a1 == v
            D[i & 1] |= (a0 & 255) << (8 * (i >> 1))
            D[2 + (i & 1)] |= (a1 & 255) << (8 * (i >> 1))
        for j in range(4):
            out[j * 9 + nd] = D[j]
    return out


def split_blocks(w, tb, xd):
    be = [nl8_lookup(w[q] & 0x0F0F0F0F, tb) for q in range(9)]
    bo = [nl8_lookup((w[q] >> 4) & 0x0F0F0F0F, tb) for q in range(9)]
    a0, a1 = [0, 0], [0, 0]
    for j in range(2):
        for q in range(9):
            dst = a0 if q < 5 else a1
            dst[j] = sdot4(be[q], xd[(2 * j) * 9 + q], dst[j])
            dst[j] = sdot4(bo[q], xd[(2 * j + 1) * 9 + q], dst[j])
    return a0[0] + 256 * a0[1], a1[0] + 256 * a1[1]


def test_split_pair_exact_dot_products():
    """Gate/up (two blocks of a row, kmask 63) and down (one block read by
    two rows, kmask 31): the launch's sums equal sum table[code] * a."""
    rng = np.random.default_rng(34)
    for cb in random_tables(rng, 6):
        tb = [int.from_bytes(bytes(np.array(cb, dtype=np.int8).view(np.uint8)[4 * i:4 * i + 4]), "little")
              for i in range(4)]
        for trial in range(30):
            pair = rng.integers(0, 256, 36, dtype=np.uint8).tobytes()
            w = list(struct.unpack("<9I", pair))
            c0, c1 = block_codes(pair[:18]), block_codes(pair[18:])
            for kmask in (63, 31):
                n = kmask + 1
                a = rng.integers(-(1 << 14), (1 << 14) + 1, n)
                if trial == 0:
                    a[:] = (1 << 14) * (1 if kmask == 63 else -1)  # the extremes
                A0, A1 = split_blocks(w, tb, digit_words8(a, kmask))
                assert A0 == sum(cb[c0[i]] * int(a[i & kmask]) for i in range(32))
                assert A1 == sum(cb[c1[i]] * int(a[(32 + i) & kmask]) for i in range(32))
