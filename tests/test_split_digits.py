"""CPU check of the column-split decode launch's integer dot-product scheme.

The launch (csrc/moe_split.hip) multiplies weight bytes, read as 32-bit words
of eight nibbles, by words of signed radix-16 activation digits with
v_dot8_i32_i4.  This test models those layouts in Python -- which k each
nibble of each word multiplies, how the digits are cut, how a 3-bit code is
assembled as one nibble from its low bits and its third bit (with the -4a
term taken from the block's sum of a) -- and checks that the sums
are the exact integer dot products sum (code - bias) * a of each block, for
both formats, for a pair of blocks of one row (gate/up) and for the same
block of two rows (down), including the extreme activations +-2^14.  A wrong
nibble order, digit, mask or shift in the model fails it; the kernel's own
results are checked against the oracle by the GPU tests.
"""
import numpy as np
import pytest


def nibble_k(bits, nd, i):
    h = i & 1
    if bits == 4:
        beta = 4 * nd + (i >> 1)
        if 2 <= beta <= 17:
            return beta - 2 + 16 * h
        if 20 <= beta <= 35:
            return 32 + beta - 20 + 16 * h
        return -1
    # 3-bit: nibble-dword 4B + m holds codes 8 (m & 1) + 4 (m >> 1) + j (+16 in
    # the high nibble) of block B, byte j
    B, m = nd >> 2, nd & 3
    return 32 * B + 8 * (m & 1) + 4 * (m >> 1) + (i >> 1) + 16 * h


def digit_words(bits, a, kmask):
    """The digit words of one pair, [digit][word]."""
    nnd = 9 if bits == 4 else 8
    out = [0] * (4 * nnd)
    for nd in range(nnd):
        D = [0] * 4
        for i in range(8):
            kk = nibble_k(bits, nd, i)
            v = int(a[kk & kmask]) if kk >= 0 else 0
            u = v + 0x8888
            assert 0 <= u < (1 << 16)
            for j in range(4):
                D[j] |= ((u >> (4 * j)) & 15) << (4 * i)
        for j in range(4):
            out[j * nnd + nd] = D[j] ^ 0x88888888
    return out


def sdot8(a, b, c):
    for i in range(8):
        x, y = (a >> 4 * i) & 15, (b >> 4 * i) & 15
        c += (x - 16 if x >= 8 else x) * (y - 16 if y >= 8 else y)
    return c


def radix16(acc):
    v = acc[-1]
    for j in range(len(acc) - 2, -1, -1):
        v = (v << 4) + acc[j]
    return v


def words(b):
    return [int.from_bytes(bytes(b[4 * i:4 * i + 4]), "little") for i in range(len(b) // 4)]


def block_sums(bits, pair_bytes, xd, S0, S1):
    w = words(pair_bytes)
    if bits == 4:
        wx = [x ^ 0x88888888 for x in w]
        a0, a1 = [0] * 4, [0] * 4
        for j in range(4):
            for q in range(5):
                a0[j] = sdot8(wx[q], xd[j * 9 + q], a0[j])
            for q in range(5, 9):
                a1[j] = sdot8(wx[q], xd[j * 9 + q], a1[j])
        return radix16(a0), radix16(a1)
    align = lambda hi, lo: (((hi << 32) | lo) >> 16) & 0xFFFFFFFF
    L = [[align(w[1], w[0]), align(w[2], w[1])], [w[4], w[5]]]
    Q = [align(w[3], w[2]), w[6]]
    spread = lambda t: ((t & 0xFFFFFF) * 0x810204) & 0x04040404
    C = []
    for B in range(2):
        for m in range(4):
            c0 = 8 * (m & 1) + 4 * (m >> 1)
            n = ((L[B][m >> 1] >> 2) if m & 1 else L[B][m >> 1]) & 0x33333333
            C.append(n | spread((Q[B] >> c0) & 15) | (spread((Q[B] >> (c0 + 16)) & 15) << 4))
    a0, a1 = [-4 * S0, 0, 0, 0], [-4 * S1, 0, 0, 0]
    for j in range(4):
        for q in range(4):
            a0[j] = sdot8(C[q], xd[j * 8 + q], a0[j])
        for q in range(4, 8):
            a1[j] = sdot8(C[q], xd[j * 8 + q], a1[j])
    return radix16(a0), radix16(a1)


def block_bytes(bits, codes, scale_bits):
    b = [scale_bits & 255, scale_bits >> 8]
    if bits == 4:
        return b + [int(codes[i] | (codes[i + 16] << 4)) for i in range(16)]
    for i in range(8):
        b.append(sum((int(codes[i + 8 * f]) & 3) << (2 * f) for f in range(4)))
    hb = sum(((int(codes[i]) >> 2) & 1) << i for i in range(32))
    return b + list(hb.to_bytes(4, "little"))


@pytest.mark.parametrize("bits", [4, 3])
def test_nibble_dot_products_are_exact(bits):
    rng = np.random.default_rng(7)
    bias = 8 if bits == 4 else 4
    for trial in range(60):
        codes = rng.integers(0, 2 ** bits, size=(2, 32))
        pb = block_bytes(bits, codes[0], 0x3A5C) + block_bytes(bits, codes[1], 0x2B11)
        a = rng.integers(-16384, 16385, size=64)
        if trial % 5 == 0:
            a = rng.choice([-16384, 16384], size=64)
        # gate/up: two blocks of one row, 64 distinct activations
        got = block_sums(bits, pb, digit_words(bits, a, 63), int(a[:32].sum()), int(a[32:].sum()))
        assert got == (int(np.dot(codes[0] - bias, a[:32])), int(np.dot(codes[1] - bias, a[32:])))
        # down: the same block of two rows, one slice of 32 activations
        h = a[:32]
        got = block_sums(bits, pb, digit_words(bits, h, 31), int(h.sum()), int(h.sum()))
        assert got == (int(np.dot(codes[0] - bias, h)), int(np.dot(codes[1] - bias, h)))
