"""CPU check of the column-split decode launch's integer dot-product scheme.

The launch (csrc/moe_split.hip) multiplies weight bytes, read as 32-bit words
of eight nibbles, by words of signed radix-16 activation digits with
v_dot8_i32_i4.  This test models those layouts in Python -- which k each
nibble of each word multiplies, how the digits are cut, how 3-bit codes are
split into their low bits and their third bit -- and checks that the sums
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
    if nd < 10:
        w = nd >> 1
        beta = 4 * w + (4 if w >= 3 else 0) + (i >> 1)
        if 2 <= beta <= 9:
            B, j = 0, beta - 2
        elif 16 <= beta <= 23:
            B, j = 1, beta - 16
        else:
            return -1
        f = (3 if h else 1) if (nd & 1) else (2 if h else 0)
        return 32 * B + j + 8 * f
    u = nd - 10
    return 32 * (u >> 2) + 4 * i + (u & 3)


def digit_words(bits, a, kmask):
    """The digit words of one pair: 4-bit [digit][word]; 3-bit [low word][digit] then [third word][digit]."""
    nnd = 9 if bits == 4 else 18
    out = [0] * (36 if bits == 4 else 80)
    for nd in range(nnd):
        third = bits == 3 and nd >= 10
        D = [0] * 5
        for i in range(8):
            kk = nibble_k(bits, nd, i)
            v = int(a[kk & kmask]) if kk >= 0 else 0
            u = 4 * v + 0x88888 if third else v + 0x8888
            assert 0 <= u < (1 << 20)
            for j in range(5):
                D[j] |= ((u >> (4 * j)) & 15) << (4 * i)
        D = [d ^ 0x88888888 for d in D]
        if bits == 4:
            for j in range(4):
                out[j * 9 + nd] = D[j]
        elif not third:
            for j in range(4):
                out[nd * 4 + j] = D[j]
        else:
            for j in range(5):
                out[40 + (nd - 10) * 5 + j] = D[j]
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
    lw = [w[0], w[1], w[2], w[4], w[5]]
    N = []
    for x in lw:
        N += [x & 0x33333333, (x >> 2) & 0x33333333]
    h0 = (((w[3] << 32) | w[2]) >> 16) & 0xFFFFFFFF
    M = [(h0 >> s) & 0x11111111 for s in range(4)] + [(w[6] >> s) & 0x11111111 for s in range(4)]
    a0, a1 = [-4 * S0, 0, 0, 0, 0], [-4 * S1, 0, 0, 0, 0]
    for j in range(5):
        if j < 4:
            for nd in range(6):
                a0[j] = sdot8(N[nd], xd[nd * 4 + j], a0[j])
            for nd in range(6, 10):
                a1[j] = sdot8(N[nd], xd[nd * 4 + j], a1[j])
        for u in range(4):
            a0[j] = sdot8(M[u], xd[40 + u * 5 + j], a0[j])
        for u in range(4, 8):
            a1[j] = sdot8(M[u], xd[40 + u * 5 + j], a1[j])
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
