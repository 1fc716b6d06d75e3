"""CPU model of the 3-bit operand path of the matrix-core decode launch (no GPU).

A lane of k-group g feeds the weights 8g .. 8g+7 of a block.  It assembles
their eight codes one per byte (a shift and mask of the low-part bytes; the
third bits spread to bit 2 of each byte by one 24-bit multiply), looks each
up in a byte table of the high bytes of fp16(code - 4) (v_perm_b32: selector
byte k < 4 picks byte k of the second source, 4..7 byte k-4 of the first, 12
the constant zero), and interleaves them with zero low bytes.  This models
those integer steps bit for bit and checks them against the block format's
own definition (the weight = code minus 4, as an exact fp16), for both blocks
of a gate/up pair (dword realignment of the first block, the aligned second
one) and for a down block at an even and at an odd row of a column block
(rows 14 bytes apart, read as five dwords from the one at or below the
block's start)."""
import struct

import numpy as np

from test_prefill_dequant import alignbit, perm


def fp16_bits(x):
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def mul24(a, b):
    return ((a & 0xFFFFFF) * (b & 0xFFFFFF)) & 0xFFFFFFFF


def unpack3(qs0, qs1, qh, g):
    """The eight fp16 bit patterns a lane of k-group g feeds, in slot order."""
    l0 = (qs0 >> (2 * g)) & 0x03030303
    l1 = (qs1 >> (2 * g)) & 0x03030303
    t0 = (qh >> (8 * g)) & 15
    t1 = (qh >> (8 * g + 4)) & 15
    c0 = (mul24(t0, 0x810204) & 0x04040404) | l0
    c1 = (mul24(t1, 0x810204) & 0x04040404) | l1
    h0 = perm(0x42403C00, 0xBCC0C2C4, c0)
    h1 = perm(0x42403C00, 0xBCC0C2C4, c1)
    words = [perm(h0, h0, 0x050C040C), perm(h0, h0, 0x070C060C), perm(h1, h1, 0x050C040C), perm(h1, h1, 0x070C060C)]
    return [(w >> (16 * k)) & 0xFFFF for w in words for k in range(2)]


def reference(block):
    """fp16(code - 4) of weights 0..31 of a 14-byte block, from the format."""
    qs, qh = block[2:10], int.from_bytes(block[10:14], "little")
    codes = [((qs[i & 7] >> (2 * (i >> 3))) & 3) | (((qh >> i) & 1) << 2) for i in range(32)]
    return [fp16_bits(c - 4) for c in codes]


def test_table_is_fp16_of_code_minus_4():
    # the table's bytes are the high bytes of fp16(c - 4), whose low bytes are zero
    for c in range(8):
        bits = fp16_bits(c - 4)
        assert bits & 0xFF == 0
        table = (0x42403C00 << 32) | 0xBCC0C2C4
        assert (table >> (8 * c)) & 0xFF == bits >> 8


def test_gate_up_pair():
    rng = np.random.default_rng(21)
    for _ in range(500):
        pair = rng.integers(0, 256, 28, dtype=np.uint8).tobytes()
        w = list(struct.unpack("<7I", pair))
        # block 0: bytes 0..13 (fields two bytes into a dword); block 1: 14..27 (aligned fields)
        fields = [
            (w[0] & 0xFFFF, alignbit(w[1], w[0], 16), alignbit(w[2], w[1], 16), alignbit(w[3], w[2], 16)),
            (w[3] >> 16, w[4], w[5], w[6]),
        ]
        for blk in range(2):
            b = pair[14 * blk:14 * blk + 14]
            d, qs0, qs1, qh = fields[blk]
            assert d == int.from_bytes(b[0:2], "little")
            got = sum((unpack3(qs0, qs1, qh, g) for g in range(4)), [])
            assert got == reference(b)


def test_down_block_both_parities():
    rng = np.random.default_rng(22)
    for _ in range(300):
        buf = rng.integers(0, 256, 64, dtype=np.uint8).tobytes()
        for n in range(2):  # row parity
            a0 = 16 + 14 * n  # the block's first byte (4-aligned for even rows, 2 past for odd ones)
            rd = lambda o: int.from_bytes(buf[o:o + 4], "little")
            q = a0 + 2
            qa, sh = q & ~3, q & 3
            base = a0 & ~3
            dw, r0, r1, r2, r3 = rd(base), rd(qa), rd(qa + 4), rd(qa + 8), rd(base + 12)
            assert (dw >> (16 * n)) & 0xFFFF == int.from_bytes(buf[a0:a0 + 2], "little")
            got = sum((unpack3(alignbit(r1, r0, 8 * sh), alignbit(r2, r1, 8 * sh), alignbit(r3, r2, 8 * sh), g)
                       for g in range(4)), [])
            assert got == reference(buf[a0:a0 + 14])
            # an odd row's reads end with its block; an even row's reach two bytes
            # into the next row (an even row is never a column block's last)
            assert max(qa + 12, base + 16) <= a0 + 14 + (2 if n == 0 else 0)
