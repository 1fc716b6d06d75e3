"""Independent numpy formulations used to pin the oracle.

These are written from the format statement and the layer's definition as
whole-array operations (a dense-with-mask MoE, matrix products), a different
formulation from the oracle's per-expert loops, so that an indexing or
ordering mistake in one shows up against the other.
"""
import numpy as np


def half_bits_to_f64(h):
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


NL4 = 20  # non-linear 4-bit: the 4-bit layout, codes index a 16-entry int8 table
BLOCK_BYTES = {4: 18, 3: 14, NL4: 18}


def dequant_blocks(raw: np.ndarray, bits: int, codebook=None) -> np.ndarray:
    """raw uint8 [nblk * B] -> float64 [nblk, 32]."""
    B = BLOCK_BYTES[bits]
    blk = np.asarray(raw, dtype=np.uint8).reshape(-1, B)
    d = half_bits_to_f64(blk[:, 0].astype(np.uint16) | (blk[:, 1].astype(np.uint16) << 8))
    if bits == NL4:
        qs = blk[:, 2:18]
        codes = np.concatenate([qs & 0x0F, qs >> 4], axis=1).astype(np.int64)
        table = np.asarray(codebook, dtype=np.int8).astype(np.float64)
        return d[:, None] * table[codes]
    if bits == 4:
        qs = blk[:, 2:18]
        codes = np.concatenate([qs & 0x0F, qs >> 4], axis=1).astype(np.int64)
        bias = 8
    else:
        ql = blk[:, 2:10].astype(np.int64)
        qh = (blk[:, 10].astype(np.int64) | (blk[:, 11].astype(np.int64) << 8)
              | (blk[:, 12].astype(np.int64) << 16) | (blk[:, 13].astype(np.int64) << 24))
        i = np.arange(32)
        lo = (ql[:, i % 8] >> (2 * (i // 8))) & 3
        hi = (qh[:, None] >> i[None, :]) & 1
        codes = lo | (hi << 2)
        bias = 4
    return d[:, None] * (codes - bias).astype(np.float64)


def dequant_matrix(raw, bits, rows, cols, codebook=None):
    return dequant_blocks(raw, bits, codebook).reshape(rows, cols)


def dequant_expert(blob, bits, H, F, down_bits=None, codebook=None):
    """gate, up ([F,H], `bits`) and down ([H,F], `down_bits`, default `bits`)."""
    db = bits if down_bits is None else down_bits
    mg = H * (F // 32) * BLOCK_BYTES[bits]
    md = H * (F // 32) * BLOCK_BYTES[db]
    blob = np.asarray(blob, dtype=np.uint8)
    assert blob.size == 2 * mg + md
    return (dequant_matrix(blob[:mg], bits, F, H, codebook), dequant_matrix(blob[mg:2 * mg], bits, F, H, codebook),
            dequant_matrix(blob[2 * mg:], db, H, F, codebook))


def swiglu_mlp(X, Wg, Wu, Wd):
    """X [T,H] -> [T,H]: (silu(X Wg^T) * (X Wu^T)) Wd^T."""
    G = X @ Wg.T
    U = X @ Wu.T
    Hh = G / (1.0 + np.exp(-G)) * U
    return Hh @ Wd.T


def x_to_f64(x, x_code):
    return np.asarray(x, dtype=np.float64) if x_code == 0 else bf16_bits_to_f64(x)


def dense_masked_layer(x, x_code, logits, k, bits, H, F, routed, shared=None, s_bits=None, s_F=None,
                       down_bits=None, codebook=None):
    """Every expert on every row, weighted by a [T,E] mask that is the softmax
    of the k selected logits and zero elsewhere; plus the shared expert.
    bits: gate/up width, down_bits: down width (default bits), for the routed
    and the shared experts alike."""
    X = x_to_f64(x, x_code)
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    order = np.argsort(-L.astype(np.float64), axis=1, kind="stable")[:, :k]
    M = np.zeros((T, E))
    for t in range(T):
        sel = L[t, order[t]].astype(np.float64)
        ex = np.exp(sel - sel.max())
        M[t, order[t]] = ex / ex.sum()
    db = bits if down_bits is None else down_bits
    eb = H * (F // 32) * (2 * BLOCK_BYTES[bits] + BLOCK_BYTES[db])
    Y = np.zeros((T, H))
    for e in range(E):
        if not M[:, e].any():
            continue
        Wg, Wu, Wd = dequant_expert(routed[e * eb:(e + 1) * eb], bits, H, F, db, codebook)
        Y += M[:, e:e + 1] * swiglu_mlp(X, Wg, Wu, Wd)
    if shared is not None:
        sb = bits if s_bits is None else s_bits
        sF = F if s_F is None else s_F
        Wg, Wu, Wd = dequant_expert(shared, sb, H, sF, db, codebook)
        Y += swiglu_mlp(X, Wg, Wu, Wd)
    return Y, order.astype(np.int32), M
