"""Seeded synthetic inputs for the routed-expert MoE layer.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds the workload recipes (shapes, value distributions, routing skew) and
the encoder that packs Gaussian weights into the quantized block layout; it
holds none of the layer's own arithmetic (no routing, grouping, dequant, FFN
or combine).  Every random draw comes from
``numpy.random.default_rng(SeedSequence([config_id, layer, tensor_id, base_seed, ...]))``
so layers and tensors are independent and reproducible.

Block layout (the decoder side is written independently in the oracle and in
the HIP kernels):
  * 4-bit, 18 bytes per 32 weights: fp16 scale d (little-endian), then 16
    bytes; byte i holds code i in its low nibble and code i+16 in its high
    nibble; weight = d * (code - 8).
  * 3-bit, 14 bytes per 32 weights: fp16 scale d, 8 bytes of 2-bit low parts
    (code i's low two bits at bit 2*(i//8) of byte i%8), then a 32-bit
    little-endian word whose bit i is code i's third bit; weight = d*(code-4).
  * non-linear 4-bit (format code 20), 18 bytes: the 4-bit layout, weight =
    d * codebook[code] with a 16-entry table of signed 8-bit values (the
    pages name the format but print no table; the table is an input).
  * A matrix [rows][cols] is stored row by row, cols/32 blocks per row; an
    expert is gate [F][H] | up [F][H] | down [H][F]; experts back to back.
    Gate and up share one bit width, down may have another (``down_bits``).

The 4-bit block of 32 values in 18 bytes is the one the forum thread "把
Strata 搬上 SGLang 引擎 的嘗試" names in §四; the nibble order and the whole
3-bit layout are readings of points the pages leave open.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TID_X, TID_LOGITS, TID_ROUTED, TID_SHARED, TID_PERM, TID_ROUTER = 0, 1, 2, 3, 4, 5
BITS_NL4 = 20  # the non-linear 4-bit format's code


def nl4_test_codebook() -> tuple:
    """A non-linear, monotone table of 16 signed 8-bit values for the tests:
    127 * sign(t) * |t|^1.6 at t = (i - 7.5) / 7.5, rounded."""
    t = (np.arange(16) - 7.5) / 7.5
    return tuple(int(v) for v in np.rint(127.0 * np.sign(t) * np.abs(t) ** 1.6))


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload: the MoE layer's shapes and input recipe."""
    name: str
    cid: int            # seed namespace
    hidden: int
    n_experts: int
    ffn: int
    top_k: int
    shared_ffn: int     # 0 = no shared expert
    rows: tuple         # tokens per window/chunk
    bits: int
    x_dtype: str        # "f32" or "bf16"
    logits: tuple       # ("normal", sigma) or ("zipf", s)
    layers: int
    weight_cid: int = 0  # seed namespace of the weights (0 = cid)
    down_bits: int = 0   # bit width of the down projection (0 = bits, the gate/up width)
    codebook: tuple = ()  # the non-linear 4-bit format's 16 values (when a width is 20)

    @property
    def wcid(self) -> int:
        return self.weight_cid or self.cid

    @property
    def dbits(self) -> int:
        return self.down_bits or self.bits

    @property
    def fmt(self) -> int:
        """Format code: gate/up bits in the low byte, down bits in the next (0 = the same)."""
        return format_code(self.bits, self.down_bits)

    @property
    def block_bytes(self) -> int:
        return block_bytes(self.bits)

    @property
    def expert_bytes(self) -> int:
        return expert_bytes(self.bits, self.hidden, self.ffn, self.down_bits)

    @property
    def shared_bytes(self) -> int:
        return expert_bytes(self.bits, self.hidden, self.shared_ffn, self.down_bits) if self.shared_ffn else 0


CONFIGS = {
    # tiny correctness layer: fp32 activations, 4-bit weights
    "tiny": Config("tiny", 1, 256, 8, 512, 2, 512, (4,), 4, "f32", ("normal", 1.0), 1),
    # one decode slot, 128 experts, 4-bit
    "decode": Config("decode", 2, 2048, 128, 768, 8, 768, (1,), 4, "bf16", ("normal", 2.0), 48),
    # 8 slots x (token + proposal) = 16 rows, Zipf(1.1) routing, 3-bit
    "mtp16": Config("mtp16", 3, 2048, 128, 768, 8, 768, (16,), 3, "bf16", ("zipf", 1.1), 48),
    # 512 experts, top-10, 3-bit, 1 and 4 rows per window
    "e512": Config("e512", 4, 2048, 512, 512, 10, 512, (1, 4), 3, "bf16", ("normal", 2.0), 48),
    # a 2048-token prefill chunk over the same layer (same weights as e512)
    "prefill": Config("prefill", 5, 2048, 512, 512, 10, 512, (2048,), 3, "bf16", ("zipf", 1.1), 48,
                      weight_cid=4),
}


def block_bytes(bits: int) -> int:
    return {4: 18, 3: 14, BITS_NL4: 18}[bits]


def format_code(bits: int, down_bits: int = 0) -> int:
    return bits | ((down_bits if down_bits and down_bits != bits else 0) << 8)


def expert_bytes(bits: int, hidden: int, ffn: int, down_bits: int = 0) -> int:
    return hidden * (ffn // 32) * (2 * block_bytes(bits) + block_bytes(down_bits or bits))


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


# --------------------------------------------------------------------------
# scalar encodings
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# weight encoder (symmetric absmax, fp16 scale)
# --------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, d16: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes [nblk, 32] (0..2^bits-1) and fp16 scales [nblk] into
    nblk consecutive blocks; returns uint8 [nblk * block_bytes]."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, 32)
    nblk = codes.shape[0]
    d16 = np.ascontiguousarray(np.asarray(d16, dtype=np.float16).reshape(nblk))
    out = np.empty((nblk, block_bytes(bits)), dtype=np.uint8)
    out[:, 0:2] = d16.view(np.uint8).reshape(nblk, 2)
    if bits in (4, BITS_NL4):
        out[:, 2:18] = (codes[:, :16] & 0x0F) | ((codes[:, 16:] & 0x0F) << 4)
    elif bits == 3:
        lo = codes & 3
        ql = np.zeros((nblk, 8), dtype=np.uint8)
        for f in range(4):
            ql |= lo[:, 8 * f:8 * f + 8] << (2 * f)
        out[:, 2:10] = ql
        # little-endian bit order: bit i of the 32-bit word = third bit of code i
        out[:, 10:14] = np.packbits((codes >> 2) & 1, axis=1, bitorder="little")
    else:
        raise ValueError(bits)
    return out.reshape(-1)


def quantize(w: np.ndarray, bits: int, codebook=None) -> np.ndarray:
    """Quantize a [rows, cols] float32 matrix along its rows in blocks of 32:
    d = fp16(absmax / qmax), code = clip(rint(w / d), -qmax, qmax) + 2^(bits-1)
    with qmax = 2^(bits-1) - 1 (all codes = bias when the block is zero).
    Non-linear 4-bit: d = fp16(absmax / max|codebook|), code = the entry
    nearest w / d (on a tie the smaller value; among equal values the lower
    code)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    if bits == BITS_NL4:
        cb = np.asarray(codebook, dtype=np.float32).reshape(16)
        order = np.argsort(cb, kind="stable")
        srt = cb[order]
        mids = (srt[1:] + srt[:-1]) * np.float32(0.5)  # boundaries between neighbouring values
        blk = w.reshape(-1, 32)
        amax = np.abs(blk).max(axis=1)
        d16 = (amax / np.float32(np.abs(cb).max())).astype(np.float16)
        d32 = d16.astype(np.float32)
        safe = np.where(d32 > 0, d32, np.float32(1.0))
        codes = order[np.searchsorted(mids, blk / safe[:, None], side="left")].astype(np.uint8)
        return pack_codes(codes, d16, bits)
    qmax = (1 << (bits - 1)) - 1
    bias = 1 << (bits - 1)
    blk = w.reshape(-1, 32)
    amax = np.abs(blk).max(axis=1)
    d16 = (amax / np.float32(qmax)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 > 0, d32, np.float32(1.0))
    q = np.rint(blk / safe[:, None])
    np.clip(q, -qmax, qmax, out=q)
    q[d32 == 0] = 0
    codes = (q + bias).astype(np.uint8)
    return pack_codes(codes, d16, bits)


def quantize_torch(w, bits: int, codebook=None):
    """The encoder of ``quantize`` in torch, on w's device (any device): the
    same steps in the same fp32/fp16 arithmetic, so the same bytes for the
    same w.  w: float32 tensor [..., cols] (cols % 32 == 0) -> uint8 tensor
    [nblk * block_bytes], blocks in row-major order."""
    import torch
    w = w.contiguous().to(torch.float32)
    if bits == BITS_NL4:
        cb = torch.tensor(codebook, dtype=torch.float32, device=w.device).reshape(16)
        srt, order = torch.sort(cb, stable=True)
        mids = (srt[1:] + srt[:-1]) * 0.5
        blk = w.reshape(-1, 32)
        nblk = blk.shape[0]
        amax = blk.abs().amax(dim=1)
        d16 = (amax / cb.abs().max()).to(torch.float16)
        d32 = d16.to(torch.float32)
        safe = torch.where(d32 > 0, d32, torch.ones_like(d32))
        codes = order[torch.searchsorted(mids, (blk / safe[:, None]).contiguous(), right=False)].to(torch.uint8)
        out = torch.empty((nblk, 18), dtype=torch.uint8, device=w.device)
        dv = d16.view(torch.int16).to(torch.int32)
        out[:, 0] = (dv & 0xFF).to(torch.uint8)
        out[:, 1] = ((dv >> 8) & 0xFF).to(torch.uint8)
        out[:, 2:18] = (codes[:, :16] & 0x0F) | ((codes[:, 16:] & 0x0F) << 4)
        return out.reshape(-1)
    if bits not in (3, 4):
        raise ValueError(bits)
    qmax = (1 << (bits - 1)) - 1
    bias = 1 << (bits - 1)
    blk = w.reshape(-1, 32)
    nblk = blk.shape[0]
    amax = blk.abs().amax(dim=1)
    d16 = (amax / torch.tensor(float(qmax), dtype=torch.float32, device=w.device)).to(torch.float16)
    d32 = d16.to(torch.float32)
    safe = torch.where(d32 > 0, d32, torch.ones_like(d32))
    q = torch.round(blk / safe[:, None])  # round half to even, as np.rint
    q.clamp_(-qmax, qmax)
    q[d32 == 0] = 0
    codes = (q + bias).to(torch.uint8)
    out = torch.empty((nblk, block_bytes(bits)), dtype=torch.uint8, device=w.device)
    dv = d16.view(torch.int16).to(torch.int32)
    out[:, 0] = (dv & 0xFF).to(torch.uint8)
    out[:, 1] = ((dv >> 8) & 0xFF).to(torch.uint8)
    if bits == 4:
        out[:, 2:18] = (codes[:, :16] & 0x0F) | ((codes[:, 16:] & 0x0F) << 4)
    elif bits == 3:
        lo = codes & 3
        ql = torch.zeros((nblk, 8), dtype=torch.uint8, device=w.device)
        for f in range(4):
            ql |= lo[:, 8 * f:8 * f + 8] << (2 * f)
        out[:, 2:10] = ql
        hb = ((codes >> 2) & 1).to(torch.int64)
        word = (hb << torch.arange(32, device=w.device, dtype=torch.int64)).sum(dim=1)
        for j in range(4):
            out[:, 10 + j] = ((word >> (8 * j)) & 0xFF).to(torch.uint8)
    else:
        raise ValueError(bits)
    return out.reshape(-1)


def _torch_seed(*key: int) -> int:
    return int(np.random.SeedSequence([int(k) for k in key]).generate_state(1, dtype=np.uint64)[0] >> 1)


def routed_weights_torch(cfg: Config, layer: int, device, base_seed: int = 0, chunk: int = 32,
                         std: float = 0.02):
    """All routed experts of one layer generated and quantized on `device`
    (the benchmark's fast path for 48 layers of hundreds of experts): the
    same recipe as ``routed_weights`` (N(0, std) gate, up, down per expert,
    quantized per block of 32), drawn from torch's generator seeded per
    (config, layer, expert, base_seed), so other values than the numpy
    generator gives.  Returns a uint8 tensor [E * expert_bytes] on `device`."""
    import torch
    H, F, E, bits = cfg.hidden, cfg.ffn, cfg.n_experts, cfg.bits
    eb = cfg.expert_bytes
    mb = H * (F // 32) * block_bytes(bits)  # bytes of the gate (and the up) matrix
    out = torch.empty(E * eb, dtype=torch.uint8, device=device)
    cb = cfg.codebook or None
    gen = torch.Generator(device=device)
    for e0 in range(0, E, chunk):
        n = min(chunk, E - e0)
        gu = torch.empty((n, 2, F, H), device=device, dtype=torch.float32)
        dn = torch.empty((n, H, F), device=device, dtype=torch.float32)
        for i in range(n):
            gen.manual_seed(_torch_seed(cfg.wcid, layer, TID_ROUTED, base_seed, e0 + i, 1))
            gu[i].normal_(0.0, std, generator=gen)
            dn[i].normal_(0.0, std, generator=gen)
        view = out[e0 * eb:(e0 + n) * eb].view(n, eb)
        view[:, :2 * mb] = quantize_torch(gu, bits, cb).view(n, 2 * mb)
        view[:, 2 * mb:] = quantize_torch(dn, cfg.dbits, cb).view(n, eb - 2 * mb)
        del gu, dn
    return out


def expert_blob(rg: np.random.Generator, hidden: int, ffn: int, bits: int, std: float = 0.02,
                down_bits: int = 0, codebook=None) -> np.ndarray:
    """One expert: N(0, std) gate [F,H], up [F,H] (bits), down [H,F]
    (down_bits, 0 = bits), quantized (codebook: the non-linear format's table)."""
    g = rg.standard_normal((ffn, hidden), dtype=np.float32) * np.float32(std)
    u = rg.standard_normal((ffn, hidden), dtype=np.float32) * np.float32(std)
    d = rg.standard_normal((hidden, ffn), dtype=np.float32) * np.float32(std)
    return np.concatenate([quantize(g, bits, codebook), quantize(u, bits, codebook),
                           quantize(d, down_bits or bits, codebook)])


def _threads(n: int | None) -> int:
    if n:
        return n
    return max(1, min(16, os.cpu_count() or 1))


def routed_weights(cfg: Config, layer: int, base_seed: int = 0, threads: int | None = None,
                   out: np.ndarray | None = None) -> np.ndarray:
    """All routed experts of one layer, back to back: uint8 [E * expert_bytes]."""
    eb = cfg.expert_bytes
    buf = out if out is not None else np.empty(cfg.n_experts * eb, dtype=np.uint8)

    def one(e):
        buf[e * eb:(e + 1) * eb] = expert_blob(rng(cfg.wcid, layer, TID_ROUTED, base_seed, e),
                                               cfg.hidden, cfg.ffn, cfg.bits, down_bits=cfg.down_bits,
                                               codebook=cfg.codebook or None)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(one, range(cfg.n_experts)))
    return buf


def shared_weights(cfg: Config, layer: int, base_seed: int = 0) -> np.ndarray | None:
    if not cfg.shared_ffn:
        return None
    return expert_blob(rng(cfg.wcid, layer, TID_SHARED, base_seed), cfg.hidden, cfg.shared_ffn, cfg.bits,
                       down_bits=cfg.down_bits, codebook=cfg.codebook or None)


# --------------------------------------------------------------------------
# activations and router logits
# --------------------------------------------------------------------------

def activations(cfg: Config, layer: int, T: int, base_seed: int = 0) -> np.ndarray:
    """x [T, H]: float32 N(0,1), or its bf16 rounding as uint16 bit patterns."""
    x = rng(cfg.cid, layer, TID_X, base_seed, T).standard_normal((T, cfg.hidden), dtype=np.float32)
    if cfg.x_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def logits(cfg: Config, layer: int, T: int, base_seed: int = 0) -> np.ndarray:
    """Router logits [T, E] float32.

    ("normal", s): i.i.d. N(0, s).  ("zipf", a): expert popularity p_r ∝ r^-a
    over a seeded per-layer permutation of expert ids, logits = log p + Gumbel(0,1)
    i.i.d., so that top-k draws k distinct experts with probability ∝ p
    (Gumbel-top-k) and rows share the popular experts."""
    kind, par = cfg.logits
    rg = rng(cfg.cid, layer, TID_LOGITS, base_seed, T)
    E = cfg.n_experts
    if kind == "normal":
        return (rg.standard_normal((T, E)) * par).astype(np.float32)
    if kind == "zipf":
        perm = rng(cfg.cid, layer, TID_PERM, base_seed).permutation(E)
        ranks = np.arange(1, E + 1, dtype=np.float64)
        p = ranks ** (-float(par))
        p /= p.sum()
        logp = np.empty(E, dtype=np.float64)
        logp[perm] = np.log(p)
        return (logp[None, :] + rg.gumbel(size=(T, E))).astype(np.float32)
    raise ValueError(kind)


def router_weights(cfg: Config, layer: int, base_seed: int = 0) -> np.ndarray:
    """The router matrix W [E, H] as bf16 bit patterns (uint16): i.i.d.
    N(0, s / sqrt(H)) with s the logit scale of the recipe (the "normal"
    sigma, or 1), so that x W^T for x ~ N(0,1) has about the recipe's
    logit spread."""
    kind, par = cfg.logits
    s = float(par) if kind == "normal" else 1.0
    w = rng(cfg.cid, layer, TID_ROUTER, base_seed).standard_normal((cfg.n_experts, cfg.hidden))
    return f32_to_bf16_bits((w * (s / np.sqrt(cfg.hidden))).astype(np.float32))


@dataclasses.dataclass
class LayerInputs:
    cfg: Config
    layer: int
    T: int
    x: np.ndarray          # [T,H] float32 or uint16 (bf16 bits)
    logits: np.ndarray     # [T,E] float32
    routed: np.ndarray     # uint8 [E * expert_bytes]
    shared: np.ndarray | None

    @property
    def x_code(self) -> int:
        return 0 if self.cfg.x_dtype == "f32" else 1


def layer_inputs(cfg: Config, layer: int = 0, T: int | None = None, base_seed: int = 0,
                 threads: int | None = None) -> LayerInputs:
    T = cfg.rows[0] if T is None else T
    return LayerInputs(cfg, layer, T, activations(cfg, layer, T, base_seed),
                       logits(cfg, layer, T, base_seed),
                       routed_weights(cfg, layer, base_seed, threads),
                       shared_weights(cfg, layer, base_seed))


def scaled_config(cfg: Config, name: str | None = None, **changes) -> Config:
    """A reduced copy of a workload (same recipe, other sizes), for tests the
    oracle must finish in seconds."""
    return dataclasses.replace(cfg, name=name or (cfg.name + "_scaled"), **changes)
