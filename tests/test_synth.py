"""The torch encoder (used by the benchmark to build 48 layers of weights on
the device) writes the same bytes as the numpy encoder the oracle's pins
check, for the same weights (CPU only)."""
import numpy as np
import pytest
import torch

from quantized_routed_expert_amd import synth


@pytest.mark.parametrize("bits", [3, 4, synth.BITS_NL4])
def test_quantize_torch_matches_numpy(bits):
    rg = np.random.default_rng(5 + bits)
    w = (rg.standard_normal((96, 512)) * 0.02).astype(np.float32)
    w[3, :32] = 0.0                 # an all-zero block: d = 0, every code the bias
    w[5, 32:64] *= np.float32(1e-30)  # a block whose fp16 scale underflows to 0
    w[7, 5] = np.float32(0.9)       # one large weight dominating its block
    w[9, 64:96] = np.float32(-0.0)
    w[11, 96:128] = np.linspace(-1, 1, 32, dtype=np.float32)  # codes at .5 boundaries
    cb = synth.nl4_test_codebook() if bits == synth.BITS_NL4 else None
    a = synth.quantize(w, bits, cb)
    b = synth.quantize_torch(torch.from_numpy(w), bits, cb).numpy()
    assert np.array_equal(a, b)


def test_nl4_quantizer_picks_nearest():
    """The non-linear encoder picks a table entry nearest w / d for every
    weight (brute force over the 16 entries), for an ordered and an
    unordered table."""
    rg = np.random.default_rng(8)
    w = (rg.standard_normal((16, 256)) * 0.02).astype(np.float32)
    for cb in (synth.nl4_test_codebook(), tuple(((c * 37 + 11) % 256) - 128 for c in range(16))):
        raw = synth.quantize(w, synth.BITS_NL4, cb).reshape(-1, 18)
        d = raw[:, :2].copy().view(np.float16).astype(np.float32).ravel()
        codes = np.concatenate([raw[:, 2:] & 15, raw[:, 2:] >> 4], axis=1)
        v = w.reshape(-1, 32) / d[:, None]
        table = np.array(cb, dtype=np.float32)
        best = np.abs(v[:, :, None] - table[None, None, :]).min(axis=2)
        assert np.allclose(np.abs(v - table[codes]), best, rtol=0, atol=1e-4)


def test_routed_weights_torch_layout():
    """Expert blobs of the device generator: the right size, gate|up|down of
    N(0, 0.02) weights (scale bytes of plausible magnitude), independent per
    layer and reproducible per seed."""
    cfg = synth.scaled_config(synth.CONFIGS["e512"], name="gen", n_experts=5, hidden=256, ffn=256)
    a = synth.routed_weights_torch(cfg, 0, "cpu", chunk=2).numpy()
    b = synth.routed_weights_torch(cfg, 0, "cpu", chunk=3).numpy()
    c = synth.routed_weights_torch(cfg, 1, "cpu").numpy()
    assert a.size == cfg.n_experts * cfg.expert_bytes
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    d = a.reshape(-1, cfg.block_bytes)[:, :2].copy().view(np.float16).astype(np.float64).ravel()
    # absmax of 32 N(0, 0.02) draws over qmax = 3: around 0.015
    assert 0.008 < np.median(d) < 0.025
