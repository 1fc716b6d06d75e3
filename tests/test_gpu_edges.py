"""Edge cases through the C ABI against the oracle (GPU): decode with more
experts than the fused router takes, activations of extreme magnitude, the
routing heat counters and the device error word.

Bar: routing bit-exact; outputs within max |err| <= 2e-3 * rms(oracle),
plus fp32's smallest normal magnitude (2^-126) where the oracle's values
fall below fp32's normal range."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL, DevLayer, oracle_forward, rel_err
from quantized_routed_expert_amd import moe, synth

pytestmark = pytest.mark.gpu

D, P = moe.PATH_DECODE, moe.PATH_PREFILL
FP32_TINY = 2.0 ** -126


def _cfg(base, **kw):
    return synth.scaled_config(synth.CONFIGS[base], **kw)


def _check(orc, li, path, abs_floor=0.0):
    y, idx, w = DevLayer(li).forward(path)
    yr, ir, wr = oracle_forward(orc, li)
    assert np.array_equal(idx, ir), "routing differs"
    assert np.all(np.isfinite(y))
    rms = float(np.sqrt(np.mean(yr ** 2)))
    err = float(np.max(np.abs(y.astype(np.float64) - yr)))
    print(f"    max|err| {err:.3e}  rms {rms:.3e}", flush=True)
    assert err <= TOL * rms + abs_floor, (err, rms)


# ---- decode with E > 1024: router and grouping launches, then the decode launch ----

@pytest.mark.parametrize("T", [1, 8])
@pytest.mark.parametrize("bits", [3, 4])
def test_decode_many_experts(orc, T, bits):
    """More experts than the fused routing takes (1500 > 1024): the layer runs
    k_route + the grouping launches + the decode launch on the given grouping
    (split launch for T = 1, matrix-core launch for T = 8)."""
    print(f"[edges] decode E=1500 T={T} bits={bits}", flush=True)
    cfg = _cfg("e512", name=f"e1500_{bits}", n_experts=1500, hidden=1024, ffn=256, shared_ffn=256, top_k=8,
               bits=bits)
    li = synth.layer_inputs(cfg, T=T, threads=4)
    _check(orc, li, D)


# ---- activations of extreme magnitude ------------------------------------------

@pytest.mark.parametrize("T,path", [(1, D), (3, D), (8, D), (16, D), (40, P)])
def test_tiny_magnitude_rows(orc, T, path):
    """Rows scaled by 2^-58 (their h falls below 2^-113: a power-of-two scale
    of the h slices beyond fp32's exponent range) and by 2^-120 (the
    activations' own scale beyond it): finite outputs that match the
    oracle (values under fp32's normal range underflow, hence the floor)."""
    base = synth.layer_inputs(_cfg("decode", name="tinymag", n_experts=16, hidden=512, ffn=256, shared_ffn=256),
                              T=T, threads=2)
    xf = synth.bf16_bits_to_f32(base.x).astype(np.float64)
    for e in (-58, -120):
        print(f"[edges] tiny rows T={T} path={path} scale 2^{e}", flush=True)
        xs = synth.f32_to_bf16_bits((xf * 2.0 ** e).astype(np.float32))
        li = dataclasses.replace(base, x=xs)
        _check(orc, li, path, abs_floor=FP32_TINY)
    # fp32 activations down in fp32's subnormal range
    fb = synth.layer_inputs(_cfg("tiny", name="tinymag32", n_experts=8), T=T, threads=2)
    li = dataclasses.replace(fb, x=(fb.x.astype(np.float64) * 2.0 ** -140).astype(np.float32))
    print(f"[edges] fp32 subnormal rows T={T} path={path}", flush=True)
    _check(orc, li, path, abs_floor=FP32_TINY)


def test_mixed_row_magnitudes(orc):
    """Rows of very different magnitudes in one window: each row has its own
    power-of-two scale, so the small rows keep their precision."""
    li = synth.layer_inputs(_cfg("decode", name="mixmag", n_experts=16, hidden=512, ffn=256, shared_ffn=256),
                            T=4, threads=2)
    xf = synth.bf16_bits_to_f32(li.x).astype(np.float64)
    xf *= (2.0 ** np.array([0, -30, 20, -50], dtype=np.float64))[:, None]
    li = dataclasses.replace(li, x=synth.f32_to_bf16_bits(xf.astype(np.float32)))
    y, idx, _ = DevLayer(li).forward(D)
    yr, ir, _ = oracle_forward(orc, li)
    assert np.array_equal(idx, ir)
    for t in range(4):
        e = rel_err(y[t], yr[t])
        print(f"    row {t}: rel err {e:.3e}", flush=True)
        assert e <= TOL, (t, e)


# ---- routing heat ----------------------------------------------------------------

@pytest.mark.parametrize("name,T,path,scale", [
    ("decode", 1, D, {}),                                       # split launch
    ("e512", 4, D, {}),                                         # split launch, 4 rows
    ("mtp16", 16, D, {}),                                       # matrix-core launch
    ("e512", 2048, P, {"hidden": 512, "ffn": 256}),             # prefill path
    ("e512", 8, D, {"n_experts": 1500, "hidden": 512, "ffn": 256, "shared_ffn": 256}),  # E > 1024
])
def test_heat_counts(orc, name, T, path, scale):
    """heat[e] += the number of pairs routed to e: bit-exact against the
    oracle's grouping (offsets differences), accumulated over calls."""
    print(f"[heat] {name} T={T} path={path} {scale}", flush=True)
    cfg = _cfg(name, name=f"heat_{name}", **scale) if scale else synth.CONFIGS[name]
    li = synth.layer_inputs(cfg, T=T, threads=8)
    dl = DevLayer(li)
    E, k = cfg.n_experts, cfg.top_k
    ri, _ = orc.route(li.logits, k)
    ro, _, _ = orc.group(ri, E)
    counts = np.diff(ro).astype(np.int64)
    assert counts.sum() == T * k
    base = np.random.default_rng(3).integers(0, 1000, E).astype(np.int32)
    heat = torch.from_numpy(base.copy()).to(DEV)
    ws = moe.workspace(T, E, k, cfg.hidden, cfg.ffn, cfg.shared_ffn, path)
    y = torch.empty((T, cfg.hidden), dtype=torch.float32, device=DEV)
    for rep in (1, 2):
        moe.layer_forward(dl.x, dl.logits, k, dl.routed, dl.shared, y, ws, path=path, heat=heat)
        torch.cuda.synchronize()
        assert moe.workspace_error(ws) == 0
        got = heat.cpu().numpy().astype(np.int64)
        assert np.array_equal(got, base + rep * counts), rep
    # without the buffer nothing is counted (and nothing else changes)
    moe.layer_forward(dl.x, dl.logits, k, dl.routed, dl.shared, y, ws, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(heat.cpu().numpy().astype(np.int64), base + 2 * counts)


def test_heat_per_layer_rows(orc):
    """One heat row per layer: each layer's call adds to its own row only."""
    cfg = synth.CONFIGS["e512"]
    E, k = cfg.n_experts, cfg.top_k
    heat = torch.zeros((3, E), dtype=torch.int32, device=DEV)
    ws = moe.workspace(4, E, k, cfg.hidden, cfg.ffn, cfg.shared_ffn, D)
    exp = np.zeros((3, E), dtype=np.int64)
    for layer in range(3):
        li = synth.layer_inputs(cfg, layer=layer, T=4)
        dl = DevLayer(li)
        y = torch.empty((4, cfg.hidden), dtype=torch.float32, device=DEV)
        moe.layer_forward(dl.x, dl.logits, k, dl.routed, dl.shared, y, ws, path=D, heat=heat[layer])
        ri, _ = orc.route(li.logits, k)
        exp[layer] = np.bincount(ri.reshape(-1), minlength=E)
    torch.cuda.synchronize()
    assert np.array_equal(heat.cpu().numpy().astype(np.int64), exp)


# ---- the device error word --------------------------------------------------------

def test_error_word_clear_after_calls(orc):
    """After correct calls of every launch family on one workspace the error
    word reads 0 (a malformed grouping sets bit 1 and is reported)."""
    cfg = synth.CONFIGS["e512"]
    ws = moe.workspace(16, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, cfg.shared_ffn, D)
    for T in (1, 4, 16):
        li = synth.layer_inputs(cfg, T=T, layer=5)
        DevLayer(li).forward(D, ws=ws)
        assert moe.workspace_error(ws, clear=False) == 0
    # a grouping whose active list claims an expert id out of range
    T, k = 2, cfg.top_k
    li = synth.layer_inputs(cfg, T=T, layer=6)
    dl = DevLayer(li)
    ri, rw = orc.route(li.logits, k)
    ro, rp, ra = orc.group(ri, cfg.n_experts)
    bad = ra.copy()
    bad[1] = cfg.n_experts + 7
    out = torch.zeros((T * k, cfg.hidden), dtype=torch.float32, device=DEV)
    moe.expert_ffn(dl.x, dl.routed, torch.from_numpy(ro).to(DEV), torch.from_numpy(np.ascontiguousarray(rp)).to(DEV),
                   torch.from_numpy(bad).to(DEV), k, out, ws, pair_w=torch.from_numpy(rw.astype(np.float32)).to(DEV),
                   path=D)
    torch.cuda.synchronize()
    assert moe.workspace_error(ws) & moe.ERR_BAD_GROUPING
    assert moe.workspace_error(ws) == 0  # cleared by the read before
    # the workspace still serves correct calls afterwards
    y, idx, _ = dl.forward(D, ws=ws)
    yr, ir, _ = oracle_forward(orc, li)
    assert np.array_equal(idx, ir) and rel_err(y, yr) <= TOL
