"""The router projection (moe_router_logits) and the router + layer stack
through the C ABI against the oracle (GPU).

Logits bar, per element, from the arithmetic: bf16 x bf16 products are exact
in fp32 and the H products (plus eight partial tiles) are summed in fp32, so
|err| <= (H + 8) * 2^-24 * sum_h |x_h w_h|; fp32 x enters as bf16 hi + lo,
which adds 2^-17 * sum_h |x_h w_h|.

Stack bar: the layer consumes the GPU's fp32 logits, and the oracle's layer
is run on those same logits, so both take the top-k decision on the same
values: routing bit-exact, outputs within max |err| <= 2e-3 * rms(oracle)."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL, DevLayer, rel_err, x_to_dev
from quantized_routed_expert_amd import moe, synth

pytestmark = pytest.mark.gpu


def _wdev(w_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(w_bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _bound(x, x_code, w_bits):
    X = np.abs(synth.bf16_bits_to_f32(x).astype(np.float64) if x_code == 1 else x.astype(np.float64))
    W = np.abs(synth.bf16_bits_to_f32(w_bits).astype(np.float64))
    H = X.shape[1]
    c = (H + 8) * 2.0 ** -24 + (2.0 ** -17 if x_code == 0 else 0.0)
    return c * (X @ W.T)


@pytest.mark.parametrize("name,T", [("decode", 1), ("decode", 16), ("e512", 4), ("e512", 2048), ("tiny", 4),
                                    ("tiny", 37)])
def test_router_logits(orc, name, T):
    print(f"[router] {name} T={T}", flush=True)
    cfg = synth.CONFIGS[name]
    x = synth.activations(cfg, 0, T)
    w = synth.router_weights(cfg, 0)
    got = moe.router_logits(x_to_dev(x, cfg.x_dtype), _wdev(w))
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    code = 0 if cfg.x_dtype == "f32" else 1
    ref = orc.router_logits(x, code, w)
    err = np.abs(got - ref)
    b = _bound(x, code, w)
    print(f"    max err {err.max():.3e}, max err/bound {np.max(err / np.maximum(b, 1e-300)):.3e}", flush=True)
    assert np.all(err <= b)
    assert rel_err(got, ref) <= 1e-5


def test_router_batch_invariance():
    """A row's logits are bitwise the same alone, in a 16-row window and in
    a 2048-row chunk; two runs give the same bits."""
    cfg = synth.CONFIGS["e512"]
    x = synth.activations(cfg, 3, 2048)
    w = _wdev(synth.router_weights(cfg, 3))
    xd = x_to_dev(x, cfg.x_dtype)
    full = moe.router_logits(xd, w).cpu().numpy()
    again = moe.router_logits(xd, w).cpu().numpy()
    assert np.array_equal(full, again)
    win = moe.router_logits(xd[100:116].contiguous(), w).cpu().numpy()
    assert np.array_equal(win, full[100:116])
    for t in (0, 5, 2047):
        one = moe.router_logits(xd[t:t + 1].contiguous(), w).cpu().numpy()
        assert np.array_equal(one[0], full[t])


@pytest.mark.parametrize("name,T", [("decode", 1), ("mtp16", 16), ("e512", 4), ("prefill", 2048)])
def test_router_layer_stack(orc, name, T):
    """Router projection, then the layer on its logits, for three layers in
    one captured graph, replayed with eager calls between the replays; every
    replay bitwise the eager pass, each layer within the oracle's bar."""
    print(f"[stack] {name} T={T}", flush=True)
    cfg = synth.CONFIGS[name]
    path = moe.PATH_AUTO
    layers = []
    for l in range(3):
        li = synth.layer_inputs(cfg, layer=l, T=T)
        dl = DevLayer(li)
        dl.w_router = synth.router_weights(cfg, l)
        dl.wr = _wdev(dl.w_router)
        dl.lg = torch.empty((T, cfg.n_experts), dtype=torch.float32, device=DEV)
        dl.y = torch.empty((T, cfg.hidden), dtype=torch.float32, device=DEV)
        dl.idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=DEV)
        layers.append(dl)
    ws = moe.workspace(T, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, cfg.shared_ffn, path)
    s = torch.cuda.Stream()

    def one_pass():
        for dl in layers:
            moe.router_logits(dl.x, dl.wr, logits=dl.lg, stream=s)
            moe.layer_forward(dl.x, dl.lg, cfg.top_k, dl.routed, dl.shared, dl.y, ws, topk_idx=dl.idx, path=path,
                              stream=s)

    with torch.cuda.stream(s):
        one_pass()
    torch.cuda.synchronize()
    assert moe.workspace_error(ws) == 0
    eager = [(dl.lg.cpu().numpy(), dl.y.cpu().numpy(), dl.idx.cpu().numpy()) for dl in layers]
    for dl, (lg, y, idx) in zip(layers, eager):
        li = dl.li
        yr, ir, _ = orc.layer_forward(li.x, li.x_code, lg, cfg.top_k, cfg.fmt, cfg.ffn, li.routed, li.shared,
                                      s_ffn=cfg.shared_ffn or None)
        assert np.array_equal(idx, ir)
        e = rel_err(y, yr)
        print(f"    layer rel err {e:.3e}", flush=True)
        assert e <= TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            one_pass()
    for _ in range(3):
        for dl in layers:
            dl.y.fill_(float("nan"))
            dl.lg.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for dl, (lg, y, idx) in zip(layers, eager):
            assert np.array_equal(dl.lg.cpu().numpy(), lg)
            assert np.array_equal(dl.y.cpu().numpy(), y)
        with torch.cuda.stream(s):
            one_pass()  # eager work between the replays
        torch.cuda.synchronize()
    assert moe.workspace_error(ws) == 0
