"""moe_layer_forward_noalloc (the layer with the library's static device
scratch, for callers that cannot allocate) against moe_layer_forward with a
caller workspace, through the C ABI (GPU).

Two calls in a row, the second on a smaller window, then a third of one row:
the same kernels run, so the outputs, routing and heat are bitwise those of
the workspace entry point, and within the oracle's bar."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL, DevLayer, layer_inputs, oracle_forward, rel_err
from quantized_routed_expert_amd import moe, synth

pytestmark = pytest.mark.gpu


def _noalloc(dl, heat=None, path=moe.PATH_AUTO):
    cfg = dl.cfg
    T, k = dl.T, cfg.top_k
    y = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    moe.layer_forward_noalloc(dl.x, dl.logits, k, dl.routed, dl.shared, y, idx, w, path=path, heat=heat)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def test_noalloc_matches_workspace_entry(orc):
    for name, T in (("mtp16", 16), ("e512", 4), ("decode", 1)):
        print(f"[noalloc] {name} T={T}", flush=True)
        li = layer_inputs(name, T)
        dl = DevLayer(li)
        cfg = li.cfg
        heat_a = torch.zeros(cfg.n_experts, dtype=torch.int32, device=DEV)
        heat_b = torch.zeros(cfg.n_experts, dtype=torch.int32, device=DEV)
        yb, ib, wb = _noalloc(dl, heat=heat_b)
        ws = moe.workspace(T, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, cfg.shared_ffn)
        ya = torch.empty((T, cfg.hidden), dtype=torch.float32, device=DEV)
        moe.layer_forward(dl.x, dl.logits, cfg.top_k, dl.routed, dl.shared, ya, ws, heat=heat_a)
        torch.cuda.synchronize()
        assert moe.workspace_error(ws) == 0
        ya = ya.cpu().numpy()
        yr, ir, _ = oracle_forward(orc, li)
        assert np.array_equal(ib, ir)
        assert np.array_equal(yb, ya), name
        assert np.array_equal(heat_a.cpu().numpy(), heat_b.cpu().numpy())
        e = rel_err(yb, yr)
        print(f"    rel err {e:.3e}", flush=True)
        assert e <= TOL


def test_noalloc_repeat_and_graph(orc):
    """Back-to-back calls and graph replays on the shared scratch stay exact."""
    li = layer_inputs("e512", 4)
    dl = DevLayer(li)
    y0 = _noalloc(dl)[0]
    for _ in range(3):
        assert np.array_equal(_noalloc(dl)[0], y0)
    cfg = li.cfg
    y = torch.empty((4, cfg.hidden), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        moe.layer_forward_noalloc(dl.x, dl.logits, cfg.top_k, dl.routed, dl.shared, y, stream=s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            moe.layer_forward_noalloc(dl.x, dl.logits, cfg.top_k, dl.routed, dl.shared, y, stream=s)
    for _ in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), y0)
        assert np.array_equal(_noalloc(dl)[0], y0)  # eager calls between the replays


def test_noalloc_rejects_oversize():
    """A 2048-token prefill chunk needs more than the static scratch: refused
    before any launch, the output untouched."""
    cfg = synth.CONFIGS["e512"]
    need = moe.workspace_bytes(2048, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, cfg.shared_ffn)
    assert need > moe.NOALLOC_SCRATCH_BYTES
    li = synth.layer_inputs(synth.scaled_config(cfg, name="big", n_experts=16), T=2048, threads=8)
    dl = DevLayer(li)
    y = torch.full((2048, cfg.hidden), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError) as ex:
        moe.layer_forward_noalloc(dl.x, dl.logits, li.cfg.top_k, dl.routed, dl.shared, y)
    assert ex.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))
