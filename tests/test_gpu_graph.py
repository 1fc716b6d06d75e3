"""The layer captured in a HIP graph (as a 48-layer pass is): every replay
matches the eager result bitwise, with eager work and synchronizations
between replays (GPU)."""
import numpy as np
import pytest
import torch

from gpu_util import DevLayer, layer_inputs
from quantized_routed_expert_amd import moe, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T,path", [("decode", 1, moe.PATH_DECODE), ("mtp16", 16, moe.PATH_DECODE),
                                         ("prefill", 300, moe.PATH_PREFILL)])
def test_graph_replays(name, T, path):
    print(f"[graph] {name} T={T} path={path}", flush=True)
    cfg = synth.CONFIGS[name]
    layers = [DevLayer(synth.layer_inputs(cfg, layer=i, T=T)) for i in range(3)]
    ws = moe.workspace(T, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, cfg.shared_ffn, path)
    ys = [torch.zeros((T, cfg.hidden), device="cuda:0") for _ in layers]
    eager = []
    for dl, y in zip(layers, ys):
        moe.layer_forward(dl.x, dl.logits, cfg.top_k, dl.routed, dl.shared, y, ws, path=path)
        torch.cuda.synchronize()
        eager.append(y.cpu().numpy().copy())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for dl, y in zip(layers, ys):
                moe.layer_forward(dl.x, dl.logits, cfg.top_k, dl.routed, dl.shared, y, ws, path=path,
                                  stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for y in ys:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(ys):
            assert np.array_equal(y.cpu().numpy(), eager[i]), (rep, i)
        # eager work between replays on the same workspace
        moe.layer_forward(layers[0].x, layers[0].logits, cfg.top_k, layers[0].routed, layers[0].shared,
                          ys[0], ws, path=path)
        torch.cuda.synchronize()
        assert np.array_equal(ys[0].cpu().numpy(), eager[0])
