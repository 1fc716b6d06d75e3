"""Per-projection weight formats through the C ABI against the oracle (GPU):
gate/up in one bit width and down in the other (the thread's §三 decode
table pairs a 2- or 3-bit gate/up format with a 4-bit down format), on every
launch family: the column-split decode (1-4 rows), the matrix-core decode
(5-16 rows), the prefill GEMMs, and the expert FFN entry point.

Bar: routing bit-exact; outputs within max |err| <= 2e-3 * rms(oracle)."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL, DevLayer, oracle_forward, rel_err, x_to_dev
from quantized_routed_expert_amd import moe, synth

pytestmark = pytest.mark.gpu

D, P = moe.PATH_DECODE, moe.PATH_PREFILL
PAIRS = [(3, 4), (4, 3)]


def _check(orc, li, path):
    y, idx, w = DevLayer(li).forward(path)
    yr, ir, wr = oracle_forward(orc, li)
    assert np.array_equal(idx, ir), "routing differs"
    assert np.all(np.isfinite(y))
    e = rel_err(y, yr)
    print(f"    rel err {e:.3e}", flush=True)
    assert e <= TOL, e


@pytest.mark.parametrize("bg,bd", PAIRS)
@pytest.mark.parametrize("name,T,path", [
    ("e512", 1, D), ("e512", 4, D), ("e512", 2, D),   # column-split launch
    ("mtp16", 16, D), ("e512", 8, D),                 # matrix-core launch
    ("e512", 64, P),                                  # prefill GEMMs
])
def test_mixed_formats_full_shapes(orc, bg, bd, name, T, path):
    """The workloads' layer shapes (hidden 2048, 128 or 512 experts) with
    gate/up and down in different widths, routed and shared experts alike."""
    print(f"[formats] {name} T={T} path={path} gate/up {bg}-bit down {bd}-bit", flush=True)
    cfg = dataclasses.replace(synth.CONFIGS[name], name=f"{name}_{bg}{bd}", bits=bg, down_bits=bd)
    _check(orc, synth.layer_inputs(cfg, T=T), path)


@pytest.mark.parametrize("bg,bd", PAIRS)
def test_mixed_formats_edge_shapes(orc, bg, bd):
    """Other widths: fp32 activations, a shared expert of another FFN width,
    no shared expert, hidden 256 .. 1024, k = E."""
    cases = [
        (synth.scaled_config(synth.CONFIGS["tiny"], name="mf_tiny"), (1, 3, 4, 9, 16, 40)),
        (synth.scaled_config(synth.CONFIGS["decode"], name="mf_h512", n_experts=16, hidden=512, ffn=256,
                             shared_ffn=1024), (1, 2, 4, 5, 16, 33)),
        (synth.scaled_config(synth.CONFIGS["e512"], name="mf_h1024", n_experts=40, hidden=1024, ffn=768,
                             shared_ffn=0), (1, 4, 12)),
        (synth.scaled_config(synth.CONFIGS["tiny"], name="mf_kE", n_experts=6, top_k=6), (2, 7)),
    ]
    for base, Ts in cases:
        cfg = dataclasses.replace(base, bits=bg, down_bits=bd)
        for T in Ts:
            for path in ((D, P) if T <= 16 else (P,)):
                print(f"[formats] {cfg.name} T={T} path={path} {bg}/{bd}", flush=True)
                _check(orc, synth.layer_inputs(cfg, T=T, threads=4), path)


@pytest.mark.parametrize("bg,bd", PAIRS)
@pytest.mark.parametrize("T,path", [(2, D), (12, D), (70, P)])
def test_mixed_formats_expert_ffn(orc, bg, bd, T, path):
    """moe_expert_ffn on a given grouping, per-pair rows."""
    cfg = synth.scaled_config(synth.CONFIGS["e512"], name=f"mf_ffn{bg}{bd}", n_experts=24, hidden=512, ffn=512,
                              bits=bg, down_bits=bd)
    li = synth.layer_inputs(cfg, T=T, threads=4)
    ri, rw = orc.route(li.logits, cfg.top_k)
    ro, rp, ra = orc.group(ri, cfg.n_experts)
    ref = orc.expert_ffn(li.x, li.x_code, cfg.top_k, cfg.fmt, cfg.n_experts, cfg.hidden, cfg.ffn, li.routed,
                         ro, rp, ra, rw)
    x = x_to_dev(li.x, cfg.x_dtype)
    _, qw = moe.prepare_qweights(torch.from_numpy(li.routed).to(DEV), bg, cfg.n_experts, cfg.hidden, cfg.ffn,
                                 down_bits=bd)
    out = torch.full((T * cfg.top_k, cfg.hidden), float("nan"), device=DEV)
    ws = moe.workspace(T, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, 0, path)
    moe.expert_ffn(x, qw, torch.from_numpy(ro).to(DEV), torch.from_numpy(np.ascontiguousarray(rp)).to(DEV),
                   torch.from_numpy(ra).to(DEV), cfg.top_k, out, ws,
                   pair_w=torch.from_numpy(rw.astype(np.float32)).to(DEV), path=path)
    torch.cuda.synchronize()
    assert moe.workspace_error(ws) == 0
    e = rel_err(out.cpu().numpy(), ref)
    print(f"[formats] expert_ffn T={T} path={path} {bg}/{bd}: rel err {e:.3e}", flush=True)
    assert e <= TOL


@pytest.mark.parametrize("bg,bd", PAIRS)
def test_mixed_prepare_order(bg, bd):
    """moe_prepare_qweights with per-projection widths: gate and up byte for
    byte, down blocks (of the down width) moved to index c*H + h."""
    cfg = synth.scaled_config(synth.CONFIGS["e512"], name="mf_prep", n_experts=3, hidden=512, ffn=256, bits=bg,
                              down_bits=bd)
    raw = synth.routed_weights(cfg, 0)
    dev, _ = moe.prepare_qweights(torch.from_numpy(raw).to(DEV), bg, 3, cfg.hidden, cfg.ffn, down_bits=bd)
    got = dev.cpu().numpy().reshape(3, -1)
    H, F = cfg.hidden, cfg.ffn
    gu = 2 * F * (H // 32) * synth.block_bytes(bg)
    bbd = synth.block_bytes(bd)
    exp = raw.reshape(3, -1).copy()
    exp[:, gu:] = exp[:, gu:].reshape(3, H, F // 32, bbd).transpose(0, 2, 1, 3).reshape(3, -1)
    assert np.array_equal(got, exp)
