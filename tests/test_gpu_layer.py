"""The whole layer (moe_layer_forward) and the expert FFN (moe_expert_ffn)
through the C ABI against the oracle (GPU).

Bar: routing bit-exact; outputs within max |err| <= 2e-3 * rms(oracle)."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL, DevLayer, layer_inputs, oracle_forward, rel_err, x_to_dev
from quantized_routed_expert_amd import moe, synth

pytestmark = pytest.mark.gpu

D, P = moe.PATH_DECODE, moe.PATH_PREFILL


def _check(orc, li, path, rows=None, tol=TOL):
    dl = DevLayer(li)
    y, idx, w = dl.forward(path)
    yr, ir, wr = oracle_forward(orc, li, rows=rows)
    assert np.array_equal(idx, ir), "routing differs"
    assert np.max(np.abs(w - wr)) <= 2e-6
    yy = y if rows is None else y[rows]
    assert np.all(np.isfinite(y))
    e = rel_err(yy, yr)
    print(f"    rel err {e:.3e}", flush=True)
    assert e <= tol, e
    return y


# ---- the five workloads at their own sizes (one layer) -------------------------

@pytest.mark.parametrize("name,T,path", [
    ("tiny", 4, D), ("tiny", 4, P),
    ("decode", 1, D), ("decode", 1, P),
    ("mtp16", 16, D),
    ("e512", 1, D), ("e512", 4, D), ("e512", 4, P),
])
def test_workload_full(orc, name, T, path):
    print(f"[layer] {name} T={T} path={path}", flush=True)
    _check(orc, layer_inputs(name, T), path)


@pytest.mark.parametrize("layer", [0, 31])
def test_prefill_chunk_full(orc, layer):
    """The whole 2048-token chunk (512 experts, top-10, Zipf routing) in the
    launch configuration the benchmark times, every row and output compared
    with the oracle (OpenMP over rows)."""
    print(f"[layer] prefill T=2048 layer={layer}, all rows (oracle on {orc.set_threads(0)} threads)", flush=True)
    li = synth.layer_inputs(synth.CONFIGS["prefill"], layer=layer, T=2048)
    _check(orc, li, P)


def test_mtp16_other_layers(orc):
    for layer in (1, 47):
        print(f"[layer] mtp16 layer={layer}", flush=True)
        _check(orc, synth.layer_inputs(synth.CONFIGS["mtp16"], layer=layer, T=16), D)


# ---- reduced shapes that the oracle runs whole, with ragged tiles ---------------

def _cfg(base, **kw):
    return synth.scaled_config(synth.CONFIGS[base], **kw)


@pytest.mark.parametrize("T", [17, 65, 200])
def test_prefill_scaled_full(orc, T):
    """Full comparison on the prefill path with ragged 64-row tiles."""
    print(f"[layer] prefill scaled T={T}", flush=True)
    cfg = _cfg("prefill", name="pf_scaled", hidden=512, n_experts=24, ffn=256, shared_ffn=512)
    _check(orc, synth.layer_inputs(cfg, T=T, threads=4), P)


def test_prefill_fp32_x(orc):
    print("[layer] prefill fp32 activations", flush=True)
    cfg = _cfg("tiny", name="tiny_pf", n_experts=16, top_k=4)
    _check(orc, synth.layer_inputs(cfg, T=40, threads=2), P)


def test_decode_no_shared_mixed_f(orc):
    print("[layer] decode without shared / shared with other F", flush=True)
    cfg = _cfg("mtp16", name="noshared", shared_ffn=0, n_experts=32, hidden=1024, ffn=512)
    _check(orc, synth.layer_inputs(cfg, T=5, threads=4), D)
    cfg = _cfg("decode", name="fs", shared_ffn=1024, n_experts=16, hidden=512, ffn=256)
    _check(orc, synth.layer_inputs(cfg, T=3, threads=4), D)
    _check(orc, synth.layer_inputs(cfg, T=3, threads=4), P)


def test_edge_cases(orc):
    # top-k = E (every expert on every row), one expert, all-equal logits (ties)
    print("[layer] k = E", flush=True)
    cfg = _cfg("tiny", name="kE", n_experts=6, top_k=6)
    _check(orc, synth.layer_inputs(cfg, T=16, threads=2), D)
    print("[layer] E = k = 1", flush=True)
    cfg = _cfg("tiny", name="e1", n_experts=1, top_k=1)
    _check(orc, synth.layer_inputs(cfg, T=9, threads=2), D)
    print("[layer] equal logits", flush=True)
    li = synth.layer_inputs(_cfg("e512", name="tie", n_experts=64), T=16, threads=4)
    li = dataclasses.replace(li, logits=np.zeros_like(li.logits))
    _check(orc, li, D)
    print("[layer] zero activations", flush=True)
    li = dataclasses.replace(li, x=np.zeros_like(li.x))
    y = DevLayer(li).forward(D)[0]
    assert np.all(y == 0.0)
    print("[layer] large-magnitude activations", flush=True)
    li = synth.layer_inputs(_cfg("decode", name="big", n_experts=16, hidden=512, ffn=256, shared_ffn=256),
                            T=4, threads=2)
    xb = (synth.bf16_bits_to_f32(li.x) * 3000.0).astype(np.float32)
    li = dataclasses.replace(li, x=synth.f32_to_bf16_bits(xb))
    _check(orc, li, D)
    _check(orc, li, P)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_split_launch_shapes(orc, T):
    """Windows of one to four rows take the column-split launch (integer dot
    products): both weight formats, fp32 and bf16 activations, every hidden
    size it takes (256 .. 2048), with and without a shared expert (of another
    width), k = E, E = k = 1, tied logits, zero and large activations."""
    cases = [
        ("tiny", _cfg("tiny", name="sp_tiny")),                                   # H 256, fp32 x, 4-bit
        ("h512", _cfg("decode", name="sp_h512", n_experts=16, hidden=512, ffn=256, shared_ffn=1024)),
        ("h1024_3b", _cfg("e512", name="sp_h1024", n_experts=40, hidden=1024, ffn=768, shared_ffn=0)),
        ("kE", _cfg("tiny", name="sp_kE", n_experts=6, top_k=6)),
        ("e1", _cfg("tiny", name="sp_e1", n_experts=1, top_k=1)),
        ("k32", _cfg("e512", name="sp_k32", n_experts=64, top_k=32, hidden=256, ffn=256, shared_ffn=256)),
    ]
    for tag, cfg in cases:
        print(f"[split] {tag} T={T}", flush=True)
        _check(orc, synth.layer_inputs(cfg, T=T, threads=2), D)
    print(f"[split] tied logits T={T}", flush=True)
    li = synth.layer_inputs(_cfg("e512", name="sp_tie", n_experts=64, hidden=512, ffn=256, shared_ffn=256),
                            T=T, threads=2)
    li = dataclasses.replace(li, logits=np.zeros_like(li.logits))
    _check(orc, li, D)
    print(f"[split] zero activations T={T}", flush=True)
    y = DevLayer(dataclasses.replace(li, x=np.zeros_like(li.x))).forward(D)[0]
    assert np.all(y == 0.0)
    print(f"[split] large activations T={T}", flush=True)
    li = synth.layer_inputs(_cfg("decode", name="sp_big", n_experts=16, hidden=512, ffn=256, shared_ffn=256),
                            T=T, threads=2)
    xb = (synth.bf16_bits_to_f32(li.x) * 3000.0).astype(np.float32)
    _check(orc, dataclasses.replace(li, x=synth.f32_to_bf16_bits(xb)), D)
    print(f"[split] real workloads T={T}", flush=True)
    _check(orc, layer_inputs("decode", T), D)
    _check(orc, layer_inputs("e512", T), D)


def test_decode_matches_prefill(orc):
    """The two kernel families agree with each other on the same inputs."""
    print("[layer] decode vs prefill kernels", flush=True)
    li = layer_inputs("mtp16", 16)
    dl = DevLayer(li)
    yd = dl.forward(D)[0]
    yp = dl.forward(P)[0]
    assert rel_err(yd, yp) <= TOL


# ---- determinism and batch invariance -------------------------------------------

def test_run_twice_bitwise():
    print("[layer] run twice", flush=True)
    for name, T, path in [("mtp16", 16, D), ("e512", 4, D), ("decode", 1, D), ("e512", 2, D), ("tiny", 3, D),
                          ("prefill", 512, P)]:
        li = layer_inputs(name, T) if T == synth.CONFIGS[name].rows[0] else synth.layer_inputs(
            synth.CONFIGS[name], T=T)
        dl = DevLayer(li)
        cfg = li.cfg
        ws = moe.workspace(T, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, cfg.shared_ffn, path)
        a = dl.forward(path, ws=ws)[0]
        b = dl.forward(path, ws=ws)[0]
        assert np.array_equal(a, b), (name, T)


def test_batch_invariance_decode():
    """A row's routing is bitwise the same in any window; its output is
    bitwise the same in any window served by the same launch: the 16-row
    window against 8-row windows (matrix-core launch, 5-16 rows), and 4-row
    and 2-row windows against single rows (column-split launch, 1-4 rows),
    both weight formats."""
    print("[layer] batch invariance", flush=True)
    li = layer_inputs("mtp16", 16)
    y16, i16, w16 = DevLayer(li).forward(D)
    for t0 in (0, 8):
        sub = dataclasses.replace(li, T=8, x=li.x[t0:t0 + 8].copy(), logits=li.logits[t0:t0 + 8].copy())
        y8, i8, w8 = DevLayer(sub).forward(D)
        assert np.array_equal(i8, i16[t0:t0 + 8]), t0
        assert np.array_equal(w8, w16[t0:t0 + 8]), t0
        assert np.array_equal(y8, y16[t0:t0 + 8]), t0
    for t in range(16):
        one = dataclasses.replace(li, T=1, x=li.x[t:t + 1].copy(), logits=li.logits[t:t + 1].copy())
        _, i1, w1 = DevLayer(one).forward(D)
        assert np.array_equal(i1[0], i16[t]), t
        assert np.array_equal(w1[0], w16[t]), t
    for name in ("decode", "e512"):
        li4 = layer_inputs(name, 4)
        y4, i4, w4 = DevLayer(li4).forward(D)
        sub = dataclasses.replace(li4, T=2, x=li4.x[1:3].copy(), logits=li4.logits[1:3].copy())
        y2, _, _ = DevLayer(sub).forward(D)
        assert np.array_equal(y2, y4[1:3]), name
        for t in range(4):
            one = dataclasses.replace(li4, T=1, x=li4.x[t:t + 1].copy(), logits=li4.logits[t:t + 1].copy())
            y1, i1, w1 = DevLayer(one).forward(D)
            assert np.array_equal(i1[0], i4[t]), (name, t)
            assert np.array_equal(w1[0], w4[t]), (name, t)
            assert np.array_equal(y1[0], y4[t]), (name, t)


def test_workspace_reuse_across_shapes(orc):
    """One workspace serves calls of different sizes in a row (its counters
    return to zero after every call)."""
    print("[layer] workspace reuse", flush=True)
    cfg = synth.CONFIGS["e512"]
    ws = moe.workspace(16, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, cfg.shared_ffn, D)
    for T in (4, 1, 16, 2, 3, 1, 4):
        li = synth.layer_inputs(cfg, T=T, layer=T)
        y, idx, _ = DevLayer(li).forward(D, ws=ws)
        yr, ir, _ = oracle_forward(orc, li)
        assert np.array_equal(idx, ir)
        assert rel_err(y, yr) <= TOL, T


# ---- the expert FFN entry point on a given grouping -------------------------------

@pytest.mark.parametrize("name,T,path", [("tiny", 4, D), ("mtp16", 16, D), ("e512", 4, P), ("tiny", 40, P),
                                         ("decode", 1, D), ("e512", 2, D), ("tiny", 2, D), ("e512", 4, D)])
def test_expert_ffn(orc, name, T, path):
    print(f"[expert_ffn] {name} T={T} path={path}", flush=True)
    cfg = synth.CONFIGS[name]
    li = synth.layer_inputs(cfg, T=T)
    ri, rw = orc.route(li.logits, cfg.top_k)
    ro, rp, ra = orc.group(ri, cfg.n_experts)
    ref = orc.expert_ffn(li.x, li.x_code, cfg.top_k, cfg.bits, cfg.n_experts, cfg.hidden, cfg.ffn,
                         li.routed, ro, rp, ra, rw)
    x = x_to_dev(li.x, cfg.x_dtype)
    routed_t, qw = moe.prepare_qweights(torch.from_numpy(li.routed).to(DEV), cfg.bits, cfg.n_experts, cfg.hidden,
                                        cfg.ffn)
    off = torch.from_numpy(ro).to(DEV)
    pairs = torch.from_numpy(np.ascontiguousarray(rp)).to(DEV)
    act = torch.from_numpy(ra).to(DEV)
    pw = torch.from_numpy(rw.astype(np.float32)).to(DEV)
    out = torch.full((T * cfg.top_k, cfg.hidden), float("nan"), device=DEV)
    ws = moe.workspace(T, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, 0, path)
    moe.expert_ffn(x, qw, off, pairs, act, cfg.top_k, out, ws, pair_w=pw, path=path)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert rel_err(got, ref) <= TOL


# ---- negative control -----------------------------------------------------------

def test_negative_control_corrupted_expert(orc):
    """Flip one byte of a selected expert on the device: the parity check must
    go red, so a green check carries evidence."""
    print("[layer] negative control", flush=True)
    li = layer_inputs("decode", 1)
    cfg = li.cfg
    dl = DevLayer(li)
    y0 = dl.forward(D)[0]
    yr, ir, _ = oracle_forward(orc, li)
    assert rel_err(y0, yr) <= TOL
    e = int(ir[0, 0])
    eb = cfg.expert_bytes
    # a down-projection block of the top expert: scale byte (high) of block 0,
    # row 0 (the first down block in either block order)
    off = e * eb + 2 * cfg.ffn * (cfg.hidden // 32) * cfg.block_bytes + 1
    dl.routed_t[off] ^= 0x40
    y1 = dl.forward(D)[0]
    assert rel_err(y1, yr) > TOL


# ---- weight preparation ---------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "e512"])
def test_prepare_qweights_order(name):
    """moe_prepare_qweights is a pure reordering: gate and up byte for byte,
    down block (h, c) moved to index c*H + h (checked against a numpy
    transpose of the blocks; both formats)."""
    print(f"[prepare] {name}", flush=True)
    cfg = synth.CONFIGS[name]
    li = layer_inputs(name, 1)
    n = 3
    raw = np.ascontiguousarray(li.routed[: n * cfg.expert_bytes])
    dev, _ = moe.prepare_qweights(torch.from_numpy(raw).to(DEV), cfg.bits, n, cfg.hidden, cfg.ffn)
    got = dev.cpu().numpy().reshape(n, -1)
    H, F, bb = cfg.hidden, cfg.ffn, cfg.block_bytes
    gu = 2 * F * (H // 32) * bb
    exp = raw.reshape(n, -1).copy()
    exp[:, gu:] = exp[:, gu:].reshape(n, H, F // 32, bb).transpose(0, 2, 1, 3).reshape(n, -1)
    assert np.array_equal(got, exp)


# ---- prefill tile heights: groups at every 16/32/64-row boundary ------------------

@pytest.mark.parametrize("bits,x_dtype", [(3, "bf16"), (4, "f32"), (3, "f32"), (4, "bf16")])
def test_prefill_group_size_boundaries(orc, bits, x_dtype):
    """moe_expert_ffn on the prefill path with a hand-made grouping (top-1):
    group sizes straddle the 16-, 32- and 64-row tile heights and need several
    64-row tiles, so every tile height, ragged last tiles and multi-tile
    groups are compared element by element with the oracle."""
    counts = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 129]
    E = len(counts) + 1  # one expert with no rows
    print(f"[prefill groups] bits={bits} x={x_dtype} counts={counts}", flush=True)
    cfg = synth.scaled_config(synth.CONFIGS["prefill"], name=f"pf_groups{bits}", bits=bits, x_dtype=x_dtype,
                              hidden=512, n_experts=E, ffn=256, shared_ffn=0, top_k=1)
    T = sum(counts)
    li = synth.layer_inputs(cfg, T=T)
    ids = np.concatenate([np.full(c, e + 1, dtype=np.int32) for e, c in enumerate(counts)])
    rng = np.random.default_rng(7)
    idx = rng.permutation(ids).reshape(T, 1).astype(np.int32)
    ro, rp, ra = orc.group(idx, E)
    assert [int(ro[e + 1] - ro[e]) for e in range(E)] == [0] + counts
    rw = rng.uniform(0.25, 1.0, T).astype(np.float64)
    ref = orc.expert_ffn(li.x, li.x_code, 1, bits, E, cfg.hidden, cfg.ffn, li.routed, ro, rp, ra, rw)
    x = x_to_dev(li.x, cfg.x_dtype)
    routed_t, qw = moe.prepare_qweights(torch.from_numpy(li.routed).to(DEV), bits, E, cfg.hidden, cfg.ffn)
    out = torch.full((T, cfg.hidden), float("nan"), device=DEV)
    ws = moe.workspace(T, E, 1, cfg.hidden, cfg.ffn, 0, P)
    moe.expert_ffn(x, qw, torch.from_numpy(ro).to(DEV), torch.from_numpy(np.ascontiguousarray(rp)).to(DEV),
                   torch.from_numpy(ra).to(DEV), 1, out, ws, pair_w=torch.from_numpy(rw.astype(np.float32)).to(DEV),
                   path=P)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    e = rel_err(got, ref)
    print(f"    rel err {e:.3e}", flush=True)
    assert e <= TOL


def test_prefill_many_experts(orc):
    """More than 1024 groups in one chunk (1,071 active experts + the shared
    one): the plan's general ranking and the GEMMs' slot plan at its largest."""
    print("[layer] prefill E=1100 T=512", flush=True)
    cfg = _cfg("e512", name="pf_e1100", n_experts=1100, hidden=256, ffn=256, shared_ffn=256, top_k=8)
    li = synth.layer_inputs(cfg, T=512, threads=4)
    _check(orc, li, P)
