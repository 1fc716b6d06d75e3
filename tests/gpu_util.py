"""Helpers for the GPU parity tests: seeded inputs to device, one call
through the C ABI, and the parity measure against the oracle."""
import functools

import numpy as np
import torch

from quantized_routed_expert_amd import moe, synth

DEV = "cuda:0"
TOL = 2e-3  # max |err| <= TOL * rms(oracle output)


def x_to_dev(x: np.ndarray, x_dtype: str) -> torch.Tensor:
    if x_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


class DevLayer:
    """A layer's seeded inputs resident on the GPU."""

    def __init__(self, li: synth.LayerInputs):
        cfg = li.cfg
        self.li = li
        self.cfg = cfg
        self.T = li.T
        self.x = x_to_dev(li.x, cfg.x_dtype)
        self.logits = torch.from_numpy(li.logits).to(DEV)
        # the pages' block order on the host, converted once on the device
        cb = cfg.codebook or None
        self.routed_t, self.routed = moe.prepare_qweights(torch.from_numpy(li.routed).to(DEV), cfg.bits,
                                                          cfg.n_experts, cfg.hidden, cfg.ffn,
                                                          down_bits=cfg.down_bits, codebook=cb)
        self.shared_t = None
        self.shared = None
        if li.shared is not None:
            self.shared_t, self.shared = moe.prepare_qweights(torch.from_numpy(li.shared).to(DEV), cfg.bits, 1,
                                                              cfg.hidden, cfg.shared_ffn, down_bits=cfg.down_bits,
                                                              codebook=cb)

    def forward(self, path=moe.PATH_AUTO, ws=None, want_routing=True):
        cfg = self.cfg
        T, k = self.T, cfg.top_k
        if ws is None:
            ws = moe.workspace(T, cfg.n_experts, k, cfg.hidden, cfg.ffn, cfg.shared_ffn, path)
        y = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float32, device=DEV)
        idx = torch.full((T, k), -1, dtype=torch.int32, device=DEV) if want_routing else None
        w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV) if want_routing else None
        moe.layer_forward(self.x, self.logits, k, self.routed, self.shared, y, ws, idx, w, path=path)
        torch.cuda.synchronize()
        assert moe.workspace_error(ws) == 0, "device error word set"
        return (y.cpu().numpy(), None if idx is None else idx.cpu().numpy(),
                None if w is None else w.cpu().numpy())


@functools.lru_cache(maxsize=8)
def layer_inputs(name: str, T: int, layer: int = 0, seed: int = 0):
    return synth.layer_inputs(synth.CONFIGS[name], layer=layer, T=T, base_seed=seed)


def oracle_forward(orc, li: synth.LayerInputs, rows=None):
    cfg = li.cfg
    return orc.layer_forward(li.x, li.x_code, li.logits, cfg.top_k, cfg.fmt, cfg.ffn, li.routed, li.shared,
                             s_ffn=cfg.shared_ffn or None, rows=rows, codebook=cfg.codebook or None)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(np.asarray(ref, dtype=np.float64) ** 2)))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref))) / max(rms, 1e-30)
