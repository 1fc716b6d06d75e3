"""Python binding of the C ABI in include/moe.h (argument marshalling only).

Every step of the layer runs in the HIP library libmoe_gfx950.so; this module
only turns torch tensors into device pointers and sizes, passes the current
stream as an int64 and raises on a non-zero status.  It never computes any
part of the layer itself and has no fallback: if the library is missing it
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gfx950.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_LAUNCH = -4
MOE_ERR_DEVICE = -5

DTYPE_F32, DTYPE_BF16 = 0, 1
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2
DECODE_MAX_ROWS = 16
LAYOUT_ROWS, LAYOUT_PREPARED = 0, 1

EXPORTS = ["moe_version", "moe_status_string", "moe_expert_bytes", "moe_workspace_bytes",
           "moe_prepare_qweights", "moe_workspace_error", "moe_router_logits", "moe_route", "moe_group", "moe_expert_ffn",
           "moe_layer_forward", "moe_layer_forward_noalloc"]
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024

# bits of the workspace error word (moe_workspace_error)
ERR_WAIT_TIMEOUT = 1
ERR_BAD_GROUPING = 2


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


class QWeights(ctypes.Structure):
    """moe_qweights: device pointer + format and shape of a set of experts."""
    _fields_ = [("data", ctypes.c_void_p), ("bits", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("down_bits", ctypes.c_int32), ("codebook", ctypes.c_int8 * 16)]


BITS_NL4 = 20  # the non-linear 4-bit format (4-bit layout, codes index a 16-entry int8 table)


def _qw(data_ptr, bits, n_experts, hidden, ffn, layout, down_bits, codebook) -> QWeights:
    q = QWeights(ctypes.c_void_p(data_ptr), bits, n_experts, hidden, ffn, layout, down_bits)
    if codebook is not None:
        cb = [int(v) for v in codebook]
        if len(cb) != 16 or any(v < -128 or v > 127 for v in cb):
            raise ValueError("codebook: 16 values in -128..127")
        q.codebook = (ctypes.c_int8 * 16)(*cb)
    return q


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} (run quantized_routed_expert_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.moe_version.restype = ctypes.c_int
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_expert_bytes.restype = i64
        L.moe_expert_bytes.argtypes = [i32, i32, i32, i32]
        L.moe_workspace_bytes.restype = i64
        L.moe_workspace_bytes.argtypes = [i32] * 7
        L.moe_prepare_qweights.restype = ctypes.c_int
        L.moe_prepare_qweights.argtypes = [ctypes.POINTER(QWeights), vp, i64]
        L.moe_workspace_error.restype = ctypes.c_int
        L.moe_workspace_error.argtypes = [vp, i64, ctypes.POINTER(ctypes.c_uint32), i32, i64]
        L.moe_router_logits.restype = ctypes.c_int
        L.moe_router_logits.argtypes = [vp, i32, i32, i32, vp, i32, vp, i64]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [vp, i32, i32, i32, vp, vp, i64]
        L.moe_group.restype = ctypes.c_int
        L.moe_group.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, i64, i64]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [vp, i32, i32, ctypes.POINTER(QWeights), vp, vp, vp, vp, i32, vp, i32,
                                     vp, i64, i64]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward.argtypes = [vp, i32, vp, i32, i32, ctypes.POINTER(QWeights),
                                        ctypes.POINTER(QWeights), vp, vp, vp, vp, i32, vp, i64, i64]
        L.moe_layer_forward_noalloc.restype = ctypes.c_int
        L.moe_layer_forward_noalloc.argtypes = [vp, i32, vp, i32, i32, ctypes.POINTER(QWeights),
                                                ctypes.POINTER(QWeights), vp, vp, vp, vp, i32, i64]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoeError(rc, where)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _xcode(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return DTYPE_F32
    if x.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")


def qweights_at(data_ptr, bits: int, n_experts: int, hidden: int, ffn: int, layout: int,
                down_bits: int = 0, codebook=None) -> QWeights:
    """QWeights for a raw device address (an int or ctypes.c_void_p)."""
    if isinstance(data_ptr, ctypes.c_void_p):
        data_ptr = data_ptr.value
    return _qw(data_ptr, bits, n_experts, hidden, ffn, layout, down_bits, codebook)


def qweights(data: torch.Tensor, bits: int, n_experts: int, hidden: int, ffn: int, layout: int,
             down_bits: int = 0, codebook=None) -> QWeights:
    """Describe a uint8 device tensor holding n_experts expert blobs in the
    given block order (LAYOUT_ROWS or LAYOUT_PREPARED); gate/up in `bits`,
    down in `down_bits` (0: the same); codebook: the 16 int8 values of the
    non-linear format (BITS_NL4)."""
    return _qw(data.data_ptr(), bits, n_experts, hidden, ffn, layout, down_bits, codebook)


def prepare_qweights(data: torch.Tensor, bits: int, n_experts: int, hidden: int, ffn: int, out=None,
                     stream=None, down_bits: int = 0, codebook=None):
    """Blobs in the pages' row-by-row order (uint8 device tensor) -> a new
    tensor in the order the compute calls read; returns (tensor, QWeights)."""
    if out is None:
        out = torch.empty_like(data)
    src = _qw(data.data_ptr(), bits, n_experts, hidden, ffn, LAYOUT_ROWS, down_bits, codebook)
    _check(lib().moe_prepare_qweights(ctypes.byref(src), _ptr(out), _stream(stream)), "moe_prepare_qweights")
    return out, qweights(out, bits, n_experts, hidden, ffn, LAYOUT_PREPARED, down_bits, codebook)


def expert_bytes(bits: int, hidden: int, ffn: int, down_bits: int = 0) -> int:
    return int(lib().moe_expert_bytes(bits, down_bits, hidden, ffn))


def workspace_bytes(T: int, E: int, k: int, hidden: int, ffn: int, shared_ffn: int = 0,
                    path: int = PATH_AUTO) -> int:
    n = int(lib().moe_workspace_bytes(T, E, k, hidden, ffn, shared_ffn, path))
    if n < 0:
        raise MoeError(n, "moe_workspace_bytes")
    return n


def workspace(T, E, k, hidden, ffn, shared_ffn=0, path=PATH_AUTO, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of the required size (uint8 device tensor)."""
    return torch.zeros(max(workspace_bytes(T, E, k, hidden, ffn, shared_ffn, path), 1), dtype=torch.uint8,
                       device=device)


def workspace_error(ws: torch.Tensor, clear: bool = True, stream=None) -> int:
    """The workspace's device error word (0 after correct calls); waits for
    the stream and, with clear, resets the word."""
    v = ctypes.c_uint32(0)
    _check(lib().moe_workspace_error(_ptr(ws), ws.numel(), ctypes.byref(v), 1 if clear else 0, _stream(stream)),
           "moe_workspace_error")
    return int(v.value)


def router_logits(x: torch.Tensor, w_router: torch.Tensor, logits=None, stream=None) -> torch.Tensor:
    """x [T, H] fp32/bf16, w_router [E, H] bf16 (device) -> logits [T, E] fp32."""
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.dtype != torch.bfloat16 or tuple(w_router.shape) != (E, H):
        raise TypeError("w_router must be a bf16 [E, H] tensor")
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check(lib().moe_router_logits(_ptr(x), _xcode(x), T, H, _ptr(w_router), E, _ptr(logits), _stream(stream)),
           "moe_router_logits")
    return logits


def route(logits: torch.Tensor, k: int, topk_idx=None, topk_w=None, stream=None):
    T, E = logits.shape
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_w), _stream(stream)), "moe_route")
    return topk_idx, topk_w


def group(topk_idx: torch.Tensor, E: int, ws: torch.Tensor, offsets=None, pairs=None, active=None,
          stream=None):
    T, k = topk_idx.shape
    dev = topk_idx.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    pairs = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev) if pairs is None else pairs
    active = torch.empty(E + 1, dtype=torch.int32, device=dev) if active is None else active
    _check(lib().moe_group(_ptr(topk_idx), T, E, k, _ptr(offsets), _ptr(pairs), _ptr(active), _ptr(ws),
                           ws.numel(), _stream(stream)), "moe_group")
    return offsets, pairs, active


def expert_ffn(x: torch.Tensor, w: QWeights, offsets, pairs, active, k: int, out_pairs: torch.Tensor,
               ws: torch.Tensor, pair_w=None, path: int = PATH_AUTO, stream=None):
    T = x.shape[0]
    _check(lib().moe_expert_ffn(_ptr(x), _xcode(x), T, ctypes.byref(w), _ptr(offsets), _ptr(pairs),
                                _ptr(active), _ptr(pair_w), k, _ptr(out_pairs), path, _ptr(ws), ws.numel(),
                                _stream(stream)), "moe_expert_ffn")
    return out_pairs


def layer_forward(x: torch.Tensor, logits: torch.Tensor, k: int, routed: QWeights, shared: QWeights | None,
                  y: torch.Tensor, ws: torch.Tensor, topk_idx=None, topk_w=None, path: int = PATH_AUTO,
                  stream=None, heat=None):
    """heat: optional int32 [E] device tensor; the call adds its per-expert
    pair counts to it (routing heat)."""
    T = x.shape[0]
    _check(lib().moe_layer_forward(_ptr(x), _xcode(x), _ptr(logits), T, k, ctypes.byref(routed),
                                   ctypes.byref(shared) if shared is not None else None, _ptr(y),
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(heat), path, _ptr(ws), ws.numel(),
                                   _stream(stream)),
           "moe_layer_forward")
    return y


def layer_forward_noalloc(x: torch.Tensor, logits: torch.Tensor, k: int, routed: QWeights,
                          shared: QWeights | None, y: torch.Tensor, topk_idx=None, topk_w=None,
                          path: int = PATH_AUTO, stream=None, heat=None):
    """moe_layer_forward_noalloc: the layer with the library's static device
    scratch instead of a workspace (nothing is allocated)."""
    T = x.shape[0]
    _check(lib().moe_layer_forward_noalloc(_ptr(x), _xcode(x), _ptr(logits), T, k, ctypes.byref(routed),
                                           ctypes.byref(shared) if shared is not None else None, _ptr(y),
                                           _ptr(topk_idx), _ptr(topk_w), _ptr(heat), path, _stream(stream)),
           "moe_layer_forward_noalloc")
    return y
