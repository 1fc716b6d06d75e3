"""CPU oracle of the quantized routed-expert MoE layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product path (the HIP library and its
binding) never touches it.  The arithmetic lives in ``oracle.c`` (plain C,
binary64); this module only marshals numpy arrays into it.

Every function here is pinned by CPU tests against something other than
itself: golden blocks written from the format statement, closed forms,
brute force and invariants.  No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(out_path: str | None = None, extra_flags: list[str] | None = None, openmp: bool = True) -> str:
    """Compile oracle.c with gcc -O2 (and OpenMP over rows unless openmp is
    False) into a shared library; returns its path."""
    out = out_path or _LIB_PATH
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", out, _SRC, "-lm"]
    if openmp:
        cmd[1:1] = ["-fopenmp"]
    if extra_flags:
        cmd[1:1] = extra_flags
    subprocess.run(cmd, check=True)
    return out


def _bind(lib):
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    u8p = ctypes.c_void_p
    lib.orc_version.restype = ctypes.c_int
    lib.orc_set_threads.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_half_to_double.restype = ctypes.c_double
    lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_double.restype = ctypes.c_double
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_set_codebook.restype = None
    lib.orc_set_codebook.argtypes = [ctypes.c_void_p]
    lib.orc_block_bytes.restype = ctypes.c_int
    lib.orc_block_bytes.argtypes = [ctypes.c_int]
    lib.orc_format_bits.restype = ctypes.c_int
    lib.orc_format_bits.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.orc_expert_bytes.restype = ctypes.c_int64
    lib.orc_expert_bytes.argtypes = [ctypes.c_int] * 3
    lib.orc_dequant_block.restype = None
    lib.orc_dequant_block.argtypes = [ctypes.c_int, u8p, f64p]
    lib.orc_dequant_matrix.restype = ctypes.c_int
    lib.orc_dequant_matrix.argtypes = [ctypes.c_int, u8p, ctypes.c_int, ctypes.c_int, f64p]
    lib.orc_router_logits.restype = ctypes.c_int
    lib.orc_router_logits.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_int, f64p]
    lib.orc_route.restype = ctypes.c_int
    lib.orc_route.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p, f64p]
    lib.orc_group.restype = ctypes.c_int
    lib.orc_group.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p, i32p, i32p]
    lib.orc_expert_ffn.restype = ctypes.c_int
    lib.orc_expert_ffn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p,
                                   i32p, i32p, i32p, ctypes.c_void_p, f64p]
    lib.orc_layer_forward.restype = ctypes.c_int
    lib.orc_layer_forward.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, u8p, ctypes.c_int, ctypes.c_int, u8p,
                                      ctypes.c_int, ctypes.c_void_p, f64p, i32p, f64p]
    return lib


def load(path: str | None = None, rebuild_if_missing: bool = True):
    """Load (building if absent) the oracle library.  With ``path`` given,
    load that build instead of the default one (used by negative controls)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            if not rebuild_if_missing:
                raise RuntimeError("oracle library not built")
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a: np.ndarray, ctype=None):
    assert a.flags["C_CONTIGUOUS"]
    if ctype is None:
        return ctypes.c_void_p(a.ctypes.data)
    return a.ctypes.data_as(ctypes.POINTER(ctype))


X_F32, X_BF16 = 0, 1
BITS_NL4 = 20  # the non-linear 4-bit block (4-bit layout, codes index a 16-entry int8 table)


class Oracle:
    """Thin numpy front end over one build of oracle.c."""

    def __init__(self, lib=None):
        self.lib = lib or load()

    def set_threads(self, n: int = 0) -> int:
        """Threads for the loops over rows (n <= 0 keeps the current count);
        returns the count in use (1 for a serial build)."""
        return self.lib.orc_set_threads(int(n))

    # -- scalar formats ---------------------------------------------------
    def half_to_double(self, h: int) -> float:
        return self.lib.orc_half_to_double(int(h))

    def bf16_to_double(self, b: int) -> float:
        return self.lib.orc_bf16_to_double(int(b))

    # -- blocks -----------------------------------------------------------
    def set_codebook(self, cb) -> None:
        """The 16 signed 8-bit values that the non-linear 4-bit format's codes index."""
        c = np.ascontiguousarray(np.asarray(cb, dtype=np.int8).reshape(16))
        self.lib.orc_set_codebook(_ptr(c))

    def _cb(self, codebook):
        if codebook is not None:
            self.set_codebook(codebook)

    def block_bytes(self, bits: int) -> int:
        return self.lib.orc_block_bytes(bits)

    def format_bits(self, fmt: int, down: bool) -> int:
        """Bit width of the gate/up (down=False) or down projection of a format code."""
        return self.lib.orc_format_bits(fmt, 1 if down else 0)

    def expert_bytes(self, fmt: int, hidden: int, ffn: int) -> int:
        return self.lib.orc_expert_bytes(fmt, hidden, ffn)

    def dequant_block(self, bits: int, blk: bytes | np.ndarray, codebook=None) -> np.ndarray:
        self._cb(codebook)
        b = np.ascontiguousarray(np.frombuffer(bytes(blk), dtype=np.uint8))
        assert b.size == self.block_bytes(bits)
        out = np.zeros(32, dtype=np.float64)
        self.lib.orc_dequant_block(bits, _ptr(b), _ptr(out, ctypes.c_double))
        return out

    def dequant_matrix(self, bits: int, m: np.ndarray, rows: int, cols: int, codebook=None) -> np.ndarray:
        self._cb(codebook)
        m = np.ascontiguousarray(m, dtype=np.uint8)
        assert m.size >= rows * (cols // 32) * self.block_bytes(bits)
        out = np.zeros((rows, cols), dtype=np.float64)
        rc = self.lib.orc_dequant_matrix(bits, _ptr(m), rows, cols, _ptr(out, ctypes.c_double))
        assert rc == 0
        return out

    def dequant_expert(self, fmt: int, blob: np.ndarray, hidden: int, ffn: int, codebook=None):
        """(gate [F,H], up [F,H], down [H,F]) of one expert blob of format fmt."""
        self._cb(codebook)
        blob = np.ascontiguousarray(blob, dtype=np.uint8)
        bg, bd = self.format_bits(fmt, False), self.format_bits(fmt, True)
        mb = hidden * (ffn // 32) * self.block_bytes(bg)
        assert blob.size == self.expert_bytes(fmt, hidden, ffn)
        g = self.dequant_matrix(bg, blob[:mb], ffn, hidden)
        u = self.dequant_matrix(bg, blob[mb:2 * mb], ffn, hidden)
        d = self.dequant_matrix(bd, blob[2 * mb:], hidden, ffn)
        return g, u, d

    # -- router projection, router and grouping ----------------------------
    def router_logits(self, x: np.ndarray, x_dtype: int, w_router: np.ndarray) -> np.ndarray:
        """x [T,H] (fp32, or bf16 bits as uint16), w_router [E,H] bf16 bits
        (uint16) -> logits [T,E] float64."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w_router, dtype=np.uint16)
        T, H = x.shape
        E = w.shape[0]
        assert w.shape[1] == H
        out = np.zeros((T, E), dtype=np.float64)
        rc = self.lib.orc_router_logits(_ptr(x), x_dtype, T, H, _ptr(w), E, _ptr(out, ctypes.c_double))
        if rc:
            raise ValueError(f"orc_router_logits rc={rc}")
        return out

    def route(self, logits: np.ndarray, k: int):
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        T, E = logits.shape
        idx = np.zeros((T, k), dtype=np.int32)
        w = np.zeros((T, k), dtype=np.float64)
        rc = self.lib.orc_route(_ptr(logits), T, E, k, _ptr(idx, ctypes.c_int32),
                                _ptr(w, ctypes.c_double))
        if rc:
            raise ValueError(f"orc_route rc={rc}")
        return idx, w

    def group(self, idx: np.ndarray, E: int):
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, k = idx.shape
        offsets = np.zeros(E + 1, dtype=np.int32)
        pairs = np.zeros(max(T * k, 1), dtype=np.int32)
        active = np.zeros(E + 1, dtype=np.int32)
        rc = self.lib.orc_group(_ptr(idx, ctypes.c_int32), T, E, k, _ptr(offsets, ctypes.c_int32),
                                _ptr(pairs, ctypes.c_int32), _ptr(active, ctypes.c_int32))
        if rc:
            raise ValueError(f"orc_group rc={rc}")
        return offsets, pairs[:T * k], active

    # -- FFN and layer --------------------------------------------------------
    def expert_ffn(self, x: np.ndarray, x_dtype: int, k: int, fmt: int, E: int, hidden: int,
                   ffn: int, blobs: np.ndarray, offsets, pairs, active, pair_w=None, codebook=None):
        self._cb(codebook)
        x = np.ascontiguousarray(x)
        T = x.shape[0]
        blobs = np.ascontiguousarray(blobs, dtype=np.uint8)
        offsets = np.ascontiguousarray(offsets, dtype=np.int32)
        pairs = np.ascontiguousarray(pairs if len(pairs) else np.zeros(1, np.int32), dtype=np.int32)
        active = np.ascontiguousarray(active, dtype=np.int32)
        out = np.zeros((T * k, hidden), dtype=np.float64)
        pw = None
        if pair_w is not None:
            pw = np.ascontiguousarray(pair_w, dtype=np.float64).reshape(-1)
        rc = self.lib.orc_expert_ffn(_ptr(x), x_dtype, T, k, fmt, E, hidden, ffn, _ptr(blobs),
                                     _ptr(offsets, ctypes.c_int32), _ptr(pairs, ctypes.c_int32),
                                     _ptr(active, ctypes.c_int32),
                                     _ptr(pw) if pw is not None else None,
                                     _ptr(out, ctypes.c_double))
        if rc:
            raise ValueError(f"orc_expert_ffn rc={rc}")
        return out

    def layer_forward(self, x: np.ndarray, x_dtype: int, logits: np.ndarray, k: int, fmt: int,
                      ffn: int, routed: np.ndarray, shared: np.ndarray | None = None,
                      s_fmt: int | None = None, s_ffn: int | None = None, rows=None, codebook=None):
        """fmt / s_fmt: format codes of the routed / shared experts (a bit
        width 3, 4 or 20 (non-linear 4-bit), or gate/up bits | down bits << 8);
        codebook: the non-linear format's 16 int8 values (shared by both).
        Returns (y [n_rows, H] float64, idx [T,k] int32, w [T,k] float64)."""
        self._cb(codebook)
        x = np.ascontiguousarray(x)
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        T, E = logits.shape
        H = x.shape[1]
        routed = np.ascontiguousarray(routed, dtype=np.uint8)
        s_fmt = fmt if s_fmt is None else s_fmt
        s_ffn = ffn if s_ffn is None else s_ffn
        sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.uint8)
        rws = None
        nr = T
        if rows is not None:
            rws = np.ascontiguousarray(rows, dtype=np.int32)
            nr = rws.size
        y = np.zeros((nr, H), dtype=np.float64)
        idx = np.zeros((T, k), dtype=np.int32)
        w = np.zeros((T, k), dtype=np.float64)
        rc = self.lib.orc_layer_forward(_ptr(x), x_dtype, _ptr(logits), T, E, k, H, fmt, ffn,
                                        _ptr(routed), s_fmt, s_ffn,
                                        _ptr(sh) if sh is not None else None, nr,
                                        _ptr(rws) if rws is not None else None,
                                        _ptr(y, ctypes.c_double), _ptr(idx, ctypes.c_int32),
                                        _ptr(w, ctypes.c_double))
        if rc:
            raise ValueError(f"orc_layer_forward rc={rc}")
        return y, idx, w
