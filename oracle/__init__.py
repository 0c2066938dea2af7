"""CPU oracle for GGUF block-quantized matmul — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it and
shares no code with it.

This module is argument marshalling around ``gqo.c`` (plain C, fp64), built
with gcc into ``oracle/_build/libgqo.so``.  The formats, the dequantization
order and the readings taken where the pages are silent are documented at the
top of ``gqo.c``.  ``Oracle(plant=k)`` loads a separate build with deliberate
mistake k compiled in; it exists only for the tests that show the pins reject
such mistakes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqo.c")
_BUILD = os.path.join(_HERE, "_build")

# This project's own type numbering (the pages give none).
TYPES = {"f32": 0, "f16": 1, "q4_0": 2, "q5_0": 3, "q8_0": 4, "q4_k": 5, "q6_k": 6,
         "q4_1": 7, "q5_k": 8, "q2_k": 9, "q3_k": 10}
QUANT_TYPES = ["q4_0", "q5_0", "q8_0", "q4_k", "q6_k", "q4_1", "q5_k", "q2_k", "q3_k"]


def _lib_path(plant: int) -> str:
    return os.path.join(_BUILD, "libgqo.so" if plant == 0 else f"libgqo_plant{plant}.so")


def build(force: bool = True, plant: int = 0) -> str:
    """Compile gqo.c with gcc (-O2, OpenMP, no FP contraction, no fast-math)."""
    os.makedirs(_BUILD, exist_ok=True)
    lib = _lib_path(plant)
    if force or not os.path.exists(lib):
        tmp = lib + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wno-unused-function",
               f"-DGQO_PLANT={int(plant)}", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


def _tid(t) -> int:
    if isinstance(t, str):
        if t not in TYPES:
            raise ValueError(f"unknown type {t!r}")
        return TYPES[t]
    return int(t)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    def __init__(self, plant: int = 0):
        path = _lib_path(plant)
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(force=True, plant=plant)
        lib = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.gqo_block_info.argtypes = [ci, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.gqo_half_to_double.argtypes = [ctypes.c_uint16]
        lib.gqo_half_to_double.restype = ctypes.c_double
        lib.gqo_half_up.argtypes = [ctypes.c_double]
        lib.gqo_half_up.restype = ctypes.c_uint16
        lib.gqo_half_rne.argtypes = [ctypes.c_float]
        lib.gqo_half_rne.restype = ctypes.c_uint16
        lib.gqo_quantize.argtypes = [ci, vp, i64, i64, vp]
        lib.gqo_dequant_f32.argtypes = [ci, vp, i64, i64, vp]
        lib.gqo_dequant_f64.argtypes = [ci, vp, i64, i64, vp]
        lib.gqo_matmul_f64.argtypes = [ci, vp, i64, i64, vp, i64, vp, vp, ci]
        lib.gqo_rmsnorm_f64.argtypes = [vp, i64, vp, ctypes.c_double, ci, vp]
        lib.gqo_swiglu_f64.argtypes = [vp, vp, i64, vp]
        lib.gqo_attn_decode_f64.argtypes = [ci, vp, vp, i64, i64, i64, vp, i64, vp]
        self.lib = lib
        self.plant = plant

    def block_info(self, t):
        """(weights per block, bytes per block)."""
        qk, bb = ctypes.c_int64(), ctypes.c_int64()
        if self.lib.gqo_block_info(_tid(t), ctypes.byref(qk), ctypes.byref(bb)) != 0:
            raise ValueError(f"unknown type {t!r}")
        return qk.value, bb.value

    def row_bytes(self, t, cols: int) -> int:
        qk, bb = self.block_info(t)
        if cols % qk:
            raise ValueError("cols must be a multiple of the block size")
        return cols // qk * bb

    def half_to_double(self, h: int) -> float:
        return self.lib.gqo_half_to_double(h)

    def half_up(self, v: float) -> int:
        return self.lib.gqo_half_up(v)

    def half_rne(self, f: float) -> int:
        return self.lib.gqo_half_rne(f)

    def quantize(self, w: np.ndarray, t) -> np.ndarray:
        """Quantize fp32 w[rows, cols] into a flat uint8 blob (row-major blocks)."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        rows, cols = w.shape
        blob = np.zeros(rows * self.row_bytes(t, cols), dtype=np.uint8)
        rc = self.lib.gqo_quantize(_tid(t), _ptr(w), rows, cols, _ptr(blob))
        if rc:
            raise ValueError(f"gqo_quantize failed ({rc})")
        return blob

    def _blob(self, blob, t, rows, cols):
        blob = np.ascontiguousarray(blob, dtype=np.uint8)
        if blob.size < rows * self.row_bytes(t, cols):
            raise ValueError("blob too small")
        return blob

    def dequant_f32(self, blob: np.ndarray, t, rows: int, cols: int) -> np.ndarray:
        blob = self._blob(blob, t, rows, cols)
        out = np.empty((rows, cols), dtype=np.float32)
        rc = self.lib.gqo_dequant_f32(_tid(t), _ptr(blob), rows, cols, _ptr(out))
        if rc:
            raise ValueError(f"gqo_dequant_f32 failed ({rc})")
        return out

    def dequant_f64(self, blob: np.ndarray, t, rows: int, cols: int) -> np.ndarray:
        blob = self._blob(blob, t, rows, cols)
        out = np.empty((rows, cols), dtype=np.float64)
        rc = self.lib.gqo_dequant_f64(_tid(t), _ptr(blob), rows, cols, _ptr(out))
        if rc:
            raise ValueError(f"gqo_dequant_f64 failed ({rc})")
        return out

    def matmul_f64(self, blob: np.ndarray, t, rows: int, cols: int, x: np.ndarray,
                   threads: int = 1):
        """Return (y, yabs), both float64 [n_tok, rows]: y = W^ x, yabs = sum |w*x|.

        x is [n_tok, cols] of any float dtype; it is widened exactly to fp64."""
        blob = self._blob(blob, t, rows, cols)
        x = np.ascontiguousarray(np.atleast_2d(x).astype(np.float64))
        if x.shape[1] != cols:
            raise ValueError("x has the wrong number of columns")
        n = x.shape[0]
        y = np.empty((n, rows), dtype=np.float64)
        yabs = np.empty((n, rows), dtype=np.float64)
        rc = self.lib.gqo_matmul_f64(_tid(t), _ptr(blob), rows, cols, _ptr(x), n,
                                     _ptr(y), _ptr(yabs), int(threads))
        if rc:
            raise ValueError(f"gqo_matmul_f64 failed ({rc})")
        return y, yabs


    def rmsnorm_f64(self, x: np.ndarray, w: np.ndarray, eps: float, half_x: bool = False):
        """RMSNorm of the vector x with weights w (fp64; see gqo.h)."""
        x = np.ascontiguousarray(np.asarray(x).reshape(-1).astype(np.float64))
        w = np.ascontiguousarray(np.asarray(w).reshape(-1).astype(np.float64))
        if w.size != x.size:
            raise ValueError("x and w differ in length")
        out = np.empty_like(x)
        rc = self.lib.gqo_rmsnorm_f64(_ptr(x), x.size, _ptr(w), float(eps), int(bool(half_x)), _ptr(out))
        if rc:
            raise ValueError(f"gqo_rmsnorm_f64 failed ({rc})")
        return out

    def swiglu_f64(self, g: np.ndarray, u: np.ndarray):
        """silu(g) * u elementwise (fp64)."""
        g = np.ascontiguousarray(np.asarray(g, dtype=np.float64))
        u = np.ascontiguousarray(np.asarray(u, dtype=np.float64))
        if g.shape != u.shape:
            raise ValueError("g and u differ in shape")
        out = np.empty_like(g)
        rc = self.lib.gqo_swiglu_f64(_ptr(g), _ptr(u), g.size, _ptr(out))
        if rc:
            raise ValueError(f"gqo_swiglu_f64 failed ({rc})")
        return out


    def attn_decode_f64(self, k_cache: np.ndarray, v_cache: np.ndarray, t, kv_len: int,
                        n_kv: int, head_dim: int, q: np.ndarray) -> np.ndarray:
        """Decode-step GQA attention over quantized K/V caches (fp64; see gqo.h).
        q: [n_heads][head_dim]; returns [n_heads][head_dim]."""
        q = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
        n_heads = q.shape[0]
        rb = self.row_bytes(t, head_dim)
        for c in (k_cache, v_cache):
            if c.size != kv_len * n_kv * rb:
                raise ValueError("cache size does not match kv_len * n_kv rows")
        out = np.empty((n_heads, head_dim), dtype=np.float64)
        rc = self.lib.gqo_attn_decode_f64(_tid(t), _ptr(np.ascontiguousarray(k_cache)),
                                          _ptr(np.ascontiguousarray(v_cache)), kv_len, n_kv,
                                          head_dim, _ptr(q), n_heads, _ptr(out))
        if rc:
            raise ValueError(f"gqo_attn_decode_f64 failed ({rc})")
        return out


_default = None


def _load() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(0)
    return _default


def block_info(t):
    return _load().block_info(t)


def row_bytes(t, cols):
    return _load().row_bytes(t, cols)


def half_to_double(h):
    return _load().half_to_double(h)


def half_up(v):
    return _load().half_up(v)


def half_rne(f):
    return _load().half_rne(f)


def quantize(w, t):
    return _load().quantize(w, t)


def dequant_f32(blob, t, rows, cols):
    return _load().dequant_f32(blob, t, rows, cols)


def dequant_f64(blob, t, rows, cols):
    return _load().dequant_f64(blob, t, rows, cols)


def matmul_f64(blob, t, rows, cols, x, threads=1):
    return _load().matmul_f64(blob, t, rows, cols, x, threads)


def rmsnorm_f64(x, w, eps, half_x=False):
    return _load().rmsnorm_f64(x, w, eps, half_x)


def swiglu_f64(g, u):
    return _load().swiglu_f64(g, u)


def attn_decode_f64(k_cache, v_cache, t, kv_len, n_kv, head_dim, q):
    return _load().attn_decode_f64(k_cache, v_cache, t, kv_len, n_kv, head_dim, q)
