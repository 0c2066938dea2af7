"""gguf_quant_matmul_amd — GGUF block-quantized GEMV / matmul on MI355X.

Thin Python binding over the C ABI of ``libgq.so`` (see ``include/gq.h``):
argument marshalling only.  Every step of the computation runs in the HIP
kernels of the library; PyTorch supplies device memory and the current HIP
stream.  Importing this package does not load the library; the first call
does, and raises if ``libgq.so`` has not been built (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgq.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "gq.h")

F32, F16, Q4_0, Q5_0, Q8_0, Q4_K, Q6_K, Q4_1, Q5_K, Q2_K, Q3_K = range(11)
TYPES = {"f32": F32, "f16": F16, "q4_0": Q4_0, "q5_0": Q5_0, "q8_0": Q8_0,
         "q4_k": Q4_K, "q6_k": Q6_K, "q4_1": Q4_1, "q5_k": Q5_K, "q2_k": Q2_K, "q3_k": Q3_K}
QUANT_TYPES = ["q4_0", "q5_0", "q8_0", "q4_k", "q6_k", "q4_1", "q5_k", "q2_k", "q3_k"]

_lib = None


class GQError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code})")


def lib():
    """The loaded libgq.so (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m gguf_quant_matmul_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.gq_type_info.argtypes = [ci, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.gq_type_info.restype = ci
        L.gq_row_bytes.argtypes = [ci, i64]
        L.gq_row_bytes.restype = i64
        L.gq_strerror.argtypes = [ci]
        L.gq_strerror.restype = ctypes.c_char_p
        L.gq_matmul.argtypes = [vp, ci, i64, i64, vp, vp, i64, vp]
        L.gq_matmul.restype = ci
        L.gq_matmul_ex.argtypes = [vp, ci, i64, i64, vp, ci, vp, i64, vp]
        L.gq_matmul_ex.restype = ci
        L.gq_matmul_path.argtypes = [vp, ci, i64, i64, vp, ci, vp, i64, ci, vp]
        L.gq_matmul_path.restype = ci
        L.gq_matmul_decode.argtypes = [vp, vp, ci, i64, i64, vp, ci, vp, ctypes.c_float, vp, vp]
        L.gq_matmul_decode.restype = ci
        L.gq_attn_decode_workspace_bytes.argtypes = [i64, ci, ci, ci]
        L.gq_attn_decode_workspace_bytes.restype = i64
        L.gq_attn_decode.argtypes = [vp, vp, ci, i64, ci, ci, vp, ci, vp, vp, i64, vp]
        L.gq_attn_decode.restype = ci
        L.gq_attn_decode_noalloc.argtypes = [vp, vp, ci, i64, ci, ci, vp, ci, vp, vp]
        L.gq_attn_decode_noalloc.restype = ci
        L.gq_probe_stream_read.argtypes = [vp, i64, vp, vp]
        L.gq_probe_stream_read.restype = ci
        L.gq_dequant.argtypes = [vp, ci, i64, i64, vp, ci, vp]
        L.gq_dequant.restype = ci
        L.gq_quantize.argtypes = [vp, ci, i64, i64, vp, vp]
        L.gq_quantize.restype = ci
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Names of the functions declared in include/gq.h."""
    with open(HEADER) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(gq_\w+)\s*\(", text, re.M)))


def _tid(t) -> int:
    if isinstance(t, str):
        if t not in TYPES:
            raise ValueError(f"unknown type {t!r}")
        return TYPES[t]
    return int(t)


def strerror(code: int) -> str:
    return lib().gq_strerror(int(code)).decode()


def type_info(t):
    qk, bb = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().gq_type_info(_tid(t), ctypes.byref(qk), ctypes.byref(bb))
    if rc:
        raise GQError(rc, "gq_type_info")
    return qk.value, bb.value


def row_bytes(t, cols: int) -> int:
    r = lib().gq_row_bytes(_tid(t), int(cols))
    if r < 0:
        raise GQError(int(r), "gq_row_bytes")
    return int(r)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


PATH_AUTO, PATH_GEMV, PATH_WEIGHT_STREAM, PATH_TILED = range(4)


def matmul(blob, t, rows: int, cols: int, x, out=None, stream=None, path: int = PATH_AUTO):
    """y[n, rows] = W^ x for x [n, cols] (fp32 or fp16, CUDA).  fp32 result.
    path: the kernel family (gq_matmul_path); PATH_AUTO chooses."""
    import torch
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dtype not in (torch.float32, torch.float16):
        raise TypeError("x must be float32 or float16")
    x = x.contiguous()
    n = x.shape[0]
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=x.device)
    xt = F16 if x.dtype == torch.float16 else F32
    rc = lib().gq_matmul_path(blob.data_ptr(), _tid(t), rows, cols, x.data_ptr(), xt,
                              out.data_ptr(), n, int(path), _stream(stream))
    if rc:
        raise GQError(rc, "gq_matmul_path")
    return out


def matmul_decode(blob, t, rows: int, cols: int, x, up=None, norm_weight=None, eps: float = 1e-5,
                  out=None, stream=None):
    """One token: y[rows] = W^ RMSNorm(x) (norm_weight given) or W^ x, or with
    `up` (a second blob of the same type and shape) silu(W^ xin) * (U^ xin)."""
    import torch
    x = x.reshape(-1)
    if x.dtype not in (torch.float32, torch.float16):
        raise TypeError("x must be float32 or float16")
    x = x.contiguous()
    if norm_weight is not None:
        if norm_weight.dtype != torch.float32:
            raise TypeError("norm_weight must be float32")
        norm_weight = norm_weight.contiguous()
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=x.device)
    xt = F16 if x.dtype == torch.float16 else F32
    rc = lib().gq_matmul_decode(blob.data_ptr(), None if up is None else up.data_ptr(), _tid(t),
                                rows, cols, x.data_ptr(), xt,
                                None if norm_weight is None else norm_weight.data_ptr(),
                                float(eps), out.data_ptr(), _stream(stream))
    if rc:
        raise GQError(rc, "gq_matmul_decode")
    return out


def attn_decode_workspace_bytes(kv_len: int, n_kv_heads: int, n_heads: int, head_dim: int) -> int:
    n = lib().gq_attn_decode_workspace_bytes(kv_len, n_kv_heads, n_heads, head_dim)
    if n < 0:
        raise GQError(int(n), "gq_attn_decode_workspace_bytes")
    return int(n)


def attn_decode(k_cache, v_cache, t, kv_len: int, n_kv_heads: int, head_dim: int, q,
                out=None, workspace=None, stream=None):
    """One decode step of GQA attention over q8_0 / q4_0 K and V caches
    (uint8 CUDA blobs, [kv_len][n_kv_heads][head_dim] rows); q fp32
    [n_heads, head_dim].  Returns out fp32 [n_heads, head_dim]."""
    import torch
    if q.dtype != torch.float32:
        raise TypeError("q must be float32")
    q = q.contiguous()
    n_heads = q.shape[0]
    need = attn_decode_workspace_bytes(kv_len, n_kv_heads, n_heads, head_dim)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((n_heads, head_dim), dtype=torch.float32, device=q.device)
    rc = lib().gq_attn_decode(k_cache.data_ptr(), v_cache.data_ptr(), _tid(t), kv_len,
                              n_kv_heads, head_dim, q.data_ptr(), n_heads, out.data_ptr(),
                              workspace.data_ptr(), workspace.numel(), _stream(stream))
    if rc:
        raise GQError(rc, "gq_attn_decode")
    return out


def attn_decode_noalloc(k_cache, v_cache, t, kv_len: int, n_kv_heads: int, head_dim: int, q,
                        out, stream=None):
    """attn_decode through gq_attn_decode_noalloc: the library's fixed
    device array serves as workspace; out (fp32 [n_heads, head_dim], CUDA)
    is given by the caller, so the call itself allocates nothing."""
    import torch
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise TypeError("q must be contiguous float32")
    rc = lib().gq_attn_decode_noalloc(k_cache.data_ptr(), v_cache.data_ptr(), _tid(t), kv_len,
                                      n_kv_heads, head_dim, q.data_ptr(), q.shape[0],
                                      out.data_ptr(), _stream(stream))
    if rc:
        raise GQError(rc, "gq_attn_decode_noalloc")
    return out


PROBE_OUT_WORDS = 2048


def probe_stream_read(buf, out=None, stream=None):
    """Streaming read of a contiguous CUDA tensor's bytes (the measured
    bandwidth ceiling); returns the int32 tensor of per-workgroup XORs."""
    import torch
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if out is None:
        out = torch.empty(PROBE_OUT_WORDS, dtype=torch.int32, device=buf.device)
    rc = lib().gq_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                    out.data_ptr(), _stream(stream))
    if rc:
        raise GQError(rc, "gq_probe_stream_read")
    return out


def dequant(blob, t, rows: int, cols: int, dtype=None, out=None, stream=None):
    """Dequantized weights [rows, cols] as fp32 (default) or fp16 (RNE)."""
    import torch
    dtype = dtype or torch.float32
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=blob.device)
    ot = F16 if out.dtype == torch.float16 else F32
    rc = lib().gq_dequant(blob.data_ptr(), _tid(t), rows, cols, out.data_ptr(), ot,
                          _stream(stream))
    if rc:
        raise GQError(rc, "gq_dequant")
    return out


def quantize(w, t, out=None, stream=None):
    """Blob (uint8, CUDA) of fp32 weights w [rows, cols] quantized on the GPU."""
    import torch
    w = w.contiguous()
    if w.dtype != torch.float32:
        raise TypeError("w must be float32")
    rows, cols = w.shape
    if out is None:
        out = torch.empty(rows * row_bytes(t, cols), dtype=torch.uint8, device=w.device)
    rc = lib().gq_quantize(w.data_ptr(), _tid(t), rows, cols, out.data_ptr(), _stream(stream))
    if rc:
        raise GQError(rc, "gq_quantize")
    return out
