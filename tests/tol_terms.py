"""Terms of the error bounds the GPU paths meet on arbitrary blocks.

On blocks the quantizer makes (and on any scaling of weights or fp32
activations) every path meets the plain bar

    |y - y_ref| <= 1e-3 * sum_c |w^[r,c] x[t,c]|.

Two further terms appear on arbitrary bytes, each derived from the arithmetic
of a path:

  * factored Q4_K, Q5_K and Q2_K sums.  The batch-1 GEMV forms, per sub-block,
    a * sum(q x) - b * sum(x) (w = a q - b, Hitchhiker's Guide §11.2), and the
    weight-stream kernel d * P_k - dmin * P_m with P_k = sum((sc q) x) and
    P_m = sum(m x).  Each sum is rounded relative to its own magnitude, so the
    error is bounded by eps_f * F with F = sum_c (|a_c| q_c + |b_c|) |x_c|, not
    by sum |w x|: where a q and b nearly cancel, sum |w x| can be far below F.
    fp32 sums of at most 64 terms, the lane tree and the matrix-core
    accumulation give eps_f <= ~40 * 2^-24; the tests use 2^-16.
  * fp16 range in the matrix-core paths.  Operands are brought into fp16 by
    exact powers of two (per weight row in the tiled GEMM, from the largest
    bound U = the magnitude the block's fields allow; per token and slab or
    step for fp32 activations, from the largest |x|), so only values below
    2^-24 of the row's largest U (or of the token's largest |x|) fall into
    fp16's subnormal range, each with an absolute error <= 2^-34 U (or
    2^-34 max|x|).  The tests use 2^-30 (U_row sum|x| + max|x| sum|w|).

This module only reads block fields (layouts as stated for the oracle: R1, R2
for Q4_K) with NumPy; a CPU test checks that a q - b rebuilt here equals the
oracle's fp64 dequantization on random bytes.
"""
from __future__ import annotations

import numpy as np

QK = {"q4_0": 32, "q5_0": 32, "q8_0": 32, "q4_k": 256, "q6_k": 256, "q4_1": 32, "q5_k": 256,
      "q2_k": 256, "q3_k": 256}
BB = {"q4_0": 18, "q5_0": 22, "q8_0": 34, "q4_k": 144, "q6_k": 210, "q4_1": 20, "q5_k": 176,
      "q2_k": 84, "q3_k": 110}
FACTORED = ("q4_k", "q5_k", "q2_k")       # paths that sum a q and b apart
EPS_FACTORED = 2.0 ** -16
EPS_RANGE = 2.0 ** -30


def _f16(b2: np.ndarray) -> np.ndarray:
    """Little-endian fp16 fields (last axis of 2 bytes) as float64."""
    u = b2[..., 0].astype(np.uint16) | (b2[..., 1].astype(np.uint16) << 8)
    return u.view(np.float16).astype(np.float64)


def q4k_parts(blob: np.ndarray, rows: int, cols: int, t: str = "q4_k"):
    """Per weight (a, q, b) of Q4_K (or Q5_K, Q2_K) blocks with w = a q - b:
    a = d sc_i, b = dmin m_i (fp64), q the 4-bit (5-bit, 2-bit) code; arrays
    of shape [rows, cols].  Q5_K (R15): the fifth-bit plane at bytes 16..47,
    codes from byte 48.  Q2_K (R16): scale/min bytes 4..19 (low nibble scale,
    high nibble min, 16 weights each), 2-bit codes from byte 20, byte 8g+k
    holding elements 32g+k+8u at bits 2u."""
    nb = cols // 256
    if t == "q2_k":
        blk = blob.reshape(rows, nb, 84)
        d = _f16(blk[..., 0:2])
        dmin = _f16(blk[..., 2:4])
        sm = blk[..., 4:20].astype(np.int64)
        sc, mn = sm & 15, sm >> 4                                          # [rows, nb, 16]
        pl = blk[..., 20:84].reshape(rows, nb, 8, 8).astype(np.int64)      # [g][k]
        q = np.stack([(pl >> (2 * u)) & 3 for u in range(4)], axis=-2)    # [g][u][k]
        q = q.reshape(rows, nb, 256).astype(np.float64)                    # element 32g + 8u + k
        a = (d[..., None] * sc)[..., None] * np.ones(16)
        b = (dmin[..., None] * mn)[..., None] * np.ones(16)
        return a.reshape(rows, cols), q.reshape(rows, cols), b.reshape(rows, cols)
    q5 = (t == "q5_k")
    blk = blob.reshape(rows, nb, BB[t])
    d = _f16(blk[..., 0:2])
    dmin = _f16(blk[..., 2:4])
    bits = np.unpackbits(blk[..., 4:16], axis=-1, bitorder="little")      # 96 bits, LSB first
    fields = (bits.reshape(rows, nb, 16, 6).astype(np.int64) << np.arange(6)).sum(axis=-1)
    sc, mn = fields[..., 0::2], fields[..., 1::2]                          # [rows, nb, 8]
    o = 48 if q5 else 16
    qs = blk[..., o:o + 128].reshape(rows, nb, 8, 16)
    q = np.concatenate([qs & 15, qs >> 4], axis=-1).astype(np.float64)    # element k, k + 16
    if q5:
        hb = np.unpackbits(blk[..., 16:48], axis=-1, bitorder="little")   # bit e: element e
        q = q + 16.0 * hb.reshape(rows, nb, 8, 32)
    a = (d[..., None] * sc)[..., None] * np.ones(32)
    b = (dmin[..., None] * mn)[..., None] * np.ones(32)
    return a.reshape(rows, cols), q.reshape(rows, cols), b.reshape(rows, cols)


def row_bound(blob: np.ndarray, t: str, rows: int, cols: int) -> np.ndarray:
    """Per row, the largest block bound U (largest |w| the fields allow)."""
    blk = blob.reshape(rows, cols // QK[t], BB[t])
    d = np.abs(_f16(blk[..., 0:2]))
    if t == "q4_k":
        u = 945.0 * d + 63.0 * np.abs(_f16(blk[..., 2:4]))
    elif t == "q5_k":
        u = 1953.0 * d + 63.0 * np.abs(_f16(blk[..., 2:4]))
    elif t == "q4_1":
        u = 15.0 * d + np.abs(_f16(blk[..., 2:4]))
    elif t == "q2_k":
        u = 45.0 * d + 15.0 * np.abs(_f16(blk[..., 2:4]))
    else:
        u = {"q6_k": 4096.0, "q8_0": 128.0, "q4_0": 8.0, "q5_0": 16.0, "q3_k": 252.0}[t] * d
    return u.max(axis=1)


def tolerance(blob, t, rows, cols, x, yabs, w64):
    """The bound above for y [n, rows] against the oracle: yabs = sum |w x|
    from the oracle, w64 the oracle's fp64 dequantization [rows, cols]."""
    ax = np.abs(np.asarray(x, dtype=np.float64).reshape(-1, cols))
    tol = 1e-3 * yabs
    if t in FACTORED:
        a, q, b = q4k_parts(blob, rows, cols, t)
        tol = tol + EPS_FACTORED * (ax @ (np.abs(a) * q + np.abs(b)).T)
    u = row_bound(blob, t, rows, cols)
    tol = tol + EPS_RANGE * (ax.sum(axis=1)[:, None] * u[None, :]
                             + ax.max(axis=1)[:, None] * np.abs(w64).sum(axis=1)[None, :])
    return tol


def finite_scales(blob: np.ndarray, t: str) -> np.ndarray:
    """A copy of a (random-byte) blob whose fp16 scale fields are finite:
    an all-ones exponent (Inf / NaN) is lowered to 30."""
    out = blob.copy()
    blk = out.reshape(-1, BB[t])
    for off in ((0, 2) if t in ("q4_k", "q5_k", "q4_1", "q2_k") else (0,)):
        hi = blk[:, off + 1]
        bad = (hi & 0x7C) == 0x7C
        hi[bad] &= 0xFB                                   # exponent 31 -> 30
    return out
