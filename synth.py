"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method (no packing, no quantization,
no dequantization and no dot products).  It draws fp32 weight matrices, fp32
or fp16 activations and random bytes from NumPy's PCG64 generator, and it
names the workload shapes.  Blocks are made from these draws either by the
CPU oracle (tests) or by the library's own GPU quantizer (bench).

Value distributions follow the workloads the pages discuss (Llama-7B-shaped
and Llama-3-8B-shaped layers quantized with the Q4_K_M recipe): weights drawn
from N(0, 0.02^2), optionally with 1 % of weights scaled by 10 (outliers),
activations from N(0, 1).
"""
from __future__ import annotations

import numpy as np


def weights(rows: int, cols: int, seed: int, std: float = 0.02,
            outlier_frac: float = 0.0, outlier_scale: float = 10.0) -> np.ndarray:
    """fp32 [rows, cols] ~ N(0, std^2); each weight independently, with
    probability ``outlier_frac``, is multiplied by ``outlier_scale``."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(std)
    if outlier_frac > 0.0:
        mask = rng.random((rows, cols), dtype=np.float32) < outlier_frac
        w[mask] *= np.float32(outlier_scale)
    return w


def activations(n_tok: int, cols: int, seed: int, dtype: str = "f32") -> np.ndarray:
    """[n_tok, cols] ~ N(0, 1) drawn in fp32; ``dtype='f16'`` rounds the draws
    to fp16 (round to nearest even, NumPy's conversion)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_tok, cols), dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype != "f32":
        raise ValueError(dtype)
    return x


def norm_weights(cols: int, seed: int) -> np.ndarray:
    """fp32 [cols] ~ N(1, 0.1^2): RMSNorm weights of a trained layer sit
    near one (the page's module initializes them to ones)."""
    rng = np.random.default_rng(seed)
    return (1.0 + 0.1 * rng.standard_normal(cols)).astype(np.float32)


def random_bytes(n: int, seed: int) -> np.ndarray:
    """Uniform random bytes (fuzz blobs: every bit pattern, NaN/Inf scales too)."""
    return np.random.default_rng(seed).integers(0, 256, size=n, dtype=np.uint8)


def dyadic(shape, seed: int, lo: int = -64, hi: int = 64, shift: int = 4) -> np.ndarray:
    """fp64 values k / 2^shift with integer k in [lo, hi): exact in every format."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=shape).astype(np.float64) / float(1 << shift)


# Workload shapes: (name, type, rows, cols).  rows = output features,
# cols = input features, as in nn.Linear.
SINGLE_Q4K_2048 = [("w", "q4_k", 2048, 2048)]

LLAMA7B_LAYER_Q4KM = [
    ("attn_q", "q4_k", 4096, 4096),
    ("attn_k", "q4_k", 4096, 4096),
    ("attn_v", "q4_k", 4096, 4096),
    ("attn_o", "q4_k", 4096, 4096),
    ("ffn_gate", "q4_k", 11008, 4096),
    ("ffn_up", "q4_k", 11008, 4096),
    ("ffn_down", "q6_k", 4096, 11008),
]

PER_TYPE_SWEEP_4096 = [
    ("q5_0", "q5_0", 4096, 4096),
    ("q6_k", "q6_k", 4096, 4096),
    ("q8_0", "q8_0", 4096, 4096),
    ("head", "q6_k", 32000, 4096),
]

GEMM_Q4K_11008 = [("ffn_up", "q4_k", 11008, 4096)]
GEMM_TOKENS = [1, 8, 64, 512]

LLAMA3_8B_LAYER_Q4KM = [
    ("attn_q", "q4_k", 4096, 4096),
    ("attn_k", "q4_k", 1024, 4096),
    ("attn_v", "q4_k", 1024, 4096),
    ("attn_o", "q4_k", 4096, 4096),
    ("ffn_gate", "q4_k", 14336, 4096),
    ("ffn_up", "q4_k", 14336, 4096),
    ("ffn_down", "q6_k", 4096, 14336),
    ("output", "q6_k", 128256, 4096),
]
LLAMA3_8B_TOKENS = [1, 8, 64]
