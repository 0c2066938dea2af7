"""GPU parity at the full workload sizes, in the launch configurations the
bench times, checked on sampled output rows (all tokens) against the oracle.

Workloads (shapes as rows x cols, rows = output features):
  * a single Q4_K GEMV at 2048 x 2048 (checked in full);
  * a Llama-7B-shaped decode layer in the Q4_K_M mix at batch 1;
  * a per-type sweep at 4096 x 4096 (Q5_0, Q6_K, Q8_0, 1 % outliers at 10x)
    plus a 32000 x 4096 Q6_K output head, and Q4_1 and Q5_K at 4096 x 4096
    at 1, 8, 64 and 512 tokens;
  * Q4_K 11008 x 4096 with fp16 activations at 1, 8, 64 and 512 tokens;
  * a Llama-3-8B-shaped layer set at 1, 8 and 64 tokens, with the
    128256 x 4096 Q6_K head.
"""
import functools

import numpy as np
import pytest
import torch

import gguf_quant_matmul_amd as gq
import oracle
import synth
from test_gpu_parity import check_matmul, say, to_dev

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def blob_for(t, rows, cols, seed, outliers):
    w = synth.weights(rows, cols, seed=seed, outlier_frac=outliers)
    b = oracle.quantize(w, t)
    del w
    return b


def sample_rows(rows, k=384, seed=0):
    rng = np.random.default_rng(seed)
    mid = rng.choice(rows, size=min(k, rows), replace=False)
    edge = np.r_[0:min(32, rows), max(0, rows - 32):rows]
    return np.unique(np.concatenate([mid, edge]))


def run_case(t, rows, cols, n, xdt, seed, outliers=0.0, full=False):
    say(f"fullsize {t} {rows}x{cols} n={n} x={xdt}")
    blob = blob_for(t, rows, cols, seed, outliers)
    bd = to_dev(blob)
    x = synth.activations(n, cols, seed=seed + 1, dtype=xdt)
    y = gq.matmul(bd, t, rows, cols, to_dev(x)).cpu().numpy()
    del bd
    idx = None if full else sample_rows(rows, seed=seed)
    return check_matmul(y, blob, t, rows, cols, x, rows_idx=idx, label=f"{t} {rows}x{cols} n={n}")


def test_single_q4k_2048():
    run_case("q4_k", 2048, 2048, 1, "f32", seed=1000, full=True)


@pytest.mark.parametrize("name,t,rows,cols", synth.LLAMA7B_LAYER_Q4KM[3:])
def test_llama7b_layer_batch1(name, t, rows, cols):
    run_case(t, rows, cols, 1, "f32", seed=2000 + rows + cols)


@pytest.mark.parametrize("name,t,rows,cols", synth.PER_TYPE_SWEEP_4096)
def test_per_type_sweep(name, t, rows, cols):
    run_case(t, rows, cols, 1, "f32", seed=3000 + rows, outliers=0.01)


@pytest.mark.parametrize("n", synth.GEMM_TOKENS)
def test_q4k_11008_fp16_tokens(n):
    run_case("q4_k", 11008, 4096, n, "f16", seed=4000)


@pytest.mark.parametrize("name,t,rows,cols", synth.LLAMA3_8B_LAYER_Q4KM)
def test_llama3_8b_layer(name, t, rows, cols):
    for n in synth.LLAMA3_8B_TOKENS:
        run_case(t, rows, cols, n, "f32" if n == 1 else "f16", seed=5000 + rows + cols)


@pytest.mark.parametrize("t", ["q4_1", "q5_k", "q2_k", "q3_k"])
def test_new_types_4096(t):
    """The block types beyond the Q4_K_M recipe at a full 4096 x 4096 size,
    through the GEMV (fp32 x) and the batched paths (fp16 x)."""
    for n in synth.GEMM_TOKENS:
        run_case(t, 4096, 4096, n, "f32" if n == 1 else "f16", seed=6000, outliers=0.01)
