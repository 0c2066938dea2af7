"""Decode attention over a q8_0 / q4_0 KV cache on the GPU (gq_attn_decode
through the C ABI) against the oracle.

Bar, carried from the per-dot-product bar to the output: every score
s_t = q . K^_t / sqrt(head_dim) is taken to be within
D_t = 1e-4 * sum_c |q_c K^_tc| / sqrt(head_dim) of the exact value (fp32
sums of 32 exact products and a short tree: actual error ~1e-6 of that
scale); a perturbation of at most D = max_t D_t moves each softmax weight by
a factor within [e^-2D, e^2D], so
    |out - out_ref| <= (1e-3 + e^(2D) - 1) * sum_t p_t |V^_t|
per output, the 1e-3 covering the fp32 exponentials and weighted sums.
Inputs: K and V rows drawn N(0, 1) and quantized by the oracle's quantizer
(cache entries are activations of order one), q ~ N(0, 1), optionally
scaled up to make the softmax sharp.
"""
import os
import sys

import numpy as np
import pytest
import torch

import gguf_quant_matmul_amd as gq
import oracle
import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_cache(t, kv_len, n_kv, head_dim, seed):
    rows = kv_len * n_kv
    k = synth.activations(rows, head_dim, seed=seed)
    v = synth.activations(rows, head_dim, seed=seed + 1)
    return oracle.quantize(k, t), oracle.quantize(v, t)


def reference(kb, vb, t, kv_len, n_kv, head_dim, q):
    """Oracle output and the bound above."""
    out = oracle.attn_decode_f64(kb, vb, t, kv_len, n_kv, head_dim, q)
    n_heads = q.shape[0]
    n_rep = n_heads // n_kv
    kd = oracle.dequant_f64(kb, t, kv_len * n_kv, head_dim).reshape(kv_len, n_kv, head_dim)
    vd = oracle.dequant_f64(vb, t, kv_len * n_kv, head_dim).reshape(kv_len, n_kv, head_dim)
    tol = np.empty_like(out)
    scale = 1.0 / np.sqrt(head_dim)
    for h in range(n_heads):
        g = h // n_rep
        s = kd[:, g, :] @ q[h] * scale
        dmax = 1e-4 * float(np.max(np.abs(kd[:, g, :]) @ np.abs(q[h]))) * scale
        p = np.exp(s - s.max())
        p /= p.sum()
        tol[h] = (1e-3 + np.expm1(2 * dmax)) * (p @ np.abs(vd[:, g, :]))
    return out, tol


def run(kb, vb, t, kv_len, n_kv, head_dim, q):
    kd, vd = torch.from_numpy(kb).cuda(), torch.from_numpy(vb).cuda()
    out = gq.attn_decode(kd, vd, t, kv_len, n_kv, head_dim, torch.from_numpy(q.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHAPES = [("q8_0", 1, 2, 4, 128, 1.0),       # one position: the value row
          ("q8_0", 37, 4, 8, 64, 1.0),       # one ragged chunk
          ("q4_0", 300, 8, 40, 128, 1.0),    # 5 query heads per KV head
          ("q8_0", 1000, 2, 32, 128, 1.0),   # 16 query heads per KV head, several chunks
          ("q4_0", 129, 1, 3, 256, 1.0),     # head_dim 256
          ("q8_0", 5000, 8, 64, 128, 8.0),   # sharp softmax across many chunks
          ("q4_0", 4097, 8, 32, 64, 4.0),
          ("q8_0", 700, 4, 4, 128, 1.0),     # one query head per KV head
          ("q4_0", 2048, 8, 16, 128, 2.0),   # whole chunks only, 2 heads per KV head
          ("q8_0", 513, 2, 32, 256, 1.0),    # head_dim 256, 16 heads per KV head
          ("q8_0", 8192, 1, 8, 128, 1.0),    # one KV head, 8 query heads, 128 whole chunks
          ("q8_0", 32868, 8, 40, 128, 1.0),  # 129 chunks per KV head, the last ragged
          ("q4_0", 16400, 16, 32, 128, 2.0)]  # 65 chunks x 16 KV heads


@pytest.mark.parametrize("t,kv_len,n_kv,n_heads,head_dim,qs", SHAPES)
def test_attn_decode_parity(t, kv_len, n_kv, n_heads, head_dim, qs):
    say(f"attn {t} kv_len={kv_len} n_kv={n_kv} n_heads={n_heads} head_dim={head_dim} q x{qs}")
    kb, vb = make_cache(t, kv_len, n_kv, head_dim, seed=kv_len + head_dim)
    q = synth.activations(n_heads, head_dim, seed=kv_len + 7).astype(np.float64) * qs
    q = q.astype(np.float32).astype(np.float64)
    got = run(kb, vb, t, kv_len, n_kv, head_dim, q)
    ref, tol = reference(kb, vb, t, kv_len, n_kv, head_dim, q)
    err = np.abs(got - ref)
    say(f"  max |err| / bound = {float(np.max(err / np.maximum(tol, 1e-300))):.3e}")
    assert np.all(err <= tol), f"{int((err > tol).sum())} outputs beyond the bound"


@pytest.mark.parametrize("t", ["q8_0", "q4_0"])
def test_attn_decode_full_size(t):
    """The measured workload: 32k cached positions, 8 KV heads, 40 query
    heads, head_dim 128 (the 30B-class cache of the Hitchhiker's Guide
    §13.2), every output against the oracle; two runs are bit-identical."""
    kv_len, n_kv, n_heads, hd = 32768, 8, 40, 128
    say(f"attn full size {t}")
    kb, vb = make_cache(t, kv_len, n_kv, hd, seed=31)
    q = synth.activations(n_heads, hd, seed=32).astype(np.float64)
    a = run(kb, vb, t, kv_len, n_kv, hd, q)
    b = run(kb, vb, t, kv_len, n_kv, hd, q)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ref, tol = reference(kb, vb, t, kv_len, n_kv, hd, q)
    err = np.abs(a - ref)
    say(f"  max |err| / bound = {float(np.max(err / np.maximum(tol, 1e-300))):.3e}")
    assert np.all(err <= tol)


def test_attn_decode_closed_forms():
    """Values constant per KV head (g + 1, as quantized) come back unchanged
    for any query, selecting KV head h // n_rep for query head h; a zero
    query gives the mean of the value rows."""
    kv_len, n_kv, n_heads, hd = 777, 4, 16, 128
    rb = gq.row_bytes("q8_0", hd)
    kb, _ = make_cache("q8_0", kv_len, n_kv, hd, seed=5)
    vals = np.array([[g + 1.0] * hd for _ in range(kv_len) for g in range(n_kv)], dtype=np.float32)
    vb = oracle.quantize(vals, "q8_0")
    q = synth.activations(n_heads, hd, seed=6).astype(np.float64)
    got = run(kb, vb, "q8_0", kv_len, n_kv, hd, q)
    vd = oracle.dequant_f64(vb, "q8_0", kv_len * n_kv, hd).reshape(kv_len, n_kv, hd)
    want = vd[0][np.arange(n_heads) // (n_heads // n_kv)]      # ~ g + 1, as quantized
    assert np.allclose(got, want, rtol=1e-4, atol=0)
    _, vb2 = make_cache("q8_0", kv_len, n_kv, hd, seed=9)
    got = run(kb, vb2, "q8_0", kv_len, n_kv, hd, np.zeros((n_heads, hd)))
    vd = oracle.dequant_f64(vb2, "q8_0", kv_len * n_kv, hd).reshape(kv_len, n_kv, hd)
    want = vd.mean(axis=0)[np.arange(n_heads) // (n_heads // n_kv)]
    assert np.allclose(got, want, rtol=0, atol=1e-5 * float(np.abs(vd).max()))
    assert rb == 136
