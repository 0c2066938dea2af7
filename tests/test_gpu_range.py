"""GPU parity at the edges of the number formats, on every kernel path.

  * fp32 activations scaled by 2^-30, 2^-20 and 2^20 (and per token by
    2^-40 .. 2^40) at 2, 40, 130 and 512 tokens through the weight-stream
    kernel, the tiled GEMM and the automatic choice, and at one token through
    the GEMV: the plain bar |y - y_ref| <= 1e-3 sum |w x| (the matrix-core
    paths bring fp32 x into fp16 range by exact powers of two);
  * blobs quantized from weights scaled by 2^-16 and 2^20 (block scales
    near the fp16 subnormal range and near its top): the plain bar on every
    path and both activation types;
  * random-byte blobs with finite scales, and blocks built so that a q and b
    (w = a q - b, Hitchhiker's Guide §11.2) cancel exactly or nearly: the
    bound of tests/tol_terms.py (the plain bar plus the factored-sum and
    fp16-range terms derived there), on every path and the fused decode call;
  * the decode attention with fp32 queries scaled by 2^-20 and 2^20, and
    with query heads of one KV head 2^40 apart.
"""
import os
import sys

import numpy as np
import pytest
import torch

import gguf_quant_matmul_amd as gq
import oracle
import synth
import tol_terms

pytestmark = pytest.mark.gpu

QK = tol_terms.QK
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
SHAPES = {"q4_k": (75, 768), "q6_k": (70, 768), "q8_0": (75, 352), "q5_0": (75, 288),
          "q4_0": (75, 320), "q4_1": (75, 352), "q5_k": (70, 768), "q2_k": (70, 768),
          "q3_k": (70, 768)}
BATCH_PATHS = [("auto", gq.PATH_AUTO), ("stream", gq.PATH_WEIGHT_STREAM),
               ("tiled", gq.PATH_TILED)]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda:0"))


def run(bd, t, rows, cols, x, path):
    return gq.matmul(bd, t, rows, cols, to_dev(x), path=path).cpu().numpy().astype(np.float64)


def check_plain(y, ref, rabs, label):
    err = np.abs(y - ref)
    ratio = float(np.max(err / np.maximum(rabs, 1e-300)))
    say(f"  {label}: max |err| / sum|w x| = {ratio:.3e}")
    bad = ~(err <= 1e-3 * rabs)
    assert not bad.any(), f"{label}: {int(bad.sum())} outputs beyond 1e-3 sum|w x| (worst {ratio:.3e})"


def check_bound(y, ref, tol, label):
    err = np.abs(y - ref)
    ratio = float(np.max(err / np.maximum(tol, 1e-300)))
    say(f"  {label}: max |err| / bound = {ratio:.3e}")
    bad = ~(err <= tol)
    assert not bad.any(), f"{label}: {int(bad.sum())} outputs beyond the bound (worst {ratio:.3e})"


def every_path(t, n):
    """(label, path) pairs that accept n tokens."""
    if n == 1:
        return [("gemv", gq.PATH_GEMV)]
    return BATCH_PATHS


# ---------------------------------------------------------------- scaled fp32 activations

@pytest.mark.parametrize("t", gq.QUANT_TYPES)
def test_fp32_x_scaled_every_path(t):
    rows, cols = SHAPES[t]
    blob = oracle.quantize(synth.weights(rows, cols, seed=700), t)
    bd = to_dev(blob)
    for n in (1, 2, 40, 130, 512):
        x0 = synth.activations(n, cols, seed=701 + n)
        ref0, abs0 = oracle.matmul_f64(blob, t, rows, cols, x0, threads=THREADS)
        for e in (-30, -20, 20):
            x = (x0 * np.float32(2.0 ** e)).astype(np.float32)
            ref, rabs = ref0 * 2.0 ** e, abs0 * 2.0 ** e     # exact: power-of-two scaling
            for label, path in every_path(t, n):
                say(f"scaled x {t} {rows}x{cols} n={n} x*2^{e} {label}")
                check_plain(run(bd, t, rows, cols, x, path), ref, rabs, f"{t} n={n} 2^{e} {label}")


@pytest.mark.parametrize("t", gq.QUANT_TYPES)
def test_fp32_x_scale_per_token(t):
    """Tokens of one call scaled by 2^-40 .. 2^40: each token's own scale."""
    rows, cols = SHAPES[t]
    blob = oracle.quantize(synth.weights(rows, cols, seed=710), t)
    bd = to_dev(blob)
    for n in (9, 40, 130):
        e = np.array([(-40, -20, 0, 20, 40, -33, 17)[i % 7] for i in range(n)], dtype=np.float64)
        x = (synth.activations(n, cols, seed=711 + n) * (2.0 ** e)[:, None]).astype(np.float32)
        ref, rabs = oracle.matmul_f64(blob, t, rows, cols, x, threads=THREADS)
        for label, path in BATCH_PATHS:
            say(f"per-token scaled x {t} n={n} {label}")
            check_plain(run(bd, t, rows, cols, x, path), ref, rabs, f"{t} n={n} {label}")


# ---------------------------------------------------------------- scaled blocks

@pytest.mark.parametrize("t", gq.QUANT_TYPES)
@pytest.mark.parametrize("e", [-16, 20])
def test_scaled_blocks_every_path(t, e):
    """Weights scaled by 2^e before quantization: block scales near fp16's
    subnormal range (2^-16) or near its top (2^20)."""
    rows, cols = SHAPES[t]
    w = synth.weights(rows, cols, seed=720) * np.float32(2.0 ** e)
    blob = oracle.quantize(w, t)
    bd = to_dev(blob)
    for xdt in ("f32", "f16"):
        for n in (1, 2, 40, 130):
            if n == 1 and xdt == "f16":
                continue
            x = synth.activations(n, cols, seed=721 + n, dtype=xdt)
            ref, rabs = oracle.matmul_f64(blob, t, rows, cols, x, threads=THREADS)
            for label, path in every_path(t, n):
                say(f"scaled blocks {t} 2^{e} n={n} x={xdt} {label}")
                check_plain(run(bd, t, rows, cols, x, path), ref, rabs,
                            f"{t} 2^{e} n={n} {xdt} {label}")


# ---------------------------------------------------------------- arbitrary blocks

def _pack_q4k(d16, dmin16, sc, mn, codes):
    """One Q4_K block from fields (R1: 16 six-bit fields LSB first, scale of
    sub-block i in field 2i, min in 2i + 1; R2: sub-block i's bytes 16i..,
    low nibble element 32i + k, high nibble 32i + k + 16)."""
    stream = 0
    for i in range(8):
        stream |= (int(sc[i]) & 63) << (12 * i)
        stream |= (int(mn[i]) & 63) << (12 * i + 6)
    raw = int(d16).to_bytes(2, "little") + int(dmin16).to_bytes(2, "little")
    raw += stream.to_bytes(12, "little")
    for i in range(8):
        c = codes[32 * i:32 * i + 32]
        raw += bytes((int(c[k]) & 15) | ((int(c[k + 16]) & 15) << 4) for k in range(16))
    return raw


def _pack_q6k(d16, sc, codes):
    """One Q6_K block (R4): fp16 d, 16 int8 scales, low nibbles of group g in
    bytes 16g.. (element 32g + k low, 32g + k + 16 high), then the 2-bit high
    parts, byte 8g + k holding element 32g + k + 8u at bits 2u."""
    raw = int(d16).to_bytes(2, "little") + bytes(int(s) & 0xFF for s in sc)
    for g in range(8):
        c = codes[32 * g:32 * g + 32]
        raw += bytes((int(c[k]) & 15) | ((int(c[k + 16]) & 15) << 4) for k in range(16))
    for g in range(8):
        c = codes[32 * g:32 * g + 32]
        raw += bytes(sum(((int(c[k + 8 * u]) >> 4) & 3) << (2 * u) for u in range(4)) for k in range(8))
    return raw


def cancellation_blob(t, rows, cols, seed):
    """Rows of blocks whose products cancel: Q4_K with a q = b exactly (codes
    15, sc 1, m 15, d = dmin) or nearly (dmin one fp16 step below d), Q6_K
    with every code 32 (w = 0) or 33; other rows from the quantizer."""
    rng = np.random.default_rng(seed)
    blob = oracle.quantize(synth.weights(rows, cols, seed=seed), t)
    rb = blob.size // rows
    out = blob.reshape(rows, rb).copy()
    nb = cols // 256
    for r in range(0, rows, 2):
        raw = b""
        for b in range(nb):
            d16 = int(rng.choice([0x1C00, 0x2400, 0x3C00, 0x5800]))
            if t == "q4_k":
                dmin16 = d16 if (r + b) % 3 else d16 - 1
                raw += _pack_q4k(d16, dmin16, [1] * 8, [15] * 8, [15] * 256)
            else:
                code = 32 if (r + b) % 3 else 33
                raw += _pack_q6k(d16, rng.integers(-127, 128, size=16), [code] * 256)
        out[r] = np.frombuffer(raw, dtype=np.uint8)
    return out.reshape(-1)


def _arbitrary(kind, t, rows, cols, seed):
    if kind == "random":
        rb = oracle.row_bytes(t, cols)
        return tol_terms.finite_scales(synth.random_bytes(rows * rb, seed=seed), t)
    return cancellation_blob(t, rows, cols, seed)


CASES = [("random", t) for t in gq.QUANT_TYPES] + [("cancel", "q4_k"), ("cancel", "q6_k")]


@pytest.mark.parametrize("kind,t", CASES)
def test_arbitrary_blocks_every_path(kind, t):
    rows, cols = SHAPES[t]
    blob = _arbitrary(kind, t, rows, cols, seed=730)
    bd = to_dev(blob)
    w64 = oracle.dequant_f64(blob, t, rows, cols)
    for xdt in ("f32", "f16"):
        for n in (1, 2, 9, 40, 130):
            if n == 1 and xdt == "f16":
                continue
            x = synth.activations(n, cols, seed=731 + n, dtype=xdt)
            ref, rabs = oracle.matmul_f64(blob, t, rows, cols, x, threads=THREADS)
            tol = tol_terms.tolerance(blob, t, rows, cols, x, rabs, w64)
            for label, path in every_path(t, n):
                say(f"{kind} blocks {t} n={n} x={xdt} {label}")
                check_bound(run(bd, t, rows, cols, x, path), ref, tol,
                            f"{kind} {t} n={n} {xdt} {label}")


@pytest.mark.parametrize("kind,t", CASES)
def test_arbitrary_blocks_fused_decode(kind, t):
    """The fused decode call (RMSNorm prologue) on the same blocks: the bound
    with the oracle's normalized input in place of x."""
    rows, cols = SHAPES[t]
    blob = _arbitrary(kind, t, rows, cols, seed=740)
    bd = to_dev(blob)
    w64 = oracle.dequant_f64(blob, t, rows, cols)
    x = synth.activations(1, cols, seed=741)[0]
    nw = synth.norm_weights(cols, seed=742)
    xin = oracle.rmsnorm_f64(x.astype(np.float64), nw, 1e-5)
    ref, rabs = oracle.matmul_f64(blob, t, rows, cols, xin[None, :], threads=THREADS)
    tol = tol_terms.tolerance(blob, t, rows, cols, xin[None, :], rabs, w64)
    say(f"{kind} blocks fused decode {t}")
    y = gq.matmul_decode(bd, t, rows, cols, to_dev(x), norm_weight=to_dev(nw), eps=1e-5)
    check_bound(y.cpu().numpy().astype(np.float64)[None, :], ref, tol, f"{kind} {t} decode+norm")
    y = gq.matmul_decode(bd, t, rows, cols, to_dev(x))
    ref, rabs = oracle.matmul_f64(blob, t, rows, cols, x[None, :], threads=THREADS)
    tol = tol_terms.tolerance(blob, t, rows, cols, x[None, :], rabs, w64)
    check_bound(y.cpu().numpy().astype(np.float64)[None, :], ref, tol, f"{kind} {t} decode")


def test_exact_cancellation_is_zero_on_exact_paths():
    """Q4_K blocks with a q = b for every weight (w = 0 exactly): the tiled
    GEMM (B = RNE_fp16 of the exact zero) returns exactly 0 for those rows."""
    t, rows, cols = "q4_k", 64, 512
    raw = b"".join(_pack_q4k(0x3C00, 0x3C00, [1] * 8, [15] * 8, [15] * 256) for _ in range(rows * 2))
    blob = np.frombuffer(raw, dtype=np.uint8).copy()
    assert np.all(oracle.dequant_f64(blob, t, rows, cols) == 0.0)
    x = synth.activations(40, cols, seed=750)
    y = run(to_dev(blob), t, rows, cols, x, gq.PATH_TILED)
    assert np.all(y == 0.0)


# ---------------------------------------------------------------- attention queries

def _scaled_cache(t, kv_len, n_kv, hd, e, seed):
    """K drawn N(0, 1) * 2^-e and V N(0, 1), quantized by the oracle: with
    queries scaled by 2^e the scores stay of order one."""
    k = synth.activations(kv_len * n_kv, hd, seed=seed) * np.float32(2.0 ** -e)
    v = synth.activations(kv_len * n_kv, hd, seed=seed + 1)
    return oracle.quantize(k, t), oracle.quantize(v, t)


@pytest.mark.parametrize("t", ["q8_0", "q4_0"])
@pytest.mark.parametrize("e", [-20, 20])
def test_attn_scaled_query(t, e):
    """fp32 queries of magnitude 2^e (outside fp16 for e = 20, below its
    normal range for e = -20): the part kernel brings each head's q into
    fp16 range by a power of two; the attention tests' bound applies."""
    from test_gpu_attn import reference, run as attn_run
    kv_len, n_kv, hd, n_heads = 600, 2, 128, 10
    kc, vc = _scaled_cache(t, kv_len, n_kv, hd, e, seed=760)
    q = (synth.activations(n_heads, hd, seed=762) * np.float32(2.0 ** e)).astype(np.float64)
    say(f"attention {t} q*2^{e}")
    ref, tol = reference(kc, vc, t, kv_len, n_kv, hd, q)
    got = attn_run(kc, vc, t, kv_len, n_kv, hd, q).astype(np.float64)
    err = np.abs(got - ref)
    say(f"  max err / bound = {float(np.max(err / np.maximum(tol, 1e-300))):.3e}")
    assert np.all(err <= tol)


def test_attn_query_scale_per_head():
    """Query heads of one KV head at 2^20 and 2^-20 alternately: each head
    needs its own power of two (another head's would overflow fp16)."""
    from test_gpu_attn import reference, run as attn_run
    kv_len, n_kv, hd, n_heads = 500, 2, 128, 8
    kc, vc = _scaled_cache("q8_0", kv_len, n_kv, hd, 20, seed=770)
    sc = np.array([2.0 ** (20 if h % 2 == 0 else -20) for h in range(n_heads)])
    q = synth.activations(n_heads, hd, seed=772).astype(np.float64) * sc[:, None]
    q = q.astype(np.float32).astype(np.float64)
    say("attention per-head query scales")
    ref, tol = reference(kc, vc, "q8_0", kv_len, n_kv, hd, q)
    got = attn_run(kc, vc, "q8_0", kv_len, n_kv, hd, q).astype(np.float64)
    err = np.abs(got - ref)
    say(f"  max err / bound = {float(np.max(err / np.maximum(tol, 1e-300))):.3e}")
    assert np.all(err <= tol)
