"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (stated in the design notes):
  * dequantization and quantization: bit-exact (NaN compared as NaN);
  * GEMV / matmul: |y_gpu - y_ref| <= 1e-3 * sum_c |w^[r,c] * x[t,c]| for every
    output, with y_ref the oracle's fp64 dequant-then-dot.
Every input is seeded (synth.py).  Blobs come from the oracle's quantizer
unless a test checks the GPU quantizer itself.
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

QK = {"q4_0": 32, "q5_0": 32, "q8_0": 32, "q4_k": 256, "q6_k": 256, "q4_1": 32, "q5_k": 256,
      "q2_k": 256, "q3_k": 256}
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
TOL = 1e-3


def dev():
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def check_matmul(y_gpu, blob, t, rows, cols, x, rows_idx=None, label=""):
    """Compare y_gpu [n, rows] (numpy) with the oracle on all or sampled rows."""
    if rows_idx is None:
        ref, rabs = oracle.matmul_f64(blob, t, rows, cols, x, threads=THREADS)
        got = y_gpu.astype(np.float64)
    else:
        rb = oracle.row_bytes(t, cols)
        sub = blob.reshape(rows, rb)[rows_idx].reshape(-1)
        ref, rabs = oracle.matmul_f64(sub, t, len(rows_idx), cols, x, threads=THREADS)
        got = y_gpu[:, rows_idx].astype(np.float64)
    err = np.abs(got - ref)
    ratio = float(np.max(err / np.maximum(rabs, 1e-300)))
    say(f"  {label} max |err| / sum|w*x| = {ratio:.3e}")
    bad = ~(err <= TOL * rabs)
    assert not bad.any(), f"{label}: {int(bad.sum())} outputs beyond tolerance, worst ratio {ratio:.3e}"
    return ratio


def quantized(t, rows, cols, seed, outliers=0.01):
    w = synth.weights(rows, cols, seed=seed, outlier_frac=outliers)
    return w, oracle.quantize(w, t)


# ---------------------------------------------------------------- dequant / quantize

@pytest.mark.parametrize("t", gq.QUANT_TYPES)
def test_dequant_bit_exact(t):
    rows, cols = 37, 3 * QK[t]
    say(f"dequant {t} {rows}x{cols}")
    _, blob = quantized(t, rows, cols, seed=11)
    bd = to_dev(blob)
    y32 = gq.dequant(bd, t, rows, cols).cpu().numpy()
    y16 = gq.dequant(bd, t, rows, cols, dtype=torch.float16).cpu().numpy()
    ref = oracle.dequant_f32(blob, t, rows, cols)
    assert np.array_equal(y32.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(y16.view(np.uint16), ref.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("t", gq.QUANT_TYPES)
def test_dequant_fuzz_bytes(t):
    """Random bytes: every field pattern, including NaN/Inf/subnormal scales."""
    rows, cols = 64, 4 * QK[t]
    say(f"dequant fuzz {t}")
    blob = synth.random_bytes(rows * oracle.row_bytes(t, cols), seed=5)
    y = gq.dequant(to_dev(blob), t, rows, cols).cpu().numpy()
    ref = oracle.dequant_f32(blob, t, rows, cols)
    both_nan = np.isnan(y) & np.isnan(ref)
    same = y.view(np.uint32) == ref.view(np.uint32)
    assert np.all(both_nan | same)


@pytest.mark.parametrize("t", gq.QUANT_TYPES)
def test_quantize_bit_exact(t):
    rows, cols = 50, 3 * QK[t]
    say(f"quantize {t}")
    w = synth.weights(rows, cols, seed=21, outlier_frac=0.02)
    # special rows: zeros, constant, all positive, all negative, tiny (fp16
    # subnormal scales), huge (saturating scales)
    w[0] = 0.0
    w[1] = 0.0312
    w[2] = np.abs(w[2])
    w[3] = -np.abs(w[3])
    w[4] *= 1e-5
    w[5] *= 1e7
    blob = gq.quantize(to_dev(w), t).cpu().numpy()
    ref = oracle.quantize(w, t)
    assert np.array_equal(blob, ref), f"{int((blob != ref).sum())} bytes differ"


# ---------------------------------------------------------------- GEMV (n = 1)

GEMV_SHAPES = {
    "q4_k": [(1, 256), (37, 2304), (257, 4096), (130, 16384)],
    "q6_k": [(1, 256), (37, 2304), (257, 11008), (64, 14336)],
    "q5_k": [(1, 256), (37, 2304), (257, 4096), (130, 11008)],
    "q2_k": [(1, 256), (37, 2304), (257, 4096), (130, 11008)],
    "q3_k": [(1, 256), (37, 2304), (257, 4096), (64, 14336)],
    "q4_1": [(1, 32), (37, 96), (257, 4096), (33, 2080)],
    "q8_0": [(1, 32), (37, 96), (257, 4096), (33, 2080)],
    "q5_0": [(1, 32), (37, 96), (257, 4096), (33, 2080)],
    "q4_0": [(1, 32), (37, 96), (257, 4096), (33, 2080)],
}


@pytest.mark.parametrize("t", gq.QUANT_TYPES)
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_gemv_parity(t, xdt):
    for i, (rows, cols) in enumerate(GEMV_SHAPES[t]):
        say(f"gemv {t} {rows}x{cols} x={xdt}")
        _, blob = quantized(t, rows, cols, seed=100 + i)
        x = synth.activations(1, cols, seed=200 + i, dtype=xdt)
        y = gq.matmul(to_dev(blob), t, rows, cols, to_dev(x)).cpu().numpy()
        check_matmul(y, blob, t, rows, cols, x, label=f"{t} {rows}x{cols} {xdt}")


# ---------------------------------------------------------------- matrix cores (n >= 2)

MM_SHAPES = {"q4_k": (75, 512), "q6_k": (75, 768), "q8_0": (75, 352), "q5_0": (75, 288),
             "q4_0": (75, 320), "q4_1": (75, 352), "q5_k": (75, 768), "q2_k": (75, 768),
             "q3_k": (75, 768)}


@pytest.mark.parametrize("t", gq.QUANT_TYPES)
@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_mfma_parity(t, xdt):
    rows, cols = MM_SHAPES[t]
    _, blob = quantized(t, rows, cols, seed=31)
    bd = to_dev(blob)
    for n in (2, 7, 16, 33, 64, 100, 130):
        say(f"mfma {t} {rows}x{cols} n={n} x={xdt}")
        x = synth.activations(n, cols, seed=40 + n, dtype=xdt)
        y = gq.matmul(bd, t, rows, cols, to_dev(x)).cpu().numpy()
        check_matmul(y, blob, t, rows, cols, x, label=f"{t} n={n} {xdt}")
        if n > 64:                               # both kernel families past 64 tokens
            for path in (gq.PATH_WEIGHT_STREAM, gq.PATH_TILED):
                y = gq.matmul(bd, t, rows, cols, to_dev(x), path=path).cpu().numpy()
                check_matmul(y, blob, t, rows, cols, x, label=f"{t} n={n} {xdt} path {path}")


@pytest.mark.parametrize("t", gq.QUANT_TYPES)
def test_mfma_many_slabs_and_rows(t):
    """Rows split into many 16-row tiles and the columns into 16 slabs shared
    by several waves; for the 32-weight types the last slab is partial
    (4000 columns = 125 blocks)."""
    rows, cols = 300, (4096 if QK[t] == 256 else 4000)
    _, blob = quantized(t, rows, cols, seed=32)
    bd = to_dev(blob)
    for n, xdt in ((8, "f16"), (9, "f16"), (40, "f16"), (5, "f32"), (40, "f32")):
        say(f"mfma {t} {rows}x{cols} n={n} x={xdt}")
        x = synth.activations(n, cols, seed=33 + n, dtype=xdt)
        y = gq.matmul(bd, t, rows, cols, to_dev(x)).cpu().numpy()
        check_matmul(y, blob, t, rows, cols, x, label=f"{t} {rows}x{cols} n={n} {xdt}")


@pytest.mark.parametrize("t,rows,cols,n,xdt", [
    ("q5_0", 4096, 4000, 24, "f16"),     # 32-token pass, 256 tiles: the larger LDS budget
    ("q8_0", 4096, 4000, 30, "f16"),
    ("q8_0", 2048, 4000, 40, "f16"),     # two 32-token passes over 128 tiles
    ("q4_0", 4095, 2080, 9, "f32"),      # 65 blocks per row (2-byte-aligned rows), ragged tile
    ("q5_0", 1000, 1056, 3, "f16"),      # 33 blocks: a slab with one block
])
def test_mmv_32weight_staged(t, rows, cols, n, xdt):
    """The 32-weight types' small-batch path (blocks loaded whole and
    regrouped through LDS), including rows with an odd block count and a last
    slab of one block: sampled rows (every token) against the oracle."""
    _, blob = quantized(t, rows, cols, seed=151)
    bd = to_dev(blob)
    rng = np.random.default_rng(152)
    idx = np.unique(np.concatenate([rng.choice(rows, 80, replace=False), np.r_[0:24, rows - 24:rows]]))
    say(f"mmv 32-weight staged {t} {rows}x{cols} n={n} x={xdt}")
    x = synth.activations(n, cols, seed=153 + n, dtype=xdt)
    y = gq.matmul(bd, t, rows, cols, to_dev(x), path=gq.PATH_WEIGHT_STREAM).cpu().numpy()
    check_matmul(y, blob, t, rows, cols, x, rows_idx=idx, label=f"{t} {rows}x{cols} n={n} {xdt}")


@pytest.mark.parametrize("t,rows,cols,ns", [
    ("q4_k", 32768, 256, ((5, "f16"), (24, "f16"), (8, "f32"))),
    ("q6_k", 32005, 512, ((8, "f16"), (30, "f16"), (3, "f32"))),
    ("q4_k", 11008, 512, ((24, "f16"), (64, "f16"))),   # 32-token passes, 344 tile pairs
    ("q5_k", 4112, 512, ((40, "f16"),)),                 # 257 tiles: the last pair has one
    ("q3_k", 8208, 256, ((20, "f16"),)),
    ("q2_k", 8200, 256, ((33, "f16"),)),                 # 513 tiles, the last one ragged
    ("q4_k", 14352, 256, ((12, "f16"),)),                # 16-token pass, 449 pairs, ragged
    ("q6_k", 11008, 256, ((20, "f32"),)),                # fp32 x, 344 pairs x 2 passes
    ("q5_k", 19216, 256, ((16, "f32"),)),                # fp32 x, 601 pairs, ragged
    ("q4_k", 11008, 256, ((64, "f32"),)),                # fp32 x, four passes
])
def test_mmv_two_tiles_per_wave(t, rows, cols, ns):
    """Tall K-quant matrices (over 2000 16-row tiles), and 16- and 32-token
    passes with enough tile pairs, where each wave takes two tiles sharing
    its activation slab; the last tile ragged: sampled rows (every token)
    against the oracle."""
    _, blob = quantized(t, rows, cols, seed=141)
    bd = to_dev(blob)
    rng = np.random.default_rng(142)
    idx = np.unique(np.concatenate([rng.choice(rows, 96, replace=False), np.r_[0:40, rows - 40:rows]]))
    for n, xdt in ns:
        say(f"mmv two tiles {t} {rows}x{cols} n={n} x={xdt}")
        x = synth.activations(n, cols, seed=143 + n, dtype=xdt)
        y = gq.matmul(bd, t, rows, cols, to_dev(x), path=gq.PATH_WEIGHT_STREAM).cpu().numpy()
        check_matmul(y, blob, t, rows, cols, x, rows_idx=idx, label=f"{t} {rows}x{cols} n={n} {xdt}")


@pytest.mark.parametrize("t,rows,cols,ns", [
    ("q4_k", 16400, 512, ((8, "f16"), (16, "f16"), (5, "f32"), (40, "f16"))),
    ("q6_k", 8200, 768, ((8, "f16"), (3, "f32"), (24, "f16"))),
])
def test_mmv_tall_matrices(t, rows, cols, ns):
    """Small batches on tall matrices (over a thousand 16-row tiles, the last
    one ragged) with fp16 and fp32 activations, one and several token
    passes: checked in full against the oracle."""
    _, blob = quantized(t, rows, cols, seed=96)
    bd = to_dev(blob)
    for n, xdt in ns:
        say(f"mmv tall {t} {rows}x{cols} n={n} x={xdt}")
        x = synth.activations(n, cols, seed=97 + n, dtype=xdt)
        y = gq.matmul(bd, t, rows, cols, to_dev(x)).cpu().numpy()
        check_matmul(y, blob, t, rows, cols, x, label=f"{t} {rows}x{cols} n={n} {xdt}")


@pytest.mark.parametrize("t,rows,cols,n,xdt", [
    ("q4_k", 256, 8192, 128, "f16"),     # one tile of 128 K steps
    ("q6_k", 512, 4096, 200, "f32"),     # 4 tiles (2 x 2, the token tiles ragged), fp32 x
    ("q8_0", 600, 2400, 96, "f16"),      # 3 x 1 tiles, 38 K steps: a partial last unit
    ("q5_0", 300, 1056, 140, "f32"),     # 17 K steps, ragged rows and tokens
    ("q6_k", 4096, 512, 200, "f16"),     # 64 x 64 tiles in 4 K groups, ragged token tile
    ("q4_0", 4000, 1056, 150, "f16"),    # the same with ragged rows; 17 K steps: groups
                                         # of 8, 8, 1 and none
])
def test_gemm_few_tiles(t, rows, cols, n, xdt):
    """Prefill shapes with few tiles and long or ragged K (a partial last
    K step for the 32-weight types, ragged rows and token tiles): checked in
    full against the oracle, and three calls in a row agree bit for bit."""
    _, blob = quantized(t, rows, cols, seed=91)
    bd = to_dev(blob)
    say(f"gemm few tiles {t} {rows}x{cols} n={n} x={xdt}")
    x = synth.activations(n, cols, seed=92, dtype=xdt)
    xd = to_dev(x)
    ys = [gq.matmul(bd, t, rows, cols, xd, path=gq.PATH_TILED).cpu().numpy() for _ in range(3)]
    for y in ys[1:]:
        assert np.array_equal(y.view(np.uint32), ys[0].view(np.uint32))
    check_matmul(ys[0], blob, t, rows, cols, x, label=f"{t} {rows}x{cols} n={n} {xdt}")


@pytest.mark.parametrize("t,rows,cols,n", [
    ("q6_k", 4096, 11008, 512),          # 64 tiles x 172 K steps over every CU
    ("q4_k", 11008, 4096, 768),          # 258 tiles: one more than a wave of 256
])
def test_gemm_partial_wave_full_size(t, rows, cols, n):
    """Full-size prefill shapes whose tiles do not fill whole waves of CUs
    (the FFN down projection's 64 tiles of 172 K steps; 258 tiles): sampled
    rows against the oracle, and two calls bit-identical."""
    _, blob = quantized(t, rows, cols, seed=93)
    bd = to_dev(blob)
    say(f"gemm partial wave {t} {rows}x{cols} n={n}")
    x = synth.activations(n, cols, seed=94, dtype="f16")
    xd = to_dev(x)
    y0 = gq.matmul(bd, t, rows, cols, xd, path=gq.PATH_TILED).cpu().numpy()
    y1 = gq.matmul(bd, t, rows, cols, xd, path=gq.PATH_TILED).cpu().numpy()
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    rng = np.random.default_rng(95)
    idx = np.unique(np.concatenate([rng.choice(rows, 96, replace=False), np.r_[0:16, rows - 16:rows]]))
    check_matmul(y0, blob, t, rows, cols, x, rows_idx=idx, label=f"{t} {rows}x{cols} n={n}")


@pytest.mark.parametrize("t,rows,cols,n,xdt", [
    ("q4_k", 32768, 256, 100, "f16"),    # 128 tiles of 256 x 128: the large tile shape, ragged tokens
    ("q8_0", 8400, 512, 1030, "f32"),    # 297 large tiles -> 128 x 128 tiles, ragged rows and tokens
    ("q6_k", 1000, 768, 77, "f16"),      # few tiles -> 32-row tiles in 4 K groups, ragged
    ("q4_0", 4096, 4096, 512, "f16"),    # 64 large tiles -> 256 tiles of 128 x 64
    ("q6_k", 1000, 768, 40, "f32"),      # fp32 x up to 64 tokens: 128 x 64 tiles
    ("q5_k", 8200, 512, 40, "f16"),      # > 256 32-row tiles: 64-row tiles in 4 K groups, ragged
    ("q4_1", 9000, 768, 64, "f16"),      # 64 x 64 in 4 K groups, the last group past the end of K
    ("q6_k", 2000, 768, 460, "f16"),     # Q6_K, 128 tiles of 128 x 64 -> 64 x 128 in 2 K groups
])
def test_gemm_tile_shapes(t, rows, cols, n, xdt):
    """Each tile shape of the tiled GEMM (chosen by how many CUs the tiles
    cover, and for up to 64 tokens or few tiles with K split over groups of
    one workgroup) with ragged edges: sampled rows (all tokens) against the
    oracle, and two calls bit-identical."""
    _, blob = quantized(t, rows, cols, seed=97)
    bd = to_dev(blob)
    say(f"gemm tile shape {t} {rows}x{cols} n={n} x={xdt}")
    x = synth.activations(n, cols, seed=98, dtype=xdt)
    xd = to_dev(x)
    y0 = gq.matmul(bd, t, rows, cols, xd, path=gq.PATH_TILED).cpu().numpy()
    y1 = gq.matmul(bd, t, rows, cols, xd, path=gq.PATH_TILED).cpu().numpy()
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    rng = np.random.default_rng(99)
    idx = np.unique(np.concatenate([rng.choice(rows, 64, replace=False), np.r_[0:8, rows - 136:rows]]))
    check_matmul(y0, blob, t, rows, cols, x, rows_idx=idx, label=f"{t} {rows}x{cols} n={n} {xdt}")


@pytest.mark.parametrize("t,rows,cols,n,xdt", [
    ("q6_k", 4096, 14336, 128, "f16"),   # few GEMM tiles over a long K: two 64-token chunks
    ("q4_k", 4096, 4096, 65, "f16"),     # chunks of 33 and 32
    ("q4_k", 1024, 4096, 130, "f32"),    # three chunks (44, 43, 43), fp32 x
])
def test_batch_chunks_past_64_tokens(t, rows, cols, n, xdt):
    """Past 64 tokens on shapes with few GEMM tiles the automatic choice runs
    the weight-stream kernel in chunks: bit-identical to asking for that path,
    and against the oracle on sampled rows (all tokens)."""
    _, blob = quantized(t, rows, cols, seed=301)
    bd = to_dev(blob)
    say(f"batch chunks {t} {rows}x{cols} n={n} x={xdt}")
    x = synth.activations(n, cols, seed=302, dtype=xdt)
    xd = to_dev(x)
    ya = gq.matmul(bd, t, rows, cols, xd).cpu().numpy()
    yw = gq.matmul(bd, t, rows, cols, xd, path=gq.PATH_WEIGHT_STREAM).cpu().numpy()
    assert np.array_equal(ya.view(np.uint32), yw.view(np.uint32))
    rng = np.random.default_rng(303)
    idx = np.unique(np.concatenate([rng.choice(rows, 64, replace=False), np.r_[0:8, rows - 8:rows]]))
    check_matmul(ya, blob, t, rows, cols, x, rows_idx=idx, label=f"{t} {rows}x{cols} n={n} {xdt}")


# ---------------------------------------------------------------- decode-layer fusions

def decode_reference(blob, up, t, rows, cols, x, xdt, nw, eps):
    """(y_ref, tolerance) for gq_matmul_decode from the oracle: RMSNorm of x
    (when nw is given), then W^ x or silu(W^ x) * (U^ x).  The gated form's
    bound carries the matmul bar through h = silu(g) u: |silu'| <= 1.1, so
    |dh| <= 1.1 |dg| (|u| + |du|) + |silu(g)| |du| with |dg|, |du| within
    1e-3 of sum |w x|, plus a few fp32 roundings of h."""
    xin = x.astype(np.float64).reshape(-1)
    if nw is not None:
        xin = oracle.rmsnorm_f64(xin, nw, eps, half_x=(xdt == "f16"))
    g, ga = oracle.matmul_f64(blob, t, rows, cols, xin[None, :], threads=THREADS)
    g, ga = g[0], ga[0]
    if up is None:
        return g, TOL * ga
    u, ua = oracle.matmul_f64(up, t, rows, cols, xin[None, :], threads=THREADS)
    u, ua = u[0], ua[0]
    h = oracle.swiglu_f64(g, u)
    sg = np.abs(oracle.swiglu_f64(g, np.ones_like(g)))
    tol = 1.1 * TOL * ga * (np.abs(u) + TOL * ua) + TOL * sg * ua + 1e-6 * np.abs(h)
    return h, tol


DECODE_SHAPES = [("q4_k", 300, 4096), ("q6_k", 96, 11008), ("q8_0", 300, 352),
                 ("q5_0", 75, 288), ("q4_0", 130, 2048), ("q4_k", 200, 768),
                 ("q4_1", 130, 2080), ("q5_k", 120, 4096), ("q2_k", 120, 4096),
                 ("q3_k", 96, 11008)]


@pytest.mark.parametrize("t,rows,cols", DECODE_SHAPES)
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_decode_fused(t, rows, cols, xdt):
    """RMSNorm prologue and SwiGLU epilogue of gq_matmul_decode against the
    oracle, in every combination; with neither, the call is bit-identical to
    gq_matmul_ex at one token."""
    _, blob = quantized(t, rows, cols, seed=121)
    _, upb = quantized(t, rows, cols, seed=122)
    bd, ud = to_dev(blob), to_dev(upb)
    x = synth.activations(1, cols, seed=123, dtype=xdt)[0]
    nw = synth.norm_weights(cols, seed=124)
    xd, nd = to_dev(x), to_dev(nw)
    plain = gq.matmul(bd, t, rows, cols, xd).cpu().numpy()[0]
    none = gq.matmul_decode(bd, t, rows, cols, xd).cpu().numpy()
    assert np.array_equal(plain.view(np.uint32), none.view(np.uint32))
    for norm in (False, True):
        for glu in (False, True):
            if not (norm or glu):
                continue
            say(f"decode {t} {rows}x{cols} x={xdt} norm={norm} glu={glu}")
            y = gq.matmul_decode(bd, t, rows, cols, xd, up=ud if glu else None,
                                 norm_weight=nd if norm else None, eps=1e-5).cpu().numpy()
            ref, tol = decode_reference(blob, upb if glu else None, t, rows, cols, x, xdt,
                                        nw if norm else None, 1e-5)
            err = np.abs(y.astype(np.float64) - ref)
            say(f"  max err / tol = {float(np.max(err / np.maximum(tol, 1e-300))):.3e}")
            assert np.all(err <= tol), (norm, glu, int(np.sum(err > tol)))


def test_decode_fused_deterministic_and_scale_free():
    """The normalized path repeats bit for bit, and RMSNorm makes the result
    independent of a power-of-two scaling of x (exact in fp32 and fp16)."""
    t, rows, cols = "q4_k", 512, 4096
    _, blob = quantized(t, rows, cols, seed=125)
    _, upb = quantized(t, rows, cols, seed=126)
    bd, ud = to_dev(blob), to_dev(upb)
    x = synth.activations(1, cols, seed=127)[0]
    nw = to_dev(synth.norm_weights(cols, seed=128))
    a = gq.matmul_decode(bd, t, rows, cols, to_dev(x), up=ud, norm_weight=nw, eps=0.0).cpu().numpy()
    b = gq.matmul_decode(bd, t, rows, cols, to_dev(x), up=ud, norm_weight=nw, eps=0.0).cpu().numpy()
    c = gq.matmul_decode(bd, t, rows, cols, to_dev(x * np.float32(8.0)), up=ud, norm_weight=nw,
                         eps=0.0).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


# ---------------------------------------------------------------- exact special cases

def _q8_unit_blob(codes):
    rows, cols = codes.shape
    blocks = codes.reshape(rows, cols // 32, 32).astype(np.int8).view(np.uint8)
    head = np.zeros((rows, cols // 32, 2), dtype=np.uint8)
    head[..., 1] = 0x3C                                  # d = 1.0
    return np.concatenate([head, blocks], axis=2).reshape(-1)


@pytest.mark.parametrize("n", [1, 9])
def test_integer_reduction_exact(n):
    """Q8_0 with d = 1 and small-integer x is an exact integer product."""
    rng = np.random.default_rng(3)
    rows, cols = 70, 512
    codes = rng.integers(-128, 128, size=(rows, cols))
    xi = rng.integers(-16, 17, size=(n, cols))
    blob = _q8_unit_blob(codes)
    say(f"integer reduction n={n}")
    x = xi.astype(np.float16) if n > 1 else xi.astype(np.float32)
    y = gq.matmul(to_dev(blob), "q8_0", rows, cols, to_dev(x)).cpu().numpy()
    assert np.array_equal(y.astype(np.int64), xi @ codes.T)


@pytest.mark.parametrize("xdt", ["f16", "f32"])
@pytest.mark.parametrize("n", [1, 3, 40])
def test_identity_reduction(n, xdt):
    """Q8_0 with d = 1 and one code 1 per row (row r picks column r): y = x.
    Exact for fp16 x; fp32 x at n >= 2 is split into two fp16 parts, which
    keeps all but the last 2 bits of the fp32 significand."""
    rows = cols = 256
    codes = np.eye(rows, cols, dtype=np.int64)
    x = synth.activations(n, cols, seed=90 + n, dtype=xdt)
    say(f"identity n={n} x={xdt}")
    y = gq.matmul(to_dev(_q8_unit_blob(codes)), "q8_0", rows, cols, to_dev(x)).cpu().numpy()
    xs = x.astype(np.float64)
    if xdt == "f16" or n == 1:
        assert np.array_equal(y.astype(np.float64), xs)
    else:
        assert np.all(np.abs(y - xs) <= 2.0 ** -21 * np.abs(xs) + 2.0 ** -25)


def _scale_by_two(blob, t, rows, cols):
    qk, bb = oracle.block_info(t)
    b = blob.copy().reshape(-1, bb)
    offs = [0, 2] if t in ("q4_k", "q5_k", "q4_1", "q2_k") else [0]     # d, and dmin or m
    for off in offs:
        h = b[:, off].astype(np.uint16) | (b[:, off + 1].astype(np.uint16) << 8)
        mag = h & 0x7FFF
        assert np.all((mag >> 10) < 30)
        h = np.where(mag >= 0x0400, h + 0x0400, (h & 0x8000) | (mag << 1)).astype(np.uint16)
        b[:, off] = (h & 0xFF).astype(np.uint8)
        b[:, off + 1] = (h >> 8).astype(np.uint8)
    return b.reshape(-1)


@pytest.mark.parametrize("t", gq.QUANT_TYPES)
def test_power_of_two_scaling_is_exact(t):
    """Doubling every fp16 scale doubles y bit for bit, at any summation order."""
    rows, cols = 64, 2 * QK[t] if QK[t] == 256 else 256
    _, blob = quantized(t, rows, cols, seed=55)
    b2 = _scale_by_two(blob, t, rows, cols)
    for n, xdt in ((1, "f32"), (20, "f16")):
        say(f"pow2 {t} n={n}")
        x = to_dev(synth.activations(n, cols, seed=56, dtype=xdt))
        y1 = gq.matmul(to_dev(blob), t, rows, cols, x).cpu().numpy()
        y2 = gq.matmul(to_dev(b2), t, rows, cols, x).cpu().numpy()
        assert np.array_equal(y2, 2 * y1)


def test_deterministic_run_to_run():
    t, rows, cols = "q6_k", 4096, 4096
    _, blob = quantized(t, rows, cols, seed=60)
    bd = to_dev(blob)
    for n, xdt in ((1, "f32"), (64, "f16")):
        say(f"determinism n={n}")
        x = to_dev(synth.activations(n, cols, seed=61, dtype=xdt))
        a = gq.matmul(bd, t, rows, cols, x).cpu().numpy()
        b = gq.matmul(bd, t, rows, cols, x).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_nan_scale_propagates():
    t, rows, cols = "q4_k", 16, 512
    _, blob = quantized(t, rows, cols, seed=70)
    blob = blob.copy()
    rb = oracle.row_bytes(t, cols)
    blob[3 * rb + 144 + 0] = 0x00
    blob[3 * rb + 144 + 1] = 0x7E                         # d of row 3, block 1 = NaN
    for n, xdt in ((1, "f32"), (5, "f16")):
        say(f"nan propagation n={n}")
        x = to_dev(synth.activations(n, cols, seed=71, dtype=xdt))
        y = gq.matmul(to_dev(blob), t, rows, cols, x).cpu().numpy()
        assert np.all(np.isnan(y[:, 3]))
        assert np.all(np.isfinite(np.delete(y, 3, axis=1)))


def test_zero_tokens_and_tiny():
    t = "q4_k"
    _, blob = quantized(t, 1, 256, seed=80)
    bd = to_dev(blob)
    say("zero tokens")
    out = torch.empty((0, 1), dtype=torch.float32, device=dev())
    x = torch.zeros((0, 256), dtype=torch.float32, device=dev())
    assert gq.lib().gq_matmul(bd.data_ptr(), gq.Q4_K, 1, 256, x.data_ptr(), out.data_ptr(), 0, None) == 0
    x1 = synth.activations(1, 256, seed=81)
    y = gq.matmul(bd, t, 1, 256, to_dev(x1)).cpu().numpy()
    check_matmul(y, blob, t, 1, 256, x1, label="1x256")


@pytest.mark.parametrize("nbytes", [0, 16, 16 * 1000 + 16, 29491200, 40 << 20])
def test_probe_stream_read_reads_every_word(nbytes):
    """The streaming-read probe (the measured bandwidth ceiling) reads every
    byte: the XOR of its per-workgroup outputs equals the buffer's."""
    say(f"probe {nbytes} bytes")
    host = synth.random_bytes(nbytes, seed=nbytes + 5)
    buf = to_dev(host) if nbytes else torch.empty(0, dtype=torch.uint8, device=dev())
    out = gq.probe_stream_read(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32)) if nbytes else np.uint32(0)
    assert got == want
