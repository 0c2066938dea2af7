"""Oracle-free invariants of the GPU matmul paths.

Each check compares the library with itself; the tolerance scale
S[t, r] = sum_c |w^[r, c] x[t, c]| comes from the library's own
dequantization (bit-exact against the oracle elsewhere), so nothing here
reads the oracle:

  * permuting whole block-rows of the blob permutes y's columns, bit for bit
    (every output's sums run inside its own row's lanes, whatever the row's
    position in a tile);
  * linearity in x: y(a x1 + b x2) = a y(x1) + b y(x2) within
    1e-3 (|a| S(x1) + |b| S(x2) + S(x3)) plus the rounding of the combined
    input x3 (2^-23 for fp32, 2^-10 for fp16, times sum_c |w^| |x3|);
  * a batch of N tokens equals N single-token calls within
    2e-3 S per output (both sides meet the 1e-3 bar).

Every path is checked: the batch-1 GEMV, the weight stream and the tiled
GEMM (forced), for fp32 and fp16 activations.
"""
import sys

import numpy as np
import pytest
import torch

import gguf_quant_matmul_amd as gq
import synth

pytestmark = pytest.mark.gpu

QK = {"q4_0": 32, "q5_0": 32, "q8_0": 32, "q4_k": 256, "q6_k": 256, "q4_1": 32, "q5_k": 256,
      "q2_k": 256, "q3_k": 256}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def blob_for(t, rows, cols, seed):
    w = torch.from_numpy(synth.weights(rows, cols, seed=seed, outlier_frac=0.01)).cuda()
    return gq.quantize(w, t)


def scale_of(blob, t, rows, cols, x):
    """S[t, r] = sum_c |w^[r, c] x[t, c]| and sum_c |w^[r, c]| |x| in fp64."""
    w = gq.dequant(blob, t, rows, cols).double().abs()
    xa = x.double().abs().reshape(-1, cols)
    return xa @ w.T


def run(blob, t, rows, cols, x, path=None):
    kw = {} if path is None else {"path": path}
    return gq.matmul(blob, t, rows, cols, x, **kw).double()


PATHS = [
    ("gemv", None, 1),
    ("stream", gq.PATH_WEIGHT_STREAM, 8),
    ("stream", gq.PATH_WEIGHT_STREAM, 40),
    ("tiled", gq.PATH_TILED, 48),
    ("tiled", gq.PATH_TILED, 200),
]


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q5_k", "q4_1", "q2_k", "q3_k"])
@pytest.mark.parametrize("name,path,n", PATHS)
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_row_permutation_permutes_y(t, name, path, n, xdt):
    rows, cols = 300, 2 * 256                   # ragged against every tile height
    say(f"permutation {t} {name} n={n} x={xdt}")
    blob = blob_for(t, rows, cols, seed=41)
    rb = blob.numel() // rows
    perm = torch.from_numpy(np.random.default_rng(42).permutation(rows)).cuda()
    pblob = blob.view(rows, rb)[perm].contiguous().view(-1)
    x = torch.from_numpy(synth.activations(n, cols, seed=43, dtype=xdt)).cuda()
    y = run(blob, t, rows, cols, x, path)
    yp = run(pblob, t, rows, cols, x, path)
    assert torch.equal(yp, y[:, perm]), f"{t} {name}: a row's result depends on its position"


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q5_0"])
@pytest.mark.parametrize("name,path,n", PATHS)
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_linear_in_x(t, name, path, n, xdt):
    rows, cols = 130, 4 * 256
    say(f"linearity {t} {name} n={n} x={xdt}")
    blob = blob_for(t, rows, cols, seed=51)
    x1 = torch.from_numpy(synth.activations(n, cols, seed=52, dtype="f32")).cuda().double()
    x2 = torch.from_numpy(synth.activations(n, cols, seed=53, dtype="f32")).cuda().double()
    a, b = 3.0, -0.5
    tdt = torch.float16 if xdt == "f16" else torch.float32
    x1d, x2d = x1.to(tdt), x2.to(tdt)
    x3d = (a * x1d.double() + b * x2d.double()).to(tdt)
    y1, y2, y3 = (run(blob, t, rows, cols, v, path) for v in (x1d, x2d, x3d))
    s1, s2, s3 = (scale_of(blob, t, rows, cols, v) for v in (x1d, x2d, x3d))
    # the combined input is the rounded a x1 + b x2: its own rounding moves y by at most
    # sum_c |w^| |x3 - (a x1 + b x2)|
    wabs = gq.dequant(blob, t, rows, cols).double().abs()
    dx = (x3d.double() - (a * x1d.double() + b * x2d.double())).abs()
    tol = 1e-3 * (abs(a) * s1 + abs(b) * s2 + s3) + dx @ wabs.T
    err = (y3 - (a * y1 + b * y2)).abs()
    ratio = float((err / tol.clamp_min(1e-300)).max())
    say(f"  max err / bound = {ratio:.3e}")
    assert bool((err <= tol).all()), f"{t} {name}: linearity beyond the bound ({ratio:.3e})"


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q4_1", "q5_k", "q2_k", "q3_k"])
@pytest.mark.parametrize("n,path", [(8, None), (40, None), (70, None),
                                    (24, gq.PATH_TILED), (33, gq.PATH_WEIGHT_STREAM)])
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_batch_equals_single_calls(t, n, path, xdt):
    rows, cols = 200, 2 * 256
    say(f"batch vs single {t} n={n} path={path} x={xdt}")
    blob = blob_for(t, rows, cols, seed=61)
    x = torch.from_numpy(synth.activations(n, cols, seed=62, dtype=xdt)).cuda()
    yb = run(blob, t, rows, cols, x, path)
    ys = torch.cat([run(blob, t, rows, cols, x[i:i + 1]) for i in range(n)])
    s = scale_of(blob, t, rows, cols, x)
    err = (yb - ys).abs()
    ratio = float((err / s.clamp_min(1e-300)).max())
    say(f"  max err / S = {ratio:.3e}")
    assert bool((err <= 2e-3 * s).all()), f"{t} n={n}: batch and single calls differ ({ratio:.3e})"
