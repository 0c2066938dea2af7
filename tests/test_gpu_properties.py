"""Property tests of the GPU matmul against the oracle over shapes and
seeds (hypothesis): rows in [1, 300], whole blocks per row, token counts
around every pass and tile boundary, fp32 and fp16 activations, each path
(automatic, weight stream, tiled), every block type.  Deterministic
(derandomized); each case is checked in full against the oracle's bar
(|y - y_ref| <= 1e-3 sum_c |w^ x|)."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import gguf_quant_matmul_amd as gq
import oracle
import synth
from test_gpu_parity import check_matmul, say

pytestmark = pytest.mark.gpu

TYPES = ["q4_0", "q5_0", "q8_0", "q4_k", "q6_k", "q4_1", "q5_k", "q2_k", "q3_k"]
QK = {"q4_0": 32, "q5_0": 32, "q8_0": 32, "q4_k": 256, "q6_k": 256, "q4_1": 32, "q5_k": 256,
      "q2_k": 256, "q3_k": 256}
PATHS = {"auto": gq.PATH_AUTO, "stream": gq.PATH_WEIGHT_STREAM, "tiled": gq.PATH_TILED}


@settings(max_examples=80, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(t=st.sampled_from(TYPES), rows=st.integers(1, 300), blocks=st.integers(1, 6),
       n=st.sampled_from([1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 32, 33, 47, 63, 64, 65, 70]),
       xdt=st.sampled_from(["f32", "f16"]), path=st.sampled_from(sorted(PATHS)),
       seed=st.integers(0, 2**31 - 1))
def test_matmul_random_shapes(t, rows, blocks, n, xdt, path, seed):
    cols = blocks * QK[t]
    if n == 1:
        path = "auto"                           # one token: the GEMV
    say(f"random shape {t} {rows}x{cols} n={n} x={xdt} path={path} seed={seed}")
    w = synth.weights(rows, cols, seed=seed, outlier_frac=0.01)
    blob = oracle.quantize(w, t)
    x = synth.activations(n, cols, seed=seed + 1, dtype=xdt)
    y = gq.matmul(torch.from_numpy(blob).cuda(), t, rows, cols, torch.from_numpy(x).cuda(),
                  path=PATHS[path]).cpu().numpy()
    check_matmul(y, blob, t, rows, cols, x, label=f"{t} {rows}x{cols} n={n}")
