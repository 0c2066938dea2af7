"""Property tests of the oracle over shapes and seeds (hypothesis, CPU).

The same properties the fixed pins check, drawn over many shapes and
seeds: quantize -> dequantize within half a quantization step (the
quantizer's definition), the fp32 dequantization one rounding of the exact
value, the fp64 dot within its summation bound of the exact rational dot
on dyadic inputs, and every stored fp16 field finite.  Runs are
deterministic (derandomized)."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import synth
from oracle_pins import _exact_dot, _roundtrip_bound
from fractions import Fraction

TYPES = ["q4_0", "q5_0", "q8_0", "q4_k", "q6_k", "q4_1", "q5_k"]
QK = {"q4_0": 32, "q5_0": 32, "q8_0": 32, "q4_k": 256, "q6_k": 256, "q4_1": 32, "q5_k": 256}
SETTINGS = settings(max_examples=40, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.function_scoped_fixture])


@SETTINGS
@given(t=st.sampled_from(TYPES), rows=st.integers(1, 40), blocks=st.integers(1, 4),
       seed=st.integers(0, 2**31 - 1), outliers=st.sampled_from([0.0, 0.01, 0.2]),
       std=st.sampled_from([1e-6, 0.02, 3.0]))
def test_roundtrip_within_half_step(oracle, t, rows, blocks, seed, outliers, std):
    cols = blocks * QK[t]
    w = synth.weights(rows, cols, seed=seed, std=std, outlier_frac=outliers)
    blob = oracle.quantize(w, t)
    got = oracle.dequant_f64(blob, t, rows, cols)
    assert np.all(np.isfinite(got))
    err = np.abs(got - w.astype(np.float64))
    bound = _roundtrip_bound(w, t) * (1 + 1e-9) + 1e-12
    assert np.all(err <= bound), float((err / bound).max())


@SETTINGS
@given(t=st.sampled_from(TYPES), rows=st.integers(1, 40), blocks=st.integers(1, 4),
       seed=st.integers(0, 2**31 - 1))
def test_f32_dequant_is_one_rounding(oracle, t, rows, blocks, seed):
    cols = blocks * QK[t]
    blob = oracle.quantize(synth.weights(rows, cols, seed=seed, outlier_frac=0.01), t)
    w32 = oracle.dequant_f32(blob, t, rows, cols)
    w64 = oracle.dequant_f64(blob, t, rows, cols)
    assert np.array_equal(w32, w64.astype(np.float32))


@SETTINGS
@given(t=st.sampled_from(TYPES), rows=st.integers(1, 3), blocks=st.integers(1, 2),
       n=st.integers(1, 2), seed=st.integers(0, 2**31 - 1))
def test_dot_within_bound_of_exact(oracle, t, rows, blocks, n, seed):
    cols = blocks * QK[t]
    blob = oracle.quantize(synth.weights(rows, cols, seed=seed, outlier_frac=0.05), t)
    w64 = oracle.dequant_f64(blob, t, rows, cols)
    x = synth.dyadic((n, cols), seed=seed + 1)
    y, yabs = oracle.matmul_f64(blob, t, rows, cols, x)
    for tok in range(n):
        for r, (s, sa) in enumerate(_exact_dot(w64, x[tok])):
            bound = Fraction(cols * 2.0 ** -53 * float(sa))
            assert abs(Fraction(y[tok, r]) - s) <= bound
            assert abs(Fraction(yabs[tok, r]) - sa) <= bound
