"""The test-side field reader behind tests/tol_terms.py, pinned to the oracle:
Q4_K, Q5_K and Q2_K weights rebuilt as a q - b from the fields it reads equal the oracle's
fp64 dequantization on random bytes (finite scales), and every row's block
bound covers every decoded weight of the row."""
import numpy as np
import pytest

import synth
import tol_terms


@pytest.mark.parametrize("t", ["q4_k", "q5_k", "q2_k"])
def test_q4k_parts_rebuild_the_oracle_dequant(oracle, t):
    o = oracle._load()
    rows, cols = 40, 512
    blob = tol_terms.finite_scales(synth.random_bytes(rows * o.row_bytes(t, cols), seed=81), t)
    a, q, b = tol_terms.q4k_parts(blob, rows, cols, t)
    assert np.array_equal(a * q - b, o.dequant_f64(blob, t, rows, cols))


@pytest.mark.parametrize("t", ["q4_0", "q5_0", "q8_0", "q4_k", "q6_k", "q4_1", "q5_k", "q2_k",
                               "q3_k"])
def test_row_bound_covers_every_weight(oracle, t):
    o = oracle._load()
    rows, cols = 30, 2 * tol_terms.QK[t]
    blob = tol_terms.finite_scales(synth.random_bytes(rows * o.row_bytes(t, cols), seed=82), t)
    w = np.abs(o.dequant_f64(blob, t, rows, cols))
    assert np.all(np.isfinite(w))
    assert np.all(w.max(axis=1) <= tol_terms.row_bound(blob, t, rows, cols))
