"""The CPU oracle against its pins, and the pins against planted mistakes."""
import numpy as np
import pytest

import oracle_pins as P
import synth


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle, pin):
    pin(oracle._load())


# Each deliberate mistake compiled into a separate oracle build must be caught
# by at least one pin.
PLANTS = {1: "nibble order swapped", 2: "Q4_K min sign", 3: "Q4_K scale/min swapped",
          4: "Q6_K offset", 5: "dot drops a column", 6: "dot reads x transposed",
          7: "RMSNorm drops eps", 8: "SiLU exponent sign",
          9: "attention without 1/sqrt(head_dim)", 10: "attention head mapping h % n_kv",
          11: "unsaturated (Inf) block scale", 12: "Q4_1 min sign",
          13: "Q5_K fifth bits of the neighbouring element", 14: "Q2_K scale/min nibbles swapped",
          15: "Q3_K code offset 3", 16: "2-bit code plane in element order"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda k: PLANTS[k])
def test_planted_mistake_is_caught(plant):
    import oracle
    o = oracle.Oracle(plant)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin rejects plant {plant} ({PLANTS[plant]})"


def test_half_to_double_all_encodings(oracle):
    """fp16 decoding against NumPy's binary16 for all 65536 encodings."""
    o = oracle._load()
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = np.array([o.half_to_double(int(v)) for v in h])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (got == ref))


def test_half_rne_matches_numpy(oracle):
    """fp32 -> fp16 rounding against NumPy's IEEE conversion, ties included."""
    o = oracle._load()
    rng = np.random.default_rng(1)
    f = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-5).astype(np.float32),      # fp16 subnormals
        (rng.standard_normal(1000) * 3e4).astype(np.float32),       # near overflow
        np.array([65504, 65519.99, 65520, 1e6, -65520, 0.0, -0.0, 2.0 ** -25,
                  2.0 ** -26, 3 * 2.0 ** -26], np.float32),
    ])
    # exact halfway points between neighbouring fp16 values
    hs = rng.integers(0, 0x7BFF, size=1000).astype(np.uint16)
    lo = hs.view(np.float16).astype(np.float64)
    hi = (hs + 1).view(np.float16).astype(np.float64)
    f = np.concatenate([f, ((lo + hi) / 2).astype(np.float32)])
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    got = np.array([o.half_rne(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_half_up_is_smallest_cover(oracle):
    o = oracle._load()
    v = np.abs(np.random.default_rng(2).standard_normal(3000)) * 10.0 ** np.random.default_rng(3).uniform(-8, 4, 3000)
    for x in v:
        h = o.half_up(float(x))
        assert o.half_to_double(h) >= x
        assert h == 0 or o.half_to_double(h - 1) < x


def test_quantize_rejects_bad_shapes(oracle):
    o = oracle._load()
    with pytest.raises(ValueError):
        o.quantize(np.zeros((2, 100), np.float32), "q4_k")
    with pytest.raises(ValueError):
        o.block_info("iq4_xs")


def test_matmul_zero_tokens(oracle):
    o = oracle._load()
    w = synth.weights(4, 256, seed=1)
    blob = o.quantize(w, "q4_k")
    y, _ = o.matmul_f64(blob, "q4_k", 4, 256, np.zeros((0, 256)))
    assert y.shape == (0, 4)


def test_threads_do_not_change_results(oracle):
    o = oracle._load()
    w = synth.weights(64, 512, seed=5)
    blob = o.quantize(w, "q6_k")
    x = synth.activations(3, 512, seed=6)
    y1, _ = o.matmul_f64(blob, "q6_k", 64, 512, x, threads=1)
    y4, _ = o.matmul_f64(blob, "q6_k", 64, 512, x, threads=4)
    assert np.array_equal(y1, y4)
