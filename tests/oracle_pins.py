"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the given oracle instance
disagrees with what the pages or mathematics fix.  ``tests/test_oracle.py`` runs
them on the real oracle (all must pass) and on builds with a deliberate mistake
compiled in (at least one must fail for each).

What each pin rests on:
  * golden blocks: hand-chosen fields packed by the byte layouts of the pages
    (or the stated readings), with weights from the pages' dequant formulas;
  * byte counts and bits per weight printed on the pages;
  * exact rational arithmetic (fractions.Fraction) for the fp64 dot;
  * textbook reductions: Q8_0 with d = 1 is an integer matrix product (NumPy
    int64), Q4_K with constant codes per sub-block reduces to per-sub-block sums;
  * invariants: power-of-two scaling is exact, row permutation permutes y,
    n tokens in one call equal n calls;
  * the quantizer's round-trip error bound derived from its definition;
  * RMSNorm and SiLU: closed forms, identities and invariants;
  * decode attention over a quantized KV cache: closed forms (one position,
    zero query, two positions), the query-to-KV head mapping, and invariance
    under permuting the cached positions.
"""
from __future__ import annotations

import glob
import json
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
QTYPES = ["q4_0", "q5_0", "q8_0", "q4_k", "q6_k", "q4_1", "q5_k", "q2_k", "q3_k"]


def golden_fixtures():
    out = []
    for p in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        with open(p) as fh:
            out.append((os.path.basename(p), json.load(fh)))
    return out


def pin_golden(o):
    """Hand-built blocks decode to the pages' formula on their fields."""
    for name, fx in golden_fixtures():
        raw = np.frombuffer(bytes.fromhex(fx["hex"]), dtype=np.uint8)
        qk, bb = o.block_info(fx["type"])
        assert raw.size == bb, name
        w64 = o.dequant_f64(raw, fx["type"], 1, qk)[0]
        w32 = o.dequant_f32(raw, fx["type"], 1, qk)[0]
        exp = np.array(fx["expected"], dtype=np.float64)
        exp32 = np.array(fx["expected_f32"], dtype=np.float32)
        assert np.array_equal(w64, exp), (name, np.nonzero(w64 != exp)[0][:5])
        assert np.array_equal(w32.view(np.uint32), exp32.view(np.uint32)), name


def pin_sizes(o):
    """Bytes per block and bits per weight as the pages print them."""
    # Q4_0: 18 B per 32 weights, 4.5 bpw (Hitchhiker's Guide §11.1 figure).
    assert o.block_info("q4_0") == (32, 18)
    # Q4_K: 2+2+12+128 = 144 B per 256 weights, 4.5 bpw (§11.2; 12 — llama.cpp).
    assert o.block_info("q4_k") == (256, 2 + 2 + 12 + 128)
    for t in ("q4_0", "q4_k"):
        qk, bb = o.block_info(t)
        assert bb * 8 / qk == 4.5
    # Q6_K: the "Other k-quants" table prints 6.6 bits per weight.
    qk, bb = o.block_info("q6_k")
    assert qk == 256 and round(bb * 8 / qk, 1) == 6.6
    # Q8_0 (Q4_0 structure, 8-bit codes) and Q5_0 (4+1 bit codes).
    assert o.block_info("q8_0") == (32, 2 + 32)
    assert o.block_info("q5_0") == (32, 2 + 4 + 16)
    # Q4_1: Q4_0's block plus an fp16 min (5.0 bpw); Q5_K: Q4_K plus one fifth
    # bit per weight, 5.5 bpw, inside the table's 5.5-5.7 for Q5_K_S / _M.
    assert o.block_info("q4_1") == (32, 2 + 2 + 16)
    qk, bb = o.block_info("q5_k")
    assert qk == 256 and bb == 144 + 256 // 8 and 5.5 <= bb * 8 / qk <= 5.7
    # Q2_K and Q3_K (same table: 2.5-2.6 and 3.4-4.0 bits per weight on
    # 256-weight super-blocks): 2-bit codes with 4-bit scales and mins per 16
    # weights plus fp16 d and dmin; 3-bit codes with 6-bit scales per 16
    # weights plus fp16 d.
    qk, bb = o.block_info("q2_k")
    assert qk == 256 and bb == 2 + 2 + 16 + 64 and 2.5 <= round(bb * 8 / qk, 1) <= 2.6
    qk, bb = o.block_info("q3_k")
    assert qk == 256 and bb == 2 + 12 + 64 + 32 and 3.4 <= bb * 8 / qk <= 4.0


def _exact_dot(w64, x):
    out = []
    for r in range(w64.shape[0]):
        s = Fraction(0)
        sa = Fraction(0)
        for c in range(w64.shape[1]):
            p = Fraction(float(w64[r, c])) * Fraction(float(x[c]))
            s += p
            sa += abs(p)
        out.append((s, sa))
    return out


def pin_fraction_dot(o):
    """fp64 dot within the sequential-summation bound of the exact rational dot."""
    for k, t in enumerate(QTYPES):
        qk, _ = o.block_info(t)
        rows, cols = 3, 2 * qk
        w = synth.weights(rows, cols, seed=100 + k, outlier_frac=0.05)
        blob = o.quantize(w, t)
        w64 = o.dequant_f64(blob, t, rows, cols)
        x = synth.dyadic((2, cols), seed=200 + k)
        y, yabs = o.matmul_f64(blob, t, rows, cols, x)
        for tok in range(2):
            for r, (s, sa) in enumerate(_exact_dot(w64, x[tok])):
                bound = cols * 2.0 ** -53 * float(sa)
                assert abs(Fraction(y[tok, r]) - s) <= Fraction(bound), (t, tok, r)
                assert abs(Fraction(yabs[tok, r]) - sa) <= Fraction(bound), (t, tok, r)


def _q8_blob(codes: np.ndarray) -> np.ndarray:
    """Q8_0 blob with d = 1.0 (fp16 0x3C00) and the given int8 codes [rows, cols]."""
    rows, cols = codes.shape
    blocks = codes.reshape(rows, cols // 32, 32).astype(np.int8).view(np.uint8)
    head = np.zeros((rows, cols // 32, 2), dtype=np.uint8)
    head[..., 0], head[..., 1] = 0x00, 0x3C
    return np.concatenate([head, blocks], axis=2).reshape(-1)


def pin_q8_integer(o):
    """Q8_0 with d = 1 and integer x is an exact integer matrix product."""
    rng = np.random.default_rng(7)
    rows, cols, n = 5, 96, 3
    codes = rng.integers(-128, 128, size=(rows, cols))
    xi = rng.integers(-1000, 1000, size=(n, cols))
    y, _ = o.matmul_f64(_q8_blob(codes), "q8_0", rows, cols, xi.astype(np.float64))
    assert np.array_equal(y, (xi @ codes.T).astype(np.float64))


def _q4k_const_blob(d16, dmin16, sc, mn, code):
    """One Q4_K block whose 256 codes all equal ``code`` (layout-order free)."""
    v = 0
    for i in range(8):
        v |= sc[i] << (12 * i)
        v |= mn[i] << (12 * i + 6)
    head = bytes([d16 & 0xFF, d16 >> 8, dmin16 & 0xFF, dmin16 >> 8]) + v.to_bytes(12, "little")
    return np.frombuffer(head + bytes([code | (code << 4)]) * 128, dtype=np.uint8)


def pin_q4k_structured(o):
    """Constant codes: y = sum_i (d*sc_i*c - dmin*m_i) * (sum of x over sub-block i)."""
    sc = [3, 60, 17, 1, 44, 9, 33, 25]
    mn = [5, 0, 63, 12, 7, 30, 2, 48]
    d, dmin = 0.0078125, 0.001953125          # fp16 0x2000, 0x1800
    x = synth.dyadic((1, 256), seed=11)
    for code in (0, 5, 15):
        blob = _q4k_const_blob(0x2000, 0x1800, sc, mn, code)
        y, _ = o.matmul_f64(blob, "q4_k", 1, 256, x)
        want = sum((d * sc[i] * code - dmin * mn[i]) * x[0, 32 * i:32 * i + 32].sum()
                   for i in range(8))
        assert abs(y[0, 0] - want) <= 1e-12 * max(1.0, abs(want)), (code, y[0, 0], want)


def pin_pow2_and_perm(o):
    """Doubling d (and dmin) doubles y exactly; permuting rows permutes y."""
    offs = {"q4_0": [0], "q5_0": [0], "q8_0": [0], "q4_k": [0, 2], "q6_k": [0], "q4_1": [0, 2],
            "q5_k": [0, 2], "q2_k": [0, 2], "q3_k": [0]}
    for k, t in enumerate(QTYPES):
        qk, bb = o.block_info(t)
        rows, cols = 6, 2 * qk
        w = synth.weights(rows, cols, seed=300 + k)
        blob = o.quantize(w, t)
        x = synth.activations(2, cols, seed=400 + k).astype(np.float64)
        y, _ = o.matmul_f64(blob, t, rows, cols, x)
        b2 = blob.copy().reshape(-1, bb)
        for off in offs[t]:
            h = b2[:, off].astype(np.uint16) | (b2[:, off + 1].astype(np.uint16) << 8)
            mag = h & 0x7FFF
            assert np.all((mag >> 10) < 30)               # room for one more exponent step
            # normal: exponent + 1; subnormal (and zero): the encoding doubles
            h = np.where(mag >= 0x0400, h + 0x0400, (h & 0x8000) | (mag << 1)).astype(np.uint16)
            b2[:, off] = (h & 0xFF).astype(np.uint8)
            b2[:, off + 1] = (h >> 8).astype(np.uint8)
        y2, _ = o.matmul_f64(b2.reshape(-1), t, rows, cols, x)
        assert np.array_equal(y2, 2.0 * y), t
        rb = cols // qk * bb
        perm = np.random.default_rng(k).permutation(rows)
        bp = blob.reshape(rows, rb)[perm].reshape(-1)
        yp, _ = o.matmul_f64(bp, t, rows, cols, x)
        assert np.array_equal(yp, y[:, perm]), t
        # n tokens in one call equal one call per token
        for tok in range(2):
            y1, _ = o.matmul_f64(blob, t, rows, cols, x[tok:tok + 1])
            assert np.array_equal(y1[0], y[tok]), t


def pin_f32_is_one_rounding(o):
    """The fp32 dequant rounds at most once: it equals fp32(fp64 dequant)."""
    for k, t in enumerate(QTYPES):
        qk, _ = o.block_info(t)
        rows, cols = 8, 4 * qk
        w = synth.weights(rows, cols, seed=500 + k, outlier_frac=0.01)
        blob = o.quantize(w, t)
        w32 = o.dequant_f32(blob, t, rows, cols)
        w64 = o.dequant_f64(blob, t, rows, cols)
        assert np.array_equal(w32, w64.astype(np.float32)), t


def _roundtrip_bound(w: np.ndarray, t: str) -> np.ndarray:
    """Per-weight bound on |w - dequant(quantize(w))| from the quantizer's
    definition (covering fp16 scales rounded up by at most 2^-10 relative,
    codes rounded to nearest)."""
    up = 1.0 + 2.0 ** -9
    w = w.astype(np.float64)
    if t in ("q4_0", "q5_0", "q8_0"):
        L = {"q4_0": 7, "q5_0": 15, "q8_0": 127}[t]
        a = np.abs(w.reshape(-1, 32)).max(axis=1, keepdims=True)
        d = a / L * up + 2.0 ** -24
        return np.broadcast_to(d / 2, (a.shape[0], 32)).reshape(w.shape)
    if t in ("q6_k", "q3_k"):
        L, F = (31.0, 127.0) if t == "q6_k" else (3.0, 63.0)
        ts = np.abs(w.reshape(-1, 16, 16)).max(axis=2, keepdims=True) / L
        d = ts.max(axis=1, keepdims=True) / F * up + 2.0 ** -24                 # [blocks,1,1]
        step = ts + d
        return np.broadcast_to(step / 2, (ts.shape[0], 16, 16)).reshape(w.shape)
    if t == "q4_1":
        b = w.reshape(-1, 32)
        lo, hi = b.min(axis=1, keepdims=True), b.max(axis=1, keepdims=True)
        span = (hi - lo) + np.abs(lo) * 2.0 ** -10 + 2.0 ** -24      # m is an fp16 <= lo
        d = span / 15.0 * up + 2.0 ** -24
        return np.broadcast_to(d / 2, b.shape).reshape(w.shape)
    # q4_k, q5_k, q2_k
    L = {"q5_k": 31.0, "q4_k": 15.0, "q2_k": 3.0}[t]
    F = 15.0 if t == "q2_k" else 63.0              # levels of the scale and min fields
    n = 16 if t == "q2_k" else 8                   # sub-blocks per super-block
    sb = w.reshape(-1, n, 256 // n)
    lo = np.minimum(sb.min(axis=2), 0.0)
    hi = sb.max(axis=2)
    M = -lo
    dmin = M.max(axis=1, keepdims=True) / F * up + 2.0 ** -24
    sp = (hi + M + dmin) / L
    d = sp.max(axis=1, keepdims=True) / F * up + 2.0 ** -24
    step = sp + d
    return np.broadcast_to((step / 2)[..., None], sb.shape).reshape(w.shape)


def pin_roundtrip(o):
    """Quantize -> dequantize stays within half a quantization step."""
    for k, t in enumerate(QTYPES):
        qk, _ = o.block_info(t)
        rows, cols = 16, 4 * qk
        for frac in (0.0, 0.01):
            w = synth.weights(rows, cols, seed=600 + k, outlier_frac=frac)
            blob = o.quantize(w, t)
            err = np.abs(o.dequant_f64(blob, t, rows, cols) - w.astype(np.float64))
            bound = _roundtrip_bound(w, t) * (1 + 1e-9) + 1e-12
            assert np.all(err <= bound), (t, frac, float((err / bound).max()))
        # special blocks: all zero, all equal, all positive
        for w in (np.zeros((1, qk), np.float32), np.full((1, qk), 0.03, np.float32),
                  np.abs(synth.weights(1, qk, seed=7))):
            blob = o.quantize(w, t)
            err = np.abs(o.dequant_f64(blob, t, 1, qk) - w.astype(np.float64))
            assert np.all(err <= _roundtrip_bound(w, t) * (1 + 1e-9) + 1e-12), t


def _f16_field(blob, off):
    return int(blob[off]) | (int(blob[off + 1]) << 8)


def pin_quantize_saturation(o):
    """A block whose absmax needs a scale above the largest finite fp16
    (65504) stores 65504 (0x7BFF), not Inf, and its extreme codes clamp at
    the ends of their range, so its weights decode finite with the extremes
    at the largest magnitudes the fields allow; an in-range block of the same
    shape still meets the round trip.  Block: a ramp from -A to A with A four
    times the largest magnitude the type can represent."""
    top = 65504.0
    big = {"q4_0": top * 7, "q5_0": top * 15, "q8_0": top * 127, "q6_k": top * 127 * 31,
           "q4_k": top * 63 * 15, "q5_k": top * 63 * 31, "q4_1": top * 16,
           "q2_k": top * 15 * 3, "q3_k": top * 63 * 3}
    for t in QTYPES:
        qk, _ = o.block_info(t)
        ramp = np.linspace(-1.0, 1.0, qk)
        w = (ramp * 4.0 * big[t]).astype(np.float32)[None, :]
        blob = o.quantize(w, t)
        assert _f16_field(blob, 0) == 0x7BFF, (t, hex(_f16_field(blob, 0)))
        w64 = o.dequant_f64(blob, t, 1, qk)[0]
        assert np.all(np.isfinite(w64)), t
        if t in ("q4_k", "q5_k"):
            assert _f16_field(blob, 2) == 0x7BFF, (t, "dmin")
            # sub-block 0 all negative: code 0 at min 63; sub-block 7 all
            # positive: the top code at scale 63, min 0
            top_code = 31 if t == "q5_k" else 15
            assert w64[0] == -top * 63 and w64[-1] == top * 63 * top_code, (t, w64[0], w64[-1])
        elif t == "q4_1":
            # the min saturates at -65504 (0xFBFF), codes 0 and 15 at the ends
            assert _f16_field(blob, 2) == 0xFBFF, (t, hex(_f16_field(blob, 2)))
            assert w64[0] == -top and w64[-1] == 14 * top, (t, w64[0], w64[-1])
        elif t == "q6_k":
            assert int(blob[2]) == 127 and int(blob[2 + 15]) == 127, t      # scales clamp at 127
            assert w64[0] == -big[t] and w64[-1] == big[t], t
        elif t == "q2_k":
            # min and scale fields clamp at 15: sub-block 0 all negative ends at
            # code 0 under min 15, sub-block 15 all positive at code 3, scale 15
            assert _f16_field(blob, 2) == 0x7BFF, (t, "dmin")
            assert int(blob[4]) >> 4 == 15 and int(blob[4 + 15]) & 15 == 15, t
            assert w64[0] == -top * 15 and w64[-1] == big[t], (t, w64[0], w64[-1])
        elif t == "q3_k":
            assert int(blob[2]) & 63 == 63, t                                # scale 0 at 63
            assert w64[0] == -big[t] and w64[-1] == big[t], (t, w64[0], w64[-1])
        else:
            assert w64[0] == -big[t] and w64[-1] == big[t], (t, w64[0], w64[-1])
        assert np.all(np.abs(w64) <= big[t]), t
        wi = (ramp * 0.05).astype(np.float32)[None, :]
        bi = o.quantize(wi, t)
        err = np.abs(o.dequant_f64(bi, t, 1, qk) - wi.astype(np.float64))
        assert np.all(err <= _roundtrip_bound(wi, t) * (1 + 1e-9) + 1e-12), t


def pin_rmsnorm(o):
    """RMSNorm ("How LLM Inference Engines Work", "RMSNorm") against closed
    forms and invariants: x = (3, 4) has mean square 12.5, so eps = 3.5 gives
    the scale 1/sqrt(16) = 1/4 exactly; a constant vector with eps = 0
    normalizes to its sign; with eps = 0 a positive rescaling of x changes
    nothing and the output's mean square (unit weights) is 1; the weights
    multiply elementwise; fp16 inputs round x*s to binary16 (NumPy's) first."""
    out = o.rmsnorm_f64(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 3.5)
    assert np.array_equal(out, np.array([0.75, 2.0])), out
    out = o.rmsnorm_f64(np.full(7, -2.5), np.ones(7), 0.0)
    assert np.array_equal(out, np.full(7, -1.0)), out
    rng = np.random.default_rng(11)
    x = rng.standard_normal(4096)
    w = rng.standard_normal(4096)
    a = o.rmsnorm_f64(x, np.ones(4096), 0.0)
    assert abs(np.mean(a * a) - 1.0) < 1e-12
    b = o.rmsnorm_f64(x * 37.0, np.ones(4096), 0.0)
    assert np.allclose(a, b, rtol=1e-13, atol=0)
    c = o.rmsnorm_f64(x, w, 1e-5)
    assert np.allclose(c, o.rmsnorm_f64(x, np.ones(4096), 1e-5) * w, rtol=1e-15, atol=0)
    # eps enters as mean + eps: x = 0 stays 0 (and finite) for eps > 0
    assert np.array_equal(o.rmsnorm_f64(np.zeros(5), np.ones(5), 1e-6), np.zeros(5))
    xh = rng.standard_normal(1000).astype(np.float16).astype(np.float64)
    s = 1.0 / np.sqrt(np.mean(xh * xh) + 1e-5)
    got = o.rmsnorm_f64(xh, np.ones(1000), 1e-5, half_x=True)
    ref = (xh * s).astype(np.float32).astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref), int(np.sum(got != ref))


def pin_swiglu(o):
    """SiLU ("SwiGLU Feed-Forward Network") against identities and closed
    forms: silu(0) = 0; silu(v) - silu(-v) = v (sigmoid(v) + sigmoid(-v) = 1);
    sigmoid(ln 3) = 3/4 so silu(ln 3) = (3/4) ln 3; silu(v) ~ v for large v and
    ~ 0 for very negative v; the up projection multiplies elementwise."""
    v = np.linspace(-30, 30, 601)
    one = np.ones_like(v)
    sp, sn = o.swiglu_f64(v, one), o.swiglu_f64(-v, one)
    assert np.allclose(sp - sn, v, rtol=0, atol=1e-12)
    assert o.swiglu_f64(np.array([0.0]), np.array([5.0]))[0] == 0.0
    l3 = np.log(3.0)
    assert abs(o.swiglu_f64(np.array([l3]), np.array([1.0]))[0] - 0.75 * l3) < 1e-15
    assert abs(o.swiglu_f64(np.array([50.0]), np.array([1.0]))[0] - 50.0) < 1e-12
    assert abs(o.swiglu_f64(np.array([-50.0]), np.array([1.0]))[0]) < 1e-18
    u = np.linspace(-2, 3, 601)
    assert np.allclose(o.swiglu_f64(v, u), sp * u, rtol=1e-15, atol=0)


def _q8_rows(codes, d_bits=0x3C00):
    """Q8_0 blob from int8 codes [rows][32k] with one fp16 scale per block
    (the Hitchhiker's Guide §11.1 layout: fp16 d, then the codes); d = 1.0
    by default (0x3C00)."""
    codes = np.asarray(codes, dtype=np.int64)
    rows, cols = codes.shape
    out = bytearray()
    for r in range(rows):
        for b in range(cols // 32):
            out += int(d_bits).to_bytes(2, "little")
            out += bytes((int(v) & 0xFF) for v in codes[r, 32 * b:32 * b + 32])
    return np.frombuffer(bytes(out), dtype=np.uint8)


def pin_attention(o):
    """Decode attention over a quantized KV cache ("How LLM Inference Engines
    Work", "Grouped-Query Attention (GQA) and KV Cache") against closed
    forms: one cached position gives its value row exactly (softmax of one
    score is 1); a zero query scores every position 0, so the output is the
    mean of the value rows; two positions whose scores differ by D weigh
    their values 1 : exp(D), with D = q.k / sqrt(head_dim); when each KV
    head's values are the constant g + 1, query head h returns
    h // (n_heads / n_kv) + 1 (the head mapping of the page's expand); and
    permuting the cached positions changes nothing."""
    rng = np.random.default_rng(21)
    hd, n_kv, n_heads = 64, 4, 8
    # one position
    k1 = _q8_rows(rng.integers(-127, 128, (n_kv, hd)))
    v1 = _q8_rows(rng.integers(-127, 128, (n_kv, hd)))
    q = rng.standard_normal((n_heads, hd))
    out = o.attn_decode_f64(k1, v1, "q8_0", 1, n_kv, hd, q)
    vd = o.dequant_f64(v1, "q8_0", n_kv, hd)
    assert np.array_equal(out, vd[np.arange(n_heads) // 2]), "one position"
    # zero query: the mean of the values
    T = 37
    kc = _q8_rows(rng.integers(-127, 128, (T * n_kv, hd)))
    vc = _q8_rows(rng.integers(-127, 128, (T * n_kv, hd)))
    out = o.attn_decode_f64(kc, vc, "q8_0", T, n_kv, hd, np.zeros((n_heads, hd)))
    vd = o.dequant_f64(vc, "q8_0", T * n_kv, hd).reshape(T, n_kv, hd)
    ref = vd.mean(axis=0)[np.arange(n_heads) // 2]
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-13), "zero query"
    # two positions, one head: K0 = 0, K1 = c at dim 5; q = a at dim 5
    c, a = 90, 0.37
    kk = np.zeros((2, 32), dtype=np.int64)
    kk[1, 5] = c
    vv = np.array([[-40] * 32, [100] * 32])
    qq = np.zeros((1, 32))
    qq[0, 5] = a
    out = o.attn_decode_f64(_q8_rows(kk), _q8_rows(vv), "q8_0", 2, 1, 32, qq)
    D = a * c / np.sqrt(32.0)
    ref = (-40.0 + 100.0 * np.exp(D)) / (1.0 + np.exp(D))
    assert np.allclose(out, ref, rtol=1e-14, atol=0), (out[0, 0], ref)
    # head mapping: V of KV head g is the constant g + 1
    vg = np.array([[g + 1] * hd for t in range(T) for g in range(n_kv)])
    out = o.attn_decode_f64(kc, _q8_rows(vg), "q8_0", T, n_kv, hd, q)
    ref = (np.arange(n_heads) // 2 + 1.0)[:, None] * np.ones((1, hd))
    assert np.allclose(out, ref, rtol=1e-14, atol=0), "head mapping"
    # permutation of positions
    perm = rng.permutation(T)
    rb = o.row_bytes("q8_0", hd)
    kr = kc.reshape(T, n_kv * rb)[perm].reshape(-1)
    vr = vc.reshape(T, n_kv * rb)[perm].reshape(-1)
    a1 = o.attn_decode_f64(kc, vc, "q8_0", T, n_kv, hd, q)
    a2 = o.attn_decode_f64(kr, vr, "q8_0", T, n_kv, hd, q)
    assert np.allclose(a1, a2, rtol=1e-12, atol=1e-12), "position permutation"


ALL_PINS = [pin_golden, pin_sizes, pin_fraction_dot, pin_q8_integer, pin_q4k_structured,
            pin_quantize_saturation,
            pin_pow2_and_perm, pin_f32_is_one_rounding, pin_roundtrip, pin_rmsnorm, pin_swiglu,
            pin_attention]
