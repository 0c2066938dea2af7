"""Writes the hand-built block fixtures in this folder.

Each fixture is one block whose fields are chosen by hand (listed in the
fixture), packed into bytes by the byte layout the pages give or, where they
are silent, by the reading stated in the fixture, together with the weights
the pages' dequantization formula gives for those fields.  The packing here is
written independently of the oracle (plain integer bit placement from field
values), and the expected weights come from the formula on the fields, never
from a decoder.  Nothing here calls the oracle or the GPU library.

Run: python tests/golden/make_golden.py   (rewrites the *.json fixtures)
"""
from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def f16_bits_of(value: Fraction) -> int:
    """Encoding of an fp16 that represents ``value`` exactly (asserted)."""
    import numpy as np
    h = np.float16(float(value))
    assert Fraction(float(h)) == value, value
    return int(h.view(np.uint16))


def frac_f32(v: Fraction) -> float:
    """Round an exact rational to fp32 (via fp64, exact for these values)."""
    import numpy as np
    f = float(v)
    assert Fraction(f) == v                  # fits fp64 exactly
    return float(np.float32(f))


def dump(name, obj):
    with open(os.path.join(HERE, name), "w") as fh:
        json.dump(obj, fh, indent=1)
        fh.write("\n")


def q4_0():
    d = Fraction(1, 2)
    codes = [j for j in range(16)] + [15 - j for j in range(16)]   # element -> code
    raw = struct.pack("<H", f16_bits_of(d))
    raw += bytes((codes[j] & 15) | ((codes[j + 16] & 15) << 4) for j in range(16))
    exp = [d * (q - 8) for q in codes]
    dump("q4_0_ramp.json", {
        "type": "q4_0",
        "citation": "How LLM Inference Engines Work, 'Loading GGUF Models' (18-byte "
                    "block: fp16 scale, then 16 bytes whose low nibbles are elements "
                    "0..15 and high nibbles elements 16..31, offset -8); Hitchhiker's "
                    "Guide Lab 01 §11.1, Q4_0 block figure (w ~= d*(q-8)).",
        "fields": {"d": str(d), "codes": codes},
        "hex": raw.hex(),
        "expected": [float(v) for v in exp],
        "expected_f32": [frac_f32(v) for v in exp],
    })


def q8_0():
    d = Fraction(1, 4)
    codes = [((37 * j) % 256) - 128 for j in range(32)]
    raw = struct.pack("<H", f16_bits_of(d)) + bytes(q & 0xFF for q in codes)
    exp = [d * q for q in codes]
    dump("q8_0_signed.json", {
        "type": "q8_0",
        "citation": "Hitchhiker's Guide Lab 01 §11.1: Q8_0 has the Q4_0 structure with "
                    "8-bit codes. Reading: fp16 d first, then 32 two's-complement int8 "
                    "codes, w = d*q.",
        "fields": {"d": str(d), "codes": codes},
        "hex": raw.hex(),
        "expected": [float(v) for v in exp],
        "expected_f32": [frac_f32(v) for v in exp],
    })


def q5_0():
    d = Fraction(1, 8)
    codes = [(7 * j + 3) % 32 for j in range(32)]
    qh = 0
    for j, q in enumerate(codes):
        qh |= ((q >> 4) & 1) << j
    raw = struct.pack("<HI", f16_bits_of(d), qh)
    raw += bytes((codes[j] & 15) | ((codes[j + 16] & 15) << 4) for j in range(16))
    exp = [d * (q - 16) for q in codes]
    dump("q5_0_mixed.json", {
        "type": "q5_0",
        "citation": "Local LLM inference, 'The mmap backend' names Q5_0 in the Q4_K_M "
                    "recipe; the layout is not on the pages. Reading: fp16 d, a "
                    "little-endian 32-bit word whose bit j is bit 4 of code j, then 16 "
                    "bytes of low nibbles in the Q4_0 order of 'Loading GGUF Models'; "
                    "w = d*(q-16).",
        "fields": {"d": str(d), "codes": codes},
        "hex": raw.hex(),
        "expected": [float(v) for v in exp],
        "expected_f32": [frac_f32(v) for v in exp],
    })


def pack6(fields):
    """16 six-bit fields, LSB-first, as one 96-bit little-endian integer."""
    v = 0
    for k, f in enumerate(fields):
        assert 0 <= f < 64
        v |= f << (6 * k)
    return v.to_bytes(12, "little")


def q4_k(name, d, dmin, sc, mn, lo_nib, hi_nib, note):
    fields = []
    for i in range(8):
        fields += [sc[i], mn[i]]
    raw = struct.pack("<HH", f16_bits_of(d), f16_bits_of(dmin)) + pack6(fields)
    codes = [0] * 256
    qs = bytearray()
    for i in range(8):
        for k in range(16):
            a, b = lo_nib(i, k), hi_nib(i, k)
            codes[32 * i + k] = a
            codes[32 * i + k + 16] = b
            qs.append(a | (b << 4))
    raw += bytes(qs)
    assert len(raw) == 144
    exp = [(d * sc[j // 32]) * codes[j] - dmin * mn[j // 32] for j in range(256)]
    dump(name, {
        "type": "q4_k",
        "citation": "Hitchhiker's Guide Lab 01 §11.2 (Q4_K super-block figure: d, dmin, "
                    "8 six-bit scales + 8 six-bit mins, 256 four-bit codes; w = (d*sc)*q "
                    "- dmin*m) and 12 — llama.cpp / GGUF, 'Q4_K_M — bit layout in "
                    "exquisite detail' (field sizes 2+2+12+128 = 144 B; sub-block i uses "
                    "6-bit fields 2i (scale) and 2i+1 (min)). Readings: the 16 fields "
                    "are one LSB-first 96-bit little-endian stream; sub-block i owns "
                    "code bytes 16i..16i+15 in the Q4_0 nibble order. " + note,
        "fields": {"d": str(d), "dmin": str(dmin), "sc": sc, "m": mn, "codes": codes},
        "hex": raw.hex(),
        "expected": [float(v) for v in exp],
        "expected_f32": [frac_f32(v) for v in exp],
    })


def q6_k():
    d = Fraction(1, 1024)
    sc = [8 * s - 60 for s in range(16)]
    codes = [(11 * j + 5) % 64 for j in range(256)]
    raw = struct.pack("<H", f16_bits_of(d)) + bytes(s & 0xFF for s in sc)
    ql = bytearray()
    qh = bytearray()
    for g in range(8):
        for k in range(16):
            ql.append((codes[32 * g + k] & 15) | ((codes[32 * g + k + 16] & 15) << 4))
    for g in range(8):
        for k in range(8):
            h = 0
            for u in range(4):
                h |= ((codes[32 * g + k + 8 * u] >> 4) & 3) << (2 * u)
            qh.append(h)
    raw += bytes(ql) + bytes(qh)
    assert len(raw) == 210
    exp = [d * (sc[j // 16] * (codes[j] - 32)) for j in range(256)]
    dump("q6_k_signed.json", {
        "type": "q6_k",
        "citation": "12 — llama.cpp / GGUF, table 'Other k-quants at a glance': Q6_K is "
                    "6.6 bits per weight over a 256-weight super-block; the layout is "
                    "not on the pages. Reading: fp16 d; 16 signed int8 scales (one per "
                    "16 weights); 128 bytes of low nibbles (Q4_0 order per 32-weight "
                    "group); 64 bytes of 2-bit high parts, byte 8g+k holding elements "
                    "32g+k+8u at bits 2u..2u+1; w = d*(sc*(q-32)); 210 B = 6.5625 bpw.",
        "fields": {"d": str(d), "sc": sc, "codes": codes},
        "hex": raw.hex(),
        "expected": [float(v) for v in exp],
        "expected_f32": [frac_f32(v) for v in exp],
    })


def q4_1():
    d, m = Fraction(3, 16), Fraction(-5, 4)
    codes = [(9 * j + 2) % 16 for j in range(32)]
    raw = struct.pack("<HH", f16_bits_of(d), f16_bits_of(m) if m >= 0 else
                      0x8000 | f16_bits_of(-m))
    raw += bytes(codes[j] | (codes[j + 16] << 4) for j in range(16))
    assert len(raw) == 20
    exp = [d * q + m for q in codes]
    dump("q4_1_min.json", {
        "type": "q4_1",
        "citation": "How LLM Inference Engines Work, 'Loading GGUF Models' names Q4_1 "
                    "among the GGUF formats; the layout is not on the pages. Reading: the "
                    "Q4_0 block of that section with a signed fp16 min after the fp16 "
                    "scale (the asymmetric range of Hitchhiker's Guide §11.2 item 2): "
                    "d, m, then 16 bytes of codes in Q4_0 nibble order; w = d*q + m; "
                    "20 B per 32 weights = 5.0 bpw.",
        "fields": {"d": str(d), "m": str(m), "codes": codes},
        "hex": raw.hex(),
        "expected": [float(v) for v in exp],
        "expected_f32": [frac_f32(v) for v in exp],
    })


def q5_k():
    d, dmin = Fraction(1, 128), Fraction(3, 256)
    sc = [62 - 7 * i for i in range(8)]
    mn = [9 * i for i in range(8)]
    codes = [(13 * j + 7) % 32 for j in range(256)]
    fields = []
    for i in range(8):
        fields += [sc[i], mn[i]]
    raw = struct.pack("<HH", f16_bits_of(d), f16_bits_of(dmin)) + pack6(fields)
    qh = 0
    for e, q in enumerate(codes):
        qh |= ((q >> 4) & 1) << e
    raw += qh.to_bytes(32, "little")
    for i in range(8):
        for k in range(16):
            raw += bytes([(codes[32 * i + k] & 15) | ((codes[32 * i + k + 16] & 15) << 4)])
    assert len(raw) == 176
    exp = [(d * sc[j // 32]) * codes[j] - dmin * mn[j // 32] for j in range(256)]
    dump("q5_k_fields.json", {
        "type": "q5_k",
        "citation": "12 — llama.cpp / GGUF, table 'Other k-quants at a glance': Q5_K_S / _M "
                    "at 5.5-5.7 bits per weight over a 256-weight super-block; the layout "
                    "is not on the pages. Reading: the Q4_K super-block of Hitchhiker's "
                    "Guide §11.2 (d, dmin, 16 six-bit fields as one LSB-first 96-bit "
                    "stream, field 2i scale and 2i+1 min of sub-block i) with a 32-byte "
                    "plane of fifth bits after the fields (bit e of the little-endian "
                    "256-bit plane is bit 4 of element e's code, as Q5_0's 32-bit word), "
                    "then the 128 code bytes in Q4_0 nibble order per sub-block; "
                    "w = (d*sc)*q - dmin*m with q in 0..31; 176 B = 5.5 bpw.",
        "fields": {"d": str(d), "dmin": str(dmin), "sc": sc, "m": mn, "codes": codes},
        "hex": raw.hex(),
        "expected": [float(v) for v in exp],
        "expected_f32": [frac_f32(v) for v in exp],
    })


def plane2(codes):
    """64 bytes of 2-bit fields: byte 8g+k holds elements 32g+k+8u at bits 2u..2u+1."""
    out = bytearray()
    for g in range(8):
        for k in range(8):
            v = 0
            for u in range(4):
                c = codes[32 * g + k + 8 * u]
                assert 0 <= c < 4
                v |= c << (2 * u)
            out.append(v)
    return bytes(out)


def q2_k():
    d, dmin = Fraction(1, 64), Fraction(3, 512)
    sc = [15 - s for s in range(16)]                      # 15 .. 0
    mn = [(7 * s + 3) % 16 for s in range(16)]
    codes = [(7 * e + e // 32) % 4 for e in range(256)]
    raw = struct.pack("<HH", f16_bits_of(d), f16_bits_of(dmin))
    raw += bytes(sc[s] | (mn[s] << 4) for s in range(16))
    raw += plane2(codes)
    assert len(raw) == 84
    exp = [(d * sc[e // 16]) * codes[e] - dmin * mn[e // 16] for e in range(256)]
    dump("q2_k_fields.json", {
        "type": "q2_k",
        "citation": "12 — llama.cpp / GGUF, table 'Other k-quants at a glance': Q2_K at "
                    "2.5-2.6 bits per weight over a 256-weight super-block; the layout is "
                    "not on the pages. Reading: the two-level scale/min recipe of "
                    "Hitchhiker's Guide §11.2 at 2 bits: fp16 d, fp16 dmin, 16 bytes whose "
                    "low nibble is the scale and high nibble the min of a 16-weight "
                    "sub-block, then 64 bytes of 2-bit codes, byte 8g+k holding elements "
                    "32g+k+8u at bits 2u..2u+1; w = (d*sc)*q - dmin*m with q in 0..3; "
                    "84 B = 2.625 bpw.",
        "fields": {"d": str(d), "dmin": str(dmin), "sc": sc, "m": mn, "codes": codes},
        "hex": raw.hex(),
        "expected": [float(v) for v in exp],
        "expected_f32": [frac_f32(v) for v in exp],
    })


def q3_k():
    d = Fraction(1, 32)
    sc = [63, 0] + [4 * s + 1 for s in range(14)]
    codes = [(3 * e + e // 16) % 8 for e in range(256)]
    raw = struct.pack("<H", f16_bits_of(d)) + pack6(sc)
    raw += plane2([c & 3 for c in codes])
    qh = 0
    for e, c in enumerate(codes):
        qh |= ((c >> 2) & 1) << e
    raw += qh.to_bytes(32, "little")
    assert len(raw) == 110
    exp = [d * (sc[e // 16] * (codes[e] - 4)) for e in range(256)]
    dump("q3_k_fields.json", {
        "type": "q3_k",
        "citation": "12 — llama.cpp / GGUF, table 'Other k-quants at a glance': Q3_K_S / _M "
                    "/ _L at 3.4-4.0 bits per weight over a 256-weight super-block; the "
                    "layout is not on the pages. Reading: symmetric like Q6_K: fp16 d, 16 "
                    "unsigned six-bit scales (one per 16 weights) as one LSB-first 96-bit "
                    "stream, 64 bytes of the codes' low 2 bits (byte 8g+k holding elements "
                    "32g+k+8u at bits 2u..2u+1), then a 32-byte plane whose bit e is bit 2 "
                    "of element e's code; w = d*(sc*(q-4)) with q in 0..7; 110 B = "
                    "3.4375 bpw.",
        "fields": {"d": str(d), "sc": sc, "codes": codes},
        "hex": raw.hex(),
        "expected": [float(v) for v in exp],
        "expected_f32": [frac_f32(v) for v in exp],
    })


if __name__ == "__main__":
    q4_0()
    q8_0()
    q5_0()
    q4_k("q4_k_fields.json", Fraction(1, 256), Fraction(1, 512),
         [63 - 5 * i for i in range(8)], [7 * i + 5 for i in range(8)],
         lambda i, k: (k + i) % 16, lambda i, k: (5 * k + 3 * i + 1) % 16,
         "Scales 63..28 and mins 5..54 use all six bits of each field.")
    # d = 1, dmin = the smallest normal fp16 plus one ulp: a*q - b needs ~33 bits,
    # so the fp32 dequant rounds exactly once (expected_f32 is that rounding).
    q4_k("q4_k_rounding.json", Fraction(1), Fraction(1025, 1024 * 16384),
         [63, 1, 17, 40, 63, 2, 33, 9], [63, 63, 1, 30, 0, 62, 45, 7],
         lambda i, k: 15 - (k % 16), lambda i, k: (k * 3) % 16,
         "Extreme fields: d = 1.0, dmin = 2^-14 * 1025/1024, so the single fp32 "
         "rounding of a*q - b is exercised.")
    q6_k()
    q4_1()
    q5_k()
    q2_k()
    q3_k()
