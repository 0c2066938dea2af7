/*
 * gqo.c — plain, slow CPU oracle for GGUF block-quantized matmul.
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, the smoke check and bench.py's
 * CPU-baseline leg, never by the GPU library, which shares no code with it.
 *
 * Sources (page title, then section / figure):
 *  [HG]  "Hitchhiker's Guide — Lab 01: Air-Gapped LLM Serving",
 *        §11.1 (block-wise scales, w ~= d*q; Q4_0 block figure; Q8_0 "same
 *        structure with 8-bit codes") and §11.2 (Q4_K super-block figure and
 *        its dequant formula; two-level scales; asymmetric mins).
 *  [LC]  "12 — llama.cpp / GGUF / Local Inference Mastery", section
 *        "Q4_K_M — bit layout in exquisite detail" (field sizes, per-sub-block
 *        dequant pseudo-code with fields 2i / 2i+1) and the table
 *        "Other k-quants at a glance" (Q6_K: 6.6 bits per weight, 256 weights).
 *  [NL]  "How LLM Inference Engines Work", section "Loading GGUF Models"
 *        (Q4_0 decoder: fp16 scale first, low nibbles are elements 0..15,
 *        high nibbles elements 16..31, offset -8).
 *  [LK]  "Local LLM inference (experimental, --features llm)", section
 *        "The mmap backend" (Q4_K_M mixes Q4_K, Q5_0, Q6_K, Q8_0, F32 and
 *        dequantizes every block inside the dot product).
 *  [NL]  also sections "RMSNorm" (scale by the reciprocal root of the mean
 *        square plus eps, computed in float32, the product cast back to the
 *        input's type, then times the weight) and "SwiGLU Feed-Forward
 *        Network" (SiLU of the gate projection times the up projection).
 *  [NL]  also section "Grouped-Query Attention (GQA) and KV Cache" (scores
 *        q.k / sqrt(head_dim) over the cached positions, softmax, the
 *        weighted sum of the values; query head h reads KV head h / n_rep
 *        where n_rep = query heads per KV head) and [HG] §13.2 (the KV cache
 *        itself stored as q8_0 or q4_0 blocks).
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  R1 Q4_K 6-bit fields: one 96-bit little-endian stream, field k at bits
 *     6k..6k+5; sub-block i uses field 2i as scale and 2i+1 as min [LC].
 *  R2 Q4_K codes: sub-block i owns qs bytes 16i..16i+15 in the Q4_0 nibble
 *     order of [NL] (byte k: low nibble -> element k, high -> element k+16).
 *  R3 Q5_0: d fp16, then a 32-bit word of fifth bits, then 16 bytes of low
 *     nibbles in Q4_0 order; w = d*(q-16).
 *  R4 Q6_K: d fp16, 16 signed 8-bit scales (one per 16 weights), 128 bytes of
 *     low nibbles (Q4_0 order per 32-weight group), 64 bytes of 2-bit high
 *     parts; w = d*(sc*(q-32)); 210 bytes = 6.5625 bpw, which the pages round
 *     to 6.6 [LC table].
 *  R5 Q8_0: d fp16 then 32 two's-complement int8 codes; w = d*q [HG §11.1].
 *  R6 fp32 dequant order: Q4_K computes a = d*sc and b = dmin*m in fp32 (both
 *     exact), t = a*q (exact) and then one rounding in t - b.  Q6_K forms the
 *     integer k = sc*(q-32) first, then d*k (exact).  The others are d*(q-off)
 *     (exact).  The pages' "-> fp16" comments are not followed: fp32 is used.
 *  R14 Q4_1 (named only, [NL] list of formats): Q4_0's block with an fp16
 *     min after the scale: d @0, m @2, qs[16] @4 in Q4_0 nibble order;
 *     w = d*q + m (the block minimum carried as a signed fp16, so the 16
 *     levels span [m, m + 15d]: [HG §11.2] item 2's asymmetric range); 20
 *     bytes per 32 weights = 5.0 bpw.  fp32 order: d*q exact, one rounding
 *     in d*q + m.
 *  R15 Q5_K (256-weight super-block at 5.5-5.7 bpw [LC table]): Q4_K's
 *     fields plus one fifth bit per weight, d @0, dmin @2, scales[12] @4 (R1),
 *     qh[32] @16, qs[128] @48 (R2); bit e of the 256-bit little-endian qh
 *     field is bit 4 of element e's code (as Q5_0's qh word, R3); q in
 *     [0, 31], w = (d*sc_i)*q - dmin*m_i in the fp32 order of R6.  176
 *     bytes = 5.5 bpw, Q4_K's 4.5 plus the fifth bit.
 *  R16 Q2_K (256-weight super-block at 2.5-2.6 bpw [LC table]): Q4_K's
 *     two-level recipe at 2 bits, d @0, dmin @2, scales[16] @4 (byte s:
 *     low nibble = scale, high nibble = min of the 16-weight sub-block s),
 *     qs[64] @20: byte 8g+k holds elements 32g+k+8u at bits 2u..2u+1 (the
 *     2-bit plane order of R4's high parts); q in [0, 3], w = (d*sc_s)*q -
 *     dmin*m_s in the fp32 order of R6.  84 bytes = 2.625 bpw.
 *  R17 Q3_K (256-weight super-block at 3.4-4.0 bpw [LC table]): symmetric
 *     like Q6_K, d @0, scales[12] @2 (16 unsigned six-bit fields in R1's
 *     96-bit stream, field s = scale of the 16-weight sub-block s), ql[64]
 *     @14 (low 2 bits of each code in R16's plane order), qh[32] @78 (bit e
 *     of the little-endian 256-bit plane = bit 2 of element e's code, as
 *     R15's fifth bits); q in [0, 7], w = d*(sc_s*(q-4)) with the integer
 *     formed first (exact).  110 bytes = 3.4375 bpw.
 *  R13 Quantized KV cache: K and V are each [kv_len][n_kv][head_dim], row
 *     (t, g) = t*n_kv + g quantized along head_dim in blocks of the cache's
 *     type (the page's cache tensor is [batch, positions, kv heads, head
 *     dim]; blocks run along the contiguous dimension as in a weight row).
 *  R7 Quantizer (used only to make test inputs): symmetric absmax per block
 *     for Q4_0/Q5_0/Q8_0/Q6_K sub-blocks and min/scale for Q4_K, in fp64, with
 *     stored fp16 scales rounded UP so every weight is covered; codes are
 *     rounded half away from zero.  A block whose cover would exceed the
 *     largest finite fp16 stores 65504 instead (the pages store every scale as
 *     an fp16, [HG §11.1]; an infinite scale would decode to NaN or Inf), so
 *     its codes clamp at the ends of their range.  Q4_1: m is the largest
 *     fp16 <= the block minimum (saturating at -65504), d the cover of
 *     (max - m)/15, q = clamp(rnd((w - m)/d), 0, 15).  Q5_K: as Q4_K with 31
 *     levels per sub-block instead of 15.  Q2_K: as Q4_K over 16-weight
 *     sub-blocks with 3 levels and 15-level scale and min fields.  Q3_K: as
 *     Q6_K with codes clamp(rnd(w/step), -3, 3) + 4 and 63-level scales.
 */
#include "gqo.h"
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* GQO_PLANT selects a deliberate mistake, compiled only into separate test
 * builds that check the pins reject it; the normal build uses 0:
 *   1 nibble order swapped, 2 Q4_K min added instead of subtracted,
 *   3 Q4_K scale/min fields swapped, 4 Q6_K offset 31 instead of 32,
 *   5 dot drops the last column, 6 dot reads x transposed,
 *   7 RMSNorm leaves out eps, 8 SiLU uses exp(+v),
 *   9 attention scores without the 1/sqrt(head_dim) scale,
 *   10 query head h reads KV head h % n_kv instead of h / n_rep,
 *   11 a block scale with no finite cover is stored as Inf,
 *   12 Q4_1 min subtracted instead of added,
 *   13 Q5_K fifth bits read from element e ^ 1,
 *   14 Q2_K scale and min nibbles swapped,
 *   15 Q3_K code offset 3 instead of 4,
 *   16 Q2_K / Q3_K 2-bit plane read with k and u swapped. */
#ifndef GQO_PLANT
#define GQO_PLANT 0
#endif

/* ---------------------------------------------------------------- fp16 */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double gqo_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero or subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1.f) * 2^(e-15) */
    return sign ? -v : v;
}

/* Positive finite fp16 encodings 0x0000..0x7BFF are ordered like their
 * values, so the smallest one >= v is found by bisection. */
uint16_t gqo_half_up(double v) {
    if (!(v > 0.0)) return 0;                       /* 0, or NaN treated as 0 */
    if (v > 65504.0) return 0x7C00;                 /* no finite fp16 covers v */
    uint16_t lo = 0, hi = 0x7BFF;                   /* invariant: val(hi) >= v */
    while (lo < hi) {
        uint16_t mid = (uint16_t)((lo + hi) / 2);
        if (gqo_half_to_double(mid) >= v) hi = mid; else lo = (uint16_t)(mid + 1);
    }
    return hi;
}

/* Round to nearest, ties to even fraction; beyond the largest finite value the
 * halfway point to 2^16 decides overflow, as IEEE rounding does. */
uint16_t gqo_half_rne(float f) {
    if (isnan(f)) return 0x7E00;
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (a >= 65520.0) return sign | 0x7C00;
    /* largest encoding with value <= a */
    uint16_t lo = 0, hi = 0x7BFF;
    while (lo < hi) {
        uint16_t mid = (uint16_t)((lo + hi + 1) / 2);
        if (gqo_half_to_double(mid) <= a) lo = mid; else hi = (uint16_t)(mid - 1);
    }
    double vlo = gqo_half_to_double(lo);
    if (vlo == a || lo == 0x7BFF) return sign | lo;
    double vhi = gqo_half_to_double((uint16_t)(lo + 1));
    double dlo = a - vlo, dhi = vhi - a;            /* exact in fp64 */
    uint16_t r;
    if (dlo < dhi) r = lo;
    else if (dhi < dlo) r = (uint16_t)(lo + 1);
    else r = (lo & 1) ? (uint16_t)(lo + 1) : lo;    /* tie: even fraction */
    return sign | r;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }

/* ---------------------------------------------------------------- types */

int gqo_block_info(int type, int64_t *qk, int64_t *bb) {
    int64_t k, b;
    switch (type) {
    case GQO_F32:  k = 1;   b = 4;   break;
    case GQO_F16:  k = 1;   b = 2;   break;
    case GQO_Q4_0: k = 32;  b = 18;  break;   /* 2 + 16      [HG §11.1] */
    case GQO_Q5_0: k = 32;  b = 22;  break;   /* 2 + 4 + 16  (R3) */
    case GQO_Q8_0: k = 32;  b = 34;  break;   /* 2 + 32      (R5) */
    case GQO_Q4_K: k = 256; b = 144; break;   /* 2+2+12+128  [HG §11.2, LC] */
    case GQO_Q6_K: k = 256; b = 210; break;   /* 2+16+128+64 (R4) */
    case GQO_Q4_1: k = 32;  b = 20;  break;   /* 2 + 2 + 16  (R14) */
    case GQO_Q5_K: k = 256; b = 176; break;   /* 2+2+12+32+128 (R15) */
    case GQO_Q2_K: k = 256; b = 84;  break;   /* 2+2+16+64   (R16) */
    case GQO_Q3_K: k = 256; b = 110; break;   /* 2+12+64+32  (R17) */
    default: return -1;
    }
    if (qk) *qk = k;
    if (bb) *bb = b;
    return 0;
}

static int check(int type, const void *p, int64_t rows, int64_t cols, const void *q) {
    int64_t qk, bb;
    if (gqo_block_info(type, &qk, &bb) != 0) return -1;
    if (rows < 0 || cols <= 0 || cols % qk != 0) return -2;
    if (!p || !q) return -3;
    return 0;
}

/* ---------------------------------------------------------------- codes of one block */

/* Unpacks the integer codes of one block into q[] (length QK) and its header
 * fields.  Field meanings per type are given at the top of the file. */
typedef struct {
    double d, dmin;        /* fp16 scales as exact doubles; dmin: Q4_K and Q5_K's
                              super-min, Q4_1's min m */
    uint16_t d16, dmin16;
    int sc[16], mn[16];    /* Q4_K: 8 scale + 8 min 6-bit fields; Q6_K: 16 int8 scales;
                              Q2_K: 16 four-bit scales and mins; Q3_K: 16 six-bit scales */
    int q[256];
} block_t;

/* 64 bytes of 2-bit fields for 256 elements: byte 8g+k holds elements
 * 32g+k+8u at bits 2u..2u+1 (R16, R17; R4's high-part order). */
static void unpack_2bit_plane(const uint8_t *p, int *q) {
    for (int g = 0; g < 8; g++)
        for (int k = 0; k < 8; k++)
            for (int u = 0; u < 4; u++) {
                const int e = (GQO_PLANT == 16) ? 32 * g + 4 * k + u : 32 * g + k + 8 * u;
                q[e] = (p[8 * g + k] >> (2 * u)) & 3;
            }
}

static void unpack_block(int type, const uint8_t *b, block_t *o) {
    o->d16 = rd16(b);
    o->d = gqo_half_to_double(o->d16);
    o->dmin16 = 0;
    o->dmin = 0.0;
    switch (type) {
    case GQO_Q4_0:                           /* [NL]: low nibbles 0..15, high 16..31 */
        for (int j = 0; j < 16; j++) {
            o->q[j] = b[2 + j] & 0x0F;
            o->q[j + 16] = b[2 + j] >> 4;
            if (GQO_PLANT == 1) { int t = o->q[j]; o->q[j] = o->q[j + 16]; o->q[j + 16] = t; }
        }
        break;
    case GQO_Q8_0:                           /* R5 */
        for (int j = 0; j < 32; j++) o->q[j] = (int)(int8_t)b[2 + j];
        break;
    case GQO_Q5_0: {                         /* R3 */
        uint32_t qh = (uint32_t)b[2] | ((uint32_t)b[3] << 8) | ((uint32_t)b[4] << 16) |
                      ((uint32_t)b[5] << 24);
        for (int j = 0; j < 16; j++) {
            o->q[j] = (b[6 + j] & 0x0F) | (int)(((qh >> j) & 1) << 4);
            o->q[j + 16] = (b[6 + j] >> 4) | (int)(((qh >> (j + 16)) & 1) << 4);
        }
        break;
    }
    case GQO_Q4_1:                           /* R14 */
        o->dmin16 = rd16(b + 2);
        o->dmin = gqo_half_to_double(o->dmin16);
        for (int j = 0; j < 16; j++) {
            o->q[j] = b[4 + j] & 0x0F;
            o->q[j + 16] = b[4 + j] >> 4;
        }
        break;
    case GQO_Q5_K:                           /* R15: Q4_K's fields and a plane of fifth bits */
    case GQO_Q4_K: {
        const int qs = (type == GQO_Q5_K) ? 48 : 16;
        o->dmin16 = rd16(b + 2);
        o->dmin = gqo_half_to_double(o->dmin16);
        /* R1: 96-bit little-endian stream of 16 six-bit fields */
        for (int k = 0; k < 16; k++) {
            int v = 0;
            for (int t = 0; t < 6; t++) {
                int bit = 6 * k + t;
                v |= ((b[4 + bit / 8] >> (bit % 8)) & 1) << t;
            }
            if ((k % 2 == 0) != (GQO_PLANT == 3)) o->sc[k / 2] = v; else o->mn[k / 2] = v;
        }
        /* R2 */
        for (int i = 0; i < 8; i++)
            for (int k = 0; k < 16; k++) {
                uint8_t byte = b[qs + 16 * i + k];
                o->q[32 * i + k] = (GQO_PLANT == 1) ? byte >> 4 : byte & 0x0F;
                o->q[32 * i + k + 16] = (GQO_PLANT == 1) ? byte & 0x0F : byte >> 4;
            }
        if (type == GQO_Q5_K)                /* R15: bit e of qh, element e */
            for (int e = 0; e < 256; e++) {
                int src = (GQO_PLANT == 13) ? (e ^ 1) : e;
                o->q[e] |= ((b[16 + src / 8] >> (src % 8)) & 1) << 4;
            }
        break;
    }
    case GQO_Q2_K:                           /* R16 */
        o->dmin16 = rd16(b + 2);
        o->dmin = gqo_half_to_double(o->dmin16);
        for (int s = 0; s < 16; s++) {
            const int lo = b[4 + s] & 0x0F, hi = b[4 + s] >> 4;
            o->sc[s] = (GQO_PLANT == 14) ? hi : lo;
            o->mn[s] = (GQO_PLANT == 14) ? lo : hi;
        }
        unpack_2bit_plane(b + 20, o->q);
        break;
    case GQO_Q3_K: {                         /* R17 */
        for (int k = 0; k < 16; k++) {       /* R1's 96-bit stream of six-bit fields */
            int v = 0;
            for (int t = 0; t < 6; t++) {
                int bit = 6 * k + t;
                v |= ((b[2 + bit / 8] >> (bit % 8)) & 1) << t;
            }
            o->sc[k] = v;
        }
        unpack_2bit_plane(b + 14, o->q);
        for (int e = 0; e < 256; e++) o->q[e] |= ((b[78 + e / 8] >> (e % 8)) & 1) << 2;
        break;
    }
    case GQO_Q6_K: {                         /* R4 */
        for (int s = 0; s < 16; s++) o->sc[s] = (int)(int8_t)b[2 + s];
        for (int g = 0; g < 8; g++) {
            for (int k = 0; k < 16; k++) {
                uint8_t byte = b[18 + 16 * g + k];
                o->q[32 * g + k] = byte & 0x0F;
                o->q[32 * g + k + 16] = byte >> 4;
            }
            for (int k = 0; k < 8; k++) {
                uint8_t h = b[146 + 8 * g + k];
                for (int u = 0; u < 4; u++)
                    o->q[32 * g + k + 8 * u] |= ((h >> (2 * u)) & 3) << 4;
            }
        }
        break;
    }
    }
}

/* ---------------------------------------------------------------- dequant */

/* fp32 value of element j of an unpacked block, in the order of R6. */
static float deq_f32(int type, const block_t *o, int j) {
    float d = (float)o->d;                   /* exact: fp16 -> fp32 */
    switch (type) {
    case GQO_Q4_0: return d * (float)(o->q[j] - 8);
    case GQO_Q5_0: return d * (float)(o->q[j] - 16);
    case GQO_Q8_0: return d * (float)o->q[j];
    case GQO_Q4_1: {                                   /* R14 */
        float t = d * (float)o->q[j];                  /* exact */
        float m = (float)o->dmin;                      /* exact: fp16 -> fp32 */
        return (GQO_PLANT == 12) ? t - m : t + m;      /* the one rounding */
    }
    case GQO_Q5_K:
    case GQO_Q4_K: {
        int i = j / 32;
        float a = d * (float)o->sc[i];                 /* exact */
        float b = (float)o->dmin * (float)o->mn[i];    /* exact */
        float t = a * (float)o->q[j];                  /* exact */
        return (GQO_PLANT == 2) ? t + b : t - b;       /* the one rounding */
    }
    case GQO_Q6_K: {
        int k = o->sc[j / 16] * (o->q[j] - ((GQO_PLANT == 4) ? 31 : 32));  /* integer first */
        return d * (float)k;                           /* exact */
    }
    case GQO_Q2_K: {                                   /* R16 */
        int i = j / 16;
        float a = d * (float)o->sc[i];                 /* exact */
        float b = (float)o->dmin * (float)o->mn[i];    /* exact */
        float t = a * (float)o->q[j];                  /* exact */
        return t - b;                                  /* the one rounding */
    }
    case GQO_Q3_K: {                                   /* R17 */
        int k = o->sc[j / 16] * (o->q[j] - ((GQO_PLANT == 15) ? 3 : 4));   /* integer first */
        return d * (float)k;                           /* exact */
    }
    }
    return NAN;
}

/* fp64 value of element j: the plain formula, exact for every finite block
 * whose d and dmin exponents differ by less than about 30. */
static double deq_f64(int type, const block_t *o, int j) {
    switch (type) {
    case GQO_Q4_0: return o->d * (double)(o->q[j] - 8);
    case GQO_Q5_0: return o->d * (double)(o->q[j] - 16);
    case GQO_Q8_0: return o->d * (double)o->q[j];
    case GQO_Q4_1:                             /* R14: d*q + m */
        return o->d * (double)o->q[j] + ((GQO_PLANT == 12) ? -o->dmin : o->dmin);
    case GQO_Q5_K:
    case GQO_Q4_K: {                           /* [HG §11.2]: (d*sc)*q - dmin*m */
        int i = j / 32;
        double m = o->dmin * (double)o->mn[i];
        return (o->d * (double)o->sc[i]) * (double)o->q[j] + ((GQO_PLANT == 2) ? m : -m);
    }
    case GQO_Q6_K: return o->d * ((double)o->sc[j / 16] * (double)(o->q[j] - ((GQO_PLANT == 4) ? 31 : 32)));
    case GQO_Q2_K:                             /* R16: (d*sc)*q - dmin*m per 16 weights */
        return (o->d * (double)o->sc[j / 16]) * (double)o->q[j] - o->dmin * (double)o->mn[j / 16];
    case GQO_Q3_K:                             /* R17: d*(sc*(q-4)) */
        return o->d * ((double)o->sc[j / 16] * (double)(o->q[j] - ((GQO_PLANT == 15) ? 3 : 4)));
    }
    return NAN;
}

static void dequant_row_f64(int type, const uint8_t *row, int64_t cols, double *out) {
    int64_t qk, bb;
    gqo_block_info(type, &qk, &bb);
    if (type == GQO_F32) { for (int64_t c = 0; c < cols; c++) { float f; memcpy(&f, row + 4 * c, 4); out[c] = f; } return; }
    if (type == GQO_F16) { for (int64_t c = 0; c < cols; c++) out[c] = gqo_half_to_double(rd16(row + 2 * c)); return; }
    block_t blk;
    for (int64_t b = 0; b < cols / qk; b++) {
        unpack_block(type, row + b * bb, &blk);
        for (int j = 0; j < qk; j++) out[b * qk + j] = deq_f64(type, &blk, j);
    }
}

int gqo_dequant_f32(int type, const uint8_t *blob, int64_t rows, int64_t cols, float *out) {
    int rc = check(type, blob, rows, cols, out);
    if (rc) return rc;
    int64_t qk, bb;
    gqo_block_info(type, &qk, &bb);
    int64_t nb = rows * (cols / qk);
    if (type == GQO_F32) { memcpy(out, blob, (size_t)(rows * cols * 4)); return 0; }
    if (type == GQO_F16) { for (int64_t i = 0; i < rows * cols; i++) out[i] = (float)gqo_half_to_double(rd16(blob + 2 * i)); return 0; }
    block_t blk;
    for (int64_t b = 0; b < nb; b++) {
        unpack_block(type, blob + b * bb, &blk);
        for (int j = 0; j < qk; j++) out[b * qk + j] = deq_f32(type, &blk, j);
    }
    return 0;
}

int gqo_dequant_f64(int type, const uint8_t *blob, int64_t rows, int64_t cols, double *out) {
    int rc = check(type, blob, rows, cols, out);
    if (rc) return rc;
    int64_t qk, bb;
    gqo_block_info(type, &qk, &bb);
    int64_t rb = (cols / qk) * bb;
    for (int64_t r = 0; r < rows; r++) dequant_row_f64(type, blob + r * rb, cols, out + r * cols);
    return 0;
}

/* ---------------------------------------------------------------- matmul */

int gqo_matmul_f64(int type, const uint8_t *blob, int64_t rows, int64_t cols,
                   const double *x, int64_t n_tok, double *y, double *yabs, int threads) {
    int rc = check(type, blob, rows, cols, y);
    if (rc) return rc;
    if (n_tok < 0) return -2;
    if (n_tok > 0 && !x) return -3;
    int64_t qk, bb;
    gqo_block_info(type, &qk, &bb);
    int64_t rb = (cols / qk) * bb;
    if (threads <= 0) threads = 1;
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(threads)
    for (r = 0; r < rows; r++) {
        double *w = (double *)malloc((size_t)cols * sizeof(double));
        dequant_row_f64(type, blob + r * rb, cols, w);            /* dequant ... */
        for (int64_t t = 0; t < n_tok; t++) {                     /* ... then dot */
            const double *xt = x + t * cols;
            double s = 0.0, sa = 0.0;
            int64_t nc = (GQO_PLANT == 5) ? cols - 1 : cols;
            for (int64_t c = 0; c < nc; c++) {
                double xv = (GQO_PLANT == 6) ? x[c * n_tok + t] : xt[c];
                double p = w[c] * xv;
                s += p;
                sa += fabs(p);
            }
            y[t * rows + r] = s;
            if (yabs) yabs[t * rows + r] = sa;
        }
        free(w);
    }
    return 0;
}

/* ---------------------------------------------------------------- decode-layer steps [NL] */

int gqo_rmsnorm_f64(const double *x, int64_t cols, const double *w, double eps, int half_x,
                    double *out) {
    if (!x || !w || !out) return -3;
    if (cols < 1 || !(eps >= 0.0)) return -2;
    double ss = 0.0;
    for (int64_t c = 0; c < cols; c++) ss += x[c] * x[c];
    const double mean = ss / (double)cols;
    const double s = 1.0 / sqrt((GQO_PLANT == 7) ? mean : mean + eps);
    for (int64_t c = 0; c < cols; c++) {
        double t = x[c] * s;
        if (half_x) t = gqo_half_to_double(gqo_half_rne((float)t));   /* cast back to fp16 x */
        out[c] = t * w[c];
    }
    return 0;
}

int gqo_swiglu_f64(const double *g, const double *u, int64_t n, double *out) {
    if (!g || !u || !out) return -3;
    if (n < 0) return -2;
    for (int64_t i = 0; i < n; i++) {
        const double v = g[i];
        const double silu = v / (1.0 + exp((GQO_PLANT == 8) ? v : -v));
        out[i] = silu * u[i];
    }
    return 0;
}

/* ---------------------------------------------------------------- attention over a quantized KV cache */

int gqo_attn_decode_f64(int type, const uint8_t *k_cache, const uint8_t *v_cache, int64_t kv_len,
                        int64_t n_kv, int64_t head_dim, const double *q, int64_t n_heads,
                        double *out) {
    int64_t qk, bb;
    if (gqo_block_info(type, &qk, &bb)) return -1;
    if (!k_cache || !v_cache || !q || !out) return -3;
    if (kv_len < 1 || n_kv < 1 || n_heads < n_kv || n_heads % n_kv || head_dim < 1 ||
        head_dim % qk)
        return -2;
    const int64_t n_rep = n_heads / n_kv, rb = head_dim / qk * bb;
    double *kd = malloc(sizeof(double) * kv_len * head_dim);
    double *vd = malloc(sizeof(double) * kv_len * head_dim);
    double *s = malloc(sizeof(double) * kv_len);
    if (!kd || !vd || !s) { free(kd); free(vd); free(s); return -4; }
    const double scale = (GQO_PLANT == 9) ? 1.0 : 1.0 / sqrt((double)head_dim);
    for (int64_t g = 0; g < n_kv; g++) {
        /* the cached rows of KV head g, dequantized exactly */
        for (int64_t t = 0; t < kv_len; t++) {
            dequant_row_f64(type, k_cache + (t * n_kv + g) * rb, head_dim, kd + t * head_dim);
            dequant_row_f64(type, v_cache + (t * n_kv + g) * rb, head_dim, vd + t * head_dim);
        }
        for (int64_t h = 0; h < n_heads; h++) {
            const int64_t kvh = (GQO_PLANT == 10) ? h % n_kv : h / n_rep;
            if (kvh != g) continue;
            const double *qh = q + h * head_dim;
            double m = -INFINITY;
            for (int64_t t = 0; t < kv_len; t++) {
                double acc = 0.0;
                for (int64_t c = 0; c < head_dim; c++) acc += qh[c] * kd[t * head_dim + c];
                s[t] = acc * scale;
                if (s[t] > m) m = s[t];
            }
            double l = 0.0;
            for (int64_t t = 0; t < kv_len; t++) { s[t] = exp(s[t] - m); l += s[t]; }
            for (int64_t c = 0; c < head_dim; c++) {
                double acc = 0.0;
                for (int64_t t = 0; t < kv_len; t++) acc += s[t] * vd[t * head_dim + c];
                out[h * head_dim + c] = acc / l;
            }
        }
    }
    free(kd); free(vd); free(s);
    return 0;
}

/* ---------------------------------------------------------------- quantizer (R7) */

static double rnd_away(double v) { return round(v); }   /* C round(): half away from 0 */

static int clampi(double v, int lo, int hi) {
    if (v < lo) return lo;
    if (v > hi) return hi;
    return (int)v;
}

/* Smallest fp16 scale d with levels*d >= maxval (checked in fp64), saturating
 * at the largest finite fp16 when no finite scale covers maxval. */
static uint16_t cover_scale(double maxval, double levels) {
    uint16_t h = gqo_half_up(maxval / levels);
    if (h > 0x7BFF && GQO_PLANT != 11) h = 0x7BFF;   /* no finite cover: saturate at 65504 */
    /* make sure levels * d really covers maxval in fp64; bump one ulp if not */
    while (h < 0x7BFF && gqo_half_to_double(h) * levels < maxval) h++;
    return h;
}

/* Largest finite fp16 <= v (saturating at -65504); v finite. */
static uint16_t half_floor(double v) {
    if (v >= 0.0) {
        uint16_t h = gqo_half_up(v);
        if (h > 0x7BFF) return 0x7BFF;
        if (gqo_half_to_double(h) > v) h--;                /* h > 0 here */
        return h;
    }
    uint16_t h = gqo_half_up(-v);                          /* smallest magnitude >= |v| */
    if (h > 0x7BFF) h = 0x7BFF;
    return (uint16_t)(0x8000 | h);
}

/* Symmetric absmax block: q = clamp(rnd(w/d), -L, L) + off. [HG §11.1] */
static void quant_sym32(const float *w, int L, int off, uint16_t *d16, int *q) {
    double a = 0.0;
    for (int j = 0; j < 32; j++) if (fabs((double)w[j]) > a) a = fabs((double)w[j]);
    *d16 = cover_scale(a, (double)L);
    double d = gqo_half_to_double(*d16);
    for (int j = 0; j < 32; j++)
        q[j] = (d == 0.0) ? off : clampi(rnd_away((double)w[j] / d), -L, L) + off;
}

/* Inverse of unpack_2bit_plane for codes in 0..3. */
static void pack_2bit_plane(const int *q, uint8_t *p) {
    for (int g = 0; g < 8; g++)
        for (int k = 0; k < 8; k++) {
            int v = 0;
            for (int u = 0; u < 4; u++) v |= (q[32 * g + k + 8 * u] & 3) << (2 * u);
            p[8 * g + k] = (uint8_t)v;
        }
}

static void quant_block(int type, const float *w, uint8_t *b) {
    int q[256];
    memset(b, 0, 210);
    switch (type) {
    case GQO_Q4_0: {
        uint16_t d16; quant_sym32(w, 7, 8, &d16, q);
        wr16(b, d16);
        for (int j = 0; j < 16; j++) b[2 + j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
        break;
    }
    case GQO_Q8_0: {
        uint16_t d16; quant_sym32(w, 127, 0, &d16, q);
        wr16(b, d16);
        for (int j = 0; j < 32; j++) b[2 + j] = (uint8_t)(int8_t)q[j];
        break;
    }
    case GQO_Q5_0: {
        uint16_t d16; quant_sym32(w, 15, 16, &d16, q);
        wr16(b, d16);
        uint32_t qh = 0;
        for (int j = 0; j < 32; j++) qh |= (uint32_t)((q[j] >> 4) & 1) << j;
        for (int t = 0; t < 4; t++) b[2 + t] = (uint8_t)(qh >> (8 * t));
        for (int j = 0; j < 16; j++) b[6 + j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
        break;
    }
    case GQO_Q4_1: {      /* min and scale per block (R14, R7) */
        double lo = INFINITY, hi = -INFINITY;
        for (int j = 0; j < 32; j++) {
            double v = (double)w[j];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        uint16_t m16 = half_floor(lo);
        double m = gqo_half_to_double(m16);
        uint16_t d16 = cover_scale(hi - m, 15.0);
        double d = gqo_half_to_double(d16);
        for (int j = 0; j < 32; j++)
            q[j] = (d == 0.0) ? 0 : clampi(rnd_away(((double)w[j] - m) / d), 0, 15);
        wr16(b, d16);
        wr16(b + 2, m16);
        for (int j = 0; j < 16; j++) b[4 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
        break;
    }
    case GQO_Q5_K:        /* as Q4_K with 31 levels and a plane of fifth bits (R15) */
    case GQO_Q4_K: {      /* min/scale, two-level [HG §11.2 items 1-2] */
        const int L = (type == GQO_Q5_K) ? 31 : 15;
        const int qs = (type == GQO_Q5_K) ? 48 : 16;
        double hi[8], M[8], Mp[8], sp[8];
        double maxM = 0.0, maxs = 0.0;
        for (int i = 0; i < 8; i++) {
            double lo = 0.0, h = -INFINITY;
            for (int j = 0; j < 32; j++) {
                double v = (double)w[32 * i + j];
                if (v < lo) lo = v;
                if (v > h) h = v;
            }
            hi[i] = h;
            M[i] = -lo;                                   /* >= 0: mins are unsigned */
            if (M[i] > maxM) maxM = M[i];
        }
        uint16_t dmin16 = cover_scale(maxM, 63.0);
        double dmin = gqo_half_to_double(dmin16);
        int mn[8], sc[8];
        for (int i = 0; i < 8; i++) {
            mn[i] = (dmin == 0.0) ? 0 : clampi(ceil(M[i] / dmin), 0, 63);
            Mp[i] = dmin * (double)mn[i];                 /* >= M[i] */
            sp[i] = (hi[i] + Mp[i]) / (double)L;
            if (sp[i] > maxs) maxs = sp[i];
        }
        uint16_t d16 = cover_scale(maxs, 63.0);
        double d = gqo_half_to_double(d16);
        for (int i = 0; i < 8; i++) {
            sc[i] = (d == 0.0) ? 0 : clampi(ceil(sp[i] / d), 0, 63);
            double step = d * (double)sc[i];
            for (int j = 0; j < 32; j++)
                q[32 * i + j] = (step == 0.0) ? 0
                    : clampi(rnd_away(((double)w[32 * i + j] + Mp[i]) / step), 0, L);
        }
        wr16(b, d16);
        wr16(b + 2, dmin16);
        for (int k = 0; k < 16; k++) {                    /* R1 */
            int v = (k % 2 == 0) ? sc[k / 2] : mn[k / 2];
            for (int t = 0; t < 6; t++) {
                int bit = 6 * k + t;
                b[4 + bit / 8] |= (uint8_t)(((v >> t) & 1) << (bit % 8));
            }
        }
        for (int i = 0; i < 8; i++)                       /* R2 */
            for (int k = 0; k < 16; k++)
                b[qs + 16 * i + k] = (uint8_t)((q[32 * i + k] & 15) | ((q[32 * i + k + 16] & 15) << 4));
        if (type == GQO_Q5_K)                             /* R15 */
            for (int e = 0; e < 256; e++) b[16 + e / 8] |= (uint8_t)(((q[e] >> 4) & 1) << (e % 8));
        break;
    }
    case GQO_Q2_K: {      /* min/scale per 16-weight sub-block, two-level (R16, R7) */
        double hi[16], M[16], Mp[16], sp[16];
        double maxM = 0.0, maxs = 0.0;
        for (int s = 0; s < 16; s++) {
            double lo = 0.0, h = -INFINITY;
            for (int j = 0; j < 16; j++) {
                double v = (double)w[16 * s + j];
                if (v < lo) lo = v;
                if (v > h) h = v;
            }
            hi[s] = h;
            M[s] = -lo;                                   /* >= 0: mins are unsigned */
            if (M[s] > maxM) maxM = M[s];
        }
        uint16_t dmin16 = cover_scale(maxM, 15.0);
        double dmin = gqo_half_to_double(dmin16);
        int mn[16], sc[16];
        for (int s = 0; s < 16; s++) {
            mn[s] = (dmin == 0.0) ? 0 : clampi(ceil(M[s] / dmin), 0, 15);
            Mp[s] = dmin * (double)mn[s];                 /* >= M[s] */
            sp[s] = (hi[s] + Mp[s]) / 3.0;
            if (sp[s] > maxs) maxs = sp[s];
        }
        uint16_t d16 = cover_scale(maxs, 15.0);
        double d = gqo_half_to_double(d16);
        for (int s = 0; s < 16; s++) {
            sc[s] = (d == 0.0) ? 0 : clampi(ceil(sp[s] / d), 0, 15);
            double step = d * (double)sc[s];
            for (int j = 0; j < 16; j++)
                q[16 * s + j] = (step == 0.0) ? 0
                    : clampi(rnd_away(((double)w[16 * s + j] + Mp[s]) / step), 0, 3);
        }
        wr16(b, d16);
        wr16(b + 2, dmin16);
        for (int s = 0; s < 16; s++) b[4 + s] = (uint8_t)(sc[s] | (mn[s] << 4));
        pack_2bit_plane(q, b + 20);
        break;
    }
    case GQO_Q3_K: {      /* symmetric per 16-weight sub-block, two-level (R17, R7) */
        double t[16], maxt = 0.0;
        for (int s = 0; s < 16; s++) {
            double a = 0.0;
            for (int j = 0; j < 16; j++) if (fabs((double)w[16 * s + j]) > a) a = fabs((double)w[16 * s + j]);
            t[s] = a / 3.0;
            if (t[s] > maxt) maxt = t[s];
        }
        uint16_t d16 = cover_scale(maxt, 63.0);
        double d = gqo_half_to_double(d16);
        int sc[16];
        for (int s = 0; s < 16; s++) {
            sc[s] = (d == 0.0) ? 0 : clampi(ceil(t[s] / d), 0, 63);
            double step = d * (double)sc[s];
            for (int j = 0; j < 16; j++)
                q[16 * s + j] = (step == 0.0) ? 4
                    : clampi(rnd_away((double)w[16 * s + j] / step), -3, 3) + 4;
        }
        wr16(b, d16);
        for (int k = 0; k < 16; k++)                      /* R1's stream */
            for (int u = 0; u < 6; u++) {
                int bit = 6 * k + u;
                b[2 + bit / 8] |= (uint8_t)(((sc[k] >> u) & 1) << (bit % 8));
            }
        int lo2[256];
        for (int e = 0; e < 256; e++) lo2[e] = q[e] & 3;
        pack_2bit_plane(lo2, b + 14);
        for (int e = 0; e < 256; e++) b[78 + e / 8] |= (uint8_t)(((q[e] >> 2) & 1) << (e % 8));
        break;
    }
    case GQO_Q6_K: {      /* symmetric per 16-weight sub-block, two-level */
        double t[16], maxt = 0.0;
        for (int s = 0; s < 16; s++) {
            double a = 0.0;
            for (int j = 0; j < 16; j++) if (fabs((double)w[16 * s + j]) > a) a = fabs((double)w[16 * s + j]);
            t[s] = a / 31.0;
            if (t[s] > maxt) maxt = t[s];
        }
        uint16_t d16 = cover_scale(maxt, 127.0);
        double d = gqo_half_to_double(d16);
        int sc[16];
        for (int s = 0; s < 16; s++) {
            sc[s] = (d == 0.0) ? 0 : clampi(ceil(t[s] / d), 0, 127);
            double step = d * (double)sc[s];
            for (int j = 0; j < 16; j++)
                q[16 * s + j] = (step == 0.0) ? 32
                    : clampi(rnd_away((double)w[16 * s + j] / step), -31, 31) + 32;
        }
        wr16(b, d16);
        for (int s = 0; s < 16; s++) b[2 + s] = (uint8_t)(int8_t)sc[s];
        for (int g = 0; g < 8; g++) {                     /* R4 */
            for (int k = 0; k < 16; k++)
                b[18 + 16 * g + k] = (uint8_t)((q[32 * g + k] & 15) | ((q[32 * g + k + 16] & 15) << 4));
            for (int k = 0; k < 8; k++) {
                int h = 0;
                for (int u = 0; u < 4; u++) h |= ((q[32 * g + k + 8 * u] >> 4) & 3) << (2 * u);
                b[146 + 8 * g + k] = (uint8_t)h;
            }
        }
        break;
    }
    }
}

int gqo_quantize(int type, const float *w, int64_t rows, int64_t cols, uint8_t *blob) {
    if (type == GQO_F32 || type == GQO_F16) return -1;
    int rc = check(type, w, rows, cols, blob);
    if (rc) return rc;
    int64_t qk, bb;
    gqo_block_info(type, &qk, &bb);
    int64_t nb = rows * (cols / qk);
    uint8_t tmp[210];
    for (int64_t b = 0; b < nb; b++) {
        quant_block(type, w + b * qk, tmp);
        memcpy(blob + b * bb, tmp, (size_t)bb);
    }
    return 0;
}
