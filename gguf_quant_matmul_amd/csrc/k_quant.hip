// k_quant.hip — whole-blob dequantization and fp64 quantization kernels.
//
// Dequantization follows the fp32 operation order declared for gq_dequant in
// include/gq.h (Hitchhiker's Guide §11.1 w = d*q and §11.2
// w = (d*sc)*q - dmin*m; 12 — llama.cpp / GGUF, "Q4_K_M — bit layout in
// exquisite detail").  Quantization is the block quantizer declared for
// gq_quantize, computed in fp64 without contraction so that every code and
// scale is a deterministic function of the fp32 weights.
#include "gq_device.h"
#include "gq_launch.h"

namespace gq {

// ---------------------------------------------------------------- dequant

// Writes the 32 fp32 weights of segment s of a row (stated order).
template <int T>
__device__ __forceinline__ void seg_dequant(const uint8_t* row, int s, float w[32]) {
  const uint8_t* b = SegAddr<T>::block(row, s);
  if constexpr (T == GQ_Q4_0 || T == GQ_Q5_0 || T == GQ_Q8_0) {
    float d = h2f(ld2u(b));
    if constexpr (T == GQ_Q8_0) {
#pragma unroll
      for (int j = 0; j < 32; j++) w[j] = d * (float)(int)(int8_t)b[2 + j];
    } else {
      uint32_t qh = (T == GQ_Q5_0) ? ld4u(b + 2) : 0u;
      const uint8_t* qs = b + ((T == GQ_Q5_0) ? 6 : 2);
      const int off = (T == GQ_Q5_0) ? 16 : 8;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        int lo = (qs[j] & 15) | (int)(((qh >> j) & 1u) << 4);
        int hi = (qs[j] >> 4) | (int)(((qh >> (j + 16)) & 1u) << 4);
        w[j] = d * (float)(lo - off);
        w[j + 16] = d * (float)(hi - off);
      }
    }
  } else if constexpr (T == GQ_Q4_1) {
    const float d = h2f(ld2u(b)), m = h2f(ld2u(b + 2));
    const uint8_t* qs = b + 4;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      w[j] = fmaf(d, (float)(qs[j] & 15), m);      // d*q exact: one rounding
      w[j + 16] = fmaf(d, (float)(qs[j] >> 4), m);
    }
  } else if constexpr (T == GQ_Q4_K || T == GQ_Q5_K) {
    constexpr bool Q5 = (T == GQ_Q5_K);
    const int i = s & 7;
    u32x4 h = ld16a(b);
    float d = h2f(h.x), dmin = h2f(h.x >> 16);
    uint32_t p = q4k_pair(h.y, h.z, h.w, i);
    float a = d * (float)(p & 63u);            // exact
    float bm = dmin * (float)(p >> 6);         // exact
    const uint8_t* qs = b + (Q5 ? 48 : 16) + 16 * i;
    const uint32_t qh = Q5 ? ld4u(b + 16 + 4 * i) : 0u;   // fifth bits of the sub-block
#pragma unroll
    for (int k = 0; k < 16; k++) {
      const int c0 = (qs[k] & 15) | (int)(((qh >> k) & 1u) << 4);
      const int c1 = (qs[k] >> 4) | (int)(((qh >> (k + 16)) & 1u) << 4);
      float t0 = a * (float)c0;                // exact
      float t1 = a * (float)c1;
      w[k] = t0 - bm;                          // one rounding
      w[k + 16] = t1 - bm;
    }
  } else if constexpr (T == GQ_Q2_K) {
    const int G = s & 7;                       // elements 32G .. 32G+31 of the super-block
    const float d = h2f(ld2u(b)), dmin = h2f(ld2u(b + 2));
    const uint8_t* qs = b + 20 + 8 * G;        // byte k: elements k + 8u at bits 2u
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {           // 16-weight sub-blocks 2G, 2G+1
      const int sm = b[4 + 2 * G + hh];
      const float a = d * (float)(sm & 15);    // exact
      const float bm = dmin * (float)(sm >> 4);
#pragma unroll
      for (int p = 0; p < 16; p++) {
        const int e = 16 * hh + p;
        const int q = (qs[e & 7] >> (2 * (e >> 3))) & 3;
        const float t = a * (float)q;          // exact
        w[e] = t - bm;                         // one rounding
      }
    }
  } else if constexpr (T == GQ_Q3_K) {
    const int G = s & 7;
    const float d = h2f(ld2u(b));
    const uint8_t* ql = b + 14 + 8 * G;
    const uint32_t qh = ld4u(b + 78 + 4 * G);  // bit e: bit 2 of element 32G + e
    const int bit = 12 * G;                    // scale fields 2G, 2G+1 of the stream
    const uint32_t f = (ld4u(b + 2 + (bit >> 3)) >> (bit & 7)) & 0xFFFu;
#pragma unroll
    for (int e = 0; e < 32; e++) {
      const int q = ((ql[e & 7] >> (2 * (e >> 3))) & 3) | (int)(((qh >> e) & 1u) << 2);
      const int sc = (e < 16) ? (int)(f & 63u) : (int)(f >> 6);
      w[e] = d * (float)(sc * (q - 4));        // integer first, then exact
    }
  } else {  // GQ_Q6_K
    const int g = s & 7;
    float d = h2f(ld2u(b));
    int sc0 = (int)(int8_t)b[2 + 2 * g], sc1 = (int)(int8_t)b[3 + 2 * g];
    const uint8_t* ql = b + 18 + 16 * g;
    const uint8_t* qh = b + 146 + 8 * g;
#pragma unroll
    for (int e = 0; e < 32; e++) {
      int lo = (e < 16) ? (ql[e] & 15) : (ql[e - 16] >> 4);
      int hi = (qh[e & 7] >> (2 * (e >> 3))) & 3;
      int q = lo | (hi << 4);
      int k = ((e < 16) ? sc0 : sc1) * (q - 32);   // integer first
      w[e] = d * (float)k;                          // exact
    }
  }
}

template <int T, bool F16OUT>
__global__ void __launch_bounds__(256) k_dequant(const uint8_t* __restrict__ blob,
                                                 int64_t rows, int nseg, int64_t row_bytes,
                                                 void* __restrict__ out) {
  int64_t gs = (int64_t)blockIdx.x * 256 + threadIdx.x;   // global segment
  if (gs >= rows * nseg) return;
  int64_t r = gs / nseg;
  int s = (int)(gs - r * nseg);
  float w[32];
  seg_dequant<T>(blob + r * row_bytes, s, w);
  if constexpr (F16OUT) {
    _Float16* o = (_Float16*)out + gs * 32;
#pragma unroll
    for (int j = 0; j < 32; j += 8) {
      f16x8 v;
#pragma unroll
      for (int k = 0; k < 8; k++) v[k] = (_Float16)w[j + k];     // RNE
      *reinterpret_cast<f16x8*>(o + j) = v;
    }
  } else {
    float* o = (float*)out + gs * 32;
#pragma unroll
    for (int j = 0; j < 32; j += 4)
      *reinterpret_cast<f32x4*>(o + j) = f32x4{w[j], w[j + 1], w[j + 2], w[j + 3]};
  }
}

// ---------------------------------------------------------------- quantize (fp64)

#pragma clang fp contract(off)

__device__ double d_h2d(uint32_t h) {   // fp16 bits -> fp64, exact
  return (double)h2f(h);
}

// Smallest finite fp16 >= v for v > 0 (0 for v <= 0), 0x7C00 if v > 65504.
__device__ uint32_t d_half_up(double v) {
  if (!(v > 0.0)) return 0u;
  if (v > 65504.0) return 0x7C00u;
  if (v < 0x1p-14) return (uint32_t)ceil(v * 0x1p24);   // subnormal steps of 2^-24
  int e;
  frexp(v, &e);                                          // v in [2^(e-1), 2^e)
  double f = ceil(ldexp(v, 11 - e));                     // significand*1024 in [1024, 2048]
  return ((uint32_t)(e - 1 + 15) << 10) + ((uint32_t)f - 1024u);
}

// fp16 scale d with levels*d >= maxval, saturating at the largest finite fp16.
__device__ uint32_t d_cover(double maxval, double levels) {
  uint32_t h = d_half_up(maxval / levels);
  if (h > 0x7BFFu) h = 0x7BFFu;
  while (h < 0x7BFFu && d_h2d(h) * levels < maxval) h++;
  return h;
}

// Largest finite fp16 <= v (saturating at -65504), v finite.
__device__ uint32_t d_half_floor(double v) {
  if (v >= 0.0) {
    uint32_t h = d_half_up(v);
    if (h > 0x7BFFu) return 0x7BFFu;
    if (d_h2d(h) > v) h--;
    return h;
  }
  uint32_t h = d_half_up(-v);
  if (h > 0x7BFFu) h = 0x7BFFu;
  return 0x8000u | h;
}

__device__ int d_clampi(double v, int lo, int hi) {
  if (v < (double)lo) return lo;
  if (v > (double)hi) return hi;
  return (int)v;
}

template <int T>
__device__ void quant_block(const float* __restrict__ w, uint8_t* out) {
  if constexpr (T == GQ_Q4_0 || T == GQ_Q5_0 || T == GQ_Q8_0) {
    const int L = (T == GQ_Q4_0) ? 7 : (T == GQ_Q5_0) ? 15 : 127;
    const int off = (T == GQ_Q4_0) ? 8 : (T == GQ_Q5_0) ? 16 : 0;
    double a = 0.0;
    for (int j = 0; j < 32; j++) a = fmax(a, fabs((double)w[j]));
    uint32_t d16 = d_cover(a, (double)L);
    double d = d_h2d(d16);
    int q[32];
    for (int j = 0; j < 32; j++)
      q[j] = (d == 0.0) ? off : d_clampi(round((double)w[j] / d), -L, L) + off;
    out[0] = (uint8_t)d16;
    out[1] = (uint8_t)(d16 >> 8);
    if constexpr (T == GQ_Q8_0) {
      for (int j = 0; j < 32; j++) out[2 + j] = (uint8_t)(int8_t)q[j];
    } else if constexpr (T == GQ_Q4_0) {
      for (int j = 0; j < 16; j++) out[2 + j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
    } else {
      uint32_t qh = 0;
      for (int j = 0; j < 32; j++) qh |= (uint32_t)((q[j] >> 4) & 1) << j;
      for (int t = 0; t < 4; t++) out[2 + t] = (uint8_t)(qh >> (8 * t));
      for (int j = 0; j < 16; j++) out[6 + j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
    }
  } else if constexpr (T == GQ_Q4_1) {
    double lo = INFINITY, hi = -INFINITY;
    for (int j = 0; j < 32; j++) {
      lo = fmin(lo, (double)w[j]);
      hi = fmax(hi, (double)w[j]);
    }
    const uint32_t m16 = d_half_floor(lo);
    const double m = d_h2d(m16);
    const uint32_t d16 = d_cover(hi - m, 15.0);
    const double d = d_h2d(d16);
    int q[32];
    for (int j = 0; j < 32; j++) q[j] = (d == 0.0) ? 0 : d_clampi(round(((double)w[j] - m) / d), 0, 15);
    out[0] = (uint8_t)d16;
    out[1] = (uint8_t)(d16 >> 8);
    out[2] = (uint8_t)m16;
    out[3] = (uint8_t)(m16 >> 8);
    for (int j = 0; j < 16; j++) out[4 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
  } else if constexpr (T == GQ_Q4_K || T == GQ_Q5_K) {
    constexpr int L = (T == GQ_Q5_K) ? 31 : 15;
    constexpr int QS = (T == GQ_Q5_K) ? 48 : 16;
    double hi[8], Mp[8], sp[8];
    double M[8];
    double maxM = 0.0, maxs = 0.0;
    for (int i = 0; i < 8; i++) {
      double lo = 0.0, h = -INFINITY;
      for (int j = 0; j < 32; j++) {
        double v = (double)w[32 * i + j];
        lo = fmin(lo, v);
        h = fmax(h, v);
      }
      hi[i] = h;
      M[i] = -lo;
      maxM = fmax(maxM, M[i]);
    }
    uint32_t dmin16 = d_cover(maxM, 63.0);
    double dmin = d_h2d(dmin16);
    int mn[8], sc[8];
    for (int i = 0; i < 8; i++) {
      mn[i] = (dmin == 0.0) ? 0 : d_clampi(ceil(M[i] / dmin), 0, 63);
      Mp[i] = dmin * (double)mn[i];
      sp[i] = (hi[i] + Mp[i]) / (double)L;
      maxs = fmax(maxs, sp[i]);
    }
    uint32_t d16 = d_cover(maxs, 63.0);
    double d = d_h2d(d16);
    out[0] = (uint8_t)d16;
    out[1] = (uint8_t)(d16 >> 8);
    out[2] = (uint8_t)dmin16;
    out[3] = (uint8_t)(dmin16 >> 8);
    for (int i = 0; i < 8; i++) sc[i] = (d == 0.0) ? 0 : d_clampi(ceil(sp[i] / d), 0, 63);
    // 16 six-bit fields, field 2i = scale, 2i+1 = min, LSB-first
    uint64_t lo64 = 0, hi32 = 0;
    for (int i = 0; i < 8; i++) {
      uint64_t pair = (uint64_t)(sc[i] | (mn[i] << 6));
      int sh = 12 * i;
      if (sh + 12 <= 64) lo64 |= pair << sh;
      else if (sh >= 64) hi32 |= pair << (sh - 64);
      else { lo64 |= pair << sh; hi32 |= pair >> (64 - sh); }
    }
    for (int t = 0; t < 8; t++) out[4 + t] = (uint8_t)(lo64 >> (8 * t));
    for (int t = 0; t < 4; t++) out[12 + t] = (uint8_t)(hi32 >> (8 * t));
    if constexpr (T == GQ_Q5_K)
      for (int t = 0; t < 32; t++) out[16 + t] = 0;
    for (int i = 0; i < 8; i++) {
      double step = d * (double)sc[i];
      for (int k = 0; k < 16; k++) {
        int q0 = (step == 0.0) ? 0 : d_clampi(round(((double)w[32 * i + k] + Mp[i]) / step), 0, L);
        int q1 = (step == 0.0) ? 0 : d_clampi(round(((double)w[32 * i + k + 16] + Mp[i]) / step), 0, L);
        out[QS + 16 * i + k] = (uint8_t)((q0 & 15) | ((q1 & 15) << 4));
        if constexpr (T == GQ_Q5_K) {         // bit e of the fifth-bit plane: element e
          const int e0 = 32 * i + k, e1 = e0 + 16;
          out[16 + e0 / 8] |= (uint8_t)(((q0 >> 4) & 1) << (e0 % 8));
          out[16 + e1 / 8] |= (uint8_t)(((q1 >> 4) & 1) << (e1 % 8));
        }
      }
    }
  } else if constexpr (T == GQ_Q2_K) {
    double hi[16], M[16], Mp[16], sp[16];
    double maxM = 0.0, maxs = 0.0;
    for (int i = 0; i < 16; i++) {
      double lo = 0.0, h = -INFINITY;
      for (int j = 0; j < 16; j++) {
        double v = (double)w[16 * i + j];
        lo = fmin(lo, v);
        h = fmax(h, v);
      }
      hi[i] = h;
      M[i] = -lo;
      maxM = fmax(maxM, M[i]);
    }
    const uint32_t dmin16 = d_cover(maxM, 15.0);
    const double dmin = d_h2d(dmin16);
    int mn[16], sc[16];
    for (int i = 0; i < 16; i++) {
      mn[i] = (dmin == 0.0) ? 0 : d_clampi(ceil(M[i] / dmin), 0, 15);
      Mp[i] = dmin * (double)mn[i];
      sp[i] = (hi[i] + Mp[i]) / 3.0;
      maxs = fmax(maxs, sp[i]);
    }
    const uint32_t d16 = d_cover(maxs, 15.0);
    const double d = d_h2d(d16);
    out[0] = (uint8_t)d16;
    out[1] = (uint8_t)(d16 >> 8);
    out[2] = (uint8_t)dmin16;
    out[3] = (uint8_t)(dmin16 >> 8);
    uint8_t q[256];
    for (int i = 0; i < 16; i++) {
      sc[i] = (d == 0.0) ? 0 : d_clampi(ceil(sp[i] / d), 0, 15);
      out[4 + i] = (uint8_t)(sc[i] | (mn[i] << 4));
      const double step = d * (double)sc[i];
      for (int j = 0; j < 16; j++)
        q[16 * i + j] = (uint8_t)((step == 0.0) ? 0
                                  : d_clampi(round(((double)w[16 * i + j] + Mp[i]) / step), 0, 3));
    }
    for (int g = 0; g < 8; g++)                // byte 8g+k: elements 32g+k+8u at bits 2u
      for (int k = 0; k < 8; k++)
        out[20 + 8 * g + k] = (uint8_t)(q[32 * g + k] | (q[32 * g + k + 8] << 2) |
                                        (q[32 * g + k + 16] << 4) | (q[32 * g + k + 24] << 6));
  } else if constexpr (T == GQ_Q3_K) {
    double t[16], maxt = 0.0;
    for (int i = 0; i < 16; i++) {
      double a = 0.0;
      for (int j = 0; j < 16; j++) a = fmax(a, fabs((double)w[16 * i + j]));
      t[i] = a / 3.0;
      maxt = fmax(maxt, t[i]);
    }
    const uint32_t d16 = d_cover(maxt, 63.0);
    const double d = d_h2d(d16);
    out[0] = (uint8_t)d16;
    out[1] = (uint8_t)(d16 >> 8);
    uint8_t q[256];
    uint64_t lo64 = 0, hi32 = 0;               // 16 six-bit fields, LSB-first
    for (int i = 0; i < 16; i++) {
      const int sc = (d == 0.0) ? 0 : d_clampi(ceil(t[i] / d), 0, 63);
      const int sh = 6 * i;
      if (sh + 6 <= 64) lo64 |= (uint64_t)sc << sh;
      else if (sh >= 64) hi32 |= (uint64_t)sc << (sh - 64);
      else { lo64 |= (uint64_t)sc << sh; hi32 |= (uint64_t)sc >> (64 - sh); }
      const double step = d * (double)sc;
      for (int j = 0; j < 16; j++)
        q[16 * i + j] = (uint8_t)((step == 0.0) ? 4
                                  : d_clampi(round((double)w[16 * i + j] / step), -3, 3) + 4);
    }
    for (int k = 0; k < 8; k++) out[2 + k] = (uint8_t)(lo64 >> (8 * k));
    for (int k = 0; k < 4; k++) out[10 + k] = (uint8_t)(hi32 >> (8 * k));
    for (int g = 0; g < 8; g++)
      for (int k = 0; k < 8; k++)
        out[14 + 8 * g + k] = (uint8_t)((q[32 * g + k] & 3) | ((q[32 * g + k + 8] & 3) << 2) |
                                        ((q[32 * g + k + 16] & 3) << 4) |
                                        ((q[32 * g + k + 24] & 3) << 6));
    for (int k = 0; k < 32; k++) {
      int v = 0;
      for (int b = 0; b < 8; b++) v |= ((q[8 * k + b] >> 2) & 1) << b;
      out[78 + k] = (uint8_t)v;
    }
  } else {  // GQ_Q6_K
    double t[16], maxt = 0.0;
    for (int s = 0; s < 16; s++) {
      double a = 0.0;
      for (int j = 0; j < 16; j++) a = fmax(a, fabs((double)w[16 * s + j]));
      t[s] = a / 31.0;
      maxt = fmax(maxt, t[s]);
    }
    uint32_t d16 = d_cover(maxt, 127.0);
    double d = d_h2d(d16);
    out[0] = (uint8_t)d16;
    out[1] = (uint8_t)(d16 >> 8);
    uint8_t q[256];
    for (int s = 0; s < 16; s++) {
      int sc = (d == 0.0) ? 0 : d_clampi(ceil(t[s] / d), 0, 127);
      out[2 + s] = (uint8_t)sc;
      double step = d * (double)sc;
      for (int j = 0; j < 16; j++)
        q[16 * s + j] = (uint8_t)((step == 0.0) ? 32
                                  : d_clampi(round((double)w[16 * s + j] / step), -31, 31) + 32);
    }
    for (int g = 0; g < 8; g++) {
      for (int k = 0; k < 16; k++)
        out[18 + 16 * g + k] = (uint8_t)((q[32 * g + k] & 15) | ((q[32 * g + k + 16] & 15) << 4));
      for (int k = 0; k < 8; k++) {
        int h = 0;
        for (int u = 0; u < 4; u++) h |= ((q[32 * g + k + 8 * u] >> 4) & 3) << (2 * u);
        out[146 + 8 * g + k] = (uint8_t)h;
      }
    }
  }
}

template <int T>
__global__ void __launch_bounds__(64) k_quantize(const float* __restrict__ w, int64_t nblocks,
                                                 uint8_t* __restrict__ blob) {
  int64_t b = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (b >= nblocks) return;
  constexpr int QK = Geo<T>::QK, BB = Geo<T>::BB;
  uint8_t tmp[(BB + 1) & ~1];
  quant_block<T>(w + b * QK, tmp);
  // every block size is even and the blob is 16-B aligned: 16-bit stores
  uint16_t* o = reinterpret_cast<uint16_t*>(blob + b * BB);
  for (int k = 0; k < BB / 2; k++) o[k] = (uint16_t)(tmp[2 * k] | (tmp[2 * k + 1] << 8));
}

#pragma clang fp contract(on)

// ---------------------------------------------------------------- launchers

template <int T>
static hipError_t dequant_t(const void* blob, int64_t rows, int64_t cols, void* out, bool f16,
                            hipStream_t st) {
  int nseg = (int)(cols / 32);
  int64_t total = rows * nseg;
  dim3 grid((unsigned)((total + 255) / 256));
  int64_t rb = cols / Geo<T>::QK * Geo<T>::BB;
  if (f16)
    hipLaunchKernelGGL((k_dequant<T, true>), grid, dim3(256), 0, st, (const uint8_t*)blob, rows,
                       nseg, rb, out);
  else
    hipLaunchKernelGGL((k_dequant<T, false>), grid, dim3(256), 0, st, (const uint8_t*)blob, rows,
                       nseg, rb, out);
  return hipGetLastError();
}

hipError_t launch_dequant(int type, const void* blob, int64_t rows, int64_t cols, void* out,
                          bool f16, hipStream_t st) {
  switch (type) {
    case GQ_Q4_0: return dequant_t<GQ_Q4_0>(blob, rows, cols, out, f16, st);
    case GQ_Q5_0: return dequant_t<GQ_Q5_0>(blob, rows, cols, out, f16, st);
    case GQ_Q8_0: return dequant_t<GQ_Q8_0>(blob, rows, cols, out, f16, st);
    case GQ_Q4_K: return dequant_t<GQ_Q4_K>(blob, rows, cols, out, f16, st);
    case GQ_Q6_K: return dequant_t<GQ_Q6_K>(blob, rows, cols, out, f16, st);
    case GQ_Q4_1: return dequant_t<GQ_Q4_1>(blob, rows, cols, out, f16, st);
    case GQ_Q5_K: return dequant_t<GQ_Q5_K>(blob, rows, cols, out, f16, st);
    case GQ_Q2_K: return dequant_t<GQ_Q2_K>(blob, rows, cols, out, f16, st);
    case GQ_Q3_K: return dequant_t<GQ_Q3_K>(blob, rows, cols, out, f16, st);
  }
  return hipErrorInvalidValue;
}

template <int T>
static hipError_t quantize_t(const float* w, int64_t rows, int64_t cols, void* blob,
                             hipStream_t st) {
  int64_t nb = rows * (cols / Geo<T>::QK);
  dim3 grid((unsigned)((nb + 63) / 64));
  hipLaunchKernelGGL((k_quantize<T>), grid, dim3(64), 0, st, w, nb, (uint8_t*)blob);
  return hipGetLastError();
}

hipError_t launch_quantize(int type, const float* w, int64_t rows, int64_t cols, void* blob,
                           hipStream_t st) {
  switch (type) {
    case GQ_Q4_0: return quantize_t<GQ_Q4_0>(w, rows, cols, blob, st);
    case GQ_Q5_0: return quantize_t<GQ_Q5_0>(w, rows, cols, blob, st);
    case GQ_Q8_0: return quantize_t<GQ_Q8_0>(w, rows, cols, blob, st);
    case GQ_Q4_K: return quantize_t<GQ_Q4_K>(w, rows, cols, blob, st);
    case GQ_Q6_K: return quantize_t<GQ_Q6_K>(w, rows, cols, blob, st);
    case GQ_Q4_1: return quantize_t<GQ_Q4_1>(w, rows, cols, blob, st);
    case GQ_Q5_K: return quantize_t<GQ_Q5_K>(w, rows, cols, blob, st);
    case GQ_Q2_K: return quantize_t<GQ_Q2_K>(w, rows, cols, blob, st);
    case GQ_Q3_K: return quantize_t<GQ_Q3_K>(w, rows, cols, blob, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gq
