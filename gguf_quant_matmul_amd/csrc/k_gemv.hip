// k_gemv.hip — batch-1 GEMV over GGUF blocks, dequantized inside the dot
// product ("Local LLM inference", "The mmap backend").  Decode at batch 1
// reads every weight once and is bound by memory bandwidth ("12 — llama.cpp /
// GGUF", "The bandwidth cap"), so the kernel is built around the weight
// stream:
//   * lane <-> 32-weight segment of a row; consecutive lanes read consecutive
//     16-byte pieces of the same row, so a wave load covers ~1 KB of the blob;
//   * each wave keeps R rows in flight and reuses one x segment (held in
//     registers) for all of them;
//   * x lives in LDS as fp32 (16-byte chunks XOR-swizzled per segment so the
//     64 lanes' 16-byte reads hit distinct banks);
//   * per-segment sums are factored: Q4_K computes a*sum(q*x) - b*sum(x), from
//     w = (d*sc)*q - dmin*m of Hitchhiker's Guide §11.2, which removes the
//     per-weight scale and min operations; the other types convert each code
//     to the signed integer q - offset first, so every product is exact
//     relative to w; fp32 accumulation throughout.
#include "gq_device.h"
#include "gq_launch.h"

namespace gq {

// Raw bytes of one segment and its header, and the factored segment dot.
template <int T> struct Seg;

template <> struct Seg<GQ_Q4_K> {
  u32x4 qs, hd;
  __device__ void load(const uint8_t* row, int s) {
    const uint8_t* b = row + (size_t)(s >> 3) * 144;
    hd = ld16a(b);
    qs = ld16a(b + 16 + 16 * (s & 7));
  }
  __device__ void zero() { qs = u32x4{0, 0, 0, 0}; hd = u32x4{0, 0, 0, 0}; }
  __device__ float dot(const float* x, float xs0, float xs1, int s) const {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t lo = qs[j] & 0x0F0F0F0Fu, hi = (qs[j] >> 4) & 0x0F0F0F0Fu;
      a0 = fmaf(ub0(lo), x[4 * j + 0], a0);
      a0 = fmaf(ub1(lo), x[4 * j + 1], a0);
      a0 = fmaf(ub2(lo), x[4 * j + 2], a0);
      a0 = fmaf(ub3(lo), x[4 * j + 3], a0);
      a1 = fmaf(ub0(hi), x[16 + 4 * j + 0], a1);
      a1 = fmaf(ub1(hi), x[16 + 4 * j + 1], a1);
      a1 = fmaf(ub2(hi), x[16 + 4 * j + 2], a1);
      a1 = fmaf(ub3(hi), x[16 + 4 * j + 3], a1);
    }
    uint32_t p = q4k_pair(hd.y, hd.z, hd.w, s & 7);
    float a = h2f(hd.x) * (float)(p & 63u);
    float b = h2f(hd.x >> 16) * (float)(p >> 6);
    return a * (a0 + a1) - b * (xs0 + xs1);
  }
};

template <> struct Seg<GQ_Q6_K> {
  u32x4 ql;
  u32x2 qh;
  uint32_t sc, d;
  __device__ void load(const uint8_t* row, int s) {
    const uint8_t* b = row + (size_t)(s >> 3) * 210;
    const int g = s & 7;
    ql = ld16u(b + 18 + 16 * g);
    qh = ld8u(b + 146 + 8 * g);
    sc = ld2u(b + 2 + 2 * g);
    d = ld2u(b);
  }
  __device__ void zero() { ql = u32x4{0, 0, 0, 0}; qh = u32x2{0, 0}; sc = 0; d = 0; }
  __device__ float dot(const float* x, float, float, int) const {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t h = (j & 1) ? qh.y : qh.x;
      // signed codes q - 32 per byte, so each product is exact relative to w
      uint32_t lo = centre<32>((ql[j] & 0x0F0F0F0Fu) | q6k_hi(h, j >> 1));
      uint32_t hi = centre<32>(((ql[j] >> 4) & 0x0F0F0F0Fu) | q6k_hi(h, 2 + (j >> 1)));
      s0 = fmaf(sb0(lo), x[4 * j + 0], s0);
      s0 = fmaf(sb1(lo), x[4 * j + 1], s0);
      s0 = fmaf(sb2(lo), x[4 * j + 2], s0);
      s0 = fmaf(sb3(lo), x[4 * j + 3], s0);
      s1 = fmaf(sb0(hi), x[16 + 4 * j + 0], s1);
      s1 = fmaf(sb1(hi), x[16 + 4 * j + 1], s1);
      s1 = fmaf(sb2(hi), x[16 + 4 * j + 2], s1);
      s1 = fmaf(sb3(hi), x[16 + 4 * j + 3], s1);
    }
    float c0 = sb0(sc), c1 = sb1(sc);
    return h2f(d) * (c0 * s0 + c1 * s1);
  }
};

template <> struct Seg<GQ_Q8_0> {
  u32x4 c0, c1;
  uint32_t d;
  __device__ void load(const uint8_t* row, int s) {
    const uint8_t* b = row + (size_t)s * 34;
    d = ld2u(b);
    c0 = ld16u(b + 2);
    c1 = ld16u(b + 18);
  }
  __device__ void zero() { c0 = u32x4{0, 0, 0, 0}; c1 = c0; d = 0; }
  __device__ float dot(const float* x, float, float, int) const {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      a0 = fmaf(sb0(c0[j]), x[4 * j + 0], a0);
      a0 = fmaf(sb1(c0[j]), x[4 * j + 1], a0);
      a0 = fmaf(sb2(c0[j]), x[4 * j + 2], a0);
      a0 = fmaf(sb3(c0[j]), x[4 * j + 3], a0);
      a1 = fmaf(sb0(c1[j]), x[16 + 4 * j + 0], a1);
      a1 = fmaf(sb1(c1[j]), x[16 + 4 * j + 1], a1);
      a1 = fmaf(sb2(c1[j]), x[16 + 4 * j + 2], a1);
      a1 = fmaf(sb3(c1[j]), x[16 + 4 * j + 3], a1);
    }
    return h2f(d) * (a0 + a1);
  }
};

// Q4_0 and Q5_0: low nibbles are elements 0..15, high nibbles 16..31
// ("How LLM Inference Engines Work", "Loading GGUF Models"); Q5_0 adds bit 4.
template <int T> struct SegQ40Q50 {
  static constexpr bool Q5 = (T == GQ_Q5_0);
  u32x4 qs;
  uint32_t qh, d;
  __device__ void load(const uint8_t* row, int s) {
    const uint8_t* b = row + (size_t)s * (Q5 ? 22 : 18);
    d = ld2u(b);
    qh = Q5 ? ld4u(b + 2) : 0u;
    qs = ld16u(b + (Q5 ? 6 : 2));
  }
  __device__ void zero() { qs = u32x4{0, 0, 0, 0}; qh = 0; d = 0; }
  __device__ float dot(const float* x, float, float, int) const {
    constexpr int OFF = Q5 ? 16 : 8;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t lo = qs[j] & 0x0F0F0F0Fu, hi = (qs[j] >> 4) & 0x0F0F0F0Fu;
      if (Q5) {
        lo |= spread4_bit4(qh >> (4 * j));
        hi |= spread4_bit4(qh >> (16 + 4 * j));
      }
      lo = centre<OFF>(lo);
      hi = centre<OFF>(hi);
      a0 = fmaf(sb0(lo), x[4 * j + 0], a0);
      a0 = fmaf(sb1(lo), x[4 * j + 1], a0);
      a0 = fmaf(sb2(lo), x[4 * j + 2], a0);
      a0 = fmaf(sb3(lo), x[4 * j + 3], a0);
      a1 = fmaf(sb0(hi), x[16 + 4 * j + 0], a1);
      a1 = fmaf(sb1(hi), x[16 + 4 * j + 1], a1);
      a1 = fmaf(sb2(hi), x[16 + 4 * j + 2], a1);
      a1 = fmaf(sb3(hi), x[16 + 4 * j + 3], a1);
    }
    return h2f(d) * (a0 + a1);
  }
};
template <> struct Seg<GQ_Q4_0> : SegQ40Q50<GQ_Q4_0> {};
template <> struct Seg<GQ_Q5_0> : SegQ40Q50<GQ_Q5_0> {};

// Physical float index in LDS of logical x index f (16-byte chunks of each
// 32-float segment XOR-swizzled by the segment index).
__device__ __forceinline__ int xswz(int f) {
  int sg = f >> 5, c = (f >> 2) & 7;
  return (sg << 5) | ((c ^ (sg & 7)) << 2) | (f & 3);
}

template <int T, bool XF16, int R>
__global__ void __launch_bounds__(256) k_gemv(const uint8_t* __restrict__ blob, int rows,
                                              int cols, int64_t rb, const void* __restrict__ xv,
                                              float* __restrict__ y) {
  extern __shared__ float xsm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nseg = cols >> 5;
  const int npass = (nseg + 63) >> 6;
  const int r0 = (blockIdx.x * 4 + wave) * R;

  const uint8_t* rowp[R];
#pragma unroll
  for (int k = 0; k < R; k++) rowp[k] = blob + (int64_t)min(r0 + k, rows - 1) * rb;

  // Issue the first pass's weight loads before staging x, so the HBM latency
  // overlaps the LDS fill.
  Seg<T> cur[R], nxt[R];
  {
    const int s = lane;
#pragma unroll
    for (int k = 0; k < R; k++) {
      if (s < nseg) cur[k].load(rowp[k], s); else cur[k].zero();
    }
  }

  // Stage x (fp32) in LDS.
  for (int c4 = threadIdx.x; c4 < (cols >> 2); c4 += 256) {
    f32x4 v;
    if constexpr (XF16) {
      u32x2 h = *reinterpret_cast<const u32x2*>((const _Float16*)xv + 4 * c4);
      v = f32x4{h2f(h.x), h2f(h.x >> 16), h2f(h.y), h2f(h.y >> 16)};
    } else {
      v = reinterpret_cast<const f32x4*>(xv)[c4];
    }
    *reinterpret_cast<f32x4*>(xsm + xswz(4 * c4)) = v;
  }
  __syncthreads();

  float acc[R];
#pragma unroll
  for (int k = 0; k < R; k++) acc[k] = 0.f;

  for (int p = 0; p < npass; p++) {
    const int s = p * 64 + lane;
    if (p + 1 < npass) {
      const int sn = s + 64;
#pragma unroll
      for (int k = 0; k < R; k++) {
        if (sn < nseg) nxt[k].load(rowp[k], sn); else nxt[k].zero();
      }
    }
    if (s < nseg) {
      float x[32];
      const float* base = xsm + (s << 5);
#pragma unroll
      for (int c = 0; c < 8; c++) {
        f32x4 v = *reinterpret_cast<const f32x4*>(base + ((c ^ (s & 7)) << 2));
        x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
      }
      float xs0 = 0.f, xs1 = 0.f;            // segment sums: the Q4_K min term
      if constexpr (T == GQ_Q4_K) {
#pragma unroll
        for (int e = 0; e < 16; e++) { xs0 += x[e]; xs1 += x[16 + e]; }
      }
#pragma unroll
      for (int k = 0; k < R; k++) acc[k] += cur[k].dot(x, xs0, xs1, s);
    }
    if (p + 1 < npass) {
#pragma unroll
      for (int k = 0; k < R; k++) cur[k] = nxt[k];
    }
  }

#pragma unroll
  for (int k = 0; k < R; k++) {
    float v = wave_sum(acc[k]);
    if (lane == k && r0 + k < rows) y[r0 + k] = v;
  }
}

template <int T, bool XF16, int R>
static hipError_t gemv_launch(const void* blob, int64_t rows, int64_t cols, const void* x,
                              float* y, hipStream_t st) {
  const int64_t rb = cols / Geo<T>::QK * Geo<T>::BB;
  const size_t lds = (size_t)cols * 4;                 // cols <= 16384: at most 64 KB
  auto kern = k_gemv<T, XF16, R>;
  dim3 grid((unsigned)((rows + 4 * R - 1) / (4 * R)));
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, (const uint8_t*)blob, (int)rows, (int)cols,
                     rb, x, y);
  return hipGetLastError();
}

template <int T, bool XF16>
static hipError_t gemv_pick(const void* blob, int64_t rows, int64_t cols, const void* x, float* y,
                            hipStream_t st) {
  // Enough workgroups to fill 256 CUs: fewer rows per wave on small matrices.
  if (rows >= 8192) return gemv_launch<T, XF16, 4>(blob, rows, cols, x, y, st);
  if (rows >= 2048) return gemv_launch<T, XF16, 2>(blob, rows, cols, x, y, st);
  return gemv_launch<T, XF16, 1>(blob, rows, cols, x, y, st);
}

template <int T>
static hipError_t gemv_t(const void* blob, int64_t rows, int64_t cols, const void* x, bool xf16,
                         float* y, hipStream_t st) {
  return xf16 ? gemv_pick<T, true>(blob, rows, cols, x, y, st)
              : gemv_pick<T, false>(blob, rows, cols, x, y, st);
}

hipError_t launch_gemv(int type, const void* blob, int64_t rows, int64_t cols, const void* x,
                       bool x_f16, float* y, hipStream_t st) {
  switch (type) {
    case GQ_Q4_0: return gemv_t<GQ_Q4_0>(blob, rows, cols, x, x_f16, y, st);
    case GQ_Q5_0: return gemv_t<GQ_Q5_0>(blob, rows, cols, x, x_f16, y, st);
    case GQ_Q8_0: return gemv_t<GQ_Q8_0>(blob, rows, cols, x, x_f16, y, st);
    case GQ_Q4_K: return gemv_t<GQ_Q4_K>(blob, rows, cols, x, x_f16, y, st);
    case GQ_Q6_K: return gemv_t<GQ_Q6_K>(blob, rows, cols, x, x_f16, y, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gq
