// k_mfma.hip — small-batch and prefill matmul over GGUF blocks on the
// gfx950 matrix cores.  The weights are decoded once per token pass and
// reused for every token ("Local LLM inference", "The mmap backend": decode
// each projection weight once per input batch and reuse it across the batch
// rows); prefill is the compute-bound side of inference ("12 — llama.cpp /
// GGUF", "Prefill on CPU").
//
// Contraction: v_mfma_f32_16x16x32_f16 with A = x (16 tokens x 32 k) and
// B = W^T (32 k x 16 rows), fp32 accumulation.  The B operand is built so
// that every product is exact:
//   Q4_K  B = sc*q (<= 945, an fp16 integer); per block y += d*P, and the
//         min term dmin*sum_i m_i*sum(x over sub-block i) runs on the fp32
//         matrix op v_mfma_f32_16x16x4_f32 (Hitchhiker's Guide §11.2,
//         w = (d*sc)*q - dmin*m, rearranged per sub-block);
//   Q6_K  B = RNE_fp16(sc*(q-32)) (exact when |sc*(q-32)| <= 2048, else
//         relative error <= 2^-11); per block y += d*P;
//   Q4_0 / Q5_0 / Q8_0  B = q - offset (exact); per block y += d*P.
// Within a block the k order of each 8-element operand slice is permuted to
// match the nibble order ("How LLM Inference Engines Work", "Loading GGUF
// Models": low nibbles are elements 0..15, high nibbles 16..31), so each lane
// decodes whole 32-bit words; x is staged in LDS in the same permuted order.
//
// Work split: a workgroup is 4 waves x 16 weight rows; grid.y splits the
// tokens into passes of 16*NT.  x moves through LDS one 256-element slab at a
// time, double-buffered through registers; the next slab's weights are in
// flight while the current slab is multiplied.
#include "gq_device.h"
#include "gq_launch.h"

namespace gq {

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ f16x2 splat(float v) {
  _Float16 h = (_Float16)v;
  return f16x2{h, h};
}
__device__ __forceinline__ f16x8 pack8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// Byte pairs (bytes 0,2) and (bytes 1,3) of v as fp16 values 1024 + byte.
__device__ __forceinline__ f16x2 pair02(uint32_t v) {
  return as_h2((v & 0x00FF00FFu) | 0x64006400u);
}
__device__ __forceinline__ f16x2 pair13(uint32_t v) {
  return as_h2(((v >> 8) & 0x00FF00FFu) | 0x64006400u);
}

// The lane's share of one 256-element K slab of one weight row.  Lane group
// g = lane / 16 owns MFMA k-slices g of every 32-wide chunk.
template <int T> struct MB;

template <> struct MB<GQ_Q4_K> {     // slab = one super-block
  u32x4 hd, q0, q1;                  // header; code bytes 32g..32g+31
  __device__ void load(const uint8_t* rp, int k, int g, int) {
    const uint8_t* b = rp + (size_t)k * 144;
    hd = ld16a(b);
    q0 = ld16a(b + 16 + 32 * g);
    q1 = ld16a(b + 32 + 32 * g);
  }
};

template <> struct MB<GQ_Q6_K> {     // slab = one super-block
  u32x4 l0, l1, h;
  uint32_t sc4, d;
  __device__ void load(const uint8_t* rp, int k, int g, int) {
    const uint8_t* b = rp + (size_t)k * 210;
    l0 = ld16u(b + 18 + 32 * g);     // low nibbles of groups 2g, 2g+1
    l1 = ld16u(b + 34 + 32 * g);
    h = ld16u(b + 146 + 16 * g);     // high bits of groups 2g, 2g+1
    sc4 = ld4u(b + 2 + 4 * g);       // scales of their four 16-weight halves
    d = ld2u(b);
  }
};

template <int T> struct MB32 {       // slab = eight 32-weight blocks
  static constexpr int BB = Geo<T>::BB;
  uint32_t d[8], lo[8], hi[8];
  __device__ void load(const uint8_t* rp, int k, int g, int nblk) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int blk = k * 8 + j;
      if (blk < nblk) {
        const uint8_t* b = rp + (size_t)blk * BB;
        d[j] = ld2u(b);
        if constexpr (T == GQ_Q8_0) {
          lo[j] = ld4u(b + 2 + 4 * g);
          hi[j] = ld4u(b + 18 + 4 * g);
        } else if constexpr (T == GQ_Q5_0) {
          lo[j] = ld4u(b + 6 + 4 * g);
          hi[j] = ld4u(b + 2);       // the fifth-bit word
        } else {
          lo[j] = ld4u(b + 2 + 4 * g);
          hi[j] = 0u;
        }
      } else {
        d[j] = 0u; lo[j] = 0u; hi[j] = 0u;
      }
    }
  }
};
template <> struct MB<GQ_Q4_0> : MB32<GQ_Q4_0> {};
template <> struct MB<GQ_Q5_0> : MB32<GQ_Q5_0> {};
template <> struct MB<GQ_Q8_0> : MB32<GQ_Q8_0> {};

// LDS slot of the 16-byte A slice for token t, chunk j, lane group g.  The
// slot index is XOR-swizzled with t so 8 consecutive tokens hit 8 distinct
// groups of banks.
__device__ __forceinline__ int aslot(int t, int j, int g) {
  return t * 512 + ((((j << 2) | g) ^ (t & 7)) << 4);
}

template <int T, int NT, bool XLO>
__global__ void __launch_bounds__(256) k_mm(const uint8_t* __restrict__ blob, int rows, int cols,
                                            int64_t rb, const void* __restrict__ xv, int n,
                                            float* __restrict__ y) {
  constexpr bool KQ = (T == GQ_Q4_K || T == GQ_Q6_K);
  constexpr int NP = 16 * NT;                 // tokens per pass
  constexpr int NA = XLO ? 2 : 1;             // A planes: hi (and lo) fp16 parts of x
  constexpr int TPT = (NP + 63) / 64;         // staged tokens per thread
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][NA][NP * 512];
  __shared__ float ssum[(T == GQ_Q4_K) ? 2 : 1][(T == GQ_Q4_K) ? NP * 8 : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane & 15, g = lane >> 4;
  const int row = blockIdx.x * 64 + wave * 16 + rl;
  const uint8_t* rp = blob + (int64_t)min(row, rows - 1) * rb;
  const int tok0 = blockIdx.y * NP;
  const int nslab = (cols + 255) >> 8;
  const int nblk32 = cols >> 5;

  // ---- x staging: thread -> (token tt*64 + tid/4, quarter part = tid%4 of the slab)
  const int part = threadIdx.x & 3;
  u32x4 xr[TPT][XLO ? 16 : 8];              // 64 elements per staged token
  auto xload = [&](int k) {
#pragma unroll
    for (int i = 0; i < TPT; i++) {
      const int t = (threadIdx.x >> 2) + 64 * i;
      const int tg = tok0 + t;
      const int e0 = k * 256 + part * 64;
      const bool ok = (t < NP) && (tg < n);
#pragma unroll
      for (int c = 0; c < (XLO ? 16 : 8); c++) {
        const int eb = e0 + c * (XLO ? 4 : 8);    // first element of this 16-byte piece
        if (ok && eb < cols) {
          if constexpr (XLO) xr[i][c] = *reinterpret_cast<const u32x4*>((const float*)xv + (int64_t)tg * cols + eb);
          else xr[i][c] = *reinterpret_cast<const u32x4*>((const _Float16*)xv + (int64_t)tg * cols + eb);
        } else {
          xr[i][c] = u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  auto xstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TPT; i++) {
      const int t = (threadIdx.x >> 2) + 64 * i;
      if (t >= NP) continue;
#pragma unroll
      for (int hseg = 0; hseg < 2; hseg++) {
        const int s = part * 2 + hseg;            // segment within the slab
        float xf[32];
#pragma unroll
        for (int e = 0; e < 32; e++) {
          if constexpr (XLO) {
            // bit-cast the whole vector: clang folds a bit_cast of one
            // ext-vector element to element 0
            const f32x4 fv = __builtin_bit_cast(f32x4, xr[i][hseg * 8 + e / 4]);
            xf[e] = fv[e & 3];
          } else {
            const int c = hseg * 4 + e / 8;
            const uint32_t w = xr[i][c][(e & 7) >> 1];
            xf[e] = h2f((e & 1) ? (w >> 16) : w);
          }
        }
        if constexpr (T == GQ_Q4_K) {
          float sum = 0.f;
#pragma unroll
          for (int e = 0; e < 32; e++) sum += xf[e];
          ssum[buf][t * 8 + s] = sum;
        }
#pragma unroll
        for (int qd = 0; qd < 4; qd++) {
          const int jj = KQ ? (4 * (s & 1) + qd) : s;
          const int gg = KQ ? (s >> 1) : qd;
          const int b0 = 4 * qd;
          const int idx[8] = {b0, b0 + 2, b0 + 16, b0 + 18, b0 + 1, b0 + 3, b0 + 17, b0 + 19};
          f16x8 hv, lv;
#pragma unroll
          for (int e = 0; e < 8; e++) {
            _Float16 hh = (_Float16)xf[idx[e]];
            hv[e] = hh;
            if constexpr (XLO) lv[e] = (_Float16)(xf[idx[e]] - (float)hh);
          }
          *reinterpret_cast<f16x8*>(&xs[buf][0][aslot(t, jj, gg)]) = hv;
          if constexpr (XLO) *reinterpret_cast<f16x8*>(&xs[buf][1][aslot(t, jj, gg)]) = lv;
        }
      }
    }
  };

  f32x4v acc[NT], accm[NT];
#pragma unroll
  for (int tt = 0; tt < NT; tt++) {
    acc[tt] = f32x4v{0.f, 0.f, 0.f, 0.f};
    accm[tt] = f32x4v{0.f, 0.f, 0.f, 0.f};
  }

  MB<T> wc, wn;
  wc.load(rp, 0, g, nblk32);
  xload(0);
  xstore(0);
  __syncthreads();

  for (int k = 0; k < nslab; k++) {
    const int buf = k & 1;
    if (k + 1 < nslab) {
      wn.load(rp, k + 1, g, nblk32);
      xload(k + 1);
    }
    const uint8_t* xa = xs[buf][0];
    auto mfma_chunk = [&](int j, f16x8 B, f32x4v* P, bool first) {
#pragma unroll
      for (int tt = 0; tt < NT; tt++) {
        const int t = tt * 16 + rl;
        f16x8 A = *reinterpret_cast<const f16x8*>(xa + aslot(t, j, g));
        f32x4v c = first ? f32x4v{0.f, 0.f, 0.f, 0.f} : P[tt];
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, c, 0, 0, 0);
        if constexpr (XLO) {
          f16x8 Al = *reinterpret_cast<const f16x8*>(xs[buf][1] + aslot(t, j, g));
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, B, c, 0, 0, 0);
        }
        P[tt] = c;
      }
    };

    if constexpr (T == GQ_Q4_K) {
      const float d = h2f(wc.hd.x), dmin = h2f(wc.hd.x >> 16);
      const uint32_t pa = q4k_pair(wc.hd.y, wc.hd.z, wc.hd.w, 2 * g);
      const uint32_t pb = q4k_pair(wc.hd.y, wc.hd.z, wc.hd.w, 2 * g + 1);
      const f16x2 sa = splat((float)(pa & 63u)), na = splat(-1024.f * (float)(pa & 63u));
      const f16x2 sb = splat((float)(pb & 63u)), nb = splat(-1024.f * (float)(pb & 63u));
      f32x4v P[NT];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const uint32_t D = (j < 4) ? wc.q0[j & 3] : wc.q1[j & 3];
        const f16x2 s = (j < 4) ? sa : sb, ns = (j < 4) ? na : nb;
        const f16x2 h0 = as_h2((D & 0x000F000Fu) | 0x64006400u);
        const f16x2 h1 = as_h2(((D >> 4) & 0x000F000Fu) | 0x64006400u);
        const f16x2 h2 = as_h2(((D >> 8) & 0x000F000Fu) | 0x64006400u);
        const f16x2 h3 = as_h2(((D >> 12) & 0x000F000Fu) | 0x64006400u);
        // (1024 + q) * sc - 1024 * sc = sc * q, one rounding of an exact integer
        const f16x8 B = pack8(__builtin_elementwise_fma(h0, s, ns), __builtin_elementwise_fma(h1, s, ns),
                              __builtin_elementwise_fma(h2, s, ns), __builtin_elementwise_fma(h3, s, ns));
        mfma_chunk(j, B, P, j == 0);
      }
#pragma unroll
      for (int tt = 0; tt < NT; tt++) acc[tt] += d * P[tt];
      // min term on the fp32 matrix op: k = sub-block 4h + g
      const float bm0 = dmin * (float)(q4k_pair(wc.hd.y, wc.hd.z, wc.hd.w, g) >> 6);
      const float bm1 = dmin * (float)(q4k_pair(wc.hd.y, wc.hd.z, wc.hd.w, g + 4) >> 6);
#pragma unroll
      for (int tt = 0; tt < NT; tt++) {
        const int t = tt * 16 + rl;
        const float s0 = ssum[buf][t * 8 + g], s1 = ssum[buf][t * 8 + 4 + g];
        accm[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(s0, bm0, accm[tt], 0, 0, 0);
        accm[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(s1, bm1, accm[tt], 0, 0, 0);
      }
    } else if constexpr (T == GQ_Q6_K) {
      const float d = h2f(wc.d);
      f32x4v P[NT];
      const f16x2 off = splat(-1056.f);          // 1024 + 32
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int G = j >> 2, qd = j & 3;
        const uint32_t L = G ? wc.l1[qd] : wc.l0[qd];
        const uint32_t H = wc.h[2 * G + (qd & 1)];
        const uint32_t lo = (L & 0x0F0F0F0Fu) | q6k_hi(H, qd >> 1);
        const uint32_t hi = ((L >> 4) & 0x0F0F0F0Fu) | q6k_hi(H, 2 + (qd >> 1));
        const f16x2 sa = splat((float)(int)(int8_t)(wc.sc4 >> (16 * G)));
        const f16x2 sb = splat((float)(int)(int8_t)(wc.sc4 >> (16 * G + 8)));
        const f16x8 B = pack8((pair02(lo) + off) * sa, (pair02(hi) + off) * sb,
                              (pair13(lo) + off) * sa, (pair13(hi) + off) * sb);
        mfma_chunk(j, B, P, j == 0);
      }
#pragma unroll
      for (int tt = 0; tt < NT; tt++) acc[tt] += d * P[tt];
    } else {
      const f16x2 off = splat((T == GQ_Q8_0) ? -1152.f : (T == GQ_Q5_0) ? -1040.f : -1032.f);
#pragma unroll
      for (int j = 0; j < 8; j++) {
        uint32_t lo, hi;
        if constexpr (T == GQ_Q8_0) {
          lo = wc.lo[j] ^ 0x80808080u;
          hi = wc.hi[j] ^ 0x80808080u;
        } else {
          lo = wc.lo[j] & 0x0F0F0F0Fu;
          hi = (wc.lo[j] >> 4) & 0x0F0F0F0Fu;
          if constexpr (T == GQ_Q5_0) {
            lo |= spread4_bit4(wc.hi[j] >> (4 * g));
            hi |= spread4_bit4(wc.hi[j] >> (16 + 4 * g));
          }
        }
        const f16x8 B = pack8(pair02(lo) + off, pair02(hi) + off, pair13(lo) + off, pair13(hi) + off);
        f32x4v P[NT];
        mfma_chunk(j, B, P, true);
        const float d = h2f(wc.d[j]);
#pragma unroll
        for (int tt = 0; tt < NT; tt++) acc[tt] += d * P[tt];
      }
    }

    if (k + 1 < nslab) {
      xstore(buf ^ 1);
      wc = wn;
    }
    __syncthreads();
  }

  if (row < rows) {
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int t = tok0 + tt * 16 + 4 * g + v;
        if (t < n) {
          float r = acc[tt][v];
          if constexpr (T == GQ_Q4_K) r -= accm[tt][v];
          y[(int64_t)t * rows + row] = r;
        }
      }
    }
  }
}

template <int T, int NT, bool XLO>
static hipError_t mm_launch(const void* blob, int64_t rows, int64_t cols, const void* x, int64_t n,
                            float* y, hipStream_t st) {
  const int64_t rb = cols / Geo<T>::QK * Geo<T>::BB;
  dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((n + 16 * NT - 1) / (16 * NT)));
  hipLaunchKernelGGL((k_mm<T, NT, XLO>), grid, dim3(256), 0, st, (const uint8_t*)blob, (int)rows,
                     (int)cols, rb, x, (int)n, y);
  return hipGetLastError();
}

template <int T, bool XLO>
static hipError_t mm_pick(const void* blob, int64_t rows, int64_t cols, const void* x, int64_t n,
                          float* y, hipStream_t st) {
  if (n <= 16) return mm_launch<T, 1, XLO>(blob, rows, cols, x, n, y, st);
  if (n <= 32) return mm_launch<T, 2, XLO>(blob, rows, cols, x, n, y, st);
  // 128-token passes only where the registers allow it without spilling
  constexpr bool K = (T == GQ_Q4_K || T == GQ_Q6_K);
  if (XLO || !K || n <= 64) return mm_launch<T, 4, XLO>(blob, rows, cols, x, n, y, st);
  if constexpr (K && !XLO) return mm_launch<T, 8, false>(blob, rows, cols, x, n, y, st);
  return hipErrorInvalidValue;
}

template <int T>
static hipError_t mm_t(const void* blob, int64_t rows, int64_t cols, const void* x, bool xf16,
                       float* y, int64_t n, hipStream_t st) {
  return xf16 ? mm_pick<T, false>(blob, rows, cols, x, n, y, st)
              : mm_pick<T, true>(blob, rows, cols, x, n, y, st);
}

hipError_t launch_mfma(int type, const void* blob, int64_t rows, int64_t cols, const void* x,
                       bool x_f16, float* y, int64_t n_tok, hipStream_t st) {
  switch (type) {
    case GQ_Q4_0: return mm_t<GQ_Q4_0>(blob, rows, cols, x, x_f16, y, n_tok, st);
    case GQ_Q5_0: return mm_t<GQ_Q5_0>(blob, rows, cols, x, x_f16, y, n_tok, st);
    case GQ_Q8_0: return mm_t<GQ_Q8_0>(blob, rows, cols, x, x_f16, y, n_tok, st);
    case GQ_Q4_K: return mm_t<GQ_Q4_K>(blob, rows, cols, x, x_f16, y, n_tok, st);
    case GQ_Q6_K: return mm_t<GQ_Q6_K>(blob, rows, cols, x, x_f16, y, n_tok, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gq
