// k_gemm.hip — prefill-sized matmul (n_tok > 64) over GGUF blocks on the
// gfx950 matrix cores.  Prefill is the compute-bound side of inference
// ("12 — llama.cpp / GGUF", "Prefill on CPU"), so this is a tiled fp16 GEMM
// whose B operand is decoded from the blocks on the fly, once per 128-token
// tile ("Local LLM inference", "The mmap backend": decode once per batch,
// reuse across its rows):
//
//   * B = RNE_fp16 of the stated fp32 dequant (Hitchhiker's Guide §11.2,
//     w = (d*sc)*q - dmin*m), i.e. exactly the fp16 output of gq_dequant:
//     every weight is decoded with one fp32 fma and rounded to fp16 by
//     v_fma_mix (relative error <= 2^-11 per weight, inside the stated
//     1e-3 of sum |w*x|);
//   * workgroup tile 128 tokens x 128 weight rows, K steps of 64 columns;
//     4 waves of 64 x 64, each 2 x 2 v_mfma_f32_32x32x16_f16;
//   * both operands live in LDS, double-buffered, 16-byte chunks XOR-
//     swizzled per row so fragment reads and tile writes are conflict-free;
//   * the raw weight bytes and activations of the next D K-steps are in
//     flight in a register ring (loads complete in issue order, so both
//     streams get the same distance);
//   * fp32 activations are split into hi = RNE_fp16(x) and lo = RNE_fp16(x -
//     hi), and both pass through the matrix op;
//   * tiles are mapped so that the token tiles of one weight-row tile run on
//     one XCD (workgroups go round-robin over the 8 XCDs) and share its L2.
#include "gq_device.h"
#include "gq_launch.h"

namespace gq {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int TILE = BM * BK * 2;            // bytes of one fp16 tile (128 rows x 64)

// 16-byte chunk c (0..7) of tile row t lives at t * 128 + 16 * (c ^ swz(t)).
// Any 16 consecutive rows then use 16 distinct chunk slots of a 256-byte
// bank window (and any 8 rows 8 distinct slots of a 128-byte window).
__device__ __forceinline__ int swz(int t) { return ((t >> 1) & 7) ^ ((t & 1) << 2); }
__device__ __forceinline__ int tslot(int t, int c) { return t * 128 + ((c ^ swz(t)) << 4); }

__device__ __forceinline__ uint32_t h2pack(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
}

// ---------------------------------------------------------------------------
// Weights.  Thread (row r, half h) owns 32 columns of its row per K step: the
// "segment" sg = 2 * step + h (one Q4_K sub-block, one Q6_K group of 32, one
// 32-weight block).  BR holds its raw bytes; decode writes 4 chunks of 8
// fp16 weights.
template <int T> struct BR;
template <> struct BR<GQ_Q4_K> {
  u32x4 hd, q;
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + (sg >> 3) * 144 : kOobOff;
    hd = bld16(R, vo, 0);
    q = bld16(R, vo + 16 * (sg & 7), 16);
  }
  __device__ void decode(int sg, u32x4 out[4]) const {
    const float d = h2f(hd.x), dmin = h2f(hd.x >> 16);
    const uint32_t f = q4k_pair(hd.y, hd.z, hd.w, sg & 7);
    const float a = d * (float)(f & 63u), nb = -(dmin * (float)(f >> 6));
    const float a16 = a * 0.0625f;           // high nibbles enter as 16 q
#pragma unroll
    for (int c = 0; c < 4; c++) {            // chunk c: elements 8c .. 8c+7
      const uint32_t m = (c < 2) ? 0x0F0F0F0Fu : 0xF0F0F0F0u;
      const float s = (c < 2) ? a : a16;
      const uint32_t v0 = q[2 * (c & 1)] & m, v1 = q[2 * (c & 1) + 1] & m;
      out[c] = u32x4{h2pack(fmaf(ub0(v0), s, nb), fmaf(ub1(v0), s, nb)),
                     h2pack(fmaf(ub2(v0), s, nb), fmaf(ub3(v0), s, nb)),
                     h2pack(fmaf(ub0(v1), s, nb), fmaf(ub1(v1), s, nb)),
                     h2pack(fmaf(ub2(v1), s, nb), fmaf(ub3(v1), s, nb))};
    }
  }
};
template <> struct BR<GQ_Q6_K> {
  u32x4 ql;
  u32x2 qh;
  uint32_t sc, d;
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + (sg >> 3) * 210 : kOobOff;
    const int G = sg & 7;
    ql = bld16(R, vo + 16 * G, 18);
    qh = bld8(R, vo + 8 * G, 146);
    sc = bld2(R, vo + 2 * G, 2);
    d = bld2(R, vo, 0);
  }
  __device__ void decode(int, u32x4 out[4]) const {
    const float dd = h2f(d);
#pragma unroll
    for (int c = 0; c < 4; c++) {            // elements 8c..8c+7; scale of half c/2
      const float a = dd * (float)(int)(int8_t)(sc >> (8 * (c >> 1)));
      const float nb = -32.f * a;            // a * (q - 32) is exact in fp32
      const uint32_t L0 = ql[2 * (c & 1)], L1 = ql[2 * (c & 1) + 1];
      const int sh = 4 * (c >> 1);
      const uint32_t H0 = (c <= 2) ? (qh.x << (4 - 2 * c)) : (qh.x >> 2);
      const uint32_t H1 = (c <= 2) ? (qh.y << (4 - 2 * c)) : (qh.y >> 2);
      const uint32_t v0 = ((L0 >> sh) & 0x0F0F0F0Fu) | (H0 & 0x30303030u);
      const uint32_t v1 = ((L1 >> sh) & 0x0F0F0F0Fu) | (H1 & 0x30303030u);
      out[c] = u32x4{h2pack(fmaf(ub0(v0), a, nb), fmaf(ub1(v0), a, nb)),
                     h2pack(fmaf(ub2(v0), a, nb), fmaf(ub3(v0), a, nb)),
                     h2pack(fmaf(ub0(v1), a, nb), fmaf(ub1(v1), a, nb)),
                     h2pack(fmaf(ub2(v1), a, nb), fmaf(ub3(v1), a, nb))};
    }
  }
};
template <> struct BR<GQ_Q8_0> {
  u32x4 c0, c1;
  uint32_t d;
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + sg * 34 : kOobOff;
    d = bld2(R, vo, 0);
    c0 = bld16(R, vo, 2);
    c1 = bld16(R, vo, 18);
  }
  __device__ void decode(int, u32x4 out[4]) const {
    const float dd = h2f(d);
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const u32x4 C = (c < 2) ? c0 : c1;
      const uint32_t v0 = C[2 * (c & 1)], v1 = C[2 * (c & 1) + 1];
      out[c] = u32x4{h2pack(sb0(v0) * dd, sb1(v0) * dd), h2pack(sb2(v0) * dd, sb3(v0) * dd),
                     h2pack(sb0(v1) * dd, sb1(v1) * dd), h2pack(sb2(v1) * dd, sb3(v1) * dd)};
    }
  }
};
template <int T> struct BR4 {                // Q4_0 and Q5_0
  u32x4 c;
  uint32_t qh, d;
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + sg * Geo<T>::BB : kOobOff;
    d = bld2(R, vo, 0);
    if constexpr (T == GQ_Q5_0) {
      qh = bld4(R, vo, 2);
      c = bld16(R, vo, 6);
    } else {
      qh = 0u;
      c = bld16(R, vo, 2);
    }
  }
  __device__ void decode(int, u32x4 out[4]) const {
    const float dd = h2f(d);
    const float nb = -(float)(T == GQ_Q5_0 ? 16 : 8) * dd;
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {         // low nibbles for elements < 16
      const int sh = 4 * (cc >> 1);
      uint32_t v0 = (c[2 * (cc & 1)] >> sh) & 0x0F0F0F0Fu;
      uint32_t v1 = (c[2 * (cc & 1) + 1] >> sh) & 0x0F0F0F0Fu;
      if constexpr (T == GQ_Q5_0) {          // fifth bits of elements 8cc .. 8cc+7
        const uint32_t hb = qh >> (8 * cc);
        v0 |= (((hb & 0xFu) * 0x00204081u) & 0x01010101u) << 4;
        v1 |= ((((hb >> 4) & 0xFu) * 0x00204081u) & 0x01010101u) << 4;
      }
      out[cc] = u32x4{h2pack(fmaf(ub0(v0), dd, nb), fmaf(ub1(v0), dd, nb)),
                      h2pack(fmaf(ub2(v0), dd, nb), fmaf(ub3(v0), dd, nb)),
                      h2pack(fmaf(ub0(v1), dd, nb), fmaf(ub1(v1), dd, nb)),
                      h2pack(fmaf(ub2(v1), dd, nb), fmaf(ub3(v1), dd, nb))};
    }
  }
};
template <> struct BR<GQ_Q4_0> : BR4<GQ_Q4_0> {};
template <> struct BR<GQ_Q5_0> : BR4<GQ_Q5_0> {};

// Activations: the thread's share of one 128 x 64 tile.  fp16: load i, thread
// tid covers row (256 i + tid) / 8, chunk (256 i + tid) % 8 (8 lanes read one
// 128-byte line).  fp32: load i covers row (256 i + tid) / 16, 4 columns.
template <bool XLO> struct AR {
  u32x4 v[XLO ? 8 : 4];
};

}  // namespace

template <int T, bool XLO, int D>
__global__ void __launch_bounds__(256) k_gemm(const uint8_t* __restrict__ blob, int rows, int cols,
                                              int rb, const void* __restrict__ xv, int n,
                                              float* __restrict__ y, int tn, int tm) {
  constexpr int NA = XLO ? 2 : 1;            // activation planes: hi (and lo)
  __shared__ __attribute__((aligned(16))) uint8_t As[2][NA][TILE];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][TILE];
  constexpr int ES = XLO ? 4 : 2;

  // tile q of XCD x covers tiles x * per .. ; token tiles of a row tile adjacent
  const int total = tn * tm, per = (total + 7) >> 3;
  const int q = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (q >= total) return;                    // whole workgroup: uniform
  const int n0 = (q / tm) * BN, m0 = (q % tm) * BM;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int nr = min(BN, rows - n0), nt = min(BM, n - m0);
  const __amdgpu_buffer_rsrc_t WR = make_rsrc(blob + (int64_t)n0 * rb, (uint32_t)(nr * rb));
  const __amdgpu_buffer_rsrc_t XR =
      make_rsrc((const uint8_t*)xv + (int64_t)m0 * cols * ES, (uint32_t)(nt * cols * ES));
  const int nk = (cols + BK - 1) / BK;
  const int nseg = cols >> 5;
  const int br = tid >> 1, bh = tid & 1;     // weight row and half this thread decodes
  const int vrow = br * rb;

  auto load = [&](AR<XLO>& a, BR<T>& b, int s) {
    const int sg = 2 * s + bh;
    b.load(WR, vrow, sg, sg < nseg);
#pragma unroll
    for (int i = 0; i < (XLO ? 8 : 4); i++) {
      const int id = 256 * i + tid;
      const int t = XLO ? (id >> 4) : (id >> 3);
      const int col = s * BK + (XLO ? 4 * (id & 15) : 8 * (id & 7));
      a.v[i] = bld16(XR, col < cols ? (t * cols + col) * ES : kOobOff, 0);
    }
  };
  auto stage = [&](const AR<XLO>& a, const BR<T>& b, int s, int buf) {
#pragma unroll
    for (int i = 0; i < (XLO ? 8 : 4); i++) {
      const int id = 256 * i + tid;
      if constexpr (XLO) {
        const int t = id >> 4, c4 = id & 15;
        const f32x4 f = __builtin_bit_cast(f32x4, a.v[i]);
        float hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          hi[e] = (float)(_Float16)f[e];
          lo[e] = f[e] - hi[e];
        }
        const int o = tslot(t, c4 >> 1) + 8 * (c4 & 1);
        *reinterpret_cast<u32x2*>(&As[buf][0][o]) = u32x2{h2pack(hi[0], hi[1]), h2pack(hi[2], hi[3])};
        *reinterpret_cast<u32x2*>(&As[buf][1][o]) = u32x2{h2pack(lo[0], lo[1]), h2pack(lo[2], lo[3])};
      } else {
        *reinterpret_cast<u32x4*>(&As[buf][0][tslot(id >> 3, id & 7)]) = a.v[i];
      }
    }
    u32x4 dq[4];
    b.decode(2 * s + bh, dq);
#pragma unroll
    for (int c = 0; c < 4; c++) *reinterpret_cast<u32x4*>(&Bs[buf][tslot(br, 4 * bh + c)]) = dq[c];
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = f32x16{};

  AR<XLO> ra[D];
  BR<T> rw[D];
#pragma unroll
  for (int i = 0; i < D; i++) {
    load(ra[i], rw[i], i);                   // issued in ring order
    __builtin_amdgcn_sched_barrier(0);
  }
  stage(ra[0], rw[0], 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(ra[0], rw[0], D);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  const int fr = lane & 31, fk = lane >> 5;  // fragment row, k half
  for (int i0 = 0; i0 < nk; i0 += D) {
#pragma unroll
    for (int u = 0; u < D; u++) {
      const int i = i0 + u;
      if (i < nk) {                          // uniform
        const int buf = i & 1;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ks++) {
          f16x8 af[NA][2], bf[2];
#pragma unroll
          for (int mi = 0; mi < 2; mi++)
#pragma unroll
            for (int p = 0; p < NA; p++)
              af[p][mi] = *reinterpret_cast<const f16x8*>(&As[buf][p][tslot(wm * 64 + mi * 32 + fr, 2 * ks + fk)]);
#pragma unroll
          for (int ni = 0; ni < 2; ni++)
            bf[ni] = *reinterpret_cast<const f16x8*>(&Bs[buf][tslot(wn * 64 + ni * 32 + fr, 2 * ks + fk)]);
#pragma unroll
          for (int mi = 0; mi < 2; mi++)
#pragma unroll
            for (int ni = 0; ni < 2; ni++)
#pragma unroll
              for (int p = 0; p < NA; p++)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[p][mi], bf[ni], acc[mi][ni], 0, 0, 0);
        }
        if (i + 1 < nk) stage(ra[(u + 1) % D], rw[(u + 1) % D], i + 1, buf ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      load(ra[(u + 1) % D], rw[(u + 1) % D], i + 1 + D);   // past the last step: zeros
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }
  }

  // D lane l, register v: weight row l % 32 of the fragment, token
  // 8 (v / 4) + 4 (l / 32) + v % 4
#pragma unroll
  for (int mi = 0; mi < 2; mi++)
#pragma unroll
    for (int ni = 0; ni < 2; ni++) {
      const int r = wn * 64 + ni * 32 + fr;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int t = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * fk + (v & 3);
        if (t < nt && r < nr) y[(int64_t)(m0 + t) * rows + n0 + r] = acc[mi][ni][v];
      }
    }
}

namespace {

template <int T, bool XLO>
hipError_t gemm_t(const void* blob, int64_t rows, int64_t cols, const void* x, int64_t n, float* y,
                  hipStream_t st) {
  const int64_t rb = cols / Geo<T>::QK * Geo<T>::BB;
  const int64_t es = XLO ? 4 : 2;
  if ((int64_t)BN * rb >= kOobOff || (int64_t)BM * cols * es >= kOobOff) return hipErrorInvalidValue;
  const int64_t tn = (rows + BN - 1) / BN, tm = (n + BM - 1) / BM;
  if (tn * tm >= ((int64_t)1 << 31) / 8) return hipErrorInvalidValue;
  const int64_t grid = (tn * tm + 7) / 8 * 8;
  hipLaunchKernelGGL((k_gemm<T, XLO, XLO ? 2 : 3>), dim3((unsigned)grid), dim3(256), 0, st,
                     (const uint8_t*)blob, (int)rows, (int)cols, (int)rb, x, (int)n, y, (int)tn,
                     (int)tm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int type, const void* blob, int64_t rows, int64_t cols, const void* x,
                       bool x_f16, float* y, int64_t n_tok, hipStream_t st) {
  switch (type) {
#define GQ_GEMM_CASE(TT)                                                                  \
  case TT:                                                                                \
    return x_f16 ? gemm_t<TT, false>(blob, rows, cols, x, n_tok, y, st)                   \
                 : gemm_t<TT, true>(blob, rows, cols, x, n_tok, y, st);
    GQ_GEMM_CASE(GQ_Q4_0)
    GQ_GEMM_CASE(GQ_Q5_0)
    GQ_GEMM_CASE(GQ_Q8_0)
    GQ_GEMM_CASE(GQ_Q4_K)
    GQ_GEMM_CASE(GQ_Q6_K)
#undef GQ_GEMM_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace gq
