// k_attn.hip — one decode step of grouped-query attention over a KV cache
// stored as q8_0 or q4_0 blocks ("How LLM Inference Engines Work",
// "Grouped-Query Attention (GQA) and KV Cache"; the Hitchhiker's Guide §13.2
// for the quantized cache).  For query head h, with g = h / n_rep:
//     s[t] = q[h] . K^[t][g] / sqrt(head_dim),   out[h] = sum_t softmax(s)[t] V^[t][g]
// Decode attention reads the whole cache once per token and is bound by
// memory bandwidth, so the work is split over the cached positions to cover
// every CU, and each block is decoded where it is used:
//   * part kernel, workgroup (chunk c, KV head g): the chunk's V rows are
//     staged raw in LDS while the scores of all n_rep query heads of g are
//     formed (q in LDS, each lane one 32-element block of a K row, exact
//     integer codes times the block scale); then the chunk's softmax
//     statistics (max m, sum l of exp(s - m)) and sum_t exp(s - m) V^[t]
//     go to the workspace;
//   * combine kernel: out[h] = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c
//     with M the largest m_c, in chunk order (deterministic).
// Cache layout: [kv_len][n_kv][head_dim], row (t, g) = t * n_kv + g holding
// head_dim / 32 blocks.
#include <cmath>

#include "gq_device.h"
#include "gq_launch.h"

namespace gq {

constexpr int ATT_MAX_REP = 16;           // query heads per KV head
constexpr int ATT_LDS = 65536;            // LDS budget of the part kernel
// Largest chunk (positions) for NB blocks per row.
constexpr int ATT_CHUNK_CAP(int nb) { return nb > 4 ? 128 : 256; }

template <int KT> struct KvBlock;

template <> struct KvBlock<GQ_Q8_0> {          // fp16 d, 32 int8 codes
  static constexpr int BB = 34;
  struct Raw {
    u32x4 a, b;
    uint32_t d;
  };
  __device__ static Raw load(__amdgpu_buffer_rsrc_t r, int o) {
    return Raw{bld16(r, o, 2), bld16(r, o, 18), bld2(r, o, 0)};
  }
  // the 32 codes as exact fp32; returns the block scale
  __device__ static float decode(const Raw& raw, float (&c)[32]) {
    const u32x4 a = raw.a, b = raw.b;
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      c[4 * i] = sb0(w[i]);
      c[4 * i + 1] = sb1(w[i]);
      c[4 * i + 2] = sb2(w[i]);
      c[4 * i + 3] = sb3(w[i]);
    }
    return h2f(raw.d);
  }
  static constexpr int CODE_BYTES = 32;
  __device__ static void store_codes(const Raw& raw, uint8_t* p) {     // 16-byte aligned
    *reinterpret_cast<u32x4*>(p) = raw.a;
    *reinterpret_cast<u32x4*>(p + 16) = raw.b;
  }
  // codes j0..j0+3 (j0 a multiple of 4) of a staged block as exact fp32
  __device__ static void code4(const uint8_t* p, int j0, float (&v)[4]) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p + j0);
    v[0] = sb0(w);
    v[1] = sb1(w);
    v[2] = sb2(w);
    v[3] = sb3(w);
  }
};

template <> struct KvBlock<GQ_Q4_0> {          // fp16 d, 16 bytes: low nibbles 0..15, high 16..31
  static constexpr int BB = 18;
  struct Raw {
    u32x4 a;
    uint32_t d;
  };
  __device__ static Raw load(__amdgpu_buffer_rsrc_t r, int o) { return Raw{bld16(r, o, 2), bld2(r, o, 0)}; }
  __device__ static float decode(const Raw& raw, float (&c)[32]) {
    const u32x4 a = raw.a;
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
      c[4 * i] = ub0(lo) - 8.f;
      c[4 * i + 1] = ub1(lo) - 8.f;
      c[4 * i + 2] = ub2(lo) - 8.f;
      c[4 * i + 3] = ub3(lo) - 8.f;
      c[16 + 4 * i] = ub0(hi) - 8.f;
      c[16 + 4 * i + 1] = ub1(hi) - 8.f;
      c[16 + 4 * i + 2] = ub2(hi) - 8.f;
      c[16 + 4 * i + 3] = ub3(hi) - 8.f;
    }
    return h2f(raw.d);
  }
  static constexpr int CODE_BYTES = 16;
  __device__ static void store_codes(const Raw& raw, uint8_t* p) {
    *reinterpret_cast<u32x4*>(p) = raw.a;
  }
  // elements j0..j0+3: low nibbles of bytes j0.. for j0 < 16, else the high
  // nibbles of bytes j0 - 16..
  __device__ static void code4(const uint8_t* p, int j0, float (&v)[4]) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p + (j0 & 15));
    const uint32_t n = ((j0 & 16) ? (w >> 4) : w) & 0x0F0F0F0Fu;
    v[0] = ub0(n) - 8.f;
    v[1] = ub1(n) - 8.f;
    v[2] = ub2(n) - 8.f;
    v[3] = ub3(n) - 8.f;
  }
};

// LDS layout of the part kernel, in floats except the last (byte) region:
//   qs     [n_rep][hd]    query rows of the KV head's query heads
//   sc     [nrp][chunk]   scores, then exp(s - m); rows n_rep..nrp-1 zero
//   st     [16][2]        each head's chunk max and sum
//   vscale [nb][chunk]    V block scales as fp32 (0 past the chunk's end)
//   vcode  [chunk][cb]    V codes, cb = nb * (32 or 16) bytes per position
struct AttnLds {
  int qs, sc, st, vscale, vcode, bytes;
};
__host__ __device__ inline AttnLds attn_lds(int n_rep, int nrp, int chunk, int nb, int cb) {
  AttnLds l;
  l.qs = 0;
  l.sc = l.qs + n_rep * 32 * nb;
  l.st = l.sc + nrp * chunk;
  l.vscale = l.st + 2 * ATT_MAX_REP;
  l.vcode = l.vscale + nb * chunk;
  l.bytes = l.vcode * 4 + chunk * cb;
  return l;
}

// Query heads per KV head rounded up to the accumulator count compiled in.
__host__ __device__ inline int attn_nrp(int n_rep) {
  return n_rep <= 1 ? 1 : n_rep <= 2 ? 2 : n_rep <= 4 ? 4 : n_rep <= 8 ? 8 : 16;
}

template <int KT, int NB, int NRP>
__global__ void __launch_bounds__(256) k_attn_part(const uint8_t* __restrict__ kc,
                                                   const uint8_t* __restrict__ vc,
                                                   uint32_t cache_bytes, int kv_len, int n_kv,
                                                   int n_rep, const float* __restrict__ q,
                                                   float scale, int chunk,
                                                   float* __restrict__ part) {
  using KB = KvBlock<KT>;
  constexpr int HD = 32 * NB, BB = KB::BB, RB = NB * BB;
  constexpr int CBB = KB::CODE_BYTES, CB = NB * CBB;
  extern __shared__ float smem[];
  const AttnLds L = attn_lds(n_rep, NRP, chunk, NB, CB);
  float* const qs = smem + L.qs;
  float* const sc = smem + L.sc;
  float* const st = smem + L.st;
  float* const vscale = smem + L.vscale;
  uint8_t* const vcode = reinterpret_cast<uint8_t*>(smem + L.vcode);
  const int c = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = c * chunk;
  const int cnt = min(chunk, kv_len - t0);
  const int n_heads = n_kv * n_rep;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc, cache_bytes), rv = make_rsrc(vc, cache_bytes);

  // Every load of the chunk goes out first, so the workgroup waits one
  // memory latency: the V blocks (one block per thread and round; blocks
  // past the chunk's end read as zero) and, for the scores, NB lanes per
  // position with lane b on block b of the K row.
  constexpr int CAP = ATT_CHUNK_CAP(NB);
  constexpr int PPW = 64 / NB;                       // positions per wave and step
  constexpr int STEPS = CAP / (4 * PPW);
  constexpr int VIT = CAP * NB / 256;
  typename KB::Raw vr[VIT];
#pragma unroll
  for (int it = 0; it < VIT; it++) {
    const int qb = tid + 256 * it, lp = qb / NB, b = qb % NB;
    const int o = (lp < cnt) ? (int)(((int64_t)(t0 + lp) * n_kv + g) * RB + b * BB) : kOobOff;
    vr[it] = KB::load(rv, o);
  }
  const int b = lane % NB, sub = lane / NB;
  typename KB::Raw kr[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; s++) {
    const int lp = wave * PPW + s * 4 * PPW + sub;
    const int row = t0 + min(lp, cnt - 1);       // lanes past the chunk repeat its last row
    kr[s] = KB::load(rk, (int)(((int64_t)row * n_kv + g) * RB + b * BB));
  }
  for (int i = tid; i < n_rep * HD; i += 256) qs[i] = q[g * n_rep * HD + i];
#pragma unroll
  for (int it = 0; it < VIT; it++) {
    const int qb = tid + 256 * it, lp = qb / NB, bb = qb % NB;
    if (lp < chunk) {
      KB::store_codes(vr[it], vcode + lp * CB + bb * CBB);
      vscale[bb * chunk + lp] = h2f(vr[it].d);
    }
  }
  __syncthreads();

  // scores s = (q . K^) / sqrt(head_dim): exact integer codes times q, then
  // the block scale, then the NB blocks on the cross-lane network
#pragma unroll
  for (int s = 0; s < STEPS; s++) {
    const int base = wave * PPW + s * 4 * PPW;
    if (base >= chunk) break;
    const int lp = base + sub;
    float cv[32];
    const float d = KB::decode(kr[s], cv);
    for (int r = 0; r < n_rep; r++) {
      const float* qr = qs + r * HD + 32 * b;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 32; k += 4) {
        const f32x4 qv = *reinterpret_cast<const f32x4*>(qr + k);
        acc = fmaf(cv[k], qv.x, acc);
        acc = fmaf(cv[k + 1], qv.y, acc);
        acc = fmaf(cv[k + 2], qv.z, acc);
        acc = fmaf(cv[k + 3], qv.w, acc);
      }
      float sv = acc * d;
#pragma unroll
      for (int m = 1; m < NB; m <<= 1) sv += __shfl_xor(sv, m, 64);
      if (b == 0 && lp < chunk) sc[r * chunk + lp] = (lp < cnt) ? sv * scale : -INFINITY;
    }
  }
  __syncthreads();

  // the chunk's softmax statistics, one wave per query head; padded heads
  // get zero weights
  for (int r = wave; r < NRP; r += 4) {
    float* const sr = sc + r * chunk;
    if (r >= n_rep) {
      for (int i = lane; i < chunk; i += 64) sr[i] = 0.f;
      continue;
    }
    float m = -INFINITY;
    for (int i = lane; i < chunk; i += 64) m = fmaxf(m, sr[i]);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
    float l = 0.f;
    for (int i = lane; i < chunk; i += 64) {
      const float p = expf(sr[i] - m);
      sr[i] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      st[2 * r] = m;
      st[2 * r + 1] = l;
    }
  }
  __syncthreads();

  // sum_t exp(s - m) V^[t]: thread (dg, sl) holds output columns 4dg..4dg+3
  // of every head and takes groups of 4 positions sl, sl + TP, ...; the TP
  // slices of a column group are adjacent lanes, summed on the cross-lane
  // network at the end.
  constexpr int DG = HD / 4, TP = 256 / DG;
  const int dg = tid / TP, sl = tid % TP;
  const int blk = dg / 8, j0 = 4 * (dg % 8);
  float acc[NRP][4];
#pragma unroll
  for (int r = 0; r < NRP; r++)
#pragma unroll
    for (int e = 0; e < 4; e++) acc[r][e] = 0.f;
  const int ng = (cnt + 3) / 4;
  for (int g4 = sl; g4 < ng; g4 += TP) {
    const int lp0 = 4 * g4;
    const f32x4 sv = *reinterpret_cast<const f32x4*>(vscale + blk * chunk + lp0);
    float v[4][4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      KB::code4(vcode + (lp0 + k) * CB + blk * CBB, j0, v[k]);
#pragma unroll
      for (int e = 0; e < 4; e++) v[k][e] *= sv[k];
    }
#pragma unroll
    for (int r = 0; r < NRP; r++) {
      const f32x4 pv = *reinterpret_cast<const f32x4*>(sc + r * chunk + lp0);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        float a = acc[r][e];
        a = fmaf(pv.x, v[0][e], a);
        a = fmaf(pv.y, v[1][e], a);
        a = fmaf(pv.z, v[2][e], a);
        a = fmaf(pv.w, v[3][e], a);
        acc[r][e] = a;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NRP; r++)
#pragma unroll
    for (int e = 0; e < 4; e++)
#pragma unroll
      for (int m = 1; m < TP; m <<= 1) acc[r][e] += __shfl_xor(acc[r][e], m, 64);
  if (sl == 0) {
#pragma unroll
    for (int r = 0; r < NRP; r++) {
      if (r < n_rep) {
        float* const pr = part + ((int64_t)c * n_heads + g * n_rep + r) * (HD + 2);
#pragma unroll
        for (int e = 0; e < 4; e++) pr[4 * dg + e] = acc[r][e];
        if (dg == 0) {
          pr[HD] = st[2 * r];
          pr[HD + 1] = st[2 * r + 1];
        }
      }
    }
  }
}

// out[h][d] from the per-chunk statistics, in a fixed order: the largest
// chunk max M (a tree over thread-strided maxima), then, for every output
// column, the sums over chunks of e^(m_c - M) acc_c and e^(m_c - M) l_c,
// each thread taking every S-th chunk (S = 256 / hd) with its loads
// independent of one another, the S partial sums added in slice order.
__global__ void __launch_bounds__(256) k_attn_combine(const float* __restrict__ part,
                                                      int n_chunks, int n_heads, int hd,
                                                      float* __restrict__ out) {
  __shared__ float red[256], rden[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int64_t stride = (int64_t)n_heads * (hd + 2);
  const float* const p0 = part + (int64_t)h * (hd + 2);
  float mx = -INFINITY;
  for (int c = tid; c < n_chunks; c += 256) mx = fmaxf(mx, p0[c * stride + hd]);
  red[tid] = mx;
  __syncthreads();
  for (int k = 128; k >= 1; k >>= 1) {
    if (tid < k) red[tid] = fmaxf(red[tid], red[tid + k]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  const int S = 256 / hd, d = tid % hd, sl = tid / hd;
  float num = 0.f, den = 0.f;
#pragma unroll 8
  for (int c = sl; c < n_chunks; c += S) {
    const float* const p = p0 + c * stride;
    const float w = expf(p[hd] - mx);
    num = fmaf(w, p[d], num);
    den = fmaf(w, p[hd + 1], den);
  }
  red[tid] = num;
  rden[tid] = den;
  __syncthreads();
  if (sl == 0) {
    for (int k = 1; k < S; k++) {
      num += red[k * hd + d];
      den += rden[k * hd + d];
    }
    out[(int64_t)h * hd + d] = num / den;
  }
}

// Positions per chunk: enough chunks for ~1024 workgroups, a multiple of 64,
// at most 256 and within the LDS budget for q8_0 rows (the larger block), so
// the split does not depend on the cache's type.
AttnPlan attn_plan(int64_t kv_len, int n_kv, int n_rep, int head_dim) {
  const int nb = head_dim / 32;
  int chunk_max = ATT_CHUNK_CAP(nb);
  while (chunk_max > 64 &&
         attn_lds(n_rep, attn_nrp(n_rep), chunk_max, nb, nb * KvBlock<GQ_Q8_0>::CODE_BYTES).bytes >
             ATT_LDS)
    chunk_max -= 64;
  const int64_t target = (1024 + n_kv - 1) / n_kv;
  int64_t chunk = (kv_len + target - 1) / target;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk < 64) chunk = 64;
  if (chunk > chunk_max) chunk = chunk_max;
  AttnPlan p;
  p.chunk = (int)chunk;
  p.n_chunks = (kv_len + chunk - 1) / chunk;
  return p;
}

int64_t attn_workspace_bytes(int64_t kv_len, int n_kv, int n_heads, int head_dim) {
  const AttnPlan p = attn_plan(kv_len, n_kv, n_heads / n_kv, head_dim);
  return p.n_chunks * n_heads * (head_dim + 2) * 4;
}

template <int KT, int NB, int NRP>
static hipError_t attn_t(const void* k_cache, const void* v_cache, int64_t kv_len, int n_kv,
                         const float* q, int n_heads, float* out, float* part, hipStream_t st) {
  constexpr int HD = 32 * NB, BB = KvBlock<KT>::BB, CB = NB * KvBlock<KT>::CODE_BYTES;
  const int n_rep = n_heads / n_kv;
  const AttnPlan p = attn_plan(kv_len, n_kv, n_rep, HD);
  const AttnLds L = attn_lds(n_rep, NRP, p.chunk, NB, CB);
  const uint32_t cache_bytes = (uint32_t)(kv_len * n_kv * NB * BB);
  const float scale = (float)(1.0 / std::sqrt((double)HD));
  hipLaunchKernelGGL((k_attn_part<KT, NB, NRP>), dim3((unsigned)p.n_chunks, (unsigned)n_kv),
                     dim3(256), (size_t)L.bytes, st, (const uint8_t*)k_cache,
                     (const uint8_t*)v_cache, cache_bytes, (int)kv_len, n_kv, n_rep, q, scale,
                     p.chunk, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)n_heads), dim3(256), 0, st, part,
                     (int)p.n_chunks, n_heads, HD, out);
  return hipGetLastError();
}

template <int KT, int NB>
static hipError_t attn_rep(const void* k_cache, const void* v_cache, int64_t kv_len, int n_kv,
                           const float* q, int n_heads, float* out, float* part, hipStream_t st) {
  switch (attn_nrp(n_heads / n_kv)) {
    case 1: return attn_t<KT, NB, 1>(k_cache, v_cache, kv_len, n_kv, q, n_heads, out, part, st);
    case 2: return attn_t<KT, NB, 2>(k_cache, v_cache, kv_len, n_kv, q, n_heads, out, part, st);
    case 4: return attn_t<KT, NB, 4>(k_cache, v_cache, kv_len, n_kv, q, n_heads, out, part, st);
    case 8: return attn_t<KT, NB, 8>(k_cache, v_cache, kv_len, n_kv, q, n_heads, out, part, st);
    default: return attn_t<KT, NB, 16>(k_cache, v_cache, kv_len, n_kv, q, n_heads, out, part, st);
  }
}

template <int KT>
static hipError_t attn_hd(int head_dim, const void* k_cache, const void* v_cache, int64_t kv_len,
                          int n_kv, const float* q, int n_heads, float* out, float* part,
                          hipStream_t st) {
  switch (head_dim) {
    case 64: return attn_rep<KT, 2>(k_cache, v_cache, kv_len, n_kv, q, n_heads, out, part, st);
    case 128: return attn_rep<KT, 4>(k_cache, v_cache, kv_len, n_kv, q, n_heads, out, part, st);
    case 256: return attn_rep<KT, 8>(k_cache, v_cache, kv_len, n_kv, q, n_heads, out, part, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_decode(int kv_type, const void* k_cache, const void* v_cache,
                              int64_t kv_len, int n_kv, int head_dim, const float* q,
                              int n_heads, float* out, float* workspace, hipStream_t st) {
  switch (kv_type) {
    case GQ_Q8_0:
      return attn_hd<GQ_Q8_0>(head_dim, k_cache, v_cache, kv_len, n_kv, q, n_heads, out,
                              workspace, st);
    case GQ_Q4_0:
      return attn_hd<GQ_Q4_0>(head_dim, k_cache, v_cache, kv_len, n_kv, q, n_heads, out,
                              workspace, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gq
