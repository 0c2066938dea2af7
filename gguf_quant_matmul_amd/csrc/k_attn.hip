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
#ifndef GQ_ATT_COMBINE_UNROLL
#define GQ_ATT_COMBINE_UNROLL 16          // chunks per thread and round in the combine
#endif
#ifndef GQ_ATT_WGS
#define GQ_ATT_WGS 1024                   // part-kernel workgroups per call
#endif
#ifndef GQ_ATT_WAVES
#define GQ_ATT_WAVES 4
#endif
constexpr int ATT_WAVES(int nrp, int nb) { return nrp <= 8 && nb <= 4 ? GQ_ATT_WAVES : 1; }
// Largest chunk (positions) for NB blocks per row.
constexpr int ATT_CHUNK_CAP(int nb) { return nb > 4 ? 128 : 256; }

// Bytes of lo (0..3) and hi (4..7) as the fp16 values 1024 + byte (fp16 has
// unit spacing on [1024, 2048), so the bytes go straight into the low
// mantissa bits under the exponent byte 0x64).
__device__ __forceinline__ f16x8 bytes_1024(uint32_t lo, uint32_t hi) {
  const uint32_t e = 0x64646464u;
  const uint32_t w0 = __builtin_amdgcn_perm(e, lo, 0x04010400u);
  const uint32_t w1 = __builtin_amdgcn_perm(e, lo, 0x04030402u);
  const uint32_t w2 = __builtin_amdgcn_perm(e, hi, 0x04010400u);
  const uint32_t w3 = __builtin_amdgcn_perm(e, hi, 0x04030402u);
  return __builtin_bit_cast(f16x8, u32x4{w0, w1, w2, w3});
}

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
  // A lane's matrix-core share of a block: codes 8g .. 8g + 7 as exact
  // fp16, (1024 + (q + 128)) - 1152.  They are read as a 12-byte window of
  // the block: at byte 8g with the codes from its byte 2 (the window of
  // g = 0 starts with d), for g = 3 at byte 22 with the codes from its byte
  // 4, so no window reaches past the block.
  __device__ static int win_off(int g) { return g == 3 ? 22 : 8 * g; }
  __device__ static bool win_hi(int g) { return g == 3; }
  __device__ static f16x8 frag_codes(u32x2 c, int) {
    const f16x8 v = bytes_1024(c.x ^ 0x80808080u, c.y ^ 0x80808080u);
    return v - (_Float16)1152.f;
  }
  static constexpr int CODE_BYTES = 32;
  __device__ static void store_codes(const Raw& raw, uint8_t* p) {     // 16-byte aligned
    *reinterpret_cast<u32x4*>(p) = raw.a;
    *reinterpret_cast<u32x4*>(p + 16) = raw.b;
  }
  static constexpr float BIAS = 0.f;          // value = code - BIAS
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
  // elements 8g .. 8g + 7: low nibbles of code bytes 8g.. for g < 2, high
  // nibbles of code bytes 8(g - 2).. for g >= 2; the 12-byte window of
  // g = 0, 2 is block bytes 0..11 (d first, codes from its byte 2), of
  // g = 1, 3 block bytes 6..17 (codes from its byte 4)
  __device__ static int win_off(int g) { return (g & 1) ? 6 : 0; }
  __device__ static bool win_hi(int g) { return g & 1; }
  __device__ static f16x8 frag_codes(u32x2 c, int g) {
    const int sh = (g & 2) ? 4 : 0;
    const f16x8 v = bytes_1024((c.x >> sh) & 0x0F0F0F0Fu, (c.y >> sh) & 0x0F0F0F0Fu);
    return v - (_Float16)1032.f;
  }
  static constexpr int CODE_BYTES = 16;
  __device__ static void store_codes(const Raw& raw, uint8_t* p) {
    *reinterpret_cast<u32x4*>(p) = raw.a;
  }
  static constexpr float BIAS = 8.f;          // value = nibble - 8
  // nibbles of elements j0..j0+3 (low nibbles of bytes j0.. for j0 < 16,
  // else the high nibbles of bytes j0 - 16..) as exact fp32, bias not taken
  __device__ static void code4(const uint8_t* p, int j0, float (&v)[4]) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p + (j0 & 15));
    const uint32_t n = ((j0 & 16) ? (w >> 4) : w) & 0x0F0F0F0Fu;
    v[0] = ub0(n);
    v[1] = ub1(n);
    v[2] = ub2(n);
    v[3] = ub3(n);
  }
};

// LDS layout of the part kernel, offsets in floats:
//   qs     [n_rep][hd]    query rows of the KV head's query heads, read into
//                         registers before the scores overwrite them
//   sc     [nrp][chunk]   scores, then exp(s - m); rows n_rep..nrp-1 zero
//                         (same region as qs)
//   st     [16][2]        each head's chunk max and sum
//   qinv   [16]           2^-k of each query head's scale (q enters as q 2^k)
//   vscale [nb][chunk]    V block scales, fp16 bit patterns
//   vcode  [chunk][cb]    V codes, cb = nb * (32 or 16) bytes per position
// For q8_0 rows of 128 values and 5 query heads per KV head a 256-position
// chunk takes 40,064 bytes: four workgroups share a CU's 160 KiB.
struct AttnLds {
  int qs, sc, st, qinv, vscale, vcode, bytes;
};
__host__ __device__ inline AttnLds attn_lds(int n_rep, int nrp, int chunk, int nb, int cb) {
  AttnLds l;
  l.qs = 0;
  l.sc = 0;
  l.st = (n_rep * 32 * nb > nrp * chunk) ? n_rep * 32 * nb : nrp * chunk;
  l.qinv = l.st + 2 * ATT_MAX_REP;
  l.vscale = l.qinv + ATT_MAX_REP;
  l.vcode = l.vscale + nb * chunk / 2;
  l.bytes = l.vcode * 4 + chunk * cb;
  return l;
}

// Query heads per KV head rounded up to the accumulator count compiled in.
__host__ __device__ inline int attn_nrp(int n_rep) {
  return n_rep <= 2 ? n_rep : n_rep <= 4 ? 4 : n_rep <= 5 ? 5 : n_rep <= 8 ? 8 : 16;
}

template <int KT, int NB, int NRP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ATT_WAVES(NRP, NB))))
k_attn_part(const uint8_t* __restrict__ kc,
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
  float* const qinv = smem + L.qinv;
  uint16_t* const vscale = reinterpret_cast<uint16_t*>(smem + L.vscale);
  uint8_t* const vcode = reinterpret_cast<uint8_t*>(smem + L.vcode);
  const int c = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = c * chunk;
  const int cnt = min(chunk, kv_len - t0);
  const int n_heads = n_kv * n_rep;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc, cache_bytes), rv = make_rsrc(vc, cache_bytes);

  // Every load of the chunk goes out first (loads complete in issue order):
  // the query rows, then the V blocks and the K fragments of the scores.
  constexpr int QPT = (NRP * HD + 255) / 256;        // query values per thread, at most
  float qreg[QPT];
#pragma unroll
  for (int i = 0; i < QPT; i++) {
    const int idx = tid + 256 * i;
    qreg[i] = (idx < n_rep * HD) ? q[g * n_rep * HD + idx] : 0.f;
  }
  constexpr int CAP = ATT_CHUNK_CAP(NB);
  constexpr int TILES = CAP / 64;                    // 16-position tiles per wave
  // the V blocks: one block per thread and round; blocks past the chunk's
  // end read as zero
  constexpr int VIT = CAP * NB / 256;
  typename KB::Raw vr[VIT];
#pragma unroll
  for (int it = 0; it < VIT; it++) {
    const int qb = tid + 256 * it, lp = qb / NB, b = qb % NB;
    const int o = (lp < cnt) ? (int)(((int64_t)(t0 + lp) * n_kv + g) * RB + b * BB) : kOobOff;
    vr[it] = KB::load(rv, o);
  }
  // K for the scores on the matrix cores: tiles of 16 positions, wave w
  // taking tiles w, w + 4, ...; lane l holds position l % 16 of the tile and
  // codes 8(l / 16) .. 8(l / 16) + 7 of every block, one 12-byte window
  // load per block; the block scale is in the window of lane l % 16, which
  // the other lanes of the position read across lanes
  const int mn = lane & 15, kg = lane >> 4;
  u32x3 kw[TILES][NB];
#pragma unroll
  for (int s = 0; s < TILES; s++) {
    const int lp = 16 * (wave + 4 * s) + mn;
    const int row = t0 + min(lp, cnt - 1);       // lanes past the chunk repeat its last row
    const int o = (int)(((int64_t)row * n_kv + g) * RB);
#pragma unroll
    for (int bb = 0; bb < NB; bb++) kw[s][bb] = bld12(rk, o + bb * BB, KB::win_off(kg));
  }
#pragma unroll
  for (int i = 0; i < QPT; i++) {
    const int idx = tid + 256 * i;
    if (idx < n_rep * HD) qs[idx] = qreg[i];
  }
  // the V blocks into LDS (the loads have been in flight since the start)
#pragma unroll
  for (int it = 0; it < VIT; it++) {
    const int qb = tid + 256 * it, lp = qb / NB, bb = qb % NB;
    if (lp < chunk) {
      KB::store_codes(vr[it], vcode + lp * CB + bb * CBB);
      vscale[bb * chunk + lp] = (uint16_t)vr[it].d;
    }
  }
  __syncthreads();

  // scores s = (q . K^) / sqrt(head_dim) as 16 heads x 16 positions tiles of
  // v_mfma_f32_16x16x32_f16, one 32-element block per step: A = the query
  // rows' block as two fp16 parts (hi + lo, ~22 bits of each fp32 q 2^k,
  // with 2^k per head putting its largest |q| in [2^13, 2^14), so every fp32
  // magnitude fits), B = the block's codes (exact in fp16); each step's
  // product is scaled by the block scale of its position (exact in fp32 up
  // to one rounding) and summed in fp32, and the score takes 2^-k.  Lane l
  // of a result holds heads 4(l/16) .. +3 of position l % 16.
  float qv[NB][8];
  float qm = 0.f;
#pragma unroll
  for (int bb = 0; bb < NB; bb++) {
    const float* const qr = qs + mn * HD + 32 * bb + 8 * kg;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      qv[bb][i] = (mn < n_rep) ? qr[i] : 0.f;
      qm = fmaxf(qm, fabsf(qv[bb][i]));
    }
  }
  qm = max_rows4(qm);                            // the head's max over its 4 lane rows
  const int qk = pow2_exp_for<14>(qm);
  const float qsc = __builtin_ldexpf(1.f, qk);
  if (kg == 0) qinv[mn] = __builtin_ldexpf(1.f, -qk);
  f16x8 qh[NB], ql[NB];
#pragma unroll
  for (int bb = 0; bb < NB; bb++) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; i++) split2_scaled(qv[bb][2 * i], qv[bb][2 * i + 1], qsc, h[i], l[i]);
    qh[bb] = __builtin_bit_cast(f16x8, u32x4{h[0], h[1], h[2], h[3]});
    ql[bb] = __builtin_bit_cast(f16x8, u32x4{l[0], l[1], l[2], l[3]});
  }
  __syncthreads();                               // qs is read; sc overwrites it
  const f32x4 qiv = *reinterpret_cast<const f32x4*>(qinv + 4 * kg);
#pragma unroll
  for (int s = 0; s < TILES; s++) {
    const int tile = wave + 4 * s;
    if (16 * tile >= chunk) break;
    f32x4 sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bb = 0; bb < NB; bb++) {
      const u32x3 w = kw[s][bb];
      const bool hi = KB::win_hi(kg);
      const uint32_t a0 = hi ? w.y : w.x, a1 = hi ? w.z : w.y, sh = hi ? 0u : 16u;
      const u32x2 c8 = {__builtin_amdgcn_alignbit(a1, a0, sh), __builtin_amdgcn_alignbit(w.z, a1, sh)};
      const f16x8 B = KB::frag_codes(c8, kg);
      const uint32_t dsrc = (uint32_t)__shfl((int)w.x, mn, 64);   // d from lane mn's window
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      f32x4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[bb], B, z, 0, 0, 0);
      D = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[bb], B, D, 0, 0, 0);
      const float ds = h2f(dsrc);
#pragma unroll
      for (int v = 0; v < 4; v++) sv[v] = fmaf(D[v], ds, sv[v]);
    }
    const int lp = 16 * tile + mn;
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int r = 4 * kg + v;
      if (r < n_rep && lp < chunk) sc[r * chunk + lp] = (lp < cnt) ? (sv[v] * qiv[v]) * scale : -INFINITY;
    }
  }
  __syncthreads();

  // the chunk's softmax statistics, 16 lanes per query head (lane l of wave
  // w: head 4w + l / 16, positions 4(l % 16) + 64 i), reduced on the DPP
  // network; padded heads get zero weights
  {
    const int hr = 4 * wave + (lane >> 4), hp = 4 * (lane & 15);
    if (hr < NRP) {
      float* const sr = sc + hr * chunk;
      if (hr >= n_rep) {
        for (int i = hp; i < chunk; i += 64) *reinterpret_cast<f32x4*>(sr + i) = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        float m = -INFINITY;
        for (int i = hp; i < chunk; i += 64) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(sr + i);
          m = fmaxf(m, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
        }
        m = row16_max(m);
        float l = 0.f;
        for (int i = hp; i < chunk; i += 64) {
          f32x4 v = *reinterpret_cast<const f32x4*>(sr + i);
#pragma unroll
          for (int e = 0; e < 4; e++) v[e] = expf(v[e] - m);
          *reinterpret_cast<f32x4*>(sr + i) = v;
          l += (v.x + v.y) + (v.z + v.w);
        }
        l = row16_sum(l);
        if ((lane & 15) == 0) {
          st[2 * hr] = m;
          st[2 * hr + 1] = l;
        }
      }
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
    const u32x2 hv = *reinterpret_cast<const u32x2*>(vscale + blk * chunk + lp0);
    const f32x4 sv = {h2f(hv.x), h2f(hv.x >> 16), h2f(hv.y), h2f(hv.y >> 16)};
    float v[4][4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      KB::code4(vcode + (lp0 + k) * CB + blk * CBB, j0, v[k]);
      // (q - BIAS) d as one rounding: -BIAS d is exact (BIAS is 0 or 8)
      if constexpr (KB::BIAS != 0.f) {
        const float nb = -KB::BIAS * sv[k];
#pragma unroll
        for (int e = 0; e < 4; e++) v[k][e] = fmaf(v[k][e], sv[k], nb);
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) v[k][e] *= sv[k];
      }
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

// out[h][d] from the per-chunk statistics, in a fixed order.  Workgroup
// (h, column slice of 32): thread (d, sl) takes chunks sl, sl + 8, ...,
// GQ_ATT_COMBINE_UNROLL of them per round with all their loads in flight,
// and keeps a running max m and, at that max, num = sum e^(m_c - m) acc_c[d]
// and den = sum e^(m_c - m) l_c; the 8 slices are then merged in slice order
// at their largest m.
__global__ void __launch_bounds__(256) k_attn_combine(const float* __restrict__ part,
                                                      int n_chunks, int n_heads, int hd,
                                                      float* __restrict__ out) {
  constexpr int U = GQ_ATT_COMBINE_UNROLL;
  __shared__ float rm[256], rnum[256], rden[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int64_t stride = (int64_t)n_heads * (hd + 2);
  const float* const p0 = part + (int64_t)h * (hd + 2);
  const int d = 32 * blockIdx.y + (tid & 31), sl = tid >> 5;
  float m = -INFINITY, num = 0.f, den = 0.f;
  for (int c0 = sl; c0 < n_chunks; c0 += 8 * U) {
    float mc[U], ac[U], lc[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int c = c0 + 8 * u;
      const float* const p = p0 + (int64_t)min(c, n_chunks - 1) * stride;   // past the last: weight 0
      mc[u] = (c < n_chunks) ? p[hd] : -INFINITY;
      ac[u] = p[d];
      lc[u] = p[hd + 1];
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; u++) mx = fmaxf(mx, mc[u]);
    if (mx > -INFINITY) {
      const float r = expf(m - mx);            // 0 while nothing is summed (m = -inf)
      num *= r;
      den *= r;
#pragma unroll
      for (int u = 0; u < U; u++) {
        const float w = expf(mc[u] - mx);
        num = fmaf(w, ac[u], num);
        den = fmaf(w, lc[u], den);
      }
      m = mx;
    }
  }
  rm[tid] = m;
  rnum[tid] = num;
  rden[tid] = den;
  __syncthreads();
  if (sl == 0) {
    float M = m;
    for (int k = 1; k < 8; k++) M = fmaxf(M, rm[32 * k + (tid & 31)]);
    float nn = 0.f, dd = 0.f;
    for (int k = 0; k < 8; k++) {
      const float mk = rm[32 * k + (tid & 31)];
      const float w = (mk == -INFINITY) ? 0.f : expf(mk - M);
      nn = fmaf(w, rnum[32 * k + (tid & 31)], nn);
      dd = fmaf(w, rden[32 * k + (tid & 31)], dd);
    }
    out[(int64_t)h * hd + d] = nn / dd;
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
  const int64_t target = (GQ_ATT_WGS + n_kv - 1) / n_kv;
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
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)n_heads, HD / 32), dim3(256), 0, st, part,
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
    case 5: return attn_t<KT, NB, 5>(k_cache, v_cache, kv_len, n_kv, q, n_heads, out, part, st);
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
