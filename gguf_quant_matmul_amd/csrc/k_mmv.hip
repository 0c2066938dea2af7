// k_mmv.hip — small-batch matmul over GGUF blocks (2 <= n_tok, a few token
// passes of 8, 16 or 32) on the gfx950 matrix cores.  Each weight is decoded
// once per pass and reused for every token of the pass ("Local LLM
// inference", "The mmap backend"); with so few tokens the work is still
// bound by the weight stream ("12 — llama.cpp / GGUF", "The bandwidth cap"),
// so the kernel is built around keeping enough weight bytes in flight:
//
//   * a workgroup owns one tile of 16 weight rows; its KS waves split the
//     row's 256-weight slabs (slab s goes to wave s % KS), so even a
//     4096-row matrix spreads over every compute unit;
//   * every wave streams its slabs through a D-deep register ring that holds
//     both the weights and the matching activations: loads complete in issue
//     order, so activations fetched later than the weights would cap the
//     weights' prefetch distance at their own;
//   * activations are fetched with whole-cache-line loads (each load
//     instruction covers 8 full 128-byte lines) and moved into the matrix
//     op's A layout through the wave's own block of LDS.  Loading them
//     directly in A layout would touch 64 lines per instruction, and the
//     per-CU load pipeline, not HBM, would then set the speed;
//   * the contraction is v_mfma_f32_16x16x32_f16 with A = 16 tokens x 32 k of
//     x and B = 32 k x 16 rows of decoded weights (a 32-token pass feeds each
//     decoded B to two A tiles).  Each lane's 8 k values
//     are 8 consecutive columns; the weight bytes are put into that order
//     with v_perm_b32, which also ORs in the fp16 exponent;
//   * B holds exact integers wherever the format allows (Hitchhiker's Guide
//     §11.2, w = (d*sc)*q - dmin*m): Q4_K B = sc*q (<= 945) with the min
//     term as a second product of x with m (<= 63), both scaled by the
//     block's d and dmin in fp32; Q6_K B = RNE_fp16(sc*(q-32)) (exact unless
//     |sc*(q-32)| > 2048); Q4_0 / Q5_0 / Q8_0 B = q - offset with d applied
//     per block in fp32.  fp32 x is scaled per token and slab by a power of
//     two from the slab's largest |x| (any fp32 magnitude then fits fp16),
//     split into two fp16 parts (hi, lo) that both go through the matrix op,
//     and the slab's products take the inverse power;
//   * the KS partial tiles are summed in LDS in wave order, so the result is
//     the same on every run.
#include "gq_device.h"
#include "gq_launch.h"

namespace gq {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ f16x2 hpair(float a, float b) { return f16x2{(_Float16)a, (_Float16)b}; }
__device__ __forceinline__ f16x8 cat8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Bytes 0,1 (PAIR 0) or 2,3 (PAIR 1) of v as the low bytes of two fp16
// values whose high byte is E (v_perm_b32; selector 4 picks byte 0 of E).
template <int PAIR>
__device__ __forceinline__ f16x2 bytes_as_h2(uint32_t e4, uint32_t v) {
  return as_h2(__builtin_amdgcn_perm(e4, v, PAIR ? 0x04030402u : 0x04010400u));
}
// Eight bytes (two dwords) -> eight fp16 values with high byte E, in byte order.
__device__ __forceinline__ void bytes8(uint32_t e4, uint32_t v0, uint32_t v1, f16x2 o[4]) {
  o[0] = bytes_as_h2<0>(e4, v0);
  o[1] = bytes_as_h2<1>(e4, v0);
  o[2] = bytes_as_h2<0>(e4, v1);
  o[3] = bytes_as_h2<1>(e4, v1);
}
constexpr uint32_t kE1024 = 0x64646464u;   // fp16 0x64XX = 1024 + XX
constexpr uint32_t kE256 = 0x5C5C5C5Cu;    // fp16 0x5CXX = 256 + XX / 4

// ---------------------------------------------------------------------------
// Activation slot: one slab (256 columns) of the pass's P tokens as loaded.
// fp16: load i, lane l holds token 2i + l/32, 16-byte chunk l%32 (8 columns).
// fp32: load i, lane l holds token i, columns 4l .. 4l+3.
template <bool XLO, int P> struct XS {
  u32x4 v[XLO ? P : P / 2];
};

// The wave's LDS block: token t's 256 columns at t * 512 bytes, 16-byte chunk
// k stored at position k ^ (t & 7), so the 8 lanes that LDS serves together
// hit 8 different bank groups both when storing a load's chunks and when
// reading A fragments.  fp32 activations store hi = RNE_fp16(x s) in the
// first P rows and lo = RNE_fp16(x s - hi) in the next P, where s = 2^k is
// chosen per token and slab from the slab's largest |x| (so |x s| < 2^14:
// every fp32 magnitude fits fp16, and hi + lo keeps ~22 bits of each value
// within 2^-17 of that largest one); the slab's products are multiplied by
// 2^-k when they join the accumulators.
__device__ __forceinline__ int xslot(int t, int k) { return t * 512 + ((k ^ (t & 7)) << 4); }

// Bytes of the per-wave scale block after the weight staging: s[16], 1/s[16].
template <bool XLO> constexpr int kSB = XLO ? 128 : 0;

template <bool XLO, int P>
__device__ __forceinline__ void stage_x(uint8_t* xw, float* sv, const XS<XLO, P>& xs, int lane) {
  if constexpr (!XLO) {
#pragma unroll
    for (int i = 0; i < P / 2; i++)
      *reinterpret_cast<u32x4*>(xw + xslot(2 * i + (lane >> 5), lane & 31)) = xs.v[i];
  } else {
    // each token's largest |x| over the slab (lane l holds its columns 4l..4l+3)
    float m[P];
#pragma unroll
    for (int i = 0; i < P; i++) {
      const f32x4 f = __builtin_bit_cast(f32x4, xs.v[i]);
      m[i] = fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w)));
    }
    transposed_max<P>(m);                   // register j, row rho: token j + (P/4) rho
    if ((lane & 15) == 0) {
#pragma unroll
      for (int j = 0; j < P / 4; j++) {
        const int k = pow2_exp_for<14>(m[j]), t = j + (P / 4) * (lane >> 4);
        sv[t] = __builtin_ldexpf(1.f, k);
        sv[16 + t] = __builtin_ldexpf(1.f, -k);
      }
    }
    float s[P];                              // every lane: the scale of every token
#pragma unroll
    for (int q = 0; q < P / 4; q++) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sv + 4 * q);
      s[4 * q] = v.x; s[4 * q + 1] = v.y; s[4 * q + 2] = v.z; s[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < P; i++) {
      const f32x4 f = __builtin_bit_cast(f32x4, xs.v[i]);
      uint32_t h0, l0, h1, l1;
      split2_scaled(f.x, f.y, s[i], h0, l0);
      split2_scaled(f.z, f.w, s[i], h1, l1);
      const int o = xslot(i, lane >> 1) + 8 * (lane & 1);
      *reinterpret_cast<u32x2*>(xw + o) = u32x2{h0, h1};
      *reinterpret_cast<u32x2*>(xw + P * 512 + o) = u32x2{l0, l1};
    }
  }
}

// 1/s of the four tokens 4g .. 4g+3 whose results lane group g accumulates
// (with P = 8 tokens 8..15 repeat 0..7 and are not stored).
template <bool XLO, int P>
__device__ __forceinline__ f32x4 inv_scales(const float* sv, int g) {
  if constexpr (!XLO) return f32x4{1.f, 1.f, 1.f, 1.f};
  else return *reinterpret_cast<const f32x4*>(sv + 16 + ((4 * g) & (P - 1)));
}

// A fragment (8 consecutive columns, chunk k of the slab) of token row t.
// With P = 8 the upper 8 MFMA rows repeat rows 0..7; their results are not stored.
template <int P>
__device__ __forceinline__ f16x8 read_a(const uint8_t* xw, int t, int k) {
  const int tt = (P == 8) ? (t & 7) : t;
  return *reinterpret_cast<const f16x8*>(xw + xslot(tt, k));
}

// ---------------------------------------------------------------------------
// Weight slot: the lane's share of one slab of its row.
template <int T> struct WS;

template <> struct WS<GQ_Q4_K> {     // slab = one super-block; sub-blocks 2g, 2g+1
  u32x4 hd, q[2];
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int g) {
    hd = bld16(r, vo, 0);
    q[0] = bld16(r, vo + 32 * g, 16);
    q[1] = bld16(r, vo + 32 * g, 32);
  }
};

template <> struct WS<GQ_Q5_K> {     // Q4_K's share plus the 64 fifth bits
  u32x4 hd, q[2];
  u32x2 qh;
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int g) {
    hd = bld16(r, vo, 0);
    qh = bld8(r, vo + 8 * g, 16);
    q[0] = bld16(r, vo + 32 * g, 48);
    q[1] = bld16(r, vo + 32 * g, 64);
  }
};

template <> struct WS<GQ_Q6_K> {     // slab = one super-block; 32-groups 2g, 2g+1
  u32x4 l[2], h;
  uint32_t sc4, d;
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int g) {
    l[0] = bld16(r, vo + 32 * g, 18);
    l[1] = bld16(r, vo + 32 * g, 34);
    h = bld16(r, vo + 16 * g, 146);
    sc4 = bld4(r, vo + 4 * g, 2);
    d = bld2(r, vo, 0);
  }
};

template <> struct WS<GQ_Q2_K> {     // slab = one super-block; 16-weight sub-blocks 4g..4g+3
  uint32_t dm, sm;                   // d | dmin; their scale/min bytes
  u32x4 q;                           // code bytes of 32-groups 2g, 2g+1
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int g) {
    dm = bld4(r, vo, 0);
    sm = bld4(r, vo + 4 * g, 4);
    q = bld16(r, vo + 16 * g, 20);
  }
};

template <> struct WS<GQ_Q3_K> {     // slab = one super-block; sub-blocks 4g..4g+3
  uint32_t d, sc;                    // d; scale fields 4g.. (24 bits)
  u32x4 q;                           // low-bit plane bytes of groups 2g, 2g+1
  u32x2 qh;                          // third bits of elements 64g .. 64g+63
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int g) {
    d = bld2(r, vo, 0);
    sc = bld4(r, vo + 3 * g, 2);
    q = bld16(r, vo + 16 * g, 14);
    qh = bld8(r, vo + 8 * g, 78);
  }
};

// 32-weight types: slab = 8 blocks of the row.  Lane group g loads blocks 2g
// and 2g+1, each with whole dwords of its own bytes and a 2-byte tail (3 or
// 4 loads per block, from a 2-byte-aligned start, none reaching past its
// block), and stage_w regroups them through the wave's LDS into codes,
// scales and Q5_0 high bits, so the matrix-op steps read whole words.
template <int T> struct WS32 {
  static constexpr int BB = Geo<T>::BB;
  static constexpr int NDW = (BB - 2) / 4;   // whole dwords per block: 8, 4, 5
  static constexpr int CB = (T == GQ_Q8_0) ? 32 : 16;   // code bytes per block
  static constexpr int WD = 16 * 8 * CB;     // LDS: codes [16 rows][8 blocks][CB]
  static constexpr int WQ = WD + 256;        //      scales [16][8] fp16, then
  static constexpr int WBYTES = WQ + (T == GQ_Q5_0 ? 512 : 0);   // high bits [16][8]
  uint32_t raw[2][NDW + 1];                  // per block: dwords, then the tail
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo) {
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const int o = vo + b * BB;
#pragma unroll
      for (int k = 0; k < NDW / 4; k++) {
        const u32x4 v = bld16(r, o, 16 * k);
        raw[b][4 * k] = v.x; raw[b][4 * k + 1] = v.y; raw[b][4 * k + 2] = v.z; raw[b][4 * k + 3] = v.w;
      }
      if constexpr (NDW % 4) raw[b][NDW - 1] = bld4(r, o, 4 * (NDW - 1));
      raw[b][NDW] = bld2(r, o, 4 * NDW);
    }
  }
};
template <int T> constexpr int kWB = 0;      // weight staging bytes per wave in LDS
template <> constexpr int kWB<GQ_Q4_0> = WS32<GQ_Q4_0>::WBYTES;
template <> constexpr int kWB<GQ_Q5_0> = WS32<GQ_Q5_0>::WBYTES;
template <> constexpr int kWB<GQ_Q8_0> = WS32<GQ_Q8_0>::WBYTES;

// Bytes 2..5 of the dword pair (lo, hi).
__device__ __forceinline__ uint32_t sh16(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_alignbit(hi, lo, 16);
}

// Lane (row r, group g) writes blocks 2g, 2g+1 of its row into the LDS
// staging block ww; a block past the row's end gets scale 0 (its codes are
// whatever bytes followed, finite, and add nothing).
template <int T>
__device__ __forceinline__ void stage_w(uint8_t* ww, const WS32<T>& ws, int r, int g, bool ok_a,
                                        bool ok_b) {
  using W = WS32<T>;
  uint8_t* const c = ww + r * 8 * W::CB + 2 * g * W::CB;
  uint32_t dd = 0;
#pragma unroll
  for (int b = 0; b < 2; b++) {
    const uint32_t* D = ws.raw[b];            // bytes 0.. of the block, tail at D[NDW]
    uint8_t* const cb = c + b * W::CB;
    if constexpr (T == GQ_Q8_0) {            // d | 32 codes
      *reinterpret_cast<u32x4*>(cb) = u32x4{sh16(D[0], D[1]), sh16(D[1], D[2]), sh16(D[2], D[3]), sh16(D[3], D[4])};
      *reinterpret_cast<u32x4*>(cb + 16) = u32x4{sh16(D[4], D[5]), sh16(D[5], D[6]), sh16(D[6], D[7]), sh16(D[7], D[8])};
    } else if constexpr (T == GQ_Q4_0) {     // d | 16 code bytes
      *reinterpret_cast<u32x4*>(cb) = u32x4{sh16(D[0], D[1]), sh16(D[1], D[2]), sh16(D[2], D[3]), sh16(D[3], D[4])};
    } else {                                 // d | 4 high-bit bytes | 16 code bytes
      *reinterpret_cast<u32x4*>(cb) = u32x4{sh16(D[1], D[2]), sh16(D[2], D[3]), sh16(D[3], D[4]), sh16(D[4], D[5])};
      *reinterpret_cast<uint32_t*>(ww + W::WQ + r * 32 + 8 * g + 4 * b) = sh16(D[0], D[1]);
    }
    if (b ? ok_b : ok_a) dd |= (D[0] & 0xFFFFu) << (16 * b);
  }
  *reinterpret_cast<uint32_t*>(ww + W::WD + r * 16 + 4 * g) = dd;
}

// Q4_1: blocks are 20 dword-aligned bytes (d | m, then 16 code bytes), each
// loaded as 16 + 4 bytes and staged as codes [16][8][16], d [16][8] fp16 and
// m [16][8] fp16.
struct WSQ41 {
  static constexpr int CB = 16, WD = 16 * 8 * 16, WQ = WD + 256, WBYTES = WQ + 256;
  uint32_t raw[2][5];
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo) {
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const u32x4 v = bld16(r, vo + 20 * b, 0);
      raw[b][0] = v.x; raw[b][1] = v.y; raw[b][2] = v.z; raw[b][3] = v.w;
      raw[b][4] = bld4(r, vo + 20 * b, 16);
    }
  }
};
template <> constexpr int kWB<GQ_Q4_1> = WSQ41::WBYTES;
template <> struct WS<GQ_Q4_1> : WSQ41 {};

__device__ __forceinline__ void stage_w_q41(uint8_t* ww, const WSQ41& ws, int r, int g, bool ok_a,
                                            bool ok_b) {
  uint8_t* const c = ww + r * 8 * 16 + 2 * g * 16;
  uint32_t dd = 0, mm = 0;
#pragma unroll
  for (int b = 0; b < 2; b++) {
    const uint32_t* D = ws.raw[b];
    *reinterpret_cast<u32x4*>(c + 16 * b) = u32x4{D[1], D[2], D[3], D[4]};
    if (b ? ok_b : ok_a) {                    // blocks past the row's end: d = m = 0
      dd |= (D[0] & 0xFFFFu) << (16 * b);
      mm |= (D[0] >> 16) << (16 * b);
    }
  }
  *reinterpret_cast<uint32_t*>(ww + WSQ41::WD + r * 16 + 4 * g) = dd;
  *reinterpret_cast<uint32_t*>(ww + WSQ41::WQ + r * 16 + 4 * g) = mm;
}

template <> struct WS<GQ_Q4_0> : WS32<GQ_Q4_0> {};
template <> struct WS<GQ_Q5_0> : WS32<GQ_Q5_0> {};
template <> struct WS<GQ_Q8_0> : WS32<GQ_Q8_0> {};


// 16-token matrix-op tiles per pass: one for P = 8 or 16, two for P = 32
// (each decoded B fragment then feeds both tiles).
template <int P> constexpr int kMT = P > 16 ? P / 16 : 1;

// P[mt] += A(tile mt, chunk k) x B, with fp32 activations as hi + lo.
template <bool XLO, int P>
__device__ __forceinline__ void mma(const uint8_t* xw, int t, int k, f16x8 B, f32x4v (&Pc)[kMT<P>]) {
#pragma unroll
  for (int mt = 0; mt < kMT<P>; mt++) {
    Pc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(read_a<P>(xw, t + 16 * mt, k), B, Pc[mt], 0, 0, 0);
    if constexpr (XLO)
      Pc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(read_a<P>(xw + P * 512, t + 16 * mt, k), B,
                                                      Pc[mt], 0, 0, 0);
  }
}

// acc[mt] += the slab's contribution for this wave's 16 rows x tokens
// 16 mt .. 16 mt + 15 of the pass.
// Activation chunk of MFMA step j for lane group g: K-quant lanes own columns
// 64 g .. 64 g + 63 (their two sub-blocks), 32-weight types 32 j + 8 g.
template <int T, bool XLO, int P>
__device__ __forceinline__ void slab_mma(const uint8_t* xw, const uint8_t* ww, const float* sv, int t,
                                         const WS<T>& ws, int g, f32x4v (&acc)[kMT<P>]) {
  constexpr int MT = kMT<P>;
  const f32x4v z = {0.f, 0.f, 0.f, 0.f};
  const f32x4 iv = inv_scales<XLO, P>(sv, g);   // fp32 x: undo the slab's scale
  if constexpr (T == GQ_Q4_K || T == GQ_Q5_K) {
    const float d = h2f(ws.hd.x), dmin = h2f(ws.hd.x >> 16);
    f16x8 M[2];
    f16x2 SL[2], NL[2], SH[2], NH[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint32_t f = q4k_pair(ws.hd.y, ws.hd.z, ws.hd.w, 2 * g + h);
      const float sc = (float)(f & 63u), m = (float)(f >> 6);
      SL[h] = hpair(sc, sc);                  // low nibble q: (1024 + q) * sc - 1024 sc
      NL[h] = hpair(-1024.f * sc, -1024.f * sc);
      SH[h] = hpair(sc * 0.0625f, sc * 0.0625f);   // high nibble: (1024 + 16 q) * sc/16 - 64 sc
      NH[h] = hpair(-64.f * sc, -64.f * sc);
      const _Float16 mh = (_Float16)m;
      M[h] = f16x8{mh, mh, mh, mh, mh, mh, mh, mh};
    }
    f32x4v Pk[MT], Pm[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) Pk[mt] = Pm[mt] = z;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int h = j >> 2, qq = j & 3;       // sub-block 2g + h, eighth qq
      const uint32_t D0 = ws.q[h][2 * (qq & 1)], D1 = ws.q[h][2 * (qq & 1) + 1];
      f16x2 v[4];
      f16x2 s, n;
      if constexpr (T == GQ_Q5_K) {           // elements 8qq .. 8qq+7: codes as bytes
        const int sh = (qq < 2) ? 0 : 4;
        const uint32_t W = ws.qh[h] >> (8 * qq);
        bytes8(kE1024, ((D0 >> sh) & 0x0F0F0F0Fu) | bits_to_b4(W),
               ((D1 >> sh) & 0x0F0F0F0Fu) | bits_to_b4(W >> 4), v);
        s = SL[h];
        n = NL[h];
      } else {
        const uint32_t msk = (qq < 2) ? 0x0F0F0F0Fu : 0xF0F0F0F0u;
        bytes8(kE1024, D0 & msk, D1 & msk, v);
        s = (qq < 2) ? SL[h] : SH[h];
        n = (qq < 2) ? NL[h] : NH[h];
      }
      const f16x8 B = cat8(__builtin_elementwise_fma(v[0], s, n), __builtin_elementwise_fma(v[1], s, n),
                           __builtin_elementwise_fma(v[2], s, n), __builtin_elementwise_fma(v[3], s, n));
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const f16x8 ah = read_a<P>(xw, t + 16 * mt, 8 * g + j);
        Pk[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, B, Pk[mt], 0, 0, 0);
        Pm[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, M[h], Pm[mt], 0, 0, 0);
        if constexpr (XLO) {
          const f16x8 al = read_a<P>(xw + P * 512, t + 16 * mt, 8 * g + j);
          Pk[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, B, Pk[mt], 0, 0, 0);
          Pm[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, M[h], Pm[mt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      if constexpr (XLO) {
        acc[mt] += (d * iv) * Pk[mt];
        acc[mt] -= (dmin * iv) * Pm[mt];
      } else {
        acc[mt] += d * Pk[mt];
        acc[mt] -= dmin * Pm[mt];
      }
    }
  } else if constexpr (T == GQ_Q2_K) {
    // step j: columns 64g + 8j .. +7 = elements 8u .. 8u+7 (u = j % 4) of
    // group 2g + j / 4, bits 2u..2u+1 of its 8 plane bytes; 16-weight
    // sub-block 4g + 2 (j / 4) + u / 2.  B = sc * q (exact), the min term as
    // a second product with m, both scaled by d and dmin in fp32.
    const float d = h2f(ws.dm), dmin = h2f(ws.dm >> 16);
    f32x4v Pk[MT], Pm[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) Pk[mt] = Pm[mt] = z;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int gg = j >> 2, u = j & 3;
      const uint32_t b = ws.sm >> (8 * (2 * gg + (u >> 1)));
      const float sc = (float)(b & 15u), m = (float)((b >> 4) & 15u);
      f16x2 v[4];
      bytes8(kE1024, plane2(ws.q[2 * gg], u), plane2(ws.q[2 * gg + 1], u), v);   // 1024 + q
      const f16x2 s2 = hpair(sc, sc), n2 = hpair(-1024.f * sc, -1024.f * sc);
      const f16x8 B = cat8(__builtin_elementwise_fma(v[0], s2, n2), __builtin_elementwise_fma(v[1], s2, n2),
                           __builtin_elementwise_fma(v[2], s2, n2), __builtin_elementwise_fma(v[3], s2, n2));
      const _Float16 mh = (_Float16)m;
      const f16x8 M = f16x8{mh, mh, mh, mh, mh, mh, mh, mh};
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const f16x8 ah = read_a<P>(xw, t + 16 * mt, 8 * g + j);
        Pk[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, B, Pk[mt], 0, 0, 0);
        Pm[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, M, Pm[mt], 0, 0, 0);
        if constexpr (XLO) {
          const f16x8 al = read_a<P>(xw + P * 512, t + 16 * mt, 8 * g + j);
          Pk[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, B, Pk[mt], 0, 0, 0);
          Pm[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, M, Pm[mt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      if constexpr (XLO) {
        acc[mt] += (d * iv) * Pk[mt];
        acc[mt] -= (dmin * iv) * Pm[mt];
      } else {
        acc[mt] += d * Pk[mt];
        acc[mt] -= dmin * Pm[mt];
      }
    }
  } else if constexpr (T == GQ_Q3_K) {
    // step j as Q2_K; code q = low bits | third bit << 2, B = sc * (q - 4)
    // exactly (|B| <= 252): (1024 + q) - 1028 is exact in fp16, then the
    // product with sc
    const float d = h2f(ws.d);
    f32x4v Pk[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) Pk[mt] = z;
    const f16x2 n4 = hpair(-1028.f, -1028.f);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int gg = j >> 2, u = j & 3;
      const uint32_t hb = (gg ? ws.qh.y : ws.qh.x) >> (8 * u);   // third bits of the 8 elements
      const uint32_t c0 = plane2(ws.q[2 * gg], u) | bits_to_b2(hb);
      const uint32_t c1 = plane2(ws.q[2 * gg + 1], u) | bits_to_b2(hb >> 4);
      const float sc = (float)((ws.sc >> (6 * (2 * gg + (u >> 1)))) & 63u);
      f16x2 v[4];
      bytes8(kE1024, c0, c1, v);
      const f16x2 s2 = hpair(sc, sc);
      const f16x8 B = cat8((v[0] + n4) * s2, (v[1] + n4) * s2, (v[2] + n4) * s2, (v[3] + n4) * s2);
      mma<XLO, P>(xw, t, 8 * g + j, B, Pk);
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      if constexpr (XLO) acc[mt] += (d * iv) * Pk[mt];
      else acc[mt] += d * Pk[mt];
    }
  } else if constexpr (T == GQ_Q6_K) {
    const float d = h2f(ws.d);
    f32x4v Pk[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) Pk[mt] = z;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int h = j >> 2, qq = j & 3;       // 32-group 2g + h, eighth qq
      const uint32_t L0 = ws.l[h][2 * (qq & 1)], L1 = ws.l[h][2 * (qq & 1) + 1];
      const uint32_t H0 = ws.h[2 * h], H1 = ws.h[2 * h + 1];
      // 4 * q per byte: low 4 bits from the ql nibble, top 2 from qh bits 2qq..2qq+1
      const uint32_t c0 = ((qq < 2 ? L0 << 2 : L0 >> 2) & 0x3C3C3C3Cu) | ((H0 << (6 - 2 * qq)) & 0xC0C0C0C0u);
      const uint32_t c1 = ((qq < 2 ? L1 << 2 : L1 >> 2) & 0x3C3C3C3Cu) | ((H1 << (6 - 2 * qq)) & 0xC0C0C0C0u);
      f16x2 v[4];
      bytes8(kE256, c0, c1, v);               // 256 + q
      const float sc = (float)(int)(int8_t)(ws.sc4 >> (8 * (2 * h + (qq >> 1))));
      const f16x2 s = hpair(sc, sc), n = hpair(-288.f * sc, -288.f * sc);
      const f16x8 B = cat8(__builtin_elementwise_fma(v[0], s, n), __builtin_elementwise_fma(v[1], s, n),
                           __builtin_elementwise_fma(v[2], s, n), __builtin_elementwise_fma(v[3], s, n));
      mma<XLO, P>(xw, t, 8 * g + j, B, Pk);
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      if constexpr (XLO) acc[mt] += (d * iv) * Pk[mt];
      else acc[mt] += d * Pk[mt];
    }
  } else if constexpr (T == GQ_Q4_1) {
    // B = RNE_fp16(w 2^k) per block, w = d q + m formed exactly by the mixed
    // FMA (k puts the block's bound 15 |d| + |m| in [2^13, 2^14)); the
    // block's products take 2^-k
    const u32x4 dq = *reinterpret_cast<const u32x4*>(ww + WSQ41::WD + t * 16);   // 8 fp16 d
    const u32x4 mq = *reinterpret_cast<const u32x4*>(ww + WSQ41::WQ + t * 16);   // 8 fp16 m
    const int co = t * 8 * 16 + 8 * (g & 1), sh = 4 * (g >> 1);
    f32x4v as[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) as[mt] = z;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const u32x2 cc = *reinterpret_cast<const u32x2*>(ww + co + j * 16);
      const uint32_t c0 = (cc.x >> sh) & 0x0F0F0F0Fu, c1 = (cc.y >> sh) & 0x0F0F0F0Fu;
      const float d = h2f(dq[j >> 1] >> (16 * (j & 1))), m = h2f(mq[j >> 1] >> (16 * (j & 1)));
      const int k = pow2_exp_for<14>(fmaf(15.f, fabsf(d), fabsf(m)));
      const float s24 = __builtin_ldexpf(d, k + 24), nb = __builtin_ldexpf(m, k);
      const uint32_t e0 = c0 & 0x00FF00FFu, o0 = (c0 >> 8) & 0x00FF00FFu;
      const uint32_t e1 = c1 & 0x00FF00FFu, o1 = (c1 >> 8) & 0x00FF00FFu;
      const f16x8 B = __builtin_bit_cast(
          f16x8, u32x4{mixpair<0>(e0, o0, s24, nb), mixpair<1>(e0, o0, s24, nb),
                       mixpair<0>(e1, o1, s24, nb), mixpair<1>(e1, o1, s24, nb)});
      f32x4v Pk[MT];
#pragma unroll
      for (int mt = 0; mt < MT; mt++) Pk[mt] = z;
      mma<XLO, P>(xw, t, 4 * j + g, B, Pk);
      const float inv = __builtin_ldexpf(1.f, -k);
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        if constexpr (XLO) as[mt] += inv * Pk[mt];
        else acc[mt] += inv * Pk[mt];
      }
    }
    if constexpr (XLO) {
#pragma unroll
      for (int mt = 0; mt < MT; mt++) acc[mt] += iv * as[mt];
    }
  } else {
    using W = WS32<T>;
    const f16x2 off = (T == GQ_Q8_0) ? hpair(-1152.f, -1152.f)
                      : (T == GQ_Q5_0) ? hpair(-1040.f, -1040.f) : hpair(-1032.f, -1032.f);
    // t is the lane's row in the tile (A fragments use it as the token row)
    const u32x4 dq = *reinterpret_cast<const u32x4*>(ww + W::WD + t * 16);   // 8 fp16 scales
    u32x4 qh4[2] = {};
    if constexpr (T == GQ_Q5_0) {
      qh4[0] = *reinterpret_cast<const u32x4*>(ww + W::WQ + t * 32);
      qh4[1] = *reinterpret_cast<const u32x4*>(ww + W::WQ + t * 32 + 16);
    }
    const int co = t * 8 * W::CB + ((T == GQ_Q8_0) ? 8 * g : 8 * (g & 1));
    f32x4v as[MT];                            // fp32 x: the slab's sum before 1/s
#pragma unroll
    for (int mt = 0; mt < MT; mt++) as[mt] = z;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const u32x2 cc = *reinterpret_cast<const u32x2*>(ww + co + j * W::CB);
      uint32_t c0 = cc.x, c1 = cc.y;
      if constexpr (T == GQ_Q8_0) {
        c0 ^= 0x80808080u;                    // signed byte + 128
        c1 ^= 0x80808080u;
      } else {
        const int sh = 4 * (g >> 1);          // low nibbles for g < 2, high for g >= 2
        c0 = (c0 >> sh) & 0x0F0F0F0Fu;
        c1 = (c1 >> sh) & 0x0F0F0F0Fu;
        if constexpr (T == GQ_Q5_0) {
          const uint32_t hb = qh4[j >> 2][j & 3] >> (8 * g);   // fifth bits of elements 8g .. 8g+7
          c0 |= bits_to_b4(hb);
          c1 |= bits_to_b4(hb >> 4);
        }
      }
      f16x2 v[4];
      bytes8(kE1024, c0, c1, v);
      const f16x8 B = cat8(v[0] + off, v[1] + off, v[2] + off, v[3] + off);
      f32x4v Pk[MT];
#pragma unroll
      for (int mt = 0; mt < MT; mt++) Pk[mt] = z;
      mma<XLO, P>(xw, t, 4 * j + g, B, Pk);
      const float dj = h2f(dq[j >> 1] >> (16 * (j & 1)));
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        if constexpr (XLO) as[mt] += dj * Pk[mt];
        else acc[mt] += dj * Pk[mt];
      }
    }
    if constexpr (XLO) {
#pragma unroll
      for (int mt = 0; mt < MT; mt++) acc[mt] += iv * as[mt];
    }
  }
}

}  // namespace

// grid: tiles * passes workgroups of 64 * KS threads (a tile is RT 16-row
// tiles, one B fragment each, sharing the wave's activation slab), P tokens per pass,
// KS * P * 512 bytes of LDS (twice that for fp32 activations; the 32-weight
// types add their weight staging block per wave).  With several
// token passes the workgroup index is remapped so that the passes of one row
// tile run back to back on one XCD (workgroups go round-robin over the 8
// XCDs), where the tile's weights are still in that XCD's L2.
template <int T, bool XLO, int P, int D, int RT>
__global__ void __launch_bounds__(512) k_mmv(const uint8_t* __restrict__ blob, int rows, int cols,
                                             int rb, const void* __restrict__ xv, int n,
                                             float* __restrict__ y, int tiles, int passes) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr bool KQ = (T == GQ_Q4_K || T == GQ_Q6_K || T == GQ_Q5_K || T == GQ_Q2_K ||
                       T == GQ_Q3_K);
  constexpr int ES = XLO ? 4 : 2;
  constexpr int XB = P * 512 * (XLO ? 2 : 1);   // LDS bytes per wave: activations,
  constexpr int WB = kWB<T>;                    // then staged weights (32-weight types)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int KS = blockDim.x >> 6;
  int tile = blockIdx.x, pass = 0;
  if (passes > 1) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    tile = (slot / passes) * 8 + xcd;
    pass = slot % passes;
    if (tile >= tiles) return;                // whole workgroup: uniform
  }
  const int row0 = tile * 16 * RT, tok0 = pass * P;
  const int r = lane & 15, g = lane >> 4;
  const int nr = min(16 * RT, rows - row0), nt = min(P, n - tok0);
  const __amdgpu_buffer_rsrc_t WR = make_rsrc(blob + (int64_t)row0 * rb, (uint32_t)(nr * rb));
  const __amdgpu_buffer_rsrc_t XR =
      make_rsrc((const uint8_t*)xv + (int64_t)tok0 * cols * ES, (uint32_t)(nt * cols * ES));
  const int nslab = (cols + 255) >> 8;
  const int nblk = cols >> 5;
  const int wl = r * rb;                      // lane's row within its 16-row tile
  constexpr int SB = kSB<XLO>;                 // then fp32 x's per-token scales
  uint8_t* const xw = lds + w * (XB + WB + SB);   // this wave's activation block,
  uint8_t* const ww = xw + XB;                // weight staging block
  float* const sv = reinterpret_cast<float*>(ww + WB);   // and scales

  auto load = [&](XS<XLO, P>& xs, WS<T> (&ws)[RT], int s) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++) {
      const int wr = wl + 16 * rt * rb;
      if constexpr (KQ) {
        ws[rt].load(WR, s < nslab ? wr + s * Geo<T>::BB : kOobOff, g);
      } else {                                // blocks 8s + 2g, 8s + 2g + 1
        ws[rt].load(WR, wr + (8 * s + 2 * g) * Geo<T>::BB);
      }
    }
    // activations: whole lines; columns past the row (or past the last
    // block) and tokens past the pass read as zero
    const int c = s * 256 + (XLO ? 4 * lane : 8 * (lane & 31));
    const bool ok = KQ ? (s < nslab) : ((c >> 5) < nblk);
#pragma unroll
    for (int i = 0; i < (XLO ? P : P / 2); i++) {
      const int tok = XLO ? i : 2 * i + (lane >> 5);
      xs.v[i] = bld16(XR, ok ? (tok * cols + c) * ES : kOobOff, 0);
    }
  };

  const int cnt = (nslab - 1 - w) / KS + 1;   // this wave's slabs (w < KS <= nslab)
  constexpr int MT = kMT<P>;
  f32x4v acc[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[rt][mt] = f32x4v{0.f, 0.f, 0.f, 0.f};
  XS<XLO, P> xs[D];
  WS<T> ws[D][RT];
#pragma unroll
  for (int i = 0; i < D; i++) {
    load(xs[i], ws[i], w + i * KS);           // issued in ring order (see below)
    __builtin_amdgcn_sched_barrier(0);
  }
  // Every wave has at least one slab (KS <= slabs per row), so the loop is a
  // do-while: with a guarded loop the compiler sinks the first loads into
  // the guard in another order, and the waits in the loop follow the
  // stricter of the two orders.
  int m0 = 0;
  do {
#pragma unroll
    for (int i = 0; i < D; i++) {
      // The barriers keep the scheduler from sinking the reloads to the end
      // of the unrolled body, which would make every step wait on them all.
      // LDS operations of one wave run in order, so the block can be
      // rewritten while the previous slab's reads are still queued.
      stage_x<XLO, P>(xw, sv, xs[i], lane);
      if constexpr (!KQ) {                    // RT is 1 for these types
        const int b = 8 * (w + (m0 + i) * KS) + 2 * g;
        if constexpr (T == GQ_Q4_1) stage_w_q41(ww, ws[i][0], r, g, b < nblk, b + 1 < nblk);
        else stage_w<T>(ww, ws[i][0], r, g, b < nblk, b + 1 < nblk);
      }
#pragma unroll
      for (int rt = 0; rt < RT; rt++)         // slabs past cnt read as zeros
        slab_mma<T, XLO, P>(xw, ww, sv, r, ws[i][rt], g, acc[rt]);
      __builtin_amdgcn_sched_barrier(0);
      load(xs[i], ws[i], w + (m0 + i + D) * KS);
      __builtin_amdgcn_sched_barrier(0);
    }
    m0 += D;
  } while (m0 < cnt);

  // D lane l of tile mt holds rows (tokens) 16 mt + 4(l/16) + v of column
  // (weight row) l % 16 of its 16-row tile
  if (KS == 1) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          const int t = 16 * mt + 4 * g + v, rr = 16 * rt + r;
          if (t < nt && rr < nr) y[(int64_t)(tok0 + t) * rows + row0 + rr] = acc[rt][mt][v];
        }
    return;
  }
  __syncthreads();                            // every wave is done with its block
  f32x4v* red = reinterpret_cast<f32x4v*>(lds);   // [KS][RT][MT][64]
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int mt = 0; mt < MT; mt++) red[((w * RT + rt) * MT + mt) * 64 + lane] = acc[rt][mt];
  __syncthreads();
  for (int o = threadIdx.x; o < 256 * MT * RT; o += blockDim.x) {
    const int rt = o / (256 * MT), mt = (o >> 8) % MT, t = (o >> 4) & 15, rr = o & 15;
    const int src = 16 * (t >> 2) + rr, v = t & 3;
    float sum = 0.f;
    for (int k = 0; k < KS; k++) sum += red[((k * RT + rt) * MT + mt) * 64 + src][v];
    if (16 * mt + t < nt && 16 * rt + rr < nr)
      y[(int64_t)(tok0 + 16 * mt + t) * rows + row0 + 16 * rt + rr] = sum;
  }
}

namespace {

template <int T, bool XLO, int P, int D, int RT>
hipError_t mmv_launch(const void* blob, int64_t rows, int64_t cols, const void* x, int64_t n,
                      float* y, int ks, hipStream_t st) {
  const int64_t rb = cols / Geo<T>::QK * Geo<T>::BB;
  const int64_t es = XLO ? 4 : 2;
  // every resource and offset must stay below the out-of-range marker
  if (16 * RT * rb >= kOobOff || (int64_t)P * cols * es >= kOobOff) return hipErrorInvalidValue;
  const int64_t tiles = (rows + 16 * RT - 1) / (16 * RT), passes = (n + P - 1) / P;
  const int64_t grid = passes == 1 ? tiles : (tiles + 7) / 8 * 8 * passes;
  const size_t lds = (size_t)ks * (P * 512 * (XLO ? 2 : 1) + kWB<T> + kSB<XLO>);
  hipLaunchKernelGGL((k_mmv<T, XLO, P, D, RT>), dim3((unsigned)grid), dim3(64 * ks), lds, st,
                     (const uint8_t*)blob, (int)rows, (int)cols, (int)rb, x, (int)n, y, (int)tiles,
                     (int)passes);
  return hipGetLastError();
}

#ifndef GQ_MMV_WAVES
#define GQ_MMV_WAVES 4096                     // target waves per launch
#endif
#ifndef GQ_MMV_WAVES8
#define GQ_MMV_WAVES8 2048                    // the same for 8-token passes of fp16 x
#endif
#ifndef GQ_MMV_WAVES32
#define GQ_MMV_WAVES32 2048                   // the same for 32-token passes
#endif
#ifndef GQ_MMV_DEPTH32                        // ring depth of the 32-token passes
#define GQ_MMV_DEPTH32 1
#endif
#ifndef GQ_MMV_P32_FROM                      // fp16 x: passes of 32 tokens above this many
#define GQ_MMV_P32_FROM 16
#endif
#ifndef GQ_MMV_DEPTH
#define GQ_MMV_DEPTH 2                        // ring depth with fp16 activations
#endif
#ifndef GQ_MMV_RT2_TILES                     // 16-row tiles from which a wave takes two
#define GQ_MMV_RT2_TILES 2000
#endif

// KS: enough waves to cover the chip waves / 256 deep (waves: the launch's
// target), at most kmax per workgroup (and as many as the LDS budget holds),
// and no more than the row has slabs.
int pick_ks(int64_t rows, int64_t cols, int64_t n, int p, int lds_per_wave, int rt, int waves,
            int kmax = 8) {
  const int64_t tiles = (rows + 16 * rt - 1) / (16 * rt), passes = (n + p - 1) / p;
  const int64_t nslab = (cols + 255) / 256;
  int ks = 1;
  // 32-token passes over few tiles (the 32-weight types' staged weights on
  // top of 16 KB of activations per wave) may take 96 KB, so 4 waves still
  // split a long row (Q8_0 4096 x 11008 at 32 tokens: 39.6 -> 28.8 us)
  const int budget = (p == 32 && tiles * passes <= 256) ? 98304 : 65536;
  while (ks < kmax && (ks * 2) * lds_per_wave <= budget && tiles * passes * ks * 2 <= waves &&
         ks * 2 <= nslab)
    ks *= 2;
  return ks;
}

template <int T, bool XLO, int P>
hipError_t mmv_p(const void* blob, int64_t rows, int64_t cols, const void* x, int64_t n, float* y,
                 hipStream_t st) {
  // ring depth: as deep as the registers allow without spilling
  constexpr int D = XLO ? (P == 8 ? 2 : 1) : (P == 32) ? GQ_MMV_DEPTH32
                   : (T == GQ_Q5_0 && P == 16) ? 2 : GQ_MMV_DEPTH;
  constexpr int XB = P * 512 * (XLO ? 2 : 1) + kWB<T> + kSB<XLO>;
  // 8-token passes of fp16 x: half the waves, each splitting its row's slabs
  // over fewer waves, so a workgroup reads the activation block once for
  // twice the work (measured on MI355X: Q4_K 11008x4096 at 8 tokens 12.2 ->
  // 11.6 us, 14336x4096 14.7 -> 13.6 us, 22016x4096 20.5 -> 19.3 us; Q6_K
  // and fp32 x gain nothing or lose)
  // 32-token passes likewise (Q4_K 22016x4096 at 32 tokens 30.5 -> 28.3 us,
  // 11008x4096 at 48 27.5 -> 26.2 us; the other shapes measured are capped
  // by the LDS budget first and do not change)
  constexpr int WAVES = (P == 8 && !XLO) ? GQ_MMV_WAVES8 : (P == 32) ? GQ_MMV_WAVES32 : GQ_MMV_WAVES;
  // Two 16-row tiles per wave share each activation slab, halving the
  // activation reads, which outweigh the weights' on tall matrices and in
  // 32-token passes; they pay once the halved tile count still gives 256
  // workgroups (measured on MI355X: Q6_K 128256 x 4096 at 24 / 32 tokens
  // 201 / 216 -> 164 / 171 us; 32-token passes of Q4_K 11008 x 4096 at 24 /
  // 32 / 64 tokens 21.5 / 22.4 / 35.0 -> 18.6 / 20.3 / 27.9 us, Q6_K
  // 4096 x 11008 at 64 tokens 42.5 -> 38.8 us; with fewer workgroups, 4096
  // rows at 32 tokens, 10.8 -> 14.4 us)
  // 16-token passes of fp16 x: at most 4 waves per tile (with 8 each wave
  // has two slabs, and 8192 x 4096 at 16 tokens took 14.2 us against 11.7 with
  // 4), and two tiles per wave from 448 tile pairs (14336 x 4096: 19.2 -> 16.1
  // us, 22016 x 4096: 24.1 -> 22.3 us; 11008 x 4096, 344 pairs, 15.2 -> 15.8).
  // fp32 x, whose 16-token slab fills the registers (a 1-deep ring): two
  // tiles per wave from 600 tile pairs x passes (11008 x 4096 at 32 / 64
  // tokens 56.5 / 99.4 -> 37.9 / 70.4 us, 22016 x 4096 at 16 57.4 -> 38.7,
  // 14336 x 4096 at 32 66.1 -> 40.4; at 448 or 512, 14336 x 4096 at 16 and
  // 8192 x 4096 at 32, they lose 12 %)
  constexpr int KMAX = (P == 16 && !XLO) ? 4 : 8;
  if constexpr (T == GQ_Q4_K || T == GQ_Q6_K || T == GQ_Q5_K || T == GQ_Q2_K || T == GQ_Q3_K) {
    const int64_t tiles = (rows + 15) / 16, passes = (n + P - 1) / P;
    if (tiles >= GQ_MMV_RT2_TILES || (P == 32 && tiles / 2 * passes >= 256) ||
        (P == 16 && tiles / 2 * passes >= (XLO ? 600 : 448)))
      return mmv_launch<T, XLO, P, D, 2>(blob, rows, cols, x, n, y,
                                         pick_ks(rows, cols, n, P, XB, 2, WAVES, KMAX), st);
  }
  return mmv_launch<T, XLO, P, D, 1>(blob, rows, cols, x, n, y,
                                     pick_ks(rows, cols, n, P, XB, 1, WAVES, KMAX), st);
}

template <int T, bool XLO>
hipError_t mmv_t(const void* blob, int64_t rows, int64_t cols, const void* x, int64_t n, float* y,
                 hipStream_t st) {
  if (n <= 8) return mmv_p<T, XLO, 8>(blob, rows, cols, x, n, y, st);
  // 32-token passes (fp16 x) halve the decode work per token, which is what
  // bounds the 32-weight types and Q6_K; they need at least 256 workgroups
  // (16-row tiles x passes) to cover the chip.  Q4_K's decode is cheap, and
  // past 512 row tiles its 32-token passes pay only because they then take
  // two row tiles per wave (mmv_p).
  const int64_t tiles = (rows + 15) / 16, passes32 = (n + 31) / 32;
  const bool p32 = !XLO && n > GQ_MMV_P32_FROM && tiles * passes32 >= 256;
  if (!p32) return mmv_p<T, XLO, 16>(blob, rows, cols, x, n, y, st);
  return mmv_p<T, false, 32>(blob, rows, cols, x, n, y, st);
}

}  // namespace

hipError_t launch_mmv(int type, const void* blob, int64_t rows, int64_t cols, const void* x,
                      bool x_f16, float* y, int64_t n_tok, hipStream_t st) {
  switch (type) {
#define GQ_MMV_CASE(TT)                                                                   \
  case TT:                                                                                \
    return x_f16 ? mmv_t<TT, false>(blob, rows, cols, x, n_tok, y, st)                    \
                 : mmv_t<TT, true>(blob, rows, cols, x, n_tok, y, st);
    GQ_MMV_CASE(GQ_Q4_0)
    GQ_MMV_CASE(GQ_Q5_0)
    GQ_MMV_CASE(GQ_Q8_0)
    GQ_MMV_CASE(GQ_Q4_K)
    GQ_MMV_CASE(GQ_Q6_K)
    GQ_MMV_CASE(GQ_Q4_1)
    GQ_MMV_CASE(GQ_Q5_K)
    GQ_MMV_CASE(GQ_Q2_K)
    GQ_MMV_CASE(GQ_Q3_K)
#undef GQ_MMV_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace gq
