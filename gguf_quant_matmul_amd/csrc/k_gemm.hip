// k_gemm.hip — prefill-sized matmul (n_tok > 64) over GGUF blocks on the
// gfx950 matrix cores.  Prefill is the compute-bound side of inference
// ("12 — llama.cpp / GGUF", "Prefill on CPU"), so this is a tiled fp16 GEMM
// whose B operand is decoded from the blocks on the fly, once per 128-token
// tile ("Local LLM inference", "The mmap backend": decode once per batch,
// reuse across its rows):
//
//   * B = RNE_fp16(w 2^kr) of the stated fp32 dequant w (Hitchhiker's Guide
//     §11.2, w = (d*sc)*q - dmin*m): every weight is decoded with one fp32
//     fma on scales pre-multiplied by the row's power of two 2^kr and
//     rounded to fp16 by v_fma_mix (relative error <= 2^-11 per weight,
//     inside the stated 1e-3 of sum |w*x|), and y takes 2^-kr; kr follows
//     the largest block bound of the row seen so far (every finite fp16
//     scale then fits), the accumulators rescaled when it falls; Q4_K codes
//     reach the mix as fp16 subnormals, so they need no convert;
//   * workgroup tile 128 tokens x 256 weight rows (128 x 128 or 64 x 128
//     when that leaves fewer CUs idle), K steps of 64 columns; 32 weight
//     rows x all the tile's tokens per wave (BM/32 x 1
//     v_mfma_f32_32x32x16_f16 per 16 columns);
//   * each wave decodes its own B fragments straight into registers (no
//     redundancy, and no LDS writes for B: LDS stores run at about a third
//     of the LDS read rate here); step i + 1 is decoded while the matrix
//     cores run step i;
//   * activations are staged in LDS, double-buffered, 16-byte chunks XOR-
//     swizzled per row so fragment reads and tile writes are conflict-free;
//   * the raw weight bytes and activations of the next D K-steps are in
//     flight in a register ring (loads complete in issue order, so both
//     streams get the same distance);
//   * fp32 activations are scaled per token by a power of two 2^kx that
//     follows the running max of |x| (accumulators rescaled when it falls),
//     split into hi = RNE_fp16(x 2^kx) and lo = RNE_fp16(x 2^kx - hi), and
//     both pass through the matrix op;
//   * tiles are mapped so that the token tiles of one weight-row tile run on
//     one XCD (workgroups go round-robin over the 8 XCDs) and share its L2.
#include <type_traits>
#ifdef GQ_TUNE_ENV
#include <cstdlib>
#endif

#include "gq_device.h"
#include "gq_launch.h"

namespace gq {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int KNONE = 1 << 20;               // no nonzero block / activation seen yet
constexpr int ROWB = BK * 2;                 // bytes of one tile row (64 fp16)

// 16-byte chunk c (0..7) of tile row t lives at t * 128 + 16 * (c ^ swz(t)).
// Any 16 consecutive rows then use 16 distinct chunk slots of a 256-byte
// bank window (and any 8 rows 8 distinct slots of a 128-byte window).
__device__ __forceinline__ int swz(int t) { return ((t >> 1) & 7) ^ ((t & 1) << 2); }
__device__ __forceinline__ int tslot(int t, int c) { return t * 128 + ((c ^ swz(t)) << 4); }

// A copy the compiler cannot fold into its source.  Taking a ring slot's
// header this way frees the slot's register for the slot's next load; a
// folded copy keeps the old value in the slot's register until the loop's
// back edge, where the new load's value is then moved in, and that move
// waits for the load just issued (draining the whole ring once per
// super-block).
__device__ __forceinline__ uint32_t fresh1(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}
__device__ __forceinline__ u32x4 fresh(const u32x4& v) {
  return u32x4{fresh1(v.x), fresh1(v.y), fresh1(v.z), fresh1(v.w)};
}

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
  static constexpr bool kHeader = true;      // header shared by a super-block's 4 steps
  u32x4 hd, q;
  template <bool HDR = true>
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + (sg >> 3) * 144 : kOobOff;
    if constexpr (HDR) hd = bld16(R, vo, 0);
    q = bld16(R, vo + 16 * (sg & 7), 16);
  }
  // fields at FL * fk + FU * (step % 4) + FB of the super-block (see SbFields)
  static constexpr int NF = 2, FL[NF] = {0, 16}, FU[NF] = {0, 32}, FB[NF] = {0, 16};
  template <bool HDR = true>
  __device__ void load_at(__amdgpu_buffer_rsrc_t R, const uint32_t (&o)[NF]) {
    if constexpr (HDR) hd = bld16(R, (int)o[0], 0);
    q = bld16(R, (int)o[1], 0);
  }
  // largest |w| the block's fields allow: 945 |d| + 63 |dmin|
  __device__ static float bound(const u32x4& hd) {
    return fmaf(945.f, fabsf(h2f(hd.x)), 63.f * fabsf(h2f(hd.x >> 16)));
  }
  __device__ float bound() const { return bound(hd); }
  __device__ void decode(int sg, int k, u32x4 out[4]) const { decode(sg, hd, k, out); }
  __device__ void decode(int sg, const u32x4& hd, int k, u32x4 out[4]) const {
    const float d = __builtin_ldexpf(h2f(hd.x), k), dmin = __builtin_ldexpf(h2f(hd.x >> 16), k);
    const uint32_t f = q4k_pair(hd.y, hd.z, hd.w, sg & 7);
    const float a = d * (float)(f & 63u), nb = -(dmin * (float)(f >> 6));
    // codes enter as fp16 subnormals q * 2^-24 (high nibbles in place: 16 q)
    const float a24 = a * 16777216.f, a20 = a * 1048576.f;
#pragma unroll
    for (int c = 0; c < 4; c++) {            // chunk c: elements 8c .. 8c+7
      const uint32_t m = (c < 2) ? 0x000F000Fu : 0x00F000F0u;
      const float s = (c < 2) ? a24 : a20;
      const uint32_t w0 = q[2 * (c & 1)], w1 = q[2 * (c & 1) + 1];
      const uint32_t e0 = w0 & m, o0 = (w0 >> 8) & m;   // bytes 0, 2 / 1, 3 of w0
      const uint32_t e1 = w1 & m, o1 = (w1 >> 8) & m;
      out[c] = u32x4{mixpair<0>(e0, o0, s, nb), mixpair<1>(e0, o0, s, nb),
                     mixpair<0>(e1, o1, s, nb), mixpair<1>(e1, o1, s, nb)};
    }
  }
};
// Q5_K: Q4_K's header, the segment's 32 fifth bits, its 16 code bytes; the
// fifth bit of each code is spread into its 16-bit field (bit 4, or bit 8
// for high nibbles, which sit in place as 16 q) by a multiply that places
// bits 0 and 2 of a 4-bit group at both fields at once.
template <> struct BR<GQ_Q5_K> {
  static constexpr bool kHeader = true;
  u32x4 hd, q;
  uint32_t qh;
  template <bool HDR = true>
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + (sg >> 3) * 176 : kOobOff;
    if constexpr (HDR) hd = bld16(R, vo, 0);
    qh = bld4(R, vo + 4 * (sg & 7), 16);
    q = bld16(R, vo + 16 * (sg & 7), 48);
  }
  static constexpr int NF = 3, FL[NF] = {0, 4, 16}, FU[NF] = {0, 8, 32}, FB[NF] = {0, 16, 48};
  template <bool HDR = true>
  __device__ void load_at(__amdgpu_buffer_rsrc_t R, const uint32_t (&o)[NF]) {
    if constexpr (HDR) hd = bld16(R, (int)o[0], 0);
    qh = bld4(R, (int)o[1], 0);
    q = bld16(R, (int)o[2], 0);
  }
  __device__ static float bound(const u32x4& hd) {          // 63 * 31 |d| + 63 |dmin|
    return fmaf(1953.f, fabsf(h2f(hd.x)), 63.f * fabsf(h2f(hd.x >> 16)));
  }
  __device__ float bound() const { return bound(hd); }
  __device__ void decode(int sg, int k, u32x4 out[4]) const { decode(sg, hd, k, out); }
  __device__ void decode(int sg, const u32x4& hd, int k, u32x4 out[4]) const {
    const float d = __builtin_ldexpf(h2f(hd.x), k), dmin = __builtin_ldexpf(h2f(hd.x >> 16), k);
    const uint32_t f = q4k_pair(hd.y, hd.z, hd.w, sg & 7);
    const float a = d * (float)(f & 63u), nb = -(dmin * (float)(f >> 6));
    const float a24 = a * 16777216.f, a20 = a * 1048576.f;
#pragma unroll
    for (int c = 0; c < 4; c++) {            // chunk c: elements 8c .. 8c+7
      const uint32_t m = (c < 2) ? 0x000F000Fu : 0x00F000F0u;
      const float s = (c < 2) ? a24 : a20;
      // bits 0, 2 of a 4-bit group to bits 4, 20 (low nibbles) or 8, 24 (high)
      const uint32_t mul = (c < 2) ? 0x00040010u : 0x00400100u;
      const uint32_t pos = (c < 2) ? 0x00100010u : 0x01000100u;
      const uint32_t hb = qh >> (8 * c);      // fifth bits of elements 8c .. 8c+7
      const uint32_t w0 = q[2 * (c & 1)], w1 = q[2 * (c & 1) + 1];
      const uint32_t e0 = (w0 & m) | (((hb & 5u) * mul) & pos);
      const uint32_t o0 = ((w0 >> 8) & m) | ((((hb >> 1) & 5u) * mul) & pos);
      const uint32_t e1 = (w1 & m) | ((((hb >> 4) & 5u) * mul) & pos);
      const uint32_t o1 = ((w1 >> 8) & m) | ((((hb >> 5) & 5u) * mul) & pos);
      out[c] = u32x4{mixpair<0>(e0, o0, s, nb), mixpair<1>(e0, o0, s, nb),
                     mixpair<0>(e1, o1, s, nb), mixpair<1>(e1, o1, s, nb)};
    }
  }
};
// Q4_1: one 20-byte block per segment (d | m, 16 code bytes); B = RNE_fp16 of
// (d q + m) 2^k formed exactly by the mixed FMA.
template <> struct BR<GQ_Q4_1> {
  static constexpr bool kHeader = false;
  u32x4 a;                                   // d | m, code bytes 0..11
  uint32_t t;                                // code bytes 12..15
  template <bool HDR = true>
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + sg * 20 : kOobOff;
    a = bld16(R, vo, 0);
    t = bld4(R, vo, 16);
  }
  __device__ float bound() const { return fmaf(15.f, fabsf(h2f(a.x)), fabsf(h2f(a.x >> 16))); }
  __device__ void decode(int, int k, u32x4 out[4]) const {
    const float s = __builtin_ldexpf(h2f(a.x), k + 24), nb = __builtin_ldexpf(h2f(a.x >> 16), k);
    const uint32_t c[4] = {a.y, a.z, a.w, t};
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {         // low nibbles for elements < 16
      const int sh = 4 * (cc >> 1);
      const uint32_t w0 = c[2 * (cc & 1)] >> sh, w1 = c[2 * (cc & 1) + 1] >> sh;
      const uint32_t e0 = w0 & 0x000F000Fu, o0 = (w0 >> 8) & 0x000F000Fu;
      const uint32_t e1 = w1 & 0x000F000Fu, o1 = (w1 >> 8) & 0x000F000Fu;
      out[cc] = u32x4{mixpair<0>(e0, o0, s, nb), mixpair<1>(e0, o0, s, nb),
                      mixpair<0>(e1, o1, s, nb), mixpair<1>(e1, o1, s, nb)};
    }
  }
};
template <> struct BR<GQ_Q6_K> {
  static constexpr bool kHeader = false;
  u32x4 ql;
  u32x2 qh;
  uint32_t sc, d;
  template <bool HDR = true>
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + (sg >> 3) * 210 : kOobOff;
    const int G = sg & 7;
    ql = bld16(R, vo + 16 * G, 18);
    qh = bld8(R, vo + 8 * G, 146);
    sc = bld2(R, vo + 2 * G, 2);
    d = bld2(R, vo, 0);
  }
  static constexpr int NF = 4, FL[NF] = {16, 8, 2, 0}, FU[NF] = {32, 16, 4, 0},
                       FB[NF] = {18, 146, 2, 0};
  template <bool HDR = true>
  __device__ void load_at(__amdgpu_buffer_rsrc_t R, const uint32_t (&o)[NF]) {
    ql = bld16(R, (int)o[0], 0);
    qh = bld8(R, (int)o[1], 0);
    sc = bld2(R, (int)o[2], 0);
    d = bld2(R, (int)o[3], 0);
  }
  __device__ float bound() const { return 4096.f * fabsf(h2f(d)); }   // |sc (q - 32)| <= 4096
  __device__ void decode(int, int k, u32x4 out[4]) const {
    const float dd = __builtin_ldexpf(h2f(d), k);
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
      // codes enter as fp16 subnormals q * 2^-24; the mixed FMA rounds the
      // exact a * (q - 32) to fp16 once, as the fp32 form above does
      const float s = a * 16777216.f;
      const uint32_t e0 = v0 & 0x00FF00FFu, o0 = (v0 >> 8) & 0x00FF00FFu;   // bytes 0, 2 / 1, 3
      const uint32_t e1 = v1 & 0x00FF00FFu, o1 = (v1 >> 8) & 0x00FF00FFu;
      out[c] = u32x4{mixpair<0>(e0, o0, s, nb), mixpair<1>(e0, o0, s, nb),
                     mixpair<0>(e1, o1, s, nb), mixpair<1>(e1, o1, s, nb)};
    }
  }
};
// Q2_K: the segment (32-weight group G of a super-block) is 16-weight
// sub-blocks 2G, 2G+1; its codes are bits 2c..2c+1 of the group's 8 plane
// bytes for elements 8c .. 8c+7, so chunk c shifts them down and masks two
// 16-bit fields per dword (subnormal codes into the mixed FMA, as Q4_K).
template <> struct BR<GQ_Q2_K> {
  static constexpr bool kHeader = false;
  uint32_t dm, sm;                           // d | dmin; scale/min bytes of 2G, 2G+1
  u32x2 q;                                   // the group's 8 code bytes
  template <bool HDR = true>
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + (sg >> 3) * 84 : kOobOff;
    const int G = sg & 7;
    dm = bld4(R, vo, 0);
    sm = bld2(R, vo + 2 * G, 4);
    q = bld8(R, vo + 8 * G, 20);
  }
  static constexpr int NF = 3, FL[NF] = {0, 2, 8}, FU[NF] = {0, 4, 16}, FB[NF] = {0, 4, 20};
  template <bool HDR = true>
  __device__ void load_at(__amdgpu_buffer_rsrc_t R, const uint32_t (&o)[NF]) {
    dm = bld4(R, (int)o[0], 0);
    sm = bld2(R, (int)o[1], 0);
    q = bld8(R, (int)o[2], 0);
  }
  // largest |w| the fields allow: 15 * 3 |d| + 15 |dmin|
  __device__ float bound() const { return fmaf(45.f, fabsf(h2f(dm)), 15.f * fabsf(h2f(dm >> 16))); }
  __device__ void decode(int, int k, u32x4 out[4]) const {
    const float d = __builtin_ldexpf(h2f(dm), k + 24), dmin = __builtin_ldexpf(h2f(dm >> 16), k);
#pragma unroll
    for (int c = 0; c < 4; c++) {            // chunk c: elements 8c .. 8c+7
      const uint32_t b = sm >> (8 * (c >> 1));   // sub-block 2G + c / 2
      const float s = d * (float)(b & 15u), nb = -(dmin * (float)((b >> 4) & 15u));
      const uint32_t w0 = q.x >> (2 * c), w1 = q.y >> (2 * c);
      const uint32_t e0 = w0 & 0x00030003u, o0 = (w0 >> 8) & 0x00030003u;   // bytes 0, 2 / 1, 3
      const uint32_t e1 = w1 & 0x00030003u, o1 = (w1 >> 8) & 0x00030003u;
      out[c] = u32x4{mixpair<0>(e0, o0, s, nb), mixpair<1>(e0, o0, s, nb),
                     mixpair<0>(e1, o1, s, nb), mixpair<1>(e1, o1, s, nb)};
    }
  }
};
// Q3_K: the segment's scale fields 2G, 2G+1 (12 bits of the 96-bit stream),
// its 8 low-bit plane bytes and the 32 third bits; each code q = low | third
// << 2 is a byte (fp16 subnormal in its 16-bit field), and the mixed FMA
// rounds the exact a*(q-4) to fp16 once, a = d * sc.
template <> struct BR<GQ_Q3_K> {
  static constexpr bool kHeader = false;
  uint32_t d, sc, qh;
  u32x2 q;
  template <bool HDR = true>
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + (sg >> 3) * 110 : kOobOff;
    const int G = sg & 7;
    d = bld2(R, vo, 0);
    sc = bld4(R, vo + ((12 * G) >> 3), 2);
    q = bld8(R, vo + 8 * G, 14);
    qh = bld4(R, vo + 4 * G, 78);
  }
  // sc: (12 G) >> 3 = 3 (step % 4) + fk for G = 2 (step % 4) + fk
  static constexpr int NF = 4, FL[NF] = {0, 1, 8, 4}, FU[NF] = {0, 3, 16, 8}, FB[NF] = {0, 2, 14, 78};
  template <bool HDR = true>
  __device__ void load_at(__amdgpu_buffer_rsrc_t R, const uint32_t (&o)[NF]) {
    d = bld2(R, (int)o[0], 0);
    sc = bld4(R, (int)o[1], 0);
    q = bld8(R, (int)o[2], 0);
    qh = bld4(R, (int)o[3], 0);
  }
  __device__ float bound() const { return 252.f * fabsf(h2f(d)); }   // |sc (q - 4)| <= 252
  __device__ void decode(int sg, int k, u32x4 out[4]) const {
    const float dd = __builtin_ldexpf(h2f(d), k);
    const uint32_t f = sc >> ((12 * (sg & 7)) & 7);
#pragma unroll
    for (int c = 0; c < 4; c++) {            // chunk c: elements 8c .. 8c+7
      const float a = dd * (float)((f >> (6 * (c >> 1))) & 63u);
      const float s = a * 16777216.f, nb = -4.f * a;   // a * (q - 4) is exact in fp32
      const uint32_t v0 = plane2(q.x, c) | bits_to_b2(qh >> (8 * c));
      const uint32_t v1 = plane2(q.y, c) | bits_to_b2(qh >> (8 * c + 4));
      const uint32_t e0 = v0 & 0x00FF00FFu, o0 = (v0 >> 8) & 0x00FF00FFu;
      const uint32_t e1 = v1 & 0x00FF00FFu, o1 = (v1 >> 8) & 0x00FF00FFu;
      out[c] = u32x4{mixpair<0>(e0, o0, s, nb), mixpair<1>(e0, o0, s, nb),
                     mixpair<0>(e1, o1, s, nb), mixpair<1>(e1, o1, s, nb)};
    }
  }
};
template <> struct BR<GQ_Q8_0> {
  static constexpr bool kHeader = false;
  u32x4 c0, c1;
  uint32_t d;
  template <bool HDR = true>
  __device__ void load(__amdgpu_buffer_rsrc_t R, int vrow, int sg, bool ok) {
    const int vo = ok ? vrow + sg * 34 : kOobOff;
    d = bld2(R, vo, 0);
    c0 = bld16(R, vo, 2);
    c1 = bld16(R, vo, 18);
  }
  __device__ float bound() const { return 128.f * fabsf(h2f(d)); }
  __device__ void decode(int, int k, u32x4 out[4]) const {
    const float dd = __builtin_ldexpf(h2f(d), k);
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
  static constexpr bool kHeader = false;
  u32x4 c;
  uint32_t qh, d;
  template <bool HDR = true>
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
  __device__ float bound() const { return (T == GQ_Q5_0 ? 16.f : 8.f) * fabsf(h2f(d)); }
  __device__ void decode(int, int k, u32x4 out[4]) const {
    const float dd = __builtin_ldexpf(h2f(d), k);
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

// Activations: the thread's share of one BM x 64 tile (NT threads).  fp16:
// load i, thread tid covers row (NT i + tid) / 8, chunk (NT i + tid) % 8 (8
// lanes read one 128-byte line).  fp32: row (NT i + tid) / 16, 4 columns.
template <bool XLO, int NT, int BM> struct AR {
  static constexpr int N = BM * (XLO ? 16 : 8) / NT;
  u32x4 v[N];
};

// A super-block type's field offsets for the tiled kernel's loads: field f of
// the segment 2 * step + fk sits at FL[f] * fk + FU[f] * (step % 4) + FB[f]
// bytes into super-block step / 4 (the 32-weight types have none: N = 1).
template <int T, bool = (Geo<T>::QK == 256)> struct SbFields {
  static constexpr int N = 1;
  __device__ static constexpr int fl(int) { return 0; }
  __device__ static constexpr int fu(int) { return 0; }
  __device__ static constexpr int fb(int) { return 0; }
};
template <int T> struct SbFields<T, true> {
  static constexpr int N = BR<T>::NF;
  __device__ static constexpr int fl(int f) { return BR<T>::FL[f]; }
  __device__ static constexpr int fu(int f) { return BR<T>::FU[f]; }
  __device__ static constexpr int fb(int f) { return BR<T>::FB[f]; }
};

}  // namespace

// VALU instructions placed after each MFMA (measured best: 5; Q6_K 2, whose
// decode has more loads per weight to wait for)
#ifndef GQ_GEMM_VPM
#define GQ_GEMM_VPM (T == GQ_Q6_K ? 2 : 5)
#endif

// KS > 1 splits the K range of a tile over KS groups of BN / 32 waves: each
// group walks its own contiguous share of the K steps with its own activation
// tiles and exponents, and at the end the groups' partial tiles (each taken
// back to unit scale) are summed in group order through LDS, so the result
// does not depend on timing.  More waves per tile then hide the step latency
// where tiles are few (small batches, few weight rows, long rows).
template <int T, bool XLO, int D, int BN, int BM, int KS = 1>
__global__ void __launch_bounds__(2 * BN * KS) k_gemm(const uint8_t* __restrict__ blob, int rows, int cols,
                                                      int rb, const void* __restrict__ xv, int n,
                                                      float* __restrict__ y, int tn, int tm) {
  constexpr int NT = 2 * BN;                 // per group: BN / 32 waves, 32 weight rows each
  constexpr int MI = BM / 32;                // 32-token A fragments per 16 columns
  constexpr int NA = XLO ? 2 : 1;            // activation planes: hi (and lo)
  constexpr int ATILE = BM * ROWB;
  static_assert(D % 2 == 0, "even ring depth: LDS buffer parity is static");
  static_assert(KS == 1 || BN * 4 <= NA * 256, "the partial tiles fit the activation buffers");
  __shared__ __attribute__((aligned(16))) uint8_t As[KS * 2 * NA * ATILE];
  constexpr int ES = XLO ? 4 : 2;
  constexpr int NL = AR<XLO, NT, BM>::N;     // activation loads per thread per step
  constexpr int NW = NT / 64;
  constexpr int XKG = (3 * BM + 2 * NW + 3) / 4 * 4;   // per group (16-byte aligned):
  // fp32 x: per token the exponent change of each staged step (double-
  // buffered like the tile), the current exponent, and per wave whether any
  // token of its share changed in the step
  __shared__ __attribute__((aligned(16))) int xk[XLO ? KS * XKG : 4];

  // tile q of XCD x covers tiles x * per .. ; token tiles of a row tile adjacent
  const int total = tn * tm, per = (total + 7) >> 3;
  const int q = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (q >= total) return;                    // whole workgroup: uniform
  const int n0 = (q / tm) * BN, m0 = (q % tm) * BM;

  const int kg = (KS > 1) ? uniform((int)threadIdx.x / NT) : 0;   // K group
  const int tid = (int)threadIdx.x - kg * NT, lane = tid & 63, w = tid >> 6;
  uint8_t* const Ag = As + kg * 2 * NA * ATILE;          // the group's activation tiles
  int* const dtok = xk + kg * XKG;           // [2][BM]
  int* const ktok = dtok + 2 * BM;           // [BM]
  int* const xflag = dtok + 3 * BM;          // [2][NW]
  const int nr = min(BN, rows - n0), nt = min(BM, n - m0);
  const __amdgpu_buffer_rsrc_t WR = make_rsrc(blob + (int64_t)n0 * rb, (uint32_t)(nr * rb));
  const __amdgpu_buffer_rsrc_t XR =
      make_rsrc((const uint8_t*)xv + (int64_t)m0 * cols * ES, (uint32_t)(nt * cols * ES));
  const int nk = (cols + BK - 1) / BK;
  const int nseg = cols >> 5;
  // the group's K steps: [kbase, kbase + nkg), nkg a multiple of 4 so that a
  // super-block's steps stay in one group and in ring slots 0..3
  const int nkg = (KS > 1) ? ((nk + KS - 1) / KS + 3) / 4 * 4 : nk;
  const int kbase = kg * nkg, kend = min(nk, kbase + nkg);
  // B fragment lane: weight row 32 w + fr of the tile; k half fk = the
  // 32-column segment 2 * step + fk of the row (its chunk ks feeds MFMA ks)
  const int fr = lane & 31, fk = lane >> 5;
  const int vrow = (32 * w + fr) * rb;

  // loop-invariant offsets
  int xo[NL], aw[NL];                        // activation load i: global / LDS offsets
#pragma unroll
  for (int i = 0; i < NL; i++) {
    const int id = NT * i + tid;
    const int t = XLO ? (id >> 4) : (id >> 3);
    const int c = XLO ? 4 * (id & 15) : 8 * (id & 7);
    xo[i] = (t * cols + c) * ES;
    aw[i] = XLO ? tslot(t, (id & 15) >> 1) + 8 * (id & 1) : tslot(t, id & 7);
  }
  const int xc = XLO ? 4 * (tid & 15) : 8 * (tid & 7);   // column of every load
  int fo[BK / 16];                           // A fragment of MFMA ks: chunk 4 fk + ks
#pragma unroll
  for (int ks = 0; ks < BK / 16; ks++) fo[ks] = fr * ROWB + (((4 * fk + ks) ^ swz(fr)) << 4);

  // With a 4-deep ring, ring slot u always holds steps = u mod 4, so only
  // slot 0 (the first step of each super-block) loads the Q4_K header.
  constexpr bool SHARE = BR<T>::kHeader && D == 4;
  // s: the group's step (global step kbase + s); steps past the group's
  // range (or the row) read zeros
  // Super-block types (every row a whole number of K steps): each load's
  // offset is a per-lane part fixed for the launch plus a part common to the
  // wave for the step (kOobOff for steps past the group's range, which puts
  // the sum past every resource: the load reads zero), so a step's address
  // arithmetic is one vector add per load.
  constexpr bool SB = Geo<T>::QK == 256;
  uint32_t lf[SbFields<T>::N];               // per-lane field offsets
  if constexpr (SB) {
#pragma unroll
    for (int f = 0; f < SbFields<T>::N; f++)
      lf[f] = (uint32_t)(vrow + SbFields<T>::fl(f) * fk + SbFields<T>::fb(f));
  }
  auto load = [&](AR<XLO, NT, BM>& a, BR<T>& b, int s, auto hdr) __attribute__((always_inline)) {
    const int gs = kbase + s;
    const bool in = gs < kend;
    if constexpr (SB) {
      uint32_t o[SbFields<T>::N];
#pragma unroll
      for (int f = 0; f < SbFields<T>::N; f++)
        o[f] = lf[f] + (in ? (uint32_t)((gs >> 2) * Geo<T>::BB + SbFields<T>::fu(f) * (gs & 3))
                           : (uint32_t)kOobOff);
      b.template load_at<decltype(hdr)::value>(WR, o);
      const uint32_t ux = in ? (uint32_t)(gs * BK * ES) : (uint32_t)kOobOff;
#pragma unroll
      for (int i = 0; i < NL; i++) a.v[i] = bld16(XR, (int)((uint32_t)xo[i] + ux), 0);
    } else {
      const int sg = 2 * gs + fk;
      b.template load<decltype(hdr)::value>(WR, vrow, sg, in && sg < nseg);
      const int col = gs * BK + xc;
#pragma unroll
      for (int i = 0; i < NL; i++)
        a.v[i] = bld16(XR, (in && col < cols) ? xo[i] + gs * BK * ES : kOobOff, 0);
    }
  };
  // fp32 x: thread slot i always stages the same token, 16 threads per token
  // and step; kx[i] is that token's exponent k (x enters as hi + lo of
  // x 2^k).  It follows the running max of |x| over the steps so far, set so
  // that the max sits in [2^9, 2^10) and lowered (never raised) once a step's
  // max reaches 2^14 at the current k; the accumulators are rescaled then.
  int kx[XLO ? NL : 1];
#pragma unroll
  for (int i = 0; i < (XLO ? NL : 1); i++) kx[i] = KNONE;
  auto stage_a = [&](const AR<XLO, NT, BM>& a, int buf) __attribute__((always_inline)) {
    uint8_t* const A0 = Ag + buf * NA * ATILE;
    bool chg = false;
#pragma unroll
    for (int i = 0; i < NL; i++) {
      if constexpr (XLO) {
        const f32x4 f = __builtin_bit_cast(f32x4, a.v[i]);
        const float m = row16_max(fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
        int dl = 0;
        if (m > 0.f && m < __builtin_huge_valf()) {
          const int e = fexp(m), k = min(126, max(-126, 10 - e));
          if (kx[i] == KNONE) kx[i] = k;
          else if (e + kx[i] > 14) { dl = k - kx[i]; kx[i] = k; }
        }
        chg |= (dl != 0);
        const float sc = __builtin_ldexpf(1.f, kx[i] == KNONE ? 0 : kx[i]);
        uint32_t h0, l0, h1, l1;
        split2_scaled(f.x, f.y, sc, h0, l0);
        split2_scaled(f.z, f.w, sc, h1, l1);
        *reinterpret_cast<u32x2*>(A0 + aw[i]) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(A0 + ATILE + aw[i]) = u32x2{l0, l1};
        if ((tid & 15) == 0) {
          const int t = (NT * i + tid) >> 4;
          dtok[buf * BM + t] = dl;
          ktok[t] = kx[i];
        }
      } else {
        *reinterpret_cast<u32x4*>(A0 + aw[i]) = a.v[i];
      }
    }
    if constexpr (XLO) {
      const bool any = __builtin_amdgcn_ballot_w64(chg) != 0;
      if (lane == 0) xflag[buf * NW + w] = any ? 1 : 0;
    }
  };

  f32x16 acc[MI];
#pragma unroll
  for (int i = 0; i < MI; i++) acc[i] = f32x16{};

  AR<XLO, NT, BM> ra[D];
  BR<T> rw[D];
  u32x4 bq[2][4];                            // decoded B fragments, double-buffered
  u32x4 hcur = {0, 0, 0, 0};                 // header of the current super-block (SHARE)
  auto hflag = [](auto u) { return std::integral_constant<bool, !SHARE || decltype(u)::value == 0>{}; };
  // Weights enter B as RNE_fp16(w 2^kr), kr per row (the lane's row, both
  // k halves agree): set from the first block with a nonzero bound U (the
  // largest |w| its fields allow) so that U 2^kr sits in [2^9, 2^10), and
  // lowered when a later block's U 2^kr reaches 2^14, which rescales the
  // accumulators by the same power of two before that step's products
  // (dpend holds the change until then).  fp16 then carries every weight
  // within 2^-24 of its row's largest bound to 11 bits.
  int kr = KNONE, dpend = 0;
  auto decode = [&](BR<T>& b, int s, u32x4 out[4], auto u) __attribute__((always_inline)) {
    float U = 0.f;                           // 0: no change
    if constexpr (SHARE) {
      // the header, and so U, changes only on a super-block's first step
      if constexpr (decltype(u)::value == 0) {
        hcur = fresh(b.hd);
        U = BR<T>::bound(hcur);
      }
    } else {
      U = b.bound();
    }
    // 32-weight types: the row's two lanes hold different blocks
    if constexpr (Geo<T>::QK == 32) U = max_xor32(U);
    if (U > 0.f && U < __builtin_huge_valf()) {
      const int e = fexp(U);
      if (kr == KNONE) kr = 10 - e;         // the products so far are all zero
      else if (e + kr > 14) { dpend += 10 - e - kr; kr = 10 - e; }
    }
    const int k = (kr == KNONE) ? 0 : kr;
    if constexpr (SHARE) b.decode(2 * (kbase + s) + fk, hcur, k, out);
    else b.decode(2 * (kbase + s) + fk, k, out);
  };
  // Before step i's products: bring the accumulators to step i's exponents
  // (row: decided when step i was decoded; fp32 x: when it was staged).
  // Both only ever fall, so this is a rare, uniform branch.
  auto rescale = [&](int buf) __attribute__((always_inline)) {
    bool any = __builtin_amdgcn_ballot_w64(dpend != 0) != 0;
    if constexpr (XLO) {
      int fl = 0;
#pragma unroll
      for (int j = 0; j < NW; j++) fl |= xflag[buf * NW + j];
      any = any || __builtin_amdgcn_readfirstlane(fl) != 0;
    }
    if (any) {
#pragma unroll
      for (int mi = 0; mi < MI; mi++)
#pragma unroll
        for (int qg = 0; qg < 4; qg++) {
          int4 dt = {0, 0, 0, 0};
          if constexpr (XLO) dt = *reinterpret_cast<const int4*>(dtok + buf * BM + 32 * mi + 8 * qg + 4 * fk);
          acc[mi][4 * qg + 0] = __builtin_ldexpf(acc[mi][4 * qg + 0], dpend + dt.x);
          acc[mi][4 * qg + 1] = __builtin_ldexpf(acc[mi][4 * qg + 1], dpend + dt.y);
          acc[mi][4 * qg + 2] = __builtin_ldexpf(acc[mi][4 * qg + 2], dpend + dt.z);
          acc[mi][4 * qg + 3] = __builtin_ldexpf(acc[mi][4 * qg + 3], dpend + dt.w);
        }
    }
    dpend = 0;
  };
  static_for<D>([&](auto u) {
    load(ra[u], rw[u], u, hflag(u));         // issued in ring order
    __builtin_amdgcn_sched_barrier(0);
  });
  stage_a(ra[0], 0);
  decode(rw[0], 0, bq[0], std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  load(ra[0], rw[0], D, hflag(std::integral_constant<int, 0>{}));
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // Steps past the last read zeros (masked loads), so every unrolled step
  // runs unguarded and adds exactly nothing.
  for (int i0 = 0; i0 < nkg; i0 += D) {
    static_for<D>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const int i = i0 + u;
      constexpr int buf = u & 1;             // i0 is a multiple of D, D even
      const uint8_t* const A0 = Ag + buf * NA * ATILE;
      constexpr int sl = (u + 1) % D;        // ring slot of step i + 1
      const std::integral_constant<int, sl> slc{};
      rescale(buf);
      __builtin_amdgcn_sched_barrier(0);
      // decode step i + 1 while the matrix cores run step i
      decode(rw[sl], i + 1, bq[buf ^ 1], slc);
      // A fragments of sub-step ks + 1 are read while sub-step ks multiplies
      f16x8 af[2][NA][MI];
      auto read_a = [&](int ks, f16x8 (&f)[NA][MI]) __attribute__((always_inline)) {
#pragma unroll
        for (int mi = 0; mi < MI; mi++)
#pragma unroll
          for (int p = 0; p < NA; p++)
            f[p][mi] = *reinterpret_cast<const f16x8*>(A0 + p * ATILE + mi * 32 * ROWB + fo[ks]);
      };
      read_a(0, af[0]);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ks++) {
        if (ks + 1 < BK / 16) read_a(ks + 1, af[(ks + 1) & 1]);
        const f16x8 bf = __builtin_bit_cast(f16x8, bq[buf][ks]);
#pragma unroll
        for (int mi = 0; mi < MI; mi++)
#pragma unroll
          for (int p = 0; p < NA; p++)
            acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks & 1][p][mi], bf, acc[mi], 0, 0, 0);
      }
      stage_a(ra[sl], buf ^ 1);
#ifndef GQ_GEMM_NO_PIPE
      // Shape of this step for the scheduler: the first fragments, then each
      // MFMA followed by a share of the decode VALU and the next fragment
      // read, so the matrix cores, VALU and LDS overlap within every wave.
      __builtin_amdgcn_sched_group_barrier(0x100, MI * NA, 0);  // DS read
#pragma unroll
      for (int k = 0; k < 4 * MI * NA; k++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, GQ_GEMM_VPM, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
      }
      __builtin_amdgcn_sched_group_barrier(0x200, NL * NA, 0);  // DS write: stage last
#endif
      __builtin_amdgcn_sched_barrier(0);
      load(ra[sl], rw[sl], i + 1 + D, hflag(slc));   // past the last step: zeros
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    });
  }

  // D lane l, register v: weight row 32 w + l % 32, token 32 mi + 8 (v / 4) +
  // 4 (l / 32) + v % 4.  Steps past the last column read zeros and change
  // no exponent, so the accumulators are at (kr, ktok) here; y takes 2^-k.
  const int r = 32 * w + fr;
  const int kw = (kr == KNONE) ? 0 : kr;
  if constexpr (KS == 1) {
#pragma unroll
    for (int mi = 0; mi < MI; mi++)
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int t = mi * 32 + 8 * (v >> 2) + 4 * fk + (v & 3);
        int k = kw;
        if constexpr (XLO) k += (ktok[t] == KNONE) ? 0 : ktok[t];
        if (t < nt && r < nr) y[(int64_t)(m0 + t) * rows + n0 + r] = __builtin_ldexpf(acc[mi][v], -k);
      }
  } else {
    // each group's partial tile at unit scale into LDS (over the activation
    // tiles, which every wave is done with after the loop's last barrier),
    // then group 0 sums the KS partials in group order
    float* const red = reinterpret_cast<float*>(As);   // [KS][BN/32][16 MI][64]
#pragma unroll
    for (int mi = 0; mi < MI; mi++)
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int t = mi * 32 + 8 * (v >> 2) + 4 * fk + (v & 3);
        int k = kw;
        if constexpr (XLO) k += (ktok[t] == KNONE) ? 0 : ktok[t];
        red[((kg * (BN / 32) + w) * 16 * MI + 16 * mi + v) * 64 + lane] = __builtin_ldexpf(acc[mi][v], -k);
      }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int mi = 0; mi < MI; mi++)
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const int t = mi * 32 + 8 * (v >> 2) + 4 * fk + (v & 3);
          float sum = 0.f;
#pragma unroll
          for (int g = 0; g < KS; g++) sum += red[((g * (BN / 32) + w) * 16 * MI + 16 * mi + v) * 64 + lane];
          if (t < nt && r < nr) y[(int64_t)(m0 + t) * rows + n0 + r] = sum;
        }
    }
  }
}

namespace {

template <int T, bool XLO, int BN, int BM, int KS = 1, int D = (XLO ? 2 : 4)>
hipError_t gemm_cfg(const void* blob, int64_t rows, int64_t cols, const void* x, int64_t n, float* y,
                    hipStream_t st) {
  const int64_t rb = cols / Geo<T>::QK * Geo<T>::BB;
  const int64_t es = XLO ? 4 : 2;
  if ((int64_t)BN * rb >= kOobOff || (int64_t)BM * cols * es >= kOobOff) return hipErrorInvalidValue;
  const int64_t tn = (rows + BN - 1) / BN, tm = (n + BM - 1) / BM;
  if (tn * tm >= ((int64_t)1 << 31) / 8) return hipErrorInvalidValue;
  const int64_t grid = (tn * tm + 7) / 8 * 8;
  hipLaunchKernelGGL((k_gemm<T, XLO, D, BN, BM, KS>), dim3((unsigned)grid), dim3(2 * BN * KS), 0, st,
                     (const uint8_t*)blob, (int)rows, (int)cols, (int)rb, x, (int)n, y, (int)tn,
                     (int)tm);
  return hipGetLastError();
}

template <int T, bool XLO>
hipError_t gemm_t(const void* blob, int64_t rows, int64_t cols, const void* x, int64_t n, float* y,
                  hipStream_t st) {
  const int c = gemm_tile_config(T, rows, cols, n, !XLO);
  if constexpr (!XLO) {
    // split K: one-wave groups stage 8 loads per step each, so their ring is
    // 2 deep (4 would cost a wave per SIMD)
    if (c == 3) return gemm_cfg<T, false, 32, 64, 4, 2>(blob, rows, cols, x, n, y, st);
    // 64 x 64 split tiles: a 4-deep ring where the super-block header is
    // shared over its 4 steps (Q4_K, Q5_K), else 2 deep (measured on
    // MI355X: Q6_K 11008x4096 at 64 tokens 40.6 -> 37.8 us, 4096x14336 at 256
    // 118 -> 111 us, Q2_K / Q3_K / Q4_0 / Q5_0 / Q4_1 / Q8_0 -4 to -7 %;
    // Q4_K +6 to +8 % at 2)
    if (c == 4) return gemm_cfg<T, false, 64, 64, 4, BR<T>::kHeader ? 4 : 2>(blob, rows, cols, x, n, y, st);
    if (c == 5) return gemm_cfg<T, false, 64, 128, 2, 2>(blob, rows, cols, x, n, y, st);
  }
  if (c == 1) return gemm_cfg<T, XLO, 128, 128>(blob, rows, cols, x, n, y, st);
  if (c == 2) return gemm_cfg<T, XLO, 128, 64>(blob, rows, cols, x, n, y, st);
  return gemm_cfg<T, XLO, 256, 128>(blob, rows, cols, x, n, y, st);
}

}  // namespace

// Every tile walks its K range, so a shape with few tiles leaves CUs idle.
// fp16 x, measured on MI355X (us):
//   * up to 64 tokens, K split over 4 groups of a workgroup: 64-row tiles
//     once the rows fill 256 CUs with 32-row tiles (Q4_K 11008 x 4096 at 64
//     tokens 34.0 -> 25.9, 14336 x 4096 34.3 -> 26.5), 32-row tiles below
//     that (8192 x 4096 23.0, Q6_K 4096 x 11008 162 -> 72); no split past
//     256 64-row tiles, where 128 x 64 tiles already fill the chip (Q4_K
//     22016 x 4096 37.4 against 49.8 split, Q6_K 128256 x 4096 269 against 330);
//   * up to 256 tokens: 64 x 64 tiles in 4 K groups while those fit 256 CUs
//     and 128 x 64 tiles would be more than 64 (below 129 tokens, 128 or
//     more);
//   * more tokens: 256 x 128 tiles when they cover 128 to 256 CUs once,
//     128 x 128 past that, 128 x 64 below (Q4_K 4096 x 4096 at 512 tokens
//     62 -> 37); 32-row split-K tiles when even 128 x 64 tiles are fewer than
//     128 (Q4_K 1024 x 4096 at 512 37 -> 22); Q6_K, whose decode is the
//     longest, in 64 x 128 tiles of 2 K groups (4096 x 14336 at 512 185 -> 168).
// fp32 x keeps one K group per tile (its split variants need more registers
// than a wave has and are not built).
int gemm_tile_config(int type, int64_t rows, int64_t cols, int64_t n_tok, bool x_f16) {
  (void)cols;
#ifdef GQ_TUNE_ENV
  if (const char* e = getenv("GQ_GEMM_CFG")) {
    const int c = atoi(e);
    if (x_f16 || c < 3) return c;
  }
#endif
  const int64_t t128x64 = (rows + 127) / 128 * ((n_tok + 63) / 64);
  if (x_f16) {
    if (n_tok <= 64) {
      if ((rows + 63) / 64 > 256) return 2;  // enough 128-row tiles: no split
      return (rows + 31) / 32 > 256 ? 4 : 3;
    }
    // up to 256 tokens on few rows: 32-row split tiles up to 128 tokens
    // while 128 x 64 tiles would be fewer than 128, else 64 x 64 split tiles
    // while they fit the chip in one round and 128 x 64 tiles would be more
    // than 64 (4096 x 4096 at 192 / 256 tokens 29.1 / 30.8 -> 24.1 / 24.7 us,
    // 8192 x 4096 at 96 / 128 30.8 / 31.2 -> 24.5 / 25.9, Q6_K 4096 x 11008
    // at 192 / 256 110 / 138 -> 98 / 97, Q6_K 4096 x 14336 at 256 172 -> 118;
    // on fewer rows the 32-row tiles stay ahead: 2048 x 2048 at 160 tokens
    // 13.3 against 19.6 us; past 256 tokens the unsplit tiles)
    if (t128x64 < 128 && n_tok <= 128) return 3;
    if (n_tok <= 256 && t128x64 > 64 && (rows + 63) / 64 * ((n_tok + 63) / 64) <= 256) return 4;
    if (t128x64 < 128) return 3;
    if (type == GQ_Q6_K && t128x64 <= 256) return 5;
  }
  if (n_tok <= 64) return 2;
  const int64_t big = (rows + 255) / 256 * ((n_tok + 127) / 128);
  if (big > 256) return 1;
  return big >= 128 ? 0 : 2;
}

// A launch's time: a fixed start (first loads in flight, tail) plus the K
// steps of a tile times the measured time of one step at that tile shape,
// stretched by the tiles past one per CU.
double gemm_estimate_us(int type, int64_t rows, int64_t cols, int64_t n_tok, bool x_f16) {
  // per tile shape: rows, tokens, K groups, and a step's time per type
  // (Q4_K / Q5_K / Q2_K, Q6_K, Q8_0 / Q5_0 / Q3_K, Q4_0 / Q4_1; Q4_1 measured
  // at Q4_0's step times: 4096x4096 at 64 tokens 22.7 us tiled)
  struct Cfg {
    int64_t bn, bm, ks;
    double step_us[4];
  };
  static const Cfg cfg[6] = {
      {256, 128, 1, {1.13, 1.75, 1.4, 1.2}}, {128, 128, 1, {0.9, 1.3, 1.2, 1.0}},
      {128, 64, 1, {0.5, 0.82, 0.81, 0.6}},  {32, 64, 4, {1.2, 1.6, 1.6, 1.3}},
      {64, 64, 4, {1.4, 2.3, 2.2, 1.75}},    {64, 128, 2, {1.22, 1.5, 1.7, 1.3}}};
  int c = gemm_tile_config(type, rows, cols, n_tok, x_f16);
  if (c < 0 || c > 5) c = 0;
  const Cfg& f = cfg[c];
  const int tc = (type == GQ_Q4_K || type == GQ_Q5_K || type == GQ_Q2_K) ? 0
                 : (type == GQ_Q6_K) ? 1 : (type == GQ_Q4_0 || type == GQ_Q4_1) ? 3 : 2;
  const double tiles = (double)((rows + f.bn - 1) / f.bn * ((n_tok + f.bm - 1) / f.bm));
  const double steps = (double)(((cols + BK - 1) / BK + f.ks - 1) / f.ks);
  const double load = tiles > 256.0 ? tiles / 256.0 : 1.0;
  return 4.0 + load * steps * f.step_us[tc];
}

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
    GQ_GEMM_CASE(GQ_Q4_1)
    GQ_GEMM_CASE(GQ_Q5_K)
    GQ_GEMM_CASE(GQ_Q2_K)
    GQ_GEMM_CASE(GQ_Q3_K)
#undef GQ_GEMM_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace gq
