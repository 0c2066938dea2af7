// gq_device.h — device-side helpers shared by libgq's kernels (gfx950 only).
//
// Block layouts are the ones declared in include/gq.h.  Everything here is
// register-level bit manipulation on raw block bytes; no host code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "../../include/gq.h"

namespace gq {

// Unaligned vector types: the blob's blocks are 18, 22, 34 or 210 bytes, so
// block fields are generally not naturally aligned.  gfx950 global loads
// accept unaligned addresses; these typedefs tell the compiler so.
typedef uint32_t u32x4u __attribute__((ext_vector_type(4), aligned(1)));
typedef uint32_t u32x2u __attribute__((ext_vector_type(2), aligned(1)));
typedef uint32_t u32u __attribute__((aligned(1)));
typedef uint16_t u16u __attribute__((aligned(1)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), unrolled,
// so that register arrays indexed by the constant stay in registers.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ __forceinline__ u32x4 ld16u(const uint8_t* p) {
  u32x4u v = *reinterpret_cast<const u32x4u*>(p);
  return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ u32x4 ld16a(const uint8_t* p) {   // 16-B aligned
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8u(const uint8_t* p) {
  u32x2u v = *reinterpret_cast<const u32x2u*>(p);
  return u32x2{v.x, v.y};
}
__device__ __forceinline__ uint32_t ld4u(const uint8_t* p) {
  return *reinterpret_cast<const u32u*>(p);
}
__device__ __forceinline__ uint32_t ld2u(const uint8_t* p) {
  return *reinterpret_cast<const u16u*>(p);
}

// Raw buffer loads through a scalar resource: byte offsets are 32-bit and
// any load whose offset reaches past the resource's size returns zero without
// touching memory (the range check covers the vector offset plus the
// instruction offset).
constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit buffer resource word 3 (gfx950)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, int voff, int imm) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + imm, 0, 0));
}
__device__ __forceinline__ u32x2 bld8(__amdgpu_buffer_rsrc_t r, int voff, int imm) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff + imm, 0, 0));
}
__device__ __forceinline__ u32x3 bld12(__amdgpu_buffer_rsrc_t r, int voff, int imm) {
  return __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, voff + imm, 0, 0));
}
__device__ __forceinline__ uint32_t bld4(__amdgpu_buffer_rsrc_t r, int voff, int imm) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff + imm, 0, 0);
}
__device__ __forceinline__ uint32_t bld2(__amdgpu_buffer_rsrc_t r, int voff, int imm) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff + imm, 0, 0);
}
// A vector offset no resource reaches (resources here stay below 2^31 bytes).
constexpr int kOobOff = 0x7FFF0000;

// fp16 bit pattern (low 16 bits of h) -> fp32, exact (subnormals included).
__device__ __forceinline__ float h2f(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
  return (float)v;
}

// Byte k of w as an exact fp32: one v_cvt_f32_ubyte{k}.  Written as asm
// because the compiler otherwise folds a preceding nibble mask into a
// v_bfe_u32 + v_cvt_f32_ubyte0 pair.
__device__ __forceinline__ float ub0(uint32_t w) {
  float r; asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(w)); return r;
}
__device__ __forceinline__ float ub1(uint32_t w) {
  float r; asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(w)); return r;
}
__device__ __forceinline__ float ub2(uint32_t w) {
  float r; asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(w)); return r;
}
__device__ __forceinline__ float ub3(uint32_t w) {
  float r; asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(w)); return r;
}

// Byte k of w as a signed (two's complement) exact fp32 (v_cvt_f32_i32 with
// a sign-extending byte select).
__device__ __forceinline__ float sb0(uint32_t w) { return (float)(int)(int8_t)w; }
__device__ __forceinline__ float sb1(uint32_t w) { return (float)(int)(int8_t)(w >> 8); }
__device__ __forceinline__ float sb2(uint32_t w) { return (float)(int)(int8_t)(w >> 16); }
__device__ __forceinline__ float sb3(uint32_t w) { return (float)((int)w >> 24); }

// Four unsigned codes q (one per byte, q + 128 - off < 256) to the signed
// bytes q - off: add 128 - off to every byte (no carries), flip the sign bit.
template <int OFF>
__device__ __forceinline__ uint32_t centre(uint32_t q4) {
  return (q4 + (uint32_t)(128 - OFF) * 0x01010101u) ^ 0x80808080u;
}

// Block geometry.
template <int T> struct Geo;
template <> struct Geo<GQ_Q4_0> { static constexpr int QK = 32,  BB = 18;  };
template <> struct Geo<GQ_Q5_0> { static constexpr int QK = 32,  BB = 22;  };
template <> struct Geo<GQ_Q8_0> { static constexpr int QK = 32,  BB = 34;  };
template <> struct Geo<GQ_Q4_K> { static constexpr int QK = 256, BB = 144; };
template <> struct Geo<GQ_Q6_K> { static constexpr int QK = 256, BB = 210; };
template <> struct Geo<GQ_Q4_1> { static constexpr int QK = 32,  BB = 20;  };
template <> struct Geo<GQ_Q5_K> { static constexpr int QK = 256, BB = 176; };
template <> struct Geo<GQ_Q2_K> { static constexpr int QK = 256, BB = 84;  };
template <> struct Geo<GQ_Q3_K> { static constexpr int QK = 256, BB = 110; };

// A "segment" is 32 consecutive weights of a row: one block of the 32-weight
// types, one sub-block of Q4_K, one 32-weight group of Q6_K.  Segment s of a
// row lives in block s / (QK/32), part s % (QK/32).
template <int T> struct SegAddr {
  static constexpr int PER_BLOCK = Geo<T>::QK / 32;
  __device__ static const uint8_t* block(const uint8_t* row, int s) {
    return row + (size_t)(s / PER_BLOCK) * Geo<T>::BB;
  }
};

// Q4_K: 12-bit (scale, min) pair of sub-block i from header dwords w0..w2
// (bytes 4..15 of the block).  Field k sits at bits 6k..6k+5 of the 96-bit
// little-endian stream, so sub-block i's pair is bits 12i..12i+11.
__device__ __forceinline__ uint32_t q4k_pair(uint32_t w0, uint32_t w1, uint32_t w2, int i) {
  uint64_t lo = (uint64_t)w0 | ((uint64_t)w1 << 32);
  uint64_t hi = (uint64_t)w1 | ((uint64_t)w2 << 32);
  int sh = 12 * i;
  uint32_t v = (i <= 4) ? (uint32_t)(lo >> sh) : (uint32_t)(hi >> (sh - 32));
  return v & 0xFFFu;
}

// Q6_K: the 2-bit high parts of one quarter of a 32-weight group, moved to
// bits 4..5 of each byte.  hq is the qh dword holding bytes k = 4*(quarter&1)
// .. +3 of the group's 8 qh bytes; u selects bits 2u..2u+1.
__device__ __forceinline__ uint32_t q6k_hi(uint32_t hq, int u) {
  // ((hq >> 2u) & 0x03030303) << 4
  return (u <= 2 ? (hq << (4 - 2 * u)) : (hq >> (2 * u - 4))) & 0x30303030u;
}

// Spread 4 bits (b0..b3 of v) to bit 4 of bytes 0..3.
__device__ __forceinline__ uint32_t spread4_bit4(uint32_t v) {
  v &= 0xFu;
  return ((v & 1u) << 4) | ((v & 2u) << 11) | ((v & 4u) << 18) | ((v & 8u) << 25);
}

// Bit b (b = 0..3) of v4 to bit 4 of byte b: the multiply places bit b at
// bits b + 7k (k = 0..3), all distinct, so no carries; bit 8b is the k = b copy.
__device__ __forceinline__ uint32_t bits_to_b4(uint32_t v4) {
  return (((v4 & 0xFu) * 0x00204081u) & 0x01010101u) << 4;   // a 24-bit multiply
}

// Bit b (b = 0..3) of v4 to bit 2 of byte b (Q3_K's third bits).
__device__ __forceinline__ uint32_t bits_to_b2(uint32_t v4) {
  return (((v4 & 0xFu) * 0x00204081u) & 0x01010101u) << 2;
}

// Q2_K / Q3_K 2-bit plane: byte 8g+k holds elements 32g+k+8u at bits
// 2u..2u+1, so the codes of elements 8u .. 8u+7 of group g are bits 2u..2u+1
// of the group's 8 bytes (w0 = bytes 0..3, w1 = bytes 4..7), one per byte.
__device__ __forceinline__ uint32_t plane2(uint32_t w, int u) {
  return (w >> (2 * u)) & 0x03030303u;
}

// fp16 pair {RNE_fp16(c0 s + nb), RNE_fp16(c1 s + nb)} for codes held in
// 16-bit fields (c0 in field H of p0, c1 in field H of p1) and a scale s
// carrying a factor 2^24: a field below 1024 read as fp16 is the subnormal
// c * 2^-24 exactly, so each v_fma_mix forms the exact c * (s 2^-24) + nb and
// rounds it once, as the convert-then-mix form does, with no convert.
template <int H>
__device__ __forceinline__ uint32_t mixpair(uint32_t p0, uint32_t p1, float s, float nb) {
  uint32_t d;
  if constexpr (H == 0)
    asm("v_fma_mixlo_f16 %0, %1, %3, %4 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %2, %3, %4 op_sel_hi:[1,0,0]"
        : "=&v"(d) : "v"(p0), "v"(p1), "v"(s), "v"(nb));
  else
    asm("v_fma_mixlo_f16 %0, %1, %3, %4 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %2, %3, %4 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(d) : "v"(p0), "v"(p1), "v"(s), "v"(nb));
  return d;
}

// Wave-uniform value in a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Wave64 sum on the DPP network (no LDS round trips): quad swaps, then row
// shifts by 4 and 8, then the row broadcasts; lane 63 ends with the total,
// which readlane returns to every lane.  Lanes a DPP source does not cover
// contribute the 0 passed as the old value.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x114>(v);   // row_shr:4
  v += dpp_mov<0x118>(v);   // row_shr:8
  v += dpp_mov<0x142>(v);   // row_bcast:15
  v += dpp_mov<0x143>(v);   // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum over each aligned group of G lanes (G = 16, 32 or 64) on the DPP
// network; the group's total lands in its last lane (lane G-1 of the group).
template <int G>
__device__ __forceinline__ float group_sum_dpp(float v) {
  static_assert(G == 16 || G == 32 || G == 64, "group of 16, 32 or 64 lanes");
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x114>(v);   // row_shr:4
  v += dpp_mov<0x118>(v);   // row_shr:8: lanes 12..15 of each row hold its sum
  if (G >= 32) v += dpp_mov<0x142>(v);   // row_bcast:15: row pairs
  if (G >= 64) v += dpp_mov<0x143>(v);   // row_bcast:31: whole wave
  return v;
}

// Wave64 sum with cross-lane swaps (result valid in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Exact power-of-two scaling for fp16 matrix-core operands.  fp16 covers
// magnitudes 2^-24 .. 65504, fp32 2^-149 .. 2^128, so an fp32 value (or a
// weight decoded in fp32) is brought into fp16 range by a factor 2^k chosen
// from the largest magnitude m of the values that share it, and the fp32
// results are multiplied by 2^-k; both multiplications are exact.

// Exponent e with m in [2^(e-1), 2^e) (v_frexp_exp_i32_f32); m finite, > 0.
__device__ __forceinline__ int fexp(float m) { return __builtin_amdgcn_frexp_expf(m); }

// Scale exponent that puts m in [2^(top-1), 2^top); 0 when m is zero, NaN or
// infinite (those then reach the results unchanged); clamped to +-126 so
// that 2^k is a normal fp32 value.
template <int TOP>
__device__ __forceinline__ int pow2_exp_for(float m) {
  if (!(m > 0.f) || !(m < __builtin_huge_valf())) return 0;
  const int k = TOP - fexp(m);
  return k > 126 ? 126 : (k < -126 ? -126 : k);
}

// {RNE_fp16(x0 s), RNE_fp16(x1 s)} and {RNE_fp16(x0 s - hi0), RNE_fp16(x1 s -
// hi1)}: each mixed FMA forms the exact product (s a power of two) and rounds
// once, so hi + lo keeps ~22 bits of x s; four instructions per pair.
__device__ __forceinline__ void split2_scaled(float x0, float x1, float s, uint32_t& hi,
                                              uint32_t& lo) {
  asm("v_fma_mixlo_f16 %0, %1, %2, 0\n\tv_fma_mixhi_f16 %0, %3, %2, 0"
      : "=&v"(hi) : "v"(x0), "v"(s), "v"(x1));
  asm("v_fma_mixlo_f16 %0, %1, %2, -%4 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %3, %2, -%4 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(lo) : "v"(x0), "v"(s), "v"(x1), "v"(hi));
}

// v_permlane32_swap: lanes 32..63 of a trade places with lanes 0..31 of b
// (a = {a_lo, b_lo}, b = {a_hi, b_hi}); v_permlane16_swap: rows 1 and 3 of
// a with rows 0 and 2 of b (rows of 16 lanes).  Written as asm because the
// compiler's builtins for these return the first register for both results;
// the s_nop give the wait states around a VALU write and a permlane read.
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// max over lanes l and l ^ 32, in every lane.
__device__ __forceinline__ float max_xor32(float v) {
  float a = v, b = v;
  swap32(a, b);                              // a = {v_lo, v_lo}, b = {v_hi, v_hi}
  return fmaxf(a, b);
}

// max over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four 16-lane rows), in every lane.
__device__ __forceinline__ float max_rows4(float v) {
  float a = v, b = v;
  swap16(a, b);                              // rows {0,0,2,2} and {1,1,3,3}
  return max_xor32(fmaxf(a, b));
}

// Max over each 16-lane row, the result in every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 decltype(ctrl)::value, 0xF, 0xF,
                                                                 false));
  };
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x128>{}));   // row_ror:8
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x124>{}));   // row_ror:4
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));    // quad_perm [2,3,0,1]
  return fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{})); // quad_perm [1,0,3,2]
}

// Sum over each 16-lane row, in every lane of the row (the lanes may differ
// in the rounding order of the additions; callers keep one lane's result).
__device__ __forceinline__ float row16_sum(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 decltype(ctrl)::value, 0xF, 0xF,
                                                                 false));
  };
  v += dpp(v, std::integral_constant<int, 0x128>{});   // row_ror:8
  v += dpp(v, std::integral_constant<int, 0x124>{});   // row_ror:4
  v += dpp(v, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  return v + dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
}

// Per-column max over all 64 lanes of N columns m[0..N-1] (N = 8 or 16,
// values >= 0), transposed so that few instructions serve all columns:
// v_permlane32_swap halves the lane count per column while pairing column t
// with t + N/2, v_permlane16_swap (rows 1 and 3 of its first operand with
// rows 0 and 2 of its second) pairs t with t + N/4, and a row reduction
// finishes.  Afterwards register t (t < N/4) holds in every lane of row rho
// the max of column t + (N/4) rho.
template <int N>
__device__ __forceinline__ void transposed_max(float (&m)[N]) {
  static_assert(N == 8 || N == 16, "8 or 16 columns");
#pragma unroll
  for (int t = 0; t < N / 2; t++) {          // lanes 0..31: column t, 32..63: t + N/2
    swap32(m[t], m[t + N / 2]);
    m[t] = fmaxf(m[t], m[t + N / 2]);
  }
#pragma unroll
  for (int t = 0; t < N / 4; t++) {          // rows: t, t + N/4, t + N/2, t + 3N/4
    swap16(m[t], m[t + N / 4]);
    m[t] = row16_max(fmaxf(m[t], m[t + N / 4]));
  }
}

}  // namespace gq
