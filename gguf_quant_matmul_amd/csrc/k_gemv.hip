// k_gemv.hip — batch-1 GEMV over GGUF blocks, dequantized inside the dot
// product ("Local LLM inference", "The mmap backend").  Decode at batch 1
// reads every weight once and is bound by memory bandwidth ("12 — llama.cpp /
// GGUF", "The bandwidth cap"); on gfx950 the vector-ALU instruction count per
// weight is the second limit, so the kernel keeps it near the essential
// convert + FMA per weight:
//   * lane <-> one 64-weight slice of a row (a quarter of a Q4_K/Q6_K block,
//     or two 32-weight blocks), so block headers are decoded once per 64
//     weights;
//   * weights arrive through buffer loads on a per-row-set scalar descriptor:
//     the per-lane byte offset is loop-invariant, so no address arithmetic
//     runs per load, and reads past the descriptor's range return zero;
//   * x is staged once per workgroup in LDS as fp32 (16-byte chunks XOR-
//     swizzled per slice) with the sums of x over every 16 columns;
//   * Q4_K uses factored sub-block sums a*sum(q*x) - b*sum(x) (Hitchhiker's
//     Guide §11.2, w = (d*sc)*q - dmin*m), its codes entering their products
//     as fp16 subnormals (one mixed-precision FMA per weight, no convert);
//     Q6_K and the 32-weight types convert each code to the signed q - offset
//     so every product is exact relative to w; fp32 accumulation;
//   * persistent workgroups (as many as fit on the chip) loop over groups of
//     rows with the next group's loads in flight (a wave's first two items
//     go out before or after x is staged, by how many items it has); row
//     sums and the 16-column sums of x use the DPP network.
#include "gq_device.h"
#include "gq_launch.h"

namespace gq {

// acc + sum over the 4 bytes of w (as signed integers) * x[k].
__device__ __forceinline__ float dot4s(uint32_t w, const float* x, float acc) {
  acc = fmaf(sb0(w), x[0], acc);
  acc = fmaf(sb1(w), x[1], acc);
  acc = fmaf(sb2(w), x[2], acc);
  return fmaf(sb3(w), x[3], acc);
}

// dot4s, and the same over unsigned bytes, with each byte's convert and its
// FMA kept adjacent in one asm block: the scheduler cannot hoist a whole
// slice's converts ahead of the FMAs and hold 64 converted codes live at once
// (Q6_K's decode, or any type's with two row sets, otherwise needs enough
// registers to halve the waves per SIMD).
__device__ __forceinline__ float dot4u_asm(uint32_t w, const float* x, float acc) {
  float t;
  asm("v_cvt_f32_ubyte0 %1, %2\n\tv_fmac_f32 %0, %1, %3\n\t"
      "v_cvt_f32_ubyte1 %1, %2\n\tv_fmac_f32 %0, %1, %4\n\t"
      "v_cvt_f32_ubyte2 %1, %2\n\tv_fmac_f32 %0, %1, %5\n\t"
      "v_cvt_f32_ubyte3 %1, %2\n\tv_fmac_f32 %0, %1, %6"
      : "+v"(acc), "=&v"(t)
      : "v"(w), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
  return acc;
}
__device__ __forceinline__ float dot4s_asm(uint32_t w, const float* x, float acc) {
  float t;
  asm("v_cvt_f32_i32_sdwa %1, sext(%2) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
      "v_fmac_f32 %0, %1, %3\n\t"
      "v_cvt_f32_i32_sdwa %1, sext(%2) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1\n\t"
      "v_fmac_f32 %0, %1, %4\n\t"
      "v_cvt_f32_i32_sdwa %1, sext(%2) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
      "v_fmac_f32 %0, %1, %5\n\t"
      "v_cvt_f32_i32_sdwa %1, sext(%2) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3\n\t"
      "v_fmac_f32 %0, %1, %6"
      : "+v"(acc), "=&v"(t)
      : "v"(w), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
  return acc;
}

template <bool ASM>
__device__ __forceinline__ float dot4s_(uint32_t w, const float* x, float acc) {
  return ASM ? dot4s_asm(w, x, acc) : dot4s(w, x, acc);
}

// acc + 2^-24 (c0 x[0] + c1 x[1] + c2 x[2] + c3 x[3]) for unsigned codes c_i
// held in 16-bit fields, c0 and c2 in the low and high field of p02, c1 and c3
// in those of p13.  A field below 1024 read as fp16 is the subnormal c * 2^-24
// exactly, so each v_fma_mix_f32 takes a code straight to its fp32 product
// with x: the sum is exactly 2^-24 times the one convert + FMA gives, with the
// same roundings, while x * 2^-24 stays a normal fp32 number (|x| > 2^-102).
__device__ __forceinline__ float dot4mix(uint32_t p02, uint32_t p13, const float* x, float acc) {
  asm("v_fma_mix_f32 %0, %1, %3, %0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %0, %2, %4, %0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %0, %1, %5, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %0, %2, %6, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(acc)
      : "v"(p02), "v"(p13), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
  return acc;
}
constexpr float kSub = 16777216.f;            // 2^24: undoes the subnormal scale

// One lane's 64-weight slice of one row: raw registers and the slice dot in
// two halves of 32 weights.  voff(sl) is slice sl's byte offset in its row;
// j = sl % 4 its quarter of a K-quant block.  dot(h, x, xs, j) takes half h's
// 32 activations and the sums of x over its two 16-column quarters.  A final
// slice of a 32-weight type may have only its first block in the row; its
// second half is then never computed.
template <int T> struct Slice;

template <> struct Slice<GQ_Q4_K> {           // sub-blocks 2j, 2j+1 of a super-block
  u32x4 hd, q0, q1;
  static __device__ int voff(int sl) { return (sl >> 2) * 144; }
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int j) {
    hd = bld16(r, vo, 0);
    q0 = bld16(r, vo + 32 * j, 16);
    q1 = bld16(r, vo + 32 * j, 32);
  }
  template <bool ASM>
  __device__ float dot(int h, const float* x, const float* xs, int j) const {
    const u32x4 q = h ? q1 : q0;              // sub-block 2j + h
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {             // low nibbles: elements 4k.., high: 16+4k..
      const uint32_t u = q[k] >> 8;           // high nibbles stay in place: 16 q
      s = dot4mix(q[k] & 0x000F000Fu, u & 0x000F000Fu, x + 4 * k, s);
      t = dot4mix(q[k] & 0x00F000F0u, u & 0x00F000F0u, x + 16 + 4 * k, t);
    }
    // (scale, min) of sub-blocks 2j, 2j+1: the 24 bits at bit 24j of the
    // 96-bit field stream in header bytes 4..15
    const uint32_t lo = (j <= 1) ? hd.y : (j == 2) ? hd.z : hd.w;
    const uint32_t hi = (j <= 1) ? hd.z : hd.w;
    const uint32_t f = __builtin_amdgcn_alignbit(hi, lo, (24 * j) & 31) >> (12 * h);
    const float a = h2f(hd.x) * (float)(f & 63u) * kSub;
    const float b = h2f(hd.x >> 16) * (float)((f >> 6) & 63u);
    return fmaf(a, fmaf(t, 0.0625f, s), -b * (xs[0] + xs[1]));
  }
};

template <> struct Slice<GQ_Q6_K> {           // 32-weight groups 2j, 2j+1
  u32x4 l0, l1, h;
  uint32_t sc, d;
  static __device__ int voff(int sl) { return (sl >> 2) * 210; }
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int j) {
    l0 = bld16(r, vo + 32 * j, 18);
    l1 = bld16(r, vo + 32 * j, 34);
    h = bld16(r, vo + 16 * j, 146);
    sc = bld4(r, vo + 4 * j, 2);
    d = bld2(r, vo, 0);
  }
  template <bool ASM>
  __device__ float dot(int g, const float* x, const float*, int) const {
    // group 2j + g; codes q = low4 | high2 << 4 turned into the signed bytes
    // q - 32, so every product (q - 32) * x carries only its own rounding
    // (summing q * x and 32 * x apart would lose the difference of two
    // large sums); per 16-weight quarter sc * sum((q - 32) * x)
    const u32x4 L = g ? l1 : l0;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t H = h[2 * g + (k & 1)];
      const uint32_t lo = (L[k] & 0x0F0F0F0Fu) | q6k_hi(H, k >> 1);
      const uint32_t hi = ((L[k] >> 4) & 0x0F0F0F0Fu) | q6k_hi(H, 2 + (k >> 1));
      s0 = dot4s_asm(centre<32>(lo), x + 4 * k, s0);
      s1 = dot4s_asm(centre<32>(hi), x + 16 + 4 * k, s1);
    }
    const uint32_t sc2 = sc >> (16 * g);
    return h2f(d) * fmaf(sb1(sc2), s1, sb0(sc2) * s0);
  }
};

template <> struct Slice<GQ_Q8_0> {           // blocks 2*sl, 2*sl+1
  u32x4 c[4];
  uint32_t d0, d1;
  static __device__ int voff(int sl) { return sl * 68; }
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int) {
    d0 = bld2(r, vo, 0);
    c[0] = bld16(r, vo, 2);
    c[1] = bld16(r, vo, 18);
    d1 = bld2(r, vo, 34);
    c[2] = bld16(r, vo, 36);
    c[3] = bld16(r, vo, 52);
  }
  template <bool ASM>
  __device__ float dot(int h, const float* x, const float*, int) const {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      a = dot4s_<ASM>(c[2 * h][k], x + 4 * k, a);
      b = dot4s_<ASM>(c[2 * h + 1][k], x + 16 + 4 * k, b);
    }
    return h2f(h ? d1 : d0) * (a + b);
  }
};

// Q4_0 and Q5_0: low nibbles are elements 0..15 of a block, high nibbles
// 16..31 ("How LLM Inference Engines Work", "Loading GGUF Models"); Q5_0 adds
// a fifth bit per element from a 32-bit word.
template <int T> struct SliceQ40Q50 {
  static constexpr bool Q5 = (T == GQ_Q5_0);
  static constexpr int BB = Q5 ? 22 : 18;
  static constexpr int OFF = Q5 ? 16 : 8;
  u32x4 q0, q1;
  uint32_t d0, d1, h0, h1;
  static __device__ int voff(int sl) { return sl * 2 * BB; }
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int) {
    d0 = bld2(r, vo, 0);
    d1 = bld2(r, vo, BB);
    q0 = bld16(r, vo, Q5 ? 6 : 2);
    q1 = bld16(r, vo, BB + (Q5 ? 6 : 2));
    h0 = Q5 ? bld4(r, vo, 2) : 0u;
    h1 = Q5 ? bld4(r, vo, BB + 2) : 0u;
  }
  template <bool ASM>
  __device__ float dot(int h, const float* x, const float*, int) const {
    const u32x4 q = h ? q1 : q0;
    const uint32_t qh = h ? h1 : h0;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      uint32_t lo = q[k] & 0x0F0F0F0Fu, hi = (q[k] >> 4) & 0x0F0F0F0Fu;
      if (Q5) {
        lo |= spread4_bit4(qh >> (4 * k));
        hi |= spread4_bit4(qh >> (16 + 4 * k));
      }
      a = dot4s_<ASM>(centre<OFF>(lo), x + 4 * k, a);
      b = dot4s_<ASM>(centre<OFF>(hi), x + 16 + 4 * k, b);
    }
    return h2f(h ? d1 : d0) * (a + b);
  }
};
template <> struct Slice<GQ_Q4_0> : SliceQ40Q50<GQ_Q4_0> {};
template <> struct Slice<GQ_Q5_0> : SliceQ40Q50<GQ_Q5_0> {};

// acc + w0 x[0] + w1 x[1] + w2 x[2] + w3 x[3] with w_i = RNE_fp32(c_i a + m)
// exactly the stated dequant of codes c_i (16-bit fields: c0, c2 in p02, c1,
// c3 in p13, read as the fp16 subnormals c 2^-24) for a scale a24 = a 2^24:
// one mixed FMA forms each weight with its single rounding, one FMA
// multiplies it into the sum, so every product carries only its own
// rounding.
__device__ __forceinline__ float dot4w(uint32_t p02, uint32_t p13, float a24, float m, const float* x,
                                       float acc) {
  float w0, w1, w2, w3;
  asm("v_fma_mix_f32 %0, %4, %6, %7 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %1, %5, %6, %7 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %2, %4, %6, %7 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %3, %5, %6, %7 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
      : "v"(p02), "v"(p13), "v"(a24), "v"(m));
  acc = fmaf(w0, x[0], acc);
  acc = fmaf(w1, x[1], acc);
  acc = fmaf(w2, x[2], acc);
  return fmaf(w3, x[3], acc);
}

// Q4_1 (blocks 2 sl, 2 sl + 1): fp16 d, fp16 m, 16 code bytes in Q4_0 order;
// each weight d q + m is formed exactly as stated, then multiplied.
template <> struct Slice<GQ_Q4_1> {
  u32x4 a0, a1;                              // bytes 0..15 of each block
  uint32_t t0, t1;                           // bytes 16..19
  static __device__ int voff(int sl) { return sl * 40; }
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int) {
    a0 = bld16(r, vo, 0);
    t0 = bld4(r, vo, 16);
    a1 = bld16(r, vo, 20);
    t1 = bld4(r, vo, 36);
  }
  template <bool ASM>
  __device__ float dot(int h, const float* x, const float*, int) const {
    const u32x4 A = h ? a1 : a0;
    const uint32_t c[4] = {A.y, A.z, A.w, h ? t1 : t0};   // code bytes 0..15
    const float a24 = h2f(A.x) * kSub, m = h2f(A.x >> 16);
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {            // low nibbles: elements 4k.., high: 16+4k..
      const uint32_t u = c[k] >> 8;
      s = dot4w(c[k] & 0x000F000Fu, u & 0x000F000Fu, a24, m, x + 4 * k, s);
      t = dot4w((c[k] >> 4) & 0x000F000Fu, (u >> 4) & 0x000F000Fu, a24, m, x + 16 + 4 * k, t);
    }
    return s + t;
  }
};

// Q5_K (sub-blocks 2j, 2j+1): Q4_K's header, 8 bytes of fifth bits for the
// slice's 64 elements, 5-bit codes as bytes; factored sub-block sums as Q4_K.
template <> struct Slice<GQ_Q5_K> {
  u32x4 hd, q0, q1;
  u32x2 qh;
  static __device__ int voff(int sl) { return (sl >> 2) * 176; }
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int j) {
    hd = bld16(r, vo, 0);
    qh = bld8(r, vo + 8 * j, 16);
    q0 = bld16(r, vo + 32 * j, 48);
    q1 = bld16(r, vo + 32 * j, 64);
  }
  template <bool ASM>
  __device__ float dot(int h, const float* x, const float* xs, int j) const {
    const u32x4 q = h ? q1 : q0;              // sub-block 2j + h
    const uint32_t W = h ? qh.y : qh.x;       // its fifth bits, bit e = element e
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t lo = (q[k] & 0x0F0F0F0Fu) | bits_to_b4(W >> (4 * k));
      const uint32_t hi = ((q[k] >> 4) & 0x0F0F0F0Fu) | bits_to_b4(W >> (16 + 4 * k));
      s = dot4u_asm(lo, x + 4 * k, s);
      s = dot4u_asm(hi, x + 16 + 4 * k, s);
    }
    const uint32_t lo = (j <= 1) ? hd.y : (j == 2) ? hd.z : hd.w;
    const uint32_t hi = (j <= 1) ? hd.z : hd.w;
    const uint32_t f = __builtin_amdgcn_alignbit(hi, lo, (24 * j) & 31) >> (12 * h);
    const float a = h2f(hd.x) * (float)(f & 63u);
    const float b = h2f(hd.x >> 16) * (float)((f >> 6) & 63u);
    return fmaf(a, s, -b * (xs[0] + xs[1]));
  }
};

// Q2_K (quarter j of a super-block: 16-weight sub-blocks 4j..4j+3, 32-weight
// groups 2j, 2j+1): d | dmin, the quarter's four scale/min bytes and its 16
// code bytes.  Byte k of a group holds elements k + 8u at bits 2u; masked in
// place, bit pair u is the fp16 subnormal 4^u q 2^-24, so one mixed FMA per
// weight forms its product (powers of two undo the 4^u); factored
// sub-block sums as Q4_K, a*sum(q*x) - b*sum(x) per 16 weights.
template <> struct Slice<GQ_Q2_K> {
  uint32_t dm, sm;
  u32x4 q;
  static __device__ int voff(int sl) { return (sl >> 2) * 84; }
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int j) {
    dm = bld4(r, vo, 0);
    sm = bld4(r, vo + 4 * j, 4);
    q = bld16(r, vo + 16 * j, 20);
  }
  template <bool ASM>
  __device__ float dot(int h, const float* x, const float* xs, int) const {
    float s[4] = {0.f, 0.f, 0.f, 0.f};        // bit pair u: elements 8u .. 8u+7
#pragma unroll
    for (int c = 0; c < 2; c++) {             // bytes 4c .. 4c+3 of group 2j + h
      const uint32_t lo = q[2 * h + c], hi = lo >> 8;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const uint32_t m = 0x00030003u << (2 * u);
        s[u] = dot4mix(lo & m, hi & m, x + 4 * c + 8 * u, s[u]);
      }
    }
    // sub-blocks 4j + 2h (elements 0..15 of the group) and 4j + 2h + 1
    const uint32_t b0 = sm >> (16 * h), b1 = sm >> (16 * h + 8);
    const float d = h2f(dm) * kSub, dmin = h2f(dm >> 16);
    const float a0 = d * (float)(b0 & 15u), a1 = d * (float)(b1 & 15u);
    const float m0 = dmin * (float)((b0 >> 4) & 15u), m1 = dmin * (float)((b1 >> 4) & 15u);
    const float t0 = fmaf(s[1], 0.25f, s[0]), t1 = fmaf(s[3], 0.015625f, s[2] * 0.0625f);
    return fmaf(a0, t0, -m0 * xs[0]) + fmaf(a1, t1, -m1 * xs[1]);
  }
};

// Q3_K (quarter j: sub-blocks 4j..4j+3): d, the quarter's four scale fields
// (24 bits of the 96-bit stream), 16 low-bit plane bytes and 64 third bits;
// each code becomes the signed byte q - 4, so every product (q - 4) * x
// carries only its own rounding (as Q6_K); per 16 weights sc * sum.
template <> struct Slice<GQ_Q3_K> {
  uint32_t d, sc;
  u32x4 q;
  u32x2 qh;
  static __device__ int voff(int sl) { return (sl >> 2) * 110; }
  __device__ void load(__amdgpu_buffer_rsrc_t r, int vo, int j) {
    d = bld2(r, vo, 0);
    sc = bld4(r, vo + 3 * j, 2);              // fields 4j.. start at bit 24j
    q = bld16(r, vo + 16 * j, 14);
    qh = bld8(r, vo + 8 * j, 78);
  }
  template <bool ASM>
  __device__ float dot(int h, const float* x, const float*, int) const {
    const uint32_t H = h ? qh.y : qh.x;       // bit e: element e of group 2j + h
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int c = 0; c < 2; c++) {
      const uint32_t w = q[2 * h + c];        // plane bytes 4c .. 4c+3
#pragma unroll
      for (int u = 0; u < 4; u++) {           // elements 4c + 8u .. +3
        const uint32_t v = plane2(w, u) | bits_to_b2(H >> (4 * c + 8 * u));
        if (u < 2) s0 = dot4s_asm(centre<4>(v), x + 4 * c + 8 * u, s0);
        else s1 = dot4s_asm(centre<4>(v), x + 4 * c + 8 * u, s1);
      }
    }
    const uint32_t f = sc >> (12 * h);        // fields 4j + 2h, 4j + 2h + 1
    return h2f(d) * fmaf((float)((f >> 6) & 63u), s1, (float)(f & 63u) * s0);
  }
};

// Physical float index in LDS of logical x index f: 16-byte chunk c of slice
// s lands at chunk c ^ (s & 15), so 16 lanes reading chunk c of 16
// consecutive slices hit 16 distinct groups of 4 banks.
__device__ __forceinline__ int xswz(int f) {
  const int s = f >> 6, c = (f >> 2) & 15;
  return (s << 6) | ((c ^ (s & 15)) << 2) | (f & 3);
}

// Persistent GEMV.  LPR lanes cover a row's slices in each of npass passes
// (a wave holds 64/LPR rows side by side when rows are short); each wave takes
// R such row sets per group and walks its groups pass by pass, so the double
// buffer holds one pass whatever the row length.
// Decode-layer fusions (template F): F_NORM normalizes x (RMSNorm): fp32 x
// stages x * gamma and scales each row's sum by the norm at the end (no
// extra barrier: the per-wave sums of squares ride on the staging barrier),
// fp16 x stages RNE_fp16(x * s) * gamma after one more barrier; F_GLU walks a
// second matrix of the same shape (after a row group's passes over blob,
// the same passes over blob2) and stores silu(first sum) * second sum.
// A workgroup has W waves sharing one copy of x (W = 8 for long rows, where
// x's LDS would otherwise cap the resident waves below what registers allow).
constexpr int F_NORM = 1, F_GLU = 2;

template <int T, bool XF16, int LPR, int R, int XPT, bool XFIRST, int F = 0, int W = 4>
__global__ void __launch_bounds__(64 * W) k_gemv(const uint8_t* __restrict__ blob, int rows,
                                              int cols, int rb, const void* __restrict__ xv,
                                              float* __restrict__ y,
                                              const uint8_t* __restrict__ blob2 = nullptr,
                                              const float* __restrict__ gamma = nullptr,
                                              float eps = 0.f) {
  extern __shared__ float xsm[];           // x padded to whole slices, then 16-column sums
  constexpr bool NORM = (F & F_NORM) != 0, GLU = (F & F_GLU) != 0;
  static_assert(!GLU || R == 1, "the gated form walks one row set through both matrices");
  constexpr int RPW = 64 / LPR;            // rows side by side in a wave
  constexpr int ROWS = RPW * R;            // rows per group
  // XPT = float4 of x staged per thread: cols <= XPT * 256 * W
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int nsl = (cols + 63) >> 6;        // slices per row (the last may be half)
  const int npass = (nsl + LPR - 1) / LPR;
  const int NP = GLU ? 2 * npass : npass;  // passes per group (GLU: gate, then up)
  const int cpad = nsl << 6;
  const int ngroups = (rows + ROWS - 1) / ROWS;
  const int stride = gridDim.x * W;
  const int sub = lane / LPR;              // which of the side-by-side rows
  const int li = lane % LPR;

  // x from global first (clamped, unconditional loads), then the first pass's
  // weights, then x into LDS: the LDS stores wait only for x
  const int nc4 = cols >> 2;
  f32x4 xr[XPT], gr[NORM ? XPT : 1];
#pragma unroll
  for (int i = 0; i < XPT; i++) {
    const int cc = min((int)threadIdx.x + 64 * W * i, nc4 - 1);
    if constexpr (XF16) {
      u32x2 hh = *reinterpret_cast<const u32x2*>((const _Float16*)xv + 4 * cc);
      xr[i] = f32x4{h2f(hh.x), h2f(hh.x >> 16), h2f(hh.y), h2f(hh.y >> 16)};
    } else {
      xr[i] = reinterpret_cast<const f32x4*>(xv)[cc];
    }
    if constexpr (NORM) gr[i] = reinterpret_cast<const f32x4*>(gamma)[cc];
  }

  Slice<T> cur[R];
  // loads pass p of group grp into w; lanes past the row's last slice repeat
  // it (their sums are dropped); the descriptor ends at the matrix's last row
  auto load_item = [&](Slice<T> (&w)[R], int grp, int p) {
    const bool up = GLU && p >= npass;
    const int sl = min((up ? p - npass : p) * LPR + li, nsl - 1);
    const int vo = Slice<T>::voff(sl);
#pragma unroll
    for (int k = 0; k < R; k++) {
      const int rw0 = uniform(grp * ROWS + k * RPW);
      const int nr = max(0, min(RPW, rows - rw0));
      const uint8_t* const b = up ? blob2 : blob;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(b + (int64_t)rw0 * rb, (uint32_t)(nr * rb));
      w[k].load(rs, sub * rb + vo, sl & 3);
    }
  };
  // A wave's first two items: requested before x is staged when the waves
  // have many (the weight stream then starts at launch, and x's loads, issued
  // first, are the only ones the staging waits for), after it when they
  // have few (x then reaches every CU ahead of the weight traffic, and the
  // kernel's span is the x latency plus one or two items' work).
  int g = blockIdx.x * W + wave;
  Slice<T> nxt[R] = {};
  auto first_two = [&]() {
    if (g < ngroups) load_item(cur, g, 0);
    if (g < ngroups && (NP > 1 || g + stride < ngroups)) {
      if (NP > 1) load_item(nxt, g, 1);
      else load_item(nxt, g + stride, 0);
    }
  };
  if constexpr (!XFIRST) first_two();

  // RMSNorm ("How LLM Inference Engines Work", "RMSNorm"): s = rsqrt(mean(x^2)
  // + eps) in fp32, x' = (x * s rounded to x's type) * gamma.  Every
  // workgroup forms the sum of squares itself: per thread, then the DPP
  // network, then the W waves in order through LDS.  In fp32, sum w x' =
  // s * sum w (x gamma), so fp32 x stages x * gamma now and the rows take s
  // at the end; fp16 x must be rounded after scaling, so it waits for s.
  float* xsum = xsm + cpad;
  float* const part = xsum + (cpad >> 4);    // W floats after the column sums
  auto norm_scale = [&]() {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < W; i += 4) tot += (part[i] + part[i + 1]) + (part[i + 2] + part[i + 3]);
    return 1.f / sqrtf(tot / (float)cols + eps);
  };
  if constexpr (NORM) {
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < XPT; i++) {
      const int c4 = (int)threadIdx.x + 64 * W * i;
      const f32x4 v = (c4 < nc4) ? xr[i] : f32x4{0.f, 0.f, 0.f, 0.f};
      q += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    }
    q = group_sum_dpp<64>(q);                // the wave's total in lane 63
    if (lane == 63) part[wave] = q;
    if constexpr (XF16) {
      __syncthreads();
      const float sc = norm_scale();
#pragma unroll
      for (int i = 0; i < XPT; i++)
#pragma unroll
        for (int e = 0; e < 4; e++) xr[i][e] = (float)(_Float16)(xr[i][e] * sc) * gr[i][e];
    } else {
#pragma unroll
      for (int i = 0; i < XPT; i++)
#pragma unroll
        for (int e = 0; e < 4; e++) xr[i][e] *= gr[i][e];
    }
  }
  // x (fp32, zero-padded to whole slices) into LDS; each quad of lanes holds
  // one 16-column group, summed on the DPP network
#pragma unroll
  for (int i = 0; i < XPT; i++) {
    const int c4 = (int)threadIdx.x + 64 * W * i;
    const f32x4 v = (c4 < nc4) ? xr[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    float s = (v.x + v.y) + (v.z + v.w);
    s += dpp_mov<0xB1>(s);
    s += dpp_mov<0x4E>(s);
    if (c4 < (cpad >> 2)) {
      *reinterpret_cast<f32x4*>(xsm + xswz(4 * c4)) = v;
      if ((c4 & 3) == 0) xsum[c4 >> 2] = s;
    }
  }
  __syncthreads();
  if constexpr (XFIRST) first_two();
  constexpr bool LATE = NORM && !XF16;       // rows scaled by the norm at the end
  const float rs = LATE ? norm_scale() : 1.f;

  bool first = true;
  for (; g < ngroups; g += stride) {
    float acc[R], acc_up = 0.f;
#pragma unroll
    for (int k = 0; k < R; k++) acc[k] = 0.f;
    for (int p = 0; p < NP; p++) {
      // next item: this group's next pass, else the next group's first
      const bool more = (p + 1 < NP) || (g + stride < ngroups);
      if (more && !first) {
        if (p + 1 < NP) load_item(nxt, g, p + 1);
        else load_item(nxt, g + stride, 0);
      }
      first = false;
      const bool up = GLU && p >= npass;     // uniform: the second matrix's passes
      const int s0 = (up ? p - npass : p) * LPR + li;
      const int s = min(s0, nsl - 1);
      const bool live = s0 < nsl;
      const bool second = (2 * s + 1) * 32 < cols;   // the slice's second half is in the row
#pragma unroll
      for (int h = 0; h < 2; h++) {
        float x[32];
        const float* base = xsm + (s << 6);
#pragma unroll
        for (int c = 0; c < 8; c++) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(base + (((8 * h + c) ^ (s & 15)) << 2));
          x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
        }
        const float2 xs2 = *reinterpret_cast<const float2*>(xsum + 4 * s + 2 * h);
        const float xs[2] = {xs2.x, xs2.y};
        const bool use = live && (h == 0 || second);
#pragma unroll
        for (int k = 0; k < R; k++) {
          // two row sets: convert + FMA pairs kept together (see dot4u_asm)
          const float d = cur[k].template dot<(R > 1)>(h, x, xs, s & 3);
          if (GLU && up)
            acc_up += use ? d : 0.f;
          else
            acc[k] += use ? d : 0.f;
        }
      }
      // unconditional: without a next item the loops end here and cur is dead
#pragma unroll
      for (int k = 0; k < R; k++) cur[k] = nxt[k];
    }
    if constexpr (GLU) {
      // SwiGLU ("How LLM Inference Engines Work", "SwiGLU Feed-Forward
      // Network"): silu(gate) * up, silu(v) = v / (1 + exp(-v)), in fp32
      float gt = group_sum_dpp<LPR>(acc[0]), up = group_sum_dpp<LPR>(acc_up);
      if constexpr (LATE) { gt *= rs; up *= rs; }
      const int r = g * ROWS + sub;
      if (li == LPR - 1 && r < rows) y[r] = gt / (1.f + expf(-gt)) * up;
    } else {
#pragma unroll
      for (int k = 0; k < R; k++) {
        float v = group_sum_dpp<LPR>(acc[k]);              // valid in lane LPR-1 of each group
        if constexpr (LATE) v *= rs;
        const int r = g * ROWS + k * RPW + sub;
        if (li == LPR - 1 && r < rows) y[r] = v;
      }
    }
  }
}

#ifndef GQ_GEMV_R                 // row sets per wave when a row takes one pass
#define GQ_GEMV_R 1
#endif
#ifndef GQ_GEMV_W                 // waves per workgroup for rows of up to 8192
#define GQ_GEMV_W 4
#endif
#ifndef GQ_GEMV_LONG_W            // waves per workgroup for longer rows
#define GQ_GEMV_LONG_W 8
#endif

// Compute units of device dev, and workgroups of kern that fit on one at
// once, at most max_wps waves per SIMD (4 SIMDs per CU).
template <typename K>
static void resident_wgs(K kern, int dev, int threads, size_t lds, int max_wps, int& cus, int& per) {
  cus = 0;
  per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, (const void*)kern, threads, lds) != hipSuccess ||
      per < 1)
    per = 1;
  const int lim = max_wps * 4 * 64 / threads;
  if (per > lim) per = lim > 0 ? lim : 1;
}

// Fusion arguments of a decode-layer launch (all optional).
struct Fuse {
  const void* blob2;                       // up-projection weights: SwiGLU output
  const float* gamma;                      // RMSNorm weights: x is normalized first
  float eps;
};

template <int T, bool XF16, int LPR, int R, int XPT, int F, int W = 4>
static hipError_t gemv_launch(const void* blob, int64_t rows, int64_t cols, const void* x,
                              float* y, const Fuse& fu, hipStream_t st) {
  constexpr int RR = (F & F_GLU) ? 1 : R;
  const int64_t rb = cols / Geo<T>::QK * Geo<T>::BB;
  const int64_t cpad = (cols + 63) / 64 * 64;
  // x, its 16-column sums and W per-wave partial sums: <= 68 KB for cols <= 16384
  const size_t lds = (size_t)cpad * 4 + (size_t)(cpad / 16) * 4 + 4 * W;
  auto kern = k_gemv<T, XF16, LPR, RR, XPT, false, F, W>;
  // resident workgroups for the last (device, LDS size) this host thread
  // launched with (both orders use the same registers); per thread, so
  // concurrent callers share nothing
  struct Occ {
    int dev;
    size_t lds;
    int cus, per;
  };
  thread_local Occ occ = {-1, 0, 1, 1};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  // Rows longer than 8192 weights: one 8-wave workgroup per CU.  Each wave
  // then walks two or more rows, and the CU stages x (up to 64 KB) once
  // instead of twice (measured on MI355X: Q6_K 4096x11008 12.9 -> 12.0 us,
  // 4096x14336 15.5 -> 14.2 us, Q8_0 4096x11008 14.3 -> 13.1 us).
#ifndef GQ_GEMV_LONG_WPS
#define GQ_GEMV_LONG_WPS 2
#endif
  constexpr int kMaxWps = (W >= 8) ? GQ_GEMV_LONG_WPS : 16;
  if (occ.dev != dev || occ.lds != lds) {
    occ.dev = dev;
    occ.lds = lds;
    resident_wgs(kern, dev, 64 * W, lds, kMaxWps, occ.cus, occ.per);
  }
  const int64_t rpg = (64 / LPR) * RR;     // rows per group
  const int64_t groups = (rows + rpg - 1) / rpg;
  const int64_t wgs = (groups + W - 1) / W;
  const int64_t cap = (int64_t)occ.cus * occ.per;
  dim3 grid((unsigned)(wgs < cap ? wgs : cap));   // wgs >= 1, cap >= 1
  // items of the wave with the most: x goes first when that is at most 2
  const int64_t npass = ((cols + 63) / 64 + LPR - 1) / LPR * ((F & F_GLU) ? 2 : 1);
  const int64_t most = (groups + W * (int64_t)grid.x - 1) / (W * (int64_t)grid.x) * npass;
  const uint8_t* b2 = (const uint8_t*)fu.blob2;
  if (most <= 2)
    hipLaunchKernelGGL((k_gemv<T, XF16, LPR, RR, XPT, true, F, W>), grid, dim3(64 * W), lds, st,
                       (const uint8_t*)blob, (int)rows, (int)cols, (int)rb, x, y, b2, fu.gamma,
                       fu.eps);
  else
    hipLaunchKernelGGL(kern, grid, dim3(64 * W), lds, st, (const uint8_t*)blob, (int)rows,
                       (int)cols, (int)rb, x, y, b2, fu.gamma, fu.eps);
  return hipGetLastError();
}

// Shape dispatch: rows of up to 2048 weights share a wave (64/LPR of them);
// longer rows take several passes of 64 slices.  Rows of up to 4096 weights
// take R row sets per wave, longer ones one.  Rows of more than 8192 weights
// take 8-wave workgroups: with 4, x's LDS (> 32 KB) leaves fewer waves
// resident than registers allow, and e.g. 4096 rows then spread unevenly
// (some waves two rows, some one).
template <int T, bool XF16, int F>
static hipError_t gemv_pick(const void* blob, int64_t rows, int64_t cols, const void* x, float* y,
                            const Fuse& fu, hipStream_t st) {
  constexpr int W = GQ_GEMV_W, LW = GQ_GEMV_LONG_W;
  if (cols <= 1024) return gemv_launch<T, XF16, 16, GQ_GEMV_R, 16 / W, F, W>(blob, rows, cols, x, y, fu, st);
  if (cols <= 2048) return gemv_launch<T, XF16, 32, GQ_GEMV_R, 16 / W, F, W>(blob, rows, cols, x, y, fu, st);
  if (cols <= 4096) return gemv_launch<T, XF16, 64, GQ_GEMV_R, 16 / W, F, W>(blob, rows, cols, x, y, fu, st);
  if (cols <= 8192) return gemv_launch<T, XF16, 64, 1, 32 / W, F, W>(blob, rows, cols, x, y, fu, st);
  return gemv_launch<T, XF16, 64, 1, 64 / LW, F, LW>(blob, rows, cols, x, y, fu, st);
}

template <int T, int F>
static hipError_t gemv_f(const void* blob, int64_t rows, int64_t cols, const void* x, bool xf16,
                         float* y, const Fuse& fu, hipStream_t st) {
  return xf16 ? gemv_pick<T, true, F>(blob, rows, cols, x, y, fu, st)
              : gemv_pick<T, false, F>(blob, rows, cols, x, y, fu, st);
}

template <int T>
static hipError_t gemv_t(const void* blob, int64_t rows, int64_t cols, const void* x, bool xf16,
                         float* y, const Fuse& fu, hipStream_t st) {
  const int f = (fu.gamma ? F_NORM : 0) | (fu.blob2 ? F_GLU : 0);
  switch (f) {
    case 0: return gemv_f<T, 0>(blob, rows, cols, x, xf16, y, fu, st);
    case F_NORM: return gemv_f<T, F_NORM>(blob, rows, cols, x, xf16, y, fu, st);
    case F_GLU: return gemv_f<T, F_GLU>(blob, rows, cols, x, xf16, y, fu, st);
    default: return gemv_f<T, F_NORM | F_GLU>(blob, rows, cols, x, xf16, y, fu, st);
  }
}

hipError_t launch_gemv(int type, const void* blob, int64_t rows, int64_t cols, const void* x,
                       bool x_f16, float* y, hipStream_t st) {
  return launch_gemv_fused(type, blob, nullptr, rows, cols, x, x_f16, nullptr, 0.f, y, st);
}

hipError_t launch_gemv_fused(int type, const void* blob, const void* up_blob, int64_t rows,
                             int64_t cols, const void* x, bool x_f16, const float* norm_weight,
                             float eps, float* y, hipStream_t st) {
  const Fuse fu{up_blob, norm_weight, eps};
  switch (type) {
    case GQ_Q4_0: return gemv_t<GQ_Q4_0>(blob, rows, cols, x, x_f16, y, fu, st);
    case GQ_Q5_0: return gemv_t<GQ_Q5_0>(blob, rows, cols, x, x_f16, y, fu, st);
    case GQ_Q8_0: return gemv_t<GQ_Q8_0>(blob, rows, cols, x, x_f16, y, fu, st);
    case GQ_Q4_K: return gemv_t<GQ_Q4_K>(blob, rows, cols, x, x_f16, y, fu, st);
    case GQ_Q6_K: return gemv_t<GQ_Q6_K>(blob, rows, cols, x, x_f16, y, fu, st);
    case GQ_Q4_1: return gemv_t<GQ_Q4_1>(blob, rows, cols, x, x_f16, y, fu, st);
    case GQ_Q5_K: return gemv_t<GQ_Q5_K>(blob, rows, cols, x, x_f16, y, fu, st);
    case GQ_Q2_K: return gemv_t<GQ_Q2_K>(blob, rows, cols, x, x_f16, y, fu, st);
    case GQ_Q3_K: return gemv_t<GQ_Q3_K>(blob, rows, cols, x, x_f16, y, fu, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gq
