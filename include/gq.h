/*
 * gq.h — C ABI of libgq: matrix-vector and small-batch matrix multiplication
 * over GGUF block-quantized weights on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The pages describe GGUF weights stored as blocks, each
 * with its own fp16 scale ("Hitchhiker's Guide — Lab 01", §11.1, w ~= d*q),
 * Q4_K super-blocks of 256 weights in 8 sub-blocks of 32 with 6-bit scales
 * and mins under an fp16 super-scale and super-min (§11.2, dequant formula
 * w = (d*sc)*q - dmin*m; "12 — llama.cpp / GGUF", section "Q4_K_M — bit layout
 * in exquisite detail"), and the Q4_K_M recipe mixing Q4_K, Q5_0, Q6_K and
 * Q8_0 blocks that are dequantized inside the dot product ("Local LLM
 * inference", section "The mmap backend").  This library computes
 *
 *     y[t][r] = sum_c  W^[r][c] * x[t][c]      for t < n_tok, r < rows
 *
 * where W^ is the dequantized weight matrix.  Decode is memory-bound: each
 * weight is read once per call ("The bandwidth cap", 12 — llama.cpp / GGUF).
 *
 * Conventions shared by every entry point:
 *  - W is row-major: row r is the byte range [r*RB, (r+1)*RB) of the blob,
 *    RB = gq_row_bytes(type, cols); blocks are contiguous within a row.
 *    rows = output features, cols = input features (as in nn.Linear).
 *  - x is [n_tok][cols], y is [n_tok][rows], both row-major, contiguous.
 *  - Pointers marked "device" are HIP device (or managed) pointers; the
 *    library never allocates, frees, or keeps caller memory.
 *  - stream is a hipStream_t passed as void*; NULL is the null stream.  All
 *    work is enqueued asynchronously; the library never synchronizes, so
 *    device faults surface at the caller's next synchronization.
 *  - All argument checks run on the host before any HIP call; on a failed
 *    check nothing is enqueued.  Return value 0 is success, else a GQ_E* code.
 *  - NaN or Inf in a block's scales propagates into y; it is not an error.
 *  - The library is stateless and reentrant; calls may run concurrently on
 *    different streams.
 */
#ifndef GQ_H
#define GQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block types.  The numbering is this library's own. */
enum {
    GQ_F32  = 0,   /* activations / outputs only */
    GQ_F16  = 1,   /* activations / outputs only */
    GQ_Q4_0 = 2,   /* 32 weights, 18 B:  fp16 d, 16 B codes; w = d*(q-8) */
    GQ_Q5_0 = 3,   /* 32 weights, 22 B:  fp16 d, u32 fifth bits, 16 B codes; w = d*(q-16) */
    GQ_Q8_0 = 4,   /* 32 weights, 34 B:  fp16 d, 32 int8 codes; w = d*q */
    GQ_Q4_K = 5,   /* 256 weights, 144 B: fp16 d, fp16 dmin, 12 B 6-bit sc/m, 128 B codes */
    GQ_Q6_K = 6,   /* 256 weights, 210 B: fp16 d, 16 int8 scales, 128 B low, 64 B high bits */
    GQ_Q4_1 = 7,   /* 32 weights, 20 B:  fp16 d, fp16 m, 16 B codes; w = d*q + m */
    GQ_Q5_K = 8,   /* 256 weights, 176 B: Q4_K's fields, 32 B fifth bits, 128 B codes */
    GQ_Q2_K = 9,   /* 256 weights, 84 B: fp16 d, fp16 dmin, 16 B 4-bit sc/m, 64 B 2-bit codes */
    GQ_Q3_K = 10   /* 256 weights, 110 B: fp16 d, 12 B 6-bit sc, 64 B low 2 bits, 32 B third bits */
};

/* Error codes. */
enum {
    GQ_OK            = 0,
    GQ_EINVAL_TYPE   = -1,  /* unknown or unsupported type / x_type / out_type */
    GQ_EINVAL_SHAPE  = -2,  /* rows < 1, cols < 1, cols % block size, n_tok < 0 */
    GQ_EINVAL_PTR    = -3,  /* null pointer, or input and output ranges overlap */
    GQ_EALIGN        = -4,  /* a pointer is not 16-byte aligned */
    GQ_EOVERFLOW     = -5,  /* sizes beyond the supported range (see below) */
    GQ_EHIP          = -6   /* a HIP launch failed (the HIP error is consumed) */
};

/*
 * Byte layouts (all fields little-endian; readings where the pages are
 * silent are marked R):
 *  Q4_0: d @0; qs[16] @2; element j<16 = qs[j] & 15, j>=16 = qs[j-16] >> 4
 *        ("How LLM Inference Engines Work", "Loading GGUF Models").
 *  Q8_0: d @0; int8 q[32] @2 (R: two's complement).
 *  Q5_0: d @0; u32 qh @2, bit j = bit 4 of code j; qs[16] @6 as Q4_0 (R).
 *  Q4_K: d @0; dmin @2; scales[12] @4 = 16 six-bit fields, field k at bits
 *        6k..6k+5 of the 96-bit little-endian stream (R), sub-block i uses
 *        field 2i as scale and 2i+1 as min; qs[128] @16, sub-block i owns
 *        bytes 16i..16i+15 in Q4_0 nibble order (R).
 *        w = (d*sc_i)*q - dmin*m_i.
 *  Q6_K: d @0; int8 scales[16] @2 (one per 16 weights); ql[128] @18, group g
 *        of 32 owns bytes 16g..16g+15 in Q4_0 nibble order; qh[64] @146, byte
 *        8g+k holds bits 4..5 of elements 32g+k+8u at bits 2u..2u+1 (R).
 *        w = d*(sc*(q-32)).
 *  Q4_1: d @0; m @2 (signed); qs[16] @4 as Q4_0 (R: "How LLM Inference
 *        Engines Work", "Loading GGUF Models" names the type only).
 *        w = d*q + m.
 *  Q5_K: Q4_K's d, dmin, scales[12] @0..15; qh[32] @16, bit e of the 256-bit
 *        little-endian field = bit 4 of element e's code; qs[128] @48 as in
 *        Q4_K (R: 5.5 bpw, "Other k-quants at a glance").  q in 0..31,
 *        w = (d*sc_i)*q - dmin*m_i.
 *  Q2_K: d @0; dmin @2; 16 bytes @4, byte s = scale (low nibble) and min
 *        (high nibble) of the 16 weights 16s..16s+15; qs[64] @20, byte 8g+k
 *        holds the 2-bit codes of elements 32g+k+8u at bits 2u..2u+1 (R: 2.625
 *        bpw, "Other k-quants at a glance").  w = (d*sc_s)*q - dmin*m_s.
 *  Q3_K: d @0; 16 six-bit scales @2 in Q4_K's 96-bit stream (field s for
 *        weights 16s..16s+15); low 2 bits of the codes @14 in Q2_K's order;
 *        32 bytes @78, bit e = bit 2 of element e's code (R: 3.4375 bpw, same
 *        table).  w = d*(sc_s*(q-4)), q in 0..7.
 *
 * Limits: rows, cols and n_tok below 2^31; rows*RB, n_tok*cols and
 * n_tok*rows below 2^47; cols <= 16384 at n_tok = 1 (x is staged in 64 KB of
 * LDS); cols <= 2^21 at n_tok >= 2 (a tile of 128 tokens of x is addressed
 * with 31-bit offsets); n_tok <= 2^22; rows*cols <= 2^40 for gq_dequant and gq_quantize.
 * Beyond a limit the call returns GQ_EOVERFLOW.
 */

/* Weights per block and bytes per block of `type` (host only, no HIP call).
 * Either output pointer may be NULL. */
int gq_type_info(int type, int64_t *block_elems, int64_t *block_bytes);

/* Bytes per row for `cols` weights of `type`; a negative GQ_E* code on a bad
 * type or a cols that is not a whole number of blocks (host only). */
int64_t gq_row_bytes(int type, int64_t cols);

/* Static, human-readable text for an error code. */
const char *gq_strerror(int code);

/*
 * y = W^ x with fp32 activations.  Equivalent to gq_matmul_ex(..., GQ_F32, ...).
 *   weight_blob  device, rows*RB bytes, 16-B aligned, read only
 *   x            device, fp32 [n_tok][cols], 16-B aligned, read only
 *   y            device, fp32 [n_tok][rows], 16-B aligned, overwritten
 * n_tok = 0 is a successful no-op.  x and y must not overlap each other or
 * the blob.  Accumulation is fp32 throughout (the pages warn that fp16
 * accumulation overflows: "How LLM Inference Engines Work", "Quantization").
 */
int gq_matmul(const void *weight_blob, int ggml_type, int64_t rows, int64_t cols,
              const void *x, float *y, int64_t n_tok, void *stream);

/*
 * As gq_matmul, with x_type GQ_F32 or GQ_F16 giving the activation format.
 * For n_tok >= 2 the weights are decoded once per call and reused for every
 * token ("Local LLM inference", "The mmap backend": decode each projection
 * weight once per input batch) on the matrix cores.  fp32 activations are then
 * scaled by an exact power of two 2^k per token (and per 256-column slab in
 * the weight-stream kernel, per running maximum in the tiled GEMM) that puts
 * the largest |x| near 2^10..2^14, split into two fp16 parts, hi =
 * RNE_fp16(x 2^k) and lo = RNE_fp16(x 2^k - hi), both multiplied, and the
 * fp32 results multiplied by 2^-k: any finite fp32 magnitude is accepted,
 * about 22 of x's 24 significant bits are kept, and only values more than
 * 2^17 below the largest |x| of their scope lose relative precision (each
 * with an absolute error below 2^-34 of that largest |x|).  fp16 activations
 * are used as given.  In the weight-stream kernel (up to 32 tokens, and past
 * that when estimated faster) the decoded weights enter the products as
 * exact integers (scaled by d and dmin in fp32), except Q6_K's sc*(q-32),
 * rounded to fp16 when its magnitude exceeds 2048; in the tiled GEMM each
 * weight enters as RNE_fp16(w 2^r) of its fp32 dequant w, with a power of
 * two 2^r per weight row that follows the largest magnitude its blocks'
 * fields allow (so every finite block scale is accepted).  Either way the
 * relative error of a product is at most 2^-11.  Q4_K's min term is summed
 * apart from its scale term (w = a*q - b gives a*sum(q*x) - b*sum(x) in the
 * batch-1 GEMV and the weight-stream kernel), so on blocks where a*q and b
 * nearly cancel the error is relative to sum(|a|*q*|x| + |b|*|x|) rather
 * than to sum|w*x|; blocks a quantizer makes do not come near that.
 */
int gq_matmul_ex(const void *weight_blob, int ggml_type, int64_t rows, int64_t cols,
                 const void *x, int x_type, float *y, int64_t n_tok, void *stream);

/*
 * gq_matmul_ex with the kernel family chosen by the caller (for tests,
 * tuning and callers that know their shapes):
 *   GQ_PATH_AUTO           what gq_matmul_ex does: n_tok = 1 -> the batch-1
 *                          GEMV; up to 32 tokens -> the weight-stream
 *                          kernel; more -> the tiled matrix-core GEMM, or
 *                          the weight-stream kernel over ceil(n_tok / 64)
 *                          near-equal chunks when a cost estimate (the
 *                          GEMM's tiles walk the whole K range each, so
 *                          with few tiles it leaves CUs idle) says that is
 *                          faster;
 *   GQ_PATH_GEMV           n_tok must be 1;
 *   GQ_PATH_WEIGHT_STREAM  n_tok >= 2, in chunks of at most 64 tokens;
 *   GQ_PATH_TILED          n_tok >= 2, the tiled GEMM.
 * Results differ between paths only within the stated tolerance; each path
 * is deterministic.  A path that does not fit n_tok, or an unknown path:
 * GQ_EINVAL_SHAPE.  Other errors as for gq_matmul_ex.
 */
enum { GQ_PATH_AUTO = 0, GQ_PATH_GEMV = 1, GQ_PATH_WEIGHT_STREAM = 2, GQ_PATH_TILED = 3 };
int gq_matmul_path(const void *weight_blob, int ggml_type, int64_t rows, int64_t cols,
                   const void *x, int x_type, float *y, int64_t n_tok, int path, void *stream);

/*
 * One decode token through a transformer sublayer's projection, with the
 * steps on either side fused into the same launch:
 *   xin = norm_weight ? RMSNorm(x) : x, where RMSNorm follows "How LLM
 *         Inference Engines Work", section "RMSNorm": s = rsqrt(mean_c x[c]^2
 *         + eps) in fp32, xin[c] = (x[c] * s, rounded to fp16 when x is fp16)
 *         * norm_weight[c];
 *   y   = up_blob ? silu(W^ xin) * (U^ xin) : W^ xin, elementwise over the
 *         rows, silu(v) = v / (1 + exp(-v)) in fp32 (same page, "SwiGLU
 *         Feed-Forward Network": the gate projection through SiLU times the
 *         up projection).
 *   weight_blob  device, rows*RB bytes (the gate weights when up_blob is set)
 *   up_blob      device or NULL, a second blob of the same type and shape
 *   x            device, one token: fp32 or fp16 [cols] (x_type), read only
 *   norm_weight  device fp32 [cols] or NULL; eps >= 0 and finite
 *   y            device, fp32 [rows], overwritten; must not overlap the inputs
 * All pointers given are 16-byte aligned; cols <= 16384.  The sum of squares
 * is formed in fp32 by every workgroup in a fixed order, so the result is the
 * same on every run.  Errors as for gq_matmul_ex (a bad eps: GQ_EINVAL_SHAPE).
 */
int gq_matmul_decode(const void *weight_blob, const void *up_blob, int ggml_type, int64_t rows,
                     int64_t cols, const void *x, int x_type, const float *norm_weight,
                     float eps, float *y, void *stream);

/*
 * Dequantize the whole blob into out[rows][cols] (device, 16-B aligned).
 *   out_type GQ_F32: bit-exact with the stated fp32 operation order: Q4_K,
 *     Q5_K and Q2_K form a = d*sc and b = dmin*m in fp32 (exact) and round
 *     once in a*q - b; Q6_K and Q3_K form the integer sc*(q-32) or
 *     sc*(q-4) and multiply by d (exact); Q4_1 rounds once in d*q + m (d*q
 *     exact); the other 32-weight types compute d*(q - offset) (exact).
 *   out_type GQ_F16: round-to-nearest-even of that fp32 value.
 */
int gq_dequant(const void *weight_blob, int ggml_type, int64_t rows, int64_t cols,
               void *out, int out_type, void *stream);

/*
 * Quantize fp32 w[rows][cols] (device) into a blob (device, rows*RB bytes),
 * all arithmetic in fp64: symmetric absmax blocks for Q4_0 / Q5_0 / Q8_0 and
 * for Q6_K's 16-weight sub-blocks, min/scale sub-blocks for Q4_K ("two-level
 * scaling" and "asymmetric quantization", Hitchhiker's Guide §11.2; Q5_K
 * the same with 31 levels, Q2_K over 16-weight sub-blocks with 3 levels and
 * 4-bit fields, Q3_K as Q6_K with codes -3..3 and 6-bit scales, Q4_1 a min
 * rounded down to fp16 and a covering scale per block); stored
 * fp16 scales are rounded up so every weight is covered, codes are rounded
 * half away from zero.  Weights whose block scale would exceed the largest
 * finite fp16 saturate.  Used to make blobs from fp32 weights on the device.
 */
int gq_quantize(const float *w, int ggml_type, int64_t rows, int64_t cols,
                void *weight_blob, void *stream);

/*
 * One decode step of grouped-query attention over a KV cache stored as q8_0
 * or q4_0 blocks ("How LLM Inference Engines Work", section "Grouped-Query
 * Attention (GQA) and KV Cache"; the cache types of the Hitchhiker's Guide
 * §13.2).  For query head h and its KV head g = h / (n_heads / n_kv_heads):
 *     s[t]   = (sum_c q[h][c] * K^[t][g][c]) / sqrt(head_dim)     in fp32
 *     out[h] = sum_t softmax(s)[t] * V^[t][g]                     in fp32
 * over the cached positions t < kv_len, K^ and V^ the dequantized caches.
 *   k_cache, v_cache  device, [kv_len][n_kv_heads][head_dim] as a blob of
 *                     kv_len*n_kv_heads rows of head_dim weights quantized
 *                     along head_dim (row (t, g) = t*n_kv_heads + g,
 *                     gq_row_bytes(kv_type, head_dim) bytes each); read only
 *   kv_type           GQ_Q8_0 or GQ_Q4_0 (both caches)
 *   head_dim          64, 128 or 256; n_heads a multiple of n_kv_heads with
 *                     at most 16 query heads per KV head; kv_len >= 1
 *   q                 device fp32 [n_heads][head_dim]; out device fp32
 *                     [n_heads][head_dim], overwritten
 *   workspace         device, at least gq_attn_decode_workspace_bytes(...)
 *                     bytes (per-chunk softmax statistics), contents ignored
 *                     and overwritten; one per concurrent call
 * All pointers 16-byte aligned; out and workspace overlap nothing else.  Each
 * cache must stay within 0x7FFF0000 bytes (GQ_EOVERFLOW).  The result does not
 * depend on the run: positions are split into fixed chunks and combined in
 * order.
 */
int64_t gq_attn_decode_workspace_bytes(int64_t kv_len, int n_kv_heads, int n_heads,
                                       int head_dim);
int gq_attn_decode(const void *k_cache, const void *v_cache, int kv_type, int64_t kv_len,
                   int n_kv_heads, int head_dim, const float *q, int n_heads, float *out,
                   void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gq_attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and result, with the workspace taken from a fixed
 * array of GQ_ATTN_NOALLOC_SCRATCH_BYTES in device memory that the library
 * holds on every GPU it runs on until the process ends.  The call allocates
 * and frees nothing.  Arguments as for gq_attn_decode without the
 * workspace; the work runs on the stream's device (the current device for a
 * NULL stream).  A call whose workspace would exceed the array
 * (gq_attn_decode_workspace_bytes > GQ_ATTN_NOALLOC_SCRATCH_BYTES) returns
 * GQ_EOVERFLOW before any HIP call; a failure to find the array's device
 * address returns GQ_EHIP.  All calls on one GPU share its array: calls that
 * may overlap in time on one GPU (different streams, or host threads without
 * ordering) race and must not be issued; calls in one stream are ordered and
 * safe.  Nothing in the array needs to start at any value.
 */
#define GQ_ATTN_NOALLOC_SCRATCH_BYTES (32 << 20)
int gq_attn_decode_noalloc(const void *k_cache, const void *v_cache, int kv_type,
                           int64_t kv_len, int n_kv_heads, int head_dim, const float *q,
                           int n_heads, float *out, void *stream);

/*
 * Measurement: a plain streaming read of `bytes` bytes of device memory at
 * buf with non-temporal 128-bit loads, every byte read once, nothing else done.  Its
 * bandwidth is the practical ceiling the GEMV kernels' effective bandwidth
 * is read against (no kernel reaches the nominal HBM peak).  So that the
 * reads cannot be dropped, out (device, GQ_PROBE_OUT_WORDS 32-bit words,
 * overwritten) receives per-workgroup XORs of the buffer's 32-bit words:
 * the XOR of all of out equals the XOR of all of buf's words.
 *   buf    device, 16-byte aligned; bytes a multiple of 16, at most 2^30
 *          (GQ_EINVAL_SHAPE / GQ_EOVERFLOW otherwise); with bytes = 0 buf
 *          may be NULL and out is all zeros
 *   out    device, 16-byte aligned, must not overlap buf
 */
#define GQ_PROBE_OUT_WORDS 2048
int gq_probe_stream_read(const void *buf, int64_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* GQ_H */
