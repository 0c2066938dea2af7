/*
 * gqo.h — CPU oracle for GGUF block-quantized matmul.  TEST INFRASTRUCTURE ONLY.
 *
 * This header belongs to the oracle alone.  Only tests/, the smoke check and the
 * CPU-baseline leg of bench.py load the library built from gqo.c.  The GPU library
 * shares no code, header, table or helper with it.
 *
 * All pointers are host pointers owned by the caller.  Every function returns 0 on
 * success and a negative value on a bad argument (unknown type, shape not a whole
 * number of blocks, null pointer).
 *
 * Type codes (this project's own numbering; the pages give none):
 *   0 F32, 1 F16, 2 Q4_0, 3 Q5_0, 4 Q8_0, 5 Q4_K, 6 Q6_K, 7 Q4_1, 8 Q5_K, 9 Q2_K,
 *   10 Q3_K
 */
#ifndef GQO_H
#define GQO_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { GQO_F32 = 0, GQO_F16 = 1, GQO_Q4_0 = 2, GQO_Q5_0 = 3, GQO_Q8_0 = 4,
       GQO_Q4_K = 5, GQO_Q6_K = 6, GQO_Q4_1 = 7, GQO_Q5_K = 8, GQO_Q2_K = 9,
       GQO_Q3_K = 10 };

/* Weights per block and bytes per block of a quantized type. */
int gqo_block_info(int type, int64_t *block_elems, int64_t *block_bytes);

/* fp16 helpers, written from the IEEE binary16 definition. */
double   gqo_half_to_double(uint16_t h);
uint16_t gqo_half_up(double v);     /* smallest finite fp16 >= v, v >= 0; 0x7C00 if none */
uint16_t gqo_half_rne(float f);     /* round-to-nearest-even fp32 -> fp16 */

/* Quantize row-major fp32 w[rows][cols] into a blob of rows*(cols/QK) blocks. */
int gqo_quantize(int type, const float *w, int64_t rows, int64_t cols, uint8_t *blob);

/* Dequantize a blob.  _f32 follows the stated fp32 operation order; _f64 is exact. */
int gqo_dequant_f32(int type, const uint8_t *blob, int64_t rows, int64_t cols, float *out);
int gqo_dequant_f64(int type, const uint8_t *blob, int64_t rows, int64_t cols, double *out);

/*
 * y[t][r] = sum_c W^[r][c] * x[t][c] in fp64 (dequant-then-dot, sequential over c).
 * yabs[t][r] = sum_c |W^[r][c] * x[t][c]| (the tolerance scale); yabs may be NULL.
 * threads <= 0 means one thread.  Rows are split over OpenMP threads only.
 */
int gqo_matmul_f64(int type, const uint8_t *blob, int64_t rows, int64_t cols,
                   const double *x, int64_t n_tok, double *y, double *yabs, int threads);

/*
 * RMSNorm of one vector ("How LLM Inference Engines Work", "RMSNorm"):
 * s = 1/sqrt(mean_c x[c]^2 + eps), out[c] = (x[c]*s) * w[c] in fp64, except
 * that with half_x the product x[c]*s is first rounded to fp16 (through fp32),
 * as the page casts it back to an fp16 input's type.
 */
int gqo_rmsnorm_f64(const double *x, int64_t cols, const double *w, double eps, int half_x,
                    double *out);

/* SwiGLU output (same page, "SwiGLU Feed-Forward Network"):
 * out[i] = silu(g[i]) * u[i], silu(v) = v / (1 + exp(-v)), in fp64. */
int gqo_swiglu_f64(const double *g, const double *u, int64_t n, double *out);

/*
 * One decode step of grouped-query attention over a block-quantized KV cache
 * ("How LLM Inference Engines Work", "Grouped-Query Attention (GQA) and KV
 * Cache"; Hitchhiker's Guide §13.2 for q8_0 / q4_0 caches), in fp64:
 *   for query head h, g = h / (n_heads / n_kv):
 *     s[t]   = (sum_c q[h][c] * K^[t][g][c]) / sqrt(head_dim),   t < kv_len
 *     out[h] = sum_t softmax(s)[t] * V^[t][g]
 * k_cache, v_cache: [kv_len][n_kv][head_dim] blobs, each (t, g) row of
 * head_dim quantized along head_dim (reading R13).  q, out: [n_heads][head_dim].
 */
int gqo_attn_decode_f64(int type, const uint8_t *k_cache, const uint8_t *v_cache, int64_t kv_len,
                        int64_t n_kv, int64_t head_dim, const double *q, int64_t n_heads,
                        double *out);

#ifdef __cplusplus
}
#endif
#endif
