// gq_launch.h — host-side launchers implemented by the kernel files.
// Arguments are already validated by gq_api.cpp when these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

hipError_t launch_dequant(int type, const void* blob, int64_t rows, int64_t cols, void* out,
                          bool f16_out, hipStream_t st);
hipError_t launch_quantize(int type, const float* w, int64_t rows, int64_t cols, void* blob,
                           hipStream_t st);
// One token (n_tok == 1): the bandwidth-bound GEMV family.
hipError_t launch_gemv(int type, const void* blob, int64_t rows, int64_t cols, const void* x,
                       bool x_f16, float* y, hipStream_t st);
// One token with decode-layer fusions: RMSNorm of x first (norm_weight not
// null), and/or silu(W x) * (U x) out (up_blob not null, same type and shape).
hipError_t launch_gemv_fused(int type, const void* blob, const void* up_blob, int64_t rows,
                             int64_t cols, const void* x, bool x_f16, const float* norm_weight,
                             float eps, float* y, hipStream_t st);
// Streaming read of bytes (<= 2^30, a multiple of 16) into per-workgroup
// XORs, GQ_PROBE_OUT_WORDS of them.
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t st);
// Decode attention over a q8_0 / q4_0 KV cache ([kv_len][n_kv][head_dim],
// head_dim 64, 128 or 256, n_heads / n_kv <= 16): split over chunks of
// positions, partial statistics in workspace (attn_workspace_bytes), then
// combined.
struct AttnPlan {
  int chunk;
  int64_t n_chunks;
};
AttnPlan attn_plan(int64_t kv_len, int n_kv, int n_rep, int head_dim);
int64_t attn_workspace_bytes(int64_t kv_len, int n_kv, int n_heads, int head_dim);
hipError_t launch_attn_decode(int kv_type, const void* k_cache, const void* v_cache,
                              int64_t kv_len, int n_kv, int head_dim, const float* q,
                              int n_heads, float* out, float* workspace, hipStream_t st);
// Small batches: the weight stream on the matrix cores, 16 tokens per pass.
hipError_t launch_mmv(int type, const void* blob, int64_t rows, int64_t cols, const void* x,
                      bool x_f16, float* y, int64_t n_tok, hipStream_t st);
// Prefill-sized batches: tiled fp16 GEMM with the weights decoded per tile.
hipError_t launch_gemm(int type, const void* blob, int64_t rows, int64_t cols, const void* x,
                       bool x_f16, float* y, int64_t n_tok, hipStream_t st);
// The GEMM's tile shape (rows x tokens, K groups per tile):
//   0 = 256 x 128, 1 = 128 x 128, 2 = 128 x 64, 3 = 32 x 64 in 4 K groups,
//   4 = 64 x 64 in 4 K groups, 5 = 64 x 128 in 2 K groups;
// and the estimated time of the launch in microseconds.
int gemm_tile_config(int type, int64_t rows, int64_t cols, int64_t n_tok, bool x_f16);
double gemm_estimate_us(int type, int64_t rows, int64_t cols, int64_t n_tok, bool x_f16);
}  // namespace gq
