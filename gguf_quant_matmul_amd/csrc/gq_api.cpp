// gq_api.cpp — the C ABI declared in include/gq.h: argument validation on the
// host, then dispatch to the kernel families.  Every check runs before the
// first HIP call, so the validation is testable on a machine with no GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/gq.h"
#include "gq_launch.h"

namespace {

constexpr int64_t kDim = (int64_t)1 << 31;       // rows, cols, n_tok < 2^31
constexpr int64_t kBytes = (int64_t)1 << 47;     // any one buffer < 2^47 bytes
constexpr int64_t kMaxColsGemv = 16384;          // x staged in 64 KB of LDS
constexpr int64_t kMaxColsBatch = (int64_t)1 << 21;  // n_tok >= 2: 128 tokens of x in 31-bit offsets
constexpr int64_t kMaxTokens = (int64_t)1 << 22;  // matrix-core grid.y = n_tok / 64 < 65536
constexpr int64_t kSmallBatch = 64;               // tokens per weight-stream launch at most
constexpr int64_t kStreamOnly = 32;               // n_tok up to this: always the weight stream
constexpr int64_t kMaxElems = (int64_t)1 << 40;   // dequant / quantize grid.x < 2^31
constexpr int64_t kMaxCacheBytes = 0x7FFF0000;    // KV caches: below the kernels' out-of-range offset

bool quant_type(int t) { return t >= GQ_Q4_0 && t <= GQ_Q3_K; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int check_matrix(int type, int64_t rows, int64_t cols, int64_t* rb) {
  if (!quant_type(type)) return GQ_EINVAL_TYPE;
  if (rows < 1 || cols < 1) return GQ_EINVAL_SHAPE;
  if (rows >= kDim || cols >= kDim) return GQ_EOVERFLOW;
  int64_t r = gq_row_bytes(type, cols);
  if (r < 0) return (int)r;
  if (rows > kBytes / r) return GQ_EOVERFLOW;
  *rb = r;
  return GQ_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GQ_OK : GQ_EHIP; }

// Past 32 tokens: the matrix-core GEMM walks every tile's whole K range, so
// its time is ~ rounds of resident tiles x K steps x step time (its own
// estimate, by tile shape), while the weight-stream kernel's time grows with
// the number of 16-token passes: measured on MI355X, a pass streams
// rows*cols weights at ~150 (Q4_K, Q5_K, Q2_K, Q3_K; Q6_K ~165, the 32-weight
// types ~80) TFLOP/s.  The batch goes to the
// weight-stream kernel, in ceil(n/64) near-equal chunks of at most 64 tokens,
// when that estimate is lower.
bool small_batch_chunks_faster(int type, int64_t rows, int64_t cols, int64_t n_tok, bool x_f16) {
  const double rate = (type == GQ_Q4_K || type == GQ_Q5_K || type == GQ_Q2_K || type == GQ_Q3_K)
                          ? 150e12
                          : (type == GQ_Q6_K) ? 165e12 : 80e12;
  // fp32 x (hi + lo parts through the matrix ops) measured ~2.5x the fp16
  // figures on the tiled GEMM and ~1.9x on the weight stream (Q4_K 11008x4096
  // at 64 tokens: 95 against 70 us)
  const double gemm_us = gq::gemm_estimate_us(type, rows, cols, n_tok, x_f16) * (x_f16 ? 1.0 : 2.5);
  const double pass_us = (double)rows * (double)cols * 32.0 / rate * 1e6 * (x_f16 ? 1.0 : 1.9);
  const int64_t k = (n_tok + 63) / 64, base = n_tok / k, extra = n_tok % k;
  const int64_t passes = extra * ((base + 16) / 16) + (k - extra) * ((base + 15) / 16);
  // every chunk after the first is a launch of its own, whose start follows
  // the previous launch's tail (~2 us measured: Q4_K 4096x4096 at 80 / 96
  // tokens take 25.7 / 26.1 us on the weight stream against 20.8 / 21.2
  // tiled, while Q6_K 4096x14336 at 100 tokens takes 81 against 86)
  const double mmv_us = (double)passes * pass_us + 2.0 * (double)(k - 1);
  return mmv_us < gemm_us;
}

}  // namespace

extern "C" {

int gq_type_info(int type, int64_t* block_elems, int64_t* block_bytes) {
  int64_t qk, bb;
  switch (type) {
    case GQ_F32:  qk = 1;   bb = 4;   break;
    case GQ_F16:  qk = 1;   bb = 2;   break;
    case GQ_Q4_0: qk = 32;  bb = 18;  break;
    case GQ_Q5_0: qk = 32;  bb = 22;  break;
    case GQ_Q8_0: qk = 32;  bb = 34;  break;
    case GQ_Q4_K: qk = 256; bb = 144; break;
    case GQ_Q6_K: qk = 256; bb = 210; break;
    case GQ_Q4_1: qk = 32;  bb = 20;  break;
    case GQ_Q5_K: qk = 256; bb = 176; break;
    case GQ_Q2_K: qk = 256; bb = 84;  break;
    case GQ_Q3_K: qk = 256; bb = 110; break;
    default: return GQ_EINVAL_TYPE;
  }
  if (block_elems) *block_elems = qk;
  if (block_bytes) *block_bytes = bb;
  return GQ_OK;
}

int64_t gq_row_bytes(int type, int64_t cols) {
  int64_t qk, bb;
  int rc = gq_type_info(type, &qk, &bb);
  if (rc) return rc;
  if (cols < 1 || cols % qk) return GQ_EINVAL_SHAPE;
  if (cols >= kDim) return GQ_EOVERFLOW;
  return cols / qk * bb;
}

const char* gq_strerror(int code) {
  switch (code) {
    case GQ_OK: return "success";
    case GQ_EINVAL_TYPE: return "unknown or unsupported type";
    case GQ_EINVAL_SHAPE: return "invalid shape (rows/cols < 1, cols not a whole number of blocks, or n_tok < 0)";
    case GQ_EINVAL_PTR: return "null pointer or overlapping input/output ranges";
    case GQ_EALIGN: return "pointer not 16-byte aligned";
    case GQ_EOVERFLOW: return "size beyond the supported range";
    case GQ_EHIP: return "HIP launch failed";
  }
  return "unknown error code";
}

int gq_matmul_path(const void* weight_blob, int ggml_type, int64_t rows, int64_t cols,
                   const void* x, int x_type, float* y, int64_t n_tok, int path, void* stream) {
  int64_t rb = 0;
  int rc = check_matrix(ggml_type, rows, cols, &rb);
  if (rc) return rc;
  if (x_type != GQ_F32 && x_type != GQ_F16) return GQ_EINVAL_TYPE;
  if (n_tok < 0) return GQ_EINVAL_SHAPE;
  if (path < GQ_PATH_AUTO || path > GQ_PATH_TILED) return GQ_EINVAL_SHAPE;
  if (path == GQ_PATH_GEMV && n_tok != 1) return GQ_EINVAL_SHAPE;
  if ((path == GQ_PATH_WEIGHT_STREAM || path == GQ_PATH_TILED) && n_tok < 2 && n_tok != 0)
    return GQ_EINVAL_SHAPE;
  if (n_tok >= kDim) return GQ_EOVERFLOW;
  if (n_tok == 0) return GQ_OK;
  if (n_tok == 1 && cols > kMaxColsGemv) return GQ_EOVERFLOW;
  if (n_tok >= 2 && cols > kMaxColsBatch) return GQ_EOVERFLOW;
  if (n_tok > kMaxTokens) return GQ_EOVERFLOW;
  if (n_tok > kBytes / cols || n_tok > kBytes / rows) return GQ_EOVERFLOW;
  if (!weight_blob || !x || !y) return GQ_EINVAL_PTR;
  if (!aligned16(weight_blob) || !aligned16(x) || !aligned16(y)) return GQ_EALIGN;
  const int64_t xbytes = n_tok * cols * (x_type == GQ_F16 ? 2 : 4);
  const int64_t ybytes = n_tok * rows * 4;
  const int64_t wbytes = rows * rb;
  if (overlap(x, xbytes, y, ybytes) || overlap(weight_blob, wbytes, y, ybytes))
    return GQ_EINVAL_PTR;
  hipStream_t st = (hipStream_t)stream;
  const bool xf16 = (x_type == GQ_F16);
  if (n_tok == 1) return hip_status(gq::launch_gemv(ggml_type, weight_blob, rows, cols, x, xf16, y, st));
  if (path == GQ_PATH_AUTO)
    path = (n_tok <= kStreamOnly || small_batch_chunks_faster(ggml_type, rows, cols, n_tok, xf16))
               ? GQ_PATH_WEIGHT_STREAM
               : GQ_PATH_TILED;
  if (path == GQ_PATH_TILED)
    return hip_status(gq::launch_gemm(ggml_type, weight_blob, rows, cols, x, xf16, y, n_tok, st));
  // weight stream: ceil(n / 64) near-equal chunks of at most 64 tokens
  const int64_t xrow = cols * (xf16 ? 2 : 4);
  const int64_t k = (n_tok + kSmallBatch - 1) / kSmallBatch, base = n_tok / k;
  for (int64_t c = 0, t0 = 0; c < k; c++) {
    const int64_t nc = base + (c < n_tok % k ? 1 : 0);
    const hipError_t e = gq::launch_mmv(ggml_type, weight_blob, rows, cols,
                                        (const uint8_t*)x + t0 * xrow, xf16, y + t0 * rows, nc, st);
    if (e != hipSuccess) return GQ_EHIP;
    t0 += nc;
  }
  return GQ_OK;
}

int gq_matmul_ex(const void* weight_blob, int ggml_type, int64_t rows, int64_t cols,
                 const void* x, int x_type, float* y, int64_t n_tok, void* stream) {
  return gq_matmul_path(weight_blob, ggml_type, rows, cols, x, x_type, y, n_tok, GQ_PATH_AUTO,
                        stream);
}

int gq_matmul(const void* weight_blob, int ggml_type, int64_t rows, int64_t cols, const void* x,
              float* y, int64_t n_tok, void* stream) {
  return gq_matmul_ex(weight_blob, ggml_type, rows, cols, x, GQ_F32, y, n_tok, stream);
}

int gq_matmul_decode(const void* weight_blob, const void* up_blob, int ggml_type, int64_t rows,
                     int64_t cols, const void* x, int x_type, const float* norm_weight, float eps,
                     float* y, void* stream) {
  int64_t rb = 0;
  int rc = check_matrix(ggml_type, rows, cols, &rb);
  if (rc) return rc;
  if (x_type != GQ_F32 && x_type != GQ_F16) return GQ_EINVAL_TYPE;
  if (cols > kMaxColsGemv) return GQ_EOVERFLOW;
  if (!(eps >= 0.f) || eps > 3.4e38f) return GQ_EINVAL_SHAPE;   // NaN and inf included
  if (!weight_blob || !x || !y) return GQ_EINVAL_PTR;
  if (!aligned16(weight_blob) || !aligned16(x) || !aligned16(y) ||
      (up_blob && !aligned16(up_blob)) || (norm_weight && !aligned16(norm_weight)))
    return GQ_EALIGN;
  const int64_t xbytes = cols * (x_type == GQ_F16 ? 2 : 4);
  const int64_t ybytes = rows * 4;
  const int64_t wbytes = rows * rb;
  if (overlap(x, xbytes, y, ybytes) || overlap(weight_blob, wbytes, y, ybytes) ||
      (up_blob && overlap(up_blob, wbytes, y, ybytes)) ||
      (norm_weight && overlap(norm_weight, cols * 4, y, ybytes)))
    return GQ_EINVAL_PTR;
  return hip_status(gq::launch_gemv_fused(ggml_type, weight_blob, up_blob, rows, cols, x,
                                          x_type == GQ_F16, norm_weight, eps, y,
                                          (hipStream_t)stream));
}

static int check_attn_shape(int64_t kv_len, int n_kv_heads, int n_heads, int head_dim) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return GQ_EINVAL_SHAPE;
  if (kv_len < 1 || n_kv_heads < 1 || n_heads < n_kv_heads || n_heads % n_kv_heads ||
      n_heads / n_kv_heads > 16)
    return GQ_EINVAL_SHAPE;
  if (n_kv_heads > 65535 || kv_len >= kDim) return GQ_EOVERFLOW;
  return GQ_OK;
}

int64_t gq_attn_decode_workspace_bytes(int64_t kv_len, int n_kv_heads, int n_heads,
                                       int head_dim) {
  int rc = check_attn_shape(kv_len, n_kv_heads, n_heads, head_dim);
  if (rc) return rc;
  return gq::attn_workspace_bytes(kv_len, n_kv_heads, n_heads, head_dim);
}

// Checks shared by the attention entry points: everything but the
// workspace.  need receives the workspace bytes the call takes.
static int check_attn(const void* k_cache, const void* v_cache, int kv_type, int64_t kv_len,
                      int n_kv_heads, int head_dim, const float* q, int n_heads, const float* out,
                      int64_t* need) {
  if (kv_type != GQ_Q8_0 && kv_type != GQ_Q4_0) return GQ_EINVAL_TYPE;
  int rc = check_attn_shape(kv_len, n_kv_heads, n_heads, head_dim);
  if (rc) return rc;
  const int64_t rb = gq_row_bytes(kv_type, head_dim);
  // loads past the chunk's last position go to a byte offset no cache
  // reaches (they read as zero), so the caches stay below that offset
  if (kv_len > kMaxCacheBytes / ((int64_t)n_kv_heads * rb)) return GQ_EOVERFLOW;
  *need = gq::attn_workspace_bytes(kv_len, n_kv_heads, n_heads, head_dim);
  if (!k_cache || !v_cache || !q || !out) return GQ_EINVAL_PTR;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(out))
    return GQ_EALIGN;
  const int64_t cbytes = kv_len * n_kv_heads * rb;
  const int64_t qbytes = (int64_t)n_heads * head_dim * 4;
  if (overlap(out, qbytes, q, qbytes) || overlap(out, qbytes, k_cache, cbytes) ||
      overlap(out, qbytes, v_cache, cbytes))
    return GQ_EINVAL_PTR;
  return GQ_OK;
}

int gq_attn_decode(const void* k_cache, const void* v_cache, int kv_type, int64_t kv_len,
                   int n_kv_heads, int head_dim, const float* q, int n_heads, float* out,
                   void* workspace, int64_t workspace_bytes, void* stream) {
  int64_t need = 0;
  int rc = check_attn(k_cache, v_cache, kv_type, kv_len, n_kv_heads, head_dim, q, n_heads, out,
                      &need);
  if (rc) return rc;
  if (workspace_bytes < need) return GQ_EINVAL_SHAPE;
  if (!workspace) return GQ_EINVAL_PTR;
  if (!aligned16(workspace)) return GQ_EALIGN;
  const int64_t rb = gq_row_bytes(kv_type, head_dim);
  const int64_t cbytes = kv_len * n_kv_heads * rb;
  const int64_t qbytes = (int64_t)n_heads * head_dim * 4;
  if (overlap(out, qbytes, workspace, need) || overlap(workspace, need, q, qbytes) ||
      overlap(workspace, need, k_cache, cbytes) || overlap(workspace, need, v_cache, cbytes))
    return GQ_EINVAL_PTR;
  return hip_status(gq::launch_attn_decode(kv_type, k_cache, v_cache, kv_len, n_kv_heads,
                                           head_dim, q, n_heads, out, (float*)workspace,
                                           (hipStream_t)stream));
}

}  // extern "C"

// Workspace of gq_attn_decode_noalloc: a fixed array in device memory.  The
// runtime gives every GPU the library runs on its own copy when it loads the
// code object, held until the process ends.  In host code the name is only
// a stand-in for the symbol: the device address of a GPU's copy comes from
// hipGetSymbolAddress with that GPU current, looked up once per device.
constexpr int64_t kScratchBytes = GQ_ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of device dev's copy of scratch, or null on a HIP error.
void* scratch_on(int dev) {
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
  if (e != hipSuccess || !addr) return nullptr;
  g_scratch_ptr[dev].store(addr, std::memory_order_release);
  return addr;
}
}  // namespace

extern "C" {

int gq_attn_decode_noalloc(const void* k_cache, const void* v_cache, int kv_type, int64_t kv_len,
                           int n_kv_heads, int head_dim, const float* q, int n_heads, float* out,
                           void* stream) {
  int64_t need = 0;
  int rc = check_attn(k_cache, v_cache, kv_type, kv_len, n_kv_heads, head_dim, q, n_heads, out,
                      &need);
  if (rc) return rc;
  if (need > kScratchBytes) return GQ_EOVERFLOW;
  // the GPU the work runs on: the stream's, or the current one for NULL
  hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  if ((st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess) return GQ_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return GQ_EHIP;
  void* ws = scratch_on(dev);
  if (!ws) return GQ_EHIP;
  return hip_status(gq::launch_attn_decode(kv_type, k_cache, v_cache, kv_len, n_kv_heads,
                                           head_dim, q, n_heads, out, (float*)ws, st));
}

int gq_probe_stream_read(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
  if (bytes < 0 || bytes % 16) return GQ_EINVAL_SHAPE;
  if (bytes > ((int64_t)1 << 30)) return GQ_EOVERFLOW;
  if (!out || (bytes > 0 && !buf)) return GQ_EINVAL_PTR;
  if (!aligned16(buf) || !aligned16(out)) return GQ_EALIGN;
  if (overlap(buf, bytes, out, GQ_PROBE_OUT_WORDS * 4)) return GQ_EINVAL_PTR;
  return hip_status(gq::launch_stream_read(buf, bytes, out, (hipStream_t)stream));
}

int gq_dequant(const void* weight_blob, int ggml_type, int64_t rows, int64_t cols, void* out,
               int out_type, void* stream) {
  int64_t rb = 0;
  int rc = check_matrix(ggml_type, rows, cols, &rb);
  if (rc) return rc;
  if (out_type != GQ_F32 && out_type != GQ_F16) return GQ_EINVAL_TYPE;
  if (rows > kMaxElems / cols) return GQ_EOVERFLOW;
  if (!weight_blob || !out) return GQ_EINVAL_PTR;
  if (!aligned16(weight_blob) || !aligned16(out)) return GQ_EALIGN;
  const int64_t obytes = rows * cols * (out_type == GQ_F16 ? 2 : 4);
  if (overlap(weight_blob, rows * rb, out, obytes)) return GQ_EINVAL_PTR;
  return hip_status(gq::launch_dequant(ggml_type, weight_blob, rows, cols, out,
                                       out_type == GQ_F16, (hipStream_t)stream));
}

int gq_quantize(const float* w, int ggml_type, int64_t rows, int64_t cols, void* weight_blob,
                void* stream) {
  int64_t rb = 0;
  int rc = check_matrix(ggml_type, rows, cols, &rb);
  if (rc) return rc;
  if (rows > kMaxElems / cols) return GQ_EOVERFLOW;
  if (!w || !weight_blob) return GQ_EINVAL_PTR;
  if (!aligned16(w) || !aligned16(weight_blob)) return GQ_EALIGN;
  if (overlap(w, rows * cols * 4, weight_blob, rows * rb)) return GQ_EINVAL_PTR;
  return hip_status(gq::launch_quantize(ggml_type, w, rows, cols, weight_blob, (hipStream_t)stream));
}

}  // extern "C"
