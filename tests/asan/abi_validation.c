/*
 * Host-side argument validation of the C ABI (include/gq.h), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host side only and
 * run on a machine with no GPU.
 *
 * Every call below must be rejected (or be an n_tok = 0 no-op) before the
 * library's first HIP call: the pointers are either NULL or fake addresses
 * that nothing maps.  The library under test is compiled host-only, so no
 * kernel exists that could be launched even by mistake; a call that got past
 * validation would show up as GQ_EHIP, which fails the run.
 *
 * Two parts:
 *   1. the explicit cases of the Python ABI tests, with their exact codes;
 *   2. sweeps over extreme sizes (0, -1, block multiples, 2^31 - 1, 2^31,
 *      2^47, INT64_MAX, INT64_MIN ...) with NULL pointers, so that every
 *      size check and the products and quotients in it run on the edge values
 *      under UBSan (signed overflow, division by zero, shifts).
 * Exit status 0 when every check holds; sanitizer reports abort the run.
 *
 * With the argument --reach-runtime the driver instead makes one call that
 * passes validation (fake, aligned, disjoint pointers): it must end in the
 * runtime stand-in's trap, which shows that the trap is live.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/gq.h"

static int failures = 0;
static long checks = 0;

#define EXPECT_EQ(got, want, what)                                                      \
  do {                                                                                  \
    long long g_ = (long long)(got), w_ = (long long)(want);                            \
    checks++;                                                                           \
    if (g_ != w_) {                                                                     \
      fprintf(stderr, "FAIL %s:%d %s: got %lld want %lld\n", __FILE__, __LINE__, what,  \
              g_, w_);                                                                  \
      failures++;                                                                       \
    }                                                                                   \
  } while (0)

/* A code that a pre-HIP rejection may return. */
static void expect_rejected(int rc, int allow_ok, const char* what, long long a, long long b,
                            long long c) {
  checks++;
  const int ok = (rc == GQ_EINVAL_TYPE || rc == GQ_EINVAL_SHAPE || rc == GQ_EINVAL_PTR ||
                  rc == GQ_EALIGN || rc == GQ_EOVERFLOW || (allow_ok && rc == GQ_OK));
  if (!ok) {
    fprintf(stderr, "FAIL %s(%lld, %lld, %lld): code %d\n", what, a, b, c, rc);
    failures++;
  }
}

#define P(x) ((void*)(uintptr_t)(x))
#define FP(x) ((float*)(uintptr_t)(x))

enum { A = 0x10000, B = 0x20000, C = 0x30000, NW = 0x40000, U = 0x50000 };

static void explicit_cases(void) {
  /* type table and row bytes, out-params on exact-size heap blocks */
  int64_t* qk = (int64_t*)malloc(sizeof(int64_t));
  int64_t* bb = (int64_t*)malloc(sizeof(int64_t));
  static const int64_t want[][3] = {{GQ_F32, 1, 4},     {GQ_F16, 1, 2},     {GQ_Q4_0, 32, 18},
                                    {GQ_Q5_0, 32, 22},  {GQ_Q8_0, 32, 34},  {GQ_Q4_K, 256, 144},
                                    {GQ_Q6_K, 256, 210}, {GQ_Q4_1, 32, 20}, {GQ_Q5_K, 256, 176}};
  for (size_t i = 0; i < sizeof(want) / sizeof(want[0]); i++) {
    EXPECT_EQ(gq_type_info((int)want[i][0], qk, bb), GQ_OK, "type_info");
    EXPECT_EQ(*qk, want[i][1], "block elems");
    EXPECT_EQ(*bb, want[i][2], "block bytes");
    EXPECT_EQ(gq_type_info((int)want[i][0], NULL, bb), GQ_OK, "type_info null elems");
    EXPECT_EQ(gq_type_info((int)want[i][0], qk, NULL), GQ_OK, "type_info null bytes");
  }
  EXPECT_EQ(gq_type_info(99, qk, bb), GQ_EINVAL_TYPE, "type_info bad type");
  EXPECT_EQ(gq_type_info(-1, NULL, NULL), GQ_EINVAL_TYPE, "type_info negative type");
  free(qk);
  free(bb);
  EXPECT_EQ(gq_row_bytes(GQ_Q6_K, 11008), 9030, "row_bytes q6_k");
  EXPECT_EQ(gq_row_bytes(GQ_Q4_K, 4096), 2304, "row_bytes q4_k");
  EXPECT_EQ(gq_row_bytes(GQ_Q4_K, 100), GQ_EINVAL_SHAPE, "row_bytes ragged");

  /* every message is a NUL-terminated static string */
  for (int code = -40; code <= 40; code++) {
    const char* m = gq_strerror(code);
    checks++;
    if (!m || strlen(m) == 0) {
      fprintf(stderr, "FAIL strerror(%d)\n", code);
      failures++;
    }
  }

  /* gq_matmul */
  EXPECT_EQ(gq_matmul(P(A), 99, 16, 256, P(B), FP(C), 1, NULL), GQ_EINVAL_TYPE, "bad type");
  EXPECT_EQ(gq_matmul(P(A), GQ_F32, 16, 256, P(B), FP(C), 1, NULL), GQ_EINVAL_TYPE, "F32 weights");
  EXPECT_EQ(gq_matmul(P(A), GQ_Q4_K, 16, 100, P(B), FP(C), 1, NULL), GQ_EINVAL_SHAPE, "cols % 256");
  EXPECT_EQ(gq_matmul(P(A), GQ_Q4_K, 0, 256, P(B), FP(C), 1, NULL), GQ_EINVAL_SHAPE, "rows < 1");
  EXPECT_EQ(gq_matmul(P(A), GQ_Q4_K, 16, 256, P(B), FP(C), -1, NULL), GQ_EINVAL_SHAPE, "n_tok < 0");
  EXPECT_EQ(gq_matmul(NULL, GQ_Q4_K, 16, 256, P(B), FP(C), 1, NULL), GQ_EINVAL_PTR, "null blob");
  EXPECT_EQ(gq_matmul(P(A), GQ_Q4_K, 16, 256, NULL, FP(C), 1, NULL), GQ_EINVAL_PTR, "null x");
  EXPECT_EQ(gq_matmul(P(A + 4), GQ_Q4_K, 16, 256, P(B), FP(C), 1, NULL), GQ_EALIGN, "blob align");
  EXPECT_EQ(gq_matmul(P(A), GQ_Q4_K, 16, 256, P(B + 8), FP(C), 1, NULL), GQ_EALIGN, "x align");
  EXPECT_EQ(gq_matmul(P(A), GQ_Q4_K, 16, 256, P(B), FP(B + 16), 1, NULL), GQ_EINVAL_PTR, "y on x");
  EXPECT_EQ(gq_matmul(P(A), GQ_Q4_K, 16, 256, P(B), FP(A + 32), 1, NULL), GQ_EINVAL_PTR, "y on blob");
  EXPECT_EQ(gq_matmul(P(A), GQ_Q4_K, (int64_t)1 << 31, 256, P(B), FP(C), 1, NULL), GQ_EOVERFLOW,
            "rows 2^31");
  EXPECT_EQ(gq_matmul(P(A), GQ_Q4_K, 16, 32768, P(B), FP(C), 1, NULL), GQ_EOVERFLOW, "GEMV cols");
  EXPECT_EQ(gq_matmul(NULL, GQ_Q4_K, 16, 256, NULL, NULL, 0, NULL), GQ_OK, "n_tok 0");
  EXPECT_EQ(gq_matmul_ex(P(A), GQ_Q4_K, 16, 256, P(B), GQ_Q8_0, FP(C), 1, NULL), GQ_EINVAL_TYPE,
            "x_type");

  /* gq_matmul_path */
  EXPECT_EQ(gq_matmul_path(P(A), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(C), 2, GQ_PATH_GEMV, NULL),
            GQ_EINVAL_SHAPE, "GEMV path, two tokens");
  EXPECT_EQ(gq_matmul_path(P(A), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(C), 1, GQ_PATH_TILED, NULL),
            GQ_EINVAL_SHAPE, "tiled path, one token");
  EXPECT_EQ(gq_matmul_path(P(A), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(C), 1, GQ_PATH_WEIGHT_STREAM,
                           NULL),
            GQ_EINVAL_SHAPE, "stream path, one token");
  EXPECT_EQ(gq_matmul_path(P(A), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(C), 2, 7, NULL),
            GQ_EINVAL_SHAPE, "unknown path");
  EXPECT_EQ(gq_matmul_path(P(A), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(C), 2, -1, NULL),
            GQ_EINVAL_SHAPE, "negative path");
  EXPECT_EQ(gq_matmul_path(P(A), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(C), 0, GQ_PATH_TILED, NULL),
            GQ_OK, "no tokens");

  /* gq_matmul_decode */
  EXPECT_EQ(gq_matmul_decode(P(A), NULL, 99, 16, 256, P(B), GQ_F32, NULL, 1e-5f, FP(C), NULL),
            GQ_EINVAL_TYPE, "decode type");
  EXPECT_EQ(gq_matmul_decode(P(A), NULL, GQ_Q4_K, 16, 256, P(B), GQ_Q8_0, NULL, 1e-5f, FP(C), NULL),
            GQ_EINVAL_TYPE, "decode x_type");
  EXPECT_EQ(gq_matmul_decode(P(A), NULL, GQ_Q4_K, 16, 100, P(B), GQ_F32, NULL, 1e-5f, FP(C), NULL),
            GQ_EINVAL_SHAPE, "decode cols");
  EXPECT_EQ(gq_matmul_decode(P(A), NULL, GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(NW), -1.f, FP(C), NULL),
            GQ_EINVAL_SHAPE, "eps < 0");
  EXPECT_EQ(gq_matmul_decode(P(A), NULL, GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(NW), NAN, FP(C), NULL),
            GQ_EINVAL_SHAPE, "eps NaN");
  EXPECT_EQ(gq_matmul_decode(P(A), NULL, GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(NW), INFINITY, FP(C),
                             NULL),
            GQ_EINVAL_SHAPE, "eps inf");
  EXPECT_EQ(gq_matmul_decode(NULL, P(U), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(NW), 1e-5f, FP(C), NULL),
            GQ_EINVAL_PTR, "decode null blob");
  EXPECT_EQ(gq_matmul_decode(P(A), P(U + 4), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(NW), 1e-5f, FP(C),
                             NULL),
            GQ_EALIGN, "up blob align");
  EXPECT_EQ(gq_matmul_decode(P(A), P(U), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(NW + 8), 1e-5f, FP(C),
                             NULL),
            GQ_EALIGN, "norm align");
  EXPECT_EQ(gq_matmul_decode(P(A), P(U), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(NW), 1e-5f,
                             FP(NW + 16), NULL),
            GQ_EINVAL_PTR, "y on norm");
  EXPECT_EQ(gq_matmul_decode(P(A), P(U), GQ_Q4_K, 16, 256, P(B), GQ_F32, FP(NW), 1e-5f,
                             FP(U + 32), NULL),
            GQ_EINVAL_PTR, "y on up blob");
  EXPECT_EQ(gq_matmul_decode(P(A), P(U), GQ_Q4_K, 16, 32768, P(B), GQ_F32, FP(NW), 1e-5f, FP(C),
                             NULL),
            GQ_EOVERFLOW, "decode cols limit");

  /* gq_dequant, gq_quantize */
  EXPECT_EQ(gq_dequant(P(A), GQ_Q6_K, 4, 255, P(B), GQ_F32, NULL), GQ_EINVAL_SHAPE, "dequant cols");
  EXPECT_EQ(gq_dequant(P(A), GQ_Q6_K, 4, 256, P(B), GQ_Q4_0, NULL), GQ_EINVAL_TYPE, "dequant out");
  EXPECT_EQ(gq_dequant(P(A), GQ_Q6_K, 4, 256, P(A + 16), GQ_F32, NULL), GQ_EINVAL_PTR,
            "dequant overlap");
  EXPECT_EQ(gq_dequant(P(A), GQ_Q6_K, 4, 256, P(B + 2), GQ_F16, NULL), GQ_EALIGN, "dequant align");
  EXPECT_EQ(gq_quantize(FP(A), GQ_Q4_K, 4, 200, P(B), NULL), GQ_EINVAL_SHAPE, "quantize cols");
  EXPECT_EQ(gq_quantize(NULL, GQ_Q4_K, 4, 256, P(B), NULL), GQ_EINVAL_PTR, "quantize null");
  EXPECT_EQ(gq_quantize(FP(A), GQ_Q4_K, 4, 256, P(A + 64), NULL), GQ_EINVAL_PTR,
            "quantize overlap");

  /* gq_probe_stream_read */
  EXPECT_EQ(gq_probe_stream_read(P(A), 100, (uint32_t*)P(B), NULL), GQ_EINVAL_SHAPE, "probe 100");
  EXPECT_EQ(gq_probe_stream_read(P(A), -16, (uint32_t*)P(B), NULL), GQ_EINVAL_SHAPE, "probe -16");
  EXPECT_EQ(gq_probe_stream_read(P(A), ((int64_t)1 << 30) + 16, (uint32_t*)P(B), NULL),
            GQ_EOVERFLOW, "probe size");
  EXPECT_EQ(gq_probe_stream_read(NULL, 0, NULL, NULL), GQ_EINVAL_PTR, "probe null out");
  EXPECT_EQ(gq_probe_stream_read(P(A + 8), 64, (uint32_t*)P(B), NULL), GQ_EALIGN, "probe align");
  EXPECT_EQ(gq_probe_stream_read(P(A), 64, (uint32_t*)P(A + 32), NULL), GQ_EINVAL_PTR,
            "probe overlap");

  /* attention */
  EXPECT_EQ(gq_attn_decode_workspace_bytes(32768, 8, 40, 128), 128LL * 40 * 130 * 4, "ws 32k");
  EXPECT_EQ(gq_attn_decode_workspace_bytes(1, 1, 1, 64), 66LL * 4, "ws 1");
  EXPECT_EQ(gq_attn_decode_workspace_bytes(10, 8, 44, 128), GQ_EINVAL_SHAPE, "ws heads");
  EXPECT_EQ(gq_attn_decode_workspace_bytes(10, 2, 34, 128), GQ_EINVAL_SHAPE, "ws 17 per group");
  EXPECT_EQ(gq_attn_decode_workspace_bytes(10, 2, 4, 96), GQ_EINVAL_SHAPE, "ws head_dim");
  EXPECT_EQ(gq_attn_decode_workspace_bytes(0, 2, 4, 128), GQ_EINVAL_SHAPE, "ws kv_len");
  const uintptr_t K = 0x100000, V = 0x200000, Q = 0x300000, O = 0x310000, WS = 0x400000;
  EXPECT_EQ(gq_attn_decode(P(K), P(V), GQ_Q4_K, 100, 2, 128, FP(Q), 8, FP(O), P(WS), 1 << 20, NULL),
            GQ_EINVAL_TYPE, "attn type");
  EXPECT_EQ(gq_attn_decode(P(K), P(V), GQ_Q8_0, 100, 2, 96, FP(Q), 8, FP(O), P(WS), 1 << 20, NULL),
            GQ_EINVAL_SHAPE, "attn head_dim");
  EXPECT_EQ(gq_attn_decode(P(K), P(V), GQ_Q8_0, 100, 2, 128, FP(Q), 8, FP(O), P(WS), 100, NULL),
            GQ_EINVAL_SHAPE, "attn workspace size");
  EXPECT_EQ(gq_attn_decode(P(K), P(V), GQ_Q8_0, 100, 2, 128, FP(Q), 8, FP(O), NULL, 1 << 20, NULL),
            GQ_EINVAL_PTR, "attn null workspace");
  EXPECT_EQ(gq_attn_decode(P(K), P(V + 4), GQ_Q8_0, 100, 2, 128, FP(Q), 8, FP(O), P(WS), 1 << 20,
                           NULL),
            GQ_EALIGN, "attn align");
  EXPECT_EQ(gq_attn_decode(P(K), P(V), GQ_Q8_0, 100, 2, 128, FP(Q), 8, FP(Q + 64), P(WS), 1 << 20,
                           NULL),
            GQ_EINVAL_PTR, "attn out on q");
  EXPECT_EQ(gq_attn_decode(P(K), P(V), GQ_Q8_0, 100, 2, 128, FP(Q), 8, FP(O), P(K + 256), 1 << 20,
                           NULL),
            GQ_EINVAL_PTR, "attn workspace on K");
  EXPECT_EQ(gq_attn_decode(P(K), P(V), GQ_Q8_0, 1 << 28, 8, 128, FP(Q), 8, FP(O), P(WS), 1 << 20,
                           NULL),
            GQ_EOVERFLOW, "attn cache size");
  EXPECT_EQ(gq_attn_decode_noalloc(P(K), P(V), GQ_Q8_0, 100, 2, 96, FP(Q), 8, FP(O), NULL),
            GQ_EINVAL_SHAPE, "noalloc head_dim");
  EXPECT_EQ(gq_attn_decode_noalloc(P(K), P(V), GQ_Q8_0, 100, 2, 128, FP(Q), 8, NULL, NULL),
            GQ_EINVAL_PTR, "noalloc null out");
  /* 2^22 positions, one KV head, 16 query heads: statistics beyond the array */
  EXPECT_EQ(gq_attn_decode_noalloc(P((uint64_t)1 << 40), P((uint64_t)2 << 40), GQ_Q8_0, 1 << 22, 1,
                                   128, FP((uint64_t)3 << 40), 16, FP((uint64_t)4 << 40), NULL),
            GQ_EOVERFLOW, "noalloc beyond the array");
}

static const int64_t kEdges[] = {INT64_MIN, -((int64_t)1 << 31), -256, -1, 0, 1, 31, 32, 255, 256,
                                 4096, 16384, 16385, 32768, (int64_t)1 << 21,
                                 ((int64_t)1 << 21) + 256, ((int64_t)1 << 22) + 1,
                                 ((int64_t)1 << 31) - 1, (int64_t)1 << 31, ((int64_t)1 << 31) + 256,
                                 (int64_t)1 << 40, (int64_t)1 << 47, (int64_t)1 << 62, INT64_MAX};
#define NE ((int)(sizeof(kEdges) / sizeof(kEdges[0])))

static void sweeps(void) {
  static const int types[] = {-1, GQ_F32, GQ_F16, GQ_Q4_0, GQ_Q5_0, GQ_Q8_0, GQ_Q4_K,
                              GQ_Q6_K, GQ_Q4_1, GQ_Q5_K, 9, 1 << 30};
  const int nt = (int)(sizeof(types) / sizeof(types[0]));
  for (int ti = 0; ti < nt; ti++) {
    const int t = types[ti];
    for (int i = 0; i < NE; i++) {
      const int64_t rb = gq_row_bytes(t, kEdges[i]);
      checks++;
      if (rb == GQ_EHIP || (rb > 0 && rb > (int64_t)1 << 40)) {
        fprintf(stderr, "FAIL row_bytes(%d, %lld) = %lld\n", t, (long long)kEdges[i],
                (long long)rb);
        failures++;
      }
      for (int j = 0; j < NE; j++) {
        const int64_t rows = kEdges[i], cols = kEdges[j];
        expect_rejected(gq_dequant(NULL, t, rows, cols, NULL, GQ_F32, NULL), 0, "dequant", t, rows,
                        cols);
        expect_rejected(gq_quantize(NULL, t, rows, cols, NULL, NULL), 0, "quantize", t, rows, cols);
        expect_rejected(gq_matmul_decode(NULL, NULL, t, rows, cols, NULL, GQ_F16, NULL, 1e-5f, NULL,
                                         NULL),
                        0, "matmul_decode", t, rows, cols);
        for (int k = 0; k < NE; k++) {
          const int64_t n = kEdges[k];
          for (int path = -1; path <= 4; path++)
            expect_rejected(gq_matmul_path(NULL, t, rows, cols, NULL, GQ_F32, NULL, n, path, NULL),
                            n == 0, "matmul_path", rows, cols, n);
        }
      }
    }
  }
  static const int dims[] = {-1, 0, 32, 64, 96, 128, 256, 512, 1 << 30};
  static const int heads[] = {-8, 0, 1, 2, 7, 8, 16, 17, 64, 65535, 65536, 1 << 20, 0x7FFFFFFF};
  const int nd = (int)(sizeof(dims) / sizeof(dims[0]));
  const int nh = (int)(sizeof(heads) / sizeof(heads[0]));
  for (int i = 0; i < NE; i++)
    for (int a = 0; a < nh; a++)
      for (int b = 0; b < nh; b++)
        for (int d = 0; d < nd; d++) {
          const int64_t kv = kEdges[i];
          const int64_t ws = gq_attn_decode_workspace_bytes(kv, heads[a], heads[b], dims[d]);
          checks++;
          if (ws == GQ_EHIP || ws == 0 || ws == GQ_EINVAL_PTR || ws == GQ_EALIGN ||
              ws < GQ_EHIP) {
            fprintf(stderr, "FAIL workspace(%lld, %d, %d, %d) = %lld\n", (long long)kv, heads[a],
                    heads[b], dims[d], (long long)ws);
            failures++;
          }
          for (int kt = GQ_F32; kt <= GQ_Q5_K; kt++) {
            expect_rejected(gq_attn_decode(NULL, NULL, kt, kv, heads[a], dims[d], NULL, heads[b],
                                           NULL, NULL, INT64_MAX, NULL),
                            0, "attn", kv, heads[a], heads[b]);
            expect_rejected(gq_attn_decode_noalloc(NULL, NULL, kt, kv, heads[a], dims[d], NULL,
                                                   heads[b], NULL, NULL),
                            0, "attn_noalloc", kv, heads[a], heads[b]);
          }
        }
  for (int i = 0; i < NE; i++)
    expect_rejected(gq_probe_stream_read(NULL, kEdges[i], NULL, NULL), 0, "probe", kEdges[i], 0, 0);
}

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "--reach-runtime") == 0) {
    const int rc = gq_matmul(P(A), GQ_Q4_K, 16, 256, P(B), FP(C), 1, NULL);
    printf("validation passed the call through: code %d\n", rc);
    return 2;
  }
  explicit_cases();
  sweeps();
  if (failures) {
    fprintf(stderr, "%d of %ld checks failed\n", failures, checks);
    return 1;
  }
  printf("abi validation: %ld checks passed\n", checks);
  return 0;
}
