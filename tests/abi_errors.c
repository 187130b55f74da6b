/* Host-side error paths of every entry point of awq_mi355x.h, run against a
 * build of the library whose host code carries AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_abi_sanitized.py).  Every call here
 * is rejected during validation, before any HIP call, so no GPU is needed;
 * the sanitizers check that validation itself reads no memory it should not
 * and that the size arithmetic of the workspace queries never overflows,
 * including at the largest accepted sizes.  Prints "ok" on success. */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "awq_mi355x.h"

static int failures = 0;

#define EXPECT(expr, want)                                                        \
  do {                                                                            \
    int got_ = (int)(expr);                                                       \
    if (got_ != (int)(want)) {                                                    \
      printf("FAIL line %d: %s -> %d, want %d (%s)\n", __LINE__, #expr, got_,      \
             (int)(want), awq_last_error());                                      \
      ++failures;                                                                 \
    } else if ((want) != AWQ_OK && strlen(awq_last_error()) == 0) {               \
      printf("FAIL line %d: %s gave no message\n", __LINE__, #expr);              \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

static void* thread_main(void* arg) {
  (void)arg;
  /* a failure on this thread must not show on the main thread */
  awq_act_stats(NULL, 1, 8, NULL, NULL, 0, NULL);
  return NULL;
}

int main(void) {
  void* F = (void*)0x10000;    /* 16-byte aligned, never dereferenced on these paths */
  void* FM = (void*)0x10004;   /* misaligned */
  size_t b = 0;
  const int64_t big = (int64_t)1 << 31, k22 = (int64_t)1 << 22;

  if (awq_abi_version() != AWQ_ABI_VERSION) ++failures;
  if (strcmp(awq_status_string(99), "AWQ_ERR_UNKNOWN") != 0) ++failures;

  /* workspace sizes: every op, the largest accepted shapes, and rejections */
  EXPECT(awq_workspace_size(AWQ_OP_ACT_STATS, big - 1, 0, (big - 8), 4, 128, 20, &b), AWQ_OK);
  EXPECT(awq_workspace_size(AWQ_OP_ACT_STATS, big, 0, 8, 4, 128, 20, &b), AWQ_ERR_SHAPE);
  EXPECT(awq_workspace_size(AWQ_OP_W4A16_GEMM, big - 1, k22, 128, 4, 128, 20, &b), AWQ_OK);
  EXPECT(awq_workspace_size(AWQ_OP_W4A16_GEMM, big - 1, k22 + 1, 128, 4, 128, 20, &b), AWQ_ERR_SHAPE);
  EXPECT(awq_workspace_size(AWQ_OP_SEARCH_SCALE, big - 1, k22, k22, 4, 128, 64, &b), AWQ_OK);
  EXPECT(awq_workspace_size(AWQ_OP_SEARCH_SCALE, 1, 1, k22 + 128, 4, 128, 20, &b), AWQ_ERR_SHAPE);
  EXPECT(awq_workspace_size(AWQ_OP_SEARCH_SCALE, 1, 1, 128, 2, 128, 20, &b), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_workspace_size(AWQ_OP_SEARCH_SCALE, 1, 1, 128, 4, 64, 20, &b), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_workspace_size(AWQ_OP_SEARCH_SCALE, 1, 1, 128, 4, 128, 65, &b), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_workspace_size(AWQ_OP_CANDIDATE_SCALES, 0, 0, big - 1, 4, 128, 64, &b), AWQ_OK);
  EXPECT(awq_workspace_size(AWQ_OP_DECODE_GEMM, 64, k22, k22, 4, 128, 20, &b), AWQ_OK);
  EXPECT(awq_workspace_size(AWQ_OP_DECODE_GEMM, 65, 8, 128, 4, 128, 20, &b), AWQ_ERR_SHAPE);
  EXPECT(awq_workspace_size(AWQ_OP_CANDIDATE_SSE, big - 1, k22, 128, 4, 128, 20, &b), AWQ_OK);
  EXPECT(awq_workspace_size(AWQ_OP_SEARCH_SCALE_GRAM, k22 - 128, k22, k22 / 2, 3, 128, 64, &b), AWQ_OK);
  EXPECT(awq_workspace_size(AWQ_OP_SEARCH_SCALE_GRAM, k22 + 1, 8, 128, 4, 128, 20, &b), AWQ_ERR_SHAPE);
  EXPECT(awq_workspace_size(AWQ_OP_W4A16_GEMM_STAGED, big - 1, k22, k22, 4, 128, 20, &b), AWQ_OK);
  EXPECT(awq_workspace_size(AWQ_OP_W4A16_GEMM_STAGED, 1, 1, 100, 4, 128, 20, &b), AWQ_ERR_SHAPE);
  EXPECT(awq_workspace_size(99, 1, 1, 128, 4, 128, 20, &b), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_workspace_size(AWQ_OP_ACT_STATS, 1, 0, 8, 4, 128, 20, NULL), AWQ_ERR_NULL);

  /* statistics and candidate scales */
  EXPECT(awq_act_stats(NULL, 4, 8, F, F, 1 << 20, NULL), AWQ_ERR_NULL);
  EXPECT(awq_act_stats(F, 0, 8, F, F, 1 << 20, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_act_stats(F, 4, 12, F, F, 1 << 20, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_act_stats(FM, 4, 8, F, F, 1 << 20, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_act_stats(F, 4, 8, F, NULL, 0, NULL), AWQ_ERR_WORKSPACE);
  EXPECT(awq_candidate_scales(NULL, 8, 20, F, F, F, 1 << 20, NULL), AWQ_ERR_NULL);
  EXPECT(awq_candidate_scales(F, 0, 20, F, F, F, 1 << 20, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_candidate_scales(F, 8, 0, F, F, F, 1 << 20, NULL), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_candidate_scales(F, 8, 20, FM, F, F, 1 << 20, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_candidate_scales(F, 8, 20, F, F, F, 1, NULL), AWQ_ERR_WORKSPACE);

  /* quantize / pack in every format, and the operands */
  EXPECT(awq_quantize_pack(F, 4, 128, NULL, 5, 128, F, F, F, NULL), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_quantize_pack(F, 4, 100, NULL, 4, 128, F, F, F, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_quantize_pack(F, -1, 128, NULL, 4, 128, F, F, F, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_quantize_pack(NULL, 4, 128, NULL, 4, 128, F, F, F, NULL), AWQ_ERR_NULL);
  EXPECT(awq_quantize_pack(F, 4, 128, FM, 4, 128, F, F, F, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_quantize_pack(F, 0, 128, NULL, 4, 128, NULL, NULL, NULL, NULL), AWQ_OK);
  EXPECT(awq_quantize_pack3(F, 4, 128, NULL, 64, F, F, F, NULL), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_quantize_pack3(F, 4, 128, NULL, 128, (void*)0x10002, F, F, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_quantize_pack16(F, 4, 128, NULL, 4, 128, 7, F, F, F, NULL), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_quantize_pack16(F, 4, 128, NULL, 4, 128, AWQ_LAYOUT_INT3_DENSE, F, F, F, NULL),
         AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_quantize_pack16(F, 4, 128, NULL, 4, 128, AWQ_LAYOUT_NIBBLE, F, (void*)0x10001, F, NULL),
         AWQ_ERR_ALIGN);
  EXPECT(awq_expand_meta16(NULL, F, 4, 128, 128, F, F, NULL), AWQ_ERR_NULL);
  EXPECT(awq_expand_meta16(F, F, 4, 100, 128, F, F, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_dequant_operand(F, 4, 128, F, F, 4, 128, NULL, NULL), AWQ_ERR_NULL);
  EXPECT(awq_dequant_operand(F, 4, 128, FM, F, 4, 128, F, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_diff_operand(F, 4, k22 + 128, F, F, 4, 128, F, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_diff_operand(F, 4, 128, F, F, 3, 96, F, NULL), AWQ_ERR_UNSUPPORTED);

  /* contractions */
  EXPECT(awq_reference_gemm(F, 4, k22 + 1, 128, F, F, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_reference_gemm(NULL, 4, 8, 128, F, F, NULL), AWQ_ERR_NULL);
  EXPECT(awq_reference_gemm(F, 0, 8, 128, NULL, NULL, NULL), AWQ_OK);
  EXPECT(awq_candidate_sse(F, 4, 8, 128, F, NULL, NULL, F, 1 << 20, NULL), AWQ_ERR_NULL);
  EXPECT(awq_candidate_sse(F, 4, 8, 128, F, NULL, (double*)0x10004, F, 1 << 20, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_candidate_sse(F, 4, 8, 128, F, NULL, F, F, 0, NULL), AWQ_ERR_WORKSPACE);
  EXPECT(awq_w4a16_gemm(F, 4, 8, 128, F, F, F, 4, 128, NULL, NULL, NULL, NULL, NULL, 0, NULL),
         AWQ_ERR_NULL);
  EXPECT(awq_w4a16_gemm(F, 4, 8, 128, F, F, F, 4, 128, NULL, NULL, NULL, F, NULL, 0, NULL),
         AWQ_ERR_NULL);
  EXPECT(awq_w4a16_gemm(F, 4, 8, 128, F, F, F, 4, 128, NULL, F, NULL, F, NULL, 0, NULL),
         AWQ_ERR_WORKSPACE);
  EXPECT(awq_w4a16_gemm(F, 4, 8, 128, F, F, F, 4, 128, FM, NULL, F, NULL, NULL, 0, NULL),
         AWQ_ERR_ALIGN);
  EXPECT(awq_w3a16_gemm(F, 4, 8, 128, F, F, F, 128, NULL, NULL, NULL, NULL, NULL, 0, NULL),
         AWQ_ERR_NULL);
  EXPECT(awq_w3a16_gemm(F, 4, 8, 128, NULL, F, F, 128, NULL, NULL, F, NULL, NULL, 0, NULL),
         AWQ_ERR_NULL);
  EXPECT(awq_w3a16_gemm(F, 4, 8, 128, F, F, F, 128, NULL, F, NULL, F, NULL, 0, NULL),
         AWQ_ERR_WORKSPACE);
  EXPECT(awq_w3a16_gemm(F, 4, 8, 128, (void*)0x10002, F, F, 128, NULL, NULL, F, NULL, NULL, 0,
                        NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_w3a16_gemm(F, 4, 8, 100, F, F, F, 128, NULL, NULL, F, NULL, NULL, 0, NULL),
         AWQ_ERR_SHAPE);
  EXPECT(awq_w3a16_gemm(F, 4, 8, 128, F, F, F, 64, NULL, NULL, F, NULL, NULL, 0, NULL),
         AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_w3a16_gemm(F, 0, 8, 128, NULL, NULL, NULL, 128, NULL, NULL, NULL, NULL, NULL, 0, NULL),
         AWQ_OK);
  EXPECT(awq_w4a16_gemm_staged(F, 4, 8, 128, F, F, F, 4, 128, 3, NULL, NULL, F, NULL, F, 1 << 20,
                               NULL), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_w4a16_gemm_staged(F, 4, 8, 128, F, F, F, 4, 128, AWQ_LAYOUT_INT3_DENSE, NULL, NULL, F,
                               NULL, F, 1 << 20, NULL), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_w4a16_gemm_staged(F, 4, 8, 128, F, F, F, 4, 128, 0, NULL, NULL, F, NULL, F, 16, NULL),
         AWQ_ERR_WORKSPACE);
  EXPECT(awq_w4a16_gemm_staged(F, 4, 8, 128, (void*)0x10002, F, F, 4, 128, 0, NULL, NULL, F, NULL,
                               F, 1 << 20, NULL), AWQ_ERR_ALIGN);

  /* decode contraction in every form */
  EXPECT(awq_w4a16_decode_gemm(F, 65, 8, 128, F, F, F, 4, 128, F, NULL, 0, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_w4a16_decode_gemm(F, 4, 8, 128, F, NULL, F, 4, 128, F, NULL, 0, NULL), AWQ_ERR_NULL);
  EXPECT(awq_w4a16_decode_gemm(F, 4, 8, k22, F, F, F, 4, 128, F, NULL, 0, NULL), AWQ_ERR_WORKSPACE);
  EXPECT(awq_w3a16_decode_gemm(F, 4, 8, 128, (void*)0x10002, F, F, 128, F, NULL, 0, NULL),
         AWQ_ERR_ALIGN);
  EXPECT(awq_decode_tiles_size(8, 128, 5, 128, &b), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_decode_tiles_size(k22, k22, AWQ_LAYOUT_NIBBLE, 128, &b), AWQ_OK);
  EXPECT(awq_decode_tiles_size(8, 128, AWQ_LAYOUT_NIBBLE, 128, NULL), AWQ_ERR_NULL);
  EXPECT(awq_decode_tiles(NULL, 8, 128, AWQ_LAYOUT_NIBBLE, 128, F, NULL), AWQ_ERR_NULL);
  EXPECT(awq_decode_tiles(F, 8, 128, AWQ_LAYOUT_NIBBLE, 128, (void*)0x10004, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_decode_gemm_tiled(F, 4, 8, 128, F, NULL, F, AWQ_LAYOUT_NIBBLE, 128, F, NULL, 0, NULL),
         AWQ_ERR_NULL);
  EXPECT(awq_decode_gemm_tiled(F, 4, k22, k22, F, F, F, AWQ_LAYOUT_NIBBLE, 128, F, F, (size_t)-1,
                               NULL), AWQ_ERR_SHAPE);      /* tiles beyond 4 GiB */
  EXPECT(awq_decode_gemm_tiled_noalloc(F, 64, 24576, 28672, F, F, F, AWQ_LAYOUT_NIBBLE, 128, F,
                                       NULL), AWQ_ERR_WORKSPACE);   /* beyond the static scratch */
  EXPECT(awq_decode_gemm_tiled_noalloc(F, 4, 8, 128, F, F, F, 2, 128, F, NULL), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_decode_gemm_tiled_noalloc(F, 0, 8, 128, NULL, NULL, NULL, AWQ_LAYOUT_NIBBLE, 128, NULL,
                                       NULL), AWQ_OK);
  EXPECT(awq_decode_gemm_tiled16(F, 4, 8, 128, F, NULL, F, AWQ_LAYOUT_NIBBLE, 128, F, NULL, 0, NULL),
         AWQ_ERR_NULL);
  EXPECT(awq_decode_gemm_tiled16(F, 4, 8, 128, F, (void*)0x10001, F, AWQ_LAYOUT_NIBBLE, 128, F, NULL,
                                 0, NULL), AWQ_ERR_ALIGN);

  /* metadata tiles */
  EXPECT(awq_decode_meta_size(big - 1, k22, 128, &b), AWQ_ERR_SHAPE);
  EXPECT(awq_decode_meta_size(k22, k22, 128, &b), AWQ_OK);
  EXPECT(awq_decode_meta_size(8, 128, 128, NULL), AWQ_ERR_NULL);
  EXPECT(awq_decode_meta(NULL, F, 8, 128, 128, F, NULL), AWQ_ERR_NULL);
  EXPECT(awq_decode_meta(F, F, 8, 128, 128, (void*)0x10002, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_decode_gemm_tiled_meta(F, 4, 8, 128, F, NULL, AWQ_LAYOUT_NIBBLE, 128, F, NULL, 0, NULL),
         AWQ_ERR_NULL);
  EXPECT(awq_decode_gemm_tiled_meta(F, 4, 8, 128, F, (void*)0x10002, AWQ_LAYOUT_NIBBLE, 128, F, NULL,
                                    0, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_decode_gemm_tiled_meta(F, 65, 8, 128, F, F, AWQ_LAYOUT_NIBBLE, 128, F, NULL, 0, NULL),
         AWQ_ERR_SHAPE);
  EXPECT(awq_decode_gemm_tiled_meta(F, 4, 8, 32768, F, F, AWQ_LAYOUT_NIBBLE, 128, F, NULL, 0, NULL),
         AWQ_ERR_WORKSPACE);

  /* measured ceilings */
  {
    int64_t fl = 0;
    EXPECT(awq_ceiling_mfma(0, 10, 0, F, &fl, NULL), AWQ_ERR_SHAPE);
    EXPECT(awq_ceiling_mfma(4, 10, 0, NULL, &fl, NULL), AWQ_ERR_NULL);
    EXPECT(awq_ceiling_stream(7, F, F, 4096, 1024, NULL), AWQ_ERR_UNSUPPORTED);
    EXPECT(awq_ceiling_stream(AWQ_CEILING_COPY, F, F, 4100, 1024, NULL), AWQ_ERR_SHAPE);
    EXPECT(awq_ceiling_stream(AWQ_CEILING_COPY, F, F, 4096, 0, NULL), AWQ_ERR_SHAPE);
    EXPECT(awq_ceiling_stream(AWQ_CEILING_COPY, F, F, 4096, (1 << 24) + 1, NULL), AWQ_ERR_SHAPE);
    EXPECT(awq_ceiling_stream(AWQ_CEILING_READ, F, (void*)0x10002, 4096, 1024, NULL), AWQ_ERR_ALIGN);
  }

  /* the searches */
  EXPECT(awq_search_scale(F, 0, 128, F, 8, 4, 128, 20, F, F, F, F, F, F, F, F, 0, NULL),
         AWQ_ERR_SHAPE);
  EXPECT(awq_search_scale(F, 4, 128, F, 8, 4, 128, 20, NULL, F, F, F, F, F, F, F, 0, NULL),
         AWQ_ERR_NULL);
  EXPECT(awq_search_scale(F, 4, 128, F, 8, 4, 128, 20, F, F, F, F, F, F, F, F, 0, NULL),
         AWQ_ERR_WORKSPACE);
  EXPECT(awq_search_scale(F, 4, 128, F, 8, 4, 128, 20, F, (double*)0x10004, F, F, F, F, F, F,
                          1u << 30, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_search_scale_gram(F, 4, 128, F, 8, 4, 128, 0, F, F, F, F, F, F, F, F, 0, NULL),
         AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_search_scale_gram(F, k22 + 1, 128, F, 8, 4, 128, 20, F, F, F, F, F, F, F, F, 0, NULL),
         AWQ_ERR_SHAPE);

  /* block ops */
  EXPECT(awq_rmsnorm(F, 4, 12, F, 1e-5, F, NULL, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_rmsnorm(F, 4, 16, F, -1.0, F, NULL, NULL), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_silu_mul(F, 4, 6, F, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_silu_mul(F, 4, 8, (void*)0x10004, NULL), AWQ_ERR_ALIGN);
  EXPECT(awq_divide_rows(NULL, 4, 1, F, F, NULL), AWQ_ERR_NULL);
  EXPECT(awq_divide_rows(F, -1, 1, F, F, NULL), AWQ_ERR_SHAPE);
  EXPECT(awq_residual_add(F, F, 4, 12, F, NULL), AWQ_ERR_SHAPE);

  /* awq_last_error is per thread */
  EXPECT(awq_quantize_pack(F, 4, 100, NULL, 4, 128, F, F, F, NULL), AWQ_ERR_SHAPE);
  char before[512];
  snprintf(before, sizeof before, "%s", awq_last_error());
  pthread_t th;
  pthread_create(&th, NULL, thread_main, NULL);
  pthread_join(th, NULL);
  if (strcmp(before, awq_last_error()) != 0) {
    printf("FAIL last error changed by another thread\n");
    ++failures;
  }

  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
