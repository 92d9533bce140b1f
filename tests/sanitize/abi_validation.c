/*
 * Host-side validation layer of libnvfp4.so under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Built (with the library, whose host code is
 * instrumented) and run by tests/test_abi_sanitized_cpu.py on a host without
 * a GPU.  Every call either fails validation before any device work, or is a
 * workspace-size query; with the argument "nodevice" it also makes calls that
 * pass validation and must stop at the device check.  No pointer passed here
 * is ever dereferenced.  Exit status: the number of failed checks.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nvfp4.h"

static int failures = 0;
#define CHECK(expr, want)                                                              \
  do {                                                                                 \
    int got_ = (expr);                                                                 \
    if (got_ != (want)) {                                                              \
      fprintf(stderr, "line %d: %s -> %d, want %d\n", __LINE__, #expr, got_, (want)); \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

#define FAKE ((void *)(uintptr_t)0x100000)

int main(int argc, char **argv) {
  const int nodevice = argc > 1 && strcmp(argv[1], "nodevice") == 0;
  nvfp4_tensor t = {(uint8_t *)FAKE, (uint8_t *)FAKE, (float *)FAKE};
  nvfp4_tensor z = {0, 0, 0};
  nvfp4_tensor badg = {(uint8_t *)FAKE, (uint8_t *)FAKE, NULL};
  size_t big = (size_t)1 << 30, small = 16, sz = 0;
  float *fa = (float *)FAKE;

  /* status strings, launch counter */
  for (int c = 0; c < 8; ++c)
    if (!nvfp4_strerror(c) || !nvfp4_strerror(c)[0]) ++failures;
  if (strcmp(nvfp4_strerror(1234), "unknown status") != 0) ++failures;
  (void)nvfp4_launch_count();

  /* quantise */
  CHECK(nvfp4_quantize_act(FAKE, 7, 4, 32, 32, t, 0, FAKE, &big, NULL), NVFP4_ERR_ARG);
  CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, 4, 32, 32, t, 9, FAKE, &big, NULL), NVFP4_ERR_ARG);
  CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, 4, 24, 24, t, 0, FAKE, &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, 4, 32, 16, t, 0, FAKE, &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, -5, 32, 32, t, 0, FAKE, &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, (int64_t)1 << 40, 64, 64, t, 0, FAKE, &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize_act(NULL, NVFP4_BF16, 4, 32, 32, t, 0, FAKE, &big, NULL), NVFP4_ERR_NULL);
  CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, 4, 32, 32, badg, 0, FAKE, &big, NULL), NVFP4_ERR_NULL);
  CHECK(nvfp4_quantize_act((char *)FAKE + 2, NVFP4_BF16, 4, 32, 32, t, 0, FAKE, &big, NULL), NVFP4_ERR_ALIGN);
  CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, 4, 32, 32, t, 0, FAKE, &small, NULL), NVFP4_ERR_WORKSPACE);
  CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, 4, 32, 32, t, 0, FAKE, NULL, NULL), NVFP4_ERR_WORKSPACE);
  CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, 4, 32, 32, t, NVFP4_GS_FROM_AMAX, NULL, NULL, NULL), NVFP4_ERR_WORKSPACE);
  CHECK(nvfp4_quantize_act(NULL, NVFP4_BF16, 0, 32, 32, z, 0, FAKE, &big, NULL), NVFP4_OK);
  CHECK(nvfp4_quantize_act(NULL, NVFP4_BF16, 1024, 5120, 5120, z, 0, NULL, &sz, NULL), NVFP4_OK);
  if (sz == 0 || sz > 16384) ++failures;
  CHECK(nvfp4_quantize_act_noalloc(FAKE, NVFP4_BF16, 4, 24, 24, t, 0, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize_act_noalloc(FAKE, NVFP4_BF16, 4, 32, 32, t, NVFP4_GS_FROM_AMAX, NULL), NVFP4_ERR_ARG);
  CHECK(nvfp4_rmsnorm_quantize_act(FAKE, NVFP4_BF16, 4, 32, 32, fa, -1.0f, t, FAKE, &big, NULL), NVFP4_ERR_ARG);
  CHECK(nvfp4_rmsnorm_quantize_act(FAKE, NVFP4_BF16, 4, 32, 32, NULL, 1e-6f, t, FAKE, &big, NULL), NVFP4_ERR_NULL);

  /* contractions */
  CHECK(nvfp4_gemm(t, t, 4, 8, 100, FAKE, NVFP4_F32, 8, NULL, FAKE, &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_gemm(t, t, 4, 8, 128, FAKE, 5, 8, NULL, FAKE, &big, NULL), NVFP4_ERR_ARG);
  CHECK(nvfp4_gemm(t, t, 4, 8, 128, FAKE, NVFP4_F32, 4, NULL, FAKE, &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_gemm(t, t, 4, 6, 128, FAKE, NVFP4_F32, 6, NULL, FAKE, &big, NULL), NVFP4_ERR_ALIGN);
  CHECK(nvfp4_gemm(t, t, 4, 8, 128, FAKE, NVFP4_F32, 8, (float *)((char *)FAKE + 4), FAKE, &big, NULL),
        NVFP4_ERR_ALIGN);
  CHECK(nvfp4_gemm(z, z, 1024, 5120, 17408, NULL, NVFP4_F32, 5120, NULL, NULL, &sz, NULL), NVFP4_OK);
  CHECK(nvfp4_mlp_gu_act(t, t, t, 4, 5120, 17400, t, FAKE, &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_mlp_gu_act(t, t, t, 4, 128, 128, t, FAKE, &small, NULL), NVFP4_ERR_WORKSPACE);
  CHECK(nvfp4_mlp_gu_act(z, z, z, 1024, 5120, 17408, z, NULL, &sz, NULL), NVFP4_OK);
  CHECK(nvfp4_mlp_down(t, t, 4, 100, 64, FAKE, NVFP4_F32, 64, NULL, FAKE, &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_mlp_down(t, t, 4, 128, 64, NULL, NVFP4_F32, 64, NULL, FAKE, &big, NULL), NVFP4_ERR_NULL);
  CHECK(nvfp4_mlp_gu_act_static(t, t, badg, 4, 128, 128, t, FAKE, &big, NULL), NVFP4_ERR_NULL);
  CHECK(nvfp4_mlp_down_quant(t, t, 4, 128, 40, t, FAKE, &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_mlp(FAKE, NVFP4_BF16, 5120, NULL, 4, 5120, 17400, t, t, t, t, t, FAKE, NVFP4_F32, 5120, NULL, FAKE,
                  &big, NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_mlp(FAKE, NVFP4_BF16, 5120, NULL, 4, 5120, 17408, t, t, t, t, t, FAKE, NVFP4_F32, 5120, NULL, FAKE,
                  &small, NULL), NVFP4_ERR_WORKSPACE);
  CHECK(nvfp4_mlp(NULL, NVFP4_BF16, 5120, NULL, 1, 5120, 17408, z, z, z, z, z, NULL, NVFP4_F32, 5120, NULL, NULL,
                  &sz, NULL), NVFP4_OK);

  /* expert-grouped, routing, combine */
  CHECK(nvfp4_grouped_gemm(t, NULL, (int32_t *)FAKE, 3, 40, t, t, 256, 384, 7, FAKE, NVFP4_F32, 256, t, FAKE, &big,
                           NULL), NVFP4_ERR_ARG);
  CHECK(nvfp4_grouped_gemm(t, NULL, NULL, 3, 40, t, t, 256, 384, NVFP4_EPI_STORE, FAKE, NVFP4_F32, 256, t, FAKE,
                           &big, NULL), NVFP4_ERR_NULL);
  CHECK(nvfp4_grouped_gemm(t, NULL, (int32_t *)FAKE, 0, 40, t, t, 256, 384, NVFP4_EPI_STORE, FAKE, NVFP4_F32, 256,
                           t, FAKE, &big, NULL), NVFP4_ERR_ARG);
  CHECK(nvfp4_moe_route(fa, 16, 64, 17, 64, (int32_t *)FAKE, (int32_t *)FAKE, (int32_t *)FAKE, fa, FAKE, &big,
                        NULL), NVFP4_ERR_ARG);
  CHECK(nvfp4_moe_route(fa, 16, 64, 8, 32, (int32_t *)FAKE, (int32_t *)FAKE, (int32_t *)FAKE, fa, FAKE, &big,
                        NULL), NVFP4_ERR_SHAPE);
  CHECK(nvfp4_moe_combine(FAKE, NVFP4_F32, 64, (int32_t *)FAKE, fa, 16, 8, 60, FAKE, NVFP4_F32, 64, NULL),
        NVFP4_ERR_SHAPE);
  CHECK(nvfp4_moe_combine(FAKE, NVFP4_F32, 64, (int32_t *)FAKE, fa, 16, 0, 64, FAKE, NVFP4_F32, 64, NULL),
        NVFP4_ERR_ARG);

  /* timing window misuse */
  int64_t n = 0, d = 0;
  double ms = 0.0;
  CHECK(nvfp4_timing_begin(99, 10), NVFP4_ERR_ARG);
  CHECK(nvfp4_timing_begin(NVFP4_KC_GEMM_GLU, 0), NVFP4_ERR_ARG);
  CHECK(nvfp4_timing_end(&n, &d, &ms), NVFP4_ERR_ARG);
  CHECK(nvfp4_timing_end(NULL, &d, &ms), NVFP4_ERR_NULL);

  if (nodevice) {
    /* valid calls on a host without a GPU stop at the device check */
    CHECK(nvfp4_quantize_act(FAKE, NVFP4_BF16, 4, 32, 32, t, 0, FAKE, &big, NULL), NVFP4_ERR_DEVICE);
    CHECK(nvfp4_quantize_act_noalloc(FAKE, NVFP4_BF16, 4, 32, 32, t, 0, NULL), NVFP4_ERR_DEVICE);
    CHECK(nvfp4_gemm(t, t, 4, 8, 128, FAKE, NVFP4_F32, 8, NULL, FAKE, &big, NULL), NVFP4_ERR_DEVICE);
    CHECK(nvfp4_mlp_down(t, t, 4, 128, 64, FAKE, NVFP4_F32, 64, fa, FAKE, &big, NULL), NVFP4_ERR_DEVICE);
    CHECK(nvfp4_mlp(FAKE, NVFP4_BF16, 5120, NULL, 1, 5120, 17408, t, t, t, t, t, FAKE, NVFP4_F32, 5120, NULL, FAKE,
                    &big, NULL), NVFP4_ERR_DEVICE);
  }
  if (failures) fprintf(stderr, "%d failed checks\n", failures);
  return failures;
}
