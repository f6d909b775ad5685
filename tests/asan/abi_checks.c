/* Host-side argument checks of the C ABI, run against a build of the library
 * whose host code is instrumented with AddressSanitizer (the device code is
 * not).  No case reaches a HIP call, so no GPU is needed.  Exit status 0 when
 * every check holds; ASan aborts the process on an invalid host access. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flux3_dit.h"

static int failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed (line %d): %s [%s]\n", __LINE__, #cond, flux3_last_error()); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

/* Device-pointer stand-ins: aligned addresses that are never dereferenced on
 * the host (argument checks only look at their value). */
#define P16 ((void*)(uintptr_t)16)
#define P18 ((void*)(uintptr_t)18)

int main(void) {
  int n = -1;
  CHECK(flux3_version() >= 100);
  CHECK(flux3_build_ids(-1, 2, 0, NULL, 0, NULL, &n) == FLUX3_EINVAL);
  CHECK(strstr(flux3_last_error(), "non-negative") != NULL);
  CHECK(flux3_build_ids(1, 1, 1, NULL, 0, NULL, &n) == FLUX3_EINVAL);

  /* ids into buffers of exactly the reported size (ASan sees any overrun) */
  {
    const int ref_hw[4] = {2, 3, 1, 4};
    CHECK(flux3_build_ids(3, 5, 2, ref_hw, 7, NULL, &n) == FLUX3_OK && n == 15 + 6 + 4 + 7);
    float* ids = (float*)malloc((size_t)n * 4 * sizeof(float));
    CHECK(flux3_build_ids(3, 5, 2, ref_hw, 7, ids, &n) == FLUX3_OK);
    CHECK(ids[4 * 15 + 3] == -1.0f && ids[4 * (n - 1) + 3] == 6.0f && ids[4 * 1 + 2] == 0.5f);
    free(ids);
    int m = -1;
    CHECK(flux3_build_ids_cfg(2, 2, 1, ref_hw, 3, 5, NULL, &m) == FLUX3_OK && m == 2 * (4 + 6) + 3 + 5);
    ids = (float*)malloc((size_t)m * 4 * sizeof(float));
    CHECK(flux3_build_ids_cfg(2, 2, 1, ref_hw, 3, 5, ids, &m) == FLUX3_OK);
    free(ids);
  }
  /* schedule into an exact buffer */
  {
    float* s = (float*)malloc(17 * sizeof(float));
    CHECK(flux3_sigmas(16, 6.93, s) == FLUX3_OK && s[0] == 1.0f && s[16] == 0.0f);
    CHECK(flux3_sigmas(-1, 6.93, s) == FLUX3_EINVAL);
    free(s);
  }

  /* projections: unsupported shape, null, misaligned, bad leading dimension */
  CHECK(flux3_linear(P16, 128, P16, 128, P16, 64, NULL, 4, 64, 100, NULL) == FLUX3_EUNSUPPORTED);
  CHECK(flux3_linear(NULL, 128, P16, 128, P16, 64, NULL, 4, 64, 128, NULL) == FLUX3_EINVAL);
  CHECK(flux3_linear(P18, 128, P16, 128, P16, 64, NULL, 4, 64, 128, NULL) == FLUX3_EINVAL);
  CHECK(flux3_linear(P16, 100, P16, 128, P16, 64, NULL, 4, 64, 128, NULL) == FLUX3_EINVAL);

  /* segments that do not cover the rows, too many segments */
  {
    const int s1[3] = {0, 3, 6}, s2[3] = {0, 3, 3};
    int s3[10];
    for (int i = 0; i < 10; ++i) s3[i] = i;
    CHECK(flux3_ln_modulate(P16, 3072, P16, 3072, 7, s1, 2, P16, 9216, NULL) == FLUX3_EINVAL);
    CHECK(flux3_ln_modulate(P16, 3072, P16, 3072, 3, s2, 2, P16, 9216, NULL) == FLUX3_EINVAL);
    CHECK(flux3_ln_modulate(P16, 3072, P16, 3072, 9, s3, 9, P16, 9216, NULL) == FLUX3_EINVAL);
  }

  /* block: workspace too small or missing, missing weights */
  {
    flux3_block_weights w;
    memset(&w, 0, sizeof(w));
    w.w_in = w.w_out = w.q_scale = w.k_scale = (const uint16_t*)P16;
    const int seg[2] = {0, 10};
    CHECK(flux3_block_forward(P16, 10, seg, 1, P16, &w, P16, P16, 100, NULL) == FLUX3_EWORKSPACE);
    CHECK(flux3_block_forward(P16, 10, seg, 1, P16, &w, P16, NULL, (size_t)1 << 30, NULL) == FLUX3_EWORKSPACE);
    CHECK(flux3_block_forward(P16, 10, seg, 1, P16, NULL, P16, P16, (size_t)1 << 30, NULL) == FLUX3_EINVAL);
    w.w_in = NULL;
    CHECK(flux3_block_forward(P16, 10, seg, 1, P16, &w, P16, P16, (size_t)1 << 30, NULL) == FLUX3_EINVAL);
    CHECK(flux3_block_forward(NULL, 0, NULL, 0, NULL, NULL, NULL, NULL, 0, NULL) == FLUX3_OK);
  }

  /* attention: empty is a no-op; the balanced schedule needs its workspace */
  CHECK(flux3_attention(NULL, 3072, NULL, 3072, NULL, 3072, NULL, 3072, 0, NULL) == FLUX3_OK);
  CHECK(flux3_attention_ws(NULL, 3072, NULL, 3072, NULL, 3072, NULL, 3072, 0, NULL, 0, NULL) == FLUX3_OK);
  CHECK(flux3_attention_noalloc(NULL, 3072, NULL, 3072, NULL, 3072, NULL, 3072, 0, NULL) == FLUX3_OK);
  CHECK(flux3_attention_noalloc(NULL, 3072, P16, 3072, P16, 3072, P16, 3072, 10, NULL) == FLUX3_EINVAL);
  CHECK(flux3_attention_workspace_size(4608) > 0 && flux3_attention_workspace_size(2688) == 0);
  CHECK(flux3_attention_workspace_size(4608) <= FLUX3_ATTENTION_SCRATCH_BYTES);
  CHECK(flux3_attention_ws(P16, 3072, P16, 3072, P16, 3072, P16, 3072, 4608, P16, 1000, NULL) == FLUX3_EWORKSPACE);
  CHECK(flux3_attention_ws(P16, 3072, P16, 3072, P16, 3072, P16, 3072, 4608, NULL, (size_t)1 << 30, NULL) ==
        FLUX3_EINVAL);

  /* launch timer: argument checks (no HIP call on these paths) */
  {
    int cnt = -1;
    CHECK(flux3_timer_stop(NULL, NULL, NULL, 0, &cnt) == FLUX3_EINVAL);
    CHECK(flux3_timer_start(0, 10) == FLUX3_EINVAL);
    CHECK(flux3_timer_start(1u << 5, 10) == FLUX3_EINVAL);
    CHECK(flux3_timer_start(1u << FLUX3_TIMER_IN_PROJ, 0) == FLUX3_EINVAL);
    CHECK(flux3_timer_start(1u << FLUX3_TIMER_IN_PROJ, (1 << 20) + 1) == FLUX3_EINVAL);
  }

  /* stack and sampler: missing weights, workspace too small */
  {
    flux3_model_weights mw;
    memset(&mw, 0, sizeof(mw));
    CHECK(flux3_stack_forward(&mw, P16, 16, NULL, 0, P16, 8, P16, 0.5f, 0.4f, P16, P16, (size_t)1 << 34, NULL) ==
          FLUX3_EINVAL);
    CHECK(flux3_stack_forward(NULL, P16, 16, NULL, 0, P16, 8, P16, 0.5f, 0.4f, P16, P16, (size_t)1 << 34, NULL) ==
          FLUX3_EINVAL);
    const float sig[3] = {1.0f, 0.5f, 0.0f};
    CHECK(flux3_sample(&mw, P16, 16, NULL, 0, P16, 8, P16, sig, 2, P16, 10, NULL) != FLUX3_OK);
    CHECK(flux3_stack_workspace_size(0, 0, 512) == 0);
    CHECK(flux3_stack_workspace_size(4096, 0, 512) > flux3_block_workspace_size(4608));
    CHECK(flux3_sample_workspace_size(4096, 0, 512) >= flux3_stack_workspace_size(4096, 0, 512));
    CHECK(flux3_stack_cfg_workspace_size(4096, 0, 80, 512) > 0);
  }

  /* fp8r: unsupported product shape */
  CHECK(flux3_linear_fp8(P16, 3072, P16, P16, 3072, P16, P16, NULL, 100, 4, 100, 3072, NULL) ==
        FLUX3_EUNSUPPORTED);

  if (failures == 0) printf("abi checks: all passed\n");
  return failures == 0 ? 0 : 1;
}
