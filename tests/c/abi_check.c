/* Plain C11 user of include/pa.h: the header compiles as C, and the library's
 * host-side checks answer as documented (no call here reaches a kernel). */
#include <stdio.h>
#include <string.h>

#include "pa.h"

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

int main(void) {
  EXPECT(pa_version() >= 200);
  EXPECT(strcmp(pa_strerror(PA_OK), "ok") == 0);
  EXPECT(strcmp(pa_strerror(PA_ERR_WORKSPACE), "workspace too small") == 0);

  size_t bytes = 0;
  int32_t splits = 0;
  EXPECT(pa_decode_workspace_size(512, 16, 128, 4096, 1024, &bytes, &splits) == PA_OK);
  /* split statistics, then the shared-prefix work list (count + one int32 per
     (sequence, split)), each rounded up to 16 bytes */
  EXPECT(splits == 4 && bytes == (size_t)512 * 16 * 4 * 130 * 4 + (4 * (512 * 4 + 1) + 15) / 16 * 16);
  EXPECT(pa_decode_workspace_size(1, 2, 64, 37, 100, &bytes, &splits) == PA_ERR_UNSUPPORTED);
  EXPECT(pa_prefill_workspace_size(8, 6000, 16, 8, 128, 2048, 0, &bytes, &splits) == PA_OK);
  EXPECT(splits == 1 && bytes > 0);

  /* nothing to do: returns before any pointer is used */
  EXPECT(pa_store_kv(NULL, NULL, 1024, 128, 1024, 128, NULL, NULL, NULL, 0, 8, 128, 256, 10,
                     PA_CACHE_BSHD, PA_DTYPE_BF16, NULL) == PA_OK);
  /* null device pointers with work to do */
  EXPECT(pa_store_kv(NULL, NULL, 1024, 128, 1024, 128, NULL, NULL, NULL, 4, 8, 128, 256, 10,
                     PA_CACHE_BHSD, PA_DTYPE_BF16, NULL) == PA_ERR_INVALID_ARG);
  EXPECT(pa_store_kv(NULL, NULL, 1024, 128, 1024, 128, NULL, NULL, NULL, 4, 8, 96, 256, 10,
                     PA_CACHE_BSHD, PA_DTYPE_BF16, NULL) == PA_ERR_UNSUPPORTED);
  EXPECT(pa_decode(NULL, 2048, 128, NULL, NULL, NULL, 16, NULL, 0, 16, 8, 128, 256, 100,
                   PA_CACHE_BSHD, 4096, 1024, 0.088f, NULL, 0, PA_DTYPE_BF16, NULL) == PA_OK);
  EXPECT(pa_store_decode(NULL, NULL, 1024, 128, 1024, 128, NULL, NULL, 2048, 128, NULL, NULL,
                         NULL, 16, NULL, 4, 16, 8, 128, 256, 100, PA_CACHE_BSHD, 4096, 1024,
                         0.088f, NULL, 0, PA_DTYPE_BF16, NULL) == PA_ERR_INVALID_ARG);
  EXPECT(pa_qk_norm_rope_store(NULL, 4096, NULL, NULL, NULL, NULL, 0, 16, 8, 128, 1e-6f, 1e6,
                               NULL, 2048, NULL, NULL, 256, 10, PA_CACHE_BSHD, PA_DTYPE_BF16,
                               NULL) == PA_OK);
  EXPECT(pa_prefill_varlen(NULL, 2048, 128, NULL, NULL, NULL, NULL, NULL, 8, 8, 6000, 16, 8, 128,
                           256, 64, PA_CACHE_BSHD, 2048, 2048, 0.088f, 0, NULL, 0, NULL, 2048,
                           128, PA_DTYPE_F32, NULL) == PA_ERR_UNSUPPORTED);
  EXPECT(pa_store_prefill_varlen(NULL, NULL, 1024, 128, 1024, 128, NULL, NULL, 2048, 128, NULL,
                                 NULL, NULL, NULL, NULL, 8, 8, 6000, 16, 8, 128, 256, 64,
                                 PA_CACHE_BSHD, 2048, 2048, 0.088f, 0, NULL, 0, NULL, 2048, 128,
                                 PA_DTYPE_BF16, NULL) == PA_ERR_INVALID_ARG);
  EXPECT(pa_prefill_plan(NULL, NULL, 0, 0, 16, 8, 128, 0, 0, 0, NULL, 0, NULL) == PA_OK);
  EXPECT(pa_prefill_plan(NULL, NULL, 8, 6000, 16, 8, 128, 2048, 2048, 0, NULL, 0, NULL) ==
         PA_ERR_INVALID_ARG);
  EXPECT(pa_prefill_varlen_planned(NULL, 2048, 128, NULL, NULL, NULL, NULL, NULL, 8, 8, 6000, 16,
                                   8, 128, 256, 64, PA_CACHE_BSHD, 2048, 2048, 0.088f, 0, NULL,
                                   0, NULL, 2048, 128, PA_DTYPE_F32, NULL) == PA_ERR_UNSUPPORTED);
  EXPECT(pa_store_prefill_varlen_planned(NULL, NULL, 1024, 128, 1024, 128, NULL, NULL, 2048, 128,
                                         NULL, NULL, NULL, NULL, NULL, 8, 8, 6000, 16, 8, 128,
                                         256, 64, PA_CACHE_BSHD, 2048, 2048, 0.088f, 0, NULL, 0,
                                         NULL, 2048, 128, PA_DTYPE_BF16,
                                         NULL) == PA_ERR_INVALID_ARG);
  EXPECT(pa_decode_shared_prefix(NULL, NULL, 1024, 128, 1024, 128, NULL, NULL, 2048, 128, NULL,
                                 NULL, NULL, 16, NULL, NULL, NULL, 1, 2048, 8, 16, 8, 128, 16,
                                 100, PA_CACHE_BSHD, 4096, 512, 0.088f, NULL, 0, PA_DTYPE_F32,
                                 NULL) == PA_ERR_UNSUPPORTED);
  if (failures == 0) printf("abi_check: all checks passed\n");
  return failures == 0 ? 0 : 1;
}
