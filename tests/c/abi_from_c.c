/* A plain C99 caller of the C ABI: includes only include/fp8mi.h, links only
 * the built library, and exercises the host-side paths (version, status
 * strings, argument errors) that need no GPU.  Prints one line per check and
 * exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "fp8mi.h"

static int fails = 0;

static void expect(const char* what, int got, int want) {
  printf("%s: %d (%s)\n", what, got, got == want ? "ok" : "UNEXPECTED");
  if (got != want) ++fails;
}

int main(void) {
  /* 16-byte aligned addresses that are never dereferenced: every call below is
   * refused during host-side validation, before anything is launched. */
  void* const p = (void*)0x10000;
  const int version = fp8mi_version();
  printf("version: %d (%s)\n", version, version > 0 ? "ok" : "UNEXPECTED");
  if (version <= 0) ++fails;
  if (strcmp(fp8mi_status_string(12345), "unknown status") != 0) ++fails;
  if (strcmp(fp8mi_status_string(FP8MI_OK), "unknown status") == 0) ++fails;
  /* null input */
  expect("quantize null x",
         fp8_quantize(NULL, FP8MI_BF16, 16, 16, FP8MI_E4M3, (const float*)p, (uint8_t*)p, NULL, NULL, NULL, NULL, 0,
                      NULL),
         FP8MI_ERR_NULL);
  /* format out of range */
  expect("quantize bad format",
         fp8_quantize(p, FP8MI_BF16, 16, 16, 7, (const float*)p, (uint8_t*)p, NULL, NULL, NULL, NULL, 0, NULL),
         FP8MI_ERR_FORMAT);
  /* K not a multiple of 16 */
  expect("gemm K % 16",
         fp8_gemm((const uint8_t*)p, FP8MI_E4M3, (const uint8_t*)p, FP8MI_E4M3, 0, 64, 64, 24, (const float*)p,
                  (const float*)p, p, FP8MI_F32, FP8MI_ACCUM_EXACT, NULL),
         FP8MI_ERR_ALIGN);
  /* history length 0 */
  expect("amax_update bad length",
         fp8_amax_update((float*)p, 0, (int32_t*)p, (const float*)p, FP8MI_E4M3, (float*)p, (float*)p, NULL, NULL),
         FP8MI_ERR_SHAPE);
  return fails ? 1 : 0;
}
