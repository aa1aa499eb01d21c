/* The C-ABI from plain C99 (no C++, no Python): the header compiles under
   -std=c99 -pedantic, the library links, and the host-side paths answer as
   documented. Only calls that return before any launch are made, so no GPU
   is needed. Prints "ok" or the first failure. */
#include <stdio.h>
#include <string.h>

#include "nvfp4_gemv.h"

static int fails = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAIL %s (last error: %s)\n", what, nvfp4_last_error());
    ++fails;
  }
}

int main(void) {
  float y[4];
  int s;
  expect(nvfp4_abi_version() == NVFP4_ABI_VERSION, "abi version");
  for (s = 0; s <= 7; ++s) {
    const char* t = nvfp4_status_string((nvfp4_status)s);
    expect(t != NULL && t[0] != '\0', "status string");
  }
  expect(nvfp4_status_string((nvfp4_status)99) != NULL, "unknown status string");

  /* shapes are checked before pointers */
  expect(nvfp4_gemv(NULL, NULL, NULL, NULL, -1, 4, 32, y, NULL) == NVFP4_ERR_SHAPE,
         "gemv negative M");
  expect(strlen(nvfp4_last_error()) > 0, "last error after a failure");
  expect(nvfp4_gemv(NULL, NULL, NULL, NULL, 1, 4, 48, y, NULL) == NVFP4_ERR_SHAPE,
         "gemv K not a multiple of 32");
  expect(nvfp4_gemv(NULL, NULL, NULL, NULL, NVFP4_MAX_M + 1, 4, 32, y, NULL) ==
             NVFP4_ERR_UNSUPPORTED,
         "gemv M above the maximum");
  expect(nvfp4_gemv(NULL, NULL, NULL, NULL, 1, NVFP4_MAX_N + 1, 32, y, NULL) ==
             NVFP4_ERR_UNSUPPORTED,
         "gemv N above the maximum");
  expect(nvfp4_gemv(NULL, NULL, NULL, NULL, 1, 0, 32, y, NULL) == NVFP4_OK,
         "gemv with N = 0 does nothing");
  expect(nvfp4_moe_gemv(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 4, 64, 48, 2,
                        y, NULL, 0, NULL) == NVFP4_ERR_SHAPE,
         "moe I not a multiple of 32");

  /* workspace queries: h[M*topk, I] bf16 rounded up to 256 bytes; 0 for bad sizes */
  expect(nvfp4_moe_workspace_bytes(8, 4096, 1536, 8) == (size_t)(64 * 1536 * 2),
         "moe workspace bytes");
  expect(nvfp4_moe_workspace_bytes(1, 64, 32, 3) == 256, "moe workspace rounding");
  expect(nvfp4_moe_w4a4_workspace_bytes(-1, 64, 32, 3, 0) == 0, "w4a4 moe bad size");
  expect(nvfp4_gemv_w4a4_workspace_bytes(2, 4096) >= (size_t)(2 * 4096 * 2 + 4),
         "w4a4 gemv workspace bytes");

  if (fails == 0) printf("ok\n");
  return fails ? 1 : 0;
}
