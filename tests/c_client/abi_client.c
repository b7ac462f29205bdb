/* A plain C caller of the library: includes the public header, links
 * liblmhead.so and exercises the calls that need no GPU (size queries,
 * status strings, host-side argument checks). Exits 0 when every check
 * holds, else prints the failing check and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lmhead.h"

static int failures = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

int main(void) {
  /* pointers that pass the host checks (16-byte aligned) but are never dereferenced */
  void* fake = (void*)(uintptr_t)0x10000;
  float* ffake = (float*)fake;

  CHECK(lmhead_version() >= 300);
  CHECK(strlen(lmhead_status_string(LMHEAD_OK)) > 0);
  CHECK(lmhead_saved_bytes(0) == 1024);
  CHECK(lmhead_saved_bytes(16384) == 1024 + 4 * 16384 * 4);
  CHECK(lmhead_fwd_workspace_bytes(16384, 4096, 131072) > 0);
  CHECK(lmhead_fwd_workspace_bytes(10, 100, 1000) == 0); /* H % 64 != 0 */
  CHECK(lmhead_bwd_workspace_bytes(16384, 4096, 131072, 0) >
        (size_t)16384 * 131072 * 2); /* holds the whole batch's bf16 dZ */
  CHECK(lmhead_mfma_probe_workspace_bytes() > 0);

  /* host-side checks fail before anything is enqueued */
  CHECK(lmhead_fwd(fake, fake, fake, NULL, 8, 96, 100, 1, 1, ffake, ffake, fake, 1 << 20, fake,
                   1 << 30, NULL) == LMHEAD_ERR_UNSUPPORTED);
  CHECK(lmhead_fwd(fake, fake, fake, NULL, 8, 64, 100, 0, 1, ffake, NULL, fake, 1 << 20, fake,
                   1 << 30, NULL) == LMHEAD_ERR_INVALID_ARG);
  CHECK(lmhead_fwd_blocksparse(fake, fake, fake, NULL, 8, 64, 100, 1, 1, ffake, ffake, fake, 16,
                               fake, 1 << 30, NULL) == LMHEAD_ERR_WORKSPACE);
  CHECK(lmhead_bwd(fake, fake, fake, -1, 64, 100, 0, fake, 1 << 20, ffake, NULL, ffake, ffake, 0,
                   fake, 1 << 30, NULL) == LMHEAD_ERR_INVALID_ARG);
  CHECK(lmhead_mfma_probe(fake, 64, NULL, 64, 10, fake, 1 << 20, NULL, NULL, NULL, NULL) ==
        LMHEAD_ERR_INVALID_ARG);

  /* size limits: N <= 2^24, H <= 2^20, V <= 2^22 */
  const int64_t max_n = (int64_t)1 << 24;
  CHECK(lmhead_fwd_workspace_bytes(max_n, 64, 1000) > 0);
  CHECK(lmhead_fwd_workspace_bytes(max_n + 1, 64, 1000) == 0);
  CHECK(lmhead_bwd_workspace_bytes(max_n + 1, 64, 1000, 0) == 0);
  CHECK(lmhead_fwd(fake, fake, fake, NULL, max_n + 1, 64, 100, 1, 1, ffake, ffake, fake, 1 << 20,
                   fake, 1 << 30, NULL) == LMHEAD_ERR_UNSUPPORTED);
  CHECK(lmhead_bwd(fake, fake, fake, max_n + 1, 64, 100, 0, fake, 1 << 20, ffake, NULL, ffake,
                   ffake, 0, fake, 1 << 30, NULL) == LMHEAD_ERR_UNSUPPORTED);
  CHECK(lmhead_fwd(fake, fake, fake, NULL, 8, 64, ((int64_t)1 << 22) + 1, 1, 1, ffake, ffake, fake,
                   1 << 20, fake, 1 << 30, NULL) == LMHEAD_ERR_UNSUPPORTED);

  if (failures == 0) printf("abi client: all checks passed\n");
  return failures == 0 ? 0 : 1;
}
