/* A plain C11 consumer of libanvil.so: compiled with the host C compiler against include/anvil.h
 * alone (no HIP or torch headers), it exercises the host-side contract that needs no GPU: the
 * version, the status strings, the workspace sizes, empty stacks as no-ops and the argument checks
 * that reject a call before anything is launched.  Prints "ok" and exits 0 when every check
 * holds; otherwise names the first failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "anvil.h"

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      printf("failed: %s (line %d)\n", #cond, __LINE__);         \
      return 1;                                                  \
    }                                                            \
  } while (0)

int main(void) {
  CHECK(anvil_version() > 0);
  for (int s = ANVIL_OK; s <= ANVIL_ERR_HIP; ++s) {
    const char* msg = anvil_status_string(s);
    CHECK(msg != NULL && strlen(msg) > 0);
  }
  CHECK(anvil_status_string(12345) != NULL);

  /* workspace: the mlp bank needs at least the ping-pong X and the A and B Grams */
  const size_t ws = anvil_workspace_bytes(24, 2816, 768);
  CHECK(ws >= (size_t)24 * 2816 * 768 * 2 + (size_t)2 * 24 * 768 * 768 * 2);
  CHECK(ws % 256 == 0);
  CHECK(anvil_workspace_bytes(1, 60, 32) == 0); /* m not a multiple of 8 */
  CHECK(anvil_workspace_bytes(0, 64, 32) == 0); /* empty stack */

  /* empty stacks succeed without touching memory (null pointers allowed) */
  CHECK(anvil_bank_step(NULL, NULL, 0.95f, 0.85f, 1.0f, NULL, 0, 64, 32, NULL) == ANVIL_OK);
  CHECK(anvil_bank_step(NULL, NULL, 0.95f, 0.85f, 1.0f, NULL, 2, 0, 32, NULL) == ANVIL_OK);

  /* rejected before any launch: negative sizes, unsupported shapes, null and misaligned pointers */
  CHECK(anvil_bank_step(NULL, NULL, 0.95f, 0.85f, 1.0f, NULL, -1, 64, 32, NULL) ==
        ANVIL_ERR_INVALID_ARG);
  float* fake = (float*)(uintptr_t)0x10000; /* never dereferenced: the checks fail first */
  uint16_t* fake16 = (uint16_t*)(uintptr_t)0x20000000;
  CHECK(anvil_bank_step(fake, fake, 0.95f, 0.85f, 1.0f, fake16, 1, 60, 32, NULL) ==
        ANVIL_ERR_UNSUPPORTED);
  CHECK(anvil_bank_step(NULL, fake, 0.95f, 0.85f, 1.0f, fake16, 1, 64, 32, NULL) ==
        ANVIL_ERR_INVALID_ARG);
  CHECK(anvil_bank_step((float*)((char*)fake + 4), fake, 0.95f, 0.85f, 1.0f, fake16, 1, 64, 32,
                        NULL) == ANVIL_ERR_MISALIGNED);
  /* the output overlapping the gradient */
  CHECK(anvil_bank_step(fake, (float*)(uintptr_t)0x40000000, 0.95f, 0.85f, 1.0f,
                        (uint16_t*)fake, 1, 64, 32, NULL) == ANVIL_ERR_ALIAS);
  printf("ok\n");
  return 0;
}
