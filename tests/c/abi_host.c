/* Plain C use of the library's C interface: compiled with a C compiler against
 * include/attn.h and linked to libattn.so.  Calls only host-side entry points (the
 * split chooser, workspace sizes, status strings) and argument validation that fails
 * before any HIP call, so it runs without a GPU.  Prints "ok" on success. */
#include <stdio.h>
#include <string.h>

#include "attn.h"

static int fails = 0;
#define CHECK(cond)                                            \
  do {                                                         \
    if (!(cond)) {                                             \
      printf("FAILED line %d: %s\n", __LINE__, #cond);         \
      ++fails;                                                 \
    }                                                          \
  } while (0)

int main(void) {
  int chunk = 0, n_split = 0;
  CHECK(attn_decode_choose_split(8, 12, 4096, 64, 256, &chunk, &n_split) == ATTN_OK);
  CHECK(chunk == 192 && n_split == 22);
  CHECK(attn_decode_gqa_choose_split(8, 32, 8, 4096, 128, 256, &chunk, &n_split) == ATTN_OK);
  CHECK(chunk == 192 && n_split == 22);
  CHECK(attn_decode_choose_split(0, 12, 4096, 64, 256, &chunk, &n_split) == ATTN_ERR_INVALID_ARG);
  CHECK(strlen(attn_last_error()) > 0);
  CHECK(attn_decode_workspace_bytes(2, 3, 4, 64) == (size_t)2 * 3 * 4 * 66 * 4);
  CHECK(attn_backward_workspace_bytes(2, 8, 100) == (size_t)2 * 2 * 8 * 100 * 4);
  CHECK(strcmp(attn_status_string(ATTN_OK), "unknown status") != 0);
  /* Invalid arguments are refused before any HIP call. */
  CHECK(attn_prefill(NULL, NULL, NULL, NULL, 1, 1, 8, 64, ATTN_F16, 0, 0.125f, NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(attn_prefill((void*)16, (void*)32, (void*)48, (void*)64, 1, 1, 8, 80, ATTN_F16, 0, 0.125f, NULL) ==
        ATTN_ERR_UNSUPPORTED);
  if (fails == 0) printf("ok\n");
  return fails != 0;
}
