/* A plain-C consumer of libcpthd's C ABI (include/cpthd.h, include/cpthd_timing.h).
 *
 * Only host-side behaviour is exercised, so it runs without a GPU: workspace sizes, status strings, and
 * argument refusals that every entry point returns before anything is launched or any pointer is touched
 * (the pointers below are never dereferenced).  It checks that the headers compile as C and that a C program
 * links and calls the library with no Python or torch in between.  Built and run by tests/test_c_consumer.py;
 * prints "ok" and exits 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "cpthd.h"
#include "cpthd_timing.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      printf("FAIL line %d: %s\n", __LINE__, #cond);                  \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  /* workspace sizes for the long-context share: 131072 tokens, cp 8, 64 q / 8 kv heads, head_dim 128 */
  const size_t full = cpthd_attn_workspace_bytes(131072, 8, 64, 8, 128, 64);
  const size_t least = cpthd_attn_workspace_min_bytes(131072, 8, 64, 8, 128, 64);
  CHECK(full > 0);
  CHECK(least > 0 && least < full);
  CHECK(cpthd_attn_workspace_bytes(131072, 8, 64, 8, 48, 64) == 0);  /* head_dim outside {16, 32, 64, 128} */
  CHECK(cpthd_attn_workspace_bytes(131072, 8, 64, 7, 128, 64) == 0); /* 64 q heads over 7 kv heads */

  const char* msg = cpthd_status_string(CPTHD_ERR_HEADS);
  CHECK(msg != NULL && strlen(msg) > 0);
  CHECK(strcmp(cpthd_status_string(CPTHD_OK), cpthd_status_string(CPTHD_ERR_NULL)) != 0);

  /* fake, 256-byte aligned addresses: every call below is refused on its arguments first */
  void* const P = (void*)(size_t)0x100000;
  const int32_t* const cu = (const int32_t*)P;
  int32_t* const out = (int32_t*)P;

  CHECK(cpthd_partition_indices(NULL, 3, 28, 2, 0, CPTHD_DUAL_CHUNK_SWAP, out, NULL, NULL) == CPTHD_ERR_NULL);
  CHECK(cpthd_partition_indices(cu, 3, 28, 2, 2, CPTHD_DUAL_CHUNK_SWAP, out, NULL, NULL) == CPTHD_ERR_RANK);
  CHECK(cpthd_partition_indices(cu, 3, 28, 2, 0, 7, out, NULL, NULL) == CPTHD_ERR_STRATEGY);

  const size_t ws = cpthd_attn_workspace_bytes(64, 2, 4, 2, 16, 4);
  CHECK(cpthd_attn_plan(cu, cu, 4, 64, 64, 2, 0, CPTHD_DUAL_CHUNK_SWAP, 4, 2, 48, P, ws, NULL, NULL) ==
        CPTHD_ERR_HEADS);
  CHECK(cpthd_attn_fwd(P, P, P, cu, cu, 4, 64, 64, 2, 0, CPTHD_DUAL_CHUNK_SWAP, 4, 2, 16, 0.25f, 0, -1, 0, P,
                       (float*)P, P, ws, NULL, NULL) == CPTHD_ERR_MASK);
  CHECK(cpthd_attn_fwd(P, P, P, NULL, cu, 4, 64, 64, 2, 0, CPTHD_DUAL_CHUNK_SWAP, 4, 2, 16, 0.25f, 1, -1, 0, P,
                       (float*)P, P, ws, NULL, NULL) == CPTHD_ERR_NULL);
  CHECK(cpthd_attn_bwd(P, P, P, P, P, (const float*)P, cu, cu, 4, 64, 64, 2, 0, CPTHD_NO_LOAD_BALANCE, 4, 2, 16,
                       0.25f, 1, -1, 1, (float*)P, (float*)P, (float*)P, P, ws, NULL, NULL) == CPTHD_ERR_MASK);
  CHECK(cpthd_attn_fwd_timed(P, P, P, cu, cu, 4, 64, 64, 2, 0, 5, 4, 2, 16, 0.25f, 1, -1, 0, P, (float*)P, P, ws,
                             NULL, NULL, 0, NULL, 0) == CPTHD_ERR_STRATEGY);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
