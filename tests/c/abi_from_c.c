/*
 * The library's C ABI used from plain C99: include/pkv.h compiles as C, the
 * program links against libpkv.so, and calls whose arguments fail the
 * host-side checks return their documented status and message before any
 * HIP call (so no GPU is needed). Workspace-size queries are host
 * arithmetic. Prints "ok" and exits 0 when every check holds.
 */
#include <stdio.h>
#include <string.h>

#include "pkv.h"

static int failures = 0;

static void expect(int cond, const char *what, int line) {
  if (!cond) {
    printf("FAIL line %d: %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

static int message_has(const char *needle) {
  const char *m = pkv_last_error();
  return m != NULL && strstr(m, needle) != NULL;
}

int main(void) {
  int32_t dummy[4] = {0, 0, 0, 0};

  EXPECT(pkv_abi_version() == PKV_ABI_VERSION);

  /* index helpers: ranges and null pointers */
  EXPECT(pkv_get_seq_lens(NULL, NULL, -1, 16, NULL, NULL) == PKV_ERR_INVALID_ARG);
  EXPECT(message_has("pkv_get_seq_lens"));
  EXPECT(pkv_get_seq_lens(dummy, dummy, 1, 0, dummy, NULL) == PKV_ERR_INVALID_ARG);
  EXPECT(pkv_get_seq_lens(NULL, dummy, 1, 16, dummy, NULL) == PKV_ERR_INVALID_ARG);
  /* an empty batch is valid and launches nothing */
  EXPECT(pkv_get_seq_lens(NULL, NULL, 0, 16, NULL, NULL) == PKV_OK);
  EXPECT(pkv_get_batch_indices_positions(dummy, dummy, 1, -1, dummy, dummy, NULL) ==
         PKV_ERR_INVALID_ARG);
  EXPECT(message_has("pkv_get_batch_indices_positions"));
  EXPECT(pkv_csr_to_block_tables(dummy, dummy, 1, 0, dummy, NULL) == PKV_ERR_INVALID_ARG);
  EXPECT(message_has("pkv_csr_to_block_tables"));

  /* workspace sizes: host arithmetic only */
  EXPECT(pkv_prefill_workspace_size(4) > 0);
  EXPECT(pkv_prefill_workspace_size(100) >= pkv_prefill_workspace_size(4));
  /* one short request needs no split partials; 256 long ones do */
  EXPECT(pkv_decode_workspace_size(1, 1, 32, 8, 128, 37, -1) == 0);
  EXPECT(pkv_decode_workspace_size(256, 1, 32, 8, 128, 8192, -1) > 0);

  printf("%s\n", failures ? "FAILED" : "ok");
  return failures != 0;
}
