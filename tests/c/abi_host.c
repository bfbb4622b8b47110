/* Plain-C client of libkvq: the header compiles as C99 and the host-only
 * entry points behave as documented (no GPU needed). */
#include <stdio.h>
#include <string.h>

#include "kvq.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

int main(void) {
  int64_t k = 0, total = 0, nch = 0, rows = 0;
  CHECK(kv_keep_count(8192, 0.3, &k) == KV_OK && k == 2457);
  CHECK(kv_keep_count(10, 0.05, &k) == KV_OK && k == 1);
  CHECK(kv_keep_count(0, 0.5, &k) == KV_ERR_INVALID_ARG);
  CHECK(kv_topk_total(32, 8, 8192, 0.3, 0, &total) == KV_OK && total == 256 * 2457);
  CHECK(kv_topk_total(48, 8, 16384, 0.1, 1, &total) == KV_OK && total == 48 * 13107);
  CHECK(kv_topk_total(1, 1, 100, 0.5, 2, &total) == KV_OK && total == 50);
  CHECK(kv_topk_total(1, 1, 100, 0.5, 3, &total) == KV_ERR_UNSUPPORTED);
  CHECK(kv_topk_workspace_bytes(32, 8, 8192, 0) == 0);
  CHECK(kv_topk_workspace_bytes(32, 8, 8192, 2) > 0);
  CHECK(kv_select_tokens_workspace_bytes(65536) > 0);
  CHECK(kv_chunk_layout(131072, 32, 2048, &nch, &rows) == KV_OK && nch == 64 &&
        rows == 64 * 32 + 131072);
  CHECK(strcmp(kv_status_string(KV_ERR_CAPACITY), "KV_ERR_CAPACITY") == 0);
  CHECK(kv_last_hip_error() == 0);
  /* argument errors are reported before anything touches a device */
  CHECK(kvscore_lse(NULL, NULL, NULL, NULL, 1, 1, 4, 128, 16, 2, 0.1f, NULL) ==
        KV_ERR_INVALID_ARG);
  CHECK(kv_compact((void*)0x10000, (void*)0x10000, (const int64_t*)0x10000,
                   (const int32_t*)0x10000, (void*)0x10000, (void*)0x10000, 1, 1, 96, 8, 4,
                   NULL) == KV_ERR_UNSUPPORTED);
  printf("%s (%d failures)\n", fails ? "FAILED" : "ok", fails);
  return fails ? 1 : 0;
}
