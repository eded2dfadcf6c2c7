/* A plain C consumer of libdcptopk: it compiles against include/libdcptopk.h
 * and links the library like any C program would.  It makes only calls that
 * fail validation or have nothing to do (rows == 0), so it needs no GPU; it
 * prints one line per check and returns the number of failed checks. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "libdcptopk.h"

static int failures = 0;

static void expect(const char* what, long got, long want) {
  const int ok = got == want;
  printf("%s %s: got %ld, want %ld\n", ok ? "ok  " : "FAIL", what, got, want);
  failures += !ok;
}

int main(void) {
  dcp_topk_cand* fake_in = (dcp_topk_cand*)(uintptr_t)0x7F0000000000ull;   /* never dereferenced */
  dcp_topk_cand* fake_out = (dcp_topk_cand*)(uintptr_t)0x7F0010000000ull;
  expect("sizeof(dcp_topk_cand)", (long)sizeof(dcp_topk_cand), 8);
  expect("status string of OK", strcmp(dcp_topk_status_string(DCP_TOPK_OK), "ok"), 0);
  expect("workspace bytes, 5000 rows, dcp 4, local_k 2048",
         (long)dcp_topk_merge_workspace_bytes(5000, 4, 2048), (long)DCP_TOPK_MERGE_ROWS * 4 * 2048 * 8);
  expect("select, no rows", dcp_topk_select(NULL, 0, 8192, 2048, NULL, NULL), DCP_TOPK_OK);
  expect("select, k = 0", dcp_topk_select(fake_in, 1, 8192, 0, fake_out, NULL), DCP_TOPK_EINVAL);
  expect("select, too many candidates", dcp_topk_select(fake_in, 1, DCP_TOPK_MAX_CANDIDATES + 1, 1, fake_out, NULL),
         DCP_TOPK_EUNSUPPORTED);
  expect("split workspace bytes, 1 row, 8192 candidates, 2 parts",
         (long)dcp_topk_select_split_workspace_bytes(1, 8192, 2), 256L + 16640L + 65536L + 32768L);
  expect("split select, parts past the limit",
         dcp_topk_select_split(fake_in, 1, 8192, 2048, DCP_TOPK_SPLIT_MAX_PARTS + 1, NULL, 0, fake_out, NULL),
         DCP_TOPK_EUNSUPPORTED);
  expect("split select, no workspace", dcp_topk_select_split(fake_in, 1, 8192, 2048, 2, NULL, 0, fake_out, NULL),
         DCP_TOPK_EWORKSPACE);
  expect("pack, no rows", dcp_topk_pack(NULL, NULL, 0, NULL, 0, 0, 16, NULL, 0, NULL), DCP_TOPK_OK);
  {
    const float* sc[1] = {(const float*)(uintptr_t)0x7F0020000000ull};
    const int32_t* ix[1] = {(const int32_t*)(uintptr_t)0x7F0030000000ull};
    const int32_t* rs[1] = {(const int32_t*)(uintptr_t)0x7F0040000000ull};
    const int32_t offs[1] = {0};
    expect("fused merge, local_k not a multiple of 64",
           dcp_topk_merge_fused(sc, ix, rs, offs, 1, 4, 100, 10, fake_out, NULL), DCP_TOPK_EUNSUPPORTED);
    expect("chunked merge, workspace too small",
           dcp_topk_merge_chunked(sc, ix, rs, offs, 1, 4, 128, 10, (void*)(uintptr_t)0x7F0050000000ull, 16, fake_out,
                                  NULL),
           DCP_TOPK_EWORKSPACE);
    expect("static-scratch merge, 1024 rows of dcp 1 x 16384 (128 MiB of workspace)",
           dcp_topk_merge_chunked_static(sc, ix, rs, offs, 1, 1024, 16384, 10, fake_out, NULL), DCP_TOPK_ESCRATCH);
    expect("static-scratch merge, no rows", dcp_topk_merge_chunked_static(sc, ix, rs, offs, 1, 0, 2048, 10, NULL, NULL),
           DCP_TOPK_OK);
  }
  expect("local top-K, no rows", dcp_topk_local(NULL, 0, NULL, 0, 4096, 2048, NULL, NULL, 2048, NULL), DCP_TOPK_OK);
  expect("local top-K, k = 0",
         dcp_topk_local((const float*)fake_in, 4096, NULL, 1, 4096, 0, (float*)fake_out, (int32_t*)fake_in, 2048, NULL),
         DCP_TOPK_EINVAL);
  return failures;
}
