/* A C99 caller of libattn.so: the header compiles as plain C and every
 * validation path answers before any launch (fake, never dereferenced device
 * addresses; no GPU is needed). Exit status 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %d, want %d (%s)\n", what, got, want, attn_status_string(got));
    ++failures;
  }
}

static void* addr(int i) { return (void*)(uintptr_t)(0x1000000000ull * (uint64_t)(i + 1)); }

int main(void) {
  const int B = 1, H = 2, N = 8, d = 64;
  size_t ws = attn_bwd_workspace_bytes(B, H, N, d);
  if (ws == 0 || attn_bwd_workspace_bytes(B, H, N, 80) != 0) {
    fprintf(stderr, "FAIL workspace size\n");
    ++failures;
  }
  if (strcmp(attn_status_string(ATTN_OK), "ok") != 0) ++failures;

  expect(attn_fwd(NULL, addr(1), addr(2), addr(3), (float*)addr(4), B, H, N, d, 0.125f, NULL),
         ATTN_ERR_INVALID_ARG, "fwd null q");
  expect(attn_fwd(addr(0), addr(1), addr(2), addr(3), (float*)addr(4), B, H, N, 80, 0.125f, NULL),
         ATTN_ERR_UNSUPPORTED, "fwd d_k 80");
  expect(attn_fwd(addr(0), addr(1), addr(2), addr(0), (float*)addr(4), B, H, N, d, 0.125f, NULL),
         ATTN_ERR_INVALID_ARG, "fwd o aliases q");
  expect(attn_fwd_f32((const float*)addr(0), (const float*)addr(1), (const float*)addr(2), (float*)addr(3),
                      (float*)addr(4), 0, H, N, d, 0.125f, NULL),
         ATTN_ERR_INVALID_ARG, "fwd_f32 B = 0");
  expect(attn_fwd_ex(ATTN_DTYPE_F16, ATTN_LAYOUT_QKV_PACKED, addr(0), addr(1), addr(2), addr(3), (float*)addr(4), B,
                     H, N, d, 0.125f, 0, NULL, NULL),
         ATTN_ERR_INVALID_ARG, "fwd_ex packed k not after q");
  expect(attn_fwd_ex(ATTN_DTYPE_BF16, 7, addr(0), addr(1), addr(2), addr(3), (float*)addr(4), B, H, N, d, 0.125f, 0,
                     NULL, NULL),
         ATTN_ERR_UNSUPPORTED, "fwd_ex unknown layout");
  expect(attn_fwd_ex(ATTN_DTYPE_BF16, ATTN_LAYOUT_BHND, addr(0), addr(1), addr(2), addr(3), (float*)addr(4), B, H, N,
                     d, 0.125f, 2, NULL, NULL),
         ATTN_ERR_INVALID_ARG, "fwd_ex causal 2");
  expect(attn_bwd(addr(0), addr(1), addr(2), addr(3), (const float*)addr(4), addr(5), addr(6), addr(7), addr(8), B, H,
                  N, d, 0.125f, NULL, ws, NULL),
         ATTN_ERR_WORKSPACE, "bwd no workspace");
  expect(attn_bwd_stage(4, ATTN_DTYPE_BF16, ATTN_LAYOUT_BHND, addr(0), addr(1), addr(2), addr(3), (const float*)addr(4),
                        addr(5), addr(6), addr(7), addr(8), B, H, N, d, 0.125f, 0, NULL, addr(9), ws, NULL),
         ATTN_ERR_INVALID_ARG, "bwd stage 4");
  expect(attn_bwd_ex_noalloc(ATTN_DTYPE_BF16, ATTN_LAYOUT_BHND, addr(0), addr(1), addr(2), addr(3),
                             (const float*)addr(4), addr(5), addr(6), addr(7), addr(8), 8, 16, 16448, d, 0.125f, 0,
                             NULL, NULL),
         ATTN_ERR_WORKSPACE, "bwd_ex_noalloc beyond its 16 MiB workspace");
  expect(attn_bwd_f32((const float*)addr(0), (const float*)addr(1), (const float*)addr(2), (const float*)addr(3),
                      (const float*)addr(4), (const float*)addr(5), (float*)addr(6), (float*)addr(6), (float*)addr(8),
                      B, H, N, d, 0.125f, addr(9), ws, NULL),
         ATTN_ERR_INVALID_ARG, "bwd_f32 dq == dk");
  expect(attn_qkv_proj(ATTN_DTYPE_BF16, addr(0), addr(1), addr(0), 2, 5, 64, 2, 32, NULL), ATTN_ERR_INVALID_ARG,
         "qkv_proj output on x");
  expect(attn_qkv_proj(ATTN_DTYPE_BF16, addr(0), addr(1), addr(2), 2, 5, 60, 2, 32, NULL), ATTN_ERR_UNSUPPORTED,
         "qkv_proj D = 60");
  expect(attn_qkv_proj_bwd(ATTN_DTYPE_F16, addr(0), addr(1), addr(2), addr(3), addr(3), 2, 5, 64, 2, 32, NULL, 0,
                           NULL),
         ATTN_ERR_INVALID_ARG, "qkv_proj_bwd dx == dw");
  expect(attn_qkv_proj_bwd(ATTN_DTYPE_BF16, addr(0), addr(1), addr(2), addr(3), addr(4), 32, 196, 768, 12, 64, NULL, 0,
                           NULL),
         ATTN_ERR_WORKSPACE, "qkv_proj_bwd without its workspace");
  if (failures == 0) printf("abi_check: all checks passed\n");
  return failures == 0 ? 0 : 1;
}
