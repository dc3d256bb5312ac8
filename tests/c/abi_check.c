/* abi_check.c -- the C ABI from plain C99: the header compiles without C++,
 * the library links, and the host-only entry points (argument checks, path
 * choice, status strings) answer as the header documents. Makes no HIP call:
 * every pointer below is a stand-in address that is never dereferenced. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mi355_attn.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: got %d want %d\n", what, got, want);
    ++failures;
  }
}

int main(void) {
  const uintptr_t sz = (uintptr_t)1 << 34;
  const void *q = (const void *)(1 * sz), *k = (const void *)(2 * sz), *v = (const void *)(3 * sz);
  void *o = (void *)(4 * sz);
  float *lse = (float *)(5 * sz);

  expect("attn_fwd_validate ok", attn_fwd_validate(q, k, v, o, lse, 4, 16, 4096, 4096, 128,
                                                   0.08838835f, 0, MI355_ATTN_BF16),
         MI355_ATTN_OK);
  expect("attn_fwd_validate D=96", attn_fwd_validate(q, k, v, o, lse, 1, 1, 8, 8, 96, 1.0f, 0,
                                                     MI355_ATTN_FP32),
         MI355_ATTN_ERR_UNSUPPORTED);
  expect("attn_fwd_validate misaligned",
         attn_fwd_validate((const char *)q + 4, k, v, o, lse, 1, 1, 8, 8, 64, 1.0f, 0,
                           MI355_ATTN_FP32),
         MI355_ATTN_ERR_MISALIGNED);
  expect("attn_fwd_validate causal=2", attn_fwd_validate(q, k, v, o, lse, 1, 1, 8, 8, 64, 1.0f, 2,
                                                         MI355_ATTN_FP32),
         MI355_ATTN_ERR_INVALID_ARG);
  expect("attn_fwd empty", attn_fwd(0, 0, 0, 0, 0, 0, 4, 8, 8, 64, 1.0f, 0, MI355_ATTN_FP32, 0),
         MI355_ATTN_OK);
  expect("select small", attn_fwd_select_path(128, 4, 32, 32, 16, 0, MI355_ATTN_FP32),
         MI355_ATTN_PATH_SMALL);
  expect("select main", attn_fwd_select_path(4, 16, 4096, 4096, 128, 0, MI355_ATTN_BF16),
         MI355_ATTN_PATH_MAIN);
  expect("attn_bwd_validate fp32", attn_bwd_validate(q, k, v, o, lse, (const void *)(6 * sz),
                                                     (const void *)(7 * sz), (const void *)(8 * sz),
                                                     (const void *)(9 * sz),
                                                     (const float *)(10 * sz), 1, 1, 64, 64, 64,
                                                     0.125f, 0, MI355_ATTN_FP32),
         MI355_ATTN_ERR_UNSUPPORTED);

  const float *x = (const float *)(11 * sz), *w[5];
  for (int i = 0; i < 5; ++i) w[i] = (const float *)((12 + (uintptr_t)i) * sz);
  float *out = (float *)(17 * sz);
  expect("axial_pass_validate row", axial_pass_validate(x, out, w[0], w[1], w[2], w[3], w[4], 4, 32,
                                                        32, 64, 4, MI355_AXIAL_ROW, 1e-5f),
         MI355_ATTN_OK);
  expect("axial_pass_validate C=32", axial_pass_validate(x, out, w[0], w[1], w[2], w[3], w[4], 4,
                                                         32, 32, 32, 4, MI355_AXIAL_COL, 1e-5f),
         MI355_ATTN_ERR_UNSUPPORTED);
  expect("axial_pass_split out of place", axial_pass_split(x, out, 4, 32, 32, MI355_AXIAL_COL), 2);
  expect("axial_pass_split in place", axial_pass_split(out, out, 4, 32, 32, MI355_AXIAL_COL), 1);
  expect("axial_block empty", axial_block(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 32, 32, 64, 4,
                                          1e-5f, 0),
         MI355_ATTN_OK);

  if (strcmp(attn_status_string(MI355_ATTN_ERR_MISALIGNED), "misaligned pointer") != 0) {
    printf("FAIL status string\n");
    ++failures;
  }
  if (failures == 0) printf("abi_check: all checks passed\n");
  return failures != 0;
}
