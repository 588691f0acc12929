/*
 * Host-side driver of libfa's C ABI for the sanitizer test: every call here
 * returns from host validation before any HIP call (fake device addresses,
 * invalid descriptors, host-only helpers), so it runs without a GPU.  Built
 * and run by tests/test_host_sanitizer.py against a copy of libfa whose host
 * code carries AddressSanitizer and UndefinedBehaviorSanitizer; exit status 0
 * means every call returned the expected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

static int failures = 0;
#define EXPECT(expr, want)                                                            \
  do {                                                                                \
    int got_ = (int)(expr);                                                           \
    if (got_ != (want)) {                                                             \
      fprintf(stderr, "line %d: %s = %d, expected %d (%s)\n", __LINE__, #expr, got_, \
              (int)(want), fa_last_error());                                          \
      ++failures;                                                                     \
    }                                                                                 \
  } while (0)

#define GB ((uintptr_t)1 << 30)
static void* P(uintptr_t v) { return (void*)(v * GB); }

int main(void) {
  int32_t lens[3] = {4096, 1000, 96};
  fa_desc_t d;
  memset(&d, 0, sizeof d);
  d.dtype = FA_BF16;
  d.batch = 3;
  d.n_q_heads = 8;
  d.n_kv_heads = 2;
  d.head_dim = 128;
  d.n_comp_dims = 64;
  d.sink = 32;
  d.recent = 64;
  d.n_coef = 33;
  d.seq_len = lens;
  d.dims = (const int32_t*)P(10);
  size_t n = 0;
  uint64_t full = 0, comp = 0;

  /* workspace queries, valid and invalid */
  EXPECT(fa_decode_workspace_size(&d, &n), FA_OK);
  EXPECT(fa_project_workspace_size(&d, &n), FA_OK);
  EXPECT(fa_attend_workspace_size(&d, 40, &n), FA_OK);
  EXPECT(fa_attend_workspace_size(&d, 0, &n), FA_ERR_SHAPE);
  EXPECT(fa_attend_workspace_size(&d, 1025, &n), FA_ERR_SHAPE);
  EXPECT(fa_decode_workspace_size(NULL, &n), FA_ERR_NULL);
  EXPECT(fa_decode_workspace_size(&d, NULL), FA_ERR_NULL);
  fa_desc_t bad = d;
  bad.dtype = 9;
  EXPECT(fa_decode_workspace_size(&bad, &n), FA_ERR_DTYPE);
  bad = d;
  bad.n_q_heads = 7;
  EXPECT(fa_decode_workspace_size(&bad, &n), FA_ERR_SHAPE);
  bad = d;
  bad.n_coef = 5000;
  EXPECT(fa_project_workspace_size(&bad, &n), FA_ERR_SHAPE);
  bad = d;
  bad.seq_len = NULL;
  EXPECT(fa_decode_workspace_size(&bad, &n), FA_ERR_NULL);
  bad = d;
  bad.batch = 65;
  EXPECT(fa_decode_workspace_size(&bad, &n), FA_ERR_SHAPE);

  /* calls that fail validation before any HIP call */
  EXPECT(fa_decode(&d, NULL, P(2), P(3), P(4), P(5), (float*)P(6), (float*)P(7), 0.1f, (float*)P(8),
                   P(9), (size_t)1 << 30, NULL), FA_ERR_NULL);
  EXPECT(fa_decode(&d, P(1), P(2), P(3), P(4), P(5), (float*)P(6), (float*)P(7), 0.1f,
                   (float*)((char*)P(1) + 64), P(9), (size_t)1 << 30, NULL), FA_ERR_ALIAS);
  EXPECT(fa_decode(&d, P(1), P(2), P(3), P(4), P(5), (float*)P(6), (float*)P(7), 0.1f, (float*)P(8),
                   P(9), 16, NULL), FA_ERR_WORKSPACE);
  EXPECT(fa_attend(&d, 4, P(1), P(2), P(3), P(4), P(5), (float*)P(6), (float*)P(7), 0.1f,
                   (float*)P(8), (float*)((char*)P(8) + 64), P(9), (size_t)1 << 30, NULL), FA_ERR_ALIAS);
  EXPECT(fa_project(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), FA_ERR_NULL);
  EXPECT(fa_project(&d, P(1), NULL, (float*)((char*)P(1) + 64), NULL, NULL, NULL, P(9), (size_t)1 << 30,
                    NULL), FA_ERR_ALIAS);

  /* host-only helpers */
  /* fixed basis period: validation and fa_append's host checks (no launch) */
  bad = d;
  bad.period = 3000; /* sequence 0's middle (4000) past the period */
  EXPECT(fa_decode_workspace_size(&bad, &n), FA_ERR_SHAPE);
  bad = d;
  bad.period = -5;
  EXPECT(fa_project_workspace_size(&bad, &n), FA_ERR_SHAPE);
  bad = d;
  bad.period = 5000;
  EXPECT(fa_decode_workspace_size(&bad, &n), FA_OK);
  EXPECT(fa_append(&d, P(1), P(2), (float*)P(3), (float*)P(4), P(5), P(6), NULL), FA_ERR_SHAPE);
  EXPECT(fa_append(&bad, NULL, P(2), (float*)P(3), (float*)P(4), P(5), P(6), NULL), FA_ERR_NULL);
  EXPECT(fa_append(&bad, P(1), P(2), (float*)P(3), (float*)P(4), P(5), NULL, NULL), FA_ERR_NULL);
  EXPECT(fa_append(&bad, P(1), P(2), (float*)P(1), (float*)P(4), P(5), P(6), NULL), FA_ERR_ALIAS);
  bad.period = 4000; /* one more middle token would not fit */
  EXPECT(fa_append(&bad, P(1), P(2), (float*)P(3), (float*)P(4), P(5), P(6), NULL), FA_ERR_SHAPE);

  /* dimension analysis: workspace query and host errors (no launch) */
  EXPECT(fa_dim_sensitivity_workspace_size(&d, 4, &n), FA_OK);
  EXPECT(fa_dim_sensitivity_workspace_size(&d, 0, &n), FA_ERR_SHAPE);
  EXPECT(fa_dim_sensitivity(&d, 4, NULL, P(2), P(3), 0.1f, (float*)P(4), P(5), (size_t)1 << 40, NULL),
         FA_ERR_NULL);
  EXPECT(fa_dim_sensitivity(&d, 4, P(1), P(2), P(3), 0.1f, (float*)P(4), P(5), 64, NULL), FA_ERR_WORKSPACE);
  EXPECT(fa_dim_sensitivity(&d, 4, P(1), P(2), P(3), 0.1f, (float*)P(2), P(5), (size_t)1 << 40, NULL),
         FA_ERR_ALIAS);

  EXPECT(fa_coef_budget(4000, 0.3), 2399);
  EXPECT(fa_coef_budget(3, 0.3), 1);
  EXPECT(fa_coef_budget(0, 0.3), 0);
  EXPECT(fa_cache_bytes(&d, &full, &comp), FA_OK);
  EXPECT(full > comp, 1);
  EXPECT(fa_cache_bytes(&d, NULL, NULL), FA_OK);
  for (int s = 0; s <= 7; ++s) EXPECT(fa_status_string((fa_status_t)s) != NULL, 1);
  EXPECT(fa_last_error() != NULL, 1);
  EXPECT(fa_version() >= 100, 1);
  EXPECT(fa_time_main_kernel(P(1), NULL), FA_ERR_NULL);
  EXPECT(fa_time_main_kernel(NULL, P(2)), FA_ERR_NULL);
  EXPECT(fa_time_main_kernel(NULL, NULL), FA_OK);

  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("api_driver: all checks passed\n");
  return failures ? 1 : 0;
}
