/* Compiled as C99 against include/sdpa_attn.h and linked to the built
 * library: the header is plain C and the host-only entry points behave as it
 * documents.  No GPU is touched.  Prints "ok" and exits 0 on success. */
#include <stdio.h>
#include <string.h>

#include "sdpa_attn.h"

#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

int main(void) {
  struct attn_params p;
  memset(&p, 0, sizeof p);
  p.batch = 4;
  p.seqlen = 4096;
  p.num_heads = 32;
  p.num_gqa_groups = 8;
  p.head_dim_qk = 128;
  p.head_dim_v = 128;
  p.dtype = ATTN_BF16;
  p.mask_type = ATTN_MASK_CAUSAL;
  p.window_left = 1024;
  p.window_right = 0;
  p.scale_factor = 0.0f;
  p.softmax_type = ATTN_SOFTMAX_VANILLA;
  p.dropout_p = 0.0f;
  CHECK(attn_validate(&p) == ATTN_OK);
  CHECK(attn_fwd_workspace_size(&p) == 0);
  /* delta and LSE*log2(e) rows, B*Hq*S floats each, plus the sink partials */
  CHECK(attn_bwd_workspace_size(&p) >= 2u * 4u * 32u * 4096u * sizeof(float));

  int32_t bm = 0, bn = 0;
  CHECK(attn_fwd_tile_shape(&p, &bm, &bn) == ATTN_OK && bm > 0 && bn > 0);

  /* keys visible from rows 2000..2063 with window (1024, 0), causal */
  int32_t lo = -1, hi = -1;
  CHECK(attn_host_key_range(&p, 4096, 2000, 2063, &lo, &hi) == 1);
  CHECK(lo == 2000 - 1024 && hi == 2063);
  /* rows that see keys 4000..4095 */
  CHECK(attn_host_query_range(&p, 4096, 4000, 4095, &lo, &hi) == 1);
  CHECK(lo == 4000 && hi == 4095);
  CHECK(attn_host_dkdv_splits(&p) >= 1);

  struct attn_params bad = p;
  bad.head_dim_qk = 96;
  bad.head_dim_v = 96;
  CHECK(attn_validate(&bad) == ATTN_ERR_UNSUPPORTED);
  bad = p;
  bad.dropout_p = 1.0f;
  CHECK(attn_validate(&bad) == ATTN_ERR_INVALID_ARG);
  bad = p;
  bad.num_gqa_groups = 5;
  CHECK(attn_validate(&bad) == ATTN_ERR_INVALID_ARG);

  /* null pointers are rejected before any launch */
  CHECK(attn_fwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(attn_bwd_stage(9, &p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                       NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(strcmp(attn_status_string(ATTN_OK), "ok") == 0);
  printf("ok\n");
  return 0;
}
