/* A C program against include/headcast.h and libheadcast.so, host-only
 * calls (no device work): the header compiles as C, every host entry point
 * links, and the results match what the Python binding reports.  Prints one
 * "key value" line per result. */
#include <stdio.h>
#include <string.h>

#include "headcast.h"

int main(void) {
  hc_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.num_heads = 12; cfg.head_dim = 128; cfg.grid_h = 45; cfg.grid_w = 80;
  cfg.block_frames = 3; cfg.window_frames = 21; cfg.cell_h = 10; cfg.cell_w = 10;
  cfg.dtype = HC_BF16; cfg.softmax_scale = 0.0f; cfg.kv_format = HC_KV_SAME;
  const int8_t labels[12] = {2, 0, 3, 1, 3, 2, 2, 3, 2, 2, 0, 1};

  printf("validate %d\n", (int)hc_validate_config(&cfg));
  size_t bytes = 0;
  printf("cache_bytes_status %d\n", (int)hc_cache_bytes(&cfg, labels, &bytes));
  printf("cache_bytes %zu\n", bytes);

  /* device memory is never touched by these calls: an aligned fake address */
  hc_cache* cache = NULL;
  void* fake = (void*)((uintptr_t)1 << 40);
  printf("create %d\n", (int)hc_cache_create(&cfg, labels, fake, bytes, &cache));
  hc_cache_layout lay;
  printf("layout_status %d\n", (int)hc_cache_get_layout(cache, &lay));
  printf("n_global %d\nn_spatial %d\nn_sink %d\nn_dummy %d\nglobal_splits %d\n", lay.n_global, lay.n_spatial,
         lay.n_sink, lay.n_dummy, lay.global_splits);
  printf("destroy %d\n", (int)hc_cache_destroy(cache));

  size_t ws = 0;
  printf("workspace_status %d\n", (int)hc_classify_workspace_bytes(&cfg, &ws));
  printf("workspace %zu\n", ws);
  hc_classify_params p;
  hc_default_classify_params(&p);
  printf("theta_score %.3f\ngamma %.1f\n", p.theta_score, p.gamma);

  cfg.head_dim = 96;   /* unsupported: rejected with a message */
  const hc_status bad = hc_validate_config(&cfg);
  printf("bad %d %s\n", (int)bad, hc_status_string(bad));
  printf("message_nonempty %d\n", hc_last_error_message()[0] != '\0');
  return 0;
}
