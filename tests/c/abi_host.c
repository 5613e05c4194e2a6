/* Host-only use of the C ABI from plain C99: every declaration in eplb.h
 * compiles as C, every function links, and the host-only calls answer.
 * Touches no GPU. */
#include <stdio.h>
#include <string.h>

#include "eplb.h"

typedef void (*any_fn)(void);

int main(void) {
  /* take the address of every entry point: a missing symbol fails the link */
  const any_fn fns[] = {
      (any_fn)&eplb_load_hist,     (any_fn)&eplb_rebalance,
      (any_fn)&eplb_redirect,      (any_fn)&eplb_hist_redirect,
      (any_fn)&eplb_load_ema,      (any_fn)&eplb_ema_redirect,  (any_fn)&eplb_placement_load,
      (any_fn)&eplb_rearrange,     (any_fn)&eplb_lp_solve,
      (any_fn)&eplb_lp_redirect,   (any_fn)&eplb_lp_redirect_workspace_bytes,
      (any_fn)&eplb_status_string, (any_fn)&eplb_rebalance_lds_bytes,
      (any_fn)&eplb_rebalance_max_count, (any_fn)&eplb_lp_redirect_noalloc,
  };
  size_t i;
  for (i = 0; i < sizeof fns / sizeof fns[0]; ++i) {
    if (fns[i] == NULL) return 1;
  }
  if (strcmp(eplb_status_string(EPLB_OK), "ok") != 0) return 2;
  /* the DeepSeek-V3 prefill shape fits; a 4097-expert problem does not */
  if (eplb_rebalance_lds_bytes(256, 288, 8, 4, 32, 9) <= 0) return 3;
  if (eplb_rebalance_lds_bytes(256, 288, 8, 4, 32, 8) != -EPLB_E_CAPACITY) return 4;
  if (eplb_lp_redirect_workspace_bytes(58, 16384, 8, 256) != 58LL * 64 * 256 * 4) return 5;
  /* validation happens before any device work */
  if (eplb_rebalance(NULL, 1, 16, 24, 4, 2, 8, 5, NULL, NULL, NULL, NULL, NULL) != EPLB_E_ARG) return 6;
  /* 288 physical on 4 nodes: 9 copies at most; 8 groups on 5 nodes: global, 65 */
  if (eplb_rebalance_max_count(256, 288, 8, 4) != 9 || eplb_rebalance_max_count(256, 320, 8, 5) != 65) return 7;
  printf("abi_host ok: %zu entry points\n", sizeof fns / sizeof fns[0]);
  return 0;
}
