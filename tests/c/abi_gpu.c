/* The worked example of the EPLB pages ([EPLB-ru], «DualPipe и EPLB»,
 * section "Интерфейс и пример") through the C ABI from plain C: device
 * buffers from the HIP runtime, one eplb_rebalance call, the printed phy2log
 * of both layers compared on the host.  Needs a GPU. */
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "eplb.h"

#define CHECK(x)                                                        \
  do {                                                                  \
    if ((x) != hipSuccess) {                                            \
      fprintf(stderr, "HIP error at %s:%d\n", __FILE__, __LINE__);      \
      return 1;                                                         \
    }                                                                   \
  } while (0)

int main(void) {
  enum { B = 2, E = 12, P = 16, X = 3 };
  const int64_t load[B * E] = {90, 132, 40, 61, 104, 165, 39, 4, 73, 56, 183, 86,
                               20, 107, 104, 64, 19, 197, 187, 157, 172, 86, 16, 27};
  const int32_t want[B * P] = {5, 6, 5, 7, 8, 4, 3, 4, 10, 9, 10, 2, 0, 1, 11, 1,
                               7, 10, 6, 8, 6, 11, 8, 9, 2, 4, 5, 1, 5, 0, 3, 1};
  int64_t* d_load;
  int32_t *d_p2l, *d_l2p, *d_cnt, *d_status;
  int32_t p2l[B * P], status[B];
  int32_t rc;
  CHECK(hipMalloc((void**)&d_load, sizeof load));
  CHECK(hipMalloc((void**)&d_p2l, sizeof p2l));
  CHECK(hipMalloc((void**)&d_l2p, sizeof(int32_t) * B * E * X));
  CHECK(hipMalloc((void**)&d_cnt, sizeof(int32_t) * B * E));
  CHECK(hipMalloc((void**)&d_status, sizeof status));
  CHECK(hipMemcpy(d_load, load, sizeof load, hipMemcpyHostToDevice));
  rc = eplb_rebalance(d_load, B, E, P, 4, 2, 8, X, d_p2l, d_l2p, d_cnt, d_status, NULL);
  if (rc != EPLB_OK) {
    fprintf(stderr, "eplb_rebalance: %s\n", eplb_status_string(rc));
    return 2;
  }
  CHECK(hipMemcpy(p2l, d_p2l, sizeof p2l, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(status, d_status, sizeof status, hipMemcpyDeviceToHost));
  if (status[0] != EPLB_S_OK || status[1] != EPLB_S_OK) return 3;
  if (memcmp(p2l, want, sizeof want) != 0) {
    fprintf(stderr, "phy2log differs from the printed example\n");
    return 4;
  }
  CHECK(hipFree(d_load));
  CHECK(hipFree(d_p2l));
  CHECK(hipFree(d_l2p));
  CHECK(hipFree(d_cnt));
  CHECK(hipFree(d_status));
  printf("abi_gpu ok: worked example through the C ABI\n");
  return 0;
}
