// Placement quality on the device: the load every rank (GPU) carries under a
// placement, and the ratio of the largest to the mean.
//
// A replica takes an equal share of its expert's tokens (glossary of Part 2
// of the EPLB README translation, «DualPipe и EPLB», ai.flicky.cc), so a rank
// carries the sum of load[e] / logcnt[e] over the physical experts it holds;
// the translator's hands-on exercise 2 and the check of the worked example
// under "Интерфейс и пример" compare policies by max / mean of these loads.
//
// One wave per problem.  Lane r sums ranks r, r + 64, ... over their P / RK
// slots in slot order (double precision, one rounding per division and per
// addition); the mean is the exact int64 total (< 2^53, so exact as a double)
// divided by RK.  The work is a few gathers per slot from rows that sit in L2:
// latency-bound, a few microseconds per launch.
#include "eplb_internal.h"

namespace eplb {

namespace {

__global__ __launch_bounds__(64) void placement_load_kernel(const int64_t* __restrict__ load,
                                                            const int32_t* __restrict__ phy2log,
                                                            const int32_t* __restrict__ logcnt, int32_t E,
                                                            int32_t P, int32_t RK,
                                                            double* __restrict__ rank_load,
                                                            double* __restrict__ imbalance) {
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t* w = load + b * E;
  const int32_t* phy = phy2log + b * P;
  const int32_t* cnt = logcnt + b * E;
  double* out = rank_load + b * RK;
  const int ppr = P / RK;

  int bad = 0;
  int64_t total = 0;
  for (int e = lane; e < E; e += 64) {
    const int64_t x = w[e];
    bad |= (x < 0) | (x > kLoadMax);
    total += x;
  }
  double mx = 0.0;
  for (int r = lane; r < RK; r += 64) {
    double s = 0.0;
    for (int j = 0; j < ppr; ++j) {
      const int32_t e = phy[r * ppr + j];
      if ((uint32_t)e >= (uint32_t)E) { bad = 1; continue; }
      const int32_t c = cnt[e];
      if (c < 1) { bad = 1; continue; }
      s += (double)w[e] / (double)c;
    }
    out[r] = s;
    mx = fmax(mx, s);
  }
  const bool any_bad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
  for (int off = 32; off > 0; off >>= 1) {
    total += __shfl_xor(total, off);
    mx = fmax(mx, __shfl_xor(mx, off));
  }
  if (any_bad) {
    const double nan = __builtin_nan("");
    for (int r = lane; r < RK; r += 64) out[r] = nan;
    if (lane == 0) imbalance[b] = nan;
    return;
  }
  if (lane == 0) imbalance[b] = total == 0 ? 1.0 : mx / ((double)total / (double)RK);
}

}  // namespace

hipError_t launch_placement_load(const int64_t* load, const int32_t* phy2log, const int32_t* logcnt,
                                 int64_t B, int32_t E, int32_t P, int32_t RK, double* rank_load,
                                 double* imbalance, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  placement_load_kernel<<<(unsigned)B, 64, 0, stream>>>(load, phy2log, logcnt, E, P, RK, rank_load, imbalance);
  return hipGetLastError();
}

}  // namespace eplb
