// One pass over a step's routing ids that both counts them (the step's
// expert-load histogram, into the window ring) and redirects them with the
// placement in force, so each id is read from HBM once: 4 bytes read and 4
// written per id instead of 4 + 4 + 4 for the two passes.
//
// It is the histogram of eplb_load_hist (or eplb_load_ema) and the redirect of eplb_redirect
// (glossary of Part 2 of the EPLB README translation, «DualPipe и EPLB»,
// ai.flicky.cc: the load of an expert is the tokens routed to it; an expert
// with two copies gives each about half), done in the order a serving loop
// uses them: the ids of step s are served by the placement computed from the
// window before s, and counted into the window for the next placement.
#include "eplb_internal.h"

namespace eplb {

namespace {

__global__ __launch_bounds__(kMapThreads) void hist_redirect_kernel(
    const int32_t* __restrict__ idx, StreamSplit sp, FastDiv kdiv, bool k4, int32_t E, int32_t X, int32_t cap,
    int32_t copies, const int32_t* __restrict__ log2phy, const int32_t* __restrict__ logcnt, int32_t* __restrict__ out,
    int32_t* __restrict__ slot, int64_t* __restrict__ acc, int64_t* __restrict__ n_invalid) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t layer = blockIdx.x / sp.chunks;
  const int64_t chunk = blockIdx.x - layer * sp.chunks;
  const int tid = threadIdx.x;
  const int stride = E + 1;

  // LDS: counters [copies][E + 1], then the layer's staged map
  int32_t* counters = reinterpret_cast<int32_t*>(smem);
  const size_t cbytes = ((size_t)copies * stride * sizeof(int32_t) + 15) & ~(size_t)15;
  unsigned char* mbase = smem + cbytes;
  const LayerMapLds ml = layer_map_lds(E, cap);
  uint2* rec = reinterpret_cast<uint2*>(mbase);
  int32_t* rep = reinterpret_cast<int32_t*>(mbase + ml.o_rep);
  uint2* mlist = reinterpret_cast<uint2*>(mbase + ml.o_mlist);
  RepAlloc* alloc = reinterpret_cast<RepAlloc*>(mbase + ml.o_alloc);
  const int32_t* rows = log2phy + layer * (int64_t)E * X;
  for (int i = tid; i < copies * stride; i += kMapThreads) counters[i] = 0;
  const bool staged = stage_layer_map(logcnt + layer * E, rows, E, X, rec, rep, cap, alloc, mlist);
  int32_t* my = counters + (tid & (copies - 1)) * stride;

  const int64_t n = sp.per_layer;
  const int32_t* src = idx + layer * n;
  int32_t* dst = out + layer * n;
  const int64_t step = (int64_t)sp.chunks * kMapThreads;
  const uint32_t uE = (uint32_t)E;
  if (staged) {
    stream_map<kMapThreads, kMapUnroll>(src, dst, n, chunk, step, kdiv, k4, [&](int32_t e, uint32_t t) {
      count_id(e, uE, my);
      return map_id<true>(e, t, rec, rep, rows, uE, X);
    });
  } else {
    stream_map<kMapThreads, kMapUnroll>(src, dst, n, chunk, step, kdiv, k4, [&](int32_t e, uint32_t t) {
      count_id(e, uE, my);
      return map_id<false>(e, t, rec, rep, rows, uE, X);
    });
  }
  __syncthreads();
  flush_counts(counters, copies, E, slot + layer * E, acc + layer * E, n_invalid + layer);
}

// Count the step's ids into `slot` (cleared) and add them to `acc` and
// `n_invalid`, redirecting them on the way.  The counter copies get what the
// LDS budget leaves after the staged map (at least a map with every id of a
// placement from the rebalance: E * X entries up to kRepCap, fewer only for
// the largest E).
hipError_t launch_count_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, int32_t* slot,
                                 int64_t* acc, int64_t* n_invalid, const int32_t* log2phy, const int32_t* logcnt,
                                 int32_t X, int32_t* out, hipStream_t stream) {
  const int64_t per_layer = T * (int64_t)K;
  if (per_layer == 0) return hipSuccess;
  const StreamSplit sp = plan_stream(L, per_layer, kMapThreads, kMapUnroll, kMapBlocks);
  const FastDiv kdiv = fastdiv_make((uint32_t)K);
  auto cbytes = [&](int copies) { return ((size_t)copies * (E + 1) * 4 + 15) & ~(size_t)15; };
  const LayerMapLds ml = layer_map_plan(E, X, kMaxLdsBytes - cbytes(1));
  int copies = 16;
  while (copies > 1 && cbytes(copies) + ml.bytes > (size_t)kMaxLdsBytes) copies >>= 1;
  const size_t lds = cbytes(copies) + ml.bytes;
  const int64_t blocks = L * sp.chunks;
  hist_redirect_kernel<<<(unsigned)blocks, kMapThreads, lds, stream>>>(
      idx, sp, kdiv, K % 4 == 0, E, X, ml.cap, copies, log2phy, logcnt, out, slot, acc, n_invalid);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hist_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                                int32_t* ring, int32_t W, int64_t step, int64_t* load, int64_t* n_invalid,
                                const int32_t* log2phy, const int32_t* logcnt, int32_t X, int32_t* out,
                                hipStream_t stream) {
  if (L == 0) return hipSuccess;
  const int64_t LE = L * (int64_t)E;
  const int64_t cur = step % W;
  hipError_t err = launch_hist_prep(ring, LE, W, cur, load, n_invalid, L, stream);
  if (err != hipSuccess) return err;
  return launch_count_redirect(idx, L, T, K, E, ring + cur * LE, load, n_invalid, log2phy, logcnt, X, out,
                               stream);
}

hipError_t launch_ema_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, int32_t* count,
                               int32_t shift, int64_t* ema, int64_t* n_invalid, const int32_t* log2phy,
                               const int32_t* logcnt, int32_t X, int32_t* out, hipStream_t stream) {
  if (L == 0) return hipSuccess;
  hipError_t err = launch_ema_prep(count, L * (int64_t)E, shift, ema, n_invalid, L, stream);
  if (err != hipSuccess) return err;
  return launch_count_redirect(idx, L, T, K, E, count, ema, n_invalid, log2phy, logcnt, X, out, stream);
}

}  // namespace eplb
