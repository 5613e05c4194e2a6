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

template <bool kStaged>
__global__ __launch_bounds__(kStreamThreads) void hist_redirect_kernel(
    const int32_t* __restrict__ idx, StreamSplit sp, FastDiv kdiv, int32_t E, int32_t X, int32_t copies,
    const int32_t* __restrict__ log2phy, const int32_t* __restrict__ logcnt, int32_t* __restrict__ out,
    int32_t* __restrict__ slot, int64_t* __restrict__ acc, int64_t* __restrict__ n_invalid) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t layer = blockIdx.x / sp.chunks;
  const int64_t chunk = blockIdx.x - layer * sp.chunks;
  const int tid = threadIdx.x;
  const int stride = E + 1;

  // LDS: counters [copies][E + 1], then the per-expert records, then the rows
  int32_t* counters = reinterpret_cast<int32_t*>(smem);
  const size_t cbytes = ((size_t)copies * stride * sizeof(int32_t) + 15) & ~(size_t)15;
  uint2* info = reinterpret_cast<uint2*>(smem + cbytes);
  int32_t* stab = reinterpret_cast<int32_t*>(smem + cbytes + (size_t)E * sizeof(uint2));
  const int32_t* gtab = log2phy + layer * (int64_t)E * X;
  for (int i = tid; i < copies * stride; i += kStreamThreads) counters[i] = 0;
  stage_layer_tables<kStaged>(logcnt + layer * E, gtab, E, X, info, stab);
  __syncthreads();
  const LayerTables lt{info, kStaged ? stab : gtab, (uint32_t)E, X};
  int32_t* my = counters + (tid & (copies - 1)) * stride;
  uint32_t inv = 0;

  const int64_t n = sp.per_layer;
  const int32_t* src = idx + layer * n;
  int32_t* dst = out + layer * n;
  const int64_t step = (int64_t)sp.chunks * kStreamThreads;
  const int mis_s = (int)(((uintptr_t)src >> 2) & 3);
  const int mis_d = (int)(((uintptr_t)dst >> 2) & 3);
  if (mis_s != mis_d) {
    for (int64_t i = chunk * kStreamThreads + tid; i < n; i += step) {
      const int32_t e = src[i];
      count_id(e, (uint32_t)E, my, inv);
      dst[i] = map_id(e, fastdiv_apply((uint32_t)i, kdiv), lt);
    }
  } else {
    int64_t head = (4 - mis_s) & 3;
    if (head > n) head = n;
    const int64_t n4 = (n - head) >> 2;
    const int64_t tail0 = head + (n4 << 2);
    if (chunk == 0) {
      if (tid < head) {
        const int32_t e = src[tid];
        count_id(e, (uint32_t)E, my, inv);
        dst[tid] = map_id(e, fastdiv_apply((uint32_t)tid, kdiv), lt);
      }
      if (tail0 + tid < n) {
        const int32_t e = src[tail0 + tid];
        count_id(e, (uint32_t)E, my, inv);
        dst[tail0 + tid] = map_id(e, fastdiv_apply((uint32_t)(tail0 + tid), kdiv), lt);
      }
    }
    const i32x4* s4 = reinterpret_cast<const i32x4*>(src + head);
    i32x4* d4 = reinterpret_cast<i32x4*>(dst + head);
    const uint32_t fb = (uint32_t)head;
    for (int64_t v = chunk * kStreamThreads + tid; v < n4; v += step * kStreamUnroll) {
      i32x4 x[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const int64_t vv = v + u * step;
        if (vv < n4) x[u] = __builtin_nontemporal_load(s4 + vv);
      }
      i32x4 y[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        if (v + u * step < n4) {
          const uint32_t f = fb + (uint32_t)((v + u * step) << 2);
          count_id(x[u].x, (uint32_t)E, my, inv);
          count_id(x[u].y, (uint32_t)E, my, inv);
          count_id(x[u].z, (uint32_t)E, my, inv);
          count_id(x[u].w, (uint32_t)E, my, inv);
          y[u].x = map_id(x[u].x, fastdiv_apply(f, kdiv), lt);
          y[u].y = map_id(x[u].y, fastdiv_apply(f + 1, kdiv), lt);
          y[u].z = map_id(x[u].z, fastdiv_apply(f + 2, kdiv), lt);
          y[u].w = map_id(x[u].w, fastdiv_apply(f + 3, kdiv), lt);
        }
      }
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const int64_t vv = v + u * step;
        if (vv < n4) __builtin_nontemporal_store(y[u], d4 + vv);
      }
    }
  }
  __syncthreads();
  int32_t* cnt_out = slot + layer * E;
  unsigned long long* acc_l = reinterpret_cast<unsigned long long*>(acc + layer * E);
  for (int e = tid; e < E; e += kStreamThreads) {
    int32_t s = 0;
    for (int c = 0; c < copies; ++c) s += counters[c * stride + e];
    if (s) {
      atomicAdd(&cnt_out[e], s);
      atomicAdd(&acc_l[e], (unsigned long long)s);
    }
  }
  for (int off = 32; off > 0; off >>= 1) inv += __shfl_xor(inv, off);
  if ((tid & 63) == 0 && inv)
    atomicAdd(reinterpret_cast<unsigned long long*>(&n_invalid[layer]), (unsigned long long)inv);
}

}  // namespace

namespace {

// Clear `slot` and n_invalid, then count and redirect every id in one pass.
// Count the step's ids into `slot` (cleared) and add them to `acc` and
// `n_invalid`, redirecting them on the way.
hipError_t launch_count_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, int32_t* slot,
                                 int64_t* acc, int64_t* n_invalid, const int32_t* log2phy, const int32_t* logcnt,
                                 int32_t X, int32_t* out, hipStream_t stream) {
  hipError_t err = hipSuccess;
  const int64_t per_layer = T * (int64_t)K;
  if (per_layer > 0) {
    const StreamSplit sp = plan_stream(L, per_layer);
    const FastDiv kdiv = fastdiv_make((uint32_t)K);
    const size_t info_bytes = (size_t)E * sizeof(uint2);
    const size_t tab_bytes = (size_t)E * X * sizeof(int32_t);
    const bool staged = info_bytes + tab_bytes <= (size_t)kStageBytes;
    const size_t table_bytes = info_bytes + (staged ? tab_bytes : 0);
    int copies = 16;
    while (copies > 1 && (((size_t)copies * (E + 1) * 4 + 15) & ~(size_t)15) + table_bytes > (size_t)kMaxLdsBytes)
      copies >>= 1;
    const size_t lds = (((size_t)copies * (E + 1) * 4 + 15) & ~(size_t)15) + table_bytes;
    const int64_t blocks = L * sp.chunks;
    if (staged)
      hist_redirect_kernel<true><<<(unsigned)blocks, kStreamThreads, lds, stream>>>(
          idx, sp, kdiv, E, X, copies, log2phy, logcnt, out, slot, acc, n_invalid);
    else
      hist_redirect_kernel<false><<<(unsigned)blocks, kStreamThreads, lds, stream>>>(
          idx, sp, kdiv, E, X, copies, log2phy, logcnt, out, slot, acc, n_invalid);
    err = hipGetLastError();
  }
  return err;
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
