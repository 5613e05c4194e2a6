// Redirect of routed logical expert ids to physical replicas.
//
// An expert with c replicas hands its tokens to them in turn: token row t
// goes to replica t mod c (the glossary of Part 2 of the EPLB README
// translation, «DualPipe и EPLB», ai.flicky.cc, says an expert with two copies
// gives each about half of its tokens; the round-robin by token row is the
// rule this library fixes).  out[l][t][k] = log2phy[l][e][t mod logcnt[l][e]].
//
// HBM-bound: 4 bytes read and 4 bytes written per id.  A few workgroups per
// layer sweep the layer together (all layers at once) with 16-byte
// non-temporal loads and stores.  The layer's tables are staged in LDS first: per expert its count
// and the magic numbers of an exact division by it (so t mod c costs a
// multiply-high, a shift and a multiply-subtract), and the log2phy rows.
#include "eplb_internal.h"

namespace eplb {

namespace {


template <bool kStaged>
__global__ __launch_bounds__(kStreamThreads) void redirect_kernel(const int32_t* __restrict__ idx,
                                                                   StreamSplit sp, FastDiv kdiv,
                                                                   int32_t E, int32_t X,
                                                                   const int32_t* __restrict__ log2phy,
                                                                   const int32_t* __restrict__ logcnt,
                                                                   int32_t* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t layer = blockIdx.x / sp.chunks;
  const int64_t chunk = blockIdx.x - layer * sp.chunks;
  const int tid = threadIdx.x;

  uint2* info = reinterpret_cast<uint2*>(smem);
  int32_t* stab = reinterpret_cast<int32_t*>(smem + (size_t)E * sizeof(uint2));
  const int32_t* gtab = log2phy + layer * (int64_t)E * X;
  stage_layer_tables<kStaged>(logcnt + layer * E, gtab, E, X, info, stab);
  __syncthreads();
  const LayerTables lt{info, kStaged ? stab : gtab, (uint32_t)E, X};

  const int64_t n = sp.per_layer;
  const int32_t* src = idx + layer * n;
  int32_t* dst = out + layer * n;
  const int64_t step = (int64_t)sp.chunks * kStreamThreads;

  const int mis_s = (int)(((uintptr_t)src >> 2) & 3);
  const int mis_d = (int)(((uintptr_t)dst >> 2) & 3);
  if (mis_s != mis_d) {
    // Source and destination disagree on 16-byte phase: plain 4-byte path.
    for (int64_t i = chunk * kStreamThreads + tid; i < n; i += step)
      dst[i] = map_id(src[i], fastdiv_apply((uint32_t)i, kdiv), lt);
    return;
  }
  int64_t head = (4 - mis_s) & 3;
  if (head > n) head = n;
  const int64_t n4 = (n - head) >> 2;
  const int64_t tail0 = head + (n4 << 2);
  if (chunk == 0) {
    if (tid < head) dst[tid] = map_id(src[tid], fastdiv_apply((uint32_t)tid, kdiv), lt);
    if (tail0 + tid < n)
      dst[tail0 + tid] = map_id(src[tail0 + tid], fastdiv_apply((uint32_t)(tail0 + tid), kdiv), lt);
  }
  const i32x4* s4 = reinterpret_cast<const i32x4*>(src + head);
  i32x4* d4 = reinterpret_cast<i32x4*>(dst + head);
  const uint32_t fb = (uint32_t)head;            // id offset (within the layer) of s4[0]
  for (int64_t v = chunk * kStreamThreads + tid; v < n4; v += step * kStreamUnroll) {
    // all loads of the iteration, then all lookups, then all stores
    i32x4 x[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t vv = v + u * step;
      if (vv < n4) x[u] = __builtin_nontemporal_load(s4 + vv);
    }
    i32x4 y[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      if (v + u * step < n4) {          // t below 2^31 only for ids that exist
        const uint32_t f = fb + (uint32_t)((v + u * step) << 2);
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

}  // namespace

hipError_t launch_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                           const int32_t* log2phy, const int32_t* logcnt, int32_t X,
                           int32_t* out, hipStream_t stream) {
  const int64_t per_layer = T * (int64_t)K;
  if (L == 0 || per_layer == 0) return hipSuccess;
  const StreamSplit sp = plan_stream(L, per_layer);
  const FastDiv kdiv = fastdiv_make((uint32_t)K);
  const int64_t blocks = L * sp.chunks;
  const size_t info_bytes = (size_t)E * sizeof(uint2);
  const size_t tab_bytes = (size_t)E * X * sizeof(int32_t);
  if (info_bytes + tab_bytes <= (size_t)kStageBytes) {
    redirect_kernel<true><<<(unsigned)blocks, kStreamThreads, info_bytes + tab_bytes, stream>>>(
        idx, sp, kdiv, E, X, log2phy, logcnt, out);
  } else {
    redirect_kernel<false><<<(unsigned)blocks, kStreamThreads, info_bytes, stream>>>(
        idx, sp, kdiv, E, X, log2phy, logcnt, out);
  }
  return hipGetLastError();
}

}  // namespace eplb
