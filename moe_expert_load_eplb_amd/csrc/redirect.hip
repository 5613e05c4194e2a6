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
// non-temporal loads and stores.  Each workgroup first stages its layer's
// placement in LDS as one record per expert and the list of replica ids of
// the experts with more than one replica: an id of a single-replica expert
// is served by one LDS read, any other by a multiply-high division of its
// token row and a second LDS read.
#include "eplb_internal.h"

namespace eplb {

namespace {

__global__ __launch_bounds__(kMapThreads) void redirect_kernel(const int32_t* __restrict__ idx,
                                                                   StreamSplit sp, FastDiv kdiv, bool k4,
                                                                   int32_t E, int32_t X, int32_t cap,
                                                                   const int32_t* __restrict__ log2phy,
                                                                   const int32_t* __restrict__ logcnt,
                                                                   int32_t* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t layer = blockIdx.x / sp.chunks;
  const int64_t chunk = blockIdx.x - layer * sp.chunks;

  const LayerMapLds ml = layer_map_lds(E, cap);
  uint2* rec = reinterpret_cast<uint2*>(smem);
  int32_t* rep = reinterpret_cast<int32_t*>(smem + ml.o_rep);
  uint2* mlist = reinterpret_cast<uint2*>(smem + ml.o_mlist);
  RepAlloc* alloc = reinterpret_cast<RepAlloc*>(smem + ml.o_alloc);
  const int32_t* rows = log2phy + layer * (int64_t)E * X;
  const bool staged = stage_layer_map(logcnt + layer * E, rows, E, X, rec, rep, cap, alloc, mlist);

  const int64_t n = sp.per_layer;
  const int32_t* src = idx + layer * n;
  int32_t* dst = out + layer * n;
  const int64_t step = (int64_t)sp.chunks * kMapThreads;
  const uint32_t uE = (uint32_t)E;
  if (staged) {
    stream_map<kMapThreads, kMapUnroll>(src, dst, n, chunk, step, kdiv, k4, [&](int32_t e, uint32_t t) {
      return map_id<true>(e, t, rec, rep, rows, uE, X);
    });
  } else {
    stream_map<kMapThreads, kMapUnroll>(src, dst, n, chunk, step, kdiv, k4, [&](int32_t e, uint32_t t) {
      return map_id<false>(e, t, rec, rep, rows, uE, X);
    });
  }
}

}  // namespace

hipError_t launch_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                           const int32_t* log2phy, const int32_t* logcnt, int32_t X,
                           int32_t* out, hipStream_t stream) {
  const int64_t per_layer = T * (int64_t)K;
  if (L == 0 || per_layer == 0) return hipSuccess;
  const StreamSplit sp = plan_stream(L, per_layer, kMapThreads, kMapUnroll, kMapBlocks);
  const FastDiv kdiv = fastdiv_make((uint32_t)K);
  const int64_t blocks = L * sp.chunks;
  const LayerMapLds ml = layer_map_plan(E, X, kMaxLdsBytes);
  redirect_kernel<<<(unsigned)blocks, kMapThreads, ml.bytes, stream>>>(idx, sp, kdiv, K % 4 == 0, E, X, ml.cap,
                                                                          log2phy, logcnt, out);
  return hipGetLastError();
}

}  // namespace eplb
