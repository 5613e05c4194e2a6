// Internal declarations shared by the EPLB HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace eplb {

typedef unsigned long long u64;
typedef unsigned __int128 u128;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));   // one 16-byte vector of ids

constexpr int64_t kLoadMax = int64_t(1) << 40;   // largest accepted load
constexpr int kMaxLdsBytes = 64 * 1024;          // per-workgroup LDS budget
constexpr int kMaxE = 4096;                      // per-expert LDS tables
constexpr int kMaxX = 65535;                     // log2phy width
constexpr int kMaxCount = 16128;                 // replica count bound (< 131^2)
constexpr int kMaxP = 8192;                      // physical experts per problem
constexpr int32_t kStatusBadMap = 18;            // rearrangement: an entry out of range
constexpr int32_t kStatusBadTopology = 19;       // redistribution: an id, home or count out of range
constexpr int kLpMaxRanks = 64;                  // ranks of one redistribution problem (one wave, a lane per rank)
constexpr int kLpEnumRanks = 16;                 // up to here the optimum may come from enumerating 2^RK rank sets
constexpr int kLpMaxSlots = 64;                  // replica slots per rank
constexpr int kLpSeg = 2048;                     // ids per wave in the redirect by flows
// Launch sizes: one launch covers at most 2^32 - 1 work-items.  The largest
// launches are 512 threads per layer (streaming, from 464 layers on) or per
// problem (rebalance), and 4096 threads per problem (redistribution solve).
constexpr int64_t kMaxLayers = int64_t(1) << 22;     // layers of one streaming call
constexpr int64_t kMaxProblems = int64_t(1) << 22;   // problems of one rebalance-like call
constexpr int64_t kLpMaxProblems = (int64_t(1) << 20) - 1;   // problems of one redistribution solve
constexpr int64_t kLpMaxSegments = int64_t(1) << 25; // layers x 2048-id segments of one redirect by flows

// ---------------------------------------------------------------- helpers
// Magic numbers for floor(n / d) with 0 <= n < 2^31 and 1 <= d < 2^31
// (round-up method of Granlund and Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, Thm 4.2 with N = 31):
// l = ceil(log2 d), m = floor(2^(31+l) / d) + 1 < 2^32, and then
// floor(n / d) = umulhi(n, m) >> (l - 1) for d >= 2.  d = 1 takes the same
// form without a branch: umulhi(n + 1, 2^32 - 1) = n for n + 1 < 2^32.
struct FastDiv {
  uint32_t mul;
  int32_t shift;           // l - 1 (0 for d == 1)
  uint32_t add;            // 1 for d == 1, else 0
};

__host__ __device__ inline FastDiv fastdiv_make(uint32_t d) {
  FastDiv f;
  if (d <= 1) { f.mul = 0xffffffffu; f.shift = 0; f.add = 1; return f; }
  int l = 0;
  while ((1u << l) < d) ++l;                        // l = ceil(log2 d), 1 <= l <= 31
  u64 m = ((u64)1 << (31 + l)) / d + 1;
  f.mul = (uint32_t)m;
  f.shift = l - 1;
  f.add = 0;
  return f;
}

__host__ __device__ inline uint32_t fastdiv_apply(uint32_t n, FastDiv f) {
  return (uint32_t)(((u64)(n + f.add) * f.mul) >> 32) >> f.shift;     // v_mul_hi_u32 on the device
}

// ---------------------------------------------------------------- streaming
// Work split of a [L][n] int32 stream: `chunks` workgroups per layer, which
// take the layer's 16-byte vectors in turn (workgroup c: c*NT + tid +
// k*chunks*NT), so the workgroups of a layer sweep it together and all layers
// run at once.  Launch shapes, from sweeps on MI355X of these kernels and of
// plain copy / read streams over the same layout:
//   counting (histogram, moving average): 464 workgroups of 512 threads, 2
//     vectors in flight each, within ~5% of the read-only stream's best;
//   redirect and fused pass: 232 workgroups of 512 threads, 4 vectors in
//     flight each (as many bytes in flight as 464 x 2 with half the
//     workgroups: ~6% less time with the per-id lookups), within ~4% of the
//     copy stream's best.
constexpr int kCountThreads = 512;
constexpr int kCountUnroll = 2;
constexpr int kCountBlocks = 464;
constexpr int kMapThreads = 512;
constexpr int kMapUnroll = 4;
constexpr int kMapBlocks = 232;

struct StreamSplit {
  int64_t per_layer;       // ids per layer (T * K)
  int32_t chunks;          // workgroups per layer
};

// floor(blocks / L) workgroups per layer (at least 1, at most one per
// threads * unroll vectors).
StreamSplit plan_stream(int64_t L, int64_t per_layer, int threads, int unroll, int blocks);

// ---------------------------------------------------------------- redirect tables
// A layer's placement as a workgroup stages it in LDS for the redirect:
//   rec[e]  one 8-byte record per logical expert, {a, b}, b = off << 16 | c:
//             c = 1: a is the physical id of the expert's one replica (the
//                    original), or -1 for an unusable expert (count outside
//                    [1, X]);
//             c >= 2: a is the magic number of floor(t / c) (Granlund and
//                    Montgomery, N = 31; the shift ceil(log2 c) - 1 is
//                    recomputed from c), off the position of the expert's
//                    replicas in `rep`;
//   rec[E]  a sentinel {-1, 1} that serves every id outside [0, E);
//   rep     the c physical ids of every expert with two or more replicas,
//           expert by expert (sum of those counts: P - E + their number for
//           a placement from the rebalance).
// Single-replica experts are served from their record alone.  When the
// counts of a layer sum to more than `rep` holds (only for counts that no
// placement of the rebalance produces), the workgroup reads the replica ids
// of multi-replica experts from the global rows instead.
constexpr int kRepCap = 8192;                    // replica ids staged per layer (the largest P)

struct RepAlloc {                                // 64-bit LDS counter: experts << 32 | ids
  unsigned long long v;
};

__device__ __forceinline__ uint32_t magic_of(uint32_t c) {   // c >= 2
  const int l = 32 - __builtin_clz(c - 1u);                  // ceil(log2 c)
  return (uint32_t)((((u64)1) << (31 + l)) / c + 1);
}

// Whole workgroup; ends with a barrier.  mlist: [min(E, cap / 2)] scratch
// {offset, expert} of the multi-replica experts, in allocation order (offsets
// ascending); more of them than that cannot fit in `rep` (two ids each).
// Returns whether `rep` holds every replica id (the same for all threads).
__device__ __forceinline__ bool stage_layer_map(const int32_t* __restrict__ cnt_row,
                                                const int32_t* __restrict__ rows, int E, int X, uint2* rec,
                                                int32_t* rep, int cap, RepAlloc* alloc, uint2* mlist) {
  const uint32_t mcap = (uint32_t)(E < cap / 2 ? E : cap / 2);
  const int tid = threadIdx.x, nt = blockDim.x;
  if (tid == 0) {
    alloc->v = 0;
    rec[E] = make_uint2(0xffffffffu, 1u);
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    const int32_t c = cnt_row[e];
    uint2 r = make_uint2(0xffffffffu, 1u);
    if (c == 1) {
      r.x = (uint32_t)rows[(int64_t)e * X];
    } else if (c >= 2 && c <= X) {
      const unsigned long long old = atomicAdd(&alloc->v, (1ull << 32) | (unsigned long long)c);
      const uint32_t k = (uint32_t)(old >> 32), off = (uint32_t)old;
      if (k < mcap) mlist[k] = make_uint2(off, (uint32_t)e);
      r = make_uint2(magic_of((uint32_t)c), ((off & 0xffffu) << 16) | (uint32_t)c);
    }
    rec[e] = r;
  }
  __syncthreads();
  const unsigned long long a = alloc->v;
  const int M = (int)(a >> 32);
  const uint32_t total = (uint32_t)a;
  const bool fits = total <= (uint32_t)cap;     // then M <= cap / 2 as well
  if (fits) {
    for (uint32_t i = tid; i < total; i += nt) {
      int lo = 0, hi = M - 1;                    // the last expert whose replicas start at or before i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mlist[mid].x <= i) lo = mid;
        else hi = mid - 1;
      }
      const uint2 m = mlist[lo];
      rep[i] = rows[(int64_t)m.y * X + (i - m.x)];
    }
  }
  __syncthreads();
  return fits;
}

// Physical replica of logical id e for token row t (t < 2^31): replica
// t mod c of e, -1 for an id outside [0, E) or an unusable expert.  kStaged:
// the multi-replica ids come from `rep` in LDS, else from the global rows.
template <bool kStaged>
__device__ __forceinline__ int32_t map_id(int32_t e, uint32_t t, const uint2* rec, const int32_t* rep,
                                          const int32_t* rows, uint32_t E, int X) {
  const uint32_t ue = (uint32_t)e < E ? (uint32_t)e : E;    // E: the sentinel
  const uint2 r = rec[ue];
  const uint32_t c = r.y & 0xffffu;
  const uint32_t sh = 31u - (uint32_t)__builtin_clz((c - 1u) | 1u);
  const uint32_t q = __umulhi(t, r.x) >> sh;
  const uint32_t rr = t - q * c;
  const bool multi = c > 1u;
  int32_t v;
  if constexpr (kStaged) {
    v = rep[multi ? (r.y >> 16) + rr : 0u];
  } else {
    v = (int32_t)r.x;
    if (multi) v = rows[(int64_t)ue * X + rr];
  }
  return multi ? v : (int32_t)r.x;
}

// LDS layout of a layer's staged map: records [E + 1] (16-byte padded),
// replica ids [cap] (16-byte padded), mlist [min(E, cap / 2)], the
// allocation counter.
struct LayerMapLds {
  int cap;
  size_t o_rep, o_mlist, o_alloc, bytes;
};
__host__ __device__ inline LayerMapLds layer_map_lds(int E, int cap) {
  LayerMapLds m;
  m.cap = cap;
  m.o_rep = ((size_t)(E + 1) * 8 + 15) & ~(size_t)15;
  m.o_mlist = m.o_rep + (((size_t)cap * 4 + 15) & ~(size_t)15);
  const size_t mcap = (size_t)(E < cap / 2 ? E : cap / 2);
  m.o_alloc = m.o_mlist + ((mcap * 8 + 15) & ~(size_t)15);
  m.bytes = m.o_alloc + 16;
  return m;
}
// The staged map of a layer with E experts and log2phy width X, in at most
// `budget` bytes: room for every id the counts can name (E * X), at most
// kRepCap, fewer when the budget is short (at least 2; a layer whose counts
// need more reads the global rows).
inline LayerMapLds layer_map_plan(int E, int X, size_t budget) {
  const int64_t want = (int64_t)E * X;
  int cap = (int)(want < kRepCap ? want : kRepCap);
  if (cap < 2) cap = 2;
  while (cap > 2 && layer_map_lds(E, cap).bytes > budget) cap = cap > 64 ? cap - 64 : 2;
  return layer_map_lds(E, cap);
}

// One layer of ids through op(id, token row) -> output id, the token row of
// position i being floor(i / K) (kdiv), this
// workgroup's share: workgroup `chunk` of the layer's workgroups takes the
// 16-byte vectors chunk*NT + tid + k*step (step = workgroups * NT).  Each
// full iteration loads U vectors, then maps all their ids, then stores
// them, with no branch in between (the leftover vectors of a thread, fewer
// than U, go one at a time).  When K is a multiple of 4
// and the layer starts on a 16-byte boundary (k4), the four ids of a vector
// share one token row.  Ids before the first 16-byte boundary and after the
// last are done by workgroup 0; a destination on another 16-byte phase than
// the source goes id by id.
// Raw (untyped) buffer descriptors for gfx950: word 3 of the resource, and
// the cache-policy bits of a streaming store (sc1 = device scope, nt).
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kStoreSc1Nt = 16 | 2;

template <int NT, int U, class Op>
__device__ __forceinline__ void stream_map(const int32_t* __restrict__ src, int32_t* __restrict__ dst, int64_t n,
                                           int64_t chunk, int64_t step, FastDiv kdiv, bool k4, Op op) {
  const int tid = threadIdx.x;
  const int mis_s = (int)(((uintptr_t)src >> 2) & 3);
  const int mis_d = (int)(((uintptr_t)dst >> 2) & 3);
  auto row = [&](int64_t i) { return fastdiv_apply((uint32_t)i, kdiv); };
  if (mis_s != mis_d) {
    for (int64_t i = chunk * NT + tid; i < n; i += step) dst[i] = op(src[i], row(i));
    return;
  }
  int64_t head = (4 - mis_s) & 3;
  if (head > n) head = n;
  const int64_t n4 = (n - head) >> 2;
  const int64_t tail0 = head + (n4 << 2);
  if (chunk == 0) {
    if (tid < head) dst[tid] = op(src[tid], row(tid));
    if (tail0 + tid < n) dst[tail0 + tid] = op(src[tail0 + tid], row(tail0 + tid));
  }
  const i32x4* s4 = reinterpret_cast<const i32x4*>(src + head);
  i32x4* d4 = reinterpret_cast<i32x4*>(dst + head);
  const uint32_t fb = (uint32_t)head;            // position (within the layer) of s4[0]
  auto sweep = [&](auto one_row, auto store) {
    auto map4 = [&](const i32x4& x, int64_t v) {   // positions below 2^31: the vector exists
      const uint32_t f = fb + (uint32_t)(v << 2);
      i32x4 y;
      if constexpr (decltype(one_row)::value) {
        const uint32_t t = fastdiv_apply(f, kdiv);
        y.x = op(x.x, t);
        y.y = op(x.y, t);
        y.z = op(x.z, t);
        y.w = op(x.w, t);
      } else {
        y.x = op(x.x, fastdiv_apply(f, kdiv));
        y.y = op(x.y, fastdiv_apply(f + 1, kdiv));
        y.z = op(x.z, fastdiv_apply(f + 2, kdiv));
        y.w = op(x.w, fastdiv_apply(f + 3, kdiv));
      }
      return y;
    };
    int64_t v = chunk * NT + tid;
    for (; v + (U - 1) * step < n4; v += U * step) {
      i32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(s4 + v + u * step);
      i32x4 y[U];
#pragma unroll
      for (int u = 0; u < U; ++u) y[u] = map4(x[u], v + u * step);
#pragma unroll
      for (int u = 0; u < U; ++u) store(y[u], v + u * step);
    }
    for (; v < n4; v += step) store(map4(__builtin_nontemporal_load(s4 + v), v), v);
  };
  auto run = [&](auto store) {
    if (k4 && head == 0) sweep(std::true_type{}, store);
    else sweep(std::false_type{}, store);
  };
  if (n4 < ((int64_t)1 << 27)) {
    // below 2 GiB of vectors: buffer stores with the device-scope and
    // non-temporal bits (sc1 nt), which stream to HBM a few per cent faster
    // than plain non-temporal stores; the descriptor spans the layer's vectors
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(d4, 0, (int)(n4 * 16), kRawBufferWord3);
    run([&](const i32x4& y, int64_t v) { __builtin_amdgcn_raw_buffer_store_b128(y, rd, (int)(v * 16), 0, kStoreSc1Nt); });
  } else {
    run([&](const i32x4& y, int64_t v) { __builtin_nontemporal_store(y, d4 + v); });
  }
}

// One routing id into a workgroup's LDS counters: column e, or column E (the
// row's padding) for an id outside [0, E).
__device__ __forceinline__ void count_id(int32_t e, uint32_t E, int32_t* my) {
  atomicAdd(&my[(uint32_t)e < E ? (uint32_t)e : E], 1);
}

// A workgroup's counts ([copies][E + 1] in LDS, after a barrier) into the
// layer's step counts, its load and its invalid-id count: one global atomic
// per expert with a nonzero total.
__device__ __forceinline__ void flush_counts(const int32_t* counters, int copies, int E, int32_t* cnt_row,
                                             int64_t* acc_row, int64_t* n_invalid_l) {
  const int stride = E + 1;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    int32_t s = 0;
    for (int c = 0; c < copies; ++c) s += counters[c * stride + e];
    if (s == 0) continue;
    if (e < E) {
      atomicAdd(&cnt_row[e], s);
      atomicAdd(reinterpret_cast<unsigned long long*>(&acc_row[e]), (unsigned long long)s);
    } else {
      atomicAdd(reinterpret_cast<unsigned long long*>(n_invalid_l), (unsigned long long)s);
    }
  }
}

// ---------------------------------------------------------------- rebalance
// Everything the rebalance kernel needs about one problem shape, derived on
// the host: the effective policy, the per-node sizes, and the byte offsets of
// every LDS array.
struct RbPlan {
  int32_t E, P, Gp, Np, RK, X;
  int32_t S, En, Pn, Rn, RKn, ppr, gpn;
  int32_t KR, KP, KN;      // registers per lane for the sorted experts / GPU packs / node packs
  int32_t threads;         // workgroup size
  // LDS byte offsets
  int32_t o_kexp, o_w, o_wl, o_gsum, o_m2l, o_cnt, o_srt;
  int32_t o_gnode, o_gslot, o_gord, o_gres, o_rep, o_pk, o_posaux, o_ordr, o_ores, o_rcls;
  int32_t o_nflag, o_flags;
  int32_t pk_words;        // per-wave packing scratch, in 8-byte words
  int32_t lds_bytes;
  FastDiv fd_S, fd_En, fd_X;
};

// Returns 0 and fills `plan`, or an EPLB_E_* code.
int32_t rb_make_plan(int32_t E, int32_t P, int32_t G, int32_t N, int32_t RK, int32_t X, RbPlan* plan);

// Kernel launchers (return hipSuccess or the launch error).
hipError_t launch_hist(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                       int32_t* ring, int32_t W, int64_t step, int64_t* load,
                       int64_t* n_invalid, hipStream_t stream);
hipError_t launch_ema_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, int32_t* count,
                               int32_t shift, int64_t* ema, int64_t* n_invalid, const int32_t* log2phy,
                               const int32_t* logcnt, int32_t X, int32_t* out, hipStream_t stream);
hipError_t launch_load_ema(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                           int32_t* cnt, int32_t shift, int64_t* ema, int64_t* n_invalid,
                           hipStream_t stream);
hipError_t launch_placement_load(const int64_t* load, const int32_t* phy2log, const int32_t* logcnt,
                                 int64_t B, int32_t E, int32_t P, int32_t RK, double* rank_load,
                                 double* imbalance, hipStream_t stream);
hipError_t launch_rearrange(const int32_t* old_p2l, const int32_t* new_p2l, const int32_t* new_l2p, int64_t B,
                            int32_t E, int32_t P, int32_t RK, int32_t N, int32_t X, int32_t* plan,
                            int32_t* l2p_out, int32_t* src, int32_t* moves, int32_t* status,
                            hipStream_t stream);
int64_t rearrange_lds_bytes(int32_t E, int32_t P, int32_t N);
int64_t lp_segments(int64_t n);
// The argument rules of the redirect by flows, all but the workspace's:
// EPLB_OK or an EPLB_E_* code.
int32_t check_lp_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, const int32_t* rep,
                          const int64_t* flow, int32_t RK, int32_t R, const int32_t* out);
// Segment counts the redirect by flows keeps: one int32 per layer, 2048-id
// segment and replicated expert (at most min(E, RK * R) of them).
inline int64_t lp_redirect_counts(int64_t L, int64_t n, int32_t E, int32_t RK, int32_t R) {
  const int64_t c = (int64_t)RK * R < E ? (int64_t)RK * R : E;
  return L * lp_segments(n) * c;
}
hipError_t launch_lp_redirect(const int32_t* idx, int64_t L, int64_t n, int32_t E, const int32_t* rep,
                              const int64_t* flow, int32_t RK, int32_t R, int32_t* seg, int32_t* out,
                              hipStream_t stream);
hipError_t launch_lp_solve(const int64_t* cnt, const int32_t* home, const int32_t* rep, int64_t B, int32_t E,
                           int32_t RK, int32_t R, int64_t* lam, int64_t* flow, int64_t* rank_load,
                           int32_t* status, hipStream_t stream);
// load = sum of the window's slots other than cur, slot cur = 0, n_invalid = 0
hipError_t launch_hist_prep(int32_t* ring, int64_t LE, int32_t W, int64_t cur, int64_t* load, int64_t* n_invalid,
                            int64_t L, hipStream_t stream);
// ema = ema - floor(ema / 2^shift), cnt = 0, n_invalid = 0
hipError_t launch_ema_prep(int32_t* cnt, int64_t LE, int32_t shift, int64_t* ema, int64_t* n_invalid, int64_t L,
                           hipStream_t stream);
hipError_t launch_hist_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                                int32_t* ring, int32_t W, int64_t step, int64_t* load, int64_t* n_invalid,
                                const int32_t* log2phy, const int32_t* logcnt, int32_t X, int32_t* out,
                                hipStream_t stream);
hipError_t launch_rebalance(const int64_t* load, int64_t B, const RbPlan& plan,
                            int32_t* phy2log, int32_t* log2phy, int32_t* logcnt,
                            int32_t* status, hipStream_t stream);
hipError_t launch_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                           const int32_t* log2phy, const int32_t* logcnt, int32_t X,
                           int32_t* out, hipStream_t stream);

}  // namespace eplb
