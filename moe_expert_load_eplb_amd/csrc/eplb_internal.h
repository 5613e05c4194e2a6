// Internal declarations shared by the EPLB HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
constexpr int kLpMaxRanks = 16;                  // ranks of one redistribution problem (2^RK rank sets)
constexpr int kLpMaxSlots = 64;                  // replica slots per rank
constexpr int kLpSeg = 2048;                     // ids per wave in the redirect by flows

// ---------------------------------------------------------------- helpers
// Magic numbers for floor(n / d) with 0 <= n < 2^31 and 1 <= d < 2^31
// (round-up method of Granlund and Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, Thm 4.2 with N = 31):
// l = ceil(log2 d), m = floor(2^(31+l) / d) + 1 < 2^32, and then
// floor(n / d) = umulhi(n, m) >> (l - 1) for d >= 2; d = 1 is the identity.
struct FastDiv {
  uint32_t mul;
  int32_t shift;           // l - 1, or -1 for d == 1
};

__host__ __device__ inline FastDiv fastdiv_make(uint32_t d) {
  FastDiv f;
  if (d <= 1) { f.mul = 0; f.shift = -1; return f; }
  int l = 0;
  while ((1u << l) < d) ++l;                        // l = ceil(log2 d), 1 <= l <= 31
  u64 m = ((u64)1 << (31 + l)) / d + 1;
  f.mul = (uint32_t)m;
  f.shift = l - 1;
  return f;
}

__host__ __device__ inline uint32_t fastdiv_apply(uint32_t n, FastDiv f) {
  if (f.shift < 0) return n;
  return (uint32_t)(((u64)n * f.mul) >> 32) >> f.shift;     // v_mul_hi_u32 on the device
}

// ---------------------------------------------------------------- streaming
// Work split of a [L][n] int32 stream: `chunks` workgroups per layer, which
// take the layer's 16-byte vectors in turn (workgroup c: c*NT + tid + k*chunks*NT).
// About kStreamBlocks workgroups of kStreamThreads threads over all layers keep
// ~7.6 MB of loads in flight, which is where measured HBM throughput peaks.
constexpr int kStreamThreads = 512;
constexpr int kStreamUnroll = 2;
constexpr int kStreamBlocks = 464;

struct StreamSplit {
  int64_t per_layer;       // ids per layer (T * K)
  int32_t chunks;          // workgroups per layer
};

StreamSplit plan_stream(int64_t L, int64_t per_layer);

// ---------------------------------------------------------------- redirect helpers
// A layer's redirect tables in LDS: per expert {magic, count << 8 | (shift + 1)}
// (count 0 marks an unusable expert: its ids map to -1) and the [E][X]
// log2phy rows (in LDS when staged, else read from global memory).
struct LayerTables {
  const uint2* info;       // per expert: {magic, count << 8 | (shift + 1)}, count 0 = invalid
  const int32_t* tab;      // [E][X] log2phy rows (LDS or global)
  uint32_t E;
  int32_t X;
};

__device__ __forceinline__ int32_t map_id(int32_t e, uint32_t t, const LayerTables& lt) {
  if ((uint32_t)e >= lt.E) return -1;
  const uint2 in = lt.info[e];
  const uint32_t c = in.y >> 8;
  if (c == 0) return -1;
  const int shift = (int)(in.y & 255u) - 1;
  const uint32_t q = shift < 0 ? t : (uint32_t)(((u64)t * in.x) >> 32) >> shift;
  const uint32_t r = t - q * c;
  return lt.tab[e * lt.X + (int32_t)r];
}


template <bool kStaged>
__device__ __forceinline__ void stage_layer_tables(const int32_t* __restrict__ cnt_row,
                                                   const int32_t* __restrict__ l2p_rows, int E, int X,
                                                   uint2* info, int32_t* stab) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int32_t c = cnt_row[e];
    uint2 in = make_uint2(0u, 0u);
    if (c >= 1 && c <= X) {
      const FastDiv f = fastdiv_make((uint32_t)c);
      in = make_uint2(f.mul, ((uint32_t)c << 8) | (uint32_t)(f.shift + 1));
    }
    info[e] = in;
  }
  if (kStaged) {
    for (int i = threadIdx.x; i < E * X; i += blockDim.x) stab[i] = l2p_rows[i];
  }
}

// Stage the tables in LDS when they fit in this many bytes.
constexpr int kStageBytes = 48 * 1024;

// One routing id into a workgroup's LDS counters, or into the invalid count.
__device__ __forceinline__ void count_id(int32_t e, uint32_t E, int32_t* my, uint32_t& inv) {
  if ((uint32_t)e < E) {
    atomicAdd(&my[e], 1);
  } else {
    ++inv;
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
