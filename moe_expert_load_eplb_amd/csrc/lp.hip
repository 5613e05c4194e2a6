// Per-batch redistribution of tokens over a fixed replica topology
// (LPLB-style), solved exactly in integers.
//
// Two pages describe LPLB: «DeepSeek开源LPLB：基于线性规划的MoE负载均衡器…»
// (2048ai.net; items 4, 5 and 7: the replica topology, the LP model, the
// typical topologies) and the Machine Heart report on LPLB (wwwcj777.com,
// section «LPLB 的工作原理»).  A redundant expert links the GPU of its
// original to its own GPU; that edge carries at most the tokens routed to
// the expert in the batch; tokens move along the edges so that the loads of
// the expert-parallel group are as even as possible.  Here: the least
// largest rank load reachable with whole tokens, and one flow reaching it.
//
// One workgroup per problem (layer; with 12 or more ranks, step 2 runs over
// four workgroups per layer in a first launch):
//   1. home loads base[r] and the capacity cap[o][g] of every rank pair,
//      with LDS atomics; a bitmap catches an expert replicated twice;
//   2. the optimum, from the supply-demand theorem (Gale, 1957): a bound lam
//      is reachable iff for every set S of ranks, load(S) - cap(S -> rest)
//      <= lam * |S|, so lam* = max over S of ceil((load(S) - cap(S -> rest))
//      / |S|); the 2^RK - 1 sets are enumerated in Gray-code order (one rank
//      in or out per step; the cut changes by that rank's edges to and from
//      the set, summed from per-rank tables over 4-rank quarters of the
//      set), spread over the threads;
//   3. one wave computes a maximum flow of the feasibility network at lam*
//      (source -> rank: what it must shed; rank -> sink: what it may take)
//      by shortest augmenting paths (Edmonds and Karp, J. ACM 1972), the
//      search level by level with one lane per node; a node's predecessor is
//      the lowest-numbered node of the previous level with residual capacity,
//      which fixes one definite flow among the optimal ones;
//   4. the net flow of each rank pair is split over the pair's replica slots
//      in ascending slot order.
// Integer work throughout.  Steps 1-4 as written serve up to 16 ranks (the
// pages' 8-GPU cube and 16-GPU hypercube), where every structure fits in
// LDS; 17 to 64 ranks (a torus over several nodes) take the cut iteration
// of lp_solve_dk_kernel below, which reaches the same optimum and flow
// without enumerating rank sets.
#include <climits>

#include "eplb_internal.h"

namespace eplb {

namespace {

constexpr int kLpThreads = 1024;
constexpr int kLpMaxV = kLpEnumRanks + 2;
constexpr int kLpMaxAugment = 1 << 16;     // far above the Edmonds-Karp bound V * E for V <= 18
constexpr int kLpSplitRanks = 12;          // from 2^12 rank sets on, step 2 is spread over kLpParts workgroups
constexpr int kLpParts = 4;                // (<= kLpSplitRanks: the bounds sit in a layer's rank_load row)

__device__ __forceinline__ void lp_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// kMode 0: the whole solve in one workgroup per layer.  With many ranks the
// enumeration of step 2 is split: kMode 1 runs `parts` workgroups per layer,
// each over its share of the rank sets, and leaves its bound in
// load_out[b][part] (a scratch use of the output, rewritten at the end);
// kMode 2 then takes the largest of those and does steps 3 and 4.
template <int kMode>
__global__ __launch_bounds__(kLpThreads) void lp_solve_kernel(
    const int64_t* __restrict__ cnt, const int32_t* __restrict__ home, const int32_t* __restrict__ rep,
    int32_t E, int32_t RK, int32_t R, int32_t parts, int64_t* __restrict__ lam_out, int64_t* __restrict__ flow_out,
    int64_t* __restrict__ load_out, int32_t* __restrict__ status) {
  __shared__ unsigned long long base[kLpEnumRanks];
  __shared__ unsigned long long cap[kLpEnumRanks * kLpEnumRanks];      // cap[o * RK + g]
  __shared__ long long res[kLpMaxV * kLpMaxV];                        // residual, res[u * V + v]
  __shared__ uint32_t seen_bits[kMaxE / 32];
  __shared__ long long s_best[kLpThreads / 64];
  __shared__ long long psym[kLpEnumRanks * 4 * 16];                   // [r][quarter][4-bit subset]
  __shared__ long long wbase[kLpEnumRanks];                            // base[r] - cap(r -> every other rank)

  const int64_t b = kMode == 1 ? blockIdx.x / parts : blockIdx.x;
  const int part = kMode == 1 ? (int)(blockIdx.x - b * parts) : 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t* c = cnt + b * E;
  const int32_t* h = home + b * E;
  const int32_t* rp = rep + b * (int64_t)RK * R;
  const int V = RK + 2, src = RK, snk = RK + 1;

  for (int i = tid; i < RK; i += kLpThreads) base[i] = 0;
  for (int i = tid; i < RK * RK; i += kLpThreads) cap[i] = 0;
  for (int i = tid; i < (E + 31) / 32; i += kLpThreads) seen_bits[i] = 0;
  __syncthreads();

  // ---- 1. home loads, rank-pair capacities
  int bad = 0;
  for (int e = tid; e < E; e += kLpThreads) {
    const int64_t x = c[e];
    const int32_t r = h[e];
    const bool ok = x >= 0 && x <= kLoadMax && (uint32_t)r < (uint32_t)RK;
    bad |= !ok;
    if (ok) atomicAdd(&base[r], (unsigned long long)x);
  }
  for (int i = tid; i < RK * R; i += kLpThreads) {
    const int32_t x = rp[i];
    if (x == -1) continue;
    if ((uint32_t)x >= (uint32_t)E) { bad = 1; continue; }
    const uint32_t bit = 1u << (x & 31);
    if (atomicOr(&seen_bits[x >> 5], bit) & bit) { bad = 1; continue; }   // replicated twice
    const int32_t o = h[x], g = i / R;
    const int64_t v = c[x];
    if ((uint32_t)o < (uint32_t)RK && o != g && v >= 0 && v <= kLoadMax)
      atomicAdd(&cap[o * RK + g], (unsigned long long)v);
  }
  bad = __syncthreads_or(bad);
  int64_t* flow_b = flow_out + b * (int64_t)RK * R;
  int64_t* load_b = load_out + b * RK;
  if (kMode == 1 && bad) return;                       // the second pass reports it
  if (bad) {
    for (int i = tid; i < RK * R; i += kLpThreads) flow_b[i] = -1;
    for (int i = tid; i < RK; i += kLpThreads) load_b[i] = -1;
    if (tid == 0) {
      lam_out[b] = -1;
      status[b] = kStatusBadTopology;
    }
    return;
  }

  // ---- 2. lam* = max over rank sets S of ceil((load(S) - cap(S -> rest)) / |S|)
  // When rank r enters or leaves, giving the set T, the cut cap(T -> rest)
  // changes by cap(r -> outside T) - cap(T -> r)
  //          = cap(r -> all) - sum over g in T of (cap[r][g] + cap[g][r]),
  // and that sum is read from psym[r][q][T's bits q*4 .. q*4+3] for the
  // four quarters q of the ranks (one LDS round trip per step).
  for (int i = tid; i < kLpEnumRanks * 4 * 16; i += kLpThreads) {
    const int r = i >> 6, q = (i >> 4) & 3, m = i & 15;
    long long v = 0;
    if (r < RK)
      for (int t = 0; t < 4; ++t) {
        const int g = q * 4 + t;
        if (((m >> t) & 1) && g < RK && g != r) v += (long long)(cap[r * RK + g] + cap[g * RK + r]);
      }
    psym[i] = v;
  }
  if (tid < RK) {
    long long o = 0;
    for (int g = 0; g < RK; ++g) o += (long long)cap[tid * RK + g];
    wbase[tid] = (long long)base[tid] - o;
  }
  __syncthreads();
  // f(S) = load(S) - cap(S -> rest) changes, when rank r joins or leaves and
  // the set becomes T, by +-(base[r] - cap(r -> outside T) + cap(T -> r))
  //   = +-(wbase[r] + sum over g in T of (cap[r][g] + cap[g][r]))
  auto step_change = [&](int r, uint32_t T) {
    const long long* pr = psym + r * 64;
    return wbase[r] + pr[T & 15] + pr[16 + ((T >> 4) & 15)] + pr[32 + ((T >> 8) & 15)] + pr[48 + ((T >> 12) & 15)];
  };
  const uint32_t nsets = 1u << RK;                     // Gray index i in [1, nsets) gives S = i ^ (i >> 1)
  uint32_t lo = 1, hi = nsets;                         // this workgroup's Gray indices
  if (kMode == 1) {
    const uint32_t span = (nsets - 1 + parts - 1) / parts;
    lo = min(nsets, 1 + (uint32_t)part * span);
    hi = min(nsets, lo + span);
  }
  const uint32_t per = kMode == 2 ? 0 : (hi - lo + kLpThreads - 1) / kLpThreads;
  const uint32_t i0 = lo + (uint32_t)tid * per;
  const uint32_t i1 = min(hi, i0 + per);
  // best = the largest ceil(f(S) / |S|) so far (at least 0): a set beats it
  // exactly when f(S) > best * |S| (f <= 2^56, |S| <= 16), and only then is
  // the division made
  long long best = 0;
  if (i0 < i1) {
    uint32_t S = i0 ^ (i0 >> 1);
    long long f = 0;
    uint32_t T = 0;
    for (uint32_t m = S; m; m &= m - 1) {              // the first set, one rank at a time
      const int r = __builtin_ctz(m);
      T |= 1u << r;
      f += step_change(r, T);
    }
    auto consider = [&](uint32_t set) {
      const int k = __popc(set);
      if (f > best * k) best = (f + k - 1) / k;
    };
    consider(S);
    uint32_t i = i0 + 1;
    for (; i + 4 <= i1; i += 4) {                      // four steps' table reads in flight
      int r[4];
      uint32_t T4[4];
      long long d[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r[k] = __builtin_ctz(i + k);                   // the rank that enters or leaves
        T4[k] = (k == 0 ? S : T4[k - 1]) ^ (1u << r[k]);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) d[k] = step_change(r[k], T4[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f += ((T4[k] >> r[k]) & 1u) ? d[k] : -d[k];
        consider(T4[k]);
      }
      S = T4[3];
    }
    for (; i < i1; ++i) {
      const int r = __builtin_ctz(i);
      S ^= 1u << r;
      const long long d = step_change(r, S);
      f += ((S >> r) & 1u) ? d : -d;
      consider(S);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const long long o = __shfl_xor(best, off);
    best = o > best ? o : best;
  }
  if (lane == 0) s_best[wave] = best;
  // residual network at lam* (filled after the reduction)
  __syncthreads();
  long long lam = 0;
  for (int w = 0; w < kLpThreads / 64; ++w) lam = s_best[w] > lam ? s_best[w] : lam;
  if constexpr (kMode == 1) {
    if (tid == 0) load_b[part] = lam;
    return;
  }
  if constexpr (kMode == 2)
    for (int q = 0; q < parts; ++q) lam = load_b[q] > lam ? load_b[q] : lam;
  for (int i = tid; i < V * V; i += kLpThreads) {
    const int u = i / V, v = i - u * V;
    long long x = 0;
    if (u == src && v < RK) x = (long long)base[v] - lam > 0 ? (long long)base[v] - lam : 0;
    else if (v == snk && u < RK) x = lam - (long long)base[u] > 0 ? lam - (long long)base[u] : 0;
    else if (u < RK && v < RK && u != v) x = (long long)cap[u * RK + v];
    res[i] = x;
  }
  __syncthreads();

  // ---- 3. maximum flow at lam* (wave 0; one lane per node).  Lane v keeps
  // `in` = the set of nodes u with residual capacity u -> v, so one level of
  // the search is a bit scan and a ballot.  The path is then walked back
  // from the sink (its bottleneck from the tree edges' residuals), and `in`
  // changes only where the path did: a path edge that runs dry leaves its
  // head's set, each reverse edge joins its tail's set.
  int exhausted = 0;
  if (wave == 0) {
    const bool node = lane < V;
    uint64_t in = 0;
    if (node) {
#pragma unroll
      for (int u = 0; u < kLpMaxV; ++u)
        if (u < V) in |= (uint64_t)(res[u * V + lane] > 0) << u;
    }
    for (int it = 0; it < kLpMaxAugment; ++it) {
      uint64_t seen = 1ull << src, frontier = 1ull << src;
      int parent = -1;
      while (frontier && !((seen >> snk) & 1ull)) {
        const uint64_t cand = node && !((seen >> lane) & 1ull) ? (in & frontier) : 0;
        if (cand) parent = __builtin_ctzll(cand);
        const uint64_t found = __builtin_amdgcn_ballot_w64(cand != 0);
        seen |= found;
        frontier = found;
      }
      if (!((seen >> snk) & 1ull)) break;
      const bool reached = node && lane != src && ((seen >> lane) & 1ull);
      long long fwd = 0, bwd = 0;                      // residuals of parent -> lane and lane -> parent
      if (reached) {
        fwd = res[parent * V + lane];
        bwd = res[lane * V + parent];
      }
      uint64_t path = 0;                               // nodes on the path, source excluded
      long long bn = LLONG_MAX;
      int child = -1;                                  // this node's successor on the path
      for (int v = snk; v != src; ) {
        const int pv = __builtin_amdgcn_readlane(parent, v);
        const long long fv = (long long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(fwd >> 32), v) << 32) |
                                         (uint32_t)__builtin_amdgcn_readlane((int)fwd, v));
        bn = fv < bn ? fv : bn;
        path |= 1ull << v;
        child = lane == pv ? v : child;
        v = pv;
      }
      lp_wave_sync();
      if ((path >> lane) & 1ull) {                     // edge parent -> lane carries bn more
        const long long nf = fwd - bn;
        res[parent * V + lane] = nf;
        res[lane * V + parent] = bwd + bn;
        if (nf == 0) in &= ~(1ull << parent);
      }
      if (child >= 0) in |= 1ull << child;
      lp_wave_sync();
      if (it == kLpMaxAugment - 1) exhausted = 1;
    }
  }
  exhausted = __syncthreads_or(exhausted);
  if (exhausted) {                                     // not reachable for V <= 18; reported, never silent
    for (int i = tid; i < RK * R; i += kLpThreads) flow_b[i] = -1;
    for (int i = tid; i < RK; i += kLpThreads) load_b[i] = -1;
    if (tid == 0) {
      lam_out[b] = -1;
      status[b] = kStatusBadTopology;
    }
    return;
  }

  // ---- 4. net flow per rank pair, split over the pair's slots in slot order:
  // thread (o, g) fills the slots of rank g that replicate an expert of rank
  // o; thread (g, g) writes 0 to the slots of g that move nothing
  for (int i = tid; i < RK * RK; i += kLpThreads) {
    const int o = i / RK, g = i - o * RK;
    const long long n = o == g ? 0 : (long long)cap[o * RK + g] - res[o * V + g];
    long long left = n > 0 ? n : 0;
    for (int j = 0; j < R; ++j) {
      const int32_t x = rp[g * R + j];
      const int ox = x >= 0 ? h[x] : g;
      if (o == g) {
        if (ox == g) flow_b[g * R + j] = 0;
      } else if (ox == o) {
        const long long cx = c[x];
        const long long f = left < cx ? left : cx;
        left -= f;
        flow_b[g * R + j] = f;
      }
    }
  }
  for (int r = tid; r < RK; r += kLpThreads) {
    long long l = (long long)base[r];
    for (int g = 0; g < RK; ++g) {
      if (g == r) continue;
      const long long out_n = (long long)cap[r * RK + g] - res[r * V + g];
      const long long in_n = (long long)cap[g * RK + r] - res[g * V + r];
      l -= out_n > 0 ? out_n : 0;
      l += in_n > 0 ? in_n : 0;
    }
    load_b[r] = l;
  }
  if (tid == 0) {
    lam_out[b] = lam;
    status[b] = 0;
  }
}

// ---------------------------------------------------------------- the optimum by cuts (any RK <= 64)
// The same optimum and flow without enumerating rank sets.  Start from the
// largest of the lower bounds of the set of all ranks, ceil(total / RK), of
// each rank alone (its load minus all it can hand on) and of each pair of
// ranks, and run the maximum flow of the feasibility network at lam.  If it falls short of what
// the ranks above lam must shed, the ranks still reachable from the source
// form a set S with load(S) - cap(S -> rest) > lam * |S| (the cut that
// bounds the flow), so lam' = ceil((load(S) - cap(S -> rest)) / |S|) is a
// larger lower bound; repeat until the flow is feasible (Dinkelbach's method
// on the supply-demand bound: each round raises lam, never past the
// optimum).  The last flow is a fresh shortest-augmenting-path flow at the
// optimum, with the same predecessor rule, so it is the flow of step 3 above.
//
// One wave holds the network, a lane per rank (RK <= 64); the source and
// the sink are implicit: lane v keeps its residuals from the source and to
// the sink in registers, and `in` = the ranks u with residual u -> v.  A
// search never passes through the source (seen from the start) or the sink
// (the search ends there), so the reverse edges into them never matter.
constexpr int kLpDkThreads = 256;
constexpr int kLpMaxRounds = 1 << 12;          // rounds of the cut iteration (each one raises lam)

__host__ __device__ inline size_t lp_dk_lds_bytes(int RK, int E) {
  return (size_t)RK * RK * 16 + (size_t)RK * 8 + (((size_t)E + 31) / 32) * 4;
}

__global__ __launch_bounds__(kLpDkThreads) void lp_solve_dk_kernel(
    const int64_t* __restrict__ cnt, const int32_t* __restrict__ home, const int32_t* __restrict__ rep, int32_t E,
    int32_t RK, int32_t R, int64_t* __restrict__ lam_out, int64_t* __restrict__ flow_out,
    int64_t* __restrict__ load_out, int32_t* __restrict__ status) {
  extern __shared__ __align__(16) unsigned char lp_dk_smem[];
  unsigned long long* cap = reinterpret_cast<unsigned long long*>(lp_dk_smem);         // [RK][RK]
  long long* res = reinterpret_cast<long long*>(cap + RK * RK);                          // [RK][RK] residual
  unsigned long long* base = reinterpret_cast<unsigned long long*>(res + RK * RK);      // [RK]
  uint32_t* seen_bits = reinterpret_cast<uint32_t*>(base + RK);                          // [(E + 31) / 32]
  __shared__ long long s_lam;
  __shared__ int s_fail;

  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t* c = cnt + b * E;
  const int32_t* h = home + b * E;
  const int32_t* rp = rep + b * (int64_t)RK * R;
  int64_t* flow_b = flow_out + b * (int64_t)RK * R;
  int64_t* load_b = load_out + b * RK;

  for (int i = tid; i < RK; i += kLpDkThreads) base[i] = 0;
  for (int i = tid; i < RK * RK; i += kLpDkThreads) cap[i] = 0;
  for (int i = tid; i < (E + 31) / 32; i += kLpDkThreads) seen_bits[i] = 0;
  __syncthreads();

  // ---- home loads and rank-pair capacities (as in lp_solve_kernel)
  int bad = 0;
  for (int e = tid; e < E; e += kLpDkThreads) {
    const int64_t x = c[e];
    const int32_t r = h[e];
    const bool ok = x >= 0 && x <= kLoadMax && (uint32_t)r < (uint32_t)RK;
    bad |= !ok;
    if (ok) atomicAdd(&base[r], (unsigned long long)x);
  }
  for (int i = tid; i < RK * R; i += kLpDkThreads) {
    const int32_t x = rp[i];
    if (x == -1) continue;
    if ((uint32_t)x >= (uint32_t)E) { bad = 1; continue; }
    const uint32_t bit = 1u << (x & 31);
    if (atomicOr(&seen_bits[x >> 5], bit) & bit) { bad = 1; continue; }
    const int32_t o = h[x], g = i / R;
    const int64_t v = c[x];
    if ((uint32_t)o < (uint32_t)RK && o != g && v >= 0 && v <= kLoadMax)
      atomicAdd(&cap[o * RK + g], (unsigned long long)v);
  }
  bad = __syncthreads_or(bad);
  if (bad) {
    for (int i = tid; i < RK * R; i += kLpDkThreads) flow_b[i] = -1;
    for (int i = tid; i < RK; i += kLpDkThreads) load_b[i] = -1;
    if (tid == 0) {
      lam_out[b] = -1;
      status[b] = kStatusBadTopology;
    }
    return;
  }

  if (tid < 64) {
    const bool node = lane < RK;
    const long long bv = node ? (long long)base[lane] : 0;
    long long total = bv;
    for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);
    // lower bounds from the set of all ranks and from each rank alone
    // (its load minus all it can hand on)
    long long single = 0;
    if (node) {
      single = bv;
      for (int g = 0; g < RK; ++g) single -= (long long)cap[lane * RK + g];
    }
    // and from each pair of ranks u, v: what the two hold minus all they can
    // hand to the other ranks, over two (rounded up); the edges between u
    // and v stay inside the pair.  On the 32-rank torus batch this cut the
    // rounds from ~3.7 to ~1.4 per layer and the augmenting paths from ~53 to
    // ~12 (at most 21 in a layer, from 79), without changing the optimum the
    // rounds reach.  (Sets grown greedily from the best pair cut the mean to
    // ~9 but not the largest layer's, which sets the launch's time.)
    const long long own = single;
    long long pair = 0;
    for (int v = 0; v < RK; ++v) {
      const long long ov = (long long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(own >> 32), v) << 32) |
                                       (uint32_t)__builtin_amdgcn_readlane((int)own, v));
      if (node && lane != v) {
        const long long a = own + ov + (long long)cap[lane * RK + v] + (long long)cap[v * RK + lane];
        const long long pb = a > 0 ? (a + 1) / 2 : 0;
        pair = pb > pair ? pb : pair;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const long long o = __shfl_xor(single, off);
      single = o > single ? o : single;
      const long long q = __shfl_xor(pair, off);
      pair = q > pair ? q : pair;
    }
    long long lam = (total + RK - 1) / RK;               // total >= 0
    lam = single > lam ? single : lam;
    lam = pair > lam ? pair : lam;
    int fail = 0;
    for (int round = 0;; ++round) {
      if (round == kLpMaxRounds) { fail = 1; break; }
      // ---- the feasibility network at lam
      long long rs = node && bv > lam ? bv - lam : 0;    // source -> lane
      long long rt = node && lam > bv ? lam - bv : 0;    // lane -> sink
      long long need = rs;
      for (int off = 32; off > 0; off >>= 1) need += __shfl_xor(need, off);
      uint64_t in = 0;
      for (int u = 0; u < RK; ++u) {
        const long long cu = node ? (long long)cap[u * RK + lane] : 0;
        if (node) res[u * RK + lane] = cu;
        in |= (uint64_t)(cu > 0) << u;
      }
      lp_wave_sync();
      // ---- maximum flow by shortest augmenting paths
      long long flow = 0;
      uint64_t seen = 0;
      int it = 0;
      for (; it < kLpMaxAugment; ++it) {
        int parent = -1;                                 // 64: the source
        uint64_t frontier = __builtin_amdgcn_ballot_w64(rs > 0);
        seen = frontier;
        if (rs > 0) parent = 64;
        int last = -1;                                   // the path's rank next to the sink
        while (frontier) {
          const uint64_t ts = __builtin_amdgcn_ballot_w64(((frontier >> lane) & 1ull) && rt > 0);
          if (ts) { last = __builtin_ctzll(ts); break; }
          const uint64_t cand = node && !((seen >> lane) & 1ull) ? (in & frontier) : 0;
          if (cand) parent = __builtin_ctzll(cand);
          const uint64_t found = __builtin_amdgcn_ballot_w64(cand != 0);
          seen |= found;
          frontier = found;
        }
        if (last < 0) break;
        // residual of the tree edge into each lane, then the path from the sink back
        long long fwd = 0, bwd = 0;
        if (parent >= 0 && parent < 64) {
          fwd = res[parent * RK + lane];
          bwd = res[lane * RK + parent];
        } else if (parent == 64) {
          fwd = rs;
        }
        long long bn = (long long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(rt >> 32), last) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)rt, last));
        uint64_t path = 0;
        int child = -1;
        for (int v = last;;) {
          const int pv = __builtin_amdgcn_readlane(parent, v);
          const long long fv = (long long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(fwd >> 32), v) << 32) |
                                           (uint32_t)__builtin_amdgcn_readlane((int)fwd, v));
          bn = fv < bn ? fv : bn;
          path |= 1ull << v;
          if (pv == 64) break;
          child = lane == pv ? v : child;
          v = pv;
        }
        lp_wave_sync();
        if ((path >> lane) & 1ull) {
          if (parent == 64) {
            rs -= bn;
          } else {
            const long long nf = fwd - bn;
            res[parent * RK + lane] = nf;
            res[lane * RK + parent] = bwd + bn;
            if (nf == 0) in &= ~(1ull << parent);
          }
        }
        if (child >= 0) in |= 1ull << child;             // the reverse of the edge lane -> child
        if (lane == last) rt -= bn;
        flow += bn;
        lp_wave_sync();
      }
      if (it == kLpMaxAugment) { fail = 1; break; }
      if (flow == need) break;                           // feasible: lam is the optimum
      // the ranks reachable from the source: load(S) - cap(S -> rest) > lam |S|
      long long f = 0;
      if ((seen >> lane) & 1ull) {
        f = bv;
        for (int g = 0; g < RK; ++g)
          if (!((seen >> g) & 1ull)) f -= (long long)cap[lane * RK + g];
      }
      for (int off = 32; off > 0; off >>= 1) f += __shfl_xor(f, off);
      const int k = __popcll(seen);
      const long long next = (f + k - 1) / k;            // f > lam * k >= 0
      if (next <= lam) { fail = 1; break; }              // cannot happen; never loops
      lam = next;
    }
    if (lane == 0) {
      s_lam = lam;
      s_fail = fail;
    }
  }
  __syncthreads();
  if (s_fail) {
    for (int i = tid; i < RK * R; i += kLpDkThreads) flow_b[i] = -1;
    for (int i = tid; i < RK; i += kLpDkThreads) load_b[i] = -1;
    if (tid == 0) {
      lam_out[b] = -1;
      status[b] = kStatusBadTopology;
    }
    return;
  }
  // ---- net flow per rank pair, split over the pair's slots in slot order
  for (int i = tid; i < RK * RK; i += kLpDkThreads) {
    const int o = i / RK, g = i - o * RK;
    const long long n = o == g ? 0 : (long long)cap[o * RK + g] - res[o * RK + g];
    long long left = n > 0 ? n : 0;
    for (int j = 0; j < R; ++j) {
      const int32_t x = rp[g * R + j];
      const int ox = x >= 0 ? h[x] : g;
      if (o == g) {
        if (ox == g) flow_b[g * R + j] = 0;
      } else if (ox == o) {
        const long long cx = c[x];
        const long long f = left < cx ? left : cx;
        left -= f;
        flow_b[g * R + j] = f;
      }
    }
  }
  for (int r = tid; r < RK; r += kLpDkThreads) {
    long long l = (long long)base[r];
    for (int g = 0; g < RK; ++g) {
      if (g == r) continue;
      const long long out_n = (long long)cap[r * RK + g] - res[r * RK + g];
      const long long in_n = (long long)cap[g * RK + r] - res[g * RK + r];
      l -= out_n > 0 ? out_n : 0;
      l += in_n > 0 ? in_n : 0;
    }
    load_b[r] = l;
  }
  if (tid == 0) {
    lam_out[b] = s_lam;
    status[b] = 0;
  }
}

// ---------------------------------------------------------------- redirect by the flows
// Occurrence i (in (token, k) order within the layer) of a replicated expert
// x goes to x's replica when i < flow, else to the original.  Only the
// replicated experts need that order: each gets a compact number (its slot's
// rank among the filled slots), and the order is a per-number running count
// over the whole layer.  The layer is cut into segments of kLpSeg ids, one
// wave each: (A) count every segment's ids per compact number into the
// workspace, (B) turn the counts into exclusive prefixes over the segments,
// (C) each wave starts its counters at those prefixes and walks its segment
// 64 ids at a time.  An expert whose occurrences in the segment lie wholly
// below its flow (the next segment's prefix is at most the flow) or wholly
// at or above it is mapped by one table read; only the one segment where
// the flow runs out ranks that expert's ids: equal numbers among the lanes
// with one ballot per bit of the number (peers share every bit), so the
// numbering matches a sequential pass exactly.

// Waves per workgroup within the 64 KiB budget; a single wave whose tables
// alone exceed it (E = 4096 with 4096 filled slots: 80 KiB) still fits the
// 160 KiB of a gfx950 compute unit.
__host__ __device__ inline int lp_waves_per_block(int words_per_wave) {
  const int w = (kMaxLdsBytes / 4) / words_per_wave;
  return w < 1 ? 1 : (w > 4 ? 4 : w);
}

// cmap[e] = compact number (< C) of expert e (-1: not replicated); with
// pid/fx, the slot's physical id and its flow clamped to int32.  Returns whether the
// layer's table is bad (an id out of range, or an expert named twice).
// x0 and f0 are slot `lane`'s entry of rl and fl, read by the caller
// together with its other loads (f0 only when pid is set); slots from 64 on
// are read here.
__device__ bool lp_build_map(const int32_t* rl, const int64_t* fl, int32_t RKR, int32_t E, int32_t C,
                             int32_t* cmap, int32_t* pid, int32_t* fx, int32_t x0, int64_t f0) {
  const int lane = threadIdx.x & 63;
  for (int e = lane; e < E; e += 64) cmap[e] = -1;
  lp_wave_sync();
  int bad = 0;
  int base = 0;
  for (int i0 = 0; i0 < RKR; i0 += 64) {
    const int i = i0 + lane;
    const int32_t x = i0 == 0 ? x0 : (i < RKR ? rl[i] : -1);
    const bool inr = (uint32_t)x < (uint32_t)E;
    if (x != -1 && !inr) bad = 1;
    const uint64_t m = __builtin_amdgcn_ballot_w64(inr);
    const int c = base + __popcll(m & ((1ull << lane) - 1));
    if (inr && c >= C) bad = 1;                        // more filled slots than experts: a repeat
    if (inr && c < C) {
      if (atomicExch(&cmap[x], c) != -1) bad = 1;   // named twice
      if (pid != nullptr) {
        pid[c] = E + i;
        const int64_t f = i0 == 0 ? f0 : fl[i];
        fx[c] = f <= 0 ? 0 : (f >= 0x7fffffff ? 0x7fffffff : (int32_t)f);
      }
    }
    base += __popcll(m);
  }
  lp_wave_sync();
  return __builtin_amdgcn_ballot_w64(bad != 0) != 0;
}

__global__ __launch_bounds__(256) void lp_seg_count_kernel(const int32_t* __restrict__ idx, int64_t n, int32_t E,
                                                           const int32_t* __restrict__ rep, int32_t RKR, int32_t C,
                                                           int64_t S, int64_t LS, int32_t wpb,
                                                           int32_t* __restrict__ seg) {
  extern __shared__ int32_t lp_cnt[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t q = (int64_t)blockIdx.x * wpb + wave;
  if (q >= LS) return;                                 // whole wave; no workgroup barrier below
  const int64_t l = q / S, s = q - l * S;
  int32_t* cmap = lp_cnt + wave * (E + C);
  int32_t* cnt = cmap + E;
  for (int c = lane; c < C; c += 64) cnt[c] = 0;
  const int32_t* src = idx + l * n + s * kLpSeg;
  const int len = (int)min((int64_t)kLpSeg, n - s * kLpSeg);
  int32_t v[kLpSeg / 64];                              // the whole segment in flight at once
  if (len == kLpSeg && ((uintptr_t)src & 15) == 0) {   // uniform: counting needs no order, so 16-byte loads
    const i32x4* s4 = reinterpret_cast<const i32x4*>(src);
#pragma unroll
    for (int k = 0; k < kLpSeg / 256; ++k) {
      const i32x4 x = s4[k * 64 + lane];
      v[4 * k] = x.x;
      v[4 * k + 1] = x.y;
      v[4 * k + 2] = x.z;
      v[4 * k + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kLpSeg / 64; ++k) {
      const int i = k * 64 + lane;
      v[k] = i < len ? src[i] : -1;
    }
  }
  const int32_t* rl = rep + l * RKR;
  const int32_t x0 = lane < RKR ? rl[lane] : -1;       // with the ids: one round trip for both
  lp_build_map(rl, nullptr, RKR, E, C, cmap, nullptr, nullptr, x0, 0);
#pragma unroll
  for (int k = 0; k < kLpSeg / 64; ++k) {
    const int c = (uint32_t)v[k] < (uint32_t)E ? cmap[v[k]] : -1;
    if (c >= 0) atomicAdd(&cnt[c], 1);
  }
  lp_wave_sync();
  int32_t* dst = seg + q * C;
  for (int c = lane; c < C; c += 64) dst[c] = cnt[c];
}

// One wave per (layer, compact number), grid-stride over them: the
// segments' counts, 64 segments per pass, become exclusive prefixes by a
// wave scan.
__global__ __launch_bounds__(256) void lp_seg_scan_kernel(int32_t* __restrict__ seg, int64_t L, int64_t S,
                                                          int32_t C) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6; t < L * C; t += waves) {
    const int64_t l = t / C, c = t - l * C;
    int32_t* p = seg + l * S * C + c;
    int32_t carry = 0;
    for (int64_t s0 = 0; s0 < S; s0 += 64) {
      const int64_t sg = s0 + lane;
      const int32_t v = sg < S ? p[sg * C] : 0;
      int32_t incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(incl, off);
        incl += lane >= off ? o : 0;
      }
      if (sg < S) p[sg * C] = carry + incl - v;
      carry += __shfl(incl, 63);
    }
  }
}

__global__ __launch_bounds__(256) void lp_redirect_kernel(const int32_t* __restrict__ idx, int64_t n, int32_t E,
                                                          int32_t nbits, const int32_t* __restrict__ rep,
                                                          const int64_t* __restrict__ flow, int32_t RKR, int32_t C,
                                                          int64_t S, int64_t LS, int32_t wpb,
                                                          const int32_t* __restrict__ seg,
                                                          int32_t* __restrict__ out) {
  extern __shared__ int32_t lp_tab[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t q = (int64_t)blockIdx.x * wpb + wave;
  if (q >= LS) return;                                 // whole wave; no workgroup barrier below
  const int64_t l = q / S, s = q - l * S;
  int32_t* cmap = lp_tab + wave * (E + 4 * C);
  int32_t* run = cmap + E;                             // running occurrence count per compact number
  int32_t* pid = run + C;                              // its replica's physical id
  int32_t* fx = pid + C;                               // its replica's flow (clamped to int32)
  int32_t* nxt = fx + C;                               // the next segment's prefix
  const int32_t* src = idx + l * n + s * kLpSeg;
  int32_t* dst = out + l * n + s * kLpSeg;
  const int len = (int)min((int64_t)kLpSeg, n - s * kLpSeg);
  int32_t v[kLpSeg / 64];                              // the whole segment in flight at once
#pragma unroll
  for (int k = 0; k < kLpSeg / 64; ++k) {
    const int i = k * 64 + lane;
    v[k] = i < len ? src[i] : -1;
  }
  // the tables' first 64 entries are read with the ids (one round trip)
  const int32_t* base = seg + q * C;
  const bool has_next = s + 1 < S;
  const int32_t* rl = rep + l * RKR;
  const int64_t* fl = flow + l * RKR;
  const int32_t x0 = lane < RKR ? rl[lane] : -1;
  const int64_t f0 = lane < RKR ? fl[lane] : 0;
  const int32_t b0 = lane < C ? base[lane] : 0;
  const int32_t n0 = has_next && lane < C ? base[C + lane] : 0;
  for (int c = lane; c < C; c += 64) {
    run[c] = c == lane ? b0 : base[c];
    nxt[c] = c == lane ? n0 : (has_next ? base[C + c] : 0);
  }
  const bool bad = lp_build_map(rl, fl, RKR, E, C, cmap, pid, fx, x0, f0);
  // A replicated expert's ids in this segment all go to its replica when
  // the segment ends at or before its flow, all stay when it starts at or
  // beyond it; only in the segment where the flow runs out are they decided
  // one by one.  cmap[e] becomes -1 (stay), -2 - pid (all to the replica),
  // or the compact number (one by one).  The next segment's prefix ends this
  // one's occurrences; the layer's last segment counts as undecided.
  for (int i0 = 0; i0 < RKR && !bad; i0 += 64) {
    const int i = i0 + lane;
    const int32_t x = i0 == 0 ? x0 : (i < RKR ? rl[i] : -1);
    if ((uint32_t)x < (uint32_t)E) {
      const int c = cmap[x];
      if (c >= 0 && pid[c] == E + i) {                 // the slot that holds x's compact number
        const int32_t f = fx[c];
        if (run[c] >= f) cmap[x] = -1;
        else if (has_next && nxt[c] <= f) cmap[x] = -2 - (E + i);
      }
    }
  }
  lp_wave_sync();
  const uint64_t below = (1ull << lane) - 1;
#pragma unroll
  for (int k = 0; k < kLpSeg / 64; ++k) {
    const int i = k * 64 + lane;
    if (k * 64 >= len) break;                          // uniform
    const int32_t e = v[k];
    const bool inr = i < len && (uint32_t)e < (uint32_t)E && !bad;
    const int32_t mp = inr ? cmap[e] : -1;
    const int c = mp >= 0 ? mp : -1;
    int32_t res = inr ? (mp <= -2 ? -2 - mp : e) : -1;
    const uint64_t has = __builtin_amdgcn_ballot_w64(c >= 0);
    if (has != 0) {                                    // uniform
      uint64_t peers = has;
      for (int bit = 0; bit < nbits; ++bit) {
        const bool one = (c >> bit) & 1;
        const uint64_t m = __builtin_amdgcn_ballot_w64(c >= 0 && one);
        peers &= one ? m : ~m;
      }
      if (c >= 0) {
        const int rank = __popcll(peers & below);
        const int32_t occ = run[c] + rank;
        if (occ < fx[c]) res = pid[c];
        if (rank == 0) run[c] = occ + __popcll(peers);
      }
      lp_wave_sync();
    }
    if (i < len) dst[i] = res;
  }
}

}  // namespace

int64_t lp_segments(int64_t n) { return (n + kLpSeg - 1) / kLpSeg; }

hipError_t launch_lp_redirect(const int32_t* idx, int64_t L, int64_t n, int32_t E, const int32_t* rep,
                              const int64_t* flow, int32_t RK, int32_t R, int32_t* seg, int32_t* out,
                              hipStream_t stream) {
  const int64_t S = lp_segments(n);
  const int64_t LS = L * S;
  if (LS == 0) return hipSuccess;
  const int32_t RKR = RK * R;
  const int32_t C = RKR < E ? RKR : E;                 // compact numbers: distinct replicated experts
  int nbits = 0;
  while ((1 << nbits) < C) ++nbits;
  const int wpb_a = lp_waves_per_block(E + C);
  lp_seg_count_kernel<<<(unsigned)((LS + wpb_a - 1) / wpb_a), 64 * wpb_a, (size_t)wpb_a * (E + C) * 4, stream>>>(
      idx, n, E, rep, RKR, C, S, LS, wpb_a, seg);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t scan_blocks = (L * C + 3) / 4;         // four waves per workgroup, grid-stride beyond 2^16
  lp_seg_scan_kernel<<<(unsigned)(scan_blocks < 65536 ? scan_blocks : 65536), 256, 0, stream>>>(seg, L, S, C);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int wpb_c = lp_waves_per_block(E + 4 * C);
  lp_redirect_kernel<<<(unsigned)((LS + wpb_c - 1) / wpb_c), 64 * wpb_c, (size_t)wpb_c * (E + 4 * C) * 4, stream>>>(
      idx, n, E, nbits, rep, flow, RKR, C, S, LS, wpb_c, seg, out);
  return hipGetLastError();
}

hipError_t launch_lp_solve(const int64_t* cnt, const int32_t* home, const int32_t* rep, int64_t B, int32_t E,
                           int32_t RK, int32_t R, int64_t* lam, int64_t* flow, int64_t* rank_load,
                           int32_t* status, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (RK > kLpEnumRanks) {
    lp_solve_dk_kernel<<<(unsigned)B, kLpDkThreads, lp_dk_lds_bytes(RK, E), stream>>>(cnt, home, rep, E, RK, R, lam,
                                                                                       flow, rank_load, status);
    return hipGetLastError();
  }
  if (RK < kLpSplitRanks) {
    lp_solve_kernel<0><<<(unsigned)B, kLpThreads, 0, stream>>>(cnt, home, rep, E, RK, R, 1, lam, flow, rank_load,
                                                               status);
    return hipGetLastError();
  }
  lp_solve_kernel<1><<<(unsigned)(B * kLpParts), kLpThreads, 0, stream>>>(cnt, home, rep, E, RK, R, kLpParts, lam,
                                                                          flow, rank_load, status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  lp_solve_kernel<2><<<(unsigned)B, kLpThreads, 0, stream>>>(cnt, home, rep, E, RK, R, kLpParts, lam, flow, rank_load,
                                                             status);
  return hipGetLastError();
}

}  // namespace eplb
