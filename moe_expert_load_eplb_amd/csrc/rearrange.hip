// Rearrangement plan: turn the placement in force into a new one while moving
// as few expert weights as possible.
//
// The pages end at the placement (the rebalance assigns replicas to GPUs:
// opening section and "Алгоритм" of Part 2 of the EPLB README translation,
// «DualPipe и EPLB», ai.flicky.cc) and are silent on moving weights; this is
// the plain completion.  Positions inside a rank are interchangeable, so the
// new placement stays rank for rank and is only permuted within each rank:
// for every expert the first m old slots of the rank that hold it stay
// (m = min of its old and new copies on the rank), matched in order to the
// first m new slots holding it; the remaining new slots, ascending, take the
// freed old slots, ascending.  A freed slot fetches its expert from an old
// slot that holds it: on the same rank if possible (such a slot is always a
// kept one), else on the same node, else anywhere; the lowest slot of that
// class.  Fetch count = ppr minus the multiset overlap of each rank, the
// least a within-rank permutation allows.
//
// One workgroup per problem.  The problem's two phy2log rows live in LDS as
// 16-bit values (expert ids < 4096; bit 15 later marks "kept" / "matched"),
// with the permutation (new slot -> plan slot) and, when they fit, the lowest
// old slot of each expert overall and on each node.  The matching steps are
// short scans over one rank's slots by one thread per slot; a source on the
// node or anywhere is then one table read.  Integer work, latency-bound.
#include "eplb_internal.h"

namespace eplb {

namespace {

constexpr int kRaThreads = 256;
constexpr uint16_t kFlag = 0x8000;
constexpr uint16_t kId = 0x7fff;
constexpr int kNoSlot = 1 << 30;

// Lowest slot in [lo, hi) whose old expert is e, or kNoSlot.  No early exit:
// the LDS reads of the scan do not wait on one another.
__device__ __forceinline__ int first_holder(const uint16_t* olde, int lo, int hi, int e) {
  int q = kNoSlot;
#pragma unroll 4
  for (int x = hi - 1; x >= lo; --x) q = (olde[x] & kId) == e ? x : q;
  return q;
}

// kTables: the lowest old slot of every expert, overall and per node, are
// kept in LDS (built with atomicMin while staging), so finding a source on
// the node or anywhere is one read.  Without them (tables too large for the
// LDS budget) both are scans.
template <bool kTables>
__global__ __launch_bounds__(kRaThreads) void rearrange_kernel(
    const int32_t* __restrict__ old_p2l, const int32_t* __restrict__ new_p2l,
    const int32_t* __restrict__ new_l2p, int32_t E, int32_t P, int32_t RK, int32_t N, int32_t X,
    int32_t* __restrict__ plan, int32_t* __restrict__ l2p_out, int32_t* __restrict__ src,
    int32_t* __restrict__ moves, int32_t* __restrict__ status) {
  extern __shared__ uint32_t ra_smem[];
  // kTables: first[E], nfirst[N][E] (lowest old slot of each expert, overall
  // and per node; kNoSlot if none).  Otherwise: present[ceil(E/32)] bits.
  const int head_words = kTables ? E * (N + 1) : (E + 31) / 32;
  uint32_t* first = ra_smem;
  uint32_t* nfirst = ra_smem + E;
  uint32_t* present = ra_smem;
  uint16_t* olde = reinterpret_cast<uint16_t*>(ra_smem + head_words);   // [P] old expert (| kFlag: kept)
  uint16_t* newe = olde + P;                                        // [P] new expert (| kFlag: matched)
  uint16_t* perm = newe + P;                                        // [P] new slot -> slot in the plan
  __shared__ int32_t s_moves[3];

  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int ppr = P / RK;
  const int per_node = P / N;
  const int EX = E * X;                                             // < 2^28 by the host limits
  const int32_t* o = old_p2l + b * P;
  const int32_t* n = new_p2l + b * P;
  const int32_t* l = new_l2p + b * (int64_t)EX;
  int32_t* plan_b = plan + b * P;
  int32_t* src_b = src + b * P;
  int32_t* l2p_b = l2p_out + b * (int64_t)EX;

  // ---- stage both rows, check every entry's range
  if (tid < 3) s_moves[tid] = 0;
  for (int w = tid; w < head_words; w += kRaThreads) ra_smem[w] = kTables ? (uint32_t)kNoSlot : 0u;
  __syncthreads();
  int bad = 0;
  for (int p = tid; p < P; p += kRaThreads) {
    const int32_t a = o[p], c = n[p];
    const bool ok = (uint32_t)a < (uint32_t)E && (uint32_t)c < (uint32_t)E;
    bad |= !ok;
    olde[p] = (uint16_t)(a & kId);
    newe[p] = (uint16_t)(c & kId);
    if (ok) {
      if (kTables) {
        atomicMin(&first[a], (uint32_t)p);
        atomicMin(&nfirst[(p / per_node) * E + a], (uint32_t)p);
      } else {
        atomicOr(&present[a >> 5], 1u << (a & 31));
      }
    }
  }
#pragma unroll 4
  for (int i = tid; i < EX; i += kRaThreads) {
    const int32_t v = l[i];
    bad |= (v < -1) | (v >= P);
  }
  __syncthreads();
  for (int p = tid; p < P && !bad; p += kRaThreads) {
    const int e = newe[p];
    const bool has = kTables ? first[e] != (uint32_t)kNoSlot : ((present[e >> 5] >> (e & 31)) & 1u);
    bad |= !has;                                                    // a new expert with no old replica
  }
  bad = __syncthreads_or(bad);

  if (bad) {
    for (int p = tid; p < P; p += kRaThreads) {
      plan_b[p] = -1;
      src_b[p] = -1;
    }
    for (int i = tid; i < EX; i += kRaThreads) l2p_b[i] = -1;
    if (tid < 3) moves[b * 3 + tid] = -1;
    if (tid == 0) status[b] = kStatusBadMap;
    return;
  }

  // ---- match: the k-th new slot of a rank holding e takes the k-th old slot
  // holding e; an old slot stays if fewer earlier old slots of the rank hold
  // its expert than new slots of the rank do
  uint32_t kept = 0, matched = 0;                                   // bit j: slot tid + j * kRaThreads
  for (int j = 0, p = tid; p < P; ++j, p += kRaThreads) {
    const int base = (p / ppr) * ppr, end = base + ppr;
    const int e = newe[p], f = olde[p];
    int k = 0, before = 0, want = 0;
#pragma unroll 4
    for (int x = base; x < end; ++x) {
      const int ne = newe[x], oe = olde[x];
      k += (x < p) & (ne == e);
      before += (x < p) & (oe == f);
      want += ne == f;
    }
    int q = kNoSlot, seen = 0;
#pragma unroll 4
    for (int x = base; x < end; ++x) {
      const int hit = olde[x] == e;
      q = (hit & (seen == k) & (q == kNoSlot)) ? x : q;
      seen += hit;
    }
    if (q != kNoSlot) {
      perm[p] = (uint16_t)q;
      matched |= 1u << j;
    }
    if (before < want) kept |= 1u << j;
  }
  __syncthreads();
  for (int j = 0, p = tid; p < P; ++j, p += kRaThreads) {
    if ((kept >> j) & 1u) olde[p] |= kFlag;
    if ((matched >> j) & 1u) newe[p] |= kFlag;
  }
  __syncthreads();
  // ---- the v-th freed slot of a rank takes the v-th unmatched new slot
  for (int j = 0, q = tid; q < P; ++j, q += kRaThreads) {
    if ((kept >> j) & 1u) continue;
    const int base = (q / ppr) * ppr, end = base + ppr;
    int v = 0;
#pragma unroll 4
    for (int x = base; x < q; ++x) v += !(olde[x] & kFlag);
    int t = kNoSlot, seen = 0;
#pragma unroll 4
    for (int x = base; x < end; ++x) {
      const int free_new = !(newe[x] & kFlag);
      t = (free_new & (seen == v) & (t == kNoSlot)) ? x : t;
      seen += free_new;
    }
    if (t != kNoSlot) perm[t] = (uint16_t)q;                        // always: as many unmatched as freed
  }
  __syncthreads();
  // ---- the plan, and a source for every freed slot
  int cnt[3] = {0, 0, 0};
  for (int j = 0, p = tid; p < P; ++j, p += kRaThreads) {
    const int s = perm[p];
    const int e = newe[p] & kId;
    plan_b[s] = e;
    if ((matched >> j) & 1u) {
      src_b[s] = -1;
      continue;
    }
    const int rbase = (s / ppr) * ppr;
    int q = first_holder(olde, rbase, rbase + ppr, e), cls = 0;
    if (q == kNoSlot) {
      cls = 1;
      if (kTables) {
        q = (int)nfirst[(s / per_node) * E + e];
      } else {
        const int nbase = (s / per_node) * per_node;
        q = first_holder(olde, nbase, nbase + per_node, e);
      }
    }
    if (q == kNoSlot) {
      cls = 2;
      q = kTables ? (int)first[e] : first_holder(olde, 0, P, e);
    }
    src_b[s] = q;                                                   // found: e is present
    ++cnt[cls];
  }
  for (int c = 0; c < 3; ++c)
    if (cnt[c]) atomicAdd(&s_moves[c], cnt[c]);
#pragma unroll 4
  for (int i = tid; i < EX; i += kRaThreads) {
    const int32_t v = l[i];
    l2p_b[i] = v >= 0 ? (int32_t)perm[v] : -1;
  }
  __syncthreads();
  if (tid < 3) moves[b * 3 + tid] = s_moves[tid];
  if (tid == 0) status[b] = 0;
}

bool rearrange_tables_fit(int32_t E, int32_t P, int32_t N) {
  return (int64_t)E * (N + 1) * 4 + (int64_t)P * 6 + 64 <= kMaxLdsBytes;
}

}  // namespace

int64_t rearrange_lds_bytes(int32_t E, int32_t P, int32_t N) {
  const int64_t head = rearrange_tables_fit(E, P, N) ? (int64_t)E * (N + 1) : (E + 31) / 32;
  return head * 4 + (int64_t)P * 6;
}

hipError_t launch_rearrange(const int32_t* old_p2l, const int32_t* new_p2l, const int32_t* new_l2p, int64_t B,
                            int32_t E, int32_t P, int32_t RK, int32_t N, int32_t X, int32_t* plan,
                            int32_t* l2p_out, int32_t* src, int32_t* moves, int32_t* status,
                            hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const size_t lds = (size_t)rearrange_lds_bytes(E, P, N);
  if (rearrange_tables_fit(E, P, N))
    rearrange_kernel<true><<<(unsigned)B, kRaThreads, lds, stream>>>(old_p2l, new_p2l, new_l2p, E, P, RK, N, X,
                                                                     plan, l2p_out, src, moves, status);
  else
    rearrange_kernel<false><<<(unsigned)B, kRaThreads, lds, stream>>>(old_p2l, new_p2l, new_l2p, E, P, RK, N, X,
                                                                      plan, l2p_out, src, moves, status);
  return hipGetLastError();
}

}  // namespace eplb
