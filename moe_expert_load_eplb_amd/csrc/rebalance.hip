// Batched EPLB rebalance: one workgroup per problem (an MoE layer or a load
// snapshot), one wavefront per node, the whole problem resident in LDS and
// registers.
//
// The policy is the one of the EPLB README and its annotated source on the
// translation page «DualPipe и EPLB: конвейер в обе стороны и балансировщик
// экспертов» (ai.flicky.cc), Part 2: section "Алгоритм" (hierarchical when
// the node count divides the group count, else global), the flowchart (global
// = the same three steps with one group on one node), and the appendix's
// packing, replication and hierarchical routines:
//   step 1  sum each group's load and pack the groups onto the nodes,
//           heaviest first, each into the lightest node with room;
//   step 2  within each node, add each redundant replica to the expert with
//           the highest load per replica;
//   step 3  pack the node's physical experts (load = expert load / count)
//           onto the node's GPUs the same way as step 1.
//
// Exact integer arithmetic.  Step 2 compares u_a / c_a with u_b / c_b by
// cross-multiplication (u <= 2^40, c <= 16128, products < 2^54).  Step 3
// scales every per-replica load by D = lcm(replica counts of the node): item
// keys u * (D / c) and pack sums are exact integers, 64-bit when
// D * (node load sum) < 2^64, else 128-bit; a node with D * sum >= 2^127
// marks the problem EPLB_S_OVERFLOW.  D comes from a table of prime powers
// (the product of p over the prime powers p^k that divide some count), and
// D / c from an exact long division by c.
//
// The two greedy procedures are sequential chains.  Each runs in one
// wavefront with its state in registers, kept SORTED across the lanes (the
// element at position pos lives in register pos / 64 of lane pos % 64):
//   packing      positions hold packs ordered by (sum, pack index), full
//                packs last.  An item goes to the pack at position 0; the
//                updated pack is re-inserted at the position one ballot
//                counts, and the positions before it move down one lane
//                (DPP wave_shl).  No reduction tree, no LDS on the chain.
//                With 4 or more packs in the one-word form, RUNS of items
//                go at once: item j+s takes the pack at position s while
//                that pack stays below every earlier item's updated pack,
//                which each lane checks for its own item in parallel; up to
//                64 packs are then re-sorted by a sorting network across
//                the lanes, more in LDS.  A pack is one 64-bit word (sum,
//                pack, items), or one 32-bit word when the sums stay below
//                2^24 on at most 16 packs.
//   replication  positions hold experts ordered by (load per replica desc,
//                index asc).  The expert at position 0 gets the replica and
//                is re-inserted the same way.  With 24 to 64 replicas on a
//                node they are all taken at once instead (the D'Hondt form:
//                the first Rn of the candidates u / k in the greedy's own
//                order, found by counting and a sorting network).
// After replication the experts are already in the order step 3 visits them
// (per-replica load desc); the stable order of the node's physical experts
// (equal loads in ascending physical index) follows from prefix sums over
// that order, so no sort is needed.
#include <climits>

#include "eplb.h"
#include "eplb_internal.h"

namespace eplb {

namespace {

// ---------------------------------------------------------------- prime powers
// Every prime power q = p^k (k >= 1) up to kMaxCount, ascending, with its
// prime p and the magic numbers of a division by q.
struct PrimePowers {           // 32-bit fields: read with scalar loads
  uint32_t q[2048];
  uint32_t p[2048];
  uint32_t mul[2048];
  int32_t shift[2048];
  int count;
};

constexpr PrimePowers make_prime_powers() {
  PrimePowers t{};
  int spf[kMaxCount + 1] = {};               // smallest prime factor
  for (int i = 2; i <= kMaxCount; ++i) {
    if (spf[i] == 0) {
      for (int j = i; j <= kMaxCount; j += i)
        if (spf[j] == 0) spf[j] = i;
    }
  }
  int n = 0;
  for (int q = 2; q <= kMaxCount; ++q) {
    const int p = spf[q];
    int r = q;
    while (r % p == 0) r /= p;
    if (r == 1) {                            // q is a power of p
      int l = 0;
      while ((1 << l) < q) ++l;
      t.q[n] = (uint32_t)q;
      t.p[n] = (uint32_t)p;
      t.mul[n] = (uint32_t)((((unsigned long long)1) << (31 + l)) / (unsigned long long)q + 1);
      t.shift[n] = l - 1;
      ++n;
    }
  }
  t.count = n;
  return t;
}

__device__ __constant__ PrimePowers kPrimePowers = make_prime_powers();

// The prime powers q = p^k <= 64 with p and the mask of their multiples up
// to 64 (bit c - 1 set for c = q, 2q, ...): for counts up to 64, "q divides
// some count" is one AND with the mask of the counts present.
struct SmallPrimePowers {
  int n;
  uint32_t q[32];
  uint32_t p[32];
  unsigned long long mult[32];
};
constexpr SmallPrimePowers make_small_prime_powers() {
  SmallPrimePowers t{};
  for (int q = 2; q <= 64; ++q) {
    int p = 2;
    while (q % p != 0) ++p;                  // smallest prime factor
    int r = q;
    while (r % p == 0) r /= p;
    if (r != 1) continue;
    unsigned long long m = 0;
    for (int c = q; c <= 64; c += q) m |= 1ull << (c - 1);
    t.q[t.n] = (uint32_t)q;
    t.p[t.n] = (uint32_t)p;
    t.mult[t.n] = m;
    ++t.n;
  }
  return t;
}

// ---------------------------------------------------------------- lane helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int shl1(int x) {           // lane i <- lane i + 1 (lane 63 <- 0)
  return __builtin_amdgcn_mov_dpp(x, 0x130, 0xF, 0xF, true);
}
__device__ __forceinline__ int shr1(int x) {           // lane i <- lane i - 1 (lane 0 <- 0)
  return __builtin_amdgcn_mov_dpp(x, 0x138, 0xF, 0xF, true);
}
// Per-step records of a chain: each step shifts the record register up one
// lane and puts its value in lane 0 (no branch on the chain); after n steps
// lane i holds step n-1-i.
__device__ __forceinline__ int push_record(int rec, int x) {
  const int v = shr1(rec);
  return lane_id() == 0 ? x : v;
}
__device__ __forceinline__ int rdl(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ u64 rdl64(u64 x, int l) {
  const int lo = rdl((int)(uint32_t)x, l);
  const int hi = rdl((int)(uint32_t)(x >> 32), l);
  return ((u64)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ u64 shl1_64(u64 x) {
  const int lo = shl1((int)(uint32_t)x);
  const int hi = shl1((int)(uint32_t)(x >> 32));
  return ((u64)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ u64 ballot(bool b) { return __ballot(b); }
// Orders this wavefront's LDS accesses before and after it (no workgroup sync).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// y[pos] = x[pos + 1] over the K registers (pos = r * 64 + lane); the last
// position gets 0.
template <int K>
__device__ __forceinline__ void shift_down(const int (&x)[K], int (&y)[K]) {
#pragma unroll
  for (int r = 0; r < K; ++r) {
    int v = shl1(x[r]);
    if (r + 1 < K) {
      const int carry = rdl(x[r + 1], 0);
      if (lane_id() == 63) v = carry;
    }
    y[r] = v;
  }
}
template <int K>
__device__ __forceinline__ void shift_down64(const u64 (&x)[K], u64 (&y)[K]) {
#pragma unroll
  for (int r = 0; r < K; ++r) {
    u64 v = shl1_64(x[r]);
    if (r + 1 < K) {
      const u64 carry = rdl64(x[r + 1], 0);
      if (lane_id() == 63) v = carry;
    }
    y[r] = v;
  }
}

__device__ __forceinline__ u128 mul_u128_u64(u128 a, u64 b, bool& ovf) {
  const u64 lo = (u64)a;
  const u64 hi = (u64)(a >> 64);
  const u128 plo = (u128)lo * b;
  const u128 phi = (u128)hi * b;
  if ((u64)(phi >> 64) != 0) ovf = true;
  const u128 r = plo + ((u128)(u64)phi << 64);
  if (r < plo) ovf = true;
  return r;
}

// Wave-wide scans and reductions on DPP moves (no LDS round trips): within
// each row of 16 lanes a Hillis-Steele scan with row_shr 1, 2, 4, 8, then
// row 0's total into row 1 and row 2's into row 3 (row_bcast:15), then the
// first two rows' total into rows 2 and 3 (row_bcast:31).  Lanes without a
// source take `id`, the operation's identity.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ int dpp(int id, int x) {
  return __builtin_amdgcn_update_dpp(id, x, kCtrl, kRowMask, 0xF, false);
}
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ u64 dpp64(u64 id, u64 x) {
  const int lo = dpp<kCtrl, kRowMask>((int)(uint32_t)id, (int)(uint32_t)x);
  const int hi = dpp<kCtrl, kRowMask>((int)(uint32_t)(id >> 32), (int)(uint32_t)(x >> 32));
  return ((u64)(uint32_t)hi << 32) | (uint32_t)lo;
}
template <class T, class Op>
__device__ __forceinline__ T wave_scan_incl(T v, T id, Op op) {
  if constexpr (sizeof(T) == 8) {
    v = op(v, dpp64<0x111>(id, v));
    v = op(v, dpp64<0x112>(id, v));
    v = op(v, dpp64<0x114>(id, v));
    v = op(v, dpp64<0x118>(id, v));
    v = op(v, dpp64<0x142, 0xA>(id, v));
    v = op(v, dpp64<0x143, 0xC>(id, v));
  } else {
    v = op(v, dpp<0x111>(id, v));
    v = op(v, dpp<0x112>(id, v));
    v = op(v, dpp<0x114>(id, v));
    v = op(v, dpp<0x118>(id, v));
    v = op(v, dpp<0x142, 0xA>(id, v));
    v = op(v, dpp<0x143, 0xC>(id, v));
  }
  return v;
}
// lane i <- lane i - 1, lane 0 <- id
__device__ __forceinline__ int shr1_or(int id, int x) { return dpp<0x138>(id, x); }
__device__ __forceinline__ u64 shr1_or64(u64 id, u64 x) { return dpp64<0x138>(id, x); }

// D / c for a count c in [1, 2^14], D of `digits` 32-bit digits: long
// division digit by digit.  Each partial numerator r * 2^32 + digit is below
// c * 2^32 <= 2^46, exact as a double; its product with the correctly rounded
// 1 / c is within 2^-20 of the true quotient (below 2^32), so truncating it
// gives the quotient or one less, and the remainder check fixes the latter.
__device__ __forceinline__ u128 div_by_count(u128 D, int digits, uint32_t c) {
  const double rc = 1.0 / (double)c;
  u128 q = 0;
  u64 r = 0;
#pragma unroll
  for (int k = 3; k >= 0; --k) {
    if (k >= digits) continue;
    const u64 num = (r << 32) | (uint32_t)(D >> (32 * k));
    u64 qk = (u64)((double)num * rc);
    int64_t rem = (int64_t)(num - qk * c);
    if (rem < 0) {
      qk -= 1;
      rem += c;
    } else if (rem >= (int64_t)c) {
      qk += 1;
      rem -= c;
    }
    q = (q << 32) | qk;
    r = (u64)rem;
  }
  return q;
}

__device__ __forceinline__ u64 wave_sum64(u64 v) {
  return rdl64(wave_scan_incl<u64>(v, 0ull, [](u64 a, u64 b) { return a + b; }), 63);
}
__device__ __forceinline__ u64 wave_or64(u64 v) {
  return rdl64(wave_scan_incl<u64>(v, 0ull, [](u64 a, u64 b) { return a | b; }), 63);
}
__device__ __forceinline__ int wave_max(int v) {
  return rdl(wave_scan_incl<int>(v, INT_MIN, [](int a, int b) { return a > b ? a : b; }), 63);
}
__device__ __forceinline__ int wave_incl_sum(int v) {
  return wave_scan_incl<int>(v, 0, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ int wave_incl_max(int v) {
  return wave_scan_incl<int>(v, INT_MIN, [](int a, int b) { return a > b ? a : b; });
}
__device__ __forceinline__ int wave_incl_min(int v) {
  return wave_scan_incl<int>(v, INT_MAX, [](int a, int b) { return a < b ? a : b; });
}

// ---------------------------------------------------------------- greedy packing
// n items, visited in order (item t's key: key_of(t, w) for its KW 64-bit
// words, least significant first), go into m packs of `cap` items:
// each into the pack with the smallest sum among packs with room, lowest pack
// index on ties.  res[t] = pack * cap + arrival position of item t.
// The packs stay sorted across the K registers of the wave (m <= 64 * K);
// the element at position 0 is also kept in scalar registers.  Each step
// reads the element at position 1 before the update: after it, position 0
// holds either that element (the updated pack moved back, q > 0) or the
// updated pack itself (q == 0), so the next step starts without waiting for
// the vector update.
template <int K, int KW, class KeyOf>
__device__ void pack_sorted(KeyOf key_of, int n, int m, int cap, int32_t* res) {
  const int lane = lane_id();
  u64 s[KW][K];
  int ic[K];                                   // pack index << 16 | items in it
#pragma unroll
  for (int r = 0; r < K; ++r) {
    const int pos = r * 64 + lane;
#pragma unroll
    for (int w = 0; w < KW; ++w) s[w][r] = pos < m ? 0ull : ~0ull;
    ic[r] = pos < m ? (pos << 16) : (0x7fff << 16);
  }
  u64 s0[KW];
#pragma unroll
  for (int w = 0; w < KW; ++w) s0[w] = 0;
  int ic0 = 0;                                 // pack 0, empty
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int tn = n - t0 < 64 ? n - t0 : 64;
    u64 kk[KW];
#pragma unroll
    for (int w = 0; w < KW; ++w) kk[w] = lane < tn ? key_of(t0 + lane, w) : 0ull;
    int rec = 0;
    for (int j = 0; j < tn; ++j) {
      u64 s1[KW];
#pragma unroll
      for (int w = 0; w < KW; ++w) s1[w] = rdl64(s[w][0], 1);
      const int ic1 = rdl(ic[0], 1);
      const int c0 = ic0 & 0xffff;
      const int id0 = ic0 & ~0xffff;
      rec = push_record(rec, (ic0 >> 16) * cap + c0);
      u64 nk[KW];
      u64 carry = 0;
#pragma unroll
      for (int w = 0; w < KW; ++w) {
        const u64 t = s0[w] + rdl64(kk[w], j);
        const u64 c1 = t < s0[w] ? 1ull : 0ull;
        nk[w] = t + carry;
        carry = c1 | (nk[w] < t ? 1ull : 0ull);
      }
      const int nc = c0 + 1;
      if (nc == cap) {
#pragma unroll
        for (int w = 0; w < KW; ++w) nk[w] = ~0ull;
      }
      const int nic = id0 | nc;
      int q = 0;
#pragma unroll
      for (int r = 0; r < K; ++r) {
        if (r > 0 && q < 64 * r - 1) break;       // sorted: nothing further is below
        bool lt = (ic[r] & ~0xffff) < id0;        // decides equal sums
#pragma unroll
        for (int w = 0; w < KW; ++w) lt = (s[w][r] < nk[w]) || (s[w][r] == nk[w] && lt);
        u64 mask = __builtin_amdgcn_ballot_w64(lt);
        if (r == 0) mask &= ~1ull;
        q += __popcll(mask);
      }
      u64 sd[KW][K];
      int icd[K];
#pragma unroll
      for (int w = 0; w < KW; ++w) shift_down64<K>(s[w], sd[w]);
      shift_down<K>(ic, icd);
#pragma unroll
      for (int r = 0; r < K; ++r) {
        const int pos = r * 64 + lane;
        const bool below = pos < q;
        const bool at = pos == q;
#pragma unroll
        for (int w = 0; w < KW; ++w) s[w][r] = below ? sd[w][r] : (at ? nk[w] : s[w][r]);
        ic[r] = below ? icd[r] : (at ? nic : ic[r]);
      }
      if (q > 0) {
#pragma unroll
        for (int w = 0; w < KW; ++w) s0[w] = s1[w];
        ic0 = ic1;
      } else {
#pragma unroll
        for (int w = 0; w < KW; ++w) s0[w] = nk[w];
        ic0 = nic;
      }
    }
    if (lane < tn) res[t0 + tn - 1 - lane] = rec;
  }
}

__device__ __forceinline__ u64 shfl64(u64 x, int src) {
  const int lo = __shfl((int)(uint32_t)x, src);
  const int hi = __shfl((int)(uint32_t)(x >> 32), src);
  return ((u64)(uint32_t)hi << 32) | (uint32_t)lo;
}

// The rest of a packing once every remaining item has load 0 (its key adds
// only an item, so the sums, and with them the order of the packs, no
// longer change): the greedy fills the packs in their current order, each
// up to its capacity.  A pack at sorted position s with `fr` free slots and
// `before` free slots ahead of it takes items first + before .. + fr - 1,
// arriving after its `items` items.
__device__ __forceinline__ void fill_zero_keys_from(int fr, int before, int pack, int items, int first, int n,
                                                    int cap, int32_t* res) {
  for (int q = 0; q < fr; ++q) {
    const int t = first + before + q;
    if (t < n) res[t] = pack * cap + items + q;
  }
}
// the same for packs held one per lane (positions = lanes)
__device__ __forceinline__ void fill_zero_keys(int fr, int pack, int items, int first, int n, int cap,
                                               int32_t* res) {
  fill_zero_keys_from(fr, wave_incl_sum(fr) - fr, pack, items, first, n, cap, res);
}

// pack_words for 65 to 64 * K packs (K = 2..4 registers), with runs of items
// placed at once.  The packs' words are sorted and all distinct (a full or
// absent pack is a sentinel: all-ones sum and its pack bits, above every
// real word; real sums stay below 2^48 - 1).  Item j+s goes to the s-th
// lightest pack exactly while s is below q_t for every earlier t of the run,
// q_t being the number of packs lighter than the t-th pack after it takes
// item j+t (the packs are sorted, so "the s-th pack is lighter" is
// "s < q_t").  Every lane s tries item j+s at once: q_s by a two-level
// search of the sorted words in LDS (every GS-th word, then GS words), the
// prefix minimum of q over the lanes before s (DPP), and the run ends at the
// first lane that fails.  Its packs are then re-ranked: a run pack t lands
// at (q_t - run) + (run packs now below it, by comparing words), any other
// pack at position i at (i - run) + (run packs with q_t <= i, from a
// histogram of the q_t and its prefix sums), and each word is written to its
// new position in LDS.  The result is the sequential greedy's, item for
// item.  scr: 64 * K + 64 words and 64 * K + 1 counters of this wave's LDS
// (16-byte aligned): the sorted words, the run's updated words, the histogram.

// inclusive prefix sum over the lanes plus `carry`, which becomes the total so far
__device__ __forceinline__ int wave_incl_sum_carry(int v, int& carry) {
  const int incl = wave_incl_sum(v) + carry;
  carry = rdl(incl, 63);
  return incl;
}

template <int K, class KeyOf>
__device__ void pack_words_wide(KeyOf key_of, int n, int m, int cap, int32_t* res, u64* scr) {
  constexpr u64 kSent = 0xFFFFFFFFFFFF0000ull;
  constexpr int NP = 64 * K;                       // positions
  constexpr int GS = K <= 2 ? 8 : 16;              // words per group of the two-level search
  constexpr int NG = NP / GS;
  const int lane = lane_id();
  u64* sw = scr;                                   // [NP] words by position
  u64* su = scr + NP;                              // [64] updated word of each run candidate
  int* hist = (int*)(scr + NP + 64);               // [NP + 1] run packs by landing point
  u64 w[K];
#pragma unroll
  for (int r = 0; r < K; ++r) {
    const int pos = r * 64 + lane;
    w[r] = pos < m ? ((u64)pos << 8) : (kSent | ((u64)pos << 8) | 0xffull);
    sw[pos] = w[r];
  }
  wave_lds_sync();
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int tn = n - t0 < 64 ? n - t0 : 64;
    const u64 kk = lane < tn ? key_of(t0 + lane) : 0ull;
    const int nz = __popcll(__builtin_amdgcn_ballot_w64(lane < tn && kk != 1ull));   // items of load > 0 first
    for (int j = 0; j < nz; ) {
      const int it = j + lane;                     // this lane's candidate item
      const u64 k = shfl64(kk, it & 63);
      const bool real = w[0] < kSent;
      u64 us = w[0] + k;
      if ((int)(us & 0xff) == cap) us = kSent | (us & 0xff00ull) | 0xffull;
      su[lane] = us;
#pragma unroll
      for (int r = 0; r <= K; ++r)
        if (r < K || lane == 0) hist[r * 64 + lane] = 0;
      int b = 0;                                   // groups of GS words wholly below us
#pragma unroll
      for (int g = 0; g < NG; ++g) b += sw[GS * g + GS - 1] < us ? 1 : 0;
      const ulonglong2* f = (const ulonglong2*)(sw + GS * (b < NG ? b : NG - 1));
      int fine = 0;
#pragma unroll
      for (int h = 0; h < GS / 2; ++h) {
        const ulonglong2 fw = f[h];
        fine += (fw.x < us ? 1 : 0) + (fw.y < us ? 1 : 0);
      }
      const int q = b == NG ? NP : GS * b + fine;  // words below us
      const int pm = shr1_or(1 << 20, wave_incl_min(q));   // minimum of q over the lanes before
      const u64 vm = __builtin_amdgcn_ballot_w64(it < nz && real && lane < pm);
      const int mb = ~vm == 0 ? 64 : __builtin_ctzll(~vm);      // lane 0 is always valid
      if (lane < mb) res[t0 + j + lane] = (int)((w[0] >> 8) & 0xff) * cap + (int)(w[0] & 0xff);
      wave_lds_sync();
      if (lane < mb) atomicAdd(&hist[q], 1);
      int crun = 0;                                // run packs now below this lane's updated word
      const ulonglong2* ru = (const ulonglong2*)su;
      for (int t = 0; t < mb; t += 8) {            // eight words per round, four reads in flight
        const ulonglong2 a0 = ru[t / 2], a1 = ru[t / 2 + 1], a2 = ru[t / 2 + 2], a3 = ru[t / 2 + 3];
        crun += (a0.x < us) + (t + 1 < mb && a0.y < us) + (t + 2 < mb && a1.x < us) + (t + 3 < mb && a1.y < us) +
                (t + 4 < mb && a2.x < us) + (t + 5 < mb && a2.y < us) + (t + 6 < mb && a3.x < us) +
                (t + 7 < mb && a3.y < us);
      }
      wave_lds_sync();
      int carry = 0;
      int pos[K];
#pragma unroll
      for (int r = 0; r < K; ++r) {
        const int p = r * 64 + lane;
        const int below = wave_incl_sum_carry(hist[p], carry);   // run packs with q_t <= p
        pos[r] = (r == 0 && lane < mb) ? q - mb + crun : p - mb + below;
      }
      wave_lds_sync();
#pragma unroll
      for (int r = 0; r < K; ++r) {
        const int p = r * 64 + lane;
        if (p < m) sw[pos[r]] = (r == 0 && lane < mb) ? us : w[r];
      }
      wave_lds_sync();
#pragma unroll
      for (int r = 0; r < K; ++r) w[r] = sw[r * 64 + lane];
      j += mb;
    }
    if (nz < tn) {                                 // the rest has load 0
      int carry = 0;
#pragma unroll
      for (int r = 0; r < K; ++r) {
        const int items = (int)(w[r] & 0xff);
        const int fr = r * 64 + lane < m && w[r] < kSent ? cap - items : 0;
        const int before = wave_incl_sum_carry(fr, carry) - fr;
        fill_zero_keys_from(fr, before, (int)((w[r] >> 8) & 0xff), items, t0 + nz, n, cap, res);
      }
      return;
    }
  }
}

// The same runs for at most M <= 64 packs, all in registers and cross-lane
// moves (DPP within rows of 16, ds_bpermute across them).
// The m real packs sit sorted in lanes 0..m-1 (open packs first, then full
// ones) and lanes m..63 hold absent-pack sentinels above them.  Lane s of a
// run takes item j+s exactly while its own word is below the updated word of
// every earlier lane (that is, s < q_t for every t < s), so the run is found
// from the exclusive prefix minimum of the updated words; then the run's
// updated words and the other packs' words are put back in order by a
// bitonic sorting network over the first M lanes (6, 10, 15 or 21 stages for
// 8, 16, 32 or 64).  The next run's keys are fetched (ds_bpermute) while the
// network runs.
constexpr int kFewMinPacks = 4;        // fewer packs: runs are at most that long, the sequential form is faster

// partner of each lane in a sorting-network stage: lane ^ kX within rows of 16
template <int kX>
__device__ __forceinline__ int xlane(int x) {
  if constexpr (kX == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);        // quad_perm 1,0,3,2
  if constexpr (kX == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);        // quad_perm 2,3,0,1
  if constexpr (kX == 3) return __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, false);        // quad_perm 3,2,1,0
  if constexpr (kX == 7) return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);       // row_half_mirror
  if constexpr (kX == 15) return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);      // row_mirror
  if constexpr (kX == 4) {     // banks 0, 2 take lane + 4 (row_shl:4), banks 1, 3 lane - 4 (row_shr:4)
    const int t = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0x5, false);
    return __builtin_amdgcn_update_dpp(t, x, 0x114, 0xF, 0xA, false);
  }
  return x;
}
// lane ^ kX over the whole wave: within rows by DPP (row_ror:8 for 8), across
// rows by ds_bpermute
template <int kX>
__device__ __forceinline__ int xlane64(int x) {
  if constexpr (kX == 8) return __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);   // row_ror:8
  else if constexpr (kX >= 16) return __shfl(x, lane_id() ^ kX);
  else return xlane<kX>(x);
}
// one compare-exchange stage: the lane whose `kLow` bit is clear keeps the
// smaller word of the pair (all words distinct)
template <int kX, int kLow>
__device__ __forceinline__ u64 cx_stage(u64 x) {
  const int lo = xlane64<kX>((int)(uint32_t)x);
  const int hi = xlane64<kX>((int)(uint32_t)(x >> 32));
  const u64 px = ((u64)(uint32_t)hi << 32) | (uint32_t)lo;
  const bool lower = (lane_id() & kLow) == 0;
  return (lower == (px < x)) ? px : x;
}
// ascending sort of the words in each block of M lanes (M = 8, 16, 32, 64):
// merges of 2, 4, ..., M lanes, each a mirror stage and then half-cleaners
template <int M>
__device__ __forceinline__ u64 sort_lanes(u64 x) {
  x = cx_stage<1, 1>(x);
  x = cx_stage<3, 2>(x);
  x = cx_stage<1, 1>(x);
  x = cx_stage<7, 4>(x);
  x = cx_stage<2, 2>(x);
  x = cx_stage<1, 1>(x);
  if constexpr (M >= 16) {
    x = cx_stage<15, 8>(x);
    x = cx_stage<4, 4>(x);
    x = cx_stage<2, 2>(x);
    x = cx_stage<1, 1>(x);
  }
  if constexpr (M >= 32) {
    x = cx_stage<31, 16>(x);
    x = cx_stage<8, 8>(x);
    x = cx_stage<4, 4>(x);
    x = cx_stage<2, 2>(x);
    x = cx_stage<1, 1>(x);
  }
  if constexpr (M == 64) {
    x = cx_stage<63, 32>(x);
    x = cx_stage<16, 16>(x);
    x = cx_stage<8, 8>(x);
    x = cx_stage<4, 4>(x);
    x = cx_stage<2, 2>(x);
    x = cx_stage<1, 1>(x);
  }
  return x;
}

// One run of pack_words_few: lane s (s < M) offers item j + s (key k) to the
// s-th lightest pack; the run is the longest prefix of lanes, all below nz,
// for which that pack is lighter than every pack the run already updated.
// Places the run's items and returns their number; us: the updated words.
template <int M>
__device__ __forceinline__ int pack_run(u64 w, u64 k, int j, int nz, int cap, int32_t* res, u64& us) {
  constexpr u64 kSent = 0xFFFFFFFFFFFF0000ull;
  const int lane = lane_id();
  const bool real = w < kSent;
  us = w + k;
  if ((int)(us & 0xff) == cap) us = kSent | (us & 0xff00ull) | 0xffull;
  u64 pmin = us;                                 // prefix minimum of us within the first M lanes
  if constexpr (M <= 16) {
    pmin = min(pmin, dpp64<0x111>(~0ull, pmin));
    pmin = min(pmin, dpp64<0x112>(~0ull, pmin));
    pmin = min(pmin, dpp64<0x114>(~0ull, pmin));
    if constexpr (M == 16) pmin = min(pmin, dpp64<0x118>(~0ull, pmin));
  } else {
    pmin = wave_scan_incl<u64>(pmin, ~0ull, [](u64 a, u64 b) { return a < b ? a : b; });
  }
  const u64 before = shr1_or64(~0ull, pmin);    // over the lanes before this one
  const u64 vm = __builtin_amdgcn_ballot_w64(lane < M && j + lane < nz && real && w < before);
  const int mb = ~vm == 0 ? 64 : __builtin_ctzll(~vm);   // lane 0 is always valid; all 64 only when m = 64
  if (lane < mb) res[j + lane] = (int)((w >> 8) & 0xff) * cap + (int)(w & 0xff);
  return mb;
}

template <int M, class KeyOf>
__device__ void pack_words_few(KeyOf key_of, int n, int m, int cap, int32_t* res) {
  constexpr u64 kSent = 0xFFFFFFFFFFFF0000ull;
  const int lane = lane_id();
  u64 w = lane < m ? ((u64)lane << 8) : (kSent | ((u64)lane << 8) | 0xffull);
  if constexpr (M >= 32) {
    // Runs may start at any item: after each run the lanes read the keys of
    // the next 64 items (the read hides behind the network of 32 or 64
    // lanes).  The items of load 0 (key 1) come last; nz is the first of them
    // among the keys seen so far (successive views cover every item).
    u64 k = lane < n ? key_of(lane) : 1ull;
    int nz = n;
    {
      const u64 zm = __builtin_amdgcn_ballot_w64(lane < n && k == 1ull);
      if (zm != 0) nz = __builtin_ctzll(zm);
    }
    for (int j = 0; j < nz; ) {
      u64 us;
      const int mb = pack_run<M>(w, k, j, nz, cap, res, us);
      j += mb;
      k = j + lane < n ? key_of(j + lane) : 1ull;
      const u64 zm = __builtin_amdgcn_ballot_w64(j + lane < n && k == 1ull);
      if (zm != 0) nz = min(nz, j + (int)__builtin_ctzll(zm));
      w = sort_lanes<M>(lane < mb ? us : w);
    }
    if (nz < n) {                                // the rest has load 0
      const int items = (int)(w & 0xff);
      fill_zero_keys(lane < M && w < kSent ? cap - items : 0, (int)((w >> 8) & 0xff), items, nz, n, cap, res);
    }
  } else {
    // Short networks: the keys of 64 items at a time sit in registers and a
    // run's keys come from them by a lane shuffle (runs end at the chunk).
    for (int t0 = 0; t0 < n; t0 += 64) {
      const int tn = n - t0 < 64 ? n - t0 : 64;
      const u64 kk = lane < tn ? key_of(t0 + lane) : 0ull;
      const int nz = __popcll(__builtin_amdgcn_ballot_w64(lane < tn && kk != 1ull));   // items of load > 0 first
      u64 k = kk;                                // lane s: key of item j + s
      for (int j = 0; j < nz; ) {
        u64 us;
        const int mb = pack_run<M>(w, k, j, nz, cap, res + t0, us);
        j += mb;
        k = shfl64(kk, (j + lane) & 63);
        w = sort_lanes<M>(lane < mb ? us : w);
      }
      if (nz < tn) {                             // the rest has load 0
        const int items = (int)(w & 0xff);
        fill_zero_keys(lane < M && w < kSent ? cap - items : 0, (int)((w >> 8) & 0xff), items, t0 + nz, n, cap,
                       res);
        return;
      }
    }
  }
}

// pack_words_few on 32-bit words, sum << 8 | pack << 4 | items, for 4 to 16
// packs of at most 14 items and sums below 2^24 - 1 (a full or absent pack is
// kSent32 with its pack bits and items 0xF): one DPP move, one compare and
// one select per network stage instead of two of each.  key_of(t) = key << 8
// | 1.
template <int kX, int kLow>
__device__ __forceinline__ uint32_t cx_stage32(uint32_t x) {
  const uint32_t px = (uint32_t)xlane<kX>((int)x);
  const bool lower = (lane_id() & kLow) == 0;
  return (lower == (px < x)) ? px : x;
}
template <int M>
__device__ __forceinline__ uint32_t sort_lanes32(uint32_t x) {
  x = cx_stage32<1, 1>(x);
  x = cx_stage32<3, 2>(x);
  x = cx_stage32<1, 1>(x);
  x = cx_stage32<7, 4>(x);
  x = cx_stage32<2, 2>(x);
  x = cx_stage32<1, 1>(x);
  if constexpr (M == 16) {
    x = cx_stage32<15, 8>(x);
    x = cx_stage32<4, 4>(x);
    x = cx_stage32<2, 2>(x);
    x = cx_stage32<1, 1>(x);
  }
  return x;
}
template <int M, class KeyOf>
__device__ void pack_words_few32(KeyOf key_of, int n, int m, int cap, int32_t* res) {
  constexpr uint32_t kSent32 = 0xFFFFFF00u;
  const int lane = lane_id();
  uint32_t w = lane < m ? ((uint32_t)lane << 4) : (kSent32 | ((uint32_t)(lane & 15) << 4) | 0xFu);
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int tn = n - t0 < 64 ? n - t0 : 64;
    const uint32_t kk = lane < tn ? key_of(t0 + lane) : 0u;
    const int nz = __popcll(__builtin_amdgcn_ballot_w64(lane < tn && kk != 1u));   // items of load > 0 first
    uint32_t k = kk;                               // lane s: key of item j + s
    for (int j = 0; j < nz; ) {
      const bool real = w < kSent32;
      uint32_t us = w + k;
      if ((int)(us & 0xF) == cap) us = kSent32 | (us & 0xF0u) | 0xFu;
      uint32_t pmin = us;                          // prefix minimum of us within the first M lanes
      pmin = min(pmin, (uint32_t)dpp<0x111>(-1, (int)pmin));
      pmin = min(pmin, (uint32_t)dpp<0x112>(-1, (int)pmin));
      pmin = min(pmin, (uint32_t)dpp<0x114>(-1, (int)pmin));
      if constexpr (M == 16) pmin = min(pmin, (uint32_t)dpp<0x118>(-1, (int)pmin));
      const uint32_t before = (uint32_t)shr1_or(-1, (int)pmin);   // over the lanes before this one
      const u64 vm = __builtin_amdgcn_ballot_w64(lane < M && j + lane < nz && real && w < before);
      const int mb = __builtin_ctzll(~vm);         // lane 0 is always valid, lane M never
      if (lane < mb) res[t0 + j + lane] = (int)((w >> 4) & 0xF) * cap + (int)(w & 0xF);
      j += mb;
      k = (uint32_t)__shfl((int)kk, (j + lane) & 63);
      w = sort_lanes32<M>(lane < mb ? us : w);
    }
    if (nz < tn) {                                 // the rest has load 0
      const int items = (int)(w & 0xF);
      fill_zero_keys(lane < M && w < kSent32 ? cap - items : 0, (int)((w >> 4) & 0xF), items, t0 + nz, n, cap, res);
      return;
    }
  }
}

// The same packing with each pack in ONE 64-bit word, sum << 16 | pack << 8 |
// items, for sums below 2^48 - 1, at most 256 packs and at most 255 items per
// pack.  Words of different packs differ in the pack bits, so one unsigned
// compare orders packs by (sum, index), and one add of a pre-shifted key
// (key_of(t) = key << 16 | 1) both adds an item and counts it.  From 4 packs
// on, runs of items are placed at once (pack_words_few, pack_words_wide);
// below that, one item per step, a full pack being all ones.  A lone
// wavefront's step costs about its dependent-instruction count in issue
// slots; this form has about half the instructions of the general one.
// res[t] = pack * cap + arrival position; scr: the wave's LDS scratch for
// pack_words_wide.
template <int K, class KeyOf>
__device__ void pack_words(KeyOf key_of, int n, int m, int cap, int32_t* res, u64* scr) {
  if constexpr (K > 1 && K <= 4) {
    pack_words_wide<K>(key_of, n, m, cap, res, scr);
    return;
  }
  if constexpr (K == 1) {
    if (m >= kFewMinPacks) {
      if (m > 32) pack_words_few<64>(key_of, n, m, cap, res);
      else if (m > 16) pack_words_few<32>(key_of, n, m, cap, res);
      else if (m > 8) pack_words_few<16>(key_of, n, m, cap, res);
      else pack_words_few<8>(key_of, n, m, cap, res);
      return;
    }
  }
  const int lane = lane_id();
  u64 w[K];
#pragma unroll
  for (int r = 0; r < K; ++r) {
    const int pos = r * 64 + lane;
    w[r] = pos < m ? ((u64)pos << 8) : ~0ull;
  }
  u64 w0 = 0;                                  // pack 0, empty
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int tn = n - t0 < 64 ? n - t0 : 64;
    const u64 kk = lane < tn ? key_of(t0 + lane) : 0ull;
    int rec = 0;
    for (int j = 0; j < tn; ++j) {
      const u64 w1 = rdl64(w[0], 1);           // position 1 before this step's update
      rec = push_record(rec, (int)((w0 >> 8) & 0xff) * cap + (int)(w0 & 0xff));
      u64 nw = w0 + rdl64(kk, j);
      if ((int)(nw & 0xff) == cap) nw = ~0ull;
      int q = __popcll(__builtin_amdgcn_ballot_w64(w[0] < nw) & ~1ull);
#pragma unroll
      for (int r = 1; r < K; ++r) {
        if (q < 64 * r - 1) break;             // sorted: later registers hold nothing below nw
        q += __popcll(__builtin_amdgcn_ballot_w64(w[r] < nw));
      }
      if (K == 1 || q < 64) {
        const u64 d = shl1_64(w[0]);
        w[0] = lane < q ? d : (lane == q ? nw : w[0]);
      } else {
        u64 wd[K];
        shift_down64<K>(w, wd);
#pragma unroll
        for (int r = 0; r < K; ++r) {
          const int pos = r * 64 + lane;
          w[r] = pos < q ? wd[r] : (pos == q ? nw : w[r]);
        }
      }
      w0 = q > 0 ? w1 : nw;
    }
    if (lane < tn) res[t0 + tn - 1 - lane] = rec;
  }
}

// ---------------------------------------------------------------- replication
// The node's experts sorted by (load desc, index asc), all counts 1, are in
// (u, ci) (ci = count << 16 | local index); positions >= En hold the
// sentinel (0, 1 << 16 | 0xffff), which never moves ahead of an expert.
// Rn times: the expert at position 0 (highest load per replica, lowest index
// on ties) gets a replica and moves to its new place.  As in pack_sorted,
// position 0 is also kept in scalar registers and the next one is chosen
// from position 1 read before the update.
// One compare orders two experts: u_a / c_a before u_b / c_b (index a < b on
// ties) exactly when (u_a << 9) * c_b + (511 - a) > (u_b << 9) * c_a + (511 - b)
// (loads <= 2^40, counts < 2^14, indices < 512: below 2^63), so the chain
// keeps u << 9 and count << 16 | (511 - index) (0 for sentinels).
// rep[r] = local index | rank << 16 of the r-th replica created.
template <int K>
__device__ void replicate_sorted(u64 (&u)[K], int (&ci)[K], int Rn, int32_t* rep) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < K; ++r) {
    const int i = ci[r] & 0xffff;
    ci[r] = (ci[r] & ~0xffff) | (i < 512 ? 511 - i : 0);
    u[r] <<= 9;
  }
  u64 u0 = rdl64(u[0], 0);
  int ci0 = rdl(ci[0], 0);
  for (int r0 = 0; r0 < Rn; r0 += 64) {
    const int tn = Rn - r0 < 64 ? Rn - r0 : 64;
    int rec = 0;
    for (int j = 0; j < tn; ++j) {
      const u64 u1 = rdl64(u[0], 1);
      const int ci1 = rdl(ci[0], 1);
      const int c0 = ci0 >> 16;
      const int t0 = ci0 & 0xffff;
      rec = push_record(rec, (511 - t0) | (c0 << 16));
      const int nc = c0 + 1;
      const int nci = (nc << 16) | t0;
      int q = 0;
#pragma unroll
      for (int r = 0; r < K; ++r) {
        if (r > 0 && q < 64 * r - 1) break;       // sorted: nothing further comes first
        const u64 kp = u[r] * (u64)(uint32_t)nc + (u64)(uint32_t)(ci[r] & 0xffff);
        const u64 kq = u0 * (u64)(uint32_t)(ci[r] >> 16) + (u64)(uint32_t)t0;
        u64 mask = __builtin_amdgcn_ballot_w64(kp > kq);
        if (r == 0) mask &= ~1ull;
        q += __popcll(mask);
      }
      if (K == 1 || q < 64) {                     // only register 0 moves
        const u64 ud = shl1_64(u[0]);
        const int cid = shl1(ci[0]);
        const u64 uin = lane == q ? u0 : u[0];
        const int cin = lane == q ? nci : ci[0];
        u[0] = lane < q ? ud : uin;
        ci[0] = lane < q ? cid : cin;
      } else {
        u64 ud[K];
        int cid[K];
        shift_down64<K>(u, ud);
        shift_down<K>(ci, cid);
#pragma unroll
        for (int r = 0; r < K; ++r) {
          const int pos = r * 64 + lane;
          const bool below = pos < q;
          const bool at = pos == q;
          u[r] = below ? ud[r] : (at ? u0 : u[r]);
          ci[r] = below ? cid[r] : (at ? nci : ci[r]);
        }
      }
      if (q > 0) { u0 = u1; ci0 = ci1; } else { ci0 = nci; }
    }
    if (lane < tn) rep[r0 + tn - 1 - lane] = rec;
  }
#pragma unroll
  for (int r = 0; r < K; ++r) {              // back to count << 16 | index (sentinels: garbage index)
    ci[r] = (ci[r] & ~0xffff) | (511 - (ci[r] & 0xffff));
    u[r] >>= 9;
  }
}

// ---------------------------------------------------------------- replication by selection
// The greedy's replicas taken at once (the D'Hondt form of step 2).  Expert
// e's k-th extra replica is the candidate (e, k) of value u_e / k; the greedy
// hands out candidates in the order value desc, expert index asc, k asc
// (each expert's own candidates come in that order, and every step takes the
// first of the experts' next candidates), so its Rn replicas are the first Rn
// candidates in that order, and its creation order is theirs.  On one
// register of experts (lanes sorted by load desc, index asc, count 1 each;
// lanes without an expert hold load 0 and index 0xffff) and Rn <= 64:
//  1. the replica count x0 of the expert in lane 0 (the first in the order):
//     the largest k <= Rn whose candidate (0, k) has fewer than Rn
//     candidates ahead of it.  Lane e has floor((u_e k - t_e) / u_0) of its
//     own ahead of (0, k), t_e = 0 when its index is below lane 0's (it wins
//     ties) else 1, computed with a double reciprocal and an exact integer
//     correction; a binary search over k;
//  2. every candidate ahead of (0, x0) is taken and none behind (0, x0 + 1);
//     a lane has at most one between the two (its k there lie in an
//     interval of length u_e / u_0 <= 1), and the first Rn - rank(0, x0) - 1
//     of those are taken, ranked by counting over the lanes that have one;
//  3. the taken candidates, one per lane, go through a 64-lane sorting
//     network for the creation order (rep[r] = index | k << 16, as the
//     sequential chain records them);
//  4. the experts go through the same network for their final order (load
//     per replica desc, index asc), carrying their source lane, from which
//     load and count are fetched.
// The networks order exact integer keys: for c <= 65 and u <= 2^40,
// floor(u * 8192 / c) is strictly monotone in u / c (two distinct values
// differ by at least 1 / (c_a c_b) >= 1 / 4225) and equal for equal values,
// so ((2^53 - floor(u * 8192 / c)) << 9) | index (below 2^63) puts the larger
// u / c first and breaks ties of value to the smaller index, with one 64-bit
// compare per stage.  Each element carries a 32-bit payload along.
constexpr int kSelectMinPicks = 24;    // fewer replicas: the sequential chain is as short

// floor(u * 8192 / c): floor(u / c) by a double reciprocal (within one of it,
// u <= 2^40) and a remainder check, then the fraction's 13 bits the same way
__device__ __forceinline__ u64 ratio_floor(u64 u, uint32_t c) {
  const double rc = 1.0 / (double)c;
  u64 q = (u64)((double)u * rc);
  int64_t r = (int64_t)u - (int64_t)(q * c);
  if (r < 0) {
    q -= 1;
    r += c;
  } else if (r >= (int64_t)c) {
    q += 1;
    r -= c;
  }
  const uint32_t rs = (uint32_t)r << 13;
  uint32_t f = (uint32_t)((double)rs * rc);
  if ((f + 1) * c <= rs) f += 1;
  return (q << 13) | f;
}
__device__ __forceinline__ u64 ratio_key(u64 u, uint32_t c, int index) {
  return (((1ull << 53) - ratio_floor(u, c)) << 9) | (u64)(uint32_t)index;
}
// one compare-exchange stage on (key, payload): the lane whose kLow bit is
// clear keeps the smaller key; a lane moves only on a strict compare, so
// equal keys never duplicate a payload
template <int kX, int kLow>
__device__ __forceinline__ void cx_kv(u64& k, int& v) {
  const int plo = xlane64<kX>((int)(uint32_t)k);
  const int phi = xlane64<kX>((int)(uint32_t)(k >> 32));
  const int pv = xlane64<kX>(v);
  const u64 pk = ((u64)(uint32_t)phi << 32) | (uint32_t)plo;
  const bool lower = (lane_id() & kLow) == 0;
  const bool take = lower ? pk < k : pk > k;
  k = take ? pk : k;
  v = take ? pv : v;
}
// ascending order of the keys over the 64 lanes: merges of 2, 4, ..., 64
// lanes, each a mirror stage and then half-cleaners
__device__ __forceinline__ void sort_kv64(u64& k, int& v) {
  cx_kv<1, 1>(k, v);
  cx_kv<3, 2>(k, v);
  cx_kv<1, 1>(k, v);
  cx_kv<7, 4>(k, v);
  cx_kv<2, 2>(k, v);
  cx_kv<1, 1>(k, v);
  cx_kv<15, 8>(k, v);
  cx_kv<4, 4>(k, v);
  cx_kv<2, 2>(k, v);
  cx_kv<1, 1>(k, v);
  cx_kv<31, 16>(k, v);
  cx_kv<8, 8>(k, v);
  cx_kv<4, 4>(k, v);
  cx_kv<2, 2>(k, v);
  cx_kv<1, 1>(k, v);
  cx_kv<63, 32>(k, v);
  cx_kv<16, 16>(k, v);
  cx_kv<8, 8>(k, v);
  cx_kv<4, 4>(k, v);
  cx_kv<2, 2>(k, v);
  cx_kv<1, 1>(k, v);
}

// (u, ci) as replicate_sorted<1> takes and leaves them (ci = count << 16 |
// index); rep: Rn ints of LDS, also the scratch of the expansion.
__device__ void replicate_select(u64& u, int& ci, int Rn, int32_t* rep) {
  const int lane = lane_id();
  const int ie = ci & 0xffff;
  const u64 u0 = rdl64(u, 0);
  int x;                                  // replicas taken by this lane's expert
  if (u0 == 0) {
    x = lane == 0 ? Rn : 0;               // all loads zero: the lowest index takes every replica
  } else {
    const int i0 = rdl(ie, 0);
    const bool live = lane != 0 && u != 0;
    const u64 t = ie < i0 ? 0 : 1;
    const double r0 = 1.0 / (double)u0;
    auto ahead = [&](int k) -> int {      // this lane's candidates ahead of (0, k)
      const u64 num = live ? u * (u64)(uint32_t)k - t : 0;
      u64 q = (u64)((double)num * r0);    // num < 2^47: within one of the quotient
      if (q * u0 > num) q -= 1;
      else if ((q + 1) * u0 <= num) q += 1;
      return (int)q;
    };
    int lo = 1;
    int hi = Rn;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mid - 1 + rdl(wave_incl_sum(ahead(mid)), 63) < Rn) lo = mid;
      else hi = mid - 1;
    }
    const int a = ahead(lo);
    const int b = ahead(lo + 1);
    const int need = Rn - (lo - 1 + rdl(wave_incl_sum(a), 63)) - 1;
    const bool cand = b > a;
    const u64 cmask = ballot(cand);
    x = lane == 0 ? lo : a;
    if (need > 0) {
      if (need == __popcll(cmask)) {
        x += cand ? 1 : 0;
      } else {
        int r = 0;                        // candidates ahead of this lane's
        for (u64 m = cmask; m != 0; m &= m - 1) {
          const int f = __builtin_ctzll(m);
          const u64 uf = rdl64(u, f);
          const u64 bf = (u64)(uint32_t)rdl(b, f);
          const int jf = rdl(ie, f);
          const u64 l = uf * (u64)(uint32_t)b;
          const u64 rr = u * bf;
          r += (l > rr || (l == rr && jf < ie)) ? 1 : 0;
        }
        x += (cand && r < need) ? 1 : 0;
      }
    }
  }
  // one lane per replica: lane s < Rn takes replica k = s - off + 1 of the
  // expert whose range [off, off + x) holds s (a marker at each range start,
  // then a running maximum)
  const int off = wave_incl_sum(x) - x;
  if (lane < Rn) rep[lane] = 0;
  wave_lds_sync();
  if (x > 0) rep[off] = lane + 1;
  wave_lds_sync();
  const int mk = lane < Rn ? rep[lane] : 0;
  const int o = max(wave_incl_max(mk) - 1, 0);
  const u64 uo = shfl64(u, o);
  const int io = __shfl(ie, o);
  const int k = lane - __shfl(off, o) + 1;
  // creation order (the payload is the record); with every load zero, lane
  // 0's replicas k = 1..Rn are in order already (value 0, index, then k)
  u64 pk = lane < Rn ? ratio_key(uo, (uint32_t)k, io) : ~0ull;
  int pv = io | (k << 16);
  if (u0 != 0) sort_kv64(pk, pv);
  if (lane < Rn) rep[lane] = pv;
  // final order of the experts (the payload is the source lane); lanes
  // without an expert sort last
  u64 fk = ie != 0xffff ? ratio_key(u, (uint32_t)(x + 1), ie) : ~0ull;
  int src = lane;
  sort_kv64(fk, src);
  const u64 uf = shfl64(u, src);
  const int cf = __shfl(x + 1, src);
  const int jf = __shfl(ie, src);
  u = uf;
  ci = (cf << 16) | jf;
}

// ---------------------------------------------------------------- LDS carving

struct Smem {
  u128* kexp;      // [E]   step-3 key per mlog expert
  u64* w;          // [E]   loads, logical order
  u64* wl;         // [E]   loads, mlog order (node n: [n*En, n*En+En))
  u64* gsum;       // [Gp]
  int32_t* m2l;    // [E]
  int32_t* cnt;    // [E]   replica count per mlog expert
  int32_t* srt;    // [E]   per node: local expert index at each sorted position
  int32_t* gnode;  // [Gp]
  int32_t* gslot;  // [Gp]
  int32_t* gord;   // [Gp]  groups, heaviest first
  int32_t* gres;   // [Gp]  packing result per visiting rank
  int32_t* rep;    // [Np][Rn]
  u64* pk;         // [nscr][pk_words]  per wave: lane-parallel packing scratch
  int32_t* posaux; // [nscr][3 * En]  per wave: class start (and class size), item offset, position of expert
  int32_t* ordr;   // [nscr][Pn]  per wave: item (local expert | rank << 16) in visiting order
  int32_t* ores;   // [nscr][Pn]  per wave: packing result per visiting rank
  int32_t* rcls;   // [nscr][Rn]  per wave: class of each replica
  int32_t* nflag;  // [Np]  step-3 key form: 3 one 32-bit word per pack, 2 one 64-bit word, 1 64-bit sums, 0 128-bit sums
  int32_t* flags;  // [4]  [0]: problem status; [2..3]: the total load (u64, 8-byte aligned)
};

__device__ Smem carve(unsigned char* base, const RbPlan& p) {
  Smem s;
  s.kexp = (u128*)(base + p.o_kexp);
  s.w = (u64*)(base + p.o_w);
  s.wl = (u64*)(base + p.o_wl);
  s.gsum = (u64*)(base + p.o_gsum);
  s.m2l = (int32_t*)(base + p.o_m2l);
  s.cnt = (int32_t*)(base + p.o_cnt);
  s.srt = (int32_t*)(base + p.o_srt);
  s.gnode = (int32_t*)(base + p.o_gnode);
  s.gslot = (int32_t*)(base + p.o_gslot);
  s.gord = (int32_t*)(base + p.o_gord);
  s.gres = (int32_t*)(base + p.o_gres);
  s.rep = (int32_t*)(base + p.o_rep);
  s.pk = (u64*)(base + p.o_pk);
  s.posaux = (int32_t*)(base + p.o_posaux);
  s.ordr = (int32_t*)(base + p.o_ordr);
  s.ores = (int32_t*)(base + p.o_ores);
  s.rcls = (int32_t*)(base + p.o_rcls);
  s.nflag = (int32_t*)(base + p.o_nflag);
  s.flags = (int32_t*)(base + p.o_flags);
  return s;
}

// dst[0, n) = -1 by the workgroup: 16-byte stores between a 4-byte head and tail
__device__ void fill_minus_one(int32_t* dst, int64_t n, int tid, int nt) {
  const int64_t head0 = (int64_t)(((16u - ((uint32_t)(uintptr_t)dst & 15u)) & 15u) >> 2);
  const int64_t head = head0 < n ? head0 : n;
  if (tid < head) dst[tid] = -1;
  int4* v = (int4*)(dst + head);
  const int64_t nv = (n - head) >> 2;
  for (int64_t i = tid; i < nv; i += nt) v[i] = make_int4(-1, -1, -1, -1);
  for (int64_t i = head + nv * 4 + tid; i < n; i += nt) dst[i] = -1;
}

__device__ void write_failed(const RbPlan& p, int64_t b, int32_t code, int32_t* phy2log,
                             int32_t* log2phy, int32_t* logcnt, int32_t* status) {
  for (int i = threadIdx.x; i < p.P; i += blockDim.x) phy2log[b * p.P + i] = -1;
  for (int i = threadIdx.x; i < p.E * p.X; i += blockDim.x) log2phy[b * p.E * (int64_t)p.X + i] = -1;
  for (int i = threadIdx.x; i < p.E; i += blockDim.x) logcnt[b * p.E + i] = -1;
  if (threadIdx.x == 0) status[b] = code;
}

// ---------------------------------------------------------------- per-node phases

// After replication on the first 64 positions only (the window): the final
// order of all En > 64 experts of node n into s.srt.  Only the top Rn <= 64
// experts can take a replica (the expert at position p is preceded by the
// originals of the p experts before it, so its k-th replica ranks at least
// p + k - 1 among the picks), so the picks on the window are those on all
// positions and the other experts keep count 1 and their order.  The two
// sorted runs are merged: window expert l (lane l) finds by binary search
// how many tail experts precede it, cnt_l; tail expert j is preceded by the
// window experts with cnt_l <= j (a histogram of the cnt_l and its prefix
// sums).  Scratch: the node's part of the step-3 key array (not yet used).
template <int K>
__device__ void merge_window(const RbPlan& p, const Smem& s, int n, const u64 (&u)[K], const int (&ci)[K]) {
  const int lane = lane_id();
  const int En = p.En;
  const int T = En - 64;                             // tail experts
  u64* tk = reinterpret_cast<u64*>(s.kexp + n * En); // [T] tail keys u << 9 | (511 - index)
  int* hs = reinterpret_cast<int*>(tk + T);          // [T + 1] histogram, then its prefix sums
#pragma unroll
  for (int r = 1; r < K; ++r) {
    const int pos = r * 64 + lane;
    if (pos < En) tk[pos - 64] = (u[r] << 9) | (u64)(511 - (ci[r] & 0xffff));
  }
  for (int x = lane; x <= T; x += 64) hs[x] = 0;
  wave_lds_sync();
  // window expert: tail experts before it (a prefix of the tail)
  const u64 cl = (u64)(uint32_t)(ci[0] >> 16);
  const u64 rhs = (u[0] << 9) + (u64)(511 - (ci[0] & 0xffff));
  int lo = 0;
  int step = 1;
  while (step * 2 <= T) step *= 2;
  for (; step > 0; step >>= 1) {
    if (lo + step <= T) {
      const u64 t = tk[lo + step - 1];
      if ((t & ~(u64)511) * cl + (t & 511) > rhs) lo += step;
    }
  }
  atomicAdd(&hs[lo], 1);
  wave_lds_sync();
  int carry = 0;
  for (int x0 = 0; x0 <= T; x0 += 64) {
    const int x = x0 + lane;
    const int v = x <= T ? hs[x] : 0;
    const int incl = wave_incl_sum(v) + carry;
    carry = rdl(incl, 63);
    if (x <= T) hs[x] = incl;                       // window experts with cnt_l <= x
  }
  wave_lds_sync();
  int32_t* srt = s.srt + n * En;
  srt[lane + lo] = ci[0] & 0xffff;
#pragma unroll
  for (int r = 1; r < K; ++r) {
    const int pos = r * 64 + lane;
    if (pos < En) srt[(pos - 64) + hs[pos - 64]] = ci[r] & 0xffff;
  }
  wave_lds_sync();
}

// Step 2 and the denominators of node n (one wave): the node's experts in
// load order go through replication; counts, the final order and the exact
// step-3 keys are stored.
template <int K>
__device__ void node_replicate(const RbPlan& p, const Smem& s, int n) {
  const int lane = lane_id();
  const int En = p.En;
  // the node's experts by (load desc, local index asc): up to 64 sorted here
  // in one register, as ~(key + 1) ascending for the unique keys
  // load << 9 | (511 - local index) (loads <= 2^40, local indices < 512;
  // lanes past En: all ones); larger nodes ranked by the workgroup into srt
  u64 u[K];
  int ci[K];
  if constexpr (K == 1) {
    const u64 v = lane < En ? ~(((s.wl[n * En + lane] << 9) | (u64)(511 - lane)) + 1) : ~0ull;
    const u64 key = ~sort_lanes<64>(v) - 1;
    u[0] = lane < En ? key >> 9 : 0;
    ci[0] = (1 << 16) | (lane < En ? 511 - (int)(key & 511) : 0xffff);
  } else {
#pragma unroll
    for (int r = 0; r < K; ++r) {
      const int pos = r * 64 + lane;
      if (pos < En) {
        const int i = s.srt[n * En + pos];
        u[r] = s.wl[n * En + i];
        ci[r] = (1 << 16) | i;
      } else {
        u[r] = 0;
        ci[r] = (1 << 16) | 0xffff;
      }
    }
  }
  bool window = false;
  if constexpr (K > 1) window = p.Rn <= 64;          // En > 64 here
  if (K == 1 || window) {
    u64 uw[1] = {u[0]};
    int cw[1] = {ci[0]};
    if (p.Rn >= kSelectMinPicks && p.Rn <= 64) replicate_select(uw[0], cw[0], p.Rn, s.rep + n * p.Rn);
    else replicate_sorted<1>(uw, cw, p.Rn, s.rep + n * p.Rn);
    u[0] = uw[0];
    ci[0] = cw[0];
    if (window) merge_window<K>(p, s, n, u, ci);
  } else {
    replicate_sorted<K>(u, ci, p.Rn, s.rep + n * p.Rn);
  }

  u64 sum = 0;
  int cmax = 1;
#pragma unroll
  for (int r = 0; r < K; ++r) {
    const int pos = r * 64 + lane;
    if (pos < En) {
      const int i = ci[r] & 0xffff;
      const int c = ci[r] >> 16;
      s.cnt[n * En + i] = c;
      if (!window) s.srt[n * En + pos] = i;
      sum += u[r];
      cmax = max(cmax, c);
    }
  }
  sum = wave_sum64(sum);
  cmax = wave_max(cmax);

  // D = product of p over the prime powers p^k <= cmax dividing some count
  // (= lcm of the counts); Q = D / c by exact division.
  u128 D = 1;
  bool ovf = false;
  if (cmax <= 64) {
    u64 present = 0;                           // bit c - 1 for each count c on the node
#pragma unroll
    for (int r = 0; r < K; ++r) {
      const int pos = r * 64 + lane;
      if (pos < En) present |= 1ull << ((ci[r] >> 16) - 1);
    }
    present = wave_or64(present);
    constexpr SmallPrimePowers t = make_small_prime_powers();
#pragma unroll
    for (int i = 0; i < t.n; ++i) {
      if ((int)t.q[i] > cmax) break;
      if ((present & t.mult[i]) != 0) D *= t.p[i];   // lcm(1..64) < 2^93: no overflow
    }
  } else if (cmax <= 128) {
    // the counts up to 64 as above, then the lcm with each distinct count
    // above 64 (at most Pn / 65 of them) by Euclid on c and D mod c
    u64 present = 0, high = 0;
#pragma unroll
    for (int r = 0; r < K; ++r) {
      const int pos = r * 64 + lane;
      const int c = ci[r] >> 16;
      if (pos < En && c <= 64) present |= 1ull << (c - 1);
      if (pos < En && c > 64) high |= 1ull << (c - 65);
    }
    present = wave_or64(present);
    high = wave_or64(high);
    constexpr SmallPrimePowers t = make_small_prime_powers();
#pragma unroll
    for (int i = 0; i < t.n; ++i)
      if ((present & t.mult[i]) != 0) D *= t.p[i];
    for (u64 m = high; m != 0; m &= m - 1) {
      const uint32_t c = 65 + (uint32_t)__builtin_ctzll(m);
      const int dg = (uint32_t)(D >> 96) != 0 ? 4 : (uint32_t)(D >> 64) != 0 ? 3 : (uint32_t)(D >> 32) != 0 ? 2 : 1;
      uint32_t a = c;
      uint32_t b = (uint32_t)(D - div_by_count(D, dg, c) * c);   // D mod c
      while (b != 0) {
        const uint32_t t2 = a % b;
        a = b;
        b = t2;
      }
      D = mul_u128_u64(D, c / a, ovf);
    }
  } else {
    for (int t = 0; t < kPrimePowers.count && (int)kPrimePowers.q[t] <= cmax; ++t) {
      const uint32_t q = kPrimePowers.q[t];
      const FastDiv fd{kPrimePowers.mul[t], kPrimePowers.shift[t]};
      u64 any = 0;
#pragma unroll
      for (int r = 0; r < K; ++r) {
        const int pos = r * 64 + lane;
        const uint32_t c = (uint32_t)(ci[r] >> 16);
        any |= ballot(pos < En && fastdiv_apply(c, fd) * q == c);
      }
      if (any != 0) D = mul_u128_u64(D, kPrimePowers.p[t], ovf);
    }
  }
  const int digits = (uint32_t)(D >> 96) != 0 ? 4 : (uint32_t)(D >> 64) != 0 ? 3 : (uint32_t)(D >> 32) != 0 ? 2 : 1;
  u128 Q[K];
#pragma unroll
  for (int r = 0; r < K; ++r) {
    const uint32_t c = (uint32_t)(ci[r] >> 16) > 0 ? (uint32_t)(ci[r] >> 16) : 1u;
    Q[r] = div_by_count(D, digits, c);
  }
  const u128 total = mul_u128_u64(D, sum, ovf);
  if (lane == 0) {
    if (ovf || (total >> 127) != 0) s.flags[0] = EPLB_S_OVERFLOW;
    // key width for step 3: one 32-bit word per pack, one 64-bit word, 64-bit sums, or 128-bit sums
    const bool w32 = total < (u128)((1u << 24) - 1) && p.RKn >= kFewMinPacks && p.RKn <= 16 && p.ppr <= 14;
    s.nflag[n] = w32 ? 3 : total < (((u128)1 << 48) - 1) && p.RKn <= 256 && p.ppr <= 255 ? 2
                                                                                        : ((u64)(total >> 64) == 0 ? 1 : 0);
  }
#pragma unroll
  for (int r = 0; r < K; ++r) {
    const int pos = r * 64 + lane;
    if (pos < En) {
      bool o2 = false;                 // u * D / c <= D * sum < 2^127 once checked
      s.kexp[n * En + (ci[r] & 0xffff)] = mul_u128_u64(Q[r], u[r], o2);
    }
  }
}

// Step 3 of node n (one wave, scratch slot ws): the visiting order of the
// node's physical experts, packing onto its GPUs, and the outputs.
template <int K, int KP>
__device__ void node_place(const RbPlan& p, const Smem& s, int n, int ws,
                           int32_t* o_phy, int32_t* o_l2p, int32_t* o_cnt) {
  const int lane = lane_id();
  const int En = p.En, Pn = p.Pn, Rn = p.Rn;
  const int32_t* rep = s.rep + n * Rn;
  const int32_t* m2l = s.m2l + n * En;

  if (p.ppr == 1) {
    // One physical expert per GPU: item j sits on GPU j (identity).
    for (int j = lane; j < Pn; j += 64) {
      int li, rk;
      if (j < En) { li = j; rk = 0; }
      else { const int v = rep[j - En]; li = v & 0xffff; rk = v >> 16; }
      const int e = m2l[li];
      const int pid = n * Pn + j;
      o_phy[pid] = e;
      o_l2p[(int64_t)e * p.X + rk] = pid;
    }
  } else {
    int32_t* ordr = s.ordr + ws * Pn;
    int32_t* ores = s.ores + ws * Pn;
    int32_t* cstart = s.posaux + ws * 3 * En;   // class start of each position (a start: | class size << 16)
    int32_t* coff = cstart + En;                 // item offset of each position
    int32_t* posof = coff + En;                  // position of each local expert
    int32_t* rcls = s.rcls + ws * (Rn > 0 ? Rn : 1);
    const int width = s.nflag[n];

    // positions in the final order: (u, c, local index)
    u64 u[K];
    int c[K], li[K];
#pragma unroll
    for (int r = 0; r < K; ++r) {
      const int pos = r * 64 + lane;
      if (pos < En) {
        li[r] = s.srt[n * En + pos];
        u[r] = s.wl[n * En + li[r]];
        c[r] = s.cnt[n * En + li[r]];
      } else {
        li[r] = 0; u[r] = 0; c[r] = 0;
      }
    }
    // A class is a run of positions with equal load per replica.  Its items
    // in visiting order: the originals (ascending local index, which is
    // ascending position), then the replicas of its experts in creation order.
    int carry_off = 0, carry_start = 0;
    int stv[K];                                      // class start of each position
    u64 tiem[K];                                     // positions that tie with the one before
#pragma unroll
    for (int r = 0; r < K; ++r) {
      const int pos = r * 64 + lane;
      u64 pu = shr1_or64(0ull, u[r]);                // the previous position (DPP)
      int pc = shr1_or(0, c[r]);
      if (r > 0) {
        const u64 lu = rdl64(u[r - 1], 63);
        const int lc = rdl(c[r - 1], 63);
        if (lane == 0) { pu = lu; pc = lc; }
      }
      const bool tie = pos > 0 && pos < En && u[r] * (u64)(uint32_t)pc == pu * (u64)(uint32_t)c[r];
      tiem[r] = ballot(tie);
      const int st = max(wave_incl_max((pos < En && !tie) ? pos : -1), carry_start);
      const int incl = wave_incl_sum(pos < En ? c[r] : 0) + carry_off;
      if (pos < En) {
        cstart[pos] = st;
        coff[pos] = incl - c[r];
        posof[li[r]] = pos;
      }
      stv[r] = st;
      carry_off = rdl(incl, 63);
      carry_start = rdl(st, 63);
    }
    // the last position of each class (the next one does not tie) puts the
    // class size in the high half of its start's entry, after every start
    // above is written; readers mask the low half
#pragma unroll
    for (int r = 0; r < K; ++r) {
      const int pos = r * 64 + lane;
      const u64 next_ties = (tiem[r] >> 1) | (r + 1 < K ? (tiem[r + 1 < K ? r + 1 : r] & 1ull) << 63 : 0ull);
      if (pos < En && ((next_ties >> lane) & 1ull) == 0) cstart[stv[r]] = stv[r] | ((pos - stv[r] + 1) << 16);
    }
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < K; ++r) {              // originals
      const int pos = r * 64 + lane;
      if (pos < En) ordr[coff[stv[r]] + (pos - stv[r])] = li[r];
    }
    // Replicas: the rank of a replica among the earlier replicas of its class
    // is the count of equal class numbers before it.  Inside a chunk of 64
    // that count comes from ballots over the class number's bits (the lanes
    // that agree on every bit); earlier chunks, when a node has more than 64
    // replicas, are counted from their class numbers in LDS.
    const int cbits = En > 1 ? 32 - __builtin_clz((unsigned)(En - 1)) : 0;
    if (Rn > 64) {
      for (int rr = lane; rr < Rn; rr += 64) rcls[rr] = cstart[posof[rep[rr] & 0xffff]] & 0xffff;
      wave_lds_sync();
    }
    for (int base = 0; base < Rn; base += 64) {
      const int rr = base + lane;
      const bool act = rr < Rn;
      const int v = act ? rep[rr] : 0;
      const int cls = act ? cstart[posof[v & 0xffff]] & 0xffff : 0;
      u64 same = ballot(act);
      for (int b = 0; b < cbits; ++b) {
        const bool bit = (cls >> b) & 1;
        const u64 mb = ballot(bit);
        same &= bit ? mb : ~mb;
      }
      int before = __popcll(same & ((1ull << lane) - 1));
      for (int r2 = 0; r2 < base; r2 += 8) {
        int a[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = rcls[r2 + k];
#pragma unroll
        for (int k = 0; k < 8; ++k) before += a[k] == cls ? 1 : 0;
      }
      if (act) ordr[coff[cls] + (cstart[cls] >> 16) + before] = v;   // local index | rank << 16
    }
    wave_lds_sync();
    const u128* kexp = s.kexp + n * En;
    if (KP == 1 && width == 3) {
      auto key = [=](int t) { return ((uint32_t)kexp[ordr[t] & 0xffff] << 8) | 1u; };
      if (p.RKn > 8) pack_words_few32<16>(key, Pn, p.RKn, p.ppr, ores);
      else pack_words_few32<8>(key, Pn, p.RKn, p.ppr, ores);
    } else if (width >= 2) {
      auto key = [=](int t) { return ((u64)kexp[ordr[t] & 0xffff] << 16) | 1ull; };
      pack_words<KP>(key, Pn, p.RKn, p.ppr, ores, s.pk + ws * p.pk_words);
    } else if (width == 1) {
      auto key = [=](int t, int) { return (u64)kexp[ordr[t] & 0xffff]; };
      pack_sorted<KP, 1>(key, Pn, p.RKn, p.ppr, ores);
    } else {
      auto key = [=](int t, int w) { const u128 k = kexp[ordr[t] & 0xffff]; return w ? (u64)(k >> 64) : (u64)k; };
      pack_sorted<KP, 2>(key, Pn, p.RKn, p.ppr, ores);
    }
    wave_lds_sync();
    for (int t = lane; t < Pn; t += 64) {
      const int v = ordr[t];
      const int e = m2l[v & 0xffff];
      const int rk = v >> 16;
      const int pid = n * Pn + ores[t];
      o_phy[pid] = e;
      o_l2p[(int64_t)e * p.X + rk] = pid;
    }
  }
  // counts of the node's experts (their log2phy rows beyond the count hold
  // the -1 the kernel wrote first)
  for (int i = lane; i < En; i += 64) o_cnt[m2l[i]] = s.cnt[n * En + i];
}

// ---------------------------------------------------------------- kernel

// kFull: the many-problem form of the smallest shapes, held to 64 VGPRs so
// that eight waves fit per SIMD (at the cost of a few spilled values); with
// at most one workgroup per CU the uncapped form is used.
template <int KR, int KP, bool kFull>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 512), amdgpu_waves_per_eu(kFull && KR * KP <= 2 ? 8 : 1)))
void rebalance_kernel(const int64_t* __restrict__ load, RbPlan p,
                                                         int32_t* __restrict__ phy2log,
                                                         int32_t* __restrict__ log2phy,
                                                         int32_t* __restrict__ logcnt,
                                                         int32_t* __restrict__ status) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Smem s = carve(smem, p);
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int NT = blockDim.x;
  const int wid = tid >> 6;
  const int NW = NT >> 6;
  const int lane = lane_id();

  // ---- loads, range check
  if (tid == 0) {
    s.flags[0] = 0;
    *reinterpret_cast<u64*>(s.flags + 2) = 0;
  }
  __syncthreads();
  const int64_t* row = load + b * p.E;
  for (int e = tid; e < p.E; e += NT) {
    const int64_t v = row[e];
    if (v < 0 || v > kLoadMax) s.flags[0] = EPLB_S_BAD_LOAD;
    s.w[e] = (u64)v;
  }
  __syncthreads();
  if (s.flags[0] != 0) {
    write_failed(p, b, s.flags[0], phy2log, log2phy, logcnt, status);
    return;
  }
  // log2phy starts as all -1, written coalesced after the loads have arrived
  // (stores issued before them would hold up their wait); the placement
  // overwrites each expert's first `count` entries after the barriers below
  fill_minus_one(log2phy + b * (int64_t)p.E * p.X, (int64_t)p.E * p.X, tid, NT);

  // ---- step 1: groups -> nodes
  if (p.gpn == 1) {
    for (int g = tid; g < p.Gp; g += NT) { s.gnode[g] = g; s.gslot[g] = 0; }
  } else {
    u64* total = reinterpret_cast<u64*>(s.flags + 2);
    for (int g = wid; g < p.Gp; g += NW) {
      u64 sum = 0;
      for (int j = lane; j < p.S; j += 64) sum += s.w[g * p.S + j];
      sum = wave_sum64(sum);
      if (lane == 0) {
        s.gsum[g] = sum;
        atomicAdd(reinterpret_cast<unsigned long long*>(total), (unsigned long long)sum);
      }
    }
    __syncthreads();
    // heaviest first, equal loads in ascending group index (rank by counting):
    // by wave 0 itself for up to 64 groups, else by the whole workgroup
    auto rank_groups = [&](int g0, int gstep) {
      for (int g = g0; g < p.Gp; g += gstep) {
        const u64 wg = s.gsum[g];
        int rank = 0;
        int h = 0;
        for (; h + 8 <= p.Gp; h += 8) {            // eight reads in flight
          u64 a[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) a[k] = s.gsum[h + k];
#pragma unroll
          for (int k = 0; k < 8; ++k) rank += (a[k] > wg || (a[k] == wg && h + k < g)) ? 1 : 0;
        }
        for (; h < p.Gp; ++h) {
          const u64 wh = s.gsum[h];
          rank += (wh > wg || (wh == wg && h < g)) ? 1 : 0;
        }
        s.gord[rank] = g;
      }
    };
    if (p.Gp > 64) {
      rank_groups(tid, NT);
      __syncthreads();
    }
    if (wid == 0) {
      if (p.Gp <= 64) {
        rank_groups(lane, 64);
        wave_lds_sync();
      }
      const u64 tot = *total;
      const bool words = tot < (1ull << 48) - 1 && p.Np <= 256 && p.gpn <= 255;
      const u64* gsum = s.gsum;
      const int32_t* gord = s.gord;
      if (tot < (1u << 24) - 1 && p.Np >= kFewMinPacks && p.Np <= 16 && p.gpn <= 14) {
        auto key = [=](int t) { return ((uint32_t)gsum[gord[t]] << 8) | 1u; };
        if (p.Np > 8) pack_words_few32<16>(key, p.Gp, p.Np, p.gpn, s.gres);
        else pack_words_few32<8>(key, p.Gp, p.Np, p.gpn, s.gres);
      } else if (words) {
        auto key = [=](int t) { return (gsum[gord[t]] << 16) | 1ull; };
        if (p.KN == 1) pack_words<1>(key, p.Gp, p.Np, p.gpn, s.gres, s.pk);
        else pack_words<8>(key, p.Gp, p.Np, p.gpn, s.gres, s.pk);
      } else {
        auto key = [=](int t, int) { return gsum[gord[t]]; };
        if (p.KN == 1) pack_sorted<1, 1>(key, p.Gp, p.Np, p.gpn, s.gres);
        else pack_sorted<8, 1>(key, p.Gp, p.Np, p.gpn, s.gres);
      }
      wave_lds_sync();
      for (int t = lane; t < p.Gp; t += 64) {
        const int g = s.gord[t];
        const int v = s.gres[t];
        s.gnode[g] = v / p.gpn;
        s.gslot[g] = v - (v / p.gpn) * p.gpn;
      }
    }
  }
  __syncthreads();

  // ---- mlog order: expert g*S + j of a group at (node, slot) -> node*En + slot*S + j
  for (int e = tid; e < p.E; e += NT) {
    const int g = (int)fastdiv_apply((uint32_t)e, p.fd_S);
    const int j = e - g * p.S;
    const int m = (s.gnode[g] * p.gpn + s.gslot[g]) * p.S + j;
    s.m2l[m] = e;
    s.wl[m] = s.w[e];
  }
  __syncthreads();
  if constexpr (KR > 1) {
    // nodes of more than 64 experts: their experts by (load desc, local index
    // asc) through the unique keys load << 9 | (511 - local index) (loads <=
    // 2^40, local indices < 512), as v = ~(key + 1) ascending.  Each run of
    // 64 of a node's experts is sorted by one wave (into the logical-order
    // loads' place, dead once the mlog order is built); an expert's rank in
    // its node is then its place in its run plus, for every other run, the
    // number of that run's values below its own (binary search).  Smaller
    // nodes are sorted by their own wave in step 2.
    u64* sv = s.w;
    const int runs = (p.En + 63) >> 6;
    for (int c = wid; c < p.Np * runs; c += NW) {
      const int n = c / runs;
      const int j = (c - n * runs) * 64 + lane;
      const u64 v = j < p.En ? ~(((s.wl[n * p.En + j] << 9) | (u64)(511 - j)) + 1) : ~0ull;
      const u64 sorted = sort_lanes<64>(v);
      if (j < p.En) sv[n * p.En + j] = sorted;
    }
    __syncthreads();
    for (int c = wid; c < p.Np * runs; c += NW) {
      const int n = c / runs;
      const int r = c - n * runs;
      const int j = r * 64 + lane;
      if (j < p.En) {
        const u64* sn = sv + n * p.En;
        const u64 v = sn[j];
        int rank = lane;
        for (int o = 0; o < runs; ++o) {
          if (o == r) continue;
          const u64* a = sn + o * 64;
          const int len = min(64, p.En - o * 64);
          int lo = 0;                                // values of run o below v
#pragma unroll
          for (int step = 64; step >= 1; step >>= 1)
            if (lo + step <= len && a[lo + step - 1] < v) lo += step;
          rank += lo;
        }
        s.srt[n * p.En + rank] = 511 - (int)((~v - 1) & 511);
      }
    }
    __syncthreads();
  }

  // ---- step 2 and the denominators, one wave per node
  for (int n = wid; n < p.Np; n += NW) node_replicate<KR>(p, s, n);
  __syncthreads();
  if (s.flags[0] != 0) {
    write_failed(p, b, s.flags[0], phy2log, log2phy, logcnt, status);
    return;
  }

  // ---- step 3 and outputs, one wave per node
  int32_t* o_phy = phy2log + b * p.P;
  int32_t* o_l2p = log2phy + b * (int64_t)p.E * p.X;
  int32_t* o_cnt = logcnt + b * p.E;
  for (int n = wid; n < p.Np; n += NW) node_place<KR, KP>(p, s, n, wid, o_phy, o_l2p, o_cnt);
  if (tid == 0) status[b] = 0;
}

int regs_for(int n) {          // registers per lane to hold n sorted positions
  return n <= 64 ? 1 : n <= 128 ? 2 : n <= 256 ? 4 : 8;
}

typedef void (*RbKernel)(const int64_t*, RbPlan, int32_t*, int32_t*, int32_t*, int32_t*);

template <int KR, bool kFull>
RbKernel pick_kp(int KP) {
  switch (KP) {
    case 1: return rebalance_kernel<KR, 1, kFull>;
    case 2: return rebalance_kernel<KR, 2, kFull>;
    case 4: return rebalance_kernel<KR, 4, kFull>;
    default: return rebalance_kernel<KR, 8, kFull>;
  }
}

template <bool kFull>
RbKernel pick_kr(int KR, int KP) {   // kFull = false only
  switch (KR) {
    case 1: return pick_kp<1, kFull>(KP);
    case 2: return pick_kp<2, kFull>(KP);
    case 4: return pick_kp<4, kFull>(KP);
    default: return pick_kp<8, kFull>(KP);
  }
}

// A rebalance workgroup may take the whole LDS of a gfx950 compute unit (the
// other kernels keep to kMaxLdsBytes).
constexpr int kMaxRebalanceLdsBytes = 160 * 1024;

// Up to one workgroup per CU (256 CUs): the uncapped instantiations.
constexpr int64_t kRbFewProblems = 256;

RbKernel pick_kernel(int KR, int KP, int64_t B) {
  if (B > kRbFewProblems && KR * KP <= 2)           // the only shapes the cap changes
    return KR == 2 ? rebalance_kernel<2, 1, true> : KP == 2 ? rebalance_kernel<1, 2, true> : rebalance_kernel<1, 1, true>;
  return pick_kr<false>(KR, KP);
}

}  // namespace

int32_t rb_make_plan(int32_t E, int32_t P, int32_t G, int32_t N, int32_t RK, int32_t X, RbPlan* out) {
  if (E < 1 || P < 1 || G < 1 || N < 1 || RK < 1 || X < 1) return EPLB_E_ARG;
  const bool hier = G % N == 0;
  const int Gp = hier ? G : 1;
  const int Np = hier ? N : 1;
  if (hier && E % G != 0) return EPLB_E_DIV;
  if (RK % Np != 0 || P % RK != 0) return EPLB_E_DIV;
  if (P < E) return EPLB_E_REDUNDANCY;
  if ((int64_t)X < 1 + (int64_t)(P - E) / Np) return EPLB_E_CAPACITY;
  if (E > kMaxE || P > 2 * kMaxE || X > kMaxX) return EPLB_E_LIMIT;
  if (1 + (P - E) / Np > kMaxCount) return EPLB_E_LIMIT;
  RbPlan p{};
  p.E = E; p.P = P; p.Gp = Gp; p.Np = Np; p.RK = RK; p.X = X;
  p.S = E / Gp; p.En = E / Np; p.Pn = P / Np; p.Rn = p.Pn - p.En;
  p.RKn = RK / Np; p.ppr = P / RK; p.gpn = Gp / Np;
  if (p.En > 512 || p.RKn > 512 || Np > 512) return EPLB_E_LIMIT;
  p.KR = regs_for(p.En);
  p.KP = regs_for(p.RKn);
  p.KN = Np <= 64 ? 1 : 8;
  const int waves = Np < 4 ? 4 : (Np > 8 ? 8 : Np);
  p.threads = waves * 64;
  const int nscr = Np < waves ? Np : waves;        // waves that place nodes
  p.fd_S = fastdiv_make((uint32_t)p.S);
  p.fd_En = fastdiv_make((uint32_t)p.En);
  p.fd_X = fastdiv_make((uint32_t)X);

  int64_t off = 0;
  auto take = [&](int64_t bytes, int64_t align) {
    off = (off + align - 1) / align * align;
    const int64_t at = off;
    off += bytes;
    return (int32_t)at;
  };
  const int64_t rn1 = p.Rn > 0 ? p.Rn : 1;
  p.o_kexp = take(16ll * E, 16);
  p.o_wl = take(8ll * E, 8);
  p.o_m2l = take(4ll * E, 4);
  p.o_cnt = take(4ll * E, 4);
  p.o_srt = take(4ll * E, 4);
  p.o_rep = take(4ll * Np * rn1, 4);
  // lane-parallel packing scratch: step 3 in the one-word form with 65 to
  // 256 GPUs per node (up to 64 packs run in registers)
  const bool wide3 = p.KP > 1 && p.KP <= 4;
  const int kw = wide3 ? p.KP : 1;
  const int64_t pk_bytes = (8ll * (64 * kw + 64) + 4ll * (64 * kw + 1) + 15) / 16 * 16;
  p.pk_words = (int32_t)(pk_bytes / 8);
  p.o_pk = wide3 ? take(pk_bytes * nscr, 16) : 0;
  // Two overlaid regions: the loads and step-1 arrays die once the mlog
  // order is built; the per-wave step-3 scratch is used only after that.
  const int64_t base = (off + 15) / 16 * 16;
  off = base;
  p.o_w = take(8ll * E, 8);
  p.o_gsum = take(8ll * Gp, 8);
  p.o_gnode = take(4ll * Gp, 4);
  p.o_gslot = take(4ll * Gp, 4);
  p.o_gord = take(4ll * Gp, 4);
  p.o_gres = take(4ll * Gp, 4);
  const int64_t end1 = off;
  off = base;
  p.o_posaux = take(12ll * nscr * p.En, 4);
  p.o_ordr = take(4ll * nscr * p.Pn, 4);
  p.o_ores = take(4ll * nscr * p.Pn, 4);
  p.o_rcls = take(4ll * nscr * rn1, 4);
  if (off < end1) off = end1;
  p.o_nflag = take(4ll * Np, 4);
  p.o_flags = take(16, 8);
  off = (off + 15) / 16 * 16;
  // up to 64 KiB for every shape of the pages' workloads; wider shapes take
  // more of the CU's 160 KiB (one workgroup per CU then)
  if (off > kMaxRebalanceLdsBytes) return EPLB_E_LIMIT;
  p.lds_bytes = (int32_t)off;
  *out = p;
  return 0;
}

hipError_t launch_rebalance(const int64_t* load, int64_t B, const RbPlan& plan,
                            int32_t* phy2log, int32_t* log2phy, int32_t* logcnt,
                            int32_t* status, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  pick_kernel(plan.KR, plan.KP, B)<<<(unsigned)B, plan.threads, plan.lds_bytes, stream>>>(
      load, plan, phy2log, log2phy, logcnt, status);
  return hipGetLastError();
}

}  // namespace eplb
