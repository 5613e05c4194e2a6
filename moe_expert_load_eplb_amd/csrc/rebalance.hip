// Batched EPLB rebalance: one workgroup per problem (an MoE layer or a load
// snapshot), the whole problem resident in LDS.
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
// All arithmetic is integer and exact.  Step 2 compares u_a / c_a with
// u_b / c_b by cross-multiplication (u <= 2^40, c < 2^13, products < 2^53).
// Step 3 scales every per-replica load by D = lcm(replica counts of the
// node), so item keys u * (D / c) and pack sums are exact 128-bit integers;
// D is built from the prime factorisation of the counts, and a node with
// D * (node load sum) >= 2^127 marks the problem EPLB_S_OVERFLOW.
//
// Layout in LDS (offsets from RbPlan): loads w[E] and their node-major copy
// wl[E] ("mlog" order: node n holds wl[n*En .. n*En+En)), the mlog<->logical
// permutations, per-mlog counts, the replicas created per node, 128-bit keys
// per expert and per item, per-node sort rows, and the packing scratch.
//
// The sequential parts of the method (the greedy packs and the replication
// rounds) run one wavefront per node with wave-wide reductions; sorts and
// all elementwise phases use the whole workgroup.
#include "eplb.h"
#include "eplb_internal.h"

namespace eplb {

namespace {

#define SMALL_PRIMES 2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 41, 43, 47, 53, 59, 61, 67, \
                     71, 73, 79, 83, 89, 97, 101, 103, 107, 109, 113, 127
constexpr int kNumSmallPrimes = 31;
__device__ __constant__ int kSmallPrimes[kNumSmallPrimes] = {SMALL_PRIMES};

// ---------------------------------------------------------------- 128-bit helpers

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

__device__ __forceinline__ u64 shfl_xor_u64(u64 v, int m) {
  return (u64)__shfl_xor((unsigned long long)v, m);
}
__device__ __forceinline__ u64 shfl_u64(u64 v, int src) {
  return (u64)__shfl((unsigned long long)v, src);
}

template <typename K> struct KeyOps;
template <> struct KeyOps<u64> {
  __device__ static u64 max() { return ~0ull; }
  __device__ static u64 shfl_xor(u64 v, int m) { return shfl_xor_u64(v, m); }
};
template <> struct KeyOps<u128> {
  __device__ static u128 max() { return ~(u128)0; }
  __device__ static u128 shfl_xor(u128 v, int m) {
    const u64 lo = shfl_xor_u64((u64)v, m);
    const u64 hi = shfl_xor_u64((u64)(v >> 64), m);
    return ((u128)hi << 64) | lo;
  }
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------- sorting

// Bitonic sort of `nseg` independent rows of n2 (a power of two) item ids,
// stored back to back in `arr`.  `before(seg, a, b)` must be a strict total
// order on the ids of one row; the whole workgroup takes part.
template <class Before>
__device__ void seg_bitonic(int32_t* arr, int nseg, int n2, int log2n2, Before before) {
  const int total = nseg * n2;
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < total; i += blockDim.x) {
        const int li = i & (n2 - 1);
        if ((li & j) == 0) {
          const int seg = i >> log2n2;
          const int a = arr[i];
          const int b = arr[i + j];
          const bool asc = (li & k) == 0;
          const bool a_first = before(seg, a, b);
          if (asc != a_first) {
            arr[i] = b;
            arr[i + j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- greedy packing

// Balanced packing of n items (visited in the order given by `order`) into m
// packs of `cap` items each, by one wavefront: each item goes into the pack
// with the smallest sum among packs with room, lowest pack index on ties.
// Pack p lives in lane p % 64 (sums in psum[], counts in pcnt[], wave-private
// LDS); each lane caches its best open pack and a wave-wide argmin picks the
// winner.  result[item] = pack * cap + arrival position.
template <typename K, class KeyOf>
__device__ void wave_pack(const int32_t* order, int n, int m, int cap, KeyOf key_of,
                          int32_t* result, K* psum, int32_t* pcnt) {
  const int lane = lane_id();
  for (int p = lane; p < m; p += 64) {
    psum[p] = 0;
    pcnt[p] = 0;
  }
  int m2 = 1;
  while (m2 < m && m2 < 64) m2 <<= 1;
  // Lane-local best open pack (sum, index); index INT_MAX marks none.
  K bs = KeyOps<K>::max();
  int bp = 0x7fffffff;
  int bc = 0;
  for (int p = lane; p < m; p += 64) {
    if (bp == 0x7fffffff) { bs = 0; bp = p; bc = 0; }   // all sums are 0: lowest own index
  }
  for (int t = 0; t < n; ++t) {
    const int item = order[t];
    K s = bs;
    int p = bp;
    int c = bc;
    for (int off = 1; off < m2; off <<= 1) {
      const K os = KeyOps<K>::shfl_xor(s, off);
      const int op = __shfl_xor(p, off);
      const int oc = __shfl_xor(c, off);
      if (os < s || (os == s && op < p)) { s = os; p = op; c = oc; }
    }
    // Lanes 0 .. m2-1 now agree on the winner (p, c); it belongs to lane p % 64.
    if (lane == 0) result[item] = p * cap + c;
    if (lane == (p & 63) && p != 0x7fffffff) {
      psum[p] += key_of(item);
      pcnt[p] = c + 1;
      bs = KeyOps<K>::max();
      bp = 0x7fffffff;
      bc = 0;
      for (int q = lane; q < m; q += 64) {
        const int qc = pcnt[q];
        if (qc < cap) {
          const K qs = psum[q];
          if (qs < bs || (qs == bs && q < bp)) { bs = qs; bp = q; bc = qc; }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- replication

// Grow the node's En experts to En + Rn physical ones, one replica at a time,
// each to the expert with the highest load per replica u[i] / c[i] (lowest
// index on ties).  c[] enters as all ones.  rep[r] = expert | (rank << 16) of
// the r-th replica created (its rank is the expert's count before it).
// Also returns the node's load sum.
__device__ u64 wave_replicate(const u64* u, int32_t* c, int En, int Rn, int32_t* rep) {
  const int lane = lane_id();
  // (u, c, i) is better than (u', c', i') if u * c' > u' * c, or equal and i < i'.
  u64 bu = 0;
  int bc = 1;
  int bi = 0x7fffffff;
  u64 sum = 0;
  for (int i = lane; i < En; i += 64) {
    const u64 ui = u[i];
    sum += ui;
    if (bi == 0x7fffffff || ui * (u64)bc > bu) { bu = ui; bc = 1; bi = i; }
  }
  for (int off = 32; off > 0; off >>= 1) sum += shfl_xor_u64(sum, off);
  for (int r = 0; r < Rn; ++r) {
    u64 xu = bu;
    int xc = bc;
    int xi = bi;
    for (int off = 1; off < 64; off <<= 1) {
      const u64 ou = shfl_xor_u64(xu, off);
      const int oc = __shfl_xor(xc, off);
      const int oi = __shfl_xor(xi, off);
      const u64 lhs = ou * (u64)xc;
      const u64 rhs = xu * (u64)oc;
      if (lhs > rhs || (lhs == rhs && oi < xi)) { xu = ou; xc = oc; xi = oi; }
    }
    if (lane == 0) rep[r] = xi | (xc << 16);
    if (lane == (xi & 63)) {
      c[xi] = xc + 1;
      bu = 0;
      bc = 1;
      bi = 0x7fffffff;
      for (int i = lane; i < En; i += 64) {
        const u64 ui = u[i];
        const int ci = c[i];
        if (bi == 0x7fffffff || ui * (u64)bc > bu * (u64)ci) { bu = ui; bc = ci; bi = i; }
      }
    }
  }
  return sum;
}

// Exponent of each prime up to 127 in c; returns the cofactor.  Counts are at
// most kMaxCount < 131^2, so once the primes below 131 are divided out the
// cofactor is 1 or a single prime, which keeps the lcm built from these
// factorisations exact.
__device__ __forceinline__ int factor_small(int c, int* ex) {
  const int primes[kNumSmallPrimes] = {SMALL_PRIMES};
#pragma unroll
  for (int k = 0; k < kNumSmallPrimes; ++k) {
    const int q = primes[k];
    int e = 0;
    while (c % q == 0) { c /= q; ++e; }
    ex[k] = e;
  }
  return c;
}

// ---------------------------------------------------------------- kernel

struct Smem {
  u64* w; u64* wl; int32_t* m2l; int32_t* l2m; int32_t* cnt;
  u64* gsum; int32_t* gnode; int32_t* gslot; int32_t* gsort;
  int32_t* rep; u128* kexp; u128* ikey; int32_t* sort; int32_t* pid;
  int32_t* emax; int32_t* bigf; int32_t* big; int32_t* nbig; u64* nsum; u128* dn;
  unsigned char* psum; int32_t* pcnt; int32_t* flags;
};

__device__ Smem carve(unsigned char* base, const RbPlan& p) {
  Smem s;
  s.w = (u64*)(base + p.o_w);          s.wl = (u64*)(base + p.o_wl);
  s.m2l = (int32_t*)(base + p.o_m2l);  s.l2m = (int32_t*)(base + p.o_l2m);
  s.cnt = (int32_t*)(base + p.o_cnt);  s.gsum = (u64*)(base + p.o_gsum);
  s.gnode = (int32_t*)(base + p.o_gnode); s.gslot = (int32_t*)(base + p.o_gslot);
  s.gsort = (int32_t*)(base + p.o_gsort); s.rep = (int32_t*)(base + p.o_rep);
  s.kexp = (u128*)(base + p.o_kexp);   s.ikey = (u128*)(base + p.o_ikey);
  s.sort = (int32_t*)(base + p.o_sort); s.pid = (int32_t*)(base + p.o_pid);
  s.emax = (int32_t*)(base + p.o_emax); s.bigf = (int32_t*)(base + p.o_bigf);
  s.big = (int32_t*)(base + p.o_big);  s.nbig = (int32_t*)(base + p.o_nbig);
  s.nsum = (u64*)(base + p.o_nsum);    s.dn = (u128*)(base + p.o_dn);
  s.psum = base + p.o_psum;            s.pcnt = (int32_t*)(base + p.o_pcnt);
  s.flags = (int32_t*)(base + p.o_flags);
  return s;
}

__device__ void write_failed(const RbPlan& p, int64_t b, int32_t code, int32_t* phy2log,
                             int32_t* log2phy, int32_t* logcnt, int32_t* status) {
  for (int i = threadIdx.x; i < p.P; i += blockDim.x) phy2log[b * p.P + i] = -1;
  for (int i = threadIdx.x; i < p.E * p.X; i += blockDim.x) log2phy[b * p.E * p.X + i] = -1;
  for (int i = threadIdx.x; i < p.E; i += blockDim.x) logcnt[b * p.E + i] = -1;
  if (threadIdx.x == 0) status[b] = code;
}

__global__ __launch_bounds__(1024) void rebalance_kernel(const int64_t* __restrict__ load, RbPlan p,
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
  if (tid == 0) s.flags[0] = 0;
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

  // ---- step 1: groups -> nodes
  if (p.gpn == 1) {
    for (int g = tid; g < p.Gp; g += NT) { s.gnode[g] = g; s.gslot[g] = 0; }
  } else {
    for (int g = wid; g < p.Gp; g += NW) {
      u64 sum = 0;
      for (int j = lane; j < p.S; j += 64) sum += s.w[(int64_t)g * p.S + j];
      for (int off = 32; off > 0; off >>= 1) sum += shfl_xor_u64(sum, off);
      if (lane == 0) s.gsum[g] = sum;
    }
    for (int i = tid; i < p.G2; i += NT) s.gsort[i] = i;
    __syncthreads();
    const int Gp = p.Gp;
    const u64* gsum = s.gsum;
    int log2g = 0;
    while ((1 << log2g) < p.G2) ++log2g;
    seg_bitonic(s.gsort, 1, p.G2, log2g, [=](int, int a, int b2) {
      if (a >= Gp || b2 >= Gp) return (a < Gp) || (b2 >= Gp && a < b2);
      const u64 wa = gsum[a], wb = gsum[b2];
      return wa > wb || (wa == wb && a < b2);
    });
    if (wid == 0) {
      wave_pack<u64>(s.gsort, Gp, p.Np, p.gpn, [=](int item) { return gsum[item]; }, s.gnode,
                     (u64*)s.psum, s.pcnt);
    }
    __syncthreads();
    for (int g = tid; g < Gp; g += NT) {
      const int r = s.gnode[g];
      s.gnode[g] = r / p.gpn;
      s.gslot[g] = r - (r / p.gpn) * p.gpn;
    }
  }
  __syncthreads();

  // ---- mlog order: expert g*S + j of a group at (node, slot) -> node*En + slot*S + j
  for (int e = tid; e < p.E; e += NT) {
    const int g = (int)fastdiv_apply((uint32_t)e, p.fd_S);
    const int j = e - g * p.S;
    const int m = (s.gnode[g] * p.gpn + s.gslot[g]) * p.S + j;
    s.m2l[m] = e;
    s.l2m[e] = m;
    s.wl[m] = s.w[e];
    s.cnt[m] = 1;
  }
  // clear the per-node factorisation tables
  for (int i = tid; i < p.Np * kNumSmallPrimes; i += NT) s.emax[i] = 0;
  for (int i = tid; i < p.Np * p.bigw; i += NT) s.bigf[i] = 0;
  for (int i = tid; i < p.Np; i += NT) s.nbig[i] = 0;
  __syncthreads();

  // ---- step 2: replicas within each node (one wave per node)
  for (int n = wid; n < p.Np; n += NW) {
    const u64 sum = wave_replicate(s.wl + n * p.En, s.cnt + n * p.En, p.En, p.Rn, s.rep + n * p.Rn);
    if (lane == 0) s.nsum[n] = sum;
  }
  __syncthreads();

  // ---- step 3a: D_n = lcm of the node's counts, from their factorisations
  for (int m = tid; m < p.E; m += NT) {
    const int c = s.cnt[m];
    if (c > 1) {
      const int n = (int)fastdiv_apply((uint32_t)m, p.fd_En);
      int ex[kNumSmallPrimes];
      const int cof = factor_small(c, ex);
#pragma unroll
      for (int k = 0; k < kNumSmallPrimes; ++k)
        if (ex[k]) atomicMax(&s.emax[n * kNumSmallPrimes + k], ex[k]);
      if (cof > 1) {
        // cof is a prime above 127; list it once per node (bit cof of the
        // node's presence bitset), the list holds at most bigcap entries
        // because only counts >= 131 have such a factor.
        const unsigned bit = 1u << (cof & 31);
        if ((atomicOr((unsigned*)&s.bigf[n * p.bigw + (cof >> 5)], bit) & bit) == 0) {
          const int slot = atomicAdd(&s.nbig[n], 1);
          s.big[n * p.bigcap + slot] = cof;
        }
      }
    }
  }
  __syncthreads();
  for (int n = tid; n < p.Np; n += NT) {
    bool ovf = false;
    u128 d = 1;
    for (int k = 0; k < kNumSmallPrimes; ++k)
      for (int e = s.emax[n * kNumSmallPrimes + k]; e > 0; --e) d = mul_u128_u64(d, (u64)kSmallPrimes[k], ovf);
    for (int q = 0; q < s.nbig[n]; ++q) d = mul_u128_u64(d, (u64)s.big[n * p.bigcap + q], ovf);
    const u128 tot = mul_u128_u64(d, s.nsum[n], ovf);
    if (ovf || (tot >> 127) != 0) s.flags[0] = EPLB_S_OVERFLOW;
    s.dn[n] = d;
  }
  __syncthreads();
  if (s.flags[0] != 0) {
    write_failed(p, b, s.flags[0], phy2log, log2phy, logcnt, status);
    return;
  }

  // ---- step 3b: exact scaled loads: expert key u * (D_n / c), item keys
  for (int m = tid; m < p.E; m += NT) {
    const int c = s.cnt[m];
    const int n = (int)fastdiv_apply((uint32_t)m, p.fd_En);
    u128 q = s.dn[n];
    if (c > 1) {
      int ex[kNumSmallPrimes];
      const int cof = factor_small(c, ex);
      bool ovf = false;
      q = 1;
      for (int k = 0; k < kNumSmallPrimes; ++k)
        for (int e = s.emax[n * kNumSmallPrimes + k] - ex[k]; e > 0; --e)
          q = mul_u128_u64(q, (u64)kSmallPrimes[k], ovf);
      for (int i = 0; i < s.nbig[n]; ++i) {
        const int bq = s.big[n * p.bigcap + i];
        if (bq != cof) q = mul_u128_u64(q, (u64)bq, ovf);
      }
    }
    bool ovf = false;
    s.kexp[m] = mul_u128_u64(q, s.wl[m], ovf);     // <= D_n * u < 2^127
  }
  __syncthreads();
  for (int i = tid; i < p.Np * p.Pn2; i += NT) {
    const int n = i >> p.logPn2;
    const int j = i & (p.Pn2 - 1);
    s.sort[i] = j;
    if (j < p.Pn) {
      const int li = j < p.En ? j : (s.rep[n * p.Rn + (j - p.En)] & 0xffff);
      s.ikey[n * p.Pn + j] = s.kexp[n * p.En + li];
    }
  }
  __syncthreads();

  // ---- step 3c: heaviest first (stable), then pack onto the node's GPUs
  if (p.ppr == 1) {
    for (int i = tid; i < p.P; i += NT) s.pid[i] = i;
  } else {
    const int Pn = p.Pn;
    const u128* ikey = s.ikey;
    seg_bitonic(s.sort, p.Np, p.Pn2, p.logPn2, [=](int seg, int a, int b2) {
      if (a >= Pn || b2 >= Pn) return (a < Pn) || (b2 >= Pn && a < b2);
      const u128 ka = ikey[seg * Pn + a], kb = ikey[seg * Pn + b2];
      return ka > kb || (ka == kb && a < b2);
    });
    const int slots = p.pack_slots;
    for (int n = wid; n < p.Np; n += NW) {
      const u128* nkey = ikey + n * Pn;
      wave_pack<u128>(s.sort + n * p.Pn2, Pn, p.RKn, p.ppr, [=](int item) { return nkey[item]; },
                      s.pid + n * Pn, (u128*)s.psum + wid * slots, s.pcnt + wid * slots);
    }
    __syncthreads();
    for (int i = tid; i < p.P; i += NT) {
      const int n = i / Pn;            // Pn >= 2 here; a division per item, once
      s.pid[i] += n * Pn;
    }
  }
  __syncthreads();

  // ---- outputs
  int32_t* o_phy = phy2log + b * p.P;
  int32_t* o_l2p = log2phy + b * (int64_t)p.E * p.X;
  int32_t* o_cnt = logcnt + b * p.E;
  for (int i = tid; i < p.P; i += NT) {
    const int n = i / p.Pn;
    const int j = i - n * p.Pn;
    int li, rank;
    if (j < p.En) { li = j; rank = 0; }
    else { const int r = s.rep[n * p.Rn + (j - p.En)]; li = r & 0xffff; rank = r >> 16; }
    const int e = s.m2l[n * p.En + li];
    const int pid = s.pid[i];
    o_phy[pid] = e;
    o_l2p[(int64_t)e * p.X + rank] = pid;
  }
  for (int i = tid; i < p.E * p.X; i += NT) {
    const int e = (int)fastdiv_apply((uint32_t)i, p.fd_X);
    const int r = i - e * p.X;
    if (r >= s.cnt[s.l2m[e]]) o_l2p[i] = -1;
  }
  for (int e = tid; e < p.E; e += NT) o_cnt[e] = s.cnt[s.l2m[e]];
  if (tid == 0) status[b] = 0;
}

int pow2_at_least(int n) {
  int v = 1;
  while (v < n) v <<= 1;
  return v;
}

int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
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
  p.G2 = pow2_at_least(Gp < 2 ? 2 : Gp);
  p.Pn2 = pow2_at_least(p.Pn < 2 ? 2 : p.Pn);
  p.logPn2 = log2_exact(p.Pn2);
  int waves = Np < 4 ? 4 : (Np > 16 ? 16 : Np);
  p.threads = waves * 64;
  p.pack_slots = (p.RKn > Np ? p.RKn : Np);
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
  p.o_kexp = take(16ll * E, 16);
  p.o_ikey = take(16ll * P, 16);
  p.o_dn = take(16ll * Np, 16);
  p.o_psum = take(16ll * waves * p.pack_slots, 16);
  p.o_w = take(8ll * E, 8);
  p.o_wl = take(8ll * E, 8);
  p.o_gsum = take(8ll * Gp, 8);
  p.o_nsum = take(8ll * Np, 8);
  p.o_m2l = take(4ll * E, 4);
  p.o_l2m = take(4ll * E, 4);
  p.o_cnt = take(4ll * E, 4);
  p.o_gnode = take(4ll * Gp, 4);
  p.o_gslot = take(4ll * Gp, 4);
  p.o_gsort = take(4ll * p.G2, 4);
  p.o_rep = take(4ll * Np * (p.Rn > 0 ? p.Rn : 1), 4);
  p.o_sort = take(4ll * Np * p.Pn2, 4);
  p.o_pid = take(4ll * P, 4);
  p.o_emax = take(4ll * Np * kNumSmallPrimes, 4);
  p.bigw = (p.Rn + 2 + 31) / 32;
  p.bigcap = p.Rn / 130 + 1;
  p.o_big = take(4ll * Np * p.bigcap, 4);
  p.o_nbig = take(4ll * Np, 4);
  p.o_pcnt = take(4ll * waves * p.pack_slots, 4);
  p.o_flags = take(16, 4);
  p.o_bigf = take(4ll * Np * p.bigw, 4);
  off = (off + 15) / 16 * 16;
  if (off > kMaxLdsBytes) return EPLB_E_LIMIT;
  p.lds_bytes = (int32_t)off;
  *out = p;
  return 0;
}

hipError_t launch_rebalance(const int64_t* load, int64_t B, const RbPlan& plan,
                            int32_t* phy2log, int32_t* log2phy, int32_t* logcnt,
                            int32_t* status, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  rebalance_kernel<<<(unsigned)B, plan.threads, plan.lds_bytes, stream>>>(load, plan, phy2log, log2phy,
                                                                          logcnt, status);
  return hipGetLastError();
}

}  // namespace eplb
