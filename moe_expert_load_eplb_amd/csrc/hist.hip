// Expert-load histogram of top-k routing ids, and the load estimate built from
// it: the sum over a window of steps, or an integer moving average.
//
// The load of a logical expert is the number of tokens the router sent to it
// during the observation period (glossary of Part 2 of the EPLB README
// translation, «DualPipe и EPLB», ai.flicky.cc); the prediction uses the
// statistics of past steps, a moving average for instance (opening section of
// Part 2).  Two kernels on one stream: the first clears this step's counts
// and sets the load to the sum of the window's OTHER steps (or the moving
// average to its decayed value, ema - ema / 2^shift); the count then adds
// each workgroup's totals to both the step's counts and the load.
//
// Counting is HBM-bound: 4 bytes read per routing id.  A few workgroups per
// layer sweep the layer together with 16-byte non-temporal loads (all layers
// at once: ~1.8 workgroups of 512 threads per CU in all) and count into
// LDS-resident counters; a workgroup keeps `copies` private copies of the E
// counters (row stride E + 1, so the copies of one expert fall in different
// LDS banks) to spread the increments of a popular expert.  At the end each
// workgroup adds its E totals to the ring slot and to the load with one
// global atomic each.
#include "eplb_internal.h"

namespace eplb {

namespace {


// load[i] = sum of ring[w][i] over the window's other slots; ring[cur][i] = 0;
// n_invalid = 0.  The count kernel then adds the step's counts to both.
__global__ __launch_bounds__(256) void hist_prep_kernel(int32_t* __restrict__ ring, int64_t LE, int32_t W,
                                                        int64_t cur, int64_t* __restrict__ load,
                                                        int64_t* __restrict__ n_invalid, int64_t L) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < LE; i += stride) {
    int64_t s = 0;
    for (int w = 0; w < W; ++w)
      if (w != cur) s += ring[(int64_t)w * LE + i];
    load[i] = s;
    ring[cur * LE + i] = 0;
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < L; i += stride) n_invalid[i] = 0;
}

// One step of the integer moving average, ema <- ema - floor(ema / 2^shift) +
// cnt, in two parts: here the decay (and cnt = 0, n_invalid = 0), then the
// count kernel adds the step's counts.  Unsigned arithmetic keeps a wrap
// (values near 2^63, outside the documented range) defined; >> of the signed
// value is the floor for negative values too.
__global__ __launch_bounds__(256) void ema_prep_kernel(int32_t* __restrict__ cnt, int64_t LE, int32_t shift,
                                                       int64_t* __restrict__ ema, int64_t* __restrict__ n_invalid,
                                                       int64_t L) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < LE; i += stride) {
    const int64_t e = ema[i];
    ema[i] = (int64_t)((u64)e - (u64)(e >> shift));
    cnt[i] = 0;
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < L; i += stride) n_invalid[i] = 0;
}

// One routing id into a workgroup's LDS counters, or into the thread's count
// of ids outside [0, E).  (A branch-free form that sends those to a padding
// column measured ~3% slower here: the branch is uniform in practice.)
__device__ __forceinline__ void count_or_invalid(int32_t e, uint32_t E, int32_t* my, uint32_t& inv) {
  if ((uint32_t)e < E) atomicAdd(&my[e], 1);
  else ++inv;
}

// Workgroup c of `chunks` per layer takes the layer's 16-byte vectors
// c*NT + tid + k*chunks*NT, so the workgroups of a layer sweep it together,
// one contiguous window at a time.  Ids before the layer's first 16-byte
// boundary and after its last one are counted by workgroup 0.
__global__ __launch_bounds__(kCountThreads) void hist_count_kernel(const int32_t* __restrict__ idx,
                                                                    StreamSplit sp, int32_t E, int32_t copies,
                                                                    int32_t* __restrict__ slot,
                                                                    int64_t* __restrict__ acc,
                                                                    int64_t* __restrict__ n_invalid) {
  extern __shared__ int32_t counters[];             // [copies][E + 1]
  const int64_t layer = blockIdx.x / sp.chunks;
  const int64_t chunk = blockIdx.x - layer * sp.chunks;
  const int stride = E + 1;
  const int tid = threadIdx.x;
  constexpr int NT = kCountThreads, U = kCountUnroll;

  for (int i = tid; i < copies * stride; i += NT) counters[i] = 0;
  __syncthreads();

  const int32_t* base = idx + layer * sp.per_layer;
  const int64_t n = sp.per_layer;
  int32_t* my = counters + (tid & (copies - 1)) * stride;
  const uint32_t uE = (uint32_t)E;
  uint32_t inv = 0;

  const int misalign = (int)(((uintptr_t)base >> 2) & 3);
  int64_t head = (4 - misalign) & 3;
  if (head > n) head = n;
  const int64_t n4 = (n - head) >> 2;
  const int64_t tail0 = head + (n4 << 2);
  if (chunk == 0) {
    if (tid < head) count_or_invalid(base[tid], uE, my, inv);
    if (tail0 + tid < n) count_or_invalid(base[tail0 + tid], uE, my, inv);
  }
  const i32x4* body = reinterpret_cast<const i32x4*>(base + head);
  const int64_t step = (int64_t)sp.chunks * NT;
  for (int64_t v = chunk * NT + tid; v < n4; v += step * U) {
    i32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t vv = v + u * step;
      if (vv < n4) x[u] = __builtin_nontemporal_load(body + vv);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (v + u * step < n4) {
        count_or_invalid(x[u].x, uE, my, inv);
        count_or_invalid(x[u].y, uE, my, inv);
        count_or_invalid(x[u].z, uE, my, inv);
        count_or_invalid(x[u].w, uE, my, inv);
      }
    }
  }
  if (inv) atomicAdd(&my[E], (int32_t)inv);       // column E: this workgroup's ids outside [0, E)
  __syncthreads();
  flush_counts(counters, copies, E, slot + layer * E, acc + layer * E, n_invalid + layer);
}

int grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > 4096) g = 4096;
  return (int)g;
}

}  // namespace

StreamSplit plan_stream(int64_t L, int64_t per_layer, int threads, int unroll, int blocks) {
  StreamSplit s;
  s.per_layer = per_layer;
  const int64_t n4 = per_layer / 4;
  const int64_t per_block = (int64_t)threads * unroll;
  // Rounded down: more workgroups than fit on the chip at once leave a
  // second, mostly idle wave of workgroups (measured: 9 per layer instead of
  // 8 over 58 layers costs ~40%).
  int64_t chunks = L > 0 ? blocks / L : 1;
  const int64_t useful = (n4 + per_block - 1) / per_block;     // every thread gets a vector
  if (chunks > useful) chunks = useful;
  if (chunks < 1) chunks = 1;
  s.chunks = (int32_t)chunks;
  return s;
}

hipError_t launch_hist_prep(int32_t* ring, int64_t LE, int32_t W, int64_t cur, int64_t* load, int64_t* n_invalid,
                            int64_t L, hipStream_t stream) {
  hist_prep_kernel<<<grid_for(LE > L ? LE : L, 256), 256, 0, stream>>>(ring, LE, W, cur, load, n_invalid, L);
  return hipGetLastError();
}

hipError_t launch_ema_prep(int32_t* cnt, int64_t LE, int32_t shift, int64_t* ema, int64_t* n_invalid, int64_t L,
                           hipStream_t stream) {
  ema_prep_kernel<<<grid_for(LE > L ? LE : L, 256), 256, 0, stream>>>(cnt, LE, shift, ema, n_invalid, L);
  return hipGetLastError();
}

namespace {

// Count the step's ids into `slot` ([L][E], cleared) and add them to `acc`
// ([L][E] int64) and `n_invalid`.
hipError_t launch_count(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, int32_t* slot,
                        int64_t* acc, int64_t* n_invalid, hipStream_t stream) {
  const int64_t per_layer = T * (int64_t)K;
  if (per_layer == 0) return hipSuccess;
  const StreamSplit sp = plan_stream(L, per_layer, kCountThreads, kCountUnroll, kCountBlocks);
  int copies = 16;
  while (copies > 1 && (int64_t)copies * (E + 1) * 4 > 32 * 1024) copies >>= 1;
  const size_t lds = (size_t)copies * (E + 1) * sizeof(int32_t);
  const int64_t blocks = L * sp.chunks;
  hist_count_kernel<<<(unsigned)blocks, kCountThreads, lds, stream>>>(idx, sp, E, copies, slot, acc, n_invalid);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hist(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                       int32_t* ring, int32_t W, int64_t step, int64_t* load,
                       int64_t* n_invalid, hipStream_t stream) {
  if (L == 0) return hipSuccess;
  const int64_t LE = L * (int64_t)E;
  const int64_t cur = step % W;
  hipError_t err = launch_hist_prep(ring, LE, W, cur, load, n_invalid, L, stream);
  if (err != hipSuccess) return err;
  return launch_count(idx, L, T, K, E, ring + cur * LE, load, n_invalid, stream);
}

hipError_t launch_load_ema(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                           int32_t* cnt, int32_t shift, int64_t* ema, int64_t* n_invalid,
                           hipStream_t stream) {
  if (L == 0) return hipSuccess;
  hipError_t err = launch_ema_prep(cnt, L * (int64_t)E, shift, ema, n_invalid, L, stream);
  if (err != hipSuccess) return err;
  return launch_count(idx, L, T, K, E, cnt, ema, n_invalid, stream);
}

}  // namespace eplb
