// Reference streams for the benchmark: a plain device-to-device copy and a
// read-only pass over the same bytes, swept over launch shapes, give the
// HBM ceilings the redirect (read + write) and the histogram (read) are
// measured against on the same GPU.  Not part of the EPLB library: built
// into its own libeplb_ref.so and loaded only by bench.py.
//
// The bytes are `layers` equal rows.  Workgroup b takes row b / chunks and,
// as the streaming kernels of the library do, the row's 16-byte vectors
// (b % chunks) * NT + tid + k * chunks * NT, U of them in flight per
// iteration, with non-temporal loads; stores are non-temporal, plain, or
// buffer stores with the sc1 nt cache bits (as the library's redirect).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// kStore: 0 plain, 1 non-temporal, 2 buffer store with the device-scope and
// non-temporal bits (sc1 nt; rows below 2 GiB), the store the library's
// streaming kernels use
template <int NT, int U, int kStore>
__global__ __launch_bounds__(NT) void ref_copy_kernel(const i32x4* __restrict__ src, i32x4* __restrict__ dst,
                                                      int64_t n4l, int32_t chunks) {
  const int64_t row = blockIdx.x / chunks;
  const int64_t chunk = blockIdx.x - row * chunks;
  const i32x4* s = src + row * n4l;
  i32x4* d = dst + row * n4l;
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(d, 0, (int)(kStore == 2 ? n4l * 16 : 0), 0x00020000);
  auto store = [&](const i32x4& x, int64_t v) {
    if constexpr (kStore == 2) __builtin_amdgcn_raw_buffer_store_b128(x, rd, (int)(v * 16), 0, 16 | 2);
    else if constexpr (kStore == 1) __builtin_nontemporal_store(x, d + v);
    else d[v] = x;
  };
  const int64_t step = (int64_t)chunks * NT;
  int64_t v = chunk * NT + threadIdx.x;
  for (; v + (U - 1) * step < n4l; v += U * step) {
    i32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(s + v + u * step);
#pragma unroll
    for (int u = 0; u < U; ++u) store(x[u], v + u * step);
  }
  for (; v < n4l; v += step) store(__builtin_nontemporal_load(s + v), v);
}

// Reads every vector and folds it into one word per thread; a thread writes
// its word only when it equals a value no stream holds (so the loads cannot
// be dropped and nothing is written in practice).
template <int NT, int U>
__global__ __launch_bounds__(NT) void ref_read_kernel(const i32x4* __restrict__ src, int64_t n4l, int32_t chunks,
                                                      int32_t* __restrict__ sink) {
  const int64_t row = blockIdx.x / chunks;
  const int64_t chunk = blockIdx.x - row * chunks;
  const i32x4* s = src + row * n4l;
  const int64_t step = (int64_t)chunks * NT;
  int64_t v = chunk * NT + threadIdx.x;
  int32_t acc = 0;
  for (; v + (U - 1) * step < n4l; v += U * step) {
    i32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(s + v + u * step);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; v < n4l; v += step) {
    const i32x4 x = __builtin_nontemporal_load(s + v);
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  if (acc == 0x7fffffff) sink[0] = acc;
}

template <int NT, int U>
hipError_t launch(int mode, const void* src, void* dst, int64_t n4l, int32_t chunks, unsigned blocks,
                  hipStream_t s) {
  if (mode == 0)
    ref_read_kernel<NT, U><<<blocks, NT, 0, s>>>((const i32x4*)src, n4l, chunks, (int32_t*)dst);
  else if (mode == 1)
    ref_copy_kernel<NT, U, 1><<<blocks, NT, 0, s>>>((const i32x4*)src, (i32x4*)dst, n4l, chunks);
  else if (mode == 2)
    ref_copy_kernel<NT, U, 0><<<blocks, NT, 0, s>>>((const i32x4*)src, (i32x4*)dst, n4l, chunks);
  else
    ref_copy_kernel<NT, U, 2><<<blocks, NT, 0, s>>>((const i32x4*)src, (i32x4*)dst, n4l, chunks);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// mode 0: read src (dst, 4 bytes, is left as it is); 1: copy src to dst with
// non-temporal stores; 2: copy with plain stores; 3: copy with sc1 nt buffer
// stores (rows below 2 GiB).  The bytes are `layers`
// rows of bytes / layers each (a multiple of 16), 16-byte aligned; `chunks`
// workgroups per row of `threads` threads, `unroll` vectors in flight each.
// threads in {256, 512, 1024}, unroll in {1, 2, 4, 8}, layers * chunks
// workgroups at most 2^20.  Returns 0, 1 for an unsupported shape or
// argument, 2 for a launch error.
int32_t eplb_ref_stream(int32_t mode, const void* src, void* dst, int64_t bytes, int64_t layers, int32_t threads,
                        int32_t unroll, int32_t chunks, void* stream) {
  if (src == nullptr || dst == nullptr || bytes < 0 || layers < 1 || chunks < 1 || mode < 0 || mode > 3) return 1;
  if (bytes % (16 * layers) != 0 || layers * chunks > (1 << 20)) return 1;
  if (mode == 3 && bytes / layers >= ((int64_t)1 << 31)) return 1;
  if (((uintptr_t)src | (uintptr_t)dst) & 15) return 1;
  const int64_t n4l = bytes / 16 / layers;
  const unsigned blocks = (unsigned)(layers * chunks);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (threads * 16 + unroll) {
    case 256 * 16 + 1: e = launch<256, 1>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 256 * 16 + 2: e = launch<256, 2>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 256 * 16 + 4: e = launch<256, 4>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 256 * 16 + 8: e = launch<256, 8>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 512 * 16 + 1: e = launch<512, 1>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 512 * 16 + 2: e = launch<512, 2>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 512 * 16 + 4: e = launch<512, 4>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 512 * 16 + 8: e = launch<512, 8>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 1024 * 16 + 1: e = launch<1024, 1>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 1024 * 16 + 2: e = launch<1024, 2>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 1024 * 16 + 4: e = launch<1024, 4>(mode, src, dst, n4l, chunks, blocks, s); break;
    case 1024 * 16 + 8: e = launch<1024, 8>(mode, src, dst, n4l, chunks, blocks, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
