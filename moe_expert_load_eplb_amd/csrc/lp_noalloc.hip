// eplb_lp_redirect_noalloc: the redirect by flows of eplb_lp_redirect for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  Its per-segment
// counts live in a fixed array of this library on each GPU instead of a
// caller workspace; the kernels are those of eplb_lp_redirect.
//
// The array is a file-scope device symbol, so it exists once per GPU the
// library runs on and stays until the process ends.  Host code never passes
// its name to a kernel (on the host that name is only a stand-in): the
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept.  Every call on a GPU shares that GPU's
// array: calls that overlap in time on one GPU (on different streams, or
// from different threads) race; calls on one stream do not.  The count
// kernel writes every entry the later kernels read, so nothing in the array
// has to start at zero and no call clears it.
#include <mutex>

#include "eplb.h"
#include "eplb_internal.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) int32_t scratch[EPLB_NOALLOC_SCRATCH_BYTES / 4];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call
// on that device), or nullptr with *err set.
void* scratch_address(int32_t* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = EPLB_E_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      *err = EPLB_E_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int32_t eplb_lp_redirect_noalloc(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                                            const int32_t* rep, const int64_t* flow, int32_t RK, int32_t R,
                                            int32_t* out, void* stream) {
  int32_t rc = eplb::check_lp_redirect(idx, L, T, K, E, rep, flow, RK, R, out);
  if (rc != EPLB_OK) return rc;
  const int64_t n = T * (int64_t)K;
  if (L == 0 || n == 0) return EPLB_OK;
  if (eplb::lp_redirect_counts(L, n, E, RK, R) * 4 > EPLB_NOALLOC_SCRATCH_BYTES) return EPLB_E_LIMIT;
  void* ws = scratch_address(&rc);
  if (ws == nullptr) return rc;
  const hipError_t err = eplb::launch_lp_redirect(idx, L, n, E, rep, flow, RK, R, static_cast<int32_t*>(ws), out,
                                                  (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}
