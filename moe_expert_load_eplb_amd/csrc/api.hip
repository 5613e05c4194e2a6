// C ABI of the EPLB hot path: host-side validation, then launches.
// Declarations and the meaning of every argument: include/eplb.h.
#include "eplb.h"
#include "eplb_internal.h"

using namespace eplb;

namespace {

constexpr int64_t kMaxIdsPerLayer = (int64_t(1) << 31) - 1;

int32_t check_stream_args(const void* idx, int64_t L, int64_t T, int32_t K, int32_t E) {
  if (L < 0 || T < 0 || K < 1 || E < 1) return EPLB_E_ARG;
  if (L > 0 && T > 0 && idx == nullptr) return EPLB_E_ARG;
  if (E > kMaxE || L > kMaxLayers) return EPLB_E_LIMIT;
  if (T > kMaxIdsPerLayer / K) return EPLB_E_RANGE;
  return EPLB_OK;
}

// Whether the byte ranges [a, a + na) and [b, b + nb) share a byte (ends
// taken in 128 bits, so a range reaching past the address space still
// compares correctly).
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
  const unsigned __int128 x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (unsigned __int128)nb && y < x + (unsigned __int128)na;
}

// a * b * c bytes, saturated at 2^63 - 1 (a caller's window of W steps is
// not bounded above, so its byte count may not fit).
int64_t bytes_of(int64_t a, int64_t b, int64_t c) {
  int64_t ab = 0, abc = 0;
  if (__builtin_mul_overflow(a, b, &ab) || __builtin_mul_overflow(ab, c, &abc)) return INT64_MAX;
  return abc;
}

// A call with B problems and these input and output ranges: every pointer
// set, no output sharing a byte with an input or another output.
struct Range {
  const void* p;
  int64_t bytes;
};
// No output shares a byte with an input or another output (empty ranges and
// NULL pointers share nothing; the calls check NULLs themselves).
template <int NI, int NO>
int32_t check_disjoint(const Range (&in)[NI], const Range (&out)[NO]) {
  for (int i = 0; i < NO; ++i) {
    for (const Range& c : in)
      if (overlap(out[i].p, out[i].bytes, c.p, c.bytes)) return EPLB_E_ARG;
    for (int j = 0; j < i; ++j)
      if (overlap(out[i].p, out[i].bytes, out[j].p, out[j].bytes)) return EPLB_E_ARG;
  }
  return EPLB_OK;
}

template <int NI, int NO>
int32_t check_buffers(const Range (&in)[NI], const Range (&out)[NO]) {
  for (const Range& a : in)
    if (a.p == nullptr) return EPLB_E_ARG;
  for (const Range& a : out)
    if (a.p == nullptr) return EPLB_E_ARG;
  return check_disjoint(in, out);
}

}  // namespace

namespace eplb {

int32_t check_lp_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, const int32_t* rep,
                          const int64_t* flow, int32_t RK, int32_t R, const int32_t* out) {
  int32_t rc = check_stream_args(idx, L, T, K, E);
  if (rc != EPLB_OK) return rc;
  if (RK < 1 || R < 1) return EPLB_E_ARG;
  if (RK > kLpMaxRanks || R > kLpMaxSlots) return EPLB_E_LIMIT;
  const int64_t n = T * (int64_t)K;
  if (L * lp_segments(n) > kLpMaxSegments) return EPLB_E_LIMIT;
  if (L > 0 && n > 0) {
    if (rep == nullptr || flow == nullptr || out == nullptr) return EPLB_E_ARG;
    const int64_t slots = L * RK * (int64_t)R;
    const Range in[3] = {{idx, L * n * 4}, {rep, slots * 4}, {flow, slots * 8}};
    const Range outs[1] = {{out, L * n * 4}};
    return check_disjoint(in, outs);
  }
  return EPLB_OK;
}

}  // namespace eplb

extern "C" {

int32_t eplb_load_hist(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                       int32_t* ring, int32_t W, int64_t step,
                       int64_t* load, int64_t* n_invalid, void* stream) {
  int32_t rc = check_stream_args(idx, L, T, K, E);
  if (rc != EPLB_OK) return rc;
  if (W < 1 || step < 0) return EPLB_E_ARG;
  if (L > 0 && (ring == nullptr || load == nullptr || n_invalid == nullptr)) return EPLB_E_ARG;
  {
    const Range in[1] = {{idx, L * T * K * 4}};
    const Range out[3] = {{ring, bytes_of(W, L * E, 4)}, {load, L * E * 8}, {n_invalid, L * 8}};
    rc = check_disjoint(in, out);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_hist(idx, L, T, K, E, ring, W, step, load, n_invalid, (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int32_t eplb_rebalance(const int64_t* load, int64_t B, int32_t E, int32_t P,
                       int32_t G, int32_t N, int32_t RK, int32_t X,
                       int32_t* phy2log, int32_t* log2phy, int32_t* logcnt,
                       int32_t* status, void* stream) {
  if (B < 0) return EPLB_E_ARG;
  RbPlan plan;
  int32_t rc = rb_make_plan(E, P, G, N, RK, X, &plan);
  if (rc != EPLB_OK) return rc;
  if (B > kMaxProblems) return EPLB_E_LIMIT;
  if (B > 0) {
    const Range in[1] = {{load, B * E * 8}};
    const Range out[4] = {{phy2log, B * P * 4}, {log2phy, B * E * (int64_t)X * 4}, {logcnt, B * E * 4},
                          {status, B * 4}};
    rc = check_buffers(in, out);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_rebalance(load, B, plan, phy2log, log2phy, logcnt, status, (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int32_t eplb_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                      const int32_t* log2phy, const int32_t* logcnt, int32_t X,
                      int32_t* out, void* stream) {
  int32_t rc = check_stream_args(idx, L, T, K, E);
  if (rc != EPLB_OK) return rc;
  if (X < 1) return EPLB_E_ARG;
  if (X > kMaxX) return EPLB_E_LIMIT;
  if (L > 0 && T > 0 && (log2phy == nullptr || logcnt == nullptr || out == nullptr)) return EPLB_E_ARG;
  if (T > 0) {
    const Range in[3] = {{idx, L * T * K * 4}, {log2phy, L * E * (int64_t)X * 4}, {logcnt, L * E * 4}};
    const Range outs[1] = {{out, L * T * K * 4}};
    rc = check_disjoint(in, outs);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_redirect(idx, L, T, K, E, log2phy, logcnt, X, out, (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int32_t eplb_hist_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                           int32_t* ring, int32_t W, int64_t step, int64_t* load, int64_t* n_invalid,
                           const int32_t* log2phy, const int32_t* logcnt, int32_t X, int32_t* out,
                           void* stream) {
  int32_t rc = check_stream_args(idx, L, T, K, E);
  if (rc != EPLB_OK) return rc;
  if (W < 1 || step < 0 || X < 1) return EPLB_E_ARG;
  if (X > kMaxX) return EPLB_E_LIMIT;
  if (L > 0 && (ring == nullptr || load == nullptr || n_invalid == nullptr)) return EPLB_E_ARG;
  if (L > 0 && T > 0 && (log2phy == nullptr || logcnt == nullptr || out == nullptr)) return EPLB_E_ARG;
  {
    const int64_t tab = T > 0 ? L * E : 0;             // the tables are read only when there are ids
    const Range in[3] = {{idx, L * T * K * 4}, {log2phy, tab * X * 4}, {logcnt, tab * 4}};
    const Range outs[4] = {{ring, bytes_of(W, L * E, 4)}, {load, L * E * 8}, {n_invalid, L * 8},
                           {out, L * T * K * 4}};
    rc = check_disjoint(in, outs);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_hist_redirect(idx, L, T, K, E, ring, W, step, load, n_invalid, log2phy, logcnt, X,
                                        out, (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int32_t eplb_load_ema(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                      int32_t* count, int32_t shift, int64_t* ema, int64_t* n_invalid, void* stream) {
  int32_t rc = check_stream_args(idx, L, T, K, E);
  if (rc != EPLB_OK) return rc;
  if (shift < 0 || shift > 62) return EPLB_E_ARG;
  if (L > 0 && (count == nullptr || ema == nullptr || n_invalid == nullptr)) return EPLB_E_ARG;
  {
    const Range in[1] = {{idx, L * T * K * 4}};
    const Range out[3] = {{count, L * E * 4}, {ema, L * E * 8}, {n_invalid, L * 8}};
    rc = check_disjoint(in, out);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_load_ema(idx, L, T, K, E, count, shift, ema, n_invalid, (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int32_t eplb_ema_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, int32_t* count,
                          int32_t shift, int64_t* ema, int64_t* n_invalid, const int32_t* log2phy,
                          const int32_t* logcnt, int32_t X, int32_t* out, void* stream) {
  int32_t rc = check_stream_args(idx, L, T, K, E);
  if (rc != EPLB_OK) return rc;
  if (shift < 0 || shift > 62 || X < 1) return EPLB_E_ARG;
  if (X > kMaxX) return EPLB_E_LIMIT;
  if (L > 0 && (count == nullptr || ema == nullptr || n_invalid == nullptr)) return EPLB_E_ARG;
  if (L > 0 && T > 0 && (log2phy == nullptr || logcnt == nullptr || out == nullptr)) return EPLB_E_ARG;
  {
    const int64_t tab = T > 0 ? L * E : 0;
    const Range in[3] = {{idx, L * T * K * 4}, {log2phy, tab * X * 4}, {logcnt, tab * 4}};
    const Range outs[4] = {{count, L * E * 4}, {ema, L * E * 8}, {n_invalid, L * 8}, {out, L * T * K * 4}};
    rc = check_disjoint(in, outs);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_ema_redirect(idx, L, T, K, E, count, shift, ema, n_invalid, log2phy, logcnt, X, out,
                                       (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int32_t eplb_placement_load(const int64_t* load, const int32_t* phy2log, const int32_t* logcnt,
                            int64_t B, int32_t E, int32_t P, int32_t RK,
                            double* rank_load, double* imbalance, void* stream) {
  if (B < 0 || E < 1 || P < 1 || RK < 1) return EPLB_E_ARG;
  if (P % RK != 0) return EPLB_E_DIV;
  if (E > kMaxE || B > kMaxProblems) return EPLB_E_LIMIT;    // E * 2^40 < 2^53: the total is exact as a double
  if (B > 0) {
    const Range in[3] = {{load, B * E * 8}, {phy2log, B * P * 4}, {logcnt, B * E * 4}};
    const Range out[2] = {{rank_load, B * RK * 8}, {imbalance, B * 8}};
    const int32_t rc = check_buffers(in, out);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_placement_load(load, phy2log, logcnt, B, E, P, RK, rank_load, imbalance,
                                         (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int32_t eplb_rearrange(const int32_t* old_phy2log, const int32_t* new_phy2log, const int32_t* new_log2phy,
                       int64_t B, int32_t E, int32_t P, int32_t RK, int32_t N, int32_t X,
                       int32_t* phy2log, int32_t* log2phy, int32_t* src, int32_t* moves, int32_t* status,
                       void* stream) {
  if (B < 0 || E < 1 || P < 1 || RK < 1 || N < 1 || X < 1) return EPLB_E_ARG;
  if (P % RK != 0 || RK % N != 0) return EPLB_E_DIV;
  if (E > kMaxE || P > kMaxP || X > kMaxX || B > kMaxProblems) return EPLB_E_LIMIT;
  if (B > 0) {
    const int64_t l2p = B * E * (int64_t)X * 4;
    const Range in[3] = {{old_phy2log, B * P * 4}, {new_phy2log, B * P * 4}, {new_log2phy, l2p}};
    const Range out[5] = {{phy2log, B * P * 4}, {log2phy, l2p}, {src, B * P * 4}, {moves, B * 12}, {status, B * 4}};
    const int32_t rc = check_buffers(in, out);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_rearrange(old_phy2log, new_phy2log, new_log2phy, B, E, P, RK, N, X, phy2log, log2phy,
                                    src, moves, status, (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int32_t eplb_lp_solve(const int64_t* cnt, const int32_t* home, const int32_t* rep, int64_t B, int32_t E,
                      int32_t RK, int32_t R, int64_t* lam, int64_t* flow, int64_t* rank_load, int32_t* status,
                      void* stream) {
  if (B < 0 || E < 1 || RK < 1 || R < 1) return EPLB_E_ARG;
  if (E > kMaxE || RK > kLpMaxRanks || R > kLpMaxSlots || B > kLpMaxProblems) return EPLB_E_LIMIT;
  if (B > 0) {
    const int64_t slots = B * RK * (int64_t)R;
    const Range in[3] = {{cnt, B * E * 8}, {home, B * E * 4}, {rep, slots * 4}};
    const Range out[4] = {{lam, B * 8}, {flow, slots * 8}, {rank_load, B * RK * 8}, {status, B * 4}};
    const int32_t rc = check_buffers(in, out);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_lp_solve(cnt, home, rep, B, E, RK, R, lam, flow, rank_load, status, (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int64_t eplb_lp_redirect_workspace_bytes(int64_t L, int64_t T, int32_t K, int32_t E) {
  if (L < 0 || T < 0 || K < 1 || E < 1) return -(int64_t)EPLB_E_ARG;
  if (T > kMaxIdsPerLayer / K) return -(int64_t)EPLB_E_RANGE;
  return L * lp_segments(T * (int64_t)K) * E * (int64_t)sizeof(int32_t);
}

int32_t eplb_lp_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, const int32_t* rep,
                         const int64_t* flow, int32_t RK, int32_t R, void* workspace, int64_t workspace_bytes,
                         int32_t* out, void* stream) {
  int32_t rc = eplb::check_lp_redirect(idx, L, T, K, E, rep, flow, RK, R, out);
  if (rc != EPLB_OK) return rc;
  const int64_t n = T * (int64_t)K;
  if (L > 0 && n > 0) {
    if (workspace == nullptr) return EPLB_E_ARG;
    const int64_t need = eplb_lp_redirect_workspace_bytes(L, T, K, E);
    if (workspace_bytes < need) return EPLB_E_ARG;
    const int64_t slots = L * RK * (int64_t)R;
    const Range in[3] = {{idx, L * n * 4}, {rep, slots * 4}, {flow, slots * 8}};
    const Range outs[2] = {{out, L * n * 4}, {workspace, need}};
    rc = check_disjoint(in, outs);
    if (rc != EPLB_OK) return rc;
  }
  hipError_t err = launch_lp_redirect(idx, L, n, E, rep, flow, RK, R, static_cast<int32_t*>(workspace), out,
                                      (hipStream_t)stream);
  return err == hipSuccess ? EPLB_OK : EPLB_E_HIP;
}

int32_t eplb_rebalance_max_count(int32_t E, int32_t P, int32_t G, int32_t N) {
  if (E < 1 || P < 1 || G < 1 || N < 1) return -EPLB_E_ARG;
  const bool hier = G % N == 0;
  if (hier && E % G != 0) return -EPLB_E_DIV;
  if (P < E) return -EPLB_E_REDUNDANCY;
  const int32_t nodes = hier ? N : 1;
  return 1 + (P - E) / nodes;
}

int64_t eplb_rebalance_lds_bytes(int32_t E, int32_t P, int32_t G, int32_t N, int32_t RK, int32_t X) {
  RbPlan plan;
  int32_t rc = rb_make_plan(E, P, G, N, RK, X, &plan);
  if (rc != EPLB_OK) return -(int64_t)rc;
  return plan.lds_bytes;
}

const char* eplb_status_string(int32_t code) {
  switch (code) {
    case EPLB_OK: return "ok";
    case EPLB_E_ARG: return "invalid argument (NULL pointer or size out of range)";
    case EPLB_E_DIV: return "divisibility rule broken (E % G, RK % nodes, P % RK)";
    case EPLB_E_REDUNDANCY: return "fewer physical than logical experts";
    case EPLB_E_CAPACITY: return "log2phy width X below 1 + (P - E) / nodes";
    case EPLB_E_LIMIT: return "problem exceeds the kernels' on-chip limits";
    case EPLB_E_RANGE: return "T * K >= 2^31";
    case EPLB_E_HIP: return "HIP launch failed";
    case EPLB_S_BAD_LOAD: return "problem status: a load is negative or above 2^40";
    case EPLB_S_OVERFLOW: return "problem status: exact pack sums need 127 bits or more";
    case EPLB_S_BAD_MAP: return "problem status: a map entry is out of range or an expert has no old replica";
    case EPLB_S_BAD_TOPOLOGY: return "problem status: an id, home rank or count out of range, or an expert replicated twice";
    default: return "unknown code";
  }
}

}  // extern "C"
