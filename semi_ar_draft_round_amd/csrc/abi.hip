// The C ABI: argument checks, workspace sizing and the launch sequences.
// Every check that needs no device data happens here, before anything is
// enqueued; the kernels themselves assume valid shapes.
#include <string.h>

#include <atomic>

#include "common.hpp"
#include "rnn_head.hpp"
#include "sample_common.hpp"

namespace dspark {
// sample.hip
size_t sample_workspace_bytes(dspark_dtype dt, int R, int gamma, int V);
size_t rnn_workspace_bytes(int R, int gamma, int r);
hipError_t rnn_prepare_launch(int V, int r, int d, const uint16_t* W1, const uint16_t* Wrnn, float* P,
                              hipStream_t s);
// sts.hip
size_t sts_workspace_bytes(int N, int gamma, int G, int M);
bool sts_shape_ok(int N, int gamma, int G, int M);
hipError_t sts_launch(int N, int gamma, const float* z, const int32_t* n_acc, const float* grid, int G, int M,
                      float* T, double* ece_before, double* ece_after, double* auc, void* ws, hipStream_t s);
const char* sample_kernel_name(dspark_dtype dt, int R, int V, int r);
const char* rnn_kernel_name(dspark_dtype dt, int R, int V, int r);
hipError_t sample_launch(dspark_dtype dt, int R, int gamma, int V, int r, const void* U,
                         const void* W1, const void* W2t, const int32_t* x0, const float* G,
                         const float* g, int32_t* x, float* lse, float* logit, void* ws,
                         hipStream_t s, const RnnHead* rnn, const uint32_t* cancel, int32_t* status,
                         const SampleConf* conf, hipEvent_t ev0, hipEvent_t ev1);
// confidence.hip
hipError_t confidence_launch(dspark_dtype dt, int R, int gamma, int d, int r, int V, const void* h,
                             const void* w, const void* W1, const int32_t* x0, const int32_t* x,
                             const float* T, float* c, float* z, hipStream_t s);
// schedule.hip
size_t schedule_workspace_bytes(int R, int gamma);
hipError_t schedule_launch(int R, int gamma, const float* c, const double* sps, int mode, const int32_t* cap,
                           int32_t* ell, int32_t* admitted, double* theta_best, void* ws, hipStream_t s);
int schedule_static_slots();
hipError_t schedule_launch_static(int R, int gamma, const float* c, const double* sps, int mode, const int32_t* cap,
                                  int32_t* ell, int32_t* admitted, double* theta_best, hipStream_t s);
// verify.hip
size_t verify_greedy_workspace_bytes(int R, int gamma);
size_t acceptance_workspace_bytes(int R, int gamma, int V);
hipError_t verify_greedy_launch(dspark_dtype dt, int R, int gamma, int V, const void* target, const int32_t* row0,
                                const int32_t* x, const int32_t* ell, int32_t* n_acc, int32_t* next_tok, void* ws,
                                hipStream_t s);
hipError_t acceptance_launch(dspark_dtype dt, int R, int gamma, int V, int r, const void* target,
                             const int32_t* row0, const void* U, const void* W1, const void* W2t, const int32_t* x0,
                             const int32_t* x, const float* lse, float* c_star, void* ws, hipStream_t s,
                             const void* bvec);
size_t verify_workspace_bytes(int R, int gamma, int V);
hipError_t verify_launch(dspark_dtype dt, int R, int gamma, int V, int r, const void* target,
                         const int32_t* row0, const void* U, const void* W1, const void* W2t,
                         const int32_t* x0, const int32_t* x, const float* lse, const float* logit,
                         const int32_t* ell, const float* u_acc, const float* u_res, int32_t* n_acc,
                         int32_t* next_tok, void* ws, hipStream_t s, const void* bvec);

namespace {

constexpr int kMaxGamma = 64;
constexpr int kMaxVocab = 1 << 24;
constexpr int kMaxSchedSlots = 8191;

bool dtype_ok(dspark_dtype dt) { return dt == DSPARK_F32 || dt == DSPARK_BF16; }

// r supported by the storage type: the bf16 matrix-core tile takes whole
// k-steps of 32 with 1, 2, 4 or 8 of them in registers.
bool rank_ok(dspark_dtype dt, int r) {
  if (dt == DSPARK_BF16) return r == 32 || r == 64 || r == 128 || r == 256;
  return r >= 1 && r <= 1024;
}

bool draft_shape_ok(int R, int gamma, int V) {
  return R >= 1 && R <= 65535 && gamma >= 1 && gamma <= kMaxGamma && V >= 2 && V < kMaxVocab &&
         static_cast<int64_t>(R) * gamma <= (1LL << 30);
}

// 0 = unknown, 1 = gfx950, 2 = something else
std::atomic<int> g_device_kind[64];
std::atomic<int> g_device_cus[64];

dspark_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DSPARK_EDEVICE;
  int kind = g_device_kind[dev].load(std::memory_order_relaxed);
  if (kind == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DSPARK_EDEVICE;
    kind = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                            std::memory_order_relaxed);
    g_device_kind[dev].store(kind, std::memory_order_relaxed);
  }
  return kind == 1 ? DSPARK_OK : DSPARK_EDEVICE;
}

}  // namespace

// Compute units of the current device (valid after a successful check_device).
int compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  const int n = g_device_cus[dev].load(std::memory_order_relaxed);
  return n > 0 ? n : 1;
}

}  // namespace dspark

using namespace dspark;

extern "C" {

const char* dspark_status_string(dspark_status s) {
  switch (s) {
    case DSPARK_OK: return "success";
    case DSPARK_EINVAL: return "invalid size or pointer argument";
    case DSPARK_EDTYPE: return "unsupported data type or rank for this call";
    case DSPARK_EWORKSPACE: return "workspace missing or too small";
    case DSPARK_ELAUNCH: return "kernel launch failed";
    case DSPARK_EDEVICE: return "current device is not a gfx950 GPU";
    case DSPARK_ETIMEOUT: return "the sampler's grid barrier timed out or was cancelled (no valid draw)";
  }
  return "unknown status";
}

const char* dspark_markov_sample_kernel(dspark_dtype dt, int R, int gamma, int V, int r) {
  if (!dtype_ok(dt) || !draft_shape_ok(R, gamma, V) || !rank_ok(dt, r)) return nullptr;
  if (check_device() != DSPARK_OK) return nullptr;
  return sample_kernel_name(dt, R, V, r);
}

const char* dspark_rnn_sample_kernel(dspark_dtype dt, int R, int gamma, int V, int r) {
  if (!dtype_ok(dt) || !draft_shape_ok(R, gamma, V) || !rank_ok(dt, r)) return nullptr;
  if (check_device() != DSPARK_OK) return nullptr;
  return rnn_kernel_name(dt, R, V, r);
}

static size_t sample_ws_any(int R, int gamma, int V) {
  const size_t a = sample_workspace_bytes(DSPARK_F32, R, gamma, V), b = sample_workspace_bytes(DSPARK_BF16, R, gamma, V);
  return a > b ? a : b;
}

// The sampler's workspace (256-byte aligned), then the RNN projection partials.
static size_t rnn_sample_workspace_bytes(int R, int gamma, int V, int r) {
  return ((sample_ws_any(R, gamma, V) + 255) & ~static_cast<size_t>(255)) + rnn_workspace_bytes(R, gamma, r);
}

size_t dspark_workspace_size(dspark_ws_kind kind, int R, int gamma, int V, int r, int n_sps) {
  (void)r;
  (void)n_sps;
  switch (kind) {
    case DSPARK_WS_SAMPLE:
      if (!draft_shape_ok(R, gamma, V)) return 0;
      // the fp32 path keeps one partial per chunk, the bf16 path fewer
      return sample_workspace_bytes(DSPARK_F32, R, gamma, V) > sample_workspace_bytes(DSPARK_BF16, R, gamma, V)
                 ? sample_workspace_bytes(DSPARK_F32, R, gamma, V)
                 : sample_workspace_bytes(DSPARK_BF16, R, gamma, V);
    case DSPARK_WS_SCHEDULE:
      if (R < 1 || gamma < 1 || gamma > kMaxGamma || static_cast<int64_t>(R) * (1 + gamma) > kMaxSchedSlots) return 0;
      return schedule_workspace_bytes(R, gamma);
    case DSPARK_WS_VERIFY:
      if (!draft_shape_ok(R, gamma, V)) return 0;
      return verify_workspace_bytes(R, gamma, V);
    case DSPARK_WS_VERIFY_GREEDY:
      if (!draft_shape_ok(R, gamma, V)) return 0;
      return verify_greedy_workspace_bytes(R, gamma);
    case DSPARK_WS_ACCEPTANCE:
      if (!draft_shape_ok(R, gamma, V)) return 0;
      return acceptance_workspace_bytes(R, gamma, V);
    case DSPARK_WS_RNN_SAMPLE:
      if (!draft_shape_ok(R, gamma, V) || r < 1) return 0;
      return rnn_sample_workspace_bytes(R, gamma, V, r);
    case DSPARK_WS_STS:
      if (!sts_shape_ok(R, gamma, V, r)) return 0;
      return sts_workspace_bytes(R, gamma, V, r);
  }
  return 0;
}

dspark_status dspark_markov_sample_ex(dspark_dtype dt, int R, int gamma, int V, int r, int d, const void* U,
                                      const void* W1, const void* W2t, const int32_t* x0, const float* G,
                                      const float* g, const void* h, const void* w, const float* T, int32_t* x,
                                      float* lse, float* logit, float* c, float* z, const uint32_t* cancel,
                                      int32_t* status, void* const* events, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!dtype_ok(dt)) return DSPARK_EDTYPE;
  if (!draft_shape_ok(R, gamma, V)) return DSPARK_EINVAL;
  if (!rank_ok(dt, r)) return DSPARK_EDTYPE;
  if (!U || !W1 || !W2t || !x0 || !G || !g || !x || !lse || !logit) return DSPARK_EINVAL;
  const bool conf = h != nullptr;
  if (conf) {
    const int vec = (dt == DSPARK_BF16) ? 8 : 4;
    if (!w || !c || d < 1 || d % vec != 0 || r % vec != 0) return DSPARK_EINVAL;
  }
  if (events && (!events[0] || !events[1])) return DSPARK_EINVAL;
  if (!ws || ws_bytes < sample_workspace_bytes(dt, R, gamma, V)) return DSPARK_EWORKSPACE;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const SampleConf cf{h, w, d, T, c, z};
  const hipEvent_t e0 = events ? static_cast<hipEvent_t>(events[0]) : nullptr;
  const hipEvent_t e1 = events ? static_cast<hipEvent_t>(events[1]) : nullptr;
  if (sample_launch(dt, R, gamma, V, r, U, W1, W2t, x0, G, g, x, lse, logit, ws, s, nullptr, cancel, status,
                    conf ? &cf : nullptr, e0, e1) != hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_markov_sample(dspark_dtype dt, int R, int gamma, int V, int r, const void* U,
                                   const void* W1, const void* W2t, const int32_t* x0, const float* G,
                                   const float* g, int32_t* x, float* lse, float* logit, void* ws,
                                   size_t ws_bytes, void* stream) {
  return dspark_markov_sample_ex(dt, R, gamma, V, r, 0, U, W1, W2t, x0, G, g, nullptr, nullptr, nullptr, x, lse,
                                 logit, nullptr, nullptr, nullptr, nullptr, nullptr, ws, ws_bytes, stream);
}

dspark_status dspark_confidence(dspark_dtype dt, int R, int gamma, int d, int r, int V, const void* h,
                                const void* w, const void* W1, const int32_t* x0, const int32_t* x,
                                const float* T, float* c, float* z, void* stream) {
  if (!dtype_ok(dt)) return DSPARK_EDTYPE;
  if (!draft_shape_ok(R, gamma, V) || d < 1 || r < 1) return DSPARK_EINVAL;
  const int vec = (dt == DSPARK_BF16) ? 8 : 4;
  if (d % vec != 0 || r % vec != 0) return DSPARK_EINVAL;
  if (!h || !w || !W1 || !x0 || !x || !c) return DSPARK_EINVAL;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  if (confidence_launch(dt, R, gamma, d, r, V, h, w, W1, x0, x, T, c, z, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_schedule_ex(int R, int gamma, const float* c, const double* sps, int n_sps, int mode,
                                 const int32_t* cap, int32_t* ell, int32_t* admitted, double* theta_best,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (R < 1 || gamma < 1 || gamma > kMaxGamma) return DSPARK_EINVAL;
  if (static_cast<int64_t>(R) * (1 + gamma) > kMaxSchedSlots) return DSPARK_EINVAL;
  if (n_sps < R * (1 + gamma)) return DSPARK_EINVAL;
  if (!c || !sps || !ell) return DSPARK_EINVAL;
  if (mode != DSPARK_SCHED_EARLY_STOP && mode != DSPARK_SCHED_WHOLE_WALK && mode != DSPARK_SCHED_CAPACITY)
    return DSPARK_EINVAL;
  if (mode == DSPARK_SCHED_CAPACITY && !cap) return DSPARK_EINVAL;
  if (!ws || ws_bytes < schedule_workspace_bytes(R, gamma)) return DSPARK_EWORKSPACE;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  if (schedule_launch(R, gamma, c, sps, mode, cap, ell, admitted, theta_best, ws, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_schedule_noalloc(int R, int gamma, const float* c, const double* sps, int n_sps, int mode,
                                      const int32_t* cap, int32_t* ell, int32_t* admitted, double* theta_best,
                                      void* stream) {
  if (R < 1 || gamma < 1 || gamma > kMaxGamma) return DSPARK_EINVAL;
  if (static_cast<int64_t>(R) * (1 + gamma) > kMaxSchedSlots) return DSPARK_EINVAL;
  if (static_cast<int64_t>(R) * gamma > schedule_static_slots()) return DSPARK_EINVAL;
  if (n_sps < R * (1 + gamma)) return DSPARK_EINVAL;
  if (!c || !sps || !ell) return DSPARK_EINVAL;
  if (mode != DSPARK_SCHED_EARLY_STOP && mode != DSPARK_SCHED_WHOLE_WALK && mode != DSPARK_SCHED_CAPACITY)
    return DSPARK_EINVAL;
  if (mode == DSPARK_SCHED_CAPACITY && !cap) return DSPARK_EINVAL;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  if (schedule_launch_static(R, gamma, c, sps, mode, cap, ell, admitted, theta_best,
                             static_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_schedule(int R, int gamma, const float* c, const double* sps, int n_sps,
                              int32_t* ell, int32_t* admitted, double* theta_best, void* ws,
                              size_t ws_bytes, void* stream) {
  return dspark_schedule_ex(R, gamma, c, sps, n_sps, DSPARK_SCHED_EARLY_STOP, nullptr, ell, admitted,
                            theta_best, ws, ws_bytes, stream);
}

dspark_status dspark_verify_ex(dspark_dtype dt, int R, int gamma, int V, int r, const void* target,
                               const int32_t* row0, const void* U, const void* W1, const void* W2t, const void* bvec,
                               const int32_t* x0, const int32_t* x, const float* lse, const float* logit,
                               const int32_t* ell, const float* u_acc, const float* u_res, int32_t* n_acc,
                               int32_t* next_tok, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dt)) return DSPARK_EDTYPE;
  if (!draft_shape_ok(R, gamma, V)) return DSPARK_EINVAL;
  if (static_cast<int64_t>(R) * (gamma + 1) > 0x7FFFFFFF) return DSPARK_EINVAL;
  if (!rank_ok(dt, r)) return DSPARK_EDTYPE;
  if (!target || !U || !W1 || !W2t || !x0 || !x || !lse || !logit || !ell || !u_acc || !u_res || !n_acc ||
      !next_tok)
    return DSPARK_EINVAL;
  if (!ws || ws_bytes < verify_workspace_bytes(R, gamma, V)) return DSPARK_EWORKSPACE;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  if (verify_launch(dt, R, gamma, V, r, target, row0, U, W1, W2t, x0, x, lse, logit, ell, u_acc, u_res,
                    n_acc, next_tok, ws, static_cast<hipStream_t>(stream), bvec) != hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_verify(dspark_dtype dt, int R, int gamma, int V, int r, const void* target,
                            const int32_t* row0, const void* U, const void* W1, const void* W2t,
                            const int32_t* x0, const int32_t* x, const float* lse, const float* logit,
                            const int32_t* ell, const float* u_acc, const float* u_res, int32_t* n_acc,
                            int32_t* next_tok, void* ws, size_t ws_bytes, void* stream) {
  return dspark_verify_ex(dt, R, gamma, V, r, target, row0, U, W1, W2t, nullptr, x0, x, lse, logit, ell, u_acc,
                          u_res, n_acc, next_tok, ws, ws_bytes, stream);
}

dspark_status dspark_verify_greedy(dspark_dtype dt, int R, int gamma, int V, const void* target,
                                   const int32_t* row0, const int32_t* x, const int32_t* ell, int32_t* n_acc,
                                   int32_t* next_tok, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dt)) return DSPARK_EDTYPE;
  if (!draft_shape_ok(R, gamma, V)) return DSPARK_EINVAL;
  if (!target || !x || !ell || !n_acc || !next_tok) return DSPARK_EINVAL;
  if (!ws || ws_bytes < verify_greedy_workspace_bytes(R, gamma)) return DSPARK_EWORKSPACE;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  if (verify_greedy_launch(dt, R, gamma, V, target, row0, x, ell, n_acc, next_tok, ws,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_acceptance(dspark_dtype dt, int R, int gamma, int V, int r, const void* target,
                                const int32_t* row0, const void* U, const void* W1, const void* W2t,
                                const void* bvec, const int32_t* x0, const int32_t* x, const float* lse,
                                float* c_star, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dt)) return DSPARK_EDTYPE;
  if (!draft_shape_ok(R, gamma, V)) return DSPARK_EINVAL;
  if (!rank_ok(dt, r)) return DSPARK_EDTYPE;
  if (!target || !U || !W1 || !W2t || !x0 || !x || !lse || !c_star) return DSPARK_EINVAL;
  if (!ws || ws_bytes < acceptance_workspace_bytes(R, gamma, V)) return DSPARK_EWORKSPACE;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  if (acceptance_launch(dt, R, gamma, V, r, target, row0, U, W1, W2t, x0, x, lse, c_star, ws,
                        static_cast<hipStream_t>(stream), bvec) != hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

static dspark_status rnn_sample_impl(dspark_dtype dt, int R, int gamma, int V, int r, int d, const void* U,
                                     const void* W1, const void* W2t, const void* Wrnn, const void* h,
                                     const int32_t* x0, const float* G, const float* g, const float* P, int32_t* x,
                                     float* lse, float* logit, float* s, void* o, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!dtype_ok(dt)) return DSPARK_EDTYPE;
  if (!draft_shape_ok(R, gamma, V)) return DSPARK_EINVAL;
  if (!rank_ok(dt, r)) return DSPARK_EDTYPE;
  if (d < 1 || d > (1 << 20) || (dt == DSPARK_BF16 && d % 16 != 0)) return DSPARK_EINVAL;
  if (!U || !W1 || !W2t || !Wrnn || !h || !x0 || !G || !g || !x || !lse || !logit || !s || !o)
    return DSPARK_EINVAL;
  if (!ws || ws_bytes < rnn_sample_workspace_bytes(R, gamma, V, r)) return DSPARK_EWORKSPACE;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  const size_t off = (sample_ws_any(R, gamma, V) + 255) & ~static_cast<size_t>(255);
  const RnnHead head{Wrnn, h, d, s, o, reinterpret_cast<float*>(static_cast<char*>(ws) + off),
                     dt == DSPARK_BF16 ? P : nullptr};
  if (sample_launch(dt, R, gamma, V, r, U, W1, W2t, x0, G, g, x, lse, logit, ws, static_cast<hipStream_t>(stream),
                    &head, nullptr, nullptr, nullptr, nullptr, nullptr) != hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_rnn_sample(dspark_dtype dt, int R, int gamma, int V, int r, int d, const void* U,
                                const void* W1, const void* W2t, const void* Wrnn, const void* h,
                                const int32_t* x0, const float* G, const float* g, int32_t* x, float* lse,
                                float* logit, float* s, void* o, void* ws, size_t ws_bytes, void* stream) {
  return rnn_sample_impl(dt, R, gamma, V, r, d, U, W1, W2t, Wrnn, h, x0, G, g, nullptr, x, lse, logit, s, o, ws,
                         ws_bytes, stream);
}

dspark_status dspark_rnn_sample_ex(dspark_dtype dt, int R, int gamma, int V, int r, int d, const void* U,
                                   const void* W1, const void* W2t, const void* Wrnn, const void* h,
                                   const int32_t* x0, const float* G, const float* g, const float* P, int32_t* x,
                                   float* lse, float* logit, float* s, void* o, void* ws, size_t ws_bytes,
                                   void* stream) {
  return rnn_sample_impl(dt, R, gamma, V, r, d, U, W1, W2t, Wrnn, h, x0, G, g, P, x, lse, logit, s, o, ws,
                         ws_bytes, stream);
}

dspark_status dspark_rnn_prepare(dspark_dtype dt, int V, int r, int d, const void* W1, const void* Wrnn, float* P,
                                 void* stream) {
  if (!dtype_ok(dt)) return DSPARK_EDTYPE;
  if (dt != DSPARK_BF16 || !rank_ok(dt, r)) return DSPARK_EDTYPE;
  if (V < 2 || V >= (1 << 24) || d < 1 || d > (1 << 20) || d % 16 != 0) return DSPARK_EINVAL;
  if (!W1 || !Wrnn || !P) return DSPARK_EINVAL;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  if (rnn_prepare_launch(V, r, d, static_cast<const uint16_t*>(W1), static_cast<const uint16_t*>(Wrnn), P,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_sts_fit(int N, int gamma, const float* z, const int32_t* n_acc, const float* grid,
                             int n_grid, int n_bins, float* T, double* ece_before, double* ece_after, double* auc,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!sts_shape_ok(N, gamma, n_grid, n_bins)) return DSPARK_EINVAL;
  if (!z || !n_acc || !grid || !T || !ece_before || !ece_after || !auc) return DSPARK_EINVAL;
  if (!ws || ws_bytes < sts_workspace_bytes(N, gamma, n_grid, n_bins)) return DSPARK_EWORKSPACE;
  dspark_status st = check_device();
  if (st != DSPARK_OK) return st;
  if (sts_launch(N, gamma, z, n_acc, grid, n_grid, n_bins, T, ece_before, ece_after, auc, ws,
                 static_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ELAUNCH;
  return DSPARK_OK;
}

}  // extern "C"
