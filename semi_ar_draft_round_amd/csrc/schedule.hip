// dspark_schedule: the hardware-aware prefix scheduler (Algorithm 1), batched.
//
// Passage: DSpark reading notes, "hardware-aware prefix scheduler":
// Algorithm 1 steps 1-6, Lemma 1 (prefix closure of the ranked pool) and the
// causal early stop; caijizhuo summary, sections 三 and 四 (admit).
//
// Two launches.  schedule_rank, many work groups:
//   1. survival a_{r,j} as the fp64 left-to-right product of the fp32
//      confidences, quantised to a_fx = floor(a * 2^50) (one thread per
//      request; every work group computes all of them);
//   2. ranking: each slot gets a 64-bit key ((2^50 - a_fx) << 13) | (r*gamma + j)
//      so that ascending keys are descending a_fx, then ascending request,
//      then ascending position; slots with a_fx = 0 sort after every
//      candidate.  Survival never increases along a request, so each
//      request's keys form a sorted run, and (keys being distinct) a key's
//      rank is its position in its own run plus, for every other run, the
//      number of that run's keys below it: one fixed-depth binary descent
//      per run, the runs of each key dealt out over sixteen threads, four
//      descents in lockstep.  The key is stored at its rank in the workspace.
// schedule_kernel, one work group of 1024 threads, everything in LDS and
// registers:
//   3. tau_fx(m) = R 2^50 + the exact integer prefix sum of the ranked a_fx;
//   4. A, by mode:
//      early stop  the first m with Theta(m) <= Theta(m-1) (exact comparison
//                  of tau_fx(m) * SPS(R+m) with tau_fx(m-1) * SPS(R+m-1))
//                  gives A = m - 1;
//      whole walk  the smallest m with the largest Theta(m), m = 0..M: each
//                  thread keeps the best of its ranked slots, then a wave
//                  reduction and one pass over the wave winners, every
//                  comparison exact (the production scheduler's capacity;
//                  notes, "adapting Algorithm 1 to real hardware");
//      capacity    A = min(max(K, 0), M) with K read from device memory (the
//                  production scheduler's fill; notes, "the asynchronous fix");
//   5. l_r = number of request r's slots ranked before position A.
// Every step is integer or exact, so the result does not depend on the order
// in which threads add things up.
#include "common.hpp"

#include <atomic>
#include <mutex>

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedMaxSlots = 8192;    // keys in LDS: two buffers of 8192 * 8 bytes = 128 KiB
constexpr int kQ = 50;
constexpr uint64_t kOne = 1ull << kQ;

struct U128 {
  uint64_t hi, lo;
};

__device__ __forceinline__ U128 mul_u64(uint64_t a, uint64_t b) { return U128{__umul64hi(a, b), a * b}; }

__device__ __forceinline__ int bitlen128(U128 v) {
  if (v.hi) return 128 - __clzll(static_cast<long long>(v.hi));
  if (v.lo) return 64 - __clzll(static_cast<long long>(v.lo));
  return 0;
}

__device__ __forceinline__ U128 shl128(U128 v, int s) {
  if (s == 0) return v;
  if (s >= 64) return U128{v.lo << (s - 64), 0};
  return U128{(v.hi << s) | (v.lo >> (64 - s)), v.lo << s};
}

__device__ __forceinline__ int cmp128(U128 a, U128 b) {
  if (a.hi != b.hi) return a.hi > b.hi ? 1 : -1;
  if (a.lo != b.lo) return a.lo > b.lo ? 1 : -1;
  return 0;
}

// d = mant * 2^exp exactly, for finite d >= 0.
__device__ __forceinline__ void split_double(double d, uint64_t& mant, int& exp2) {
  const uint64_t bits = static_cast<uint64_t>(__double_as_longlong(d));
  const int eb = static_cast<int>((bits >> 52) & 0x7FF);
  const uint64_t frac = bits & ((1ull << 52) - 1);
  if (eb == 0) {
    mant = frac;
    exp2 = -1074;
  } else {
    mant = frac | (1ull << 52);
    exp2 = eb - 1075;
  }
}

// Sign of t1 * d1 - t2 * d2, exactly (t < 2^63, d finite and >= 0).
__device__ int cmp_products(uint64_t t1, double d1, uint64_t t2, double d2) {
  uint64_t m1, m2;
  int e1, e2;
  split_double(d1, m1, e1);
  split_double(d2, m2, e2);
  U128 p1 = mul_u64(t1, m1), p2 = mul_u64(t2, m2);
  const int b1 = bitlen128(p1), b2 = bitlen128(p2);
  if (b1 == 0 || b2 == 0) return (b1 != 0) - (b2 != 0);
  const int s1 = b1 + e1, s2 = b2 + e2;
  if (s1 != s2) return s1 > s2 ? 1 : -1;
  if (e1 >= e2)
    p1 = shl128(p1, e1 - e2);
  else
    p2 = shl128(p2, e2 - e1);
  return cmp128(p1, p2);
}

// The same sign, decided in double precision when the two products are
// clearly apart (each is within 2^-52 relative of its exact value, so a gap
// above 2^-40 of the larger cannot be a rounding artefact) and exactly
// otherwise.
__device__ int cmp_theta(uint64_t t1, double d1, uint64_t t2, double d2) {
  const double p1 = static_cast<double>(t1) * d1, p2 = static_cast<double>(t2) * d2;
  const double diff = p1 - p2;
  if (fabs(diff) > fmax(p1, p2) * 0x1p-40) return diff > 0 ? 1 : -1;
  return cmp_products(t1, d1, t2, d2);
}

// A point of the ranked walk: admitting the first m slots gives tau_fx = t
// and Theta = t * s (s = SPS(R + m)); m < 0 marks no point.
struct WalkPoint {
  uint64_t t;
  double s;
  int m;
};

// The better of two points: the larger Theta, the smaller m on equal Theta.
__device__ __forceinline__ WalkPoint better(WalkPoint a, WalkPoint b) {
  if (a.m < 0) return b;
  if (b.m < 0) return a;
  const int cmp = cmp_theta(a.t, a.s, b.t, b.s);
  if (cmp != 0) return cmp > 0 ? a : b;
  return a.m < b.m ? a : b;
}

// The key of slot (req, j) for j = 0 .. gamma-1 (one thread per request),
// from the confidences staged in LDS.
__device__ __forceinline__ void slot_keys(int req, int gamma, const float* cl, uint64_t* keys) {
  double s = 1.0;
  for (int j = 0; j < gamma; ++j) {
    s = s * static_cast<double>(cl[req * gamma + j]);
    const uint64_t afx = static_cast<uint64_t>(floor(s * static_cast<double>(kOne)));
    keys[req * gamma + j] = ((kOne - afx) << 13) | static_cast<uint64_t>(req * gamma + j);
  }
}

constexpr int kRankThreads = 512;
constexpr int kRankKeys = 32;                              // keys ranked per work group
constexpr int kRankParts = kRankThreads / kRankKeys;       // threads sharing a key's runs (16)
constexpr int kRankBatch = 4;                              // runs searched in lockstep per thread

__global__ __launch_bounds__(kRankThreads) void schedule_rank(int R, int gamma, const float* __restrict__ c,
                                                              uint64_t* __restrict__ ranked) {
  __shared__ uint64_t keys[kSchedMaxSlots];
  __shared__ float cl[kSchedMaxSlots];
  __shared__ int below[kRankKeys];
  const int tid = threadIdx.x;
  const int n = R * gamma;
  for (int i = tid; i < n; i += kRankThreads) cl[i] = c[i];   // one coalesced pass
  if (tid < kRankKeys) below[tid] = 0;
  __syncthreads();
  for (int req = tid; req < R; req += kRankThreads) slot_keys(req, gamma, cl, keys);
  __syncthreads();
  const int kl = tid % kRankKeys;
  const int i = blockIdx.x * kRankKeys + kl;
  if (i < n) {
    const uint64_t key = keys[i];
    const int own = i / gamma;
    int top = 1;   // highest power of two <= gamma: a fixed-depth descent
    while ((top << 1) <= gamma) top <<= 1;
    int cnt = 0;
    for (int run0 = tid / kRankKeys; run0 < R; run0 += kRankBatch * kRankParts) {
      int pos[kRankBatch];
#pragma unroll
      for (int b = 0; b < kRankBatch; ++b) pos[b] = 0;
      // pos[b] becomes the number of keys of run run0 + b kRankParts below `key`
      for (int step = top; step > 0; step >>= 1) {
#pragma unroll
        for (int b = 0; b < kRankBatch; ++b) {
          const int run = run0 + b * kRankParts;
          const int q = pos[b] + step;
          if (run < R && q <= gamma && keys[run * gamma + q - 1] < key) pos[b] = q;
        }
      }
#pragma unroll
      for (int b = 0; b < kRankBatch; ++b) {
        const int run = run0 + b * kRankParts;
        if (run < R && run != own) cnt += pos[b];
      }
    }
    atomicAdd(&below[kl], cnt);
  }
  __syncthreads();
  if (tid < kRankKeys && i < n) ranked[below[tid] + i % gamma] = keys[i];
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(int R, int gamma,
                                                                 const double* __restrict__ sps,
                                                                 int mode,
                                                                 const int32_t* __restrict__ cap,
                                                                 const uint64_t* __restrict__ ranked,
                                                                 int32_t* __restrict__ ell,
                                                                 int32_t* __restrict__ admitted,
                                                                 double* __restrict__ theta_best) {
  __shared__ uint64_t lds_small[32];   // wave totals, then scalars
  __shared__ WalkPoint wbest[kSchedThreads / kWave];
  const int tid = threadIdx.x;
  const int n = R * gamma;

  uint64_t* keys = lds_small;
  for (int req = tid; req < R; req += kSchedThreads) ell[req] = 0;
  const int P = n;   // ranked keys: keys[0 .. n)

  // 3: thread t owns ranked positions [t*8, t*8+8)
  constexpr int kPer = kSchedMaxSlots / kSchedThreads;   // 8
  const uint64_t cand_limit = kOne << 13;                // keys below are candidates
  // the step speeds of this thread's positions, SPS(R + m) for
  // m = tid * kPer - 1 .. tid * kPer + kPer - 1 (those past the pool unread),
  // fetched alongside the ranked keys rather than after them
  double sp[kPer + 1];
#pragma unroll
  for (int u = 0; u <= kPer; ++u) sp[u] = (tid * kPer + u <= P) ? sps[R + tid * kPer + u - 1] : 0.0;
  uint64_t myk[kPer];
  uint64_t local = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int p = tid * kPer + t;
    myk[t] = (p < P) ? ranked[p] : ~0ull;
    if (myk[t] < cand_limit) local += kOne - (myk[t] >> 13);
  }
  __syncthreads();                     // ell is cleared before any slot is admitted
  // exclusive prefix of the per-thread sums: a scan inside each wave, then
  // one pass over the wave totals
  uint64_t incl = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint64_t v = __shfl_up(incl, o);
    if ((tid & (kWave - 1)) >= o) incl += v;
  }
  constexpr int kWaves = kSchedThreads / kWave;
  uint64_t* wsum = keys;                                     // kWaves entries
  int* sh = reinterpret_cast<int*>(keys + kWaves);           // scalars
  if ((tid & (kWave - 1)) == kWave - 1) wsum[tid / kWave] = incl;
  if (tid == 0) {
    sh[0] = 0x7FFFFFFF;                // first drop position m
    sh[1] = 0;                         // candidate count M
  }
  __syncthreads();
  uint64_t before = 0, total = 0;
#pragma unroll
  for (int wv = 0; wv < kWaves; ++wv) {
    const uint64_t v = wsum[wv];
    before += wv < tid / kWave ? v : 0;
    total += v;
  }
  const uint64_t excl = before + incl - local;   // sum of the ranked values before this thread's
  uint64_t tau_prev = static_cast<uint64_t>(R) * kOne + excl;
  int my_first_drop = 0x7FFFFFFF;
  int my_count = 0;
  // whole walk: this thread's best point (thread 0 also holds m = 0)
  WalkPoint mine{static_cast<uint64_t>(R) * kOne, sp[0], tid == 0 ? 0 : -1};
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    if (myk[t] >= cand_limit) break;
    ++my_count;
    const int m = tid * kPer + t + 1;               // admitting the m-th ranked slot
    const uint64_t tau = tau_prev + (kOne - (myk[t] >> 13));
    const double s_m = sp[t + 1];                   // SPS(R + m)
    if (mode == DSPARK_SCHED_EARLY_STOP) {
      if (my_first_drop == 0x7FFFFFFF && cmp_theta(tau, s_m, tau_prev, sp[t]) <= 0) my_first_drop = m;
    } else if (mode == DSPARK_SCHED_WHOLE_WALK) {
      mine = better(mine, WalkPoint{tau, s_m, m});
    }
    tau_prev = tau;
  }
  // one LDS atomic per wave (the first drop and the candidate count reduced
  // in the wave first)
  int wave_drop = my_first_drop, wave_count = my_count;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    wave_drop = min(wave_drop, __shfl_xor(wave_drop, o));
    wave_count += __shfl_xor(wave_count, o);
  }
  if ((tid & (kWave - 1)) == 0) {
    if (wave_drop != 0x7FFFFFFF) atomicMin(&sh[0], wave_drop);
    if (wave_count) atomicAdd(&sh[1], wave_count);
  }
  if (mode == DSPARK_SCHED_WHOLE_WALK) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const WalkPoint other{__shfl_xor(mine.t, o), __shfl_xor(mine.s, o), __shfl_xor(mine.m, o)};
      mine = better(mine, other);
    }
    if ((tid & (kWave - 1)) == 0) wbest[tid / kWave] = mine;
  }
  __syncthreads();
  const int M = sh[1];
  int A;
  if (mode == DSPARK_SCHED_WHOLE_WALK) {
    WalkPoint b = wbest[0];
#pragma unroll
    for (int wv = 1; wv < kWaves; ++wv) b = better(b, wbest[wv]);
    A = b.m;
  } else if (mode == DSPARK_SCHED_CAPACITY) {
    A = min(max(cap[0], 0), M);
  } else {
    A = (sh[0] == 0x7FFFFFFF) ? M : sh[0] - 1;
  }
  // threshold key: the first ranked slot that is not admitted
  __syncthreads();
  uint64_t* thr = reinterpret_cast<uint64_t*>(sh + 4);
  if (tid == A / kPer) {
    uint64_t v = ~0ull;
#pragma unroll
    for (int t = 0; t < kPer; ++t)
      if (tid * kPer + t == A) v = myk[t];
    thr[0] = v;
    thr[1] = static_cast<uint64_t>(R) * kOne + excl;
    uint64_t tauA = thr[1];
#pragma unroll
    for (int t = 0; t < kPer; ++t)
      if (tid * kPer + t < A) tauA += kOne - (myk[t] >> 13);
    thr[1] = tauA;
  }
  if (A == kSchedThreads * kPer && tid == 0) {   // every slot admitted (P = 8192)
    thr[0] = ~0ull;
    thr[1] = static_cast<uint64_t>(R) * kOne + total;
  }
  __syncthreads();
  const uint64_t threshold = thr[0];

  // 5: lengths from the admitted ranked slots: the ranked prefix is
  // prefix-closed per request, so l_r is one more than the largest admitted
  // position of request r
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int p = tid * kPer + t;
    if (p < A && myk[t] < threshold) {
      const int slot = static_cast<int>(myk[t] & 0x1FFF);
      atomicMax(ell + slot / gamma, slot % gamma + 1);
    }
  }
  if (tid == 0) {
    if (admitted) admitted[0] = A;
    if (theta_best) theta_best[0] = static_cast<double>(thr[1]) * 0x1p-50 * sps[R + A - 1];
  }
}

// The ranked slot keys.
size_t schedule_workspace_bytes(int R, int gamma) {
  return (sizeof(uint64_t) * static_cast<size_t>(R) * gamma + 255) & ~static_cast<size_t>(255);
}

hipError_t schedule_launch(int R, int gamma, const float* c, const double* sps, int mode, const int32_t* cap,
                           int32_t* ell, int32_t* admitted, double* theta_best, void* ws, hipStream_t s) {
  uint64_t* ranked = static_cast<uint64_t*>(ws);
  hipLaunchKernelGGL(schedule_rank, dim3(ceil_div(R * gamma, kRankKeys)), dim3(kRankThreads), 0, s, R, gamma, c,
                     ranked);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, R, gamma, sps, mode, cap, ranked, ell,
                     admitted, theta_best);
  return hipGetLastError();
}

// The allocation-free variant's scratch: the ranked slot keys in a static
// device array instead of a caller workspace.  Every slot key is written by
// schedule_rank before schedule_kernel reads it, so nothing needs clearing.
// Each device holds its own copy until the process ends; host code reaches
// it only through the address hipGetSymbolAddress returns for the current
// device (the array's name is a host-side stand-in, not a device address).
constexpr int kStaticSlots = 8192;
static __device__ __align__(256) uint64_t scratch[kStaticSlots];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<uint64_t*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

// The scratch array's address on the current device, looked up once per
// device (nullptr on failure).
static uint64_t* schedule_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uint64_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = static_cast<uint64_t*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

int schedule_static_slots() { return kStaticSlots; }

hipError_t schedule_launch_static(int R, int gamma, const float* c, const double* sps, int mode, const int32_t* cap,
                                  int32_t* ell, int32_t* admitted, double* theta_best, hipStream_t s) {
  if (static_cast<int64_t>(R) * gamma > kStaticSlots) return hipErrorInvalidValue;
  uint64_t* p = schedule_scratch();
  if (!p) return hipErrorInvalidSymbol;
  return schedule_launch(R, gamma, c, sps, mode, cap, ell, admitted, theta_best, p, s);
}

}  // namespace dspark
