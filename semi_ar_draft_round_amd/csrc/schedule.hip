// dspark_schedule: the hardware-aware prefix scheduler (Algorithm 1), batched.
//
// Passage: DSpark reading notes, "hardware-aware prefix scheduler":
// Algorithm 1 steps 1-6, Lemma 1 (prefix closure of the ranked pool) and the
// causal early stop; caijizhuo summary, sections 三 and 四 (admit).
//
// One work group of 1024 threads, all data in LDS:
//   1. survival a_{r,j} as the fp64 left-to-right product of the fp32
//      confidences, quantised to a_fx = floor(a * 2^50) (one thread per
//      request);
//   2. ranking: each slot gets a 64-bit key ((2^50 - a_fx) << 13) | (r*gamma + j)
//      so that ascending keys are descending a_fx, then ascending request,
//      then ascending position, and the keys are sorted by a bitonic network;
//      slots with a_fx = 0 sort after every candidate;
//   3. tau_fx(m) = R 2^50 + the exact integer prefix sum of the ranked a_fx;
//   4. the first m with Theta(m) <= Theta(m-1) (exact comparison of
//      tau_fx(m) * SPS(R+m) with tau_fx(m-1) * SPS(R+m-1)) gives A = m - 1;
//   5. l_r = number of request r's slots ranked before position A.
// Every step is integer or exact, so the result does not depend on the order
// in which threads add things up.
#include "common.hpp"

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedMaxSlots = 8192;    // keys in LDS: 8192 * 8 bytes = 64 KiB
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

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(int R, int gamma, int P,
                                                                 const float* __restrict__ c,
                                                                 const double* __restrict__ sps,
                                                                 int32_t* __restrict__ ell,
                                                                 int32_t* __restrict__ admitted,
                                                                 double* __restrict__ theta_best) {
  extern __shared__ uint64_t keys[];   // P entries; reused for the scan afterwards
  const int tid = threadIdx.x;
  const int n = R * gamma;

  // 1-2: keys in LDS (one thread per request walks its positions in order)
  for (int req = tid; req < R; req += kSchedThreads) {
    double s = 1.0;
    for (int j = 0; j < gamma; ++j) {
      s = s * static_cast<double>(c[static_cast<int64_t>(req) * gamma + j]);
      const uint64_t afx = static_cast<uint64_t>(floor(s * static_cast<double>(kOne)));
      keys[req * gamma + j] = ((kOne - afx) << 13) | static_cast<uint64_t>(req * gamma + j);
    }
  }
  for (int i = n + tid; i < P; i += kSchedThreads) keys[i] = ~0ull;
  __syncthreads();

  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < P; i += kSchedThreads) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const uint64_t a = keys[i], b = keys[ixj];
          const bool up = (i & kk) == 0;
          if ((a > b) == up) {
            keys[i] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }

  // 3: thread t owns ranked positions [t*8, t*8+8)
  constexpr int kPer = kSchedMaxSlots / kSchedThreads;   // 8
  const uint64_t cand_limit = kOne << 13;                // keys below are candidates
  uint64_t myk[kPer];
  uint64_t local = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int p = tid * kPer + t;
    myk[t] = (p < P) ? keys[p] : ~0ull;
    if (myk[t] < cand_limit) local += kOne - (myk[t] >> 13);
  }
  __syncthreads();                     // keys now live in registers
  uint64_t* part = keys;               // kSchedThreads entries
  int* sh = reinterpret_cast<int*>(keys + kSchedThreads);   // scalars
  part[tid] = local;
  if (tid == 0) {
    sh[0] = 0x7FFFFFFF;                // first drop position m
    sh[1] = 0;                         // candidate count M
  }
  __syncthreads();
  for (int o = 1; o < kSchedThreads; o <<= 1) {     // inclusive scan of the partials
    const uint64_t v = (tid >= o) ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  uint64_t tau_prev = static_cast<uint64_t>(R) * kOne + (tid > 0 ? part[tid - 1] : 0);
  int my_first_drop = 0x7FFFFFFF;
  int my_count = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    if (myk[t] >= cand_limit) break;
    ++my_count;
    const int m = tid * kPer + t + 1;               // admitting the m-th ranked slot
    const uint64_t tau = tau_prev + (kOne - (myk[t] >> 13));
    if (my_first_drop == 0x7FFFFFFF &&
        cmp_products(tau, sps[R + m - 1], tau_prev, sps[R + m - 2]) <= 0)
      my_first_drop = m;
    tau_prev = tau;
  }
  if (my_first_drop != 0x7FFFFFFF) atomicMin(&sh[0], my_first_drop);
  if (my_count) atomicAdd(&sh[1], my_count);
  __syncthreads();
  const int M = sh[1];
  const int A = (sh[0] == 0x7FFFFFFF) ? M : sh[0] - 1;
  // threshold key: the first ranked slot that is not admitted
  __syncthreads();
  uint64_t* thr = reinterpret_cast<uint64_t*>(sh + 4);
  if (tid == A / kPer) {
    uint64_t v = ~0ull;
#pragma unroll
    for (int t = 0; t < kPer; ++t)
      if (tid * kPer + t == A) v = myk[t];
    thr[0] = v;
    thr[1] = static_cast<uint64_t>(R) * kOne + (tid > 0 ? part[tid - 1] : 0);
    uint64_t tauA = thr[1];
#pragma unroll
    for (int t = 0; t < kPer; ++t)
      if (tid * kPer + t < A) tauA += kOne - (myk[t] >> 13);
    thr[1] = tauA;
  }
  if (A == kSchedThreads * kPer && tid == 0) {   // every slot admitted (P = 8192)
    thr[0] = ~0ull;
    thr[1] = static_cast<uint64_t>(R) * kOne + part[kSchedThreads - 1];
  }
  __syncthreads();
  const uint64_t threshold = thr[0];

  // 5: lengths by recount (the ranked prefix is prefix-closed per request)
  for (int req = tid; req < R; req += kSchedThreads) {
    double s = 1.0;
    int cnt = 0;
    for (int j = 0; j < gamma; ++j) {
      s = s * static_cast<double>(c[static_cast<int64_t>(req) * gamma + j]);
      const uint64_t afx = static_cast<uint64_t>(floor(s * static_cast<double>(kOne)));
      const uint64_t key = ((kOne - afx) << 13) | static_cast<uint64_t>(req * gamma + j);
      if (afx > 0 && key < threshold) ++cnt;
    }
    ell[req] = cnt;
  }
  if (tid == 0) {
    if (admitted) admitted[0] = A;
    if (theta_best) theta_best[0] = static_cast<double>(thr[1]) * 0x1p-50 * sps[R + A - 1];
  }
}

size_t schedule_workspace_bytes() { return 0; }

int schedule_pow2(int n) {
  int P = 1;
  while (P < n) P <<= 1;
  return P < 2 ? 2 : P;
}

hipError_t schedule_launch(int R, int gamma, const float* c, const double* sps, int32_t* ell,
                           int32_t* admitted, double* theta_best, hipStream_t s) {
  const int P = schedule_pow2(R * gamma);
  // LDS holds max(P keys, 1024 partial sums + scalars)
  size_t lds = static_cast<size_t>(P) * sizeof(uint64_t);
  const size_t need_scan = kSchedThreads * sizeof(uint64_t) + 64;
  if (lds < need_scan) lds = need_scan;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), lds, s, R, gamma, P, c, sps, ell,
                     admitted, theta_best);
  return hipGetLastError();
}

}  // namespace dspark
