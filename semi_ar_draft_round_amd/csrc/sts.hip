// Sequential temperature scaling (DSpark reading notes, "sequential
// temperature scaling (STS)" and the per-position reliability table): for
// every drafted position k in order, the grid temperature T_k that minimises
// the ECE of the cumulative product a_k = a_{k-1} sigmoid(z_k / T_k) against
// prefix survival y_k = [n_acc >= k] (1-based k), earlier positions fixed;
// with the ECE of the raw chain (every T = 1) and the per-position ROC-AUC
// of the raw confidence among the rollouts that reached the position.
//
// Per position: a fill kernel clears the bin sums; sts_bins evaluates every
// grid temperature (and the raw chain) for every rollout and adds y - p in
// fixed point (units of 2^-32, int64) into LDS bins, then into global ones
// -- integer sums, so the result does not depend on the order of addition;
// sts_select turns the sums into ECEs and takes the first minimum; sts_update
// advances both chains; sts_auc counts, over every (accepted, rejected)
// pair of rollouts that reached the position, 2 for a higher logit of the
// accepted one and 1 for a tie (exact 64-bit integer counts).  The AUC is
// taken on the logits: the sigmoid is strictly increasing, so the order is
// the same, without the ties that rounding the sigmoid to fp32 would add.
#include "common.hpp"

namespace dspark {

constexpr int kStsThreads = 256;
constexpr int kStsMaxGrid = 256;
constexpr int kStsMaxBins = 32;
constexpr double kStsUnit = 4294967296.0;   // 2^32 fixed-point units per probability

struct StsWs {
  float* a;                 // [N] calibrated chain
  float* a_raw;             // [N] raw chain (T = 1)
  long long* bins;          // [(G + 1) * M] sums of y - p, 2^-32 units; row G is the raw chain
  int* best;                // [1] index of the chosen temperature
  unsigned long long* pairs;  // [gamma][3]: 2 * (wins) + ties, accepted count, rejected count
};

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.f / (1.f + expf(-x)); }

__global__ __launch_bounds__(kStsThreads) void sts_init(int N, int gamma, float* __restrict__ a,
                                                        float* __restrict__ a_raw,
                                                        unsigned long long* __restrict__ pairs) {
  const int i = blockIdx.x * kStsThreads + threadIdx.x;
  if (i < N) {
    a[i] = 1.f;
    a_raw[i] = 1.f;
  }
  if (i < 3 * gamma) pairs[i] = 0ull;
}

__global__ __launch_bounds__(kStsThreads) void sts_clear(int n, long long* __restrict__ bins) {
  const int i = blockIdx.x * kStsThreads + threadIdx.x;
  if (i < n) bins[i] = 0;
}

__global__ __launch_bounds__(kStsThreads) void sts_bins(int N, int gamma, int k, const float* __restrict__ z,
                                                        const int32_t* __restrict__ n_acc,
                                                        const float* __restrict__ grid, int G, int M,
                                                        const float* __restrict__ a,
                                                        const float* __restrict__ a_raw,
                                                        long long* __restrict__ bins) {
  __shared__ long long sb[(kStsMaxGrid + 1) * kStsMaxBins];
  __shared__ float sg[kStsMaxGrid];
  const int nb = (G + 1) * M;
  for (int i = threadIdx.x; i < nb; i += kStsThreads) sb[i] = 0;
  for (int i = threadIdx.x; i < G; i += kStsThreads) sg[i] = grid[i];
  __syncthreads();
  for (int n = blockIdx.x * kStsThreads + threadIdx.x; n < N; n += gridDim.x * kStsThreads) {
    const float x = z[static_cast<int64_t>(n) * gamma + k];
    const long long yv = n_acc[n] >= k + 1 ? (1ll << 32) : 0ll;
    const float ap = a[n];
    for (int t = 0; t <= G; ++t) {
      const float p = t < G ? ap * sigmoid_f32(x / sg[t]) : a_raw[n] * sigmoid_f32(x);
      const int b = min(static_cast<int>(floor(static_cast<double>(p) * M)), M - 1);
      const long long pv = static_cast<long long>(static_cast<double>(p) * kStsUnit);   // p < 2^32 units
      atomicAdd(reinterpret_cast<unsigned long long*>(&sb[t * M + b]), static_cast<unsigned long long>(yv - pv));
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += kStsThreads)
    if (sb[i] != 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(&bins[i]), static_cast<unsigned long long>(sb[i]));
}

// One wave: the ECE of each grid temperature (lanes in turn), the first
// minimum, and the raw chain's ECE.
__global__ __launch_bounds__(64) void sts_select(int N, int k, const float* __restrict__ grid, int G, int M,
                                                 const long long* __restrict__ bins, int* __restrict__ best,
                                                 float* __restrict__ T, double* __restrict__ ece_before,
                                                 double* __restrict__ ece_after) {
  const int lane = threadIdx.x;
  const double scale = 1.0 / (kStsUnit * static_cast<double>(N));
  auto ece_of = [&](int t) {
    double e = 0.0;
    for (int b = 0; b < M; ++b) e += fabs(static_cast<double>(bins[t * M + b]));
    return e * scale;
  };
  double bv = __builtin_inf();
  int bi = 0x7FFFFFFF;
  for (int t = lane; t < G; t += 64) {
    const double e = ece_of(t);
    if (e < bv) {
      bv = e;
      bi = t;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov < bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    best[0] = bi;
    T[k] = grid[bi];
    ece_after[k] = bv;
    ece_before[k] = ece_of(G);
  }
}

__global__ __launch_bounds__(kStsThreads) void sts_update(int N, int gamma, int k, const float* __restrict__ z,
                                                          const float* __restrict__ grid,
                                                          const int* __restrict__ best, float* __restrict__ a,
                                                          float* __restrict__ a_raw) {
  const int n = blockIdx.x * kStsThreads + threadIdx.x;
  if (n >= N) return;
  const float x = z[static_cast<int64_t>(n) * gamma + k];
  a[n] = a[n] * sigmoid_f32(x / grid[best[0]]);
  a_raw[n] = a_raw[n] * sigmoid_f32(x);
}

// Pair counts for the AUC of position k.  Thread = one rollout i of
// blockIdx.x's range (counted when accepted at k); blockIdx.y takes one
// chunk of the rollouts j, staged through LDS a tile at a time with the
// logit of a rollout that was not rejected at k replaced by NaN (it then
// compares false both ways).  Both must have reached k (n_acc >= k, 0-based).
constexpr int kStsAucChunks = 8;

__global__ __launch_bounds__(kStsThreads) void sts_auc(int N, int gamma, int k, const float* __restrict__ z,
                                                       const int32_t* __restrict__ n_acc,
                                                       unsigned long long* __restrict__ pairs) {
  __shared__ __attribute__((aligned(16))) float sz[kStsThreads];
  __shared__ unsigned long long red[kStsThreads / kWave][3];
  const int i = blockIdx.x * kStsThreads + threadIdx.x;
  const bool pos = i < N && n_acc[i] >= k + 1;
  const float zi = i < N ? z[static_cast<int64_t>(i) * gamma + k] : 0.f;
  const int per = ceil_div(ceil_div(N, kStsThreads), kStsAucChunks) * kStsThreads;
  const int j_lo = blockIdx.y * per, j_hi = min(N, j_lo + per);
  unsigned long long cnt = 0, negs = 0;
  for (int j0 = j_lo; j0 < j_hi; j0 += kStsThreads) {
    const int j = j0 + threadIdx.x;
    const bool neg = j < j_hi && n_acc[j] == k;
    sz[threadIdx.x] = neg ? z[static_cast<int64_t>(j) * gamma + k] : __builtin_nanf("");
    negs += (blockIdx.x == 0 && neg) ? 1ull : 0ull;
    __syncthreads();
    if (pos) {
      unsigned int c = 0;
      const float4* s4 = reinterpret_cast<const float4*>(sz);
#pragma unroll 4
      for (int q = 0; q < kStsThreads / 4; ++q) {
        const float4 v = s4[q];
        c += (zi > v.x ? 2u : 0u) + (zi == v.x ? 1u : 0u);
        c += (zi > v.y ? 2u : 0u) + (zi == v.y ? 1u : 0u);
        c += (zi > v.z ? 2u : 0u) + (zi == v.z ? 1u : 0u);
        c += (zi > v.w ? 2u : 0u) + (zi == v.w ? 1u : 0u);
      }
      cnt += c;
    }
    __syncthreads();
  }
  // the block's totals: pair count, accepted rollouts (first chunk only),
  // rejected rollouts (first block column only)
  unsigned long long v[3] = {cnt, (pos && blockIdx.y == 0) ? 1ull : 0ull, negs};
#pragma unroll
  for (int e = 0; e < 3; ++e)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v[e] += __shfl_xor(v[e], o);
  if ((threadIdx.x & 63) == 0)
    for (int e = 0; e < 3; ++e) red[threadIdx.x >> 6][e] = v[e];
  __syncthreads();
  if (threadIdx.x < 3) {
    unsigned long long t = 0;
    for (int w = 0; w < kStsThreads / kWave; ++w) t += red[w][threadIdx.x];
    if (t) atomicAdd(pairs + 3 * k + threadIdx.x, t);
  }
}

__global__ __launch_bounds__(64) void sts_auc_finish(int gamma, const unsigned long long* __restrict__ pairs,
                                                     double* __restrict__ auc) {
  const int k = threadIdx.x;
  if (k >= gamma) return;
  const unsigned long long p = pairs[3 * k + 1], n = pairs[3 * k + 2];
  auc[k] = (p == 0 || n == 0) ? __builtin_nan("")
                              : static_cast<double>(pairs[3 * k]) / (2.0 * static_cast<double>(p) * static_cast<double>(n));
}

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t sts_workspace_bytes(int N, int gamma, int G, int M) {
  return 2 * align256(sizeof(float) * N) + align256(sizeof(long long) * (G + 1) * M) + align256(sizeof(int)) +
         align256(sizeof(unsigned long long) * 3 * gamma);
}

bool sts_shape_ok(int N, int gamma, int G, int M) {
  return N >= 1 && N <= (1 << 20) && gamma >= 1 && gamma <= 64 && G >= 1 && G <= kStsMaxGrid && M >= 1 &&
         M <= kStsMaxBins;
}

hipError_t sts_launch(int N, int gamma, const float* z, const int32_t* n_acc, const float* grid, int G, int M,
                      float* T, double* ece_before, double* ece_after, double* auc, void* ws, hipStream_t s) {
  char* p = static_cast<char*>(ws);
  StsWs w;
  w.a = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * N);
  w.a_raw = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * N);
  w.bins = reinterpret_cast<long long*>(p);
  p += align256(sizeof(long long) * (G + 1) * M);
  w.best = reinterpret_cast<int*>(p);
  p += align256(sizeof(int));
  w.pairs = reinterpret_cast<unsigned long long*>(p);
  const int blocksN = ceil_div(N, kStsThreads);
  const int nbins = (G + 1) * M;
  hipLaunchKernelGGL(sts_init, dim3(ceil_div(N > 3 * gamma ? N : 3 * gamma, kStsThreads)), dim3(kStsThreads), 0, s, N,
                     gamma, w.a, w.a_raw, w.pairs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int blocksB = blocksN < 1024 ? blocksN : 1024;
  for (int k = 0; k < gamma; ++k) {
    hipLaunchKernelGGL(sts_clear, dim3(ceil_div(nbins, kStsThreads)), dim3(kStsThreads), 0, s, nbins, w.bins);
    hipLaunchKernelGGL(sts_bins, dim3(blocksB), dim3(kStsThreads), 0, s, N, gamma, k, z, n_acc, grid, G, M, w.a,
                       w.a_raw, w.bins);
    hipLaunchKernelGGL(sts_select, dim3(1), dim3(64), 0, s, N, k, grid, G, M, w.bins, w.best, T, ece_before,
                       ece_after);
    hipLaunchKernelGGL(sts_update, dim3(blocksN), dim3(kStsThreads), 0, s, N, gamma, k, z, grid, w.best, w.a,
                       w.a_raw);
    hipLaunchKernelGGL(sts_auc, dim3(blocksN, kStsAucChunks), dim3(kStsThreads), 0, s, N, gamma, k, z, n_acc,
                       w.pairs);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(sts_auc_finish, dim3(1), dim3(64), 0, s, gamma, w.pairs, auc);
  return hipGetLastError();
}

}  // namespace dspark
