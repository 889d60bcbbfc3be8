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
// advances both chains.
//
// The AUC of position k counts, over every (accepted, rejected) pair of
// rollouts that reached k, 2 for a higher logit of the accepted one and 1 for
// a tie (exact 64-bit integer counts).  It is taken on the logits: the
// sigmoid is strictly increasing, so the order is the same, without the ties
// that rounding the sigmoid to fp32 would add.  A rollout is rejected at
// exactly one position (k = n_acc), so the rejected logits of all positions
// form one set of at most N keys (k, logit); sts_auc_sort sorts it in chunks
// and sts_auc_count ranks every accepted logit in each chunk's segment for
// its position (2 below + equal = lower bound + upper bound): O(N log N)
// work per call instead of one test per pair.
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
  unsigned long long* sorted; // [ceil(N / kAucChunk) * kAucChunk] chunk-sorted rejected keys
  int* seg;                   // [ceil(N / kAucChunk)][gamma + 1] segment starts
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

// ------------------------------------------------------------------ AUC

constexpr int kAucThreads = 1024;
constexpr int kAucE = 8;                               // keys per thread in the chunk sort
constexpr int kAucChunk = kAucThreads * kAucE;         // rollouts per sorted chunk (8192)
constexpr int kAucQuery = 2048;                        // rollouts ranked per counting work group

// The logit's order-preserving unsigned image (-0 taken as +0, so the two
// compare equal as floats do); NaN never reaches it.
__device__ __forceinline__ uint32_t logit_key(float x) {
  const uint32_t u = __float_as_uint(x == 0.f ? 0.f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Ascending bitonic sort of keys[0 .. n_pad) in LDS by kAucThreads threads
// (n_pad = kAucThreads E).  Lane l of wave w holds elements w 64 E + l E +
// (0 .. E-1): a partner less than E away is in the same lane, one less than
// 64 E away in the same wave (a shuffle), any other in another wave (through
// keys[] and keys[n_pad ..], alternating, one barrier per such stage).
template <int E>
__device__ void auc_bitonic(unsigned long long* keys) {
  constexpr int n_pad = kAucThreads * E;
  const int lane = threadIdx.x & (kWave - 1);
  const int base = (threadIdx.x / kWave) * kWave * E + lane * E;
  const auto cx = [](unsigned long long a, unsigned long long o, int i, int j, int k) {
    const bool asc = (i & k) == 0, lower = (i & j) == 0;
    return (lower == asc) ? (a < o ? a : o) : (a < o ? o : a);
  };
  unsigned long long v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = keys[base + e];
  __syncthreads();
  int buf = 0;
  for (int k = 2; k <= n_pad; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kWave * E) {
        unsigned long long* b = keys + buf * n_pad;
#pragma unroll
        for (int e = 0; e < E; ++e) b[base + e] = v[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = cx(v[e], b[(base + e) ^ j], base + e, j, k);
        buf ^= 1;
      } else if (j >= E) {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = cx(v[e], __shfl_xor(v[e], j / E), base + e, j, k);
      } else {
        unsigned long long w[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          unsigned long long o = v[e ^ 1];
          if constexpr (E > 2) {
            if (j == 2) o = v[e ^ 2];
          }
          if constexpr (E > 4) {
            if (j == 4) o = v[e ^ 4];
          }
          w[e] = cx(v[e], o, base + e, j, k);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = w[e];
      }
    }
  }
  __syncthreads();   // the last LDS stage's reads are done
#pragma unroll
  for (int e = 0; e < E; ++e) keys[base + e] = v[e];
  __syncthreads();
}

// First index in s[lo, hi) whose key is not below (UPPER: not at or below) key.
template <bool UPPER>
__device__ __forceinline__ int auc_bound(const unsigned long long* s, int lo, int hi, unsigned long long key) {
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const bool left = UPPER ? s[mid] <= key : s[mid] < key;
    if (left)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Chunk c of the rollouts: the rejected logit of each rollout, as the key
// (k << 32) | logit_key (k = n_acc < gamma; rollouts accepted everywhere, or
// with a NaN logit, which compares false both ways, get ~0 and sort last),
// sorted; seg[c][k] = the first sorted index of position k (k = 0..gamma).
__global__ __launch_bounds__(kAucThreads) void sts_auc_sort(int N, int gamma, const float* __restrict__ z,
                                                           const int32_t* __restrict__ n_acc,
                                                           unsigned long long* __restrict__ sorted,
                                                           int* __restrict__ seg) {
  __shared__ unsigned long long sk[2 * kAucChunk];
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kAucChunk;
  for (int i = threadIdx.x; i < kAucChunk; i += kAucThreads) {
    const int64_t n = n0 + i;
    unsigned long long key = ~0ull;
    if (n < N) {
      const int a = n_acc[n];
      if (a >= 0 && a < gamma) {
        const float x = z[n * gamma + a];
        if (x == x) key = (static_cast<unsigned long long>(a) << 32) | logit_key(x);
      }
    }
    sk[i] = key;
  }
  __syncthreads();
  auc_bitonic<kAucE>(sk);
  for (int i = threadIdx.x; i < kAucChunk; i += kAucThreads) sorted[n0 + i] = sk[i];
  if (static_cast<int>(threadIdx.x) <= gamma)
    seg[static_cast<int64_t>(blockIdx.x) * (gamma + 1) + threadIdx.x] =
        auc_bound<false>(sk, 0, kAucChunk, static_cast<unsigned long long>(threadIdx.x) << 32);
}

// Work group (q, c): sorted chunk c in LDS, ranked against by the rollouts
// q kAucQuery .. + kAucQuery - 1.  For every position k, each rollout
// accepted at k (n_acc >= k + 1) with a logit that is not NaN adds lower +
// upper bound of its key in chunk c's segment for k; the work group's sums
// go to pairs[3k] once per wave.  The column c = 0 also counts the accepted
// (pairs[3k + 1]) and rejected (pairs[3k + 2]) rollouts, NaN logits
// included.
__global__ __launch_bounds__(kAucThreads) void sts_auc_count(int N, int gamma, const float* __restrict__ z,
                                                            const int32_t* __restrict__ n_acc,
                                                            const unsigned long long* __restrict__ sorted,
                                                            const int* __restrict__ seg,
                                                            unsigned long long* __restrict__ pairs) {
  __shared__ unsigned long long sk[kAucChunk];
  __shared__ int sseg[65];
  __shared__ unsigned long long acc[64][3];
  const int c = blockIdx.y;
  const int nk = seg[static_cast<int64_t>(c) * (gamma + 1) + gamma];   // keys of this chunk below ~0
  for (int i = threadIdx.x; i < nk; i += kAucThreads) sk[i] = sorted[static_cast<int64_t>(c) * kAucChunk + i];
  if (static_cast<int>(threadIdx.x) <= gamma) sseg[threadIdx.x] = seg[static_cast<int64_t>(c) * (gamma + 1) + threadIdx.x];
  for (int i = threadIdx.x; i < 3 * 64; i += kAucThreads) (&acc[0][0])[i] = 0ull;
  __syncthreads();
  constexpr int kPerThread = kAucQuery / kAucThreads;
  int a[kPerThread];
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * kAucQuery;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int64_t n = q0 + u * kAucThreads + threadIdx.x;
    a[u] = n < N ? n_acc[n] : -1;
  }
  const int lane = threadIdx.x & (kWave - 1);
  for (int k = 0; k < gamma; ++k) {
    unsigned long long cnt = 0;
    const int lo = sseg[k], hi = sseg[k + 1];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      if (a[u] >= k + 1 && hi > lo) {
        const float x = z[(q0 + u * kAucThreads + threadIdx.x) * gamma + k];
        if (x == x) {
          const unsigned long long key = (static_cast<unsigned long long>(k) << 32) | logit_key(x);
          cnt += static_cast<unsigned long long>(auc_bound<false>(sk, lo, hi, key) - lo) +
                 static_cast<unsigned long long>(auc_bound<true>(sk, lo, hi, key) - lo);
        }
      }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0 && cnt) atomicAdd(&acc[k][0], cnt);
    if (c == 0) {
      int np = 0, nn = 0;
#pragma unroll
      for (int u = 0; u < kPerThread; ++u) {
        np += __popcll(__ballot(a[u] >= k + 1));
        nn += __popcll(__ballot(a[u] == k));
      }
      if (lane == 0) {
        if (np) atomicAdd(&acc[k][1], static_cast<unsigned long long>(np));
        if (nn) atomicAdd(&acc[k][2], static_cast<unsigned long long>(nn));
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 3 * gamma; i += kAucThreads) {
    const unsigned long long v = (&acc[0][0])[i];
    if (v) atomicAdd(pairs + i, v);
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

static int auc_chunks(int N) { return ceil_div(N, kAucChunk); }

size_t sts_workspace_bytes(int N, int gamma, int G, int M) {
  return 2 * align256(sizeof(float) * N) + align256(sizeof(long long) * (G + 1) * M) + align256(sizeof(int)) +
         align256(sizeof(unsigned long long) * 3 * gamma) +
         align256(sizeof(unsigned long long) * static_cast<size_t>(auc_chunks(N)) * kAucChunk) +
         align256(sizeof(int) * static_cast<size_t>(auc_chunks(N)) * (gamma + 1));
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
  p += align256(sizeof(unsigned long long) * 3 * gamma);
  w.sorted = reinterpret_cast<unsigned long long*>(p);
  p += align256(sizeof(unsigned long long) * static_cast<size_t>(auc_chunks(N)) * kAucChunk);
  w.seg = reinterpret_cast<int*>(p);
  const int blocksN = ceil_div(N, kStsThreads);
  const int nbins = (G + 1) * M;
  hipLaunchKernelGGL(sts_init, dim3(ceil_div(N > 3 * gamma ? N : 3 * gamma, kStsThreads)), dim3(kStsThreads), 0, s, N,
                     gamma, w.a, w.a_raw, w.pairs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // the AUC needs only the logits and n_acc: both passes run once, up front
  hipLaunchKernelGGL(sts_auc_sort, dim3(auc_chunks(N)), dim3(kAucThreads), 0, s, N, gamma, z, n_acc, w.sorted,
                     w.seg);
  hipLaunchKernelGGL(sts_auc_count, dim3(ceil_div(N, kAucQuery), auc_chunks(N)), dim3(kAucThreads), 0, s, N, gamma,
                     z, n_acc, w.sorted, w.seg, w.pairs);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int blocksB = blocksN < 1024 ? blocksN : 1024;
  for (int k = 0; k < gamma; ++k) {
    hipLaunchKernelGGL(sts_clear, dim3(ceil_div(nbins, kStsThreads)), dim3(kStsThreads), 0, s, nbins, w.bins);
    hipLaunchKernelGGL(sts_bins, dim3(blocksB), dim3(kStsThreads), 0, s, N, gamma, k, z, n_acc, grid, G, M, w.a,
                       w.a_raw, w.bins);
    hipLaunchKernelGGL(sts_select, dim3(1), dim3(64), 0, s, N, k, grid, G, M, w.bins, w.best, T, ece_before,
                       ece_after);
    hipLaunchKernelGGL(sts_update, dim3(blocksN), dim3(kStsThreads), 0, s, N, gamma, k, z, grid, w.best, w.a,
                       w.a_raw);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(sts_auc_finish, dim3(1), dim3(64), 0, s, gamma, w.pairs, auc);
  return hipGetLastError();
}

}  // namespace dspark
