// dspark_confidence: conditional survival of every drafted position.
//
// Passage: DSpark reading notes, eq (7) (c_k = sigmoid(w^T [h_k ; W1[x_{k-1}]]))
// and the sequential temperature scaling paragraph (an order-preserving
// per-position rescaling, applied here as sigmoid(z / T_k)).
//
// One wave per (request, position): a dot product of length d over the
// hidden state plus one of length r over the previous token's W1 row, both
// with 16-byte loads and fp32 accumulation, then a wave reduction.  The
// kernel streams h once, so it is bound by HBM bandwidth: a lane issues the
// loads of up to kConfBatch pieces of the row (and of w) before it uses any,
// so a row costs one round trip to memory rather than one per piece.
#include "common.hpp"

namespace dspark {

template <typename Elt>
struct Vec16;   // sixteen bytes of storage and their elements as floats
template <>
struct Vec16<F32> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float (&o)[4]) {
    float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <>
struct Vec16<BF16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const uint16_t* p, float (&o)[8]) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// Sixteen-byte pieces per lane whose loads are in flight together (a bf16
// row of up to 8192 elements in one batch).
constexpr int kConfBatch = 16;

template <typename Elt>
__device__ __forceinline__ float dot_stride(const typename Elt::T* a, const typename Elt::T* b, int n,
                                            int lane) {
  constexpr int N = Vec16<Elt>::N;
  float acc = 0.f;
  for (int i = lane * N; i < n; i += 64 * N) {
    float va[N], vb[N];
    Vec16<Elt>::load(a + i, va);
    Vec16<Elt>::load(b + i, vb);
#pragma unroll
    for (int t = 0; t < N; ++t) acc = fmaf(va[t], vb[t], acc);
  }
  return acc;
}

template <typename Elt>
__global__ __launch_bounds__(256) void confidence_kernel(int R, int gamma, int d, int r, int V,
                                                         const typename Elt::T* __restrict__ h,
                                                         const typename Elt::T* __restrict__ w,
                                                         const typename Elt::T* __restrict__ W1,
                                                         const int32_t* __restrict__ x0,
                                                         const int32_t* __restrict__ x,
                                                         const float* __restrict__ T,
                                                         float* __restrict__ c, float* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(R) * gamma) return;
  const int req = static_cast<int>(row / gamma);
  const int k = static_cast<int>(row % gamma);
  const int prev_raw = (k == 0) ? x0[req] : x[row - 1];
  constexpr int N = Vec16<Elt>::N;
  const typename Elt::T* hrow = h + row * d;
  float acc = 0.f;
  for (int i0 = lane * N; i0 < d; i0 += 64 * N * kConfBatch) {
    uint4 hv[kConfBatch], wv[kConfBatch];
#pragma unroll
    for (int b = 0; b < kConfBatch; ++b) {
      const int i = i0 + b * 64 * N;
      if (i < d) {
        hv[b] = *reinterpret_cast<const uint4*>(hrow + i);
        wv[b] = *reinterpret_cast<const uint4*>(w + i);
      }
    }
#pragma unroll
    for (int b = 0; b < kConfBatch; ++b) {
      if (i0 + b * 64 * N < d) {
        float va[N], vb[N];
        Vec16<Elt>::load(reinterpret_cast<const typename Elt::T*>(&hv[b]), va);
        Vec16<Elt>::load(reinterpret_cast<const typename Elt::T*>(&wv[b]), vb);
#pragma unroll
        for (int t = 0; t < N; ++t) acc = fmaf(va[t], vb[t], acc);
      }
    }
  }
  const int prev = token_or_none(prev_raw, V);
  if (prev >= 0) acc += dot_stride<Elt>(W1 + static_cast<int64_t>(prev) * r, w + d, r, lane);
  const float zz = wave_reduce_sum(acc);
  if (lane == 0) {
    const float t = zz / (T ? T[k] : 1.f);
    float cc;
    if (t >= 0.f) {
      cc = 1.f / (1.f + expf(-t));
    } else {
      const float e = expf(t);
      cc = e / (1.f + e);
    }
    c[row] = cc;
    if (z) z[row] = zz;
  }
}

hipError_t confidence_launch(dspark_dtype dt, int R, int gamma, int d, int r, int V, const void* h,
                             const void* w, const void* W1, const int32_t* x0, const int32_t* x,
                             const float* T, float* c, float* z, hipStream_t s) {
  const int blocks = ceil_div(static_cast<int64_t>(R) * gamma, 4);
  if (dt == DSPARK_BF16) {
    hipLaunchKernelGGL(confidence_kernel<BF16>, dim3(blocks), dim3(256), 0, s, R, gamma, d, r, V,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w),
                       static_cast<const uint16_t*>(W1), x0, x, T, c, z);
  } else {
    hipLaunchKernelGGL(confidence_kernel<F32>, dim3(blocks), dim3(256), 0, s, R, gamma, d, r, V,
                       static_cast<const float*>(h), static_cast<const float*>(w),
                       static_cast<const float*>(W1), x0, x, T, c, z);
  }
  return hipGetLastError();
}

}  // namespace dspark
