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
#include "confidence_row.hpp"

namespace dspark {

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
  const float zz = confidence_logit<Elt>(h + row * d, w, d, W1, r, token_or_none(prev_raw, V), lane);
  if (lane == 0) {
    c[row] = sigmoid_stable(zz / (T ? T[k] : 1.f));
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
