// The confidence head on one drafted position, computed by one wave: the
// logit z = w[:d] . h_k + w[d:] . W1[x_{k-1}] (fp32 accumulation, 16-byte
// loads, the hidden-state loads of a lane issued together) and the
// temperature-scaled survival sigmoid(z / T_k) in its overflow-free form.
//
// Passage: DSpark reading notes, eq (7) and the sequential temperature
// scaling paragraph.  Shared by the standalone confidence kernel and the
// sampler's finalize step, so both compute the same sums in the same order.
#pragma once

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

// The hidden-state part of z, split so that a caller can put the first
// batch of its loads in flight together with loads of its own:
// conf_h_issue loads the lane's first kConfBatch pieces of h_k and w[:d],
// conf_h_fold adds them up (then loads and adds any further batches) and
// returns the lane's partial sum.
template <typename Elt>
struct ConfH {
  uint4 hv[kConfBatch], wv[kConfBatch];
};

template <typename Elt>
__device__ __forceinline__ void conf_h_issue(ConfH<Elt>& cb, const typename Elt::T* __restrict__ hrow,
                                             const typename Elt::T* __restrict__ w, int d, int i0) {
  constexpr int N = Vec16<Elt>::N;
#pragma unroll
  for (int b = 0; b < kConfBatch; ++b) {
    const int i = i0 + b * 64 * N;
    if (i < d) {
      cb.hv[b] = *reinterpret_cast<const uint4*>(hrow + i);
      cb.wv[b] = *reinterpret_cast<const uint4*>(w + i);
    }
  }
}

template <typename Elt>
__device__ __forceinline__ float conf_h_fold(ConfH<Elt>& cb, const typename Elt::T* __restrict__ hrow,
                                             const typename Elt::T* __restrict__ w, int d, int lane) {
  constexpr int N = Vec16<Elt>::N;
  float acc = 0.f;
  for (int i0 = lane * N; i0 < d; i0 += 64 * N * kConfBatch) {
    if (i0 != lane * N) conf_h_issue<Elt>(cb, hrow, w, d, i0);   // batches after the first
#pragma unroll
    for (int b = 0; b < kConfBatch; ++b) {
      if (i0 + b * 64 * N < d) {
        float va[N], vb[N];
        Vec16<Elt>::load(reinterpret_cast<const typename Elt::T*>(&cb.hv[b]), va);
        Vec16<Elt>::load(reinterpret_cast<const typename Elt::T*>(&cb.wv[b]), vb);
#pragma unroll
        for (int t = 0; t < N; ++t) acc = fmaf(va[t], vb[t], acc);
      }
    }
  }
  return acc;
}

// z from the lane's hidden-state partial: adds the previous token's part
// (prev in [0, V), or -1 for none) and reduces over the wave (the same value
// in every lane).
template <typename Elt>
__device__ __forceinline__ float conf_finish(float hacc, const typename Elt::T* __restrict__ w, int d,
                                             const typename Elt::T* __restrict__ W1, int r, int prev, int lane) {
  if (prev >= 0) hacc += dot_stride<Elt>(W1 + static_cast<int64_t>(prev) * r, w + d, r, lane);
  return wave_reduce_sum(hacc);
}

// z of one position (the same value in every lane).  prev is the previous
// token, already checked to lie in [0, V), or -1 for none (no W1 part).
template <typename Elt>
__device__ __forceinline__ float confidence_logit(const typename Elt::T* __restrict__ hrow,
                                                  const typename Elt::T* __restrict__ w, int d,
                                                  const typename Elt::T* __restrict__ W1, int r, int prev,
                                                  int lane) {
  ConfH<Elt> cb;
  conf_h_issue<Elt>(cb, hrow, w, d, lane * Vec16<Elt>::N);
  return conf_finish<Elt>(conf_h_fold<Elt>(cb, hrow, w, d, lane), w, d, W1, r, prev, lane);
}

// sigmoid(t) without overflow for either sign of t
__device__ __forceinline__ float sigmoid_stable(float t) {
  if (t >= 0.f) return 1.f / (1.f + expf(-t));
  const float e = expf(t);
  return e / (1.f + e);
}

}  // namespace dspark
