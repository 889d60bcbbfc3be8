// The sampler's per-position argmax keys: each work group merges its best
// (perturbed score, token) of a position into a request's 64-bit key slot
// with an atomic max; the largest key over the slots is the drawn token.
#pragma once
#include "common.hpp"

namespace dspark {

// Argmax key slots per (position, request); work group b uses slot
// b % slots.  Fewer slots mean more atomics per address, more slots more
// reads after the barrier.  The kernels with one grid barrier per position
// use four (measured faster than one, two, eight or sixteen); the one with
// a barrier per request block measured the same with four or eight and
// slower with sixteen.
constexpr int kKeySlots = 4;
constexpr int kPipeKeySlots = 4;
constexpr int kMaxKeySlots = 4;

// Token drawn at position k-1 (or the anchor at k = 0); keys are laid out
// [gamma][slots][R].
__device__ __forceinline__ int previous_token(const unsigned long long* keys, int slots, const int32_t* x0, int R,
                                              int V, int k, int req) {
  if (k == 0) return token_or_none(x0[req], V);
  unsigned long long best = 0;
  const unsigned long long* kp = keys + static_cast<int64_t>(k - 1) * slots * R + req;
  for (int s = 0; s < slots; ++s) {
    const unsigned long long v = kp[static_cast<int64_t>(s) * R];
    best = v > best ? v : best;
  }
  return token_or_none(key_token(best), V);
}

}  // namespace dspark
