// Device helpers shared by the DSpark kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr int kWave = 64;
constexpr int kChunk = 64;              // vocabulary tile of the kernels (MFMA M extent)
constexpr int kGChunk = DSPARK_CHUNK;   // tokens per chunk of the two-level Gumbel draw
static_assert(kChunk % kGChunk == 0, "a tile holds whole Gumbel chunks");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native vectors (not HIP's struct vector types): copies of these stay in
// registers instead of becoming memcpy through private memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Element type tags: storage is either fp32 or bf16 (as raw 16-bit words).
struct F32 {
  typedef float T;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return p[i]; }
};
struct BF16 {
  typedef uint16_t T;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return bf16_to_f32(p[i]); }
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Round-to-nearest-even of an fp32 value to its bf16 bit pattern.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Online log-sum-exp state: value = M + log(S).
struct Lse {
  float M, S;
};
__device__ __forceinline__ Lse lse_combine(Lse a, Lse b) {
  if (b.M == neg_inf() || b.S == 0.f) return a;
  if (a.M == neg_inf() || a.S == 0.f) return b;
  float M = fmaxf(a.M, b.M);
  return Lse{M, a.S * __expf(a.M - M) + b.S * __expf(b.M - M)};
}

// Argmax state for the Gumbel draw: highest score wins, lower token on ties.
struct Best {
  float score;
  int tok;
  float logit;
};
__device__ __forceinline__ bool better(float s1, int t1, float s2, int t2) {
  return s1 > s2 || (s1 == s2 && t1 < t2);
}
__device__ __forceinline__ Best best_combine(Best a, Best b) {
  return better(b.score, b.tok, a.score, a.tok) ? b : a;
}

// The Gumbel argmax of one drafted position is merged across work groups
// with 64-bit atomic max on a packed key: the score's bits mapped to an
// unsigned integer with the same order in the high word, and 0xFFFFFFFF - tok
// in the low word, so a larger key is a higher score or, on equal scores, a
// lower token.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ unsigned long long pack_key(float score, int tok) {
  return (static_cast<unsigned long long>(ordered_bits(score)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(tok));
}
// A token read from device memory that indexes a table: anything outside
// [0, V) is treated as "no token" (-1) so a bad input cannot address memory
// outside the table.
__device__ __forceinline__ int token_or_none(int t, int V) { return (t >= 0 && t < V) ? t : -1; }

__device__ __forceinline__ int key_token(unsigned long long key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFull));
}

// The value held by the lane 32 positions away (lane l and lane l ^ 32),
// with v_permlane32_swap: a vector permute, no LDS round trip.  The swap
// exchanges the upper half of its first operand with the lower half of its
// second, so with both operands x the first result holds x[l - 32] in the
// upper lanes and the second x[l + 32] in the lower lanes.
__device__ __forceinline__ uint32_t xor32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float xor32(float x) { return __uint_as_float(xor32(__float_as_uint(x))); }
__device__ __forceinline__ unsigned long long xor32(unsigned long long x) {
  return (static_cast<unsigned long long>(xor32(static_cast<uint32_t>(x >> 32))) << 32) |
         xor32(static_cast<uint32_t>(x));
}

__device__ __forceinline__ float wave_reduce_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_reduce_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ Lse wave_reduce_lse(Lse a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Lse b{__shfl_xor(a.M, o), __shfl_xor(a.S, o)};
    a = lse_combine(a, b);
  }
  return a;
}
__device__ __forceinline__ Best wave_reduce_best(Best a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Best b{__shfl_xor(a.score, o), __shfl_xor(a.tok, o), __shfl_xor(a.logit, o)};
    a = best_combine(a, b);
  }
  return a;
}

// Inclusive prefix sum over the 64 lanes of a wave (fixed order).
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    float t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__host__ __device__ inline int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

}  // namespace dspark
