// The Markov-head bias on matrix cores: B[req][v] = W1[prev_req] . W2t[v]
// for one 64-token chunk of the vocabulary and up to 16*NBW requests per
// wave, with bf16 inputs and fp32 accumulation (v_mfma_f32_16x16x32_bf16).
//
// Shape of the contraction (notes eq (5); cost eq (15)): M = 64 vocabulary
// rows of W2t (the chunk), N = requests, K = r.  The W2t rows of the chunk
// are one contiguous block of 64 * r bf16 in HBM; a work group copies it to
// LDS once with coalesced 16-byte loads and all of its waves read their A
// fragments from there.  Each wave keeps the W1 rows of its requests (the B
// operand) in registers for the whole launch, because they do not change
// along the vocabulary.
//
// Lane layout of the 16x16x32 bf16 MFMA, lane = 16*q + j:
//   A (16 x 32)  lane holds row j, k = 8q .. 8q+7
//   B (32 x 16)  lane holds column j, k = 8q .. 8q+7
//   D (16 x 16)  lane holds rows 4q .. 4q+3 of column j
// With A = W2t rows and B = W1 rows, lane (q, j) of M-block mb ends up with
// the bias of request j for tokens v0 + 16 mb + 4q + {0,1,2,3}: sixteen
// tokens of one chunk per lane, four lanes (q = 0..3) per request.
#pragma once

#include "common.hpp"

namespace dspark {

constexpr int kTileWaves = 4;
constexpr int kTileThreads = kTileWaves * kWave;   // 256
constexpr int kMaxKSteps = 8;                       // r <= 256

// LDS row stride of a W2t tile row: r bf16 plus 16 bytes of padding so the
// sixteen rows read by a quarter wave start in different banks.
__host__ __device__ constexpr int tile_row_bytes(int ks) { return ks * 64 + 16; }
__host__ __device__ constexpr int tile_lds_bytes(int ks) { return kChunk * tile_row_bytes(ks); }

__device__ __forceinline__ bf16x8 load_bf16x8_global(const uint16_t* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

template <int NBW, int KS>
struct WFrags {
  bf16x8 f[NBW][KS];
};

// B operand: the W1 row of each request's previous token (zeros for prev < 0).
template <int NBW, int KS>
__device__ __forceinline__ void load_w1_frags(WFrags<NBW, KS>& e, const uint16_t* W1,
                                              const int (&prev)[NBW]) {
  const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (prev[nb] >= 0) {
        e.f[nb][ks] = load_bf16x8_global(W1 + static_cast<int64_t>(prev[nb]) * (KS * 32) +
                                         ks * 32 + q * 8);
      } else {
        e.f[nb][ks] = bf16x8{};
      }
    }
  }
}

// Copy W2t rows v0 .. v0+63 (zeros past V) into LDS.
template <int KS>
__device__ __forceinline__ void load_w2_tile(uint8_t* lds, const uint16_t* W2t, int V, int v0) {
  constexpr int kPerRow = KS * 4;                 // 16-byte pieces per row
  constexpr int kTotal = kChunk * kPerRow;
#pragma unroll
  for (int t = threadIdx.x; t < kTotal; t += kTileThreads) {
    const int row = t / kPerRow;
    const int c = t % kPerRow;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (v0 + row < V)
      val = *reinterpret_cast<const uint4*>(W2t + static_cast<int64_t>(v0 + row) * (KS * 32) + c * 8);
    *reinterpret_cast<uint4*>(lds + row * tile_row_bytes(KS) + c * 16) = val;
  }
}

// acc[mb][nb][i] = bias of request (nb, j) at token v0 + 16 mb + 4q + i.
template <int NBW, int KS>
__device__ __forceinline__ void bias_tile(f32x4 (&acc)[4][NBW], const uint8_t* lds,
                                          const WFrags<NBW, KS>& e) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int q = lane >> 4;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 a[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      a[mb] = *reinterpret_cast<const bf16x8*>(lds + (mb * 16 + j) * tile_row_bytes(KS) +
                                               (ks * 32 + q * 8) * 2);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], e.f[nb][ks], acc[mb][nb], 0, 0, 0);
  }
}

// Four consecutive bf16 logits of one row starting at token `v` (a multiple
// of 4), as raw words; entries past V read as 0 (the caller masks them).
__device__ __forceinline__ uint2 load_row4(const uint16_t* row, int v, int V, bool vec_ok) {
  if (vec_ok && v + 3 < V) return *reinterpret_cast<const uint2*>(row + v);
  uint16_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (v + i < V) ? row[v + i] : uint16_t(0);
  return make_uint2(w[0] | (uint32_t(w[1]) << 16), w[2] | (uint32_t(w[3]) << 16));
}

__device__ __forceinline__ float word_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float word_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float row4_get(uint2 p, int i) {
  return i == 0 ? word_lo(p.x) : i == 1 ? word_hi(p.x) : i == 2 ? word_lo(p.y) : word_hi(p.y);
}

}  // namespace dspark
