// Pieces shared by the kernels that stream the vocabulary in 64-token tiles
// with one 16-token Gumbel chunk per lane: the -inf and zero rows that stand
// in for out-of-range logits and for a missing previous token, the lane's
// sixteen logits, and the 32x32x16 MFMA tile (W2t rows staged through
// registers into LDS in the permuted, padded layout).
#pragma once

#include "bias_tile.hpp"

namespace dspark {

// Sixteen bf16 -inf words: the logits read for tokens past V, so that they
// drop out of every reduction without a per-element test.
static __device__ u32x4 kNegInfBf16x16[2] = {{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u},
                                            {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u}};

// A W1 row of zeros (r <= 256): the B operand when there is no previous token.
static __device__ __attribute__((aligned(16))) uint16_t kZeroRow[256] = {};

// The bf16 logits of one lane's Gumbel chunk, tokens v .. v + 15 of `row`.
// VEC (V a multiple of 16): the chunk lies wholly inside the row or wholly
// past it; chunks past V read the -inf words.  Otherwise token by token.
template <bool VEC>
__device__ __forceinline__ void load_lane16(u32x4 (&u)[2], const uint16_t* row, int v, int V) {
  if constexpr (VEC) {
    const u32x4* p = v < V ? reinterpret_cast<const u32x4*>(row + v) : kNegInfBf16x16;
    u[0] = p[0];
    u[1] = p[1];
  } else {
    uint32_t w[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t lo = v + 2 * d < V ? row[v + 2 * d] : 0xFF80u;
      const uint32_t hi = v + 2 * d + 1 < V ? row[v + 2 * d + 1] : 0xFF80u;
      w[d] = lo | (hi << 16);
    }
    u[0] = u32x4{w[0], w[1], w[2], w[3]};
    u[1] = u32x4{w[4], w[5], w[6], w[7]};
  }
}

// ---------------------------------------------------------------------------
// Wide path: 32x32x16 MFMAs, two waves per SIMD at 128 requests.
//
// A work group of 2 RQ waves covers 32 RQ requests over 64-token tiles.  Wave
// w takes token half th = w & 1 (tokens 32 th .. 32 th + 31 of the tile) and
// request quarter rq = w >> 1 (requests 32 rq .. 32 rq + 31 of the group).
// Lane (h, j) of the 32x32x16 output holds column j (a request) and rows
// 8 g + 4 h + t (g, t = 0..3).  The tile rows are stored in LDS so that MFMA
// row 8 g + 4 h + t of a half is its token 16 h + 4 g + t: the lane's sixteen
// accumulators are its request's logits for the sixteen consecutive tokens
// v0 + 32 th + 16 h + (0..15), one Gumbel chunk, and every reduction of the
// chunk stays inside the lane.  Each wave reads only its half of the tile
// (16 KB at r = 256) per tile, so the LDS traffic per tile is the same as
// with four waves of 32 requests x 64 tokens, while two waves per SIMD let
// one wave's vector work run under the other's matrix products.

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Stored LDS row of tile row (token offset) t: bits [th h g1 g0 t1 t0] ->
// [th g1 g0 h t1 t0].
__host__ __device__ constexpr int row32_of_token(int t) {
  return (t & 32) | (((t >> 2) & 3) << 3) | (((t >> 4) & 1) << 2) | (t & 3);
}

template <int RQ>
__host__ __device__ constexpr int wide_threads() { return 128 * RQ; }

// The W2t tile (64 rows of r = 16 KS16 bf16) staged in registers: thread t
// takes the 16-byte pieces t, t + T, ... of the tile's contiguous block.
template <int KS16, int RQ>
struct WideW {
  static constexpr int P = 2 * KS16;   // 16-byte pieces per row
  static constexpr int T = wide_threads<RQ>();
  static constexpr int NP = (64 * P + T - 1) / T;
  u32x4 w[NP];
};

template <int KS16, int RQ>
__device__ __forceinline__ void wide_load_w(WideW<KS16, RQ>& st, const uint16_t* W2t, int V, int v0) {
  constexpr int P = WideW<KS16, RQ>::P, T = WideW<KS16, RQ>::T;
#pragma unroll
  for (int n = 0; n < WideW<KS16, RQ>::NP; ++n) {
    const int piece = n * T + static_cast<int>(threadIdx.x);
    if ((64 * P) % T == 0 || piece < 64 * P) {   // only small r leaves threads idle (wave-uniform)
      const int vrow = min(v0 + piece / P, V - 1);
      st.w[n] = *reinterpret_cast<const u32x4*>(W2t + static_cast<int64_t>(vrow) * (KS16 * 16) + (piece % P) * 8);
    }
  }
}

// Rows go to row32_of_token(row), at a stride of P + 1 pieces: the padding
// piece puts the rows one half-wave reads for an A fragment (consecutive
// stored rows, same piece) in different bank groups, and a fragment's
// address is the lane's row base plus a constant offset per k-step.
template <int KS16>
__host__ __device__ constexpr int wide_row_pieces() { return 2 * KS16 + 1; }
template <int KS16>
__host__ __device__ constexpr int wide_tile_bytes() { return 64 * wide_row_pieces<KS16>() * 16; }

template <int KS16, int RQ>
__device__ __forceinline__ void wide_store_w(uint8_t* tile, const WideW<KS16, RQ>& st) {
  constexpr int P = WideW<KS16, RQ>::P, T = WideW<KS16, RQ>::T;
#pragma unroll
  for (int n = 0; n < WideW<KS16, RQ>::NP; ++n) {
    const int piece = n * T + static_cast<int>(threadIdx.x);
    if ((64 * P) % T == 0 || piece < 64 * P) {
      const int srow = row32_of_token(piece / P);
      *reinterpret_cast<u32x4*>(tile + (srow * wide_row_pieces<KS16>() + piece % P) * 16) = st.w[n];
    }
  }
}

}  // namespace dspark
