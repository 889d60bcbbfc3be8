// The Markov-head bias on matrix cores: B[req][v] = W1[prev_req] . W2t[v]
// for one 64-token chunk of the vocabulary and up to 16*NBW requests per
// wave, with bf16 inputs and fp32 accumulation (v_mfma_f32_16x16x32_bf16).
//
// Shape of the contraction (notes eq (5); cost eq (15)): M = 64 vocabulary
// rows of W2t (the chunk), N = requests, K = r.  The W2t rows of the chunk
// are one contiguous block of 64 * r bf16 in HBM; a work group stages it
// through registers (coalesced 16-byte loads, issued two chunks ahead) into
// an LDS tile, and all of its waves read their A fragments from there.  Each
// wave keeps the W1 rows of its requests (the B operand) in registers for the
// whole launch, because they do not change along the vocabulary.
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

// A W2t tile is the chunk's 64 rows of r bf16 (KS * 4 sixteen-byte pieces
// per row), stored unpadded with the piece index XOR-swizzled by the row:
// piece c of row `row` sits in slot c ^ (row mod pieces-per-row).  The
// sixteen rows one quarter wave reads for an A fragment then fall in
// sixteen different bank groups, and the stores of a tile are conflict-free.
__host__ __device__ constexpr int tile_pieces(int ks) { return ks * 4; }
__host__ __device__ constexpr int tile_bytes(int ks) { return kChunk * ks * 64; }

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

// The same B fragments from one r-vector row per request group (a W1 row,
// or the bias vector of another head); a null row gives zeros.
template <int NBW, int KS>
__device__ __forceinline__ void load_vec_frags(WFrags<NBW, KS>& e, const uint16_t* const (&rows)[NBW]) {
  const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      e.f[nb][ks] = rows[nb] ? load_bf16x8_global(rows[nb] + ks * 32 + q * 8) : bf16x8{};
  }
}

// The W2t tile of one chunk staged in registers: the tile's 64 rows are one
// contiguous block of 64 * r bf16, so thread t takes the 16-byte pieces
// t, t + 256, ... of that block (fully coalesced); rows past V read row V-1
// (their tokens are masked by the caller).
template <int KS>
struct WRegs {
  u32x4 w[KS];
};

template <int KS>
__device__ __forceinline__ void load_w2_regs(WRegs<KS>& wr, const uint16_t* W2t, int V, int v0) {
  constexpr int P = tile_pieces(KS);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int piece = s * kTileThreads + threadIdx.x;
    const int row = piece / P;
    const int c = piece % P;
    const int vrow = min(v0 + row, V - 1);
    wr.w[s] = *reinterpret_cast<const u32x4*>(W2t + static_cast<int64_t>(vrow) * (KS * 32) + c * 8);
  }
}

template <int KS>
__device__ __forceinline__ void store_w2_tile(uint8_t* tile, const WRegs<KS>& wr) {
  constexpr int P = tile_pieces(KS);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int piece = s * kTileThreads + threadIdx.x;
    const int row = piece / P;
    const int slot = (piece % P) ^ (row & (P - 1));
    *reinterpret_cast<u32x4*>(tile + (row * P + slot) * 16) = wr.w[s];
  }
}

// Second tile layout, for kernels where each lane owns sixteen consecutive
// tokens: the tile row of token offset t (0..63) is stored at row
// lane16_row(t), which swaps the bit fields [5:4] and [3:2] of t.  Reading
// stored row 16 mb + j as A row j of M-block mb then gives lane (q, j) the
// tokens 16 q + 4 mb + i (i = 0..3) of the chunk: over the four M-blocks,
// the sixteen consecutive tokens 16 q .. 16 q + 15.
__host__ __device__ constexpr int lane16_row(int t) {
  return (((t >> 2) & 3) << 4) | (((t >> 4) & 3) << 2) | (t & 3);
}

template <int KS>
__device__ __forceinline__ void store_w2_tile_lane16(uint8_t* tile, const WRegs<KS>& wr) {
  constexpr int P = tile_pieces(KS);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int piece = s * kTileThreads + threadIdx.x;
    const int row = lane16_row(piece / P);
    const int slot = (piece % P) ^ (row & (P - 1));
    *reinterpret_cast<u32x4*>(tile + (row * P + slot) * 16) = wr.w[s];
  }
}

// acc[mb][nb] += the bias block of M-block mb for request group nb (the C
// operand comes in through acc).
template <int NBW, int KS>
__device__ __forceinline__ void bias_tile_acc(f32x4 (&acc)[4][NBW], const uint8_t* tile,
                                              const WFrags<NBW, KS>& e) {
  constexpr int P = tile_pieces(KS);
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int q = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 a[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int row = mb * 16 + j;
      const int slot = (ks * 4 + q) ^ (row & (P - 1));
      a[mb] = *reinterpret_cast<const bf16x8*>(tile + (row * P + slot) * 16);
    }
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], e.f[nb][ks], acc[mb][nb], 0, 0, 0);
  }
}

// acc[mb][nb][i] = bias of request (nb, j) at token v0 + 16 mb + 4q + i
// (tile stored by store_w2_tile).
template <int NBW, int KS>
__device__ __forceinline__ void bias_tile(f32x4 (&acc)[4][NBW], const uint8_t* tile,
                                          const WFrags<NBW, KS>& e) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bias_tile_acc<NBW, KS>(acc, tile, e);
}

// Four consecutive bf16 logits of one row starting at token `v` (a multiple
// of 4), as raw words; entries past V read as 0 (the caller masks them).
__device__ __forceinline__ u32x2 load_row4(const uint16_t* row, int v, int V, bool vec_ok) {
  if (vec_ok && v + 3 < V) return *reinterpret_cast<const u32x2*>(row + v);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (v + i < V) ? row[v + i] : 0u;
  return u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
}

// Sixteen logits of one row for this lane (chunk offsets 16 mb + 4q + i).
// VEC (V a multiple of 4): one 8-byte load per M-block; a group of four
// tokens is either wholly inside the row or wholly past V, and groups past V
// re-read the chunk's first group (their tokens are masked by the caller), so
// there is no data-dependent branch.  Otherwise the checked path.
template <bool VEC>
__device__ __forceinline__ void load_lane_logits(u32x2 (&out)[4], const uint16_t* row, int v0, int V, int q) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int v = v0 + mb * 16 + 4 * q;
    if constexpr (VEC)
      out[mb] = *reinterpret_cast<const u32x2*>(row + (v < V ? v : v0));
    else
      out[mb] = load_row4(row, v, V, false);
  }
}

__device__ __forceinline__ float word_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float word_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float row4_get(u32x2 p, int i) {
  return i == 0 ? word_lo(p.x) : i == 1 ? word_hi(p.x) : i == 2 ? word_lo(p.y) : word_hi(p.y);
}

}  // namespace dspark
