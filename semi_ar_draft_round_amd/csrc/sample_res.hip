// The Markov-head sampling loop with the bias operand W2t held on chip.
//
// Passage: DSpark reading notes, eq (4) (the bias is added inside the
// softmax) and eq (5) (Markov head B(x_{k-1}, .) = W1[x_{k-1}] W2, rank r);
// caijizhuo section 四, the sequential loop of dspark_cycle.  The draw is the
// exact two-level Gumbel-max of the other sampling kernels (chunk-level
// log-sum-exp plus chunk Gumbel, then the in-chunk argmax).
//
// Every position multiplies the same W2t (V x r) by the previous tokens' W1
// rows.  Streaming W2t from memory at every position costs more than the
// logits themselves at r = 256 (66 MB against 33 MB per position at
// R = 128, V = 129280), so this kernel keeps it on chip instead: one work
// group per compute unit owns a contiguous range of at most eight 64-token
// tiles, and each of its eight waves holds one tile's W2t rows as 32x32x16
// MFMA A fragments for the whole launch (128 registers a lane at r = 256,
// the last four k-steps in LDS; V <= 131072 on 256 compute units).  With a
// single request block (R <= 32) at r = 256, the W1 rows need so little LDS
// that two more tiles per work group fit there whole, taken by waves 0 and
// 1 after their own (V <= 163840).  A position then streams only the logits
// U_k and the chunk Gumbels.  The A fragments are loaded straight from W2t
// at launch: registers for the first k-steps, a copy into LDS (no
// registers) for the rest.
//
// Per position a wave walks the request blocks of 32: the block's logits
// seed the accumulators, the previous tokens' W1 rows (gathered into LDS
// once per position, the B operand) are multiplied in, and each lane folds
// its two 16-token chunks (one per 32-token half of the tile) into the
// request's log-sum-exp and chunk-level Gumbel-max, then draws inside the
// winning chunk.  The waves' results per request merge in LDS, and one
// thread per request merges them into the request's key slot (64-bit atomic
// max) and log-sum-exp partial, as the other sampling kernels do.  The work
// groups then meet at the grid barrier, read the keys back and gather the
// next position's W1 rows.  Logits are loaded two request blocks ahead, so
// the next position's first two blocks are in flight across the barrier.
// At r = 256 the last four k-steps of each wave's A fragments sit in LDS
// (64 KB per work group) to leave registers for those loads.  With a single
// request block the logits are loaded one position ahead instead: one
// register set for the wave's own tile, one for its LDS-held tile.
#include <hip/hip_ext.h>

#include "wide_tile.hpp"
#include "sample_keys.hpp"
#include "sample_common.hpp"

#include <atomic>
#include <type_traits>

namespace dspark {

constexpr int kResWaves = 8;
constexpr int kResThreads = kResWaves * kWave;   // 512

// Data one work group writes and others read within the launch (the RNN
// head's s and o): stored and loaded as agent-scope atomics, which are
// coherent across the dies' L2 caches without a cache write-back; the
// writers' stores have completed before they arrive at the grid barrier
// that the readers wait on.
__device__ __forceinline__ void store32_agent(void* p, uint32_t v) {
  __hip_atomic_store(static_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 load16_agent(const void* p) {
  const unsigned long long* q = static_cast<const unsigned long long*>(p);
  const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32), static_cast<uint32_t>(b),
               static_cast<uint32_t>(b >> 32)};
}

// LDS bytes of one request's W1 row (r = 16 KS16 bf16) plus a 16-byte pad,
// so the rows a half-wave reads for one B fragment fall in different banks.
template <int KS16>
__host__ __device__ constexpr int res_erow_bytes() { return KS16 * 32 + 16; }

// k-steps of each wave's A fragments kept in LDS rather than registers: at
// r = 256 the last four (the registers they free hold a second request
// block of logits in flight)
template <int KS16>
__host__ __device__ constexpr int res_lds_ksteps() { return KS16 >= 16 ? 4 : 0; }

// Tiles a work group can hold: one per wave (registers plus LDS), and at
// r = 256 with a single request block two more held wholly in LDS (one
// block's W1 rows leave room for them), so vocabularies up to 2560 tiles
// (V <= 163840 on 256 compute units) stay on chip for single requests.
template <int RB, int KS16>
__host__ __device__ constexpr int res_max_tiles() { return RB == 1 && KS16 == 16 ? kResWaves + 2 : kResWaves; }

// A request block's logits and chunk Gumbels for one lane: tokens
// 32 tb + 16 h .. + 15 of a tile for tb = 0, 1.
struct ResLane {
  u32x4 u[2][2];
  float G[2];
};

// The RNN head's arguments when the kernel runs it (see rnn_phase below).
struct ResRnn {
  const uint16_t* W;    // [3r][2r + d]: gate, candidate and output rows; columns follow z
  const float* Yh;      // [R gamma][3r]: the hidden-state part of the projection
  int d;
  float* s;             // [R][gamma][r] out: the state after each position
  uint16_t* o;          // [R][gamma][r] out: each position's bias vector
  const float* P;       // [V][3r] or null: W's W1-row columns times every W1 row (dspark_rnn_prepare)
};

// RNN: 0 the Markov head; 1 the RNN head, its step taking z = [s; W1 row]
// on the matrix cores; 2 the RNN head with the W1-row part looked up in P,
// so the step's products cover the state part only.
template <int RB, int KS16, bool VEC, int RNN = 0>
__global__ __launch_bounds__(kResThreads, 1) void sample_steps_res(
    int R, int gamma, int V, const uint16_t* __restrict__ U, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W2t, const int32_t* __restrict__ x0, const float* __restrict__ G,
    const float* __restrict__ g, SampleWs ws, int kb, int ke, const uint32_t* __restrict__ cancel, ResRnn rnn) {
  static_assert(kGChunk == 16 && kChunk == 64, "one Gumbel chunk per lane of a 32x32 output block");
  constexpr int NROWS = 32 * RB;
  constexpr int kE = res_erow_bytes<KS16>();
  constexpr int kMT = res_max_tiles<RB, KS16>();
  constexpr int NX = kMT - kResWaves;            // tiles held wholly in LDS (0 or 2)
  constexpr int KL = res_lds_ksteps<KS16>();     // k-steps of A in LDS
  constexpr int KR = KS16 - KL;                  // k-steps of A in registers
  __shared__ __attribute__((aligned(1024))) uint8_t erows[NROWS * kE];   // the W1 rows (B operand)
  __shared__ float gsh[NROWS][kGChunk];                                  // in-chunk Gumbels of the position
  __shared__ unsigned long long mkey[kMT][NROWS];                        // per-tile results, merged per request
  __shared__ float2 mlse[kMT][NROWS];
  __shared__ __attribute__((aligned(16))) bf16x8 alds[KL > 0 ? kResWaves : 1][2][KL > 0 ? KL : 1][kWave];
  __shared__ __attribute__((aligned(16))) bf16x8 xlds[NX > 0 ? NX : 1][2][NX > 0 ? KS16 : 1][kWave];
  __shared__ int barflag;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 31;
  const int h = lane >> 5;
  const int nTiles = (V + kChunk - 1) / kChunk;
  const int nG = (V + kGChunk - 1) / kGChunk;
  // the group's tiles: a contiguous range of base or base + 1 (<= kMT,
  // checked by the host); wave w owns tile t0 + w, and waves 0 and 1 also
  // tiles t0 + 8 and t0 + 9 when the group has them
  const int gx = static_cast<int>(gridDim.x), bx = static_cast<int>(blockIdx.x);
  const int base = nTiles / gx, rem = nTiles % gx;
  const int nT = base + (bx < rem ? 1 : 0);
  const int t0 = bx * base + min(bx, rem);
  const bool active = wave < nT;
  const int tile = t0 + min(wave, nT - 1);
  const int v0 = tile * kChunk;
  const bool xact = NX > 0 && wave < nT - kResWaves;   // this wave also owns an LDS-held tile
  const int xtile = t0 + kResWaves + min(wave, NX > 0 ? NX - 1 : 0);
  const int xv0 = xtile * kChunk;

  // 1. W2t: the wave's tile as A fragments, the first KR k-steps straight
  // into registers, the rest (and any LDS-held tile) straight into LDS
  bf16x8 A[2][KR > 0 ? KR : 1];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int vrow = min(v0 + token_of_row32(32 * tb + j), V - 1);
    const uint16_t* src = W2t + static_cast<int64_t>(vrow) * (KS16 * 16) + h * 8;
#pragma unroll
    for (int ks = 0; ks < KS16; ++ks) {
      if (ks < KR)
        A[tb][ks < KR ? ks : 0] = *reinterpret_cast<const bf16x8*>(src + ks * 16);
      else
        copy16_to_lds(src + ks * 16, &alds[wave][tb][ks < KR ? 0 : ks - KR][0]);
    }
  }
  if constexpr (NX > 0) {
    if (xact) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int vrow = min(xv0 + token_of_row32(32 * tb + j), V - 1);
        const uint16_t* src = W2t + static_cast<int64_t>(vrow) * (KS16 * 16) + h * 8;
#pragma unroll
        for (int ks = 0; ks < KS16; ++ks) copy16_to_lds(src + ks * 16, &xlds[wave][tb][ks][0]);
      }
    }
  }

  // 2. the W1 rows of the previous tokens (the B operand) for position k:
  // the anchors at the first position, else the tokens drawn at k - 1
  constexpr int TPR = kResThreads / NROWS;   // threads per row
  constexpr int PPR = 2 * KS16;              // 16-byte pieces per row
  auto gather_e = [&](int k, bool first) {
    const int i = static_cast<int>(threadIdx.x) / TPR;
    const int part = static_cast<int>(threadIdx.x) % TPR;
    if constexpr (RNN) {   // the head's bias vectors o_k in the W1 rows' place (written this launch)
      const uint16_t* src = i < R ? rnn.o + (static_cast<int64_t>(i) * gamma + k) * (KS16 * 16) : kZeroRow;
#pragma unroll
      for (int p = part; p < PPR; p += TPR)
        *reinterpret_cast<u32x4*>(erows + i * kE + p * 16) = load16_agent(src + p * 8);
      return;
    }
    int prev = -1;
    if (i < R) {
      if (first) {
        prev = token_or_none(x0[i], V);
      } else {
        const unsigned long long* kp = ws.keys + static_cast<int64_t>(k - 1) * kKeySlots * R + i;
        unsigned long long best = 0;
#pragma unroll
        for (int sl = 0; sl < kKeySlots; ++sl) {
          const unsigned long long v =
              __hip_atomic_load(kp + static_cast<int64_t>(sl) * R, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          best = v > best ? v : best;
        }
        prev = token_or_none(key_token(best), V);
      }
    }
    const uint16_t* src = prev >= 0 ? W1 + static_cast<int64_t>(prev) * (KS16 * 16) : kZeroRow;
#pragma unroll
    for (int p = part; p < PPR; p += TPR)
      *reinterpret_cast<u32x4*>(erows + i * kE + p * 16) = *reinterpret_cast<const u32x4*>(src + p * 8);
  };
  // the in-chunk Gumbels of position k: four floats per thread
  auto load_gq = [&](int k) {
    const int i = static_cast<int>(threadIdx.x) >> 2, q = static_cast<int>(threadIdx.x) & 3;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (i < NROWS) v = *reinterpret_cast<const f32x4*>(g + (static_cast<int64_t>(min(i, R - 1)) * gamma + k) * kGChunk + 4 * q);
    return v;
  };
  auto store_gq = [&](f32x4 v) {
    const int i = static_cast<int>(threadIdx.x) >> 2, q = static_cast<int>(threadIdx.x) & 3;
    if (i < NROWS) *reinterpret_cast<f32x4*>(&gsh[i][4 * q]) = v;
  };

  // logits and chunk Gumbels of request block rb at position k for this
  // lane, tile starting at token vt
  auto load_at = [&](ResLane& p, int k, int rb, int vt) {
    const int reqc = min(32 * rb + j, R - 1);
    const uint16_t* row = U + (static_cast<int64_t>(reqc) * gamma + k) * V;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      // the -inf stand-in is picked by address, not by value, so the loads
      // stay in flight until the step that uses them
      load_lane16<VEC>(p.u[tb], row, vt + 32 * tb + 16 * h, V);
      p.G[tb] = G[(static_cast<int64_t>(k) * nG + min(vt / kGChunk + 2 * tb + h, nG - 1)) * R + reqc];
    }
  };
  // step s = k * RB + rb (request block rb of position k), the wave's own tile
  auto load_step = [&](ResLane& p, int s) { load_at(p, s / RB, s % RB, v0); };

  // the products of one request block and tile: the logits seed the
  // accumulators and the bias is added on the matrix cores (A from
  // registers and alds, or all from xlds for an LDS-held tile)
  auto products = [&](const ResLane& cur, int rb, f32x16& acc0, f32x16& acc1, auto from_xlds) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t w0 = cur.u[0][q >> 3][(q >> 1) & 3];
      const uint32_t w1 = cur.u[1][q >> 3][(q >> 1) & 3];
      acc0[q] = __uint_as_float((q & 1) ? (w0 & 0xFFFF0000u) : (w0 << 16));
      acc1[q] = __uint_as_float((q & 1) ? (w1 & 0xFFFF0000u) : (w1 << 16));
    }
    const uint8_t* erow = erows + (32 * rb + j) * kE + h * 16;
    // B fragments two k-steps ahead of their products; the empty asm
    // with a memory clobber keeps the compiler from hoisting every read
    // of the chain to the top, which would cost KS16 x 4 registers
    if constexpr (KS16 >= 8) __builtin_amdgcn_iglp_opt(1);   // interleave the products with the vector work
    bf16x8 bc = *reinterpret_cast<const bf16x8*>(erow);
    bf16x8 bn = KS16 > 1 ? *reinterpret_cast<const bf16x8*>(erow + 32) : bc;
#pragma unroll
    for (int ks = 0; ks < KS16; ++ks) {
      const bf16x8 bnn = ks + 2 < KS16 ? *reinterpret_cast<const bf16x8*>(erow + (ks + 2) * 32) : bn;
      if constexpr (decltype(from_xlds)::value) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xlds[wave][0][ks][lane], bc, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xlds[wave][1][ks][lane], bc, acc1, 0, 0, 0);
      } else if (ks < KR) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[0][ks < KR ? ks : 0], bc, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[1][ks < KR ? ks : 0], bc, acc1, 0, 0, 0);
      } else {
        const int kl = ks < KR ? 0 : ks - KR;
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alds[wave][0][kl][lane], bc, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alds[wave][1][kl][lane], bc, acc1, 0, 0, 0);
      }
      asm volatile("" ::: "memory");
      bc = bn;
      bn = bnn;
    }
  };
  // the lane's two chunks (tokens vt + 16 h and vt + 32 + 16 h onwards), the
  // in-chunk draw on the one that wins, the merge with the request's other
  // lane; the tile's result goes to row `slot` of the per-tile results
  auto fold_store = [&](const f32x16& acc0, const f32x16& acc1, float G0, float G1, int vt, int loc, int slot) {
    LaneDraw dr;
    lane_draw_init(dr);
    f32x4 a[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = f32x4{acc0[4 * m], acc0[4 * m + 1], acc0[4 * m + 2], acc0[4 * m + 3]};
    fold_chunk(a, G0, vt + 16 * h, dr);
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = f32x4{acc1[4 * m], acc1[4 * m + 1], acc1[4 * m + 2], acc1[4 * m + 3]};
    const bool take1 = fold_chunk(a, G1, vt + 32 + 16 * h, dr);
    float bs = neg_inf();
    int bo = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(&gsh[loc][4 * m]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = 4 * m + t;
        const float sc = (take1 ? acc1[c] : acc0[c]) + gv[t];
        if (sc > bs) {
          bs = sc;
          bo = c;
        }
      }
    }
    unsigned long long key = (dr.first >= 0 && bs > neg_inf()) ? pack_key(dr.best, dr.first + bo) : 0ull;
    float M2 = dr.M2, Ts = dr.T;
    {   // the request's other lane (h ^ 1)
      const unsigned long long ok = xor32(key);
      const float M2o = xor32(M2), To = xor32(Ts);
      key = ok > key ? ok : key;
      const float Mn = fmaxf(M2, M2o);
      Ts = Ts * __builtin_amdgcn_exp2f(M2 - Mn) + To * __builtin_amdgcn_exp2f(M2o - Mn);
      M2 = Mn;
    }
    if (h == 0) {
      mkey[slot][loc] = key;
      mlse[slot][loc] = make_float2(M2, Ts);
    }
  };

  // The RNN head (DSpark reading notes, "implementation two: the RNN head",
  // eq (6)) between positions: o_k and s_k for every request, then a grid
  // barrier.  Work group b computes items b, b + gx, ...: item (jb, ib) is
  // state columns 32 jb .. 32 jb + 31 of all three parts for requests
  // 32 ib .. 32 ib + 31.  Its z rows (the state s_{k-1} rounded to bf16, then
  // the previous token's W1 row; the hidden-state part is in Yh) go to LDS
  // (the W1-row area, free here), waves 0-5 each multiply one part's 32 W
  // rows by them over one half of the 2r inner elements, and all threads
  // add the two halves and the hidden-state part (its split partials
  // already summed) and apply the gates.  o and s are stored and read back as agent-scope
  // atomics (store32_agent, load16_agent), coherent across the dies.
  // z's state rows of step item block ib at position k into LDS (the
  // W1-row area): s_{k-1} of the block's 32 requests rounded to bf16, zeros
  // at k = 0; 16 threads per request
  auto z_state = [&](int k, int ib) {
    if constexpr (RNN != 0) {
      constexpr int r = KS16 * 16;
      constexpr int kZ = (RNN == 2 ? 2 : 4) * r + 16;
      const int i = static_cast<int>(threadIdx.x) >> 4, u = static_cast<int>(threadIdx.x) & 15;
      const int rc = min(32 * ib + i, R - 1);
      uint8_t* zr = erows + i * kZ;
      const float* srow = rnn.s + (static_cast<int64_t>(rc) * gamma + (k > 0 ? k - 1 : 0)) * r;
#pragma unroll
      for (int p = u; p < r / 8; p += 16) {
        const u32x4 a = load16_agent(srow + 8 * p), b = load16_agent(srow + 8 * p + 4);
        float4 lo = make_float4(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]),
                                __uint_as_float(a[3]));
        float4 hi = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]),
                                __uint_as_float(b[3]));
        if (k == 0) lo = hi = make_float4(0.f, 0.f, 0.f, 0.f);
        const uint32_t w0 = bf16_bits_rne(lo.x) | (bf16_bits_rne(lo.y) << 16);
        const uint32_t w1 = bf16_bits_rne(lo.z) | (bf16_bits_rne(lo.w) << 16);
        const uint32_t w2 = bf16_bits_rne(hi.x) | (bf16_bits_rne(hi.y) << 16);
        const uint32_t w3 = bf16_bits_rne(hi.z) | (bf16_bits_rne(hi.w) << 16);
        *reinterpret_cast<u32x4*>(zr + 16 * p) = u32x4{w0, w1, w2, w3};
      }
    }
  };

  auto rnn_phase = [&](int k, unsigned int round) -> bool {
    if constexpr (RNN != 0) {
      constexpr bool kP = RNN == 2;
      constexpr int r = KS16 * 16;
      constexpr int kZ = (kP ? 2 : 4) * r + 16;   // bytes of a z row in LDS (r or 2r bf16 and a pad)
      constexpr int nJB = r / 32;
      const int K = 2 * r + rnn.d;
      const int nItems = nJB * ((R + 31) / 32);
      static_assert(32 * kZ <= NROWS * kE, "the z rows fit in the W1-row area");
      static_assert(6 * 16 * kWave * 4 <= NROWS * kE, "the six partial products fit in the W1-row area");
      for (int item = bx; item < nItems; item += gx) {
        const int jb = item % nJB, ib = item / nJB;
        // kP: this thread's request's previous token (the gate thread below
        // is the same thread and looks the W1-row part of y up in P)
        int pprev = -1;
        {   // z rows: 16 threads per request
          const int i = static_cast<int>(threadIdx.x) >> 4, u = static_cast<int>(threadIdx.x) & 15;
          const int rc = min(32 * ib + i, R - 1);
          int prev;
          if (k == 0) {
            prev = token_or_none(x0[rc], V);
          } else {
            const unsigned long long* kp = ws.keys + static_cast<int64_t>(k - 1) * kKeySlots * R + rc;
            unsigned long long best = 0;
#pragma unroll
            for (int sl = 0; sl < kKeySlots; ++sl) {
              const unsigned long long v =
                  __hip_atomic_load(kp + static_cast<int64_t>(sl) * R, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              best = v > best ? v : best;
            }
            prev = token_or_none(key_token(best), V);
          }
          if constexpr (kP) pprev = prev;
          // the state rows (with P, the first item's were gathered before
          // the barrier, right after the previous position's sweep)
          if (!(kP && item == bx && k > kb)) z_state(k, ib);
          uint8_t* zr = erows + i * kZ;
          if constexpr (!kP) {   // the previous token's W1 row (zeros when there is none)
            const uint16_t* erow = prev >= 0 ? W1 + static_cast<int64_t>(prev) * r : kZeroRow;
#pragma unroll
            for (int p = u; p < r / 8; p += 16)
              *reinterpret_cast<u32x4*>(zr + 2 * r + 16 * p) = *reinterpret_cast<const u32x4*>(erow + 8 * p);
          }
        }
        __syncthreads();
        f32x16 acc = {};
        if (wave < 6) {   // part g = wave / 2 over half wave % 2 of the 2r (kP: r) inner elements
          constexpr int KSH = kP ? r / 32 : r / 16;   // k-steps per half
          constexpr int B8 = KSH < 8 ? KSH : 8;
          const int gp = wave >> 1, kh = (wave & 1) * KSH;
          const uint16_t* wrow = rnn.W + static_cast<int64_t>(gp * r + 32 * jb + j) * K + 16 * kh + 8 * h;
          const uint8_t* zrow = erows + j * kZ + 32 * kh + 16 * h;
          bf16x8 a[B8];
#pragma unroll
          for (int kk = 0; kk < B8; ++kk) a[kk] = load_bf16x8_global(wrow + 16 * kk);
#pragma unroll
          for (int k0 = 0; k0 < KSH; k0 += B8) {
            // each fragment is reloaded with the next batch's right after its
            // product is issued (the last batch loads itself again)
            const int kn = k0 + B8 < KSH ? k0 + B8 : k0;
#pragma unroll
            for (int kk = 0; kk < B8; ++kk) {
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], *reinterpret_cast<const bf16x8*>(zrow + 32 * (k0 + kk)),
                                                            acc, 0, 0, 0);
              a[kk] = load_bf16x8_global(wrow + 16 * (kn + kk));
            }
          }
        }
        __syncthreads();   // every z read is done
        float* red = reinterpret_cast<float*>(erows);
        if (wave < 6) {
#pragma unroll
          for (int q = 0; q < 16; ++q) red[(wave * 16 + q) * kWave + lane] = acc[q];
        }
        __syncthreads();
        // 1024 outputs: thread t takes request 32 ib + t / 16 and columns
        // 32 jb + c and c + 1, c = 2 (t % 16) (o_k's two bf16 in one store);
        // accumulator q of lane l holds row 8 (q / 4) + 4 (l / 32) + q % 4 of
        // the part's 32 and request l % 32.  Every load goes out before the
        // first sum.
        {
          const int rl = static_cast<int>(threadIdx.x) >> 4, c0 = 2 * (static_cast<int>(threadIdx.x) & 15);
          const int req = 32 * ib + rl;
          const int rq = min(req, R - 1);
          const int64_t row = static_cast<int64_t>(rq) * gamma + k;
          const int col = 32 * jb + c0;
          float2 yh[3];
#pragma unroll
          for (int gp = 0; gp < 3; ++gp) yh[gp] = *reinterpret_cast<const float2*>(rnn.Yh + row * (3 * r) + gp * r + col);
          float2 pv[3] = {};   // kP: the W1-row part (zero without a previous token)
          if constexpr (kP) {
            const float* prow = rnn.P + static_cast<int64_t>(pprev >= 0 ? pprev : 0) * (3 * r) + col;
#pragma unroll
            for (int gp = 0; gp < 3; ++gp) {
              const float2 v = *reinterpret_cast<const float2*>(prow + gp * r);
              pv[gp] = pprev >= 0 ? v : make_float2(0.f, 0.f);
            }
          }
          // s_{k-1} of the same columns (this work group's own stores), read
          // at k = 0 too and unused there
          const u32x4 sp4 = load16_agent(rnn.s + (k > 0 ? row - 1 : row) * r + (col & ~3));
          const float sprev[2] = {__uint_as_float(sp4[col & 3]), __uint_as_float(sp4[(col & 3) + 1])};
          float sn[2];
          uint32_t ob = 0;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int c = c0 + t;
            const int q = ((c >> 3) << 2) | (c & 3);
            const int l = (((c >> 2) & 1) << 5) | rl;
            float y[3];
#pragma unroll
            for (int gp = 0; gp < 3; ++gp)
              y[gp] = (t ? yh[gp].y : yh[gp].x) +
                      ((red[(2 * gp * 16 + q) * kWave + l] + red[((2 * gp + 1) * 16 + q) * kWave + l]) +
                       (kP ? (t ? pv[gp].y : pv[gp].x) : 0.f));
            const float gate = 1.f / (1.f + expf(-y[0]));
            sn[t] = gate * (k > 0 ? sprev[t] : 0.f) + (1.f - gate) * tanhf(y[1]);
            ob |= bf16_bits_rne(tanhf(y[2])) << (16 * t);
          }
          if (req < R) {
            store32_agent(rnn.s + row * r + col, __float_as_uint(sn[0]));
            store32_agent(rnn.s + row * r + col + 1, __float_as_uint(sn[1]));
            store32_agent(rnn.o + row * r + col, ob);
          }
        }
        __syncthreads();   // the products area is reused
      }
      if (!grid_barrier(ws.bar, round, &barflag, cancel)) return false;
    }
    return true;
  };

  const int s_end = ke * RB;
  ResLane pa, pb;   // steps s and s + 1 in flight (one block: the own tile and the LDS-held tile)
  if (active) {
    load_step(pa, kb * RB);
    if (NX == 0) load_step(pb, min(kb * RB + 1, s_end - 1));
  }
  if (NX > 0 && xact) load_at(pb, kb, 0, xv0);
  if (RNN && !rnn_phase(kb, 1)) return;   // o of the first position (the launch covers all of them)
  gather_e(kb, kb == 0);
  store_gq(load_gq(kb));
  __builtin_amdgcn_s_waitcnt(0);   // the A fragments copied into LDS have landed
  __syncthreads();

  for (int k = kb; k < ke; ++k) {
    if constexpr (NX > 0) {
      // one request block: the own tile (its next position's logits go into
      // pa), then the LDS-held tile if any (pb)
      f32x16 acc0, acc1;
      if (active) {
        products(pa, 0, acc0, acc1, std::false_type{});
        const float G0 = pa.G[0], G1 = pa.G[1];
        load_step(pa, min(k + 1, ke - 1));
        fold_store(acc0, acc1, G0, G1, v0, j, wave);
      }
      if (xact) {
        products(pb, 0, acc0, acc1, std::true_type{});
        const float G0 = pb.G[0], G1 = pb.G[1];
        load_at(pb, min(k + 1, ke - 1), 0, xv0);
        fold_store(acc0, acc1, G0, G1, xv0, j, kResWaves + wave);
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        ResLane& cur = (rb & 1) ? pb : pa;
        if (active) {
          f32x16 acc0, acc1;
          products(cur, rb, acc0, acc1, std::false_type{});
          const float G0 = cur.G[0], G1 = cur.G[1];
          load_step(cur, min(k * RB + rb + 2, s_end - 1));   // unconditional: no branch near the end
          fold_store(acc0, acc1, G0, G1, v0, 32 * rb + j, wave);
        }
      }
      if (RB & 1) {   // an odd block count flips the step parity across positions
        const ResLane t = pa;
        pa = pb;
        pb = t;
      }
    }
    __syncthreads();
    // one thread per request merges the tiles (in tile order) into its key
    // slot and log-sum-exp partial
    if (static_cast<int>(threadIdx.x) < NROWS) {
      const int i = static_cast<int>(threadIdx.x);
      unsigned long long key = 0ull;
      float M2 = neg_inf(), Ts = 0.f;
      for (int w = 0; w < nT; ++w) {
        const unsigned long long ok = mkey[w][i];
        const float2 o = mlse[w][i];
        key = ok > key ? ok : key;
        const float Mn = fmaxf(M2, o.x);
        Ts = (M2 == neg_inf() ? 0.f : Ts * __builtin_amdgcn_exp2f(M2 - Mn)) +
             (o.x == neg_inf() ? 0.f : o.y * __builtin_amdgcn_exp2f(o.x - Mn));
        M2 = Mn;
      }
      if (i < R) {
        ws.lsep[(static_cast<int64_t>(k) * R + i) * gx + bx] = make_float2(M2 * kLn2, Ts);
        if (key != 0ull)
          __hip_atomic_fetch_max(ws.keys + (static_cast<int64_t>(k) * kKeySlots + bx % kKeySlots) * R + i, key,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    if (k + 1 == ke) break;
    const f32x4 gq = load_gq(k + 1);
    // with P, the first step item's state rows for position k + 1 (s_k is
    // complete: its step ended before this position's sweep) go to LDS
    // while the barrier is pending
    if constexpr (RNN == 2) {
      if (bx < (KS16 / 2) * ((R + 31) / 32)) z_state(k + 1, bx / (KS16 / 2));
    }
    // the RNN head meets twice per position: the keys of position k, then o
    // of position k + 1
    if (!grid_barrier(ws.bar, RNN ? 2 * (k + 1) : k + 1, &barflag, cancel)) return;
    if (RNN && !rnn_phase(k + 1, 2 * (k + 1) + 1)) return;
    gather_e(k + 1, false);
    store_gq(gq);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ host side

int compute_units();   // abi.hip

// Tiles a work group can hold for a shape (see res_max_tiles).
static int res_tiles_for(int R, int r) {
  return R <= 32 && r == 256 ? res_max_tiles<1, 16>() : res_max_tiles<4, 16>();
}

// Work groups of the launch: one per compute unit (at most one per tile and
// max_wgs), or 0 when some group would get more tiles than it can hold (the
// vocabulary is too large for the register files and LDS).
int res_grid_x(int R, int V, int r, int max_wgs) {
  const int nTiles = (V + kChunk - 1) / kChunk;
  int gx = compute_units();
  if (gx > nTiles) gx = nTiles;
  if (gx > max_wgs) gx = max_wgs;
  if (gx < 1) return 0;
  return (nTiles + gx - 1) / gx <= res_tiles_for(R, r) ? gx : 0;
}

template <int RB, int KS16, bool VEC, int RNN = 0>
static bool res_fits_one() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, reinterpret_cast<const void*>(&sample_steps_res<RB, KS16, VEC, RNN>), kResThreads, 0);
    v = (e == hipSuccess && n >= 1) ? 1 : 2;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1;
}

template <int KS16>
static bool res_fits_ks(int R, bool vec) {
  if (R <= 32) return vec ? res_fits_one<1, KS16, true>() : res_fits_one<1, KS16, false>();
  if (R <= 64) return vec ? res_fits_one<2, KS16, true>() : res_fits_one<2, KS16, false>();
  return vec ? res_fits_one<4, KS16, true>() : res_fits_one<4, KS16, false>();
}

// Whether the resident-W2t kernel takes a bf16 Markov-head launch of this
// shape: R <= 128, r in {32, 64, 128, 256}, at most res_tiles_for(R, r)
// tiles per work group, and the work group fits on a compute unit.
bool res_usable(int R, int V, int r, int max_wgs) {
  if (R < 1 || R > 128 || res_grid_x(R, V, r, max_wgs) == 0) return false;
  const bool vec = (V % kGChunk) == 0;
  switch (r) {
    case 32: return res_fits_ks<2>(R, vec);
    case 64: return res_fits_ks<4>(R, vec);
    case 128: return res_fits_ks<8>(R, vec);
    case 256: return res_fits_ks<16>(R, vec);
    default: return false;
  }
}

template <int RB, int KS16, bool VEC>
static void launch_res(int R, int gamma, int V, const void* U, const void* W1, const void* W2t, const int32_t* x0,
                       const float* G, const float* g, const SampleWs& w, int gx, int kb, int ke,
                       const uint32_t* cancel, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
  hipExtLaunchKernelGGL((sample_steps_res<RB, KS16, VEC>), dim3(gx), dim3(kResThreads), 0, s, ev0, ev1, 0, R, gamma,
                        V, static_cast<const uint16_t*>(U), static_cast<const uint16_t*>(W1),
                        static_cast<const uint16_t*>(W2t), x0, G, g, w, kb, ke, cancel, ResRnn{});
}

template <int KS16>
static void launch_res_ks(int R, int gamma, int V, const void* U, const void* W1, const void* W2t,
                          const int32_t* x0, const float* G, const float* g, const SampleWs& w, int gx, int kb,
                          int ke, const uint32_t* cancel, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
  const bool vec = (V % kGChunk) == 0;
#define DSPARK_RES(RB)                                                                                      \
  (vec ? launch_res<RB, KS16, true>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, kb, ke, cancel, ev0, ev1, s) \
       : launch_res<RB, KS16, false>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, kb, ke, cancel, ev0, ev1, s))
  if (R <= 32)
    DSPARK_RES(1);
  else if (R <= 64)
    DSPARK_RES(2);
  else
    DSPARK_RES(4);
#undef DSPARK_RES
}

// Launches all positions kb .. ke - 1 (the caller checked res_usable).
hipError_t res_launch(int R, int gamma, int V, int r, const void* U, const void* W1, const void* W2t,
                      const int32_t* x0, const float* G, const float* g, const SampleWs& w, int gx, int kb, int ke,
                      const uint32_t* cancel, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
  switch (r) {
    case 32: launch_res_ks<2>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, kb, ke, cancel, ev0, ev1, s); break;
    case 64: launch_res_ks<4>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, kb, ke, cancel, ev0, ev1, s); break;
    case 128: launch_res_ks<8>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, kb, ke, cancel, ev0, ev1, s); break;
    default: launch_res_ks<16>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, kb, ke, cancel, ev0, ev1, s); break;
  }
  return hipGetLastError();
}

// The RNN head in the same persistent launch (rnn_phase): 33 to 128
// requests at r = 256, 65 to 128 at r = 128 (the W1-row area must hold
// the z rows and six partial products), the tiles on chip as for the
// Markov head, and the work group fits on a compute unit.
bool res_rnn_usable(int R, int V, int r, int max_wgs) {
  if (R > 128 || res_grid_x(R, V, r, max_wgs) == 0) return false;
  const bool vec = (V % kGChunk) == 0;
  if (r == 128 && R > 64) return vec ? res_fits_one<4, 8, true, 1>() : res_fits_one<4, 8, false, 1>();
  if (r != 256 || R < 33) return false;
  if (R <= 64) return vec ? res_fits_one<2, 16, true, 1>() : res_fits_one<2, 16, false, 1>();
  return vec ? res_fits_one<4, 16, true, 1>() : res_fits_one<4, 16, false, 1>();
}

template <int RB, int KS16, bool VEC>
static void launch_res_rnn(int R, int gamma, int V, const void* U, const void* W1, const void* W2t,
                           const int32_t* x0, const float* G, const float* g, const SampleWs& w, int gx,
                           const uint32_t* cancel, const ResRnn& rn, hipStream_t s) {
  // with P, the variant whose step looks the W1-row part up, if it fits
  if (rn.P && res_fits_one<RB, KS16, VEC, 2>())
    hipLaunchKernelGGL((sample_steps_res<RB, KS16, VEC, 2>), dim3(gx), dim3(kResThreads), 0, s, R, gamma, V,
                       static_cast<const uint16_t*>(U), static_cast<const uint16_t*>(W1),
                       static_cast<const uint16_t*>(W2t), x0, G, g, w, 0, gamma, cancel, rn);
  else
    hipLaunchKernelGGL((sample_steps_res<RB, KS16, VEC, 1>), dim3(gx), dim3(kResThreads), 0, s, R, gamma, V,
                       static_cast<const uint16_t*>(U), static_cast<const uint16_t*>(W1),
                       static_cast<const uint16_t*>(W2t), x0, G, g, w, 0, gamma, cancel, rn);
}

// Launches all positions with the RNN head (the caller checked
// res_rnn_usable and computed the hidden-state partials).  P, when given,
// is W's W1-row columns applied to every W1 row (dspark_rnn_prepare).
hipError_t res_rnn_launch(int R, int gamma, int V, int r, const void* U, const void* W1, const void* W2t,
                          const int32_t* x0, const float* G, const float* g, const SampleWs& w, int gx,
                          const uint32_t* cancel, const void* Wrnn, const float* Yh, int d, float* st, void* o,
                          const float* P, hipStream_t s) {
  const ResRnn rn{static_cast<const uint16_t*>(Wrnn), Yh, d, st, static_cast<uint16_t*>(o), P};
  const bool vec = (V % kGChunk) == 0;
#define DSPARK_RES_RNN(RB, KS)                                                                   \
  (vec ? launch_res_rnn<RB, KS, true>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, cancel, rn, s) \
       : launch_res_rnn<RB, KS, false>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, cancel, rn, s))
  if (r == 128) {
    DSPARK_RES_RNN(4, 8);
  } else {
    if (R <= 64)
      DSPARK_RES_RNN(2, 16);
    else
      DSPARK_RES_RNN(4, 16);
  }
#undef DSPARK_RES_RNN
  return hipGetLastError();
}

}  // namespace dspark
