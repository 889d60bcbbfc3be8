// dspark_markov_sample: the semi-autoregressive gamma-step loop.
//
// Passage: DSpark reading notes, eq (4) (p_k(v) ∝ exp(U_k(v) + B_k(v))) and
// eq (5) (B(x_{k-1}, .) = W1[x_{k-1}] W2); caijizhuo summary, section 四
// (the sequential loop carries only the sampled token).
//
// A call is sample_init (clears the argmax keys and barrier words), the
// sweeps, and sample_finalize.  With bf16 storage one persistent launch
// (sample_steps_wide) covers all gamma positions, its work groups meeting at a
// grid barrier between positions; batches whose request groups outnumber the
// compute units (more than 32768 requests), and fp32 storage, take one
// sample_step_* launch per position instead.  Each sweep streams U_k and W2t
// once, builds the Markov bias of a 64-token tile for all requests on the
// matrix cores, and folds each 16-token Gumbel chunk into running per-request
// state: the log-sum-exp (for lse) and the chunk-level Gumbel-max (score
// LSE_c + G_c), keeping the best chunk's logits for the in-chunk draw (argmax
// of l_v + g_{v mod 16}), which is made once at the end of the sweep.  Each
// work group then merges its draw into the request's key with one 64-bit
// atomic max (four key slots per request spread the contention) and stores
// its log-sum-exp partial.  The next position reads the keys back as its
// previous tokens.  sample_finalize decodes x, merges the log-sum-exp
// partials and recomputes the logit of each drafted token.
#include <hip/hip_ext.h>

#include "bias_tile.hpp"
#include "wide_tile.hpp"
#include "sample_keys.hpp"
#include "rnn_head.hpp"
#include "sample_common.hpp"
#include "confidence_row.hpp"

#include <atomic>

namespace dspark {

// Upper bound on the work groups per position along the vocabulary (the
// bf16 kernel runs one work group per compute unit); sizes the workspace.
constexpr int kMaxSampleWGs = 1024;

template <int NBW>
__host__ __device__ constexpr int sample_reqs_per_wg() { return kTileWaves * 16 * NBW; }


// Clears the first n key words (the slots in use) and the barrier words.
__global__ __launch_bounds__(256) void sample_init(unsigned long long* keys, int64_t n, unsigned long long* bar) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n + kBarWords;
       i += static_cast<int64_t>(gridDim.x) * 256)
    (i < n ? keys[i] : bar[i - n]) = 0ull;
}


// MFMA C operand of M-block mb: the lane's tokens 4 mb .. 4 mb + 3 as fp32.
__device__ __forceinline__ f32x4 lane16_c(const u32x4 (&u)[2], int mb) {
  const uint32_t w0 = u[mb >> 1][2 * (mb & 1)];
  const uint32_t w1 = u[mb >> 1][2 * (mb & 1) + 1];
  return f32x4{__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u), __uint_as_float(w1 << 16),
               __uint_as_float(w1 & 0xFFFF0000u)};
}


// Per-chunk loads that each lane makes for itself: its sixteen logits and
// its chunk Gumbel, for every request group.
template <int NBW>
struct LaneLoads {
  u32x4 u[NBW][2];
  float G[NBW];
};

// One drafted position for a group of 16 * NBW * 4 requests over the
// vocabulary tiles blockIdx.x, blockIdx.x + gridDim.x, ... (64 tokens each).
// Lane (q, j) of wave w holds, for request group nb, request
// 64 NBW blockIdx.y + 16 (NBW w + nb) + j and the Gumbel chunk of tokens
// v0 + 16 q .. v0 + 16 q + 15: its logits seed the MFMA accumulators, which
// then hold U + B for exactly those tokens, so every reduction of the chunk
// stays inside the lane.
//
// Loads: each lane's logits and chunk Gumbels are issued two tiles ahead into
// two register sets; the W2t tile (shared by the four waves through LDS) is
// issued one tile ahead into registers and stored into the other half of a
// double-buffered LDS area after the current tile's products.
template <int NBW, int KS, bool VEC>
__global__ __launch_bounds__(kTileThreads, 1) void sample_step_bf16(
    int R, int gamma, int V, int k, const uint16_t* __restrict__ U, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W2t, const int32_t* __restrict__ x0, const float* __restrict__ G,
    const float* __restrict__ g, SampleWs ws, int nPart, const uint16_t* __restrict__ bvec) {
  static_assert(kGChunk == 16 && kChunk == 64, "one Gumbel chunk per lane and M-block column of four");
  constexpr int NROWS = sample_reqs_per_wg<NBW>();
  constexpr int kW = tile_bytes(KS);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kW];
  __shared__ float gsh[NROWS][kGChunk];        // in-chunk Gumbels of the group's requests
  // each lane's last two folded chunks per request group, one of them its
  // best: [nb][slot][mb][thread], flat
  __shared__ f32x4 keepsh[NBW * 2 * 4 * kTileThreads];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int q = lane >> 4;
  const int nTiles = (V + kChunk - 1) / kChunk;
  const int nG = (V + kGChunk - 1) / kGChunk;
  // the host launches at most one work group per tile, so nT >= 1
  const int nT = (nTiles - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                 static_cast<int>(gridDim.x);

  int req[NBW], loc[NBW];
  bool live[NBW];
  int64_t rowk[NBW];   // (request, k) row of U and g; clamped to a valid request
  int reqc[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    loc[nb] = wave * 16 * NBW + nb * 16 + j;
    req[nb] = blockIdx.y * NROWS + loc[nb];
    live[nb] = req[nb] < R;
    reqc[nb] = min(req[nb], R - 1);
    rowk[nb] = static_cast<int64_t>(reqc[nb]) * gamma + k;
  }
  const auto clampc = [&](int it) { return it < nT ? it : nT - 1; };
  const auto tile_of = [&](int it) { return static_cast<int>(blockIdx.x) + it * static_cast<int>(gridDim.x); };
  // G is [gamma][nG][R]: the lane's chunk of tile t is 4 t + q
  const float* Gk = G + static_cast<int64_t>(k) * nG * R;
  auto load_lane = [&](LaneLoads<NBW>& ll, int it) {
    const int t = tile_of(it);
    const int v = t * kChunk + q * kGChunk;
    const int gc = min(4 * t + q, nG - 1);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      load_lane16<VEC>(ll.u[nb], U + rowk[nb] * V, v, V);
      ll.G[nb] = Gk[static_cast<int64_t>(gc) * R + reqc[nb]];
    }
  };

  // the previous tokens first: the W1 rows they select gate the first products
  int prev[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) prev[nb] = !bvec && live[nb] ? previous_token(ws.keys, ws.slots, x0, R, V, k, req[nb]) : -1;
  // in-chunk Gumbels: lane q brings offsets 4q .. 4q + 3 of its request
  f32x4 gq[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) gq[nb] = *reinterpret_cast<const f32x4*>(g + rowk[nb] * kGChunk + 4 * q);
  WRegs<KS> wr;
  load_w2_regs<KS>(wr, W2t, V, tile_of(0) * kChunk);
  LaneLoads<NBW> even, odd;
  load_lane(even, 0);
  load_lane(odd, clampc(1));
  WFrags<NBW, KS> e;
  // the bias vector of each request: its previous token's W1 row, or the
  // given per-(request, position) vectors
  const uint16_t* erow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
    erow[nb] = bvec ? bvec + rowk[nb] * (KS * 32)
                    : (prev[nb] >= 0 ? W1 + static_cast<int64_t>(prev[nb]) * (KS * 32) : nullptr);
  load_vec_frags<NBW, KS>(e, erow);

  LaneDraw dr[NBW];
  int bestSlot[NBW];   // which of the lane's two keep slots holds its best chunk
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    lane_draw_init(dr[nb]);
    bestSlot[nb] = 0;
    *reinterpret_cast<f32x4*>(&gsh[loc[nb]][4 * q]) = gq[nb];
  }
  store_w2_tile_lane16<KS>(lds, wr);
  load_w2_regs<KS>(wr, W2t, V, tile_of(clampc(1)) * kChunk);
  __syncthreads();

  // Software pipeline: the products of tile `it` are formed while tile
  // it - 1 is folded, so the matrix cores and the vector ALUs of a wave work
  // on independent data.  accP holds the finished logits of the previous
  // tile.
  f32x4 accP[4][NBW];
  float GcP[NBW];
  int v0P = 0;
  // products of tile `it` (LDS half it & 1, logits from register set `cur`,
  // which is refilled with tile it + 2)
  auto products = [&](int it, LaneLoads<NBW>& cur, f32x4 (&acc)[4][NBW], float (&Gc)[NBW]) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = lane16_c(cur.u[nb], mb);
      Gc[nb] = cur.G[nb];
    }
    load_lane(cur, clampc(it + 2));
    bias_tile_acc<NBW, KS>(acc, lds + (it & 1) * kW, e);
  };
  // fold the previous tile: its logits go to the free keep slot whatever
  // happens, and the slot becomes the best one if the chunk wins (no branch)
  auto fold_prev = [&]() {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      f32x4 a[4] = {accP[0][nb], accP[1][nb], accP[2][nb], accP[3][nb]};
      const int freeSlot = bestSlot[nb] ^ 1;
      f32x4* kp = keepsh + ((nb * 2 + freeSlot) * 4) * kTileThreads + threadIdx.x;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) kp[mb * kTileThreads] = a[mb];
      if (fold_chunk(a, GcP[nb], v0P + q * kGChunk, dr[nb])) bestSlot[nb] = freeSlot;
    }
  };
  // stores tile it + 1 into the other LDS half, issues the W2t loads of
  // tile it + 2, and waits for every wave
  auto advance = [&](int it) {
    store_w2_tile_lane16<KS>(lds + ((it + 1) & 1) * kW, wr);
    load_w2_regs<KS>(wr, W2t, V, tile_of(clampc(it + 2)) * kChunk);
    __syncthreads();
  };
  auto body = [&](int it, LaneLoads<NBW>& cur) {
    f32x4 accN[4][NBW];
    float GcN[NBW];
    products(it, cur, accN, GcN);
    fold_prev();
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) accP[mb][nb] = accN[mb][nb];
      GcP[nb] = GcN[nb];
    }
    v0P = tile_of(it) * kChunk;
    advance(it);
  };

  products(0, even, accP, GcP);
  v0P = tile_of(0) * kChunk;
  advance(0);
  // pairs of tiles, so every path back to the loop head has issued both
  // register sets' loads in the same order; an odd last tile follows the loop
  int it = 1;
  for (; it + 1 < nT; it += 2) {
    body(it, odd);
    body(it + 1, even);
  }
  if (it < nT) body(it, odd);
  fold_prev();

  // the in-chunk draw on each lane's best chunk, then the best of the four
  // lanes of a request, merged across work groups by atomic max
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const float* gl = gsh[loc[nb]];
    float kept[kGChunk];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const f32x4 v = keepsh[((nb * 2 + bestSlot[nb]) * 4 + mb) * kTileThreads + threadIdx.x];
#pragma unroll
      for (int i = 0; i < 4; ++i) kept[4 * mb + i] = v[i];
    }
    float bs = neg_inf();
    int bo = 0;
#pragma unroll
    for (int c = 0; c < kGChunk; ++c) {
      const float sc = kept[c] + gl[c];
      if (sc > bs) {
        bs = sc;
        bo = c;
      }
    }
    unsigned long long key = (dr[nb].first >= 0 && bs > neg_inf()) ? pack_key(dr[nb].best, dr[nb].first + bo) : 0ull;
    float M2 = dr[nb].M2, T = dr[nb].T;
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const unsigned long long ok = __shfl_xor(key, o);
      key = ok > key ? ok : key;
      const float M2o = __shfl_xor(M2, o);
      const float To = __shfl_xor(T, o);
      const float Mn = fmaxf(M2, M2o);
      T = T * __builtin_amdgcn_exp2f(M2 - Mn) + To * __builtin_amdgcn_exp2f(M2o - Mn);
      M2 = Mn;
    }
    if (q == 0 && live[nb]) {
      ws.lsep[(static_cast<int64_t>(k) * R + req[nb]) * nPart + blockIdx.x] = make_float2(M2 * kLn2, T);
      if (key != 0ull)
        atomicMax(ws.keys + (static_cast<int64_t>(k) * ws.slots + blockIdx.x % ws.slots) * R + req[nb], key);
    }
  }
}

// W2t tiles of each work group that stay in LDS for the whole launch (the
// middle pair of its tiles): they are read from HBM once instead of once per
// position.
constexpr int kResident = 2;

// All gamma positions in one launch.  Position k + 1 needs the tokens drawn
// at position k, so the work groups meet at a grid barrier between positions;
// the loads that do not depend on the tokens (the next position's logits and
// chunk Gumbels, its first two W2t tiles) are issued before the barrier and
// land while it waits.  A work group walks its tiles in snake order (forward
// on even positions, backward on odd ones), so the W2t tile it ends a
// position with is the one it starts the next with.  Tiles are handed out in
// pairs, so every work group has an even number of positions per sweep (a
// phantom tile past the vocabulary, if the tile count is odd, reads -inf
// logits and drops out) and the two register sets keep their roles across
// positions.
template <int RQ, int KS16, bool VEC>
__global__ __launch_bounds__(wide_threads<RQ>(), 1) void sample_steps_wide(
    int R, int gamma, int V, const uint16_t* __restrict__ U, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W2t, const int32_t* __restrict__ x0, const float* __restrict__ G,
    const float* __restrict__ g, SampleWs ws, int nPart, int kb, int ke, const uint16_t* __restrict__ bvec,
    const uint32_t* __restrict__ cancel) {
  static_assert(kGChunk == 16 && kChunk == 64, "one Gumbel chunk per lane of a 32x32 output block");
  constexpr int NROWS = 32 * RQ;
  constexpr int kW = wide_tile_bytes<KS16>();   // tile bytes (padded rows)
  // two streaming slots, then the kResident tiles kept for the whole launch
  __shared__ __attribute__((aligned(1024))) uint8_t lds[(2 + kResident) * kW];
  __shared__ float gsh[NROWS][kGChunk];        // in-chunk Gumbels of the group's requests
  __shared__ float2 lsh[NROWS];                // token half 1 -> token half 0 hand-over
  __shared__ unsigned long long ksh[NROWS];
  __shared__ int barflag;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int th = wave & 1;
  const int rq = wave >> 1;
  const int j = lane & 31;
  const int h = lane >> 5;
  const int loc = rq * 32 + j;
  const int req = static_cast<int>(blockIdx.y) * NROWS + loc;
  const bool live = req < R;
  const int reqc = min(req, R - 1);
  const int lofs = 32 * th + 16 * h;   // the lane's first token in a tile
  const int nTiles = (V + kChunk - 1) / kChunk;
  const int nG = (V + kGChunk - 1) / kGChunk;
  const int nPairs = (nTiles + 1) / 2;
  // the host launches at most one work group per tile pair, so nT >= 2
  const int nT = 2 * ((nPairs - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                      static_cast<int>(gridDim.x));
  // tile at sweep position p of position k (snake order over this group's pairs)
  const auto q_at = [&](int k, int p) { return (k & 1) ? nT - 1 - p : p; };
  const auto tile_q = [&](int q) {
    return 2 * (static_cast<int>(blockIdx.x) + (q >> 1) * static_cast<int>(gridDim.x)) + (q & 1);
  };
  const auto tile_at = [&](int k, int p) { return tile_q(q_at(k, p)); };
  // a sweep position past the last belongs to the next position (the last
  // position of the launch repeats its last tile)
  const auto next_k = [&](int k, int p) { return p < nT ? k : (k + 1 < ke ? k + 1 : k); };
  const auto next_p = [&](int k, int p) { return p < nT ? p : (k + 1 < ke ? p - nT : nT - 1); };
  // the middle pair of the group's tiles stays in LDS (so that every
  // position starts on streamed tiles, whose loads are issued before the
  // grid barrier); the others stream through two slots, alternating with
  // the sweep position
  const int qr = nT / 2 - 1;
  const auto is_res = [&](int q) { return q >= qr && q < qr + kResident; };
  const auto resident = [&](int k, int p) { return is_res(q_at(next_k(k, p), next_p(k, p))); };
  const auto slot_of = [&](int k, int p) { return resident(k, p) ? 2 + q_at(k, p) - qr : (p & 1); };

  struct Lane {
    u32x4 u[2];
    float G;
  };
  auto load_lane = [&](Lane& ll, int k, int p) {
    const int k2 = next_k(k, p), p2 = next_p(k, p);
    const int t = tile_at(k2, p2);
    const int64_t row = static_cast<int64_t>(reqc) * gamma + k2;
    load_lane16<VEC>(ll.u, U + row * V, t * kChunk + lofs, V);
    ll.G = G[(static_cast<int64_t>(k2) * nG + min(4 * t + 2 * th + h, nG - 1)) * R + reqc];
  };
  auto load_w = [&](WideW<KS16, RQ>& w, int k, int p) {
    if (!resident(k, p)) wide_load_w<KS16, RQ>(w, W2t, V, tile_at(next_k(k, p), next_p(k, p)) * kChunk);
  };
  // in-chunk Gumbels of position k: each of the request's four lanes brings four offsets
  auto load_gq = [&](int k) {
    return *reinterpret_cast<const f32x4*>(g + (static_cast<int64_t>(reqc) * gamma + k) * kGChunk + 8 * th + 4 * h);
  };
  // B operand: k-step ks takes elements 16 ks + 8 h .. + 7 of the W1 row of
  // the previous token (a row of zeros when there is none: bias 0), or of
  // the request's given bias vector of position k
  bf16x8 e[KS16];
  auto load_e = [&](int prev, int k) {
    const uint16_t* w1row =
        (bvec ? bvec + (static_cast<int64_t>(reqc) * gamma + k) * (KS16 * 16)
              : prev >= 0 ? W1 + static_cast<int64_t>(prev) * (KS16 * 16) : kZeroRow) + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS16; ++ks) e[ks] = load_bf16x8_global(w1row + 16 * ks);
  };

  WideW<KS16, RQ> wr;
  Lane even, odd;
  LaneDraw dr;
  f32x16 bestL = {};   // logits of the lane's best chunk so far
  f32x16 accP;
  float GcP = 0.f;
  int v0P = 0;

  auto products = [&](int k, int p, Lane& cur, f32x16& acc, float& Gc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t w = cur.u[r >> 3][(r >> 1) & 3];
      acc[r] = __uint_as_float((r & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    Gc = cur.G;
    load_lane(cur, k, p + 2);
    // the lane's A rows: stored row 32 th + j, piece 2 ks + h at k-step ks
    const uint8_t* arow = lds + slot_of(k, p) * kW + ((32 * th + j) * wide_row_pieces<KS16>() + h) * 16;
    // A fragments in batches of eight reads ahead of their products; two
    // accumulator chains (even and odd k-steps) keep the matrix pipe busy
    constexpr int KB = KS16 < 8 ? KS16 : 8;
    f32x16 acc2 = {};
#pragma unroll
    for (int k0 = 0; k0 < KS16; k0 += KB) {
      bf16x8 a[KB];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) a[kk] = *reinterpret_cast<const bf16x8*>(arow + (k0 + kk) * 32);
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        if (kk & 1)
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], e[k0 + kk], acc2, 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], e[k0 + kk], acc, 0, 0, 0);
      }
    }
    acc += acc2;
  };
  // fold the previous tile; its logits become the best chunk's if it wins
  auto fold_prev = [&]() {
    f32x4 a[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = f32x4{accP[4 * m], accP[4 * m + 1], accP[4 * m + 2], accP[4 * m + 3]};
    const bool take = fold_chunk(a, GcP, v0P + lofs, dr);
#pragma unroll
    for (int c = 0; c < kGChunk; ++c) bestL[c] = take ? accP[c] : bestL[c];
  };
  // stores the tile of sweep position p + 1 into its streaming slot (unless
  // it is resident), issues the W2t loads of position p + 2, and waits for
  // every wave
  auto advance = [&](int k, int p) {
    if (!resident(k, p + 1)) wide_store_w<KS16, RQ>(lds + ((p + 1) & 1) * kW, wr);
    load_w(wr, k, p + 2);
    __syncthreads();
  };
  auto body = [&](int k, int p, Lane& cur) {
    f32x16 accN;
    float GcN;
    products(k, p, cur, accN, GcN);
    fold_prev();
    accP = accN;
    GcP = GcN;
    v0P = tile_at(k, p) * kChunk;
    advance(k, p);
  };

  // the first position of the launch: with W1 rows, its previous token is
  // the anchor (kb = 0)
  const int x0v = bvec ? -1 : x0[reqc];
  __builtin_amdgcn_sched_barrier(0);
  f32x4 gq = load_gq(kb);
  static_assert(kResident == 2, "the resident tiles are one pair");
  wide_load_w<KS16, RQ>(wr, W2t, V, tile_q(qr) * kChunk);
  load_lane(even, kb, 0);
  load_lane(odd, kb, 1);
  load_e(live ? token_or_none(x0v, V) : -1, kb);
  *reinterpret_cast<f32x4*>(&gsh[loc][8 * th + 4 * h]) = gq;
  wide_store_w<KS16, RQ>(lds + 2 * kW, wr);
  wide_load_w<KS16, RQ>(wr, W2t, V, tile_q(qr + 1) * kChunk);
  wide_store_w<KS16, RQ>(lds + 3 * kW, wr);
  load_w(wr, kb, 0);
  if (!resident(kb, 0)) wide_store_w<KS16, RQ>(lds, wr);
  load_w(wr, kb, 1);
  __syncthreads();

  for (int k = kb; k < ke; ++k) {
    lane_draw_init(dr);
    products(k, 0, even, accP, GcP);
    v0P = tile_at(k, 0) * kChunk;
    advance(k, 0);
    int p = 1;
    for (; p + 1 < nT; p += 2) {
      body(k, p, odd);
      body(k, p + 1, even);
    }
    body(k, p, odd);   // nT is even: the last sweep position is odd
    fold_prev();

    // the in-chunk draw on the lane's best chunk
    float bs = neg_inf();
    int bo = 0;
#pragma unroll
    for (int c = 0; c < kGChunk; ++c) {
      const float sc = bestL[c] + gsh[loc][c];
      if (sc > bs) {
        bs = sc;
        bo = c;
      }
    }
    unsigned long long key = (dr.first >= 0 && bs > neg_inf()) ? pack_key(dr.best, dr.first + bo) : 0ull;
    float M2 = dr.M2, Ts = dr.T;
    // the request's two lanes in this wave (h = 0, 1), then its two waves
    auto merge = [&](unsigned long long ok, float M2o, float To) {
      key = ok > key ? ok : key;
      const float Mn = fmaxf(M2, M2o);
      Ts = Ts * __builtin_amdgcn_exp2f(M2 - Mn) + To * __builtin_amdgcn_exp2f(M2o - Mn);
      M2 = Mn;
    };
    merge(xor32(key), xor32(M2), xor32(Ts));
    if (th == 1 && h == 0) {
      lsh[loc] = make_float2(M2, Ts);
      ksh[loc] = key;
    }
    __syncthreads();
    if (th == 0 && h == 0 && live) {
      const float2 o = lsh[loc];
      merge(ksh[loc], o.x, o.y);
      ws.lsep[(static_cast<int64_t>(k) * R + req) * nPart + blockIdx.x] = make_float2(M2 * kLn2, Ts);
      if (key != 0ull)
        __hip_atomic_fetch_max(ws.keys + (static_cast<int64_t>(k) * ws.slots + blockIdx.x % ws.slots) * R + req,
                               key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    if (k + 1 == ke) break;

    // next position: its in-chunk Gumbels are fetched before the barrier; its
    // logits and first two W2t tiles are already in flight
    gq = load_gq(k + 1);
    if (!grid_barrier(ws.bar, k + 1, &barflag, cancel)) return;
    const unsigned long long* kp = ws.keys + static_cast<int64_t>(k) * ws.slots * R + reqc;
    unsigned long long best = 0;
    for (int sl = 0; sl < ws.slots; ++sl) {
      const unsigned long long v = __hip_atomic_load(kp + static_cast<int64_t>(sl) * R, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_SYSTEM);
      best = v > best ? v : best;
    }
    load_e(live ? token_or_none(key_token(best), V) : -1, k + 1);
    *reinterpret_cast<f32x4*>(&gsh[loc][8 * th + 4 * h]) = gq;
    __syncthreads();
  }
}

// fp32 storage, any rank: one wave per (64-token tile, request), plain FMA
// bias; each sixteen-lane quarter of the wave is one Gumbel chunk.
__global__ __launch_bounds__(64) void sample_step_f32(
    int R, int gamma, int V, int r, int k, const float* __restrict__ U, const float* __restrict__ W1,
    const float* __restrict__ W2t, const int32_t* __restrict__ x0, const float* __restrict__ G,
    const float* __restrict__ g, SampleWs ws, int nPart, const float* __restrict__ bvec) {
  const int tile = blockIdx.x;
  const int req = blockIdx.y;
  const int lane = threadIdx.x;
  const int nG = (V + kGChunk - 1) / kGChunk;
  const int prev = bvec ? -1 : previous_token(ws.keys, ws.slots, x0, R, V, k, req);
  const int v = tile * kChunk + lane;
  const int64_t rowk = static_cast<int64_t>(req) * gamma + k;
  float val = neg_inf();
  if (v < V) {
    float b = 0.f;
    if (bvec || prev >= 0) {
      const float* e = bvec ? bvec + rowk * r : W1 + static_cast<int64_t>(prev) * r;
      const float* w = W2t + static_cast<int64_t>(v) * r;
      for (int i = 0; i < r; ++i) b = fmaf(e[i], w[i], b);
    }
    val = U[rowk * V + v] + b;
  }
  // the chunk's log-sum-exp and in-chunk Gumbel argmax over its sixteen lanes
  float m = val;
#pragma unroll
  for (int o = 1; o < kGChunk; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float mr = m == neg_inf() ? 0.f : m;
  float s = __expf(val - mr);
#pragma unroll
  for (int o = 1; o < kGChunk; o <<= 1) s += __shfl_xor(s, o);
  const int off = lane & (kGChunk - 1);
  Best in{v < V ? val + g[rowk * kGChunk + off] : neg_inf(), off, 0.f};
#pragma unroll
  for (int o = 1; o < kGChunk; o <<= 1) {
    Best b{__shfl_xor(in.score, o), __shfl_xor(in.tok, o), 0.f};
    in = best_combine(in, b);
  }
  const int c = tile * (kChunk / kGChunk) + lane / kGChunk;
  const bool any = c < nG && s > 0.f;
  Best ch{any ? mr + __logf(s) + G[(static_cast<int64_t>(k) * nG + c) * R + req] : neg_inf(),
          any ? c * kGChunk + in.tok : -1, 0.f};
  Lse run{mr, s};
  // the tile's best chunk and log-sum-exp over its four chunks
#pragma unroll
  for (int o = kGChunk; o < kChunk; o <<= 1) {
    Best b{__shfl_xor(ch.score, o), __shfl_xor(ch.tok, o), 0.f};
    if (b.tok >= 0 && (ch.tok < 0 || better(b.score, b.tok, ch.score, ch.tok))) ch = b;
    run = lse_combine(run, Lse{__shfl_xor(run.M, o), __shfl_xor(run.S, o)});
  }
  if (lane == 0) {
    ws.lsep[(static_cast<int64_t>(k) * R + req) * nPart + tile] = make_float2(run.M, run.S);
    if (ch.tok >= 0)
      atomicMax(ws.keys + (static_cast<int64_t>(k) * ws.slots + tile % ws.slots) * R + req,
                pack_key(ch.score, ch.tok));
  }
}

// Decode x, merge the log-sum-exp partials and recompute each drafted
// token's logit U_k(x_k) + W1[x_{k-1}] . W2t[x_k] (or the given bias vector
// of (request, k) in W1[x_{k-1}]'s place): one wave per (request, k).  With
// the confidence head asked for, the same wave then computes c_k from h_k
// and the previous token's W1 row (caijizhuo section 四: the loop scores each
// position right after drawing it).
template <typename Elt>
__global__ __launch_bounds__(256) void sample_finalize(int R, int gamma, int V, int r,
                                                       const typename Elt::T* __restrict__ U,
                                                       const typename Elt::T* __restrict__ W1,
                                                       const typename Elt::T* __restrict__ W2t,
                                                       const int32_t* __restrict__ x0, SampleWs ws,
                                                       int nPart, int32_t* __restrict__ x,
                                                       float* __restrict__ lse, float* __restrict__ logit,
                                                       const typename Elt::T* __restrict__ bvec,
                                                       int32_t* __restrict__ status, SampleConf conf) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(R) * gamma) return;
  if (status && row == 0 && lane == 0) *status = ws.bar[1] != 0u ? DSPARK_ETIMEOUT : DSPARK_OK;
  const int req = static_cast<int>(row / gamma);
  const int k = static_cast<int>(row % gamma);
  // Every load that needs no token goes out first, together: the time-out
  // flag, the key slots of positions k (the drawn token) and k - 1 (the
  // previous one), the first log-sum-exp partials and the first batch of
  // the hidden-state row.  The loads that need the tokens (the W1 and W2t
  // rows of the bias dot, the drawn token's logit, the confidence head's W1
  // part) then go out together as well: two round trips to memory per row.
  const unsigned int timed_out = ws.bar[1];
  unsigned long long kd[kMaxKeySlots], kq[kMaxKeySlots];
  const unsigned long long* kpd = ws.keys + static_cast<int64_t>(k) * ws.slots * R + req;
#pragma unroll
  for (int sl = 0; sl < kMaxKeySlots; ++sl) {
    kd[sl] = sl < ws.slots ? kpd[static_cast<int64_t>(sl) * R] : 0ull;
    kq[sl] = k > 0 && sl < ws.slots ? kpd[static_cast<int64_t>(sl - ws.slots) * R] : 0ull;
  }
  const int x0v = x0[req];
  constexpr int kLp = 4;   // partials per lane loaded up front
  const float2* lp = ws.lsep + (static_cast<int64_t>(k) * R + req) * nPart;
  float2 lpv[kLp];
#pragma unroll
  for (int q = 0; q < kLp; ++q) lpv[q] = lane + 64 * q < nPart ? lp[lane + 64 * q] : make_float2(neg_inf(), 0.f);
  using T = typename Elt::T;
  const T* hrow = conf.h ? static_cast<const T*>(conf.h) + row * conf.d : nullptr;
  const T* cw = static_cast<const T*>(conf.w);
  ConfH<Elt> cb;
  if (conf.h) conf_h_issue<Elt>(cb, hrow, cw, conf.d, lane * Vec16<Elt>::N);

  if (status && row == 0 && lane == 0) *status = timed_out != 0u ? DSPARK_ETIMEOUT : DSPARK_OK;
  unsigned long long bd = 0, bq = 0;
#pragma unroll
  for (int sl = 0; sl < kMaxKeySlots; ++sl) {
    bd = kd[sl] > bd ? kd[sl] : bd;
    bq = kq[sl] > bq ? kq[sl] : bq;
  }
  const int drawn = token_or_none(key_token(bd), V);
  const int prevk = k == 0 ? token_or_none(x0v, V) : token_or_none(key_token(bq), V);
  const int prev = bvec ? -1 : prevk;
  // the confidence head's previous token: the anchor, else the token this
  // kernel emits for position k - 1 (token 0 where no key was drawn, -1 after
  // a time-out)
  const int prev_conf = k == 0 ? prevk : (timed_out != 0u ? -1 : (prevk < 0 ? 0 : prevk));
  const int tok = drawn < 0 ? 0 : drawn;   // every position draws a token in [0, V)
  // the bias dot's first kBq elements per lane and the drawn token's logit
  constexpr int kBq = 4;
  const T* e = bvec ? bvec + row * r : (prev >= 0 ? W1 + static_cast<int64_t>(prev) * r : nullptr);
  float ev[kBq], wv[kBq];
#pragma unroll
  for (int q = 0; q < kBq; ++q) {
    const int i = lane + 64 * q;
    ev[q] = e && i < r ? Elt::load(e, i) : 0.f;
    wv[q] = e && i < r ? Elt::load(W2t, static_cast<int64_t>(tok) * r + i) : 0.f;
  }
  const float utok = Elt::load(U, row * V + tok);

  Lse run{neg_inf(), 0.f};
#pragma unroll
  for (int q = 0; q < kLp; ++q)
    if (lane + 64 * q < nPart) run = lse_combine(run, Lse{lpv[q].x, lpv[q].y});
  for (int p = lane + 64 * kLp; p < nPart; p += 64) {
    const float2 v = lp[p];
    run = lse_combine(run, Lse{v.x, v.y});
  }
  if (conf.h) {
    const float zz = conf_finish<Elt>(conf_h_fold<Elt>(cb, hrow, cw, conf.d, lane), cw, conf.d, W1, r, prev_conf,
                                      lane);
    if (lane == 0) {
      conf.c[row] = sigmoid_stable(zz / (conf.T ? conf.T[k] : 1.f));
      if (conf.z) conf.z[row] = zz;
    }
  }
  if (timed_out != 0u) {   // the persistent launch timed out at a grid barrier: no valid draw
    if (lane == 0) {
      x[row] = -1;
      lse[row] = __builtin_nanf("");
      logit[row] = __builtin_nanf("");
    }
    return;
  }
  run = wave_reduce_lse(run);
  float b = 0.f;
  if (e) {
#pragma unroll
    for (int q = 0; q < kBq; ++q)
      if (lane + 64 * q < r) b = fmaf(ev[q], wv[q], b);
    for (int i = lane + 64 * kBq; i < r; i += 64)
      b = fmaf(Elt::load(e, i), Elt::load(W2t, static_cast<int64_t>(tok) * r + i), b);
  }
  b = wave_reduce_sum(b);
  if (lane == 0) {
    x[row] = tok;
    lse[row] = run.M + logf(run.S);
    logit[row] = utok + b;
  }
}

// ------------------------------------------------------------------ host side

int compute_units();   // abi.hip

int sample_parts(dspark_dtype dt, int V) {
  const int nC = ceil_div(V, kChunk);
  return dt == DSPARK_BF16 ? (nC < kMaxSampleWGs ? nC : kMaxSampleWGs) : nC;
}

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

static size_t key_words(int R, int gamma) {   // the key area, sized for the most slots
  return static_cast<size_t>(kMaxKeySlots) * R * gamma;
}
static size_t cleared_words(int R, int gamma) {   // keys + barrier words
  return key_words(R, gamma) + kBarWords;
}
size_t sample_workspace_bytes(dspark_dtype dt, int R, int gamma, int V) {
  return align256(sizeof(unsigned long long) * cleared_words(R, gamma)) +
         sizeof(float2) * static_cast<size_t>(gamma) * R * sample_parts(dt, V);
}

static SampleWs carve(void* ws, int R, int gamma, int slots) {
  SampleWs w;
  w.slots = slots;
  w.keys = static_cast<unsigned long long*>(ws);
  w.bar = reinterpret_cast<unsigned int*>(w.keys + key_words(R, gamma));
  w.lsep = reinterpret_cast<float2*>(static_cast<char*>(ws) + align256(sizeof(unsigned long long) * cleared_words(R, gamma)));
  return w;
}

// Request groups of 64 (R <= 64) or 128 rows; one work group per compute
// unit across all groups.
static int sample_nbw(int R) { return R <= 64 ? 1 : 2; }
// Work groups along the vocabulary for the persistent 32x32x16 path: one
// per compute unit across all request groups, and at most one per tile pair,
// so the whole grid is resident at once (the grid barrier needs it).  0 when
// the request groups alone outnumber the compute units.  Every bf16 batch
// that fits takes this path: at 1 and 32 requests it measured 12 % and 16 %
// faster than one 16x16x32 launch per position.
static int wide_grid_x(int R, int V) {
  const int groups = ceil_div(R, R <= 64 ? 64 : 128);
  const int gx = compute_units() / groups;
  const int nPairs = ceil_div(ceil_div(V, kChunk), 2);
  return gx < 1 ? 0 : (gx < nPairs ? gx : nPairs);
}

static int bf16_grid_x(int R, int V) {
  const int groups = ceil_div(R, kTileWaves * 16 * sample_nbw(R));
  int gx = compute_units() / groups;
  if (gx < 1) gx = 1;
  const int nC = ceil_div(V, kChunk);
  if (gx > nC) gx = nC;
  if (gx > kMaxSampleWGs) gx = kMaxSampleWGs;
  return gx;
}

// Where each (request, position) takes its bias vector from: the previous
// token's W1 row (the Markov head, bvec null) or bvec [R][gamma][r].
struct SampleArgs {
  int R, gamma, V;
  const void *U, *W1, *W2t, *bvec;
  const int32_t* x0;
  const float *G, *g;
  const uint32_t* cancel;   // nullable: a non-zero word ends the grid-barrier waits
  hipEvent_t ev0, ev1;      // nullable: recorded at the start and the end of the position sweep
};

template <int NBW, int KS, bool VEC>
static void launch_step_bf16(const SampleArgs& a, int k, const SampleWs& w, int gx, hipStream_t s) {
  dim3 grid(gx, ceil_div(a.R, sample_reqs_per_wg<NBW>()));
  hipLaunchKernelGGL((sample_step_bf16<NBW, KS, VEC>), grid, dim3(kTileThreads), 0, s, a.R, a.gamma, a.V, k,
                     static_cast<const uint16_t*>(a.U), static_cast<const uint16_t*>(a.W1),
                     static_cast<const uint16_t*>(a.W2t), a.x0, a.G, a.g, w, gx,
                     static_cast<const uint16_t*>(a.bvec));
}

template <int RQ, int KS16, bool VEC>
static void launch_steps_wide(const SampleArgs& a, int kb, int ke, const SampleWs& w, int gx, hipStream_t s) {
  dim3 grid(gx, ceil_div(a.R, 32 * RQ));
  // with events, the runtime stamps them with the launch's own start and end
  hipExtLaunchKernelGGL((sample_steps_wide<RQ, KS16, VEC>), grid, dim3(wide_threads<RQ>()), 0, s, a.ev0, a.ev1, 0,
                        a.R, a.gamma, a.V, static_cast<const uint16_t*>(a.U), static_cast<const uint16_t*>(a.W1),
                        static_cast<const uint16_t*>(a.W2t), a.x0, a.G, a.g, w, gx, kb, ke,
                        static_cast<const uint16_t*>(a.bvec), a.cancel);
}

// Whether one work group of the persistent kernel fits on a compute unit
// (registers, LDS and threads), asked of the runtime once per device: the
// grid barrier needs the whole grid resident, one work group per compute
// unit.  When it does not fit, the sampler takes the per-position launches.
template <int RQ, int KS16, bool VEC>
static bool wide_fits() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, reinterpret_cast<const void*>(&sample_steps_wide<RQ, KS16, VEC>), wide_threads<RQ>(), 0);
    v = (e == hipSuccess && n >= 1) ? 1 : 2;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1;
}

template <int KS16>
static bool wide_fits_ks(int R, int V) {
  const bool vec = (V % kGChunk) == 0;
  if (R <= 64) return vec ? wide_fits<2, KS16, true>() : wide_fits<2, KS16, false>();
  return vec ? wide_fits<4, KS16, true>() : wide_fits<4, KS16, false>();
}

static bool wide_fits_r(int R, int V, int r) {
  switch (r / 32) {
    case 1: return wide_fits_ks<2>(R, V);
    case 2: return wide_fits_ks<4>(R, V);
    case 4: return wide_fits_ks<8>(R, V);
    default: return wide_fits_ks<16>(R, V);
  }
}

template <int KS16>
static void launch_steps_wide_ks(const SampleArgs& a, int kb, int ke, const SampleWs& w, int gx, hipStream_t s) {
  const bool vec = (a.V % kGChunk) == 0;
  if (a.R <= 64) {
    if (vec) launch_steps_wide<2, KS16, true>(a, kb, ke, w, gx, s);
    else launch_steps_wide<2, KS16, false>(a, kb, ke, w, gx, s);
  } else {
    if (vec) launch_steps_wide<4, KS16, true>(a, kb, ke, w, gx, s);
    else launch_steps_wide<4, KS16, false>(a, kb, ke, w, gx, s);
  }
}

template <int KS>
static void launch_step_bf16_ks(const SampleArgs& a, int k, const SampleWs& w, int gx, hipStream_t s) {
  // the vector path loads a lane's sixteen logits as two aligned 16-byte
  // pieces: rows must start on 16 bytes and hold whole Gumbel chunks
  const bool vec = (a.V % kGChunk) == 0;
  if (sample_nbw(a.R) == 1) {
    if (vec) launch_step_bf16<1, KS, true>(a, k, w, gx, s);
    else launch_step_bf16<1, KS, false>(a, k, w, gx, s);
  } else {
    if (vec) launch_step_bf16<2, KS, true>(a, k, w, gx, s);
    else launch_step_bf16<2, KS, false>(a, k, w, gx, s);
  }
}

// sample_res.hip: the Markov-head loop with W2t held in registers
int res_grid_x(int R, int V, int r, int max_wgs);
bool res_usable(int R, int V, int r, int max_wgs);
hipError_t res_launch(int R, int gamma, int V, int r, const void* U, const void* W1, const void* W2t,
                      const int32_t* x0, const float* G, const float* g, const SampleWs& w, int gx, int kb, int ke,
                      const uint32_t* cancel, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s);

// sample_pipe.hip: the Markov-head loop with W2t held on chip and one grid
// barrier per request block (more than 64 requests)
int pipe_grid(int R, int V, int r, int max_wgs);
hipError_t pipe_launch(int R, int gamma, int V, int r, const void* U, const void* W1, const void* W2t,
                       const int32_t* x0, const float* G, const float* g, const SampleWs& w, int gx,
                       const uint32_t* cancel, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s);

// rnn.hip: the RNN head's projection and gating for position k (reads the
// keys of position k - 1 for the previous token); the hidden-state part of
// the projection for every position (bf16), run before the first
hipError_t rnn_step_launch(dspark_dtype dt, const RnnHead& h, int R, int gamma, int V, int r, int k,
                           const void* W1, const int32_t* x0, const unsigned long long* keys, hipStream_t s);
hipError_t rnn_hproj_launch(const RnnHead& hd, int R, int gamma, int r, hipStream_t s);

// sample_res.hip: the RNN head inside the W2t-on-chip persistent launch
bool res_rnn_usable(int R, int V, int r, int max_wgs);
hipError_t res_rnn_launch(int R, int gamma, int V, int r, const void* U, const void* W1, const void* W2t,
                          const int32_t* x0, const float* G, const float* g, const SampleWs& w, int gx,
                          const uint32_t* cancel, const void* Wrnn, const float* Yh, int d, float* st, void* o,
                          const float* P, hipStream_t s);

// The kernel sample_launch runs the Markov-head positions with, for a shape
// (the same choice, in the same order).
const char* sample_kernel_name(dspark_dtype dt, int R, int V, int r) {
  if (dt == DSPARK_BF16 && pipe_grid(R, V, r, kMaxSampleWGs) > 0)
    return "sample_steps_pipe: W2t held on chip, one grid barrier per block of 32 requests, all positions in one persistent launch";
  if (dt == DSPARK_BF16 && res_usable(R, V, r, kMaxSampleWGs))
    return "sample_steps_res: W2t held in registers, all positions in one persistent launch";
  if (dt == DSPARK_BF16 && wide_fits_r(R, V, r))
    return "sample_steps_wide: W2t streamed through LDS, all positions in one persistent launch";
  return dt == DSPARK_BF16 ? "sample_step_bf16: one launch per position" : "sample_step_f32: one launch per position";
}

const char* rnn_kernel_name(dspark_dtype dt, int R, int V, int r) {
  if (dt == DSPARK_BF16 && res_rnn_usable(R, V, r, kMaxSampleWGs))
    return "sample_steps_res with the RNN step: W2t held on chip, the step between two grid barriers per position, all positions in one persistent launch";
  if (dt == DSPARK_BF16 && wide_fits_r(R, V, r))
    return "rnn_step_bf16 and a one-position sample_steps_wide launch per position: W2t streamed through LDS";
  return dt == DSPARK_BF16 ? "rnn_step_bf16 and sample_step_bf16 per position"
                           : "rnn_proj_f32, rnn_gate and sample_step_f32 per position";
}

hipError_t sample_launch(dspark_dtype dt, int R, int gamma, int V, int r, const void* U,
                         const void* W1, const void* W2t, const int32_t* x0, const float* G,
                         const float* g, int32_t* x, float* lse, float* logit, void* ws,
                         hipStream_t s, const RnnHead* rnn, const uint32_t* cancel, int32_t* status,
                         const SampleConf* conf, hipEvent_t ev0, hipEvent_t ev1) {
  const SampleConf cf = conf ? *conf : SampleConf{nullptr, nullptr, 0, nullptr, nullptr, nullptr};
  // bf16 Markov head: W2t held in registers when the vocabulary fits the
  // register files (res), else streamed through LDS at every position (wide)
  const int gxp = dt == DSPARK_BF16 && !rnn ? pipe_grid(R, V, r, kMaxSampleWGs) : 0;
  // the RNN head keeps W2t on chip too where its projection fits between
  // two grid barriers per position (rnn_phase in sample_res.hip)
  const bool rnn_res = rnn && dt == DSPARK_BF16 && res_rnn_usable(R, V, r, kMaxSampleWGs);
  const int gxr = gxp == 0 && dt == DSPARK_BF16 && ((!rnn && res_usable(R, V, r, kMaxSampleWGs)) || rnn_res)
                      ? res_grid_x(R, V, r, kMaxSampleWGs)
                      : 0;
  const int gxw = gxp == 0 && gxr == 0 && dt == DSPARK_BF16 && wide_fits_r(R, V, r) ? wide_grid_x(R, V) : 0;
  const SampleWs w = carve(ws, R, gamma, gxp > 0 ? kPipeKeySlots : kKeySlots);
  // the one-launch sweeps stamp the events themselves; the per-position
  // paths record them around all their launches
  const bool one_launch = (gxp > 0 || gxr > 0 || gxw > 0) && !rnn;
  const SampleArgs a{R, gamma, V, U, W1, W2t, rnn ? rnn->o : nullptr, x0, G, g, cancel,
                     one_launch ? ev0 : nullptr, one_launch ? ev1 : nullptr};
  const int nPart = gxp > 0 ? gxp : gxr > 0 ? gxr : gxw > 0 ? gxw : dt == DSPARK_BF16 ? bf16_grid_x(R, V) : ceil_div(V, kChunk);
  const int64_t nkeys = static_cast<int64_t>(w.slots) * R * gamma;
  hipLaunchKernelGGL(sample_init, dim3(ceil_div(nkeys + kBarWords, 256) < 1024 ? ceil_div(nkeys + kBarWords, 256) : 1024),
                     dim3(256), 0, s, w.keys, nkeys, reinterpret_cast<unsigned long long*>(w.bar));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // the positions one launch covers: all of them with the Markov head (the
  // persistent path meets at a grid barrier between positions), one at a
  // time with the RNN head (its projection runs between positions)
  const int span = rnn ? 1 : gamma;
  const bool record = ev0 && ev1 && !one_launch;
  if (record && (err = hipEventRecord(ev0, s)) != hipSuccess) return err;
  if (gxp > 0 &&
      (err = pipe_launch(R, gamma, V, r, U, W1, W2t, x0, G, g, w, gxp, cancel, ev0, ev1, s)) != hipSuccess)
    return err;
  if (gxr > 0 && !rnn &&
      (err = res_launch(R, gamma, V, r, U, W1, W2t, x0, G, g, w, gxr, 0, gamma, cancel, ev0, ev1, s)) != hipSuccess)
    return err;
  if (gxr > 0 && rnn) {
    if ((err = rnn_hproj_launch(*rnn, R, gamma, r, s)) != hipSuccess) return err;
    if ((err = res_rnn_launch(R, gamma, V, r, U, W1, W2t, x0, G, g, w, gxr, cancel, rnn->W, rnn->part, rnn->d,
                              rnn->s, rnn->o, rnn->P, s)) != hipSuccess)
      return err;
  }
  for (int kb = 0; gxp == 0 && gxr == 0 && kb < gamma; kb += span) {
    if (rnn && (err = rnn_step_launch(dt, *rnn, R, gamma, V, r, kb, W1, x0, w.keys, s)) != hipSuccess) return err;
    if (gxw > 0) {
      switch (r / 32) {
        case 1: launch_steps_wide_ks<2>(a, kb, kb + span, w, nPart, s); break;
        case 2: launch_steps_wide_ks<4>(a, kb, kb + span, w, nPart, s); break;
        case 4: launch_steps_wide_ks<8>(a, kb, kb + span, w, nPart, s); break;
        default: launch_steps_wide_ks<16>(a, kb, kb + span, w, nPart, s); break;
      }
      if ((err = hipGetLastError()) != hipSuccess) return err;
      continue;
    }
    for (int k = kb; k < kb + span; ++k) {
      if (dt == DSPARK_BF16) {
        switch (r / 32) {
          case 1: launch_step_bf16_ks<1>(a, k, w, nPart, s); break;
          case 2: launch_step_bf16_ks<2>(a, k, w, nPart, s); break;
          case 4: launch_step_bf16_ks<4>(a, k, w, nPart, s); break;
          default: launch_step_bf16_ks<8>(a, k, w, nPart, s); break;
        }
      } else {
        hipLaunchKernelGGL(sample_step_f32, dim3(nPart, R), dim3(64), 0, s, R, gamma, V, r, k,
                           static_cast<const float*>(U), static_cast<const float*>(W1),
                           static_cast<const float*>(W2t), x0, G, g, w, nPart, static_cast<const float*>(a.bvec));
      }
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  if (record && (err = hipEventRecord(ev1, s)) != hipSuccess) return err;
  const int blocks = ceil_div(static_cast<int64_t>(R) * gamma, 4);
  if (dt == DSPARK_BF16)
    hipLaunchKernelGGL(sample_finalize<BF16>, dim3(blocks), dim3(256), 0, s, R, gamma, V, r,
                       static_cast<const uint16_t*>(U), static_cast<const uint16_t*>(W1),
                       static_cast<const uint16_t*>(W2t), x0, w, nPart, x, lse, logit,
                       static_cast<const uint16_t*>(a.bvec), status, cf);
  else
    hipLaunchKernelGGL(sample_finalize<F32>, dim3(blocks), dim3(256), 0, s, R, gamma, V, r,
                       static_cast<const float*>(U), static_cast<const float*>(W1),
                       static_cast<const float*>(W2t), x0, w, nPart, x, lse, logit,
                       static_cast<const float*>(a.bvec), status, cf);
  return hipGetLastError();
}

}  // namespace dspark
