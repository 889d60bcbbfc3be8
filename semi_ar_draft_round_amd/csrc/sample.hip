// dspark_markov_sample: the semi-autoregressive gamma-step loop.
//
// Passage: DSpark reading notes, eq (4) (p_k(v) ∝ exp(U_k(v) + B_k(v))) and
// eq (5) (B(x_{k-1}, .) = W1[x_{k-1}] W2); caijizhuo summary, section 四
// (the sequential loop carries only the sampled token).
//
// A call is gamma + 2 launches: sample_init clears the argmax keys, then one
// sample_step_* launch per position, then sample_finalize.  sample_step_*
// streams U_k and W2t once, builds the Markov bias of a 64-token tile for all
// requests on the matrix cores, and folds each 16-token Gumbel chunk into
// running per-request state: the log-sum-exp (for lse) and the chunk-level
// Gumbel-max (score LSE_c + G_c), keeping the best chunk's logits for the
// in-chunk draw (argmax of l_v + g_{v mod 16}), which is made once at the end
// of the sweep.  Each work group then merges its draw into the request's key
// with one 64-bit atomic max (eight key slots per request spread the
// contention) and stores its log-sum-exp partial.  The next position's
// launch reads the keys back as its previous tokens.  sample_finalize decodes
// x, merges the log-sum-exp partials and recomputes the logit of each
// drafted token.
#include "bias_tile.hpp"

namespace dspark {

// Upper bound on the work groups per position along the vocabulary (the
// bf16 kernel runs one work group per compute unit); sizes the workspace.
constexpr int kMaxSampleWGs = 1024;
// Argmax key slots per (position, request); work group b uses slot b % 8.
constexpr int kKeySlots = 8;

template <int NBW>
__host__ __device__ constexpr int sample_reqs_per_wg() { return kTileWaves * 16 * NBW; }

struct SampleWs {
  unsigned long long* keys;   // [gamma][kKeySlots][R]
  float2* lsep;               // [gamma][R][nPart]  (M, S) log-sum-exp partials
};

// Token drawn at position k-1 (or the anchor at k = 0).
__device__ __forceinline__ int previous_token(const unsigned long long* keys, const int32_t* x0, int R,
                                              int V, int k, int req) {
  if (k == 0) return token_or_none(x0[req], V);
  unsigned long long best = 0;
  const unsigned long long* kp = keys + static_cast<int64_t>(k - 1) * kKeySlots * R + req;
#pragma unroll
  for (int s = 0; s < kKeySlots; ++s) {
    const unsigned long long v = kp[static_cast<int64_t>(s) * R];
    best = v > best ? v : best;
  }
  return token_or_none(key_token(best), V);
}

__global__ __launch_bounds__(256) void sample_init(unsigned long long* keys, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    keys[i] = 0ull;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Sixteen bf16 -inf words: the logits read for tokens past V, so that they
// drop out of every reduction without a per-element test.
__device__ u32x4 kNegInfBf16x16[2] = {{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u},
                                            {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u}};

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

// MFMA C operand of M-block mb: the lane's tokens 4 mb .. 4 mb + 3 as fp32.
__device__ __forceinline__ f32x4 lane16_c(const u32x4 (&u)[2], int mb) {
  const uint32_t w0 = u[mb >> 1][2 * (mb & 1)];
  const uint32_t w1 = u[mb >> 1][2 * (mb & 1) + 1];
  return f32x4{__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u), __uint_as_float(w1 << 16),
               __uint_as_float(w1 & 0xFFFF0000u)};
}

// Running state of one lane for one request: the log-sum-exp of every chunk
// it has folded (T * 2^M2, base 2) and the best chunk so far under the
// chunk-level Gumbel-max (score log2(e) * (LSE_c + G_c) and its first token).
// The best chunk's sixteen logits, needed for the in-chunk draw at the end,
// are kept in LDS (`keep`, four f32x4 at a stride of kTileThreads).
struct LaneDraw {
  float M2, T;
  float best;
  int first;
};

__device__ __forceinline__ void lane_draw_init(LaneDraw& d) {
  d.M2 = neg_inf();
  d.T = 0.f;
  d.best = neg_inf();
  d.first = -1;
}

// Fold one Gumbel chunk (the lane's sixteen logits l, first token `first`,
// chunk Gumbel G) into the lane's state.  Chunks with no finite logit get a
// score of -inf and add nothing.
__device__ __forceinline__ bool fold_chunk(const f32x4 (&acc)[4], float G, int first, LaneDraw& d) {
  float l[kGChunk];
#pragma unroll
  for (int c = 0; c < kGChunk; ++c) l[c] = acc[c >> 2][c & 3];
  float m = l[0];
#pragma unroll
  for (int c = 1; c < kGChunk; ++c) m = fmaxf(m, l[c]);
  const float m2 = (m == neg_inf() ? 0.f : m) * kLog2e;
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kGChunk; ++c) s4[c & 3] += __builtin_amdgcn_exp2f(fmaf(l[c], kLog2e, -m2));
  const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  const float score = fmaf(G, kLog2e, m2 + __builtin_amdgcn_logf(s));
  const float Mn = fmaxf(d.M2, m2);
  d.T = d.T * __builtin_amdgcn_exp2f(d.M2 - Mn) + s * __builtin_amdgcn_exp2f(m2 - Mn);
  d.M2 = Mn;
  const bool take = score > d.best;   // strict: the earlier chunk keeps ties
  d.best = take ? score : d.best;
  d.first = take ? first : d.first;
  return take;
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
    const float* __restrict__ g, SampleWs ws, int nPart) {
  static_assert(kGChunk == 16 && kChunk == 64, "one Gumbel chunk per lane and M-block column of four");
  constexpr int NROWS = sample_reqs_per_wg<NBW>();
  constexpr int kW = tile_bytes(KS);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kW];
  __shared__ float gsh[NROWS][kGChunk];        // in-chunk Gumbels of the group's requests
  // each lane's best chunk per request group: [nb][mb][thread], flat
  __shared__ f32x4 keepsh[NBW * 4 * kTileThreads];
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
  for (int nb = 0; nb < NBW; ++nb) prev[nb] = live[nb] ? previous_token(ws.keys, x0, R, V, k, req[nb]) : -1;
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
  load_w1_frags<NBW, KS>(e, W1, prev);

  LaneDraw dr[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    lane_draw_init(dr[nb]);
    *reinterpret_cast<f32x4*>(&gsh[loc[nb]][4 * q]) = gq[nb];
  }
  store_w2_tile_lane16<KS>(lds, wr);
  load_w2_regs<KS>(wr, W2t, V, tile_of(clampc(1)) * kChunk);
  __syncthreads();

  // tile `it` from LDS half it & 1 and register set `cur`; refills `cur` with
  // tile it + 2, then stores tile it + 1 into the other half and issues the
  // W2t loads of tile it + 2
  auto step = [&](int it, LaneLoads<NBW>& cur) {
    const int v0 = tile_of(it) * kChunk;
    f32x4 acc[4][NBW];
    float Gc[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = lane16_c(cur.u[nb], mb);
      Gc[nb] = cur.G[nb];
    }
    load_lane(cur, clampc(it + 2));
    bias_tile_acc<NBW, KS>(acc, lds + (it & 1) * kW, e);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      f32x4 a[4] = {acc[0][nb], acc[1][nb], acc[2][nb], acc[3][nb]};
      if (fold_chunk(a, Gc[nb], v0 + q * kGChunk, dr[nb])) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) keepsh[(nb * 4 + mb) * kTileThreads + threadIdx.x] = a[mb];
      }
    }
    store_w2_tile_lane16<KS>(lds + ((it + 1) & 1) * kW, wr);
    load_w2_regs<KS>(wr, W2t, V, tile_of(clampc(it + 2)) * kChunk);
    __syncthreads();
  };
  // pairs of tiles, so every path back to the loop head has issued both
  // register sets' loads in the same order; an odd last tile follows the loop
  int it = 0;
  for (; it + 1 < nT; it += 2) {
    step(it, even);
    step(it + 1, odd);
  }
  if (it < nT) step(it, even);

  // the in-chunk draw on each lane's best chunk, then the best of the four
  // lanes of a request, merged across work groups by atomic max
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const float* gl = gsh[loc[nb]];
    float kept[kGChunk];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const f32x4 v = keepsh[(nb * 4 + mb) * kTileThreads + threadIdx.x];
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
        atomicMax(ws.keys + (static_cast<int64_t>(k) * kKeySlots + blockIdx.x % kKeySlots) * R + req[nb], key);
    }
  }
}

// fp32 storage, any rank: one wave per (64-token tile, request), plain FMA
// bias; each sixteen-lane quarter of the wave is one Gumbel chunk.
__global__ __launch_bounds__(64) void sample_step_f32(
    int R, int gamma, int V, int r, int k, const float* __restrict__ U, const float* __restrict__ W1,
    const float* __restrict__ W2t, const int32_t* __restrict__ x0, const float* __restrict__ G,
    const float* __restrict__ g, SampleWs ws, int nPart) {
  const int tile = blockIdx.x;
  const int req = blockIdx.y;
  const int lane = threadIdx.x;
  const int nG = (V + kGChunk - 1) / kGChunk;
  const int prev = previous_token(ws.keys, x0, R, V, k, req);
  const int v = tile * kChunk + lane;
  const int64_t rowk = static_cast<int64_t>(req) * gamma + k;
  float val = neg_inf();
  if (v < V) {
    float b = 0.f;
    if (prev >= 0) {
      const float* e = W1 + static_cast<int64_t>(prev) * r;
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
      atomicMax(ws.keys + (static_cast<int64_t>(k) * kKeySlots + tile % kKeySlots) * R + req,
                pack_key(ch.score, ch.tok));
  }
}

// Decode x, merge the log-sum-exp partials and recompute each drafted
// token's logit U_k(x_k) + W1[x_{k-1}] . W2t[x_k]: one wave per (request, k).
template <typename Elt>
__global__ __launch_bounds__(256) void sample_finalize(int R, int gamma, int V, int r,
                                                       const typename Elt::T* __restrict__ U,
                                                       const typename Elt::T* __restrict__ W1,
                                                       const typename Elt::T* __restrict__ W2t,
                                                       const int32_t* __restrict__ x0, SampleWs ws,
                                                       int nPart, int32_t* __restrict__ x,
                                                       float* __restrict__ lse, float* __restrict__ logit) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(R) * gamma) return;
  const int req = static_cast<int>(row / gamma);
  const int k = static_cast<int>(row % gamma);
  const int drawn = previous_token(ws.keys, x0, R, V, k + 1, req);
  const int tok = drawn < 0 ? 0 : drawn;   // every position draws a token in [0, V)
  const int prev = previous_token(ws.keys, x0, R, V, k, req);
  Lse run{neg_inf(), 0.f};
  const float2* lp = ws.lsep + (static_cast<int64_t>(k) * R + req) * nPart;
  for (int p = lane; p < nPart; p += 64) {
    const float2 v = lp[p];
    run = lse_combine(run, Lse{v.x, v.y});
  }
  run = wave_reduce_lse(run);
  float b = 0.f;
  if (prev >= 0)
    for (int i = lane; i < r; i += 64)
      b = fmaf(Elt::load(W1, static_cast<int64_t>(prev) * r + i), Elt::load(W2t, static_cast<int64_t>(tok) * r + i), b);
  b = wave_reduce_sum(b);
  if (lane == 0) {
    x[row] = tok;
    lse[row] = run.M + logf(run.S);
    logit[row] = Elt::load(U, row * V + tok) + b;
  }
}

// ------------------------------------------------------------------ host side

int compute_units();   // abi.hip

int sample_parts(dspark_dtype dt, int V) {
  const int nC = ceil_div(V, kChunk);
  return dt == DSPARK_BF16 ? (nC < kMaxSampleWGs ? nC : kMaxSampleWGs) : nC;
}

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t sample_workspace_bytes(dspark_dtype dt, int R, int gamma, int V) {
  return align256(sizeof(unsigned long long) * kKeySlots * static_cast<size_t>(R) * gamma) +
         sizeof(float2) * static_cast<size_t>(gamma) * R * sample_parts(dt, V);
}

static SampleWs carve(void* ws, int R, int gamma) {
  SampleWs w;
  w.keys = static_cast<unsigned long long*>(ws);
  w.lsep = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                     align256(sizeof(unsigned long long) * kKeySlots * static_cast<size_t>(R) * gamma));
  return w;
}

// Request groups of 64 (R <= 64) or 128 rows; one work group per compute
// unit across all groups.
static int sample_nbw(int R) { return R <= 64 ? 1 : 2; }

static int bf16_grid_x(int R, int V) {
  const int groups = ceil_div(R, kTileWaves * 16 * sample_nbw(R));
  int gx = compute_units() / groups;
  if (gx < 1) gx = 1;
  const int nC = ceil_div(V, kChunk);
  if (gx > nC) gx = nC;
  if (gx > kMaxSampleWGs) gx = kMaxSampleWGs;
  return gx;
}

template <int NBW, int KS, bool VEC>
static void launch_step_bf16(int R, int gamma, int V, int k, const void* U, const void* W1,
                             const void* W2t, const int32_t* x0, const float* G, const float* g,
                             const SampleWs& w, int gx, hipStream_t s) {
  dim3 grid(gx, ceil_div(R, sample_reqs_per_wg<NBW>()));
  hipLaunchKernelGGL((sample_step_bf16<NBW, KS, VEC>), grid, dim3(kTileThreads), 0, s, R, gamma, V, k,
                     static_cast<const uint16_t*>(U), static_cast<const uint16_t*>(W1),
                     static_cast<const uint16_t*>(W2t), x0, G, g, w, gx);
}

template <int KS>
static void launch_step_bf16_ks(int R, int gamma, int V, int k, const void* U, const void* W1,
                                const void* W2t, const int32_t* x0, const float* G, const float* g,
                                const SampleWs& w, int gx, hipStream_t s) {
  // the vector path loads a lane's sixteen logits as two aligned 16-byte
  // pieces: rows must start on 16 bytes and hold whole Gumbel chunks
  const bool vec = (V % kGChunk) == 0;
  if (sample_nbw(R) == 1) {
    if (vec) launch_step_bf16<1, KS, true>(R, gamma, V, k, U, W1, W2t, x0, G, g, w, gx, s);
    else launch_step_bf16<1, KS, false>(R, gamma, V, k, U, W1, W2t, x0, G, g, w, gx, s);
  } else {
    if (vec) launch_step_bf16<2, KS, true>(R, gamma, V, k, U, W1, W2t, x0, G, g, w, gx, s);
    else launch_step_bf16<2, KS, false>(R, gamma, V, k, U, W1, W2t, x0, G, g, w, gx, s);
  }
}

hipError_t sample_launch(dspark_dtype dt, int R, int gamma, int V, int r, const void* U,
                         const void* W1, const void* W2t, const int32_t* x0, const float* G,
                         const float* g, int32_t* x, float* lse, float* logit, void* ws,
                         hipStream_t s) {
  const SampleWs w = carve(ws, R, gamma);
  const int nPart = dt == DSPARK_BF16 ? bf16_grid_x(R, V) : ceil_div(V, kChunk);
  const int64_t nkeys = static_cast<int64_t>(kKeySlots) * R * gamma;
  hipLaunchKernelGGL(sample_init, dim3(ceil_div(nkeys, 256) < 1024 ? ceil_div(nkeys, 256) : 1024),
                     dim3(256), 0, s, w.keys, nkeys);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  for (int k = 0; k < gamma; ++k) {
    if (dt == DSPARK_BF16) {
      switch (r / 32) {
        case 1: launch_step_bf16_ks<1>(R, gamma, V, k, U, W1, W2t, x0, G, g, w, nPart, s); break;
        case 2: launch_step_bf16_ks<2>(R, gamma, V, k, U, W1, W2t, x0, G, g, w, nPart, s); break;
        case 4: launch_step_bf16_ks<4>(R, gamma, V, k, U, W1, W2t, x0, G, g, w, nPart, s); break;
        default: launch_step_bf16_ks<8>(R, gamma, V, k, U, W1, W2t, x0, G, g, w, nPart, s); break;
      }
    } else {
      hipLaunchKernelGGL(sample_step_f32, dim3(nPart, R), dim3(64), 0, s, R, gamma, V, r, k,
                         static_cast<const float*>(U), static_cast<const float*>(W1),
                         static_cast<const float*>(W2t), x0, G, g, w, nPart);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int blocks = ceil_div(static_cast<int64_t>(R) * gamma, 4);
  if (dt == DSPARK_BF16)
    hipLaunchKernelGGL(sample_finalize<BF16>, dim3(blocks), dim3(256), 0, s, R, gamma, V, r,
                       static_cast<const uint16_t*>(U), static_cast<const uint16_t*>(W1),
                       static_cast<const uint16_t*>(W2t), x0, w, nPart, x, lse, logit);
  else
    hipLaunchKernelGGL(sample_finalize<F32>, dim3(blocks), dim3(256), 0, s, R, gamma, V, r,
                       static_cast<const float*>(U), static_cast<const float*>(W1),
                       static_cast<const float*>(W2t), x0, w, nPart, x, lse, logit);
  return hipGetLastError();
}

}  // namespace dspark
