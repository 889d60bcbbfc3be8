// dspark_markov_sample: the semi-autoregressive gamma-step loop.
//
// Passage: DSpark reading notes, eq (4) (p_k(v) ∝ exp(U_k(v) + B_k(v))) and
// eq (5) (B(x_{k-1}, .) = W1[x_{k-1}] W2); caijizhuo summary, section 四
// (the sequential loop carries only the sampled token).
//
// A call is gamma + 2 launches: sample_init clears the argmax keys, then one
// sample_step_* launch per position, then sample_finalize.  sample_step_*
// streams U_k and W2t once, builds the Markov bias of a 64-token chunk for
// all requests on the matrix cores, and folds the chunk into running
// per-request reductions held in registers: the log-sum-exp (for lse) and the
// two-level Gumbel argmax (chunk score LSE_c + G_c; inside the winning chunk,
// l_v + g_{v mod 64}).  At the end each work group merges its argmax into the
// request's key with one 64-bit atomic max (eight key slots per request
// spread the contention) and stores its log-sum-exp partial.  The next
// position's launch reads the keys back as its previous tokens.
// sample_finalize decodes x, merges the log-sum-exp partials and recomputes
// the logit of each drafted token.
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

// Fold one 64-token chunk of one request group into the running reductions.
// MASK: the chunk may run past V (only the last chunk of the vocabulary).
template <bool MASK, int NBW>
__device__ __forceinline__ void sample_chunk_epilogue(const f32x4 (&acc)[4][NBW], const u32x2 (&uw)[NBW][4],
                                                      const float (&Gc)[NBW], const float (&gg)[NBW][16],
                                                      int v0, int V, Lse (&run)[NBW], Best (&best)[NBW]) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    float val[16];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = acc[mb][nb][i] + row4_get(uw[nb][mb], i);
        val[mb * 4 + i] = (!MASK || v0 + mb * 16 + 4 * q + i < V) ? x : neg_inf();
      }
    float m = fmaxf(val[0], val[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) m = fmaxf(m, fmaxf(val[i], val[i + 1]));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const float mb2 = m * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += __builtin_amdgcn_exp2f(fmaf(val[i], kLog2e, -mb2));
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    // in-chunk Gumbel argmax; offsets grow with i, strict > keeps the lowest
    float bs = val[0] + gg[nb][0];
    int bo = 4 * q;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (mb == 0 && i == 0) continue;
        const float sc = val[mb * 4 + i] + gg[nb][mb * 4 + i];
        if (sc > bs) {
          bs = sc;
          bo = mb * 16 + 4 * q + i;
        }
      }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float os = __shfl_xor(bs, o);
      const int oo = __shfl_xor(bo, o);
      if (better(os, oo, bs, bo)) {
        bs = os;
        bo = oo;
      }
    }
    const float S = m + __logf(s) + Gc[nb];
    run[nb] = lse_combine(run[nb], Lse{m, s});
    if (S > best[nb].score) best[nb] = Best{S, v0 + bo, 0.f};   // earlier chunk wins ties
  }
}

// Loads of one chunk staged in registers: the W2t tile, this lane's U logits
// and chunk Gumbels.
template <int NBW, int KS>
struct SampleStage {
  WRegs<KS> w;
  u32x2 u[NBW][4];
  float G[NBW];
};

// One drafted position for every request of a group (64 or 128 rows): the
// chunks blockIdx.x, blockIdx.x + gridDim.x, ... of the vocabulary.  Loads run
// two chunks ahead in two register sets (even and odd chunks).  At the start
// of chunk i the set holding chunk i+1 is written to the other half of a
// double-buffered LDS area (W2t tile, U logits, Gumbels) and reloaded with
// chunk i+3, so the loads of chunks i+2 and i+3 are in flight while chunk i is
// reduced.  One barrier per chunk orders the LDS halves.
template <int NBW, int KS, bool VEC>
__global__ __launch_bounds__(kTileThreads, 1) void sample_step_bf16(
    int R, int gamma, int V, int k, const uint16_t* __restrict__ U, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W2t, const int32_t* __restrict__ x0, const float* __restrict__ G,
    const float* __restrict__ g, SampleWs ws, int nPart) {
  constexpr int NROWS = sample_reqs_per_wg<NBW>();
  constexpr int kW = tile_bytes(KS);
  constexpr int kU = kTileThreads * NBW * 4 * 8;       // each lane's U logits, parked per chunk
  constexpr int kG = kTileThreads * NBW * 4;            // each lane's chunk Gumbels, parked per chunk
  constexpr int kBuf = kW + kU + kG;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kBuf];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int q = lane >> 4;
  const int nC = (V + kChunk - 1) / kChunk;
  // the host launches at most one work group per chunk, so nT >= 1
  const int nT = (nC - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) / static_cast<int>(gridDim.x);

  int req[NBW];
  bool live[NBW];
  int64_t rowk[NBW];     // (request, k) row of U, G and g; clamped to a valid request
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    req[nb] = blockIdx.y * NROWS + wave * 16 * NBW + nb * 16 + j;
    live[nb] = req[nb] < R;
    rowk[nb] = static_cast<int64_t>(min(req[nb], R - 1)) * gamma + k;
  }

  auto load_stage = [&](SampleStage<NBW, KS>& st, int it) {
    const int tile = blockIdx.x + it * gridDim.x;
    const int v0 = tile * kChunk;
    load_w2_regs<KS>(st.w, W2t, V, v0);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      load_lane_logits<VEC>(st.u[nb], U + rowk[nb] * V, v0, V, q);
      st.G[nb] = G[rowk[nb] * nC + tile];
    }
  };
  auto park = [&](const SampleStage<NBW, KS>& st, int buf) {   // staged chunk -> LDS half `buf`
    store_w2_tile<KS>(lds + buf * kBuf, st.w);
    u32x2* up = reinterpret_cast<u32x2*>(lds + buf * kBuf + kW) + threadIdx.x * NBW * 4;
    float* gp = reinterpret_cast<float*>(lds + buf * kBuf + kW + kU) + threadIdx.x * NBW;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) up[nb * 4 + mb] = st.u[nb][mb];
      gp[nb] = st.G[nb];
    }
  };

  // Chunk indices past the last are clamped to it: the prefetch and park
  // below are unconditional (a conditional load would force the compiler to
  // drain every outstanding load before each park), and the few redundant
  // reloads of the last chunk are never reduced.
  const auto clampc = [&](int it) { return it < nT ? it : nT - 1; };

  // chunks 0 and 1 go out before the previous-token lookup they do not depend on
  SampleStage<NBW, KS> even, odd;
  load_stage(even, 0);
  load_stage(odd, clampc(1));
  int prev[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) prev[nb] = live[nb] ? previous_token(ws.keys, x0, R, V, k, req[nb]) : -1;
  WFrags<NBW, KS> e;
  load_w1_frags<NBW, KS>(e, W1, prev);
  // in-chunk Gumbels for this lane's sixteen offsets 16 mb + 4q + i
  float gg[NBW][16];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) gg[nb][mb * 4 + i] = g[rowk[nb] * kChunk + mb * 16 + 4 * q + i];

  Lse run[NBW];
  Best best[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    run[nb] = Lse{neg_inf(), 0.f};
    best[nb] = Best{neg_inf(), -1, 0.f};
  }
  park(even, 0);
  // every prologue load has landed before the loop, so the loop's waits only
  // ever concern the chunk being parked
  __builtin_amdgcn_s_waitcnt(0);
  load_stage(even, clampc(2));
  __syncthreads();

  // chunk `it`: park chunk it+1 from `nxt`, refill `nxt` with chunk it+3, reduce chunk it
  auto chunk = [&](int it, SampleStage<NBW, KS>& nxt) {
    const int v0 = (blockIdx.x + it * gridDim.x) * kChunk;
    const int buf = it & 1;
    park(nxt, buf ^ 1);
    load_stage(nxt, clampc(it + 3));
    u32x2 uw[NBW][4];
    float gc[NBW];
    const u32x2* up = reinterpret_cast<const u32x2*>(lds + buf * kBuf + kW) + threadIdx.x * NBW * 4;
    const float* gp = reinterpret_cast<const float*>(lds + buf * kBuf + kW + kU) + threadIdx.x * NBW;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) uw[nb][mb] = up[nb * 4 + mb];
      gc[nb] = gp[nb];
    }
    f32x4 acc[4][NBW];
    bias_tile<NBW, KS>(acc, lds + buf * kBuf, e);
    if (v0 + kChunk <= V)
      sample_chunk_epilogue<false, NBW>(acc, uw, gc, gg, v0, V, run, best);
    else
      sample_chunk_epilogue<true, NBW>(acc, uw, gc, gg, v0, V, run, best);
    __syncthreads();
  };
  // pairs of chunks, so every path back to the loop head has issued both
  // sets' loads in the same order; an odd last chunk follows the loop
  int it = 0;
  for (; it + 1 < nT; it += 2) {
    chunk(it, odd);                  // chunk it+1 (odd) is parked from `odd`
    chunk(it + 1, even);
  }
  if (it < nT) chunk(it, odd);

  if (q == 0) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if (!live[nb]) continue;
      ws.lsep[(static_cast<int64_t>(k) * R + req[nb]) * nPart + blockIdx.x] = make_float2(run[nb].M, run[nb].S);
      if (best[nb].tok >= 0)
        atomicMax(ws.keys + (static_cast<int64_t>(k) * kKeySlots + blockIdx.x % kKeySlots) * R + req[nb],
                  pack_key(best[nb].score, best[nb].tok));
    }
  }
}

// fp32 storage, any rank: one wave per (chunk, request), plain FMA bias.
__global__ __launch_bounds__(64) void sample_step_f32(
    int R, int gamma, int V, int r, int k, const float* __restrict__ U, const float* __restrict__ W1,
    const float* __restrict__ W2t, const int32_t* __restrict__ x0, const float* __restrict__ G,
    const float* __restrict__ g, SampleWs ws, int nPart) {
  const int tile = blockIdx.x;
  const int req = blockIdx.y;
  const int lane = threadIdx.x;
  const int nC = (V + kChunk - 1) / kChunk;
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
  const float m = wave_reduce_max(val);
  const float s = wave_reduce_sum(v < V ? __expf(val - m) : 0.f);
  Best bb{v < V ? val + g[rowk * kChunk + lane] : neg_inf(), v, 0.f};
  bb = wave_reduce_best(bb);
  if (lane == 0) {
    ws.lsep[(static_cast<int64_t>(k) * R + req) * nPart + tile] = make_float2(m, s);
    atomicMax(ws.keys + (static_cast<int64_t>(k) * kKeySlots + tile % kKeySlots) * R + req,
              pack_key(m + __logf(s) + G[rowk * nC + tile], bb.tok));
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
  const bool vec = (V % 4) == 0;
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
