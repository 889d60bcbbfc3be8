// The RNN head's recurrent step (DSpark reading notes, "implementation two:
// the RNN head", eq (6)): for every request,
//   z = [s_{k-1}; W1[x_{k-1}]; h_k],  y = W z  (W = [W_g; W_c; W_o]),
//   s_k = sigma(y_g) * s_{k-1} + (1 - sigma(y_g)) * tanh(y_c),  o_k = tanh(y_o),
// with s_{-1} = 0.  o_k is the r-vector the sampler's bias product takes in
// W1[x_{k-1}]'s place.  The previous token comes from the sampler's argmax
// keys of position k - 1 (the anchor at k = 0).
//
// bf16 storage: z enters the products in bf16 (its state part rounded from
// fp32 to nearest, ties to even), with fp32 accumulation on the matrix
// cores (32x32x16 MFMA).  The hidden-state part of y does not depend on the
// loop: W_h h_k for every (request, position) is one matrix product, run
// once before the first position (rnn_hproj_bf16, split along d into a few
// partials that rnn_hsum then adds in split order).  Each position then
// multiplies only the state and W1-row parts (2r of the 2r + d inner
// elements), adds the hidden-state part and applies the gates in fp32, in
// one kernel (rnn_step_bf16).
// fp32 storage: one thread per output with fp32 FMAs, then the gates.
#include "bias_tile.hpp"
#include "wide_tile.hpp"
#include "rnn_head.hpp"
#include "sample_common.hpp"

namespace dspark {

typedef float f32x16_r __attribute__((ext_vector_type(16)));


// ---- the hidden-state part, every position at once -------------------------
//
// Yh[sp][m][n] = sum over split sp's inner range of h[m][c] * W[n][2r + c]
// (m = request * gamma + position, n < 3r).  A work group computes a
// kHpBM x kHpBN block of one split: four waves, each 64 rows of h by the
// block's 96 projection rows (2 x 3 MFMA tiles).  The inner range runs in
// stages of kHpBK elements, double-buffered in LDS; a stage's loads are
// issued into registers two stages before its products and written to the
// free LDS buffer one stage before them.  In LDS a stage is 128 bytes
// per row, in 1 KB blocks of 8 rows; the 16-byte piece c of row j sits at
// slot c ^ (j mod 8), so each load instruction reads whole 128-byte lines,
// each LDS write is 1 KB contiguous, and the fragment reads (row j, piece
// 2t + half) hit eight different slots per eight lanes.
constexpr int kHpBM = 256;
constexpr int kHpBN = 96;
constexpr int kHpBK = 64;
constexpr int kHpThreads = 256;
constexpr int kHpBlocks = (kHpBM + kHpBN) / 8;          // 1 KB copy blocks per stage
constexpr int kHpCopies = kHpBlocks / (kHpThreads / kWave);   // per wave
static_assert(kHpBlocks % (kHpThreads / kWave) == 0, "copy blocks must divide over the waves");

// Splits of d: enough work groups to cover the compute units, at most
// kHpMaxSplits.
constexpr int kHpMaxSplits = 4;
int hproj_max_splits(int64_t M, int r) {
  const int64_t nN = 3 * r / kHpBN;   // 0 for the fp32 ranks that are not multiples of 32
  const int64_t tiles = ((M + kHpBM - 1) / kHpBM) * (nN > 0 ? nN : 1);
  const int64_t want = (256 + tiles - 1) / tiles;
  return static_cast<int>(want < 1 ? 1 : want > kHpMaxSplits ? kHpMaxSplits : want);
}

struct HprojPlan {
  int splits;   // partials actually written
  int per;      // stages per split
};

HprojPlan hproj_plan(int64_t M, int r, int d) {
  const int stages = ceil_div(d, kHpBK);
  int sp = hproj_max_splits(M, r);
  sp = sp < stages ? sp : stages;
  const int per = ceil_div(stages, sp);
  return HprojPlan{ceil_div(stages, per), per};
}

__device__ __forceinline__ bf16x8 hproj_frag(const uint8_t* buf, int row, int piece) {
  return *reinterpret_cast<const bf16x8*>(buf + row * 128 + ((piece ^ (row & 7)) << 4));
}

// k-step t of a stage: the wave's 64 rows of h (A) by the 96 projection rows (B)
__device__ __forceinline__ void hproj_kstep(const uint8_t* buf, f32x16_r (&acc)[2][3], int wave, int j, int hh, int t,
                                            bool ok) {
  bf16x8 a[2], bb[3];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const bf16x8 f = hproj_frag(buf, wave * 64 + mi * 32 + j, 2 * t + hh);
    a[mi] = ok ? f : bf16x8{};
  }
#pragma unroll
  for (int ni = 0; ni < 3; ++ni) {
    const bf16x8 f = hproj_frag(buf, kHpBM + ni * 32 + j, 2 * t + hh);
    bb[ni] = ok ? f : bf16x8{};
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 3; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], bb[ni], acc[mi][ni], 0, 0, 0);
}

// A work-group barrier that waits for LDS traffic only (the copies into LDS
// are waited for explicitly before it), so loads in flight stay in flight.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __launch_bounds__(kHpThreads) void rnn_hproj_bf16(int M, int N, int d, int K, int nM, int nN, int per,
                                                             const uint16_t* __restrict__ h,
                                                             const uint16_t* __restrict__ Wh,
                                                             float* __restrict__ Yh) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[(kHpBM + kHpBN) * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[(kHpBM + kHpBN) * 128];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  // work groups that share an h block (same rows and split) are numbered so
  // that they are dispatched to the same XCD (work group b goes to XCD b mod 8)
  const int T = gridDim.x;
  const int b = blockIdx.x;
  const int g = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  const int nt = g % nN;
  const int ms = g / nN;
  const int mt = ms % nM;
  const int sp = ms / nM;
  const int m0 = mt * kHpBM, n0 = nt * kHpBN;
  const int kb = sp * per * kHpBK;
  const int ke = min(d, kb + per * kHpBK);
  const int nst = ceil_div(ke - kb, kHpBK);
  // the lane's load sources: block bi = wave + 4 c (rows of h first, then of W)
  const int rib = lane >> 3;
  const int piece = (lane & 7) ^ rib;
  const uint16_t* src[kHpCopies];
#pragma unroll
  for (int c = 0; c < kHpCopies; ++c) {
    const int bi = wave + 4 * c;
    if (bi < kHpBM / 8) {
      const int m = min(m0 + 8 * bi + rib, M - 1);
      src[c] = h + static_cast<int64_t>(m) * d + kb;
    } else {
      src[c] = Wh + static_cast<int64_t>(n0 + 8 * (bi - kHpBM / 8) + rib) * K + kb;
    }
  }
  const int j = lane & 31, hh = lane >> 5;
  f32x16_r acc[2][3] = {};
  auto koff = [&](int st) {
    const int o = st * kHpBK + piece * 8;
    return kb + o < ke ? o : st * kHpBK;   // a piece past the range loads a valid one; its k-step is zeroed
  };
  // a stage's k-steps; only the last stage of a split can hold k-steps past
  // its range (d a multiple of 16, not of 64), and those multiply zeros
  // (selected without a branch)
  auto compute = [&](const uint8_t* buf, int st) {
    const int valid = (ke - kb - st * kHpBK) >> 4;
#pragma unroll
    for (int t = 0; t < kHpBK / 16; ++t) hproj_kstep(buf, acc, wave, j, hh, t, t < valid);
  };
  // two register sets: each stage's loads are issued two stages before its
  // products, written to LDS one stage before them
  u32x4 stgA[kHpCopies], stgB[kHpCopies];
  auto load_stage = [&](u32x4 (&stg)[kHpCopies], int st) {
    const int o = koff(st);
#pragma unroll
    for (int c = 0; c < kHpCopies; ++c) stg[c] = *reinterpret_cast<const u32x4*>(src[c] + o);
  };
  auto store_stage = [&](const u32x4 (&stg)[kHpCopies], uint8_t* buf) {
#pragma unroll
    for (int c = 0; c < kHpCopies; ++c) *reinterpret_cast<u32x4*>(buf + (wave + 4 * c) * 1024 + lane * 16) = stg[c];
  };
  // The loop body is one basic block: the stage count is rounded up to even
  // (a stage past the range multiplies zeros) and the loads are
  // unconditional (past the last stage they repeat it), so the compiler
  // neither sinks a load to its use nor waits for the younger register set
  // before an LDS write.
  load_stage(stgA, 0);
  load_stage(stgB, min(1, nst - 1));
  store_stage(stgA, buf0);
  lds_sync();
  for (int st = 0; st < nst; st += 2) {
    // buf0 holds stage st, stgB stage st + 1 (in flight); stage st + 2 goes to stgA
    load_stage(stgA, min(st + 2, nst - 1));
    compute(buf0, st);
    store_stage(stgB, buf1);
    lds_sync();
    load_stage(stgB, min(st + 3, nst - 1));
    compute(buf1, st + 1);
    store_stage(stgA, buf0);
    lds_sync();
  }
  float* out = Yh + static_cast<int64_t>(sp) * M * N;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = m0 + wave * 64 + mi * 32 + 8 * (q >> 2) + 4 * hh + (q & 3);
      if (m < M)
#pragma unroll
        for (int ni = 0; ni < 3; ++ni) out[static_cast<int64_t>(m) * N + n0 + ni * 32 + j] = acc[mi][ni][q];
    }
}

// ---- one position: the state and W1-row parts, the sum, the gates ----------
//
// Work group (jb, ib): state columns 32 jb .. 32 jb + 31 (rows of each of
// the three parts of W) for requests 32 ib .. 32 ib + 31.  Wave w takes the
// k-steps w, w + 4, ... of the 2r/16 over [s_{k-1}; W1[x_{k-1}]]; lane (hh,
// j) brings weight row 32 jb + j of each part (the A operands) and z of
// request 32 ib + j (the B operand).  Everything that does not wait on the
// previous token -- the weight fragments, the state fragments, the
// hidden-state partials and s_{k-1} for the gates -- is loaded before the
// keys are read.  The waves' sums meet in LDS; thread e then finishes
// (request 32 ib + e / 32, column 32 jb + e % 32), four per thread.
template <int NS>   // k-steps per wave: r / 32
__global__ __launch_bounds__(256) void rnn_step_bf16(int R, int gamma, int V, int d, int k,
                                                      const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ W1,
                                                      const int32_t* __restrict__ x0,
                                                      const unsigned long long* __restrict__ keys,
                                                      const float* __restrict__ Yh, float* __restrict__ s,
                                                      uint16_t* __restrict__ o) {
  constexpr int r = NS * 32;
  constexpr int kHalf = r / 16;   // k-steps of the state part
  __shared__ float red[3][4][16][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int j = lane & 31;
  const int hh = lane >> 5;
  const int jb = blockIdx.x, ib = blockIdx.y;
  const int K = 2 * r + d;
  const int ic = min(ib * 32 + j, R - 1);
  // the gates' inputs that need no token, loaded first
  float yh[4][3], sprev[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = threadIdx.x + 256 * u;
    const int rq = min(ib * 32 + (e >> 5), R - 1);
    const int64_t row = static_cast<int64_t>(rq) * gamma + k;
    const int col = jb * 32 + (e & 31);
#pragma unroll
    for (int g = 0; g < 3; ++g) yh[u][g] = Yh[row * (3 * r) + g * r + col];
    sprev[u] = s[(k > 0 ? row - 1 : row) * r + col];   // read at k = 0 too (any value; unused)
  }
  bf16x8 a[NS][3], bz[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int kk = (wave + 4 * u) * 16 + 8 * hh;
#pragma unroll
    for (int g = 0; g < 3; ++g)
      a[u][g] = load_bf16x8_global(W + static_cast<int64_t>(g * r + jb * 32 + j) * K + kk);
  }
  // the state part, loaded for every k-step without a branch (a k-step of
  // the W1-row part reads the state row's start and is replaced below)
  const float* srow = s + (static_cast<int64_t>(ic) * gamma + (k > 0 ? k - 1 : 0)) * r;
  float4 sv[NS][2];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int st = wave + 4 * u;
    const int kk = st < kHalf ? st * 16 + 8 * hh : 0;
    sv[u][0] = *reinterpret_cast<const float4*>(srow + kk);
    sv[u][1] = *reinterpret_cast<const float4*>(srow + kk + 4);
  }
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const float4 lo = sv[u][0], hi = sv[u][1];
    const uint32_t w0 = bf16_bits_rne(lo.x) | (bf16_bits_rne(lo.y) << 16);
    const uint32_t w1 = bf16_bits_rne(lo.z) | (bf16_bits_rne(lo.w) << 16);
    const uint32_t w2 = bf16_bits_rne(hi.x) | (bf16_bits_rne(hi.y) << 16);
    const uint32_t w3 = bf16_bits_rne(hi.z) | (bf16_bits_rne(hi.w) << 16);
    const bf16x8 v = __builtin_bit_cast(bf16x8, (uint4{w0, w1, w2, w3}));
    bz[u] = k > 0 ? v : bf16x8{};   // z's state part is zero at the first position
  }
  const int prev = previous_token(keys, kKeySlots, x0, R, V, k, ic);
  const uint16_t* erow = prev >= 0 ? W1 + static_cast<int64_t>(prev) * r : kZeroRow;
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int st = wave + 4 * u;
    const bf16x8 v = load_bf16x8_global(erow + (st >= kHalf ? st * 16 + 8 * hh - r : 0));
    if (st >= kHalf) bz[u] = v;
  }
  __builtin_amdgcn_sched_barrier(0);   // every W1-row load issued before the first product
  f32x16_r acc[3] = {};
#pragma unroll
  for (int u = 0; u < NS; ++u)
#pragma unroll
    for (int g = 0; g < 3; ++g) acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u][g], bz[u], acc[g], 0, 0, 0);
#pragma unroll
  for (int g = 0; g < 3; ++g)
#pragma unroll
    for (int q = 0; q < 16; ++q) red[g][wave][q][lane] = acc[g][q];
  __syncthreads();
  // accumulator q of lane l holds weight row 8 (q / 4) + 4 (l / 32) + q % 4
  // of the block and request l % 32
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = threadIdx.x + 256 * u;
    const int rl = e >> 5, c = e & 31;
    const int q = ((c >> 3) << 2) | (c & 3);
    const int l = (((c >> 2) & 1) << 5) | rl;
    float y[3];
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      float t = yh[u][g];
#pragma unroll
      for (int w = 0; w < 4; ++w) t += red[g][w][q][l];
      y[g] = t;
    }
    const int req = ib * 32 + rl;
    if (req < R) {
      const int64_t idx = (static_cast<int64_t>(req) * gamma + k) * r + jb * 32 + c;
      const float gate = 1.f / (1.f + expf(-y[0]));
      s[idx] = gate * (k > 0 ? sprev[u] : 0.f) + (1.f - gate) * tanhf(y[1]);
      o[idx] = static_cast<uint16_t>(bf16_bits_rne(tanhf(y[2])));
    }
  }
}

// fp32 storage: one thread per (request, output row), the whole inner range.
__global__ __launch_bounds__(256) void rnn_proj_f32(int R, int gamma, int V, int r, int d, int k,
                                                    const float* __restrict__ W, const float* __restrict__ h,
                                                    const float* __restrict__ W1, const int32_t* __restrict__ x0,
                                                    const unsigned long long* __restrict__ keys,
                                                    const float* __restrict__ s, float* __restrict__ part) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(R) * 3 * r) return;
  const int i = static_cast<int>(idx / (3 * r));
  const int n = static_cast<int>(idx % (3 * r));
  const int K = 2 * r + d;
  const int prev = previous_token(keys, kKeySlots, x0, R, V, k, i);
  const float* w = W + static_cast<int64_t>(n) * K;
  float y = 0.f;
  if (k > 0) {
    const float* srow = s + (static_cast<int64_t>(i) * gamma + k - 1) * r;
    for (int q = 0; q < r; ++q) y = fmaf(srow[q], w[q], y);
  }
  if (prev >= 0) {
    const float* erow = W1 + static_cast<int64_t>(prev) * r;
    for (int q = 0; q < r; ++q) y = fmaf(erow[q], w[r + q], y);
  }
  const float* hrow = h + (static_cast<int64_t>(i) * gamma + k) * d;
  for (int q = 0; q < d; ++q) y = fmaf(hrow[q], w[2 * r + q], y);
  part[static_cast<int64_t>(i) * 3 * r + n] = y;
}

// The gates: one thread per (request, state element); the partials are
// added in split order.
template <typename Elt>
__global__ __launch_bounds__(256) void rnn_gate(int R, int gamma, int r, int k, int nsplit,
                                                const float* __restrict__ part, float* __restrict__ s,
                                                typename Elt::T* __restrict__ o) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(R) * r) return;
  const int i = static_cast<int>(idx / r);
  const int jj = static_cast<int>(idx % r);
  float yg = 0.f, yc = 0.f, yo = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* p = part + (static_cast<int64_t>(sp) * R + i) * 3 * r;
    yg += p[jj];
    yc += p[r + jj];
    yo += p[2 * r + jj];
  }
  const int64_t row = static_cast<int64_t>(i) * gamma + k;
  const float sprev = k > 0 ? s[(row - 1) * r + jj] : 0.f;
  const float gate = 1.f / (1.f + expf(-yg));
  s[row * r + jj] = gate * sprev + (1.f - gate) * tanhf(yc);
  const float ov = tanhf(yo);
  if constexpr (sizeof(typename Elt::T) == 2)
    o[row * r + jj] = static_cast<uint16_t>(bf16_bits_rne(ov));
  else
    o[row * r + jj] = ov;
}

// The partials summed in split order into the first: float4 per thread.
__global__ __launch_bounds__(256) void rnn_hsum(int64_t n4, int S, float4* __restrict__ Yh) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 t = Yh[i];
  for (int sp = 1; sp < S; ++sp) {
    const float4 v = Yh[sp * n4 + i];
    t.x += v.x;
    t.y += v.y;
    t.z += v.z;
    t.w += v.w;
  }
  Yh[i] = t;
}

// bf16: the hidden-state part of the projection for every position
// (rnn_hproj_bf16) into hd.part, its split partials then summed in order
// into the first (rnn_hsum), so the per-position kernels read one value.
hipError_t rnn_hproj_launch(const RnnHead& hd, int R, int gamma, int r, hipStream_t s) {
  const int K = 2 * r + hd.d;
  const int64_t M = static_cast<int64_t>(R) * gamma;
  const HprojPlan pl = hproj_plan(M, r, hd.d);
  const int nM = ceil_div(M, kHpBM), nN = 3 * r / kHpBN;
  hipLaunchKernelGGL(rnn_hproj_bf16, dim3(nM * nN * pl.splits), dim3(kHpThreads), 0, s, static_cast<int>(M), 3 * r,
                     hd.d, K, nM, nN, pl.per, static_cast<const uint16_t*>(hd.h),
                     static_cast<const uint16_t*>(hd.W) + 2 * r, hd.part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || pl.splits == 1) return err;
  const int64_t n4 = M * 3 * r / 4;   // 3r is a multiple of 4
  hipLaunchKernelGGL(rnn_hsum, dim3(ceil_div(n4, 256)), dim3(256), 0, s, n4, pl.splits,
                     reinterpret_cast<float4*>(hd.part));
  return hipGetLastError();
}

// P[v] = W's W1-row columns applied to W1 row v, for every token: the
// projection kernel with W1 in h's place (V rows, inner length r) and the
// W1-row block of W (columns r .. 2r - 1) as the weights, in one split.
hipError_t rnn_prepare_launch(int V, int r, int d, const uint16_t* W1, const uint16_t* Wrnn, float* P,
                              hipStream_t s) {
  const int K = 2 * r + d;
  const int nM = ceil_div(V, kHpBM), nN = 3 * r / kHpBN;
  const int per = ceil_div(r, kHpBK);
  hipLaunchKernelGGL(rnn_hproj_bf16, dim3(nM * nN), dim3(kHpThreads), 0, s, V, 3 * r, r, K, nM, nN, per, W1,
                     Wrnn + r, P);
  return hipGetLastError();
}

hipError_t rnn_step_launch(dspark_dtype dt, const RnnHead& hd, int R, int gamma, int V, int r, int k,
                           const void* W1, const int32_t* x0, const unsigned long long* keys, hipStream_t s) {
  if (dt == DSPARK_BF16) {
    if (k == 0) {
      hipError_t err = rnn_hproj_launch(hd, R, gamma, r, s);
      if (err != hipSuccess) return err;
    }
    const dim3 grid(r / 32, ceil_div(R, 32));
    const uint16_t* Wb = static_cast<const uint16_t*>(hd.W);
    const uint16_t* W1b = static_cast<const uint16_t*>(W1);
    uint16_t* ob = static_cast<uint16_t*>(hd.o);
    switch (r) {
      case 32:
        hipLaunchKernelGGL(rnn_step_bf16<1>, grid, dim3(256), 0, s, R, gamma, V, hd.d, k, Wb, W1b, x0,
                           keys, hd.part, hd.s, ob);
        break;
      case 64:
        hipLaunchKernelGGL(rnn_step_bf16<2>, grid, dim3(256), 0, s, R, gamma, V, hd.d, k, Wb, W1b, x0,
                           keys, hd.part, hd.s, ob);
        break;
      case 128:
        hipLaunchKernelGGL(rnn_step_bf16<4>, grid, dim3(256), 0, s, R, gamma, V, hd.d, k, Wb, W1b, x0,
                           keys, hd.part, hd.s, ob);
        break;
      default:
        hipLaunchKernelGGL(rnn_step_bf16<8>, grid, dim3(256), 0, s, R, gamma, V, hd.d, k, Wb, W1b, x0,
                           keys, hd.part, hd.s, ob);
        break;
    }
  } else {
    const int nthreads = ceil_div(static_cast<int64_t>(R) * r, 256);
    hipLaunchKernelGGL(rnn_proj_f32, dim3(ceil_div(static_cast<int64_t>(R) * 3 * r, 256)), dim3(256), 0, s, R,
                       gamma, V, r, hd.d, k, static_cast<const float*>(hd.W), static_cast<const float*>(hd.h),
                       static_cast<const float*>(W1), x0, keys, hd.s, hd.part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(rnn_gate<F32>, dim3(nthreads), dim3(256), 0, s, R, gamma, r, k, 1, hd.part, hd.s,
                       static_cast<float*>(hd.o));
  }
  return hipGetLastError();
}

// bf16: the hidden-state partials [splits][R gamma][3r]; fp32: the
// projection of one position [R][3r].
size_t rnn_workspace_bytes(int R, int gamma, int r) {
  const int64_t M = static_cast<int64_t>(R) * gamma;
  const size_t a = sizeof(float) * static_cast<size_t>(hproj_max_splits(M, r)) * M * 3 * r;
  const size_t b = sizeof(float) * static_cast<size_t>(R) * 3 * r;
  return ((a > b ? a : b) + 255) & ~static_cast<size_t>(255);
}

}  // namespace dspark
