// dspark_verify: lossless rejection-sampling verification.
//
// Passage: DSpark reading notes, the speculative-decoding background (accept
// with probability min(1, p_t/p_d); at the first rejection resample from
// norm(max(0, p_t - p_d)); a bonus token from p_t when all drafts pass),
// eq (8a)-(8c) and steps 12-13 of the end-to-end loop; caijizhuo summary,
// section 四 steps 5-6 (row i of the target logits predicts draft i).
//
// Four launches:
//   verify_target_part  the needed target rows (rows 0..l_r of request r),
//                       each split into parts along the vocabulary: (max,
//                       sum) parts of the log-normaliser;
//   verify_accept       one wave per request: the parts merged into each
//                       row's log-normaliser, the target logit of each
//                       drafted token gathered, then the first i with
//                       ln u_acc >= ln p_t(x_i) - ln p_d(x_i) -> n_acc;
//   verify_residual_*   the residual row of every request in one pass over
//                       the vocabulary: p_d is rebuilt from U and the Markov
//                       bias of the previous token (same matrix-core tile as
//                       the sampler), and every 16-token chunk's mass of
//                       max(0, p_t - p_d) (or of p_t for the bonus row) and
//                       of p_t is written out;
//   verify_select       one work group per request: a prefix scan over the
//                       chunk masses picks the chunk holding u_res * Z, and
//                       the chunk's 16 masses are re-derived and scanned to
//                       the token.
#include "wide_tile.hpp"

namespace dspark {


// ---------------------------------------------------------- target normalisers

template <typename Elt>
struct RowVec;
template <>
struct RowVec<BF16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(uint4 v, float (&o)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void load(const uint16_t* p, float (&o)[8]) {
    unpack(*reinterpret_cast<const uint4*>(p), o);
  }
};
template <>
struct RowVec<F32> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(uint4 v, float (&o)[4]) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y); o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ void load(const float* p, float (&o)[4]) {
    unpack(*reinterpret_cast<const uint4*>(p), o);
  }
};

__device__ __forceinline__ Lse block_reduce_lse(Lse a, Lse* sh) {
  a = wave_reduce_lse(a);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = a;
  __syncthreads();
  Lse r = sh[0];
  for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) r = lse_combine(r, sh[w]);
  return r;
}

// Target rows are split along the vocabulary into kLseSplits parts.  Only
// rows 0..l_r of request r are needed, so every work group first builds the
// prefix of the needed-row counts (for up to kLseCompactR requests) and
// deals the needed (row, part) items out evenly: item a goes to work group
// a mod gridDim.  Larger batches walk every (row, part) item and skip the
// unneeded ones.  Each thread keeps kLseUnroll 16-byte loads in flight, and
// every item costs the same (the drafted tokens' target logits are gathered
// by verify_accept, so no item waits on a dependent load).
constexpr int kLseSplits = 8;
constexpr int kLseThreads = 256;
constexpr int kLseUnroll = 8;
constexpr int kLseCompactR = 4096;

// What a target-row part records (rows 0..l_r are the needed ones):
//   kPartLse     (max, sum exp)
//   kPartArgmax  (largest logit, its lowest index) (greedy)
enum PartMode { kPartLse = 0, kPartArgmax = 1 };

__device__ __forceinline__ int needed_rows(const int32_t* ell, int r, int gamma) {
  return min(max(ell[r], 0), gamma) + 1;
}

// The larger logit, the lower index on equal logits.
struct ArgMax {
  float m;
  int i;
};
__device__ __forceinline__ ArgMax argmax_combine(ArgMax a, ArgMax b) {
  return (b.m > a.m || (b.m == a.m && b.i < a.i)) ? b : a;
}
__device__ __forceinline__ ArgMax block_reduce_argmax(ArgMax a, ArgMax* sh) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) a = argmax_combine(a, ArgMax{__shfl_xor(a.m, o), __shfl_xor(a.i, o)});
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = a;
  __syncthreads();
  ArgMax r = sh[0];
  for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) r = argmax_combine(r, sh[w]);
  return r;
}

template <typename Elt, int MODE>
__device__ __forceinline__ void target_part_item(int r, int i, int sp, int gamma, int V, int span,
                                                 const typename Elt::T* __restrict__ target,
                                                 const int32_t* __restrict__ row0, float2* __restrict__ part,
                                                 Lse* sh) {
  constexpr int N = RowVec<Elt>::N;
  const int64_t ri = static_cast<int64_t>(r) * (gamma + 1) + i;
  const int64_t row = row0 ? static_cast<int64_t>(row0[r]) + i : ri;
  const typename Elt::T* t = target + row * V;
  const int v0 = sp * span;
  const int v1 = min(v0 + span, V);
  if constexpr (MODE == kPartArgmax) {
    // each thread visits its tokens in ascending order, so a strict > keeps
    // the lowest index of its largest logit
    ArgMax am{neg_inf(), 0x7FFFFFFF};
    if ((V % N) == 0) {
      for (int vb = v0 + static_cast<int>(threadIdx.x) * N; vb < v1; vb += kLseUnroll * N * kLseThreads) {
        float e[kLseUnroll][N];
#pragma unroll
        for (int u = 0; u < kLseUnroll; ++u) {
          const int v = vb + u * N * kLseThreads;
          RowVec<Elt>::load(t + (v < v1 ? v : v0), e[u]);
        }
#pragma unroll
        for (int u = 0; u < kLseUnroll; ++u) {
          const int v = vb + u * N * kLseThreads;
          if (v >= v1) break;
#pragma unroll
          for (int q = 0; q < N; ++q)
            if (e[u][q] > am.m || am.i == 0x7FFFFFFF) am = ArgMax{e[u][q], v + q};
        }
      }
    } else {
      for (int v = v0 + static_cast<int>(threadIdx.x); v < v1; v += kLseThreads) {
        const float e = Elt::load(t, v);
        if (e > am.m || am.i == 0x7FFFFFFF) am = ArgMax{e, v};
      }
    }
    am = block_reduce_argmax(am, reinterpret_cast<ArgMax*>(sh));
    if (threadIdx.x == 0) part[ri * kLseSplits + sp] = make_float2(am.m, __int_as_float(am.i));
    __syncthreads();   // sh is reused by the next item
    return;
  }
  Lse acc{neg_inf(), 0.f};
  if ((V % N) == 0) {
    for (int vb = v0 + static_cast<int>(threadIdx.x) * N; vb < v1; vb += kLseUnroll * N * kLseThreads) {
      float e[kLseUnroll][N];
#pragma unroll
      for (int u = 0; u < kLseUnroll; ++u) {
        const int v = vb + u * N * kLseThreads;
        RowVec<Elt>::load(t + (v < v1 ? v : v0), e[u]);
      }
#pragma unroll
      for (int u = 0; u < kLseUnroll; ++u) {
        if (vb + u * N * kLseThreads >= v1) break;
        float m = e[u][0];
#pragma unroll
        for (int q = 1; q < N; ++q) m = fmaxf(m, e[u][q]);
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < N; ++q) sum += __expf(e[u][q] - m);
        acc = lse_combine(acc, Lse{m, sum});
      }
    }
  } else {
    for (int v = v0 + static_cast<int>(threadIdx.x); v < v1; v += kLseThreads)
      acc = lse_combine(acc, Lse{Elt::load(t, v), 1.f});
  }
  acc = block_reduce_lse(acc, sh);
  if (threadIdx.x == 0) part[ri * kLseSplits + sp] = make_float2(acc.M, acc.S);
  __syncthreads();   // sh is reused by the next item
}

template <typename Elt, int MODE>
__global__ __launch_bounds__(kLseThreads) void verify_target_part(int R, int gamma, int V,
                                                                  const typename Elt::T* __restrict__ target,
                                                                  const int32_t* __restrict__ row0,
                                                                  const int32_t* __restrict__ ell,
                                                                  float2* __restrict__ part) {
  __shared__ Lse sh[kLseThreads / kWave];
  __shared__ int pref[kLseCompactR + 1];   // pref[r] = needed rows of requests < r
  constexpr int N = RowVec<Elt>::N;
  const int span = ceil_div(ceil_div(V, kLseSplits), N * kLseThreads) * N * kLseThreads;
  if (R <= kLseCompactR) {
    // counts of needed rows, then an exclusive prefix: each thread sums a
    // run of requests, the runs are scanned in one wave, then filled in
    const int per = ceil_div(R, kLseThreads);
    const int b0 = min(static_cast<int>(threadIdx.x) * per, R), b1 = min(b0 + per, R);
    int mine = 0;
    for (int q = b0; q < b1; ++q) mine += needed_rows(ell, q, gamma);
    __shared__ int wtot[kLseThreads / kWave];
    int incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if ((threadIdx.x & (kWave - 1)) >= o) incl += v;
    }
    if ((threadIdx.x & (kWave - 1)) == kWave - 1) wtot[threadIdx.x / kWave] = incl;
    __syncthreads();
    int run = incl - mine, total = 0;
#pragma unroll
    for (int wv = 0; wv < kLseThreads / kWave; ++wv) {
      run += wv < static_cast<int>(threadIdx.x / kWave) ? wtot[wv] : 0;
      total += wtot[wv];
    }
    if (threadIdx.x == 0) pref[R] = total;
    for (int q = b0; q < b1; ++q) {
      pref[q] = run;
      run += needed_rows(ell, q, gamma);
    }
    __syncthreads();
    const int64_t items = static_cast<int64_t>(pref[R]) * kLseSplits;
    for (int64_t a = blockIdx.x; a < items; a += gridDim.x) {
      const int sp = static_cast<int>(a % kLseSplits);
      const int act = static_cast<int>(a / kLseSplits);
      int lo = 0, hi = R - 1;   // the request r with pref[r] <= act < pref[r + 1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pref[mid] <= act)
          lo = mid;
        else
          hi = mid - 1;
      }
      target_part_item<Elt, MODE>(lo, act - pref[lo], sp, gamma, V, span, target, row0, part, sh);
    }
  } else {
    const int64_t items = static_cast<int64_t>(R) * (gamma + 1) * kLseSplits;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
      const int sp = static_cast<int>(it % kLseSplits);
      const int64_t ri = it / kLseSplits;
      const int r = static_cast<int>(ri / (gamma + 1));
      const int i = static_cast<int>(ri % (gamma + 1));
      const int L = needed_rows(ell, r, gamma) - 1;
      if (i > L) continue;   // uniform across the work group
      target_part_item<Elt, MODE>(r, i, sp, gamma, V, span, target, row0, part, sh);
    }
  }
}

// The target log-normalisers of the analytic acceptance: rows 0..gamma-1 of
// every request, each row whole in one work group (grid-stride over the
// rows).  Each thread folds its 16-byte vectors into a running (max, sum)
// in base 2: one exp2 per logit plus one per batch of kAccBatch vectors
// when the batch raises the thread's max (the log2-scaled max's rounding is
// taken out at the end); the next batch's loads are in
// flight while the current one is folded.  The row's (max, sum) goes to part
// 0 of the row and the other kLseSplits - 1 parts are left empty, so the
// readers merge the parts as for the split rows.
constexpr int kAccBatch = 8;

template <typename Elt>
__global__ __launch_bounds__(kLseThreads) void acceptance_target_lse(int R, int gamma, int V,
                                                                     const typename Elt::T* __restrict__ target,
                                                                     const int32_t* __restrict__ row0,
                                                                     float2* __restrict__ part) {
  constexpr float kL2e = 1.4426950408889634f;
  constexpr int N = RowVec<Elt>::N;
  constexpr int kStep = N * kLseThreads;            // elements per vector pass of the work group
  __shared__ Lse sh[kLseThreads / kWave];
  const int rows = R * gamma;
  for (int rho = blockIdx.x; rho < rows; rho += gridDim.x) {
    const int r = rho / gamma, k = rho % gamma;
    const int64_t ri = static_cast<int64_t>(r) * (gamma + 1) + k;
    const int64_t row = row0 ? static_cast<int64_t>(row0[r]) + k : ri;
    const typename Elt::T* t = target + row * V;
    // the thread's max Mn, M2 = Mn L2e rounded, and the sum of exp2(x L2e - M2)
    float Mn = neg_inf(), M2 = neg_inf(), S = 0.f;
    // batch vb: the thread's vectors at vb + u kStep, u < kAccBatch, kept as
    // raw 16-byte words until they are folded (past the row: -inf)
    auto fold = [&](const uint4 (&raw)[kAccBatch], int vb) {
      float e[kAccBatch][N];
      float m = neg_inf();
#pragma unroll
      for (int u = 0; u < kAccBatch; ++u) {
        RowVec<Elt>::unpack(raw[u], e[u]);
        const bool in = vb + u * kStep < V;
#pragma unroll
        for (int q = 0; q < N; ++q) {
          e[u][q] = in ? e[u][q] : neg_inf();
          m = fmaxf(m, e[u][q]);
        }
      }
      if (m == neg_inf()) return;                    // nothing but empty slots and -inf logits
      const float m2 = m * kL2e;
      if (m2 > M2) {
        S = S * __builtin_amdgcn_exp2f(M2 - m2);     // exp2(-inf) = 0 while S is still 0
        M2 = m2;
        Mn = m;
      }
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kAccBatch; ++u)
#pragma unroll
        for (int q = 0; q < N; ++q) s4[q & 3] += __builtin_amdgcn_exp2f(fmaf(e[u][q], kL2e, -M2));
      S += (s4[0] + s4[1]) + (s4[2] + s4[3]);
    };
    if ((V % N) == 0) {
      uint4 ra[kAccBatch], rb[kAccBatch];
      auto load = [&](uint4 (&raw)[kAccBatch], int vb) {
#pragma unroll
        for (int u = 0; u < kAccBatch; ++u) {
          const int v = vb + u * kStep;
          raw[u] = *reinterpret_cast<const uint4*>(t + (v < V ? v : 0));
        }
      };
      const int v0 = static_cast<int>(threadIdx.x) * N;
      load(ra, v0);
      for (int vb = v0; vb < V; vb += 2 * kAccBatch * kStep) {
        load(rb, vb + kAccBatch * kStep);
        fold(ra, vb);
        if (vb + kAccBatch * kStep >= V) break;
        load(ra, vb + 2 * kAccBatch * kStep);
        fold(rb, vb + kAccBatch * kStep);
      }
    } else {
      for (int v = static_cast<int>(threadIdx.x); v < V; v += kLseThreads) {
        const float x = Elt::load(t, v);
        if (x == neg_inf()) continue;
        const float x2 = x * kL2e;
        if (x2 > M2) {
          S = S * __builtin_amdgcn_exp2f(M2 - x2);
          M2 = x2;
          Mn = x;
        }
        S += __builtin_amdgcn_exp2f(fmaf(x, kL2e, -M2));
      }
    }
    // natural units for the readers: (Mn, sum of exp(x - Mn)).  Each term
    // is exp(x - Mn) 2^err with err = Mn L2e - M2, the rounding residual of
    // M2 (exact as one fma), taken out here.
    Lse acc = S > 0.f ? Lse{Mn, S * __builtin_amdgcn_exp2f(-fmaf(Mn, kL2e, -M2))} : Lse{neg_inf(), 0.f};
    acc = block_reduce_lse(acc, sh);
    if (threadIdx.x < kLseSplits)
      part[ri * kLseSplits + threadIdx.x] =
          threadIdx.x == 0 ? make_float2(acc.M, acc.S) : make_float2(neg_inf(), 0.f);
    __syncthreads();   // sh is reused by the next row
  }
}

// ------------------------------------------------------------------- accept

// One wave per request: lane i merges the parts of target row i into its
// log-normaliser (rows 0..l_r), gathers the target logit of draft i (its
// token is read before l_r is known, so the two loads overlap the part
// loads), evaluates the accept test of draft i, and the first failing draft,
// found by a ballot, ends the accepted prefix.
template <typename Elt>
__global__ __launch_bounds__(256) void verify_accept(int R, int gamma, int V, const typename Elt::T* __restrict__ target,
                                                     const int32_t* __restrict__ row0,
                                                     const int32_t* __restrict__ x,
                                                     const int32_t* __restrict__ ell,
                                                     const float2* __restrict__ part,
                                                     const float* __restrict__ logit,
                                                     const float* __restrict__ lse,
                                                     const float* __restrict__ u_acc,
                                                     float* __restrict__ lse_t, int32_t* __restrict__ n_acc) {
  const int r = blockIdx.x * 4 + static_cast<int>(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  const int64_t rbase = row0 ? static_cast<int64_t>(row0[r]) : static_cast<int64_t>(r) * (gamma + 1);
  // draft i = lane (a draft row below l_r <= gamma <= 64 is always in the first pass)
  const int xr = lane < gamma ? x[static_cast<int64_t>(r) * gamma + lane] : -1;
  const int L = min(max(ell[r], 0), gamma);
  int first_fail = L;
  for (int i0 = 0; i0 <= L; i0 += kWave) {   // gamma <= 64: at most two passes
    const int i = i0 + lane;
    bool fail = false;
    if (i <= L) {
      float txv = neg_inf();
      if (i < L) {
        const int xi = token_or_none(xr, V);
        if (xi >= 0) txv = Elt::load(target + (rbase + i) * V, xi);
      }
      const int64_t ri = static_cast<int64_t>(r) * (gamma + 1) + i;
      Lse acc{neg_inf(), 0.f};
#pragma unroll
      for (int sp = 0; sp < kLseSplits; ++sp) {
        const float2 pv = part[ri * kLseSplits + sp];
        acc = lse_combine(acc, Lse{pv.x, pv.y});
      }
      const float lt = acc.M + logf(acc.S);
      lse_t[ri] = lt;
      if (i < L) {
        const int64_t o = static_cast<int64_t>(r) * gamma + i;
        const float log_ratio = (txv - lt) - (logit[o] - lse[o]);
        fail = !(logf(u_acc[o]) < log_ratio);
      }
    }
    const unsigned long long b = __ballot(fail);
    if (b != 0ull && first_fail == L) first_fail = i0 + __ffsll(static_cast<long long>(b)) - 1;
  }
  if (lane == 0) n_acc[r] = first_fail;
}

// One wave per request, greedy verification: lane i merges the argmax parts
// of target row i (rows 0..l_r); the first draft that differs from its row's
// argmax ends the accepted prefix, and the argmax of the row where it ends
// is the next token.
__global__ __launch_bounds__(256) void verify_greedy_accept(int R, int gamma, const int32_t* __restrict__ ell,
                                                            const int32_t* __restrict__ x,
                                                            const float2* __restrict__ part,
                                                            int32_t* __restrict__ n_acc, int32_t* __restrict__ next_tok) {
  const int r = blockIdx.x * 4 + static_cast<int>(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  const int L = min(max(ell[r], 0), gamma);
  auto row_argmax = [&](int i) {
    const int64_t ri = static_cast<int64_t>(r) * (gamma + 1) + i;
    ArgMax a{neg_inf(), 0x7FFFFFFF};
#pragma unroll
    for (int sp = 0; sp < kLseSplits; ++sp) {
      const float2 pv = part[ri * kLseSplits + sp];
      a = argmax_combine(a, ArgMax{pv.x, __float_as_int(pv.y)});
    }
    return a.i;
  };
  int first_fail = L;
  for (int i0 = 0; i0 < L; i0 += kWave) {   // gamma <= 64: at most one full pass
    const int i = i0 + lane;
    const bool fail = i < L && x[static_cast<int64_t>(r) * gamma + i] != row_argmax(i);
    const unsigned long long b = __ballot(fail);
    if (b != 0ull && first_fail == L) first_fail = i0 + __ffsll(static_cast<long long>(b)) - 1;
  }
  if (lane == 0) {
    n_acc[r] = first_fail;
    next_tok[r] = row_argmax(first_fail);
  }
}

// ------------------------------------------------------- residual chunk masses

// Tiles whose chunk masses a residual work group keeps in LDS until the end
// of its sweep (4 KB each at 128 rows).
constexpr int kMassStage = 12;

// Row stride of the per-request chunk-mass arrays: ceil(V/16) rounded up to
// a multiple of four floats, so select can read them as 16-byte vectors.
__host__ __device__ __forceinline__ int mass_stride(int V) {
  return (V + 4 * kGChunk - 1) / (4 * kGChunk) * 4;
}

struct ResidualRow {
  int64_t trow;     // target row index
  int64_t urow;     // draft row index (request * gamma + n), valid when rej
  float lt, ld;     // target and draft log-normalisers of that row
  int prev;         // previous token for the Markov bias, -1 if none / not needed
  int64_t brow;     // row of the bias-vector table (W1: the previous token; or the given
                    // per-(request, position) vectors: the draft row), -1 for bias 0
  bool rej, live;
};

__device__ __forceinline__ ResidualRow residual_row(int req, int R, int gamma, int V, const int32_t* row0,
                                                    const int32_t* x0, const int32_t* x,
                                                    const int32_t* ell, const int32_t* n_acc,
                                                    const float* lse_t, const float* lse,
                                                    bool hasb) {
  ResidualRow rr{0, 0, 0.f, 0.f, -1, -1, false, false};
  if (req >= R) return rr;
  rr.live = true;
  const int L = min(max(ell[req], 0), gamma);
  const int n = min(max(n_acc[req], 0), L);
  rr.rej = n < L;
  rr.trow = row0 ? static_cast<int64_t>(row0[req]) + n : static_cast<int64_t>(req) * (gamma + 1) + n;
  rr.urow = static_cast<int64_t>(req) * gamma + (rr.rej ? n : 0);
  rr.lt = lse_t[static_cast<int64_t>(req) * (gamma + 1) + n];
  if (rr.rej) {
    rr.ld = lse[rr.urow];
    rr.prev = token_or_none((n == 0) ? x0[req] : x[static_cast<int64_t>(req) * gamma + n - 1], V);
    rr.brow = hasb ? rr.urow : rr.prev;
  }
  return rr;
}

// Row rho = r gamma + k of the analytic acceptance: target row k of request
// r against the drafter's distribution at position k (U row rho, the Markov
// bias of x_{k-1}, the sampler's normaliser lse[rho]); the target
// normaliser is merged from the row's parts.
__device__ __forceinline__ ResidualRow acceptance_row(int rho, int gamma, int V, const int32_t* row0,
                                                      const int32_t* x0, const int32_t* x, const float2* part,
                                                      const float* lse, bool hasb) {
  const int r = rho / gamma, k = rho % gamma;
  const int64_t ri = static_cast<int64_t>(r) * (gamma + 1) + k;
  ResidualRow rr;
  rr.trow = row0 ? static_cast<int64_t>(row0[r]) + k : ri;
  rr.urow = rho;
  Lse acc{neg_inf(), 0.f};
#pragma unroll
  for (int sp = 0; sp < kLseSplits; ++sp) {
    const float2 pv = part[ri * kLseSplits + sp];
    acc = lse_combine(acc, Lse{pv.x, pv.y});
  }
  rr.lt = acc.M + logf(acc.S);
  rr.ld = lse[rho];
  rr.prev = token_or_none(k == 0 ? x0[r] : x[rho - 1], V);
  rr.brow = hasb ? rho : rr.prev;
  rr.rej = true;
  rr.live = true;
  return rr;
}

// The residual row of every request, one sweep over the vocabulary in
// 64-token tiles with the sampler's 32x32x16 layout: work group = 2 RQ waves
// over 32 RQ requests, wave = (token half th, request quarter rq), lane (h, j)
// = request j and the sixteen tokens v0 + 32 th + 16 h + (0..15).  The draft
// logits U_n + B (Markov bias of the previous token on the matrix cores, U
// seeding the accumulators) and the target logits give each lane's sixteen
// values of p_t and max(0, p_t - p_d); their sums are the lane's 16-token
// chunk masses, stored directly.  Rows where every draft was accepted use
// p_t (the bonus row) and skip nothing: their draft part is computed on U
// row 0 and ignored.  W2t tiles go through registers into a double-buffered
// LDS area one tile ahead; the lane's own logits are loaded two tiles ahead
// (ACC with V a multiple of 16, whose B rows sit in LDS: the logits four
// tiles ahead and the W2t tiles two).
//
// ACC: the same sweep over the R gamma rows of the analytic acceptance
// (acceptance_row); each lane adds up min(p_t, p_d) over its tokens, and the
// request's four lanes leave one partial per work group in accp[rho][gx].
template <int RQ, int KS16, bool VEC, bool ACC>
__global__ __launch_bounds__(wide_threads<RQ>(), 1) void verify_residual_wide(
    int R, int gamma, int V, const uint16_t* __restrict__ target, const int32_t* __restrict__ row0,
    const uint16_t* __restrict__ U, const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2t,
    const int32_t* __restrict__ x0, const int32_t* __restrict__ x, const float* __restrict__ lse,
    const int32_t* __restrict__ ell, const int32_t* __restrict__ n_acc, const float* __restrict__ lse_t,
    float* __restrict__ csum, float* __restrict__ psum, const float2* __restrict__ part,
    float* __restrict__ accp, const uint16_t* __restrict__ bvec) {
  constexpr float kL2e = 1.4426950408889634f;
  constexpr int NROWS = 32 * RQ;
  constexpr int kW = wide_tile_bytes<KS16>();
  // ACC keeps the rows' B operands (W1 rows or bias vectors) in LDS rather
  // than registers, which leaves room for more tiles of logits in flight
  constexpr int kLaneAhead = ACC && VEC ? 4 : 2;   // tiles of the lane's logits in flight
  constexpr int kEB = KS16 * 32 + 16;       // bytes of an LDS B row (padded: rows of a half wave in different banks)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kW];
  __shared__ __attribute__((aligned(16))) uint8_t elds[ACC ? NROWS * kEB : 16];
  __shared__ float accsh[ACC ? NROWS : 1];
  // chunk masses of the work group's tiles, [tile][row][chunk of the tile],
  // written out together after the sweep (when the group has at most
  // kMassStage tiles; otherwise they are stored as they are made)
  __shared__ __attribute__((aligned(16))) float msh_c[ACC ? 1 : kMassStage][ACC ? 1 : NROWS][4];
  __shared__ __attribute__((aligned(16))) float msh_p[ACC ? 1 : kMassStage][ACC ? 1 : NROWS][4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int th = wave & 1;
  const int rq = wave >> 1;
  const int j = lane & 31;
  const int h = lane >> 5;
  const int nrows = ACC ? R * gamma : R;
  const int req = static_cast<int>(blockIdx.y) * NROWS + rq * 32 + j;
  const bool live = req < nrows;
  const int lofs = 32 * th + 16 * h;
  const int nTiles = (V + kChunk - 1) / kChunk;
  const int nG = (V + kGChunk - 1) / kGChunk;
  const int ldm = mass_stride(V);
  // work group b takes the contiguous tiles b per .. b per + nT - 1 (the
  // host launches ceil(nTiles / p) work groups for some p >= per, so the last
  // one starts below nTiles and nT >= 1): a request's chunk masses from one
  // work group are then one contiguous run
  const int per = (nTiles + static_cast<int>(gridDim.x) - 1) / static_cast<int>(gridDim.x);
  const int t0 = static_cast<int>(blockIdx.x) * per;
  const int nT = min(per, nTiles - t0);
  const bool staged = !ACC && nT <= kMassStage;
  const auto clampc = [&](int it) { return it < nT ? it : nT - 1; };
  const auto tile_of = [&](int it) { return t0 + it; };

  const ResidualRow rr = ACC ? acceptance_row(min(req, nrows - 1), gamma, V, row0, x0, x, part, lse, bvec)
                             : residual_row(min(req, R - 1), R, gamma, V, row0, x0, x, ell, n_acc, lse_t, lse, bvec);
  float mn = 0.f;   // ACC: the lane's sum of min(p_t, p_d)
  const uint16_t* trow = target + rr.trow * V;
  const uint16_t* urow = U + (rr.rej ? rr.urow : 0) * V;
  const float lt2 = rr.lt * kL2e;
  const float ld2 = rr.ld * kL2e;

  struct Lane {
    u32x4 t[2], u[2];
  };
  auto load_lane = [&](Lane& ll, int it) {
    const int v = tile_of(clampc(it)) * kChunk + lofs;
    load_lane16<VEC>(ll.t, trow, v, V);
    load_lane16<VEC>(ll.u, urow, v, V);
  };
  // W2t tiles in registers on their way to LDS: tile it + 1 waits in wr (in
  // wr for even it and wr2 for odd it when the tiles come two steps ahead,
  // at 128 rows per group and r >= 128)
  constexpr int kWAhead = kLaneAhead == 4 && RQ == 4 && KS16 >= 8 ? 2 : 1;
  WideW<KS16, RQ> wr, wr2;
  WideW<KS16, RQ>& wodd = kWAhead == 2 ? wr2 : wr;   // the set of odd steps
  wide_load_w<KS16, RQ>(wr, W2t, V, tile_of(0) * kChunk);
  Lane l0, l1, l2, l3;   // tiles it, it + 1, ... of the lane's logits (l2, l3 with four ahead)
  load_lane(l0, 0);
  load_lane(l1, 1);
  if constexpr (kLaneAhead == 4) {
    load_lane(l2, 2);
    load_lane(l3, 3);
  }
  bf16x8 e[KS16];
  const uint16_t* btab = bvec ? bvec : W1;
  const uint16_t* w1row = (rr.rej && rr.brow >= 0 ? btab + rr.brow * (KS16 * 16) : kZeroRow) + 8 * h;
#pragma unroll
  for (int ks = 0; ks < KS16; ++ks) e[ks] = load_bf16x8_global(w1row + 16 * ks);
  uint8_t* const erow = elds + (ACC ? (rq * 32 + j) * kEB + h * 16 : 0);   // the lane's B row (ACC)
  if constexpr (ACC) {
    if (th == 0)   // both token halves load the same rows
#pragma unroll
      for (int ks = 0; ks < KS16; ++ks) *reinterpret_cast<bf16x8*>(erow + ks * 32) = e[ks];
  }
  wide_store_w<KS16, RQ>(lds, wr);
  wide_load_w<KS16, RQ>(wr, W2t, V, tile_of(clampc(1)) * kChunk);
  if constexpr (kWAhead == 2) wide_load_w<KS16, RQ>(wr2, W2t, V, tile_of(clampc(2)) * kChunk);
  __syncthreads();

  // step it: the products read tile it from LDS; at its end tile it + 1 goes
  // from `wn` into the other LDS buffer and `wn` is reloaded with tile
  // it + 1 + kWAhead
  auto step = [&](int it, Lane& cur, WideW<KS16, RQ>& wn) {
    f32x16 acc, acc2 = {};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t w = cur.u[q >> 3][(q >> 1) & 3];
      acc[q] = __uint_as_float((q & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    float tv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t w = cur.t[q >> 3][(q >> 1) & 3];
      tv[q] = __uint_as_float((q & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    load_lane(cur, it + kLaneAhead);
    const uint8_t* arow = lds + (it & 1) * kW + ((32 * th + j) * wide_row_pieces<KS16>() + h) * 16;
    constexpr int KB = KS16 < 8 ? KS16 : 8;
#pragma unroll
    for (int k0 = 0; k0 < KS16; k0 += KB) {
      bf16x8 a[KB];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) a[kk] = *reinterpret_cast<const bf16x8*>(arow + (k0 + kk) * 32);
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const bf16x8 b = ACC ? *reinterpret_cast<const bf16x8*>(erow + (k0 + kk) * 32) : e[k0 + kk];
        if (kk & 1)
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], b, acc2, 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], b, acc, 0, 0, 0);
      }
    }
    float cs = 0.f, ps = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float at = fmaf(tv[q], kL2e, -lt2);
      const float ad = fmaf(acc[q] + acc2[q], kL2e, -ld2);
      if constexpr (ACC) {
        cs += __builtin_amdgcn_exp2f(fminf(at, ad));   // min(p_t, p_d): exp2 is monotone
      } else {
        const float pt = __builtin_amdgcn_exp2f(at);
        const float pd = __builtin_amdgcn_exp2f(ad);
        ps += pt;
        cs += rr.rej ? fmaxf(0.f, pt - pd) : pt;
      }
    }
    if constexpr (ACC) {
      mn += cs;
    } else if (staged) {
      msh_c[it][rq * 32 + j][2 * th + h] = cs;
      msh_p[it][rq * 32 + j][2 * th + h] = ps;
    } else {
      const int c16 = 4 * tile_of(it) + 2 * th + h;
      if (live && c16 < nG) {
        csum[static_cast<int64_t>(req) * ldm + c16] = cs;
        psum[static_cast<int64_t>(req) * ldm + c16] = ps;
      }
    }
    wide_store_w<KS16, RQ>(lds + ((it + 1) & 1) * kW, wn);
    wide_load_w<KS16, RQ>(wn, W2t, V, tile_of(clampc(it + 1 + kWAhead)) * kChunk);
    __syncthreads();
  };
  int it = 0;
  if constexpr (kLaneAhead == 4) {   // even steps store tiles from wr, odd steps from wodd
    for (; it + 3 < nT; it += 4) {
      step(it, l0, wr);
      step(it + 1, l1, wodd);
      step(it + 2, l2, wr);
      step(it + 3, l3, wodd);
    }
    if (it < nT) step(it, l0, wr);
    if (it + 1 < nT) step(it + 1, l1, wodd);
    if (it + 2 < nT) step(it + 2, l2, wr);
  } else {
    for (; it + 1 < nT; it += 2) {
      step(it, l0, wr);
      step(it + 1, l1, wr);
    }
    if (it < nT) step(it, l0, wr);
  }
  if (staged) {
    // the staged masses: four chunks (16 bytes) per (tile, row) item, a
    // request's items of consecutive tiles adjacent in memory
    const int row0g = static_cast<int>(blockIdx.y) * NROWS;
    for (int e = threadIdx.x; e < nT * NROWS; e += wide_threads<RQ>()) {
      const int row = e / nT, itl = e % nT;
      const int rr_ = row0g + row;
      if (rr_ >= nrows) continue;
      const int c0 = 4 * tile_of(itl);
      float* dc = csum + static_cast<int64_t>(rr_) * ldm + c0;
      float* dp = psum + static_cast<int64_t>(rr_) * ldm + c0;
      if (c0 + 3 < nG) {
        *reinterpret_cast<float4*>(dc) = *reinterpret_cast<const float4*>(msh_c[itl][row]);
        *reinterpret_cast<float4*>(dp) = *reinterpret_cast<const float4*>(msh_p[itl][row]);
      } else {
        for (int q = 0; q < 4 && c0 + q < nG; ++q) {
          dc[q] = msh_c[itl][row][q];
          dp[q] = msh_p[itl][row][q];
        }
      }
    }
  }
  if constexpr (ACC) {
    const float t = mn + xor32(mn);   // the request's two lanes of this token half
    if (th == 1 && h == 0) accsh[rq * 32 + j] = t;
    __syncthreads();
    if (th == 0 && h == 0 && live)
      accp[static_cast<int64_t>(req) * gridDim.x + blockIdx.x] = t + accsh[rq * 32 + j];
  }
}

__global__ __launch_bounds__(64) void verify_residual_f32(
    int R, int gamma, int V, int r, const float* __restrict__ target, const int32_t* __restrict__ row0,
    const float* __restrict__ U, const float* __restrict__ W1, const float* __restrict__ W2t,
    const int32_t* __restrict__ x0, const int32_t* __restrict__ x, const float* __restrict__ lse,
    const int32_t* __restrict__ ell, const int32_t* __restrict__ n_acc, const float* __restrict__ lse_t,
    float* __restrict__ csum, float* __restrict__ psum, const float* __restrict__ bvec) {
  const int tile = blockIdx.x;
  const int req = blockIdx.y;
  const int lane = threadIdx.x;
  const ResidualRow rr = residual_row(req, R, gamma, V, row0, x0, x, ell, n_acc, lse_t, lse, bvec);
  const int v = tile * kChunk + lane;
  float res = 0.f, pt = 0.f;
  if (v < V) {
    pt = __expf(target[rr.trow * V + v] - rr.lt);
    res = pt;
    if (rr.rej) {
      float b = 0.f;
      if (rr.brow >= 0) {
        const float* e = (bvec ? bvec : W1) + rr.brow * r;
        const float* w = W2t + static_cast<int64_t>(v) * r;
        for (int i = 0; i < r; ++i) b = fmaf(e[i], w[i], b);
      }
      res = fmaxf(0.f, pt - __expf(U[rr.urow * V + v] + b - rr.ld));
    }
  }
  // masses of each 16-token chunk: a reduction over each quarter of the wave
#pragma unroll
  for (int o = 1; o < kGChunk; o <<= 1) {
    res += __shfl_xor(res, o);
    pt += __shfl_xor(pt, o);
  }
  const int nG = (V + kGChunk - 1) / kGChunk;
  const int ldm = mass_stride(V);
  const int c16 = tile * (kChunk / kGChunk) + lane / kGChunk;
  if ((lane & (kGChunk - 1)) == 0 && c16 < nG) {
    csum[static_cast<int64_t>(req) * ldm + c16] = res;
    psum[static_cast<int64_t>(req) * ldm + c16] = pt;
  }
}

// fp32 storage, the analytic acceptance: one wave per (row rho, 64-token
// tile), plain FMA bias; the wave's sum of min(p_t, p_d) is the partial
// accp[rho][tile].
__global__ __launch_bounds__(64) void verify_acceptance_f32(
    int R, int gamma, int V, int r, const float* __restrict__ target, const int32_t* __restrict__ row0,
    const float* __restrict__ U, const float* __restrict__ W1, const float* __restrict__ W2t,
    const int32_t* __restrict__ x0, const int32_t* __restrict__ x, const float* __restrict__ lse,
    const float2* __restrict__ part, float* __restrict__ accp, const float* __restrict__ bvec) {
  const int rho = blockIdx.x;
  const int tile = blockIdx.y;
  const int lane = threadIdx.x;
  const ResidualRow rr = acceptance_row(rho, gamma, V, row0, x0, x, part, lse, bvec);
  const int v = tile * kChunk + lane;
  float mn = 0.f;
  if (v < V) {
    const float pt = __expf(target[rr.trow * V + v] - rr.lt);
    float b = 0.f;
    if (rr.brow >= 0) {
      const float* e = (bvec ? bvec : W1) + rr.brow * r;
      const float* w = W2t + static_cast<int64_t>(v) * r;
      for (int i = 0; i < r; ++i) b = fmaf(e[i], w[i], b);
    }
    mn = fminf(pt, __expf(U[rr.urow * V + v] + b - rr.ld));
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) mn += __shfl_xor(mn, o);
  if (lane == 0) accp[static_cast<int64_t>(rho) * gridDim.y + tile] = mn;
}

// c*[rho] = the sum of its partials, in order.
__global__ __launch_bounds__(256) void acceptance_finish(int rows, int parts, const float* __restrict__ accp,
                                                         float* __restrict__ c_star) {
  const int rho = blockIdx.x * blockDim.x + threadIdx.x;
  if (rho >= rows) return;
  const float* p = accp + static_cast<int64_t>(rho) * parts;
  float t = 0.f;
  for (int b = 0; b < parts; ++b) t += p[b];
  c_star[rho] = t;
}

// -------------------------------------------------------------------- select

// The next token of every request, one work group each: the chunk holding
// u * Z in the prefix of the chunk masses (Z their total; when the residual
// vanished, Z <= 0, the draw falls back to p_t), then the token inside that
// chunk from its sixteen recomputed values.  The masses are read as 16-byte
// vectors into registers (a run of 4 kSelVec per thread), scanned per wave and
// across the waves; the chunk's Markov biases are dot products split over
// sixteen threads per token against the previous token's W1 row in LDS.
template <typename Elt>
__global__ __launch_bounds__(256) void verify_select(
    int R, int gamma, int V, int r, const typename Elt::T* __restrict__ target,
    const int32_t* __restrict__ row0, const typename Elt::T* __restrict__ U,
    const typename Elt::T* __restrict__ W1, const typename Elt::T* __restrict__ W2t,
    const int32_t* __restrict__ x0, const int32_t* __restrict__ x, const float* __restrict__ lse,
    const int32_t* __restrict__ ell, const int32_t* __restrict__ n_acc, const float* __restrict__ lse_t,
    const float* __restrict__ u_res, const float* __restrict__ csum, const float* __restrict__ psum,
    int32_t* __restrict__ next_tok, const typename Elt::T* __restrict__ bvec) {
  constexpr int kT = 256;
  constexpr int kSelVec = 12;
  __shared__ float wsum[kT / kWave];
  __shared__ float e_row[1024];
  __shared__ float s_val[kGChunk];
  __shared__ int s_chunk, s_last;
  __shared__ float s_before, s_last_before;
  const int req = blockIdx.x;
  const int tid = threadIdx.x;
  const int nG = (V + kGChunk - 1) / kGChunk;
  const int ldm = mass_stride(V);
  const ResidualRow rr = residual_row(req, R, gamma, V, row0, x0, x, ell, n_acc, lse_t, lse, bvec);
  // the previous token's W1 row (or the given bias vector), for the bias of the chunk's tokens
  if (rr.rej && rr.brow >= 0)
    for (int i = tid; i < r; i += kT) e_row[i] = Elt::load(bvec ? bvec : W1, rr.brow * r + i);
  const int seg4 = (ldm / 4 + kT - 1) / kT;    // vectors per thread
  const int lo = tid * seg4 * 4;
  const int hi = min(nG, lo + seg4 * 4);
  const bool inreg = seg4 <= kSelVec;
  float vals[4 * kSelVec];
  bool use_pt = !rr.rej;
  const float* sums = (rr.rej ? csum : psum) + static_cast<int64_t>(req) * ldm;
  float Z = 0.f, excl = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    float local = 0.f;
    if (inreg) {
      const float4* s4 = reinterpret_cast<const float4*>(sums);
#pragma unroll
      for (int q = 0; q < kSelVec; ++q) {
        const int c = lo + 4 * q;
        const float4 f = (q < seg4 && c < ldm) ? s4[c / 4] : make_float4(0.f, 0.f, 0.f, 0.f);
        vals[4 * q] = c < nG ? f.x : 0.f;
        vals[4 * q + 1] = c + 1 < nG ? f.y : 0.f;
        vals[4 * q + 2] = c + 2 < nG ? f.z : 0.f;
        vals[4 * q + 3] = c + 3 < nG ? f.w : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4 * kSelVec; ++q) local += vals[q];
    } else {
      for (int cc = lo; cc < hi; ++cc) local += sums[cc];
    }
    float incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const float v = __shfl_up(incl, o);
      if ((tid & (kWave - 1)) >= o) incl += v;
    }
    if ((tid & (kWave - 1)) == kWave - 1) wsum[tid / kWave] = incl;
    __syncthreads();
    float before = 0.f;
    Z = 0.f;
#pragma unroll
    for (int wv = 0; wv < kT / kWave; ++wv) {
      before += wv < tid / kWave ? wsum[wv] : 0.f;
      Z += wsum[wv];
    }
    excl = before + incl - local;
    __syncthreads();
    if (Z > 0.f || use_pt) break;
    use_pt = true;                       // residual vanished: draw from p_t
    sums = psum + static_cast<int64_t>(req) * ldm;
  }
  const float thr = u_res[req] * Z;
  if (tid == 0) {
    s_chunk = 0x7FFFFFFF;
    s_last = -1;
  }
  __syncthreads();
  float run = excl;
  int first = 0x7FFFFFFF, last = -1;
  float before = 0.f, last_before = 0.f;
  auto visit = [&](int cc, float sv) {
    if (sv > 0.f) {
      last = cc;
      last_before = run;
    }
    if (first == 0x7FFFFFFF && run + sv > thr) {
      first = cc;
      before = run;
    }
    run += sv;
  };
  if (inreg) {
#pragma unroll
    for (int q = 0; q < 4 * kSelVec; ++q)
      if (lo + q < hi) visit(lo + q, vals[q]);
  } else {
    for (int cc = lo; cc < hi; ++cc) visit(cc, sums[cc]);
  }
  if (first != 0x7FFFFFFF) atomicMin(&s_chunk, first);
  if (last >= 0) atomicMax(&s_last, last);
  __syncthreads();
  if (first != 0x7FFFFFFF && first == s_chunk) s_before = before;
  if (last >= 0 && last == s_last) s_last_before = last_before;
  __syncthreads();
  // the chunk holding u * Z; rounding past the end falls back to the last
  // chunk with mass
  const bool found = s_chunk != 0x7FFFFFFF;
  const int chunk = found ? s_chunk : max(s_last, 0);
  const float base = found ? s_before : s_last_before;
  const int tk = tid / kGChunk;      // token of the chunk
  const int sl = tid % kGChunk;      // slice of its bias dot product
  const int v = chunk * kGChunk + tk;
  float tl = 0.f, ul = 0.f, b = 0.f;
  if (v < V) {
    if (sl == 0) {
      tl = Elt::load(target, rr.trow * V + v);
      if (!use_pt) ul = Elt::load(U, rr.urow * V + v);
    }
    if (!use_pt && rr.brow >= 0) {
      const typename Elt::T* w = W2t + static_cast<int64_t>(v) * r;
#pragma unroll 16
      for (int i = sl; i < r; i += kGChunk) b = fmaf(e_row[i], Elt::load(w, i), b);
    }
  }
#pragma unroll
  for (int o = 1; o < kGChunk; o <<= 1) b += __shfl_xor(b, o);
  if (sl == 0) {
    float val = 0.f;
    if (v < V) {
      const float pt = __expf(tl - rr.lt);
      val = use_pt ? pt : fmaxf(0.f, pt - __expf(ul + b - rr.ld));
    }
    s_val[tk] = val;
  }
  __syncthreads();
  if (tid < kWave) {
    const float val = tid < kGChunk ? s_val[tid] : 0.f;
    const float cum = wave_inclusive_scan(val);
    const unsigned long long hit = __ballot(tid < kGChunk && cum > thr - base);
    int off;
    if (hit) {
      off = __ffsll(static_cast<long long>(hit)) - 1;
    } else {
      const unsigned long long pos = __ballot(val > 0.f);
      off = pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
    }
    if (tid == 0) next_tok[req] = chunk * kGChunk + off;
  }
}

// ------------------------------------------------------------------ host side

struct VerifyWs {
  float* lse_t;   // [R][gamma+1]
  float2* part;   // [R][gamma+1][kLseSplits] (max, sum) parts of the target log-normalisers
  float* csum;    // [R][mass_stride(V)] residual mass of each 16-token chunk
  float* psum;    // [R][mass_stride(V)] p_t mass of each 16-token chunk
};

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t verify_workspace_bytes(int R, int gamma, int V) {
  const size_t nC = static_cast<size_t>(mass_stride(V));
  return align256(sizeof(float) * R * (gamma + 1)) + align256(sizeof(float2) * R * (gamma + 1) * kLseSplits) +
         2 * align256(sizeof(float) * R * nC);
}

static VerifyWs carve(void* ws, int R, int gamma, int V) {
  const size_t nC = static_cast<size_t>(mass_stride(V));
  char* p = static_cast<char*>(ws);
  VerifyWs w;
  w.lse_t = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * R * (gamma + 1));
  w.part = reinterpret_cast<float2*>(p);
  p += align256(sizeof(float2) * R * (gamma + 1) * kLseSplits);
  w.csum = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * R * nC);
  w.psum = reinterpret_cast<float*>(p);
  return w;
}

int compute_units();   // abi.hip

// Arguments of one residual or acceptance sweep.
struct SweepArgs {
  int R, gamma, V;
  const void *target, *U, *W1, *W2t;
  const int32_t *row0, *x0, *x, *ell, *n_acc;
  const float* lse;
  const float* lse_t;
  float *csum, *psum;
  const float2* part;
  float* accp;
  const void* bvec;   // per-(request, position) bias vectors in W1[x_prev]'s place, or null
};

// Launches the 32x32x16 sweep over `rows` rows (R residual rows, or R gamma
// acceptance rows) and returns its work groups along the vocabulary.
template <int RQ, int KS16, bool ACC>
static int launch_residual_wide(const SweepArgs& a, int rows, hipStream_t s) {
  const int nTiles = ceil_div(a.V, kChunk);
  const int groups = ceil_div(rows, 32 * RQ);
  int gx = compute_units() / groups;
  gx = gx < 1 ? 1 : (gx > nTiles ? nTiles : gx);
  gx = ceil_div(nTiles, ceil_div(nTiles, gx));   // every work group has at least one tile
  dim3 grid(gx, groups);
  const auto b16 = [](const void* p) { return static_cast<const uint16_t*>(p); };
  if (a.V % kGChunk == 0)
    hipLaunchKernelGGL((verify_residual_wide<RQ, KS16, true, ACC>), grid, dim3(wide_threads<RQ>()), 0, s, a.R,
                       a.gamma, a.V, b16(a.target), a.row0, b16(a.U), b16(a.W1), b16(a.W2t), a.x0, a.x, a.lse,
                       a.ell, a.n_acc, a.lse_t, a.csum, a.psum, a.part, a.accp, b16(a.bvec));
  else
    hipLaunchKernelGGL((verify_residual_wide<RQ, KS16, false, ACC>), grid, dim3(wide_threads<RQ>()), 0, s, a.R,
                       a.gamma, a.V, b16(a.target), a.row0, b16(a.U), b16(a.W1), b16(a.W2t), a.x0, a.x, a.lse,
                       a.ell, a.n_acc, a.lse_t, a.csum, a.psum, a.part, a.accp, b16(a.bvec));
  return gx;
}

template <int KS16, bool ACC>
static int launch_residual_wide_ks(const SweepArgs& a, int rows, hipStream_t s) {
  if (rows <= 32) return launch_residual_wide<1, KS16, ACC>(a, rows, s);
  if (rows <= 64) return launch_residual_wide<2, KS16, ACC>(a, rows, s);
  return launch_residual_wide<4, KS16, ACC>(a, rows, s);
}

template <bool ACC>
static int launch_residual_wide_r(const SweepArgs& a, int r, int rows, hipStream_t s) {
  switch (r / 32) {
    case 1: return launch_residual_wide_ks<2, ACC>(a, rows, s);
    case 2: return launch_residual_wide_ks<4, ACC>(a, rows, s);
    case 4: return launch_residual_wide_ks<8, ACC>(a, rows, s);
    default: return launch_residual_wide_ks<16, ACC>(a, rows, s);
  }
}

hipError_t verify_launch(dspark_dtype dt, int R, int gamma, int V, int r, const void* target,
                         const int32_t* row0, const void* U, const void* W1, const void* W2t,
                         const int32_t* x0, const int32_t* x, const float* lse, const float* logit,
                         const int32_t* ell, const float* u_acc, const float* u_res, int32_t* n_acc,
                         int32_t* next_tok, void* ws, hipStream_t s, const void* bvec) {
  const VerifyWs w = carve(ws, R, gamma, V);
  hipError_t err;
  const int64_t items = static_cast<int64_t>(R) * (gamma + 1) * kLseSplits;
  const int gridp = static_cast<int>(items < 4LL * compute_units() ? items : 4LL * compute_units());
  if (dt == DSPARK_BF16) {
    hipLaunchKernelGGL((verify_target_part<BF16, kPartLse>), dim3(gridp), dim3(kLseThreads), 0, s, R, gamma, V,
                       static_cast<const uint16_t*>(target), row0, ell, w.part);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(verify_accept<BF16>, dim3(ceil_div(R, 4)), dim3(256), 0, s, R, gamma, V,
                       static_cast<const uint16_t*>(target), row0, x, ell, w.part, logit, lse, u_acc, w.lse_t, n_acc);
  } else {
    hipLaunchKernelGGL((verify_target_part<F32, kPartLse>), dim3(gridp), dim3(kLseThreads), 0, s, R, gamma, V,
                       static_cast<const float*>(target), row0, ell, w.part);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(verify_accept<F32>, dim3(ceil_div(R, 4)), dim3(256), 0, s, R, gamma, V,
                       static_cast<const float*>(target), row0, x, ell, w.part, logit, lse, u_acc, w.lse_t, n_acc);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (dt == DSPARK_BF16) {
    const SweepArgs a{R, gamma, V, target, U, W1, W2t, row0, x0, x, ell, n_acc, lse, w.lse_t, w.csum, w.psum,
                      nullptr, nullptr, bvec};
    launch_residual_wide_r<false>(a, r, R, s);
  } else {
    hipLaunchKernelGGL(verify_residual_f32, dim3(ceil_div(V, kChunk), R), dim3(64), 0, s, R, gamma, V, r,
                       static_cast<const float*>(target), row0, static_cast<const float*>(U),
                       static_cast<const float*>(W1), static_cast<const float*>(W2t), x0, x, lse, ell,
                       n_acc, w.lse_t, w.csum, w.psum, static_cast<const float*>(bvec));
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (dt == DSPARK_BF16)
    hipLaunchKernelGGL(verify_select<BF16>, dim3(R), dim3(256), 0, s, R, gamma, V, r,
                       static_cast<const uint16_t*>(target), row0, static_cast<const uint16_t*>(U),
                       static_cast<const uint16_t*>(W1), static_cast<const uint16_t*>(W2t), x0, x, lse,
                       ell, n_acc, w.lse_t, u_res, w.csum, w.psum, next_tok, static_cast<const uint16_t*>(bvec));
  else
    hipLaunchKernelGGL(verify_select<F32>, dim3(R), dim3(256), 0, s, R, gamma, V, r,
                       static_cast<const float*>(target), row0, static_cast<const float*>(U),
                       static_cast<const float*>(W1), static_cast<const float*>(W2t), x0, x, lse, ell,
                       n_acc, w.lse_t, u_res, w.csum, w.psum, next_tok, static_cast<const float*>(bvec));
  return hipGetLastError();
}

// ------------------------------------------------------ greedy / acceptance

size_t verify_greedy_workspace_bytes(int R, int gamma) {
  return align256(sizeof(float2) * R * (gamma + 1) * kLseSplits);
}

size_t acceptance_workspace_bytes(int R, int gamma, int V) {
  return align256(sizeof(float2) * R * (gamma + 1) * kLseSplits) +
         align256(sizeof(float) * static_cast<size_t>(R) * gamma * ceil_div(V, kChunk));
}

static int part_grid(int R, int gamma) {
  const int64_t items = static_cast<int64_t>(R) * (gamma + 1) * kLseSplits;
  return static_cast<int>(items < 4LL * compute_units() ? items : 4LL * compute_units());
}

hipError_t verify_greedy_launch(dspark_dtype dt, int R, int gamma, int V, const void* target, const int32_t* row0,
                                const int32_t* x, const int32_t* ell, int32_t* n_acc, int32_t* next_tok, void* ws,
                                hipStream_t s) {
  float2* part = static_cast<float2*>(ws);
  const int gridp = part_grid(R, gamma);
  if (dt == DSPARK_BF16)
    hipLaunchKernelGGL((verify_target_part<BF16, kPartArgmax>), dim3(gridp), dim3(kLseThreads), 0, s, R, gamma, V,
                       static_cast<const uint16_t*>(target), row0, ell, part);
  else
    hipLaunchKernelGGL((verify_target_part<F32, kPartArgmax>), dim3(gridp), dim3(kLseThreads), 0, s, R, gamma, V,
                       static_cast<const float*>(target), row0, ell, part);
  hipError_t err;
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(verify_greedy_accept, dim3(ceil_div(R, 4)), dim3(256), 0, s, R, gamma, ell, x, part, n_acc,
                     next_tok);
  return hipGetLastError();
}

hipError_t acceptance_launch(dspark_dtype dt, int R, int gamma, int V, int r, const void* target,
                             const int32_t* row0, const void* U, const void* W1, const void* W2t, const int32_t* x0,
                             const int32_t* x, const float* lse, float* c_star, void* ws, hipStream_t s,
                             const void* bvec) {
  float2* part = static_cast<float2*>(ws);
  float* accp = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         align256(sizeof(float2) * R * (gamma + 1) * kLseSplits));
  const int rowsn = R * gamma;
  const int gridn = rowsn < 8 * compute_units() ? rowsn : 8 * compute_units();
  if (dt == DSPARK_BF16)
    hipLaunchKernelGGL(acceptance_target_lse<BF16>, dim3(gridn), dim3(kLseThreads), 0, s, R, gamma, V,
                       static_cast<const uint16_t*>(target), row0, part);
  else
    hipLaunchKernelGGL(acceptance_target_lse<F32>, dim3(gridn), dim3(kLseThreads), 0, s, R, gamma, V,
                       static_cast<const float*>(target), row0, part);
  hipError_t err;
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int rows = R * gamma;
  int parts;
  if (dt == DSPARK_BF16) {
    const SweepArgs a{R, gamma, V, target, U, W1, W2t, row0, x0, x, nullptr, nullptr, lse, nullptr, nullptr,
                      nullptr, part, accp, bvec};
    parts = launch_residual_wide_r<true>(a, r, rows, s);
  } else {
    parts = ceil_div(V, kChunk);
    hipLaunchKernelGGL(verify_acceptance_f32, dim3(rows, parts), dim3(64), 0, s, R, gamma, V, r,
                       static_cast<const float*>(target), row0, static_cast<const float*>(U),
                       static_cast<const float*>(W1), static_cast<const float*>(W2t), x0, x, lse, part, accp,
                       static_cast<const float*>(bvec));
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(acceptance_finish, dim3(ceil_div(rows, 256)), dim3(256), 0, s, rows, parts, accp, c_star);
  return hipGetLastError();
}

}  // namespace dspark
