// The Markov-head sampling loop for batches of more than 64 requests, with
// W2t held on chip and one grid barrier per block of 32 requests.
//
// Passage: DSpark reading notes, eq (4) (the bias is added inside the
// softmax) and eq (5) (Markov head B(x_{k-1}, .) = W1[x_{k-1}] W2, rank r);
// caijizhuo section 四, the sequential loop of dspark_cycle.  The draw is the
// exact two-level Gumbel-max of the other sampling kernels (chunk-level
// log-sum-exp plus chunk Gumbel, then the in-chunk argmax).
//
// The sequential dependence of the loop is per request: position k of a
// request needs only that request's token at k - 1.  This kernel walks the
// (position, request block) steps s = k * nb + rb in order, and the grid
// meets once per step instead of once per position: after step s every work
// group merges its draw of the block into the requests' key slots and
// arrives at the block's own barrier counters, while it goes on with the
// other blocks.  The keys of step s are needed again only nb steps later
// (step s + nb, the same block at the next position), so the barrier wait,
// the key read and the W1-row gather of a block all happen while the work
// group computes the blocks in between.
//
// Each of these round trips is carried by one wave at fixed points of the
// steps in between (at a step's start and between its matrix products and
// its fold), so no wave ever spins while the result is still on its way:
//   producer of step t (wave t mod 8):
//     start of step t+1   merge the waves' results, key atomics (returning)
//     middle of step t+1  once they have returned: arrive at the block's
//                         group counter
//   consumer of step c = t + nb (wave c mod 8):
//     middle of step c-2  load the block's eight group counters
//     start of step c-1   check them (wait, bounded, only if incomplete);
//                         load the block's key slots of position k - 1
//     middle of step c-1  decode the tokens; copy their W1 rows and the
//                         block's in-chunk Gumbels straight into LDS
//                         (global_load_lds, no registers)
//     end of step c-1     wait for those copies, then the work group barrier
// Two LDS slots (step parity) hold the W1 rows and in-chunk Gumbels; each
// parity has arrays of its own, so the compiler never makes a read of one
// slot wait for the copy into the other.
//
// W2t stays on chip as in the one-barrier-per-position kernel
// (sample_res.hip): one work group per compute unit owns a contiguous range
// of at most eight 64-token tiles, each wave holds one tile's A fragments
// (32x32x16 MFMA, rows permuted so a lane's sixteen accumulators are one
// Gumbel chunk) for the whole launch, in registers and, at r = 256, partly
// in LDS.  The 32 W1 rows of a slot are stored piece-major (16-byte piece p
// of row j at 512 p + 16 j): a B fragment is then 512 contiguous bytes per
// half wave, and each 1 KB copy fills two pieces of every row, so a lane
// copies only from its own request's row.
#include <hip/hip_ext.h>

#include "wide_tile.hpp"
#include "sample_keys.hpp"
#include "sample_common.hpp"

#include <atomic>

namespace dspark {

constexpr int kPipeWaves = 8;
constexpr int kPipeThreads = kPipeWaves * kWave;   // 512
constexpr int kPipeMaxTiles = kPipeWaves;          // one tile per wave
constexpr int kPipeMinBlocks = 3;                  // fewer blocks leave no steps to hide a barrier behind
constexpr int kHalfSlots = kPipeKeySlots / 2;      // key slots one lane reads

// k-steps of each wave's A fragments kept in LDS rather than registers
template <int KS16>
__host__ __device__ constexpr int pipe_lds_ksteps() { return KS16 >= 16 ? 4 : 0; }

// Work-group barrier for LDS only: the waves' LDS operations have completed,
// but their loads from memory may still be in flight (the step's logit
// loads for two steps ahead; the copies into LDS are waited for by the
// wave that issued them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Vector memory instructions of one step's logit and chunk-Gumbel loads
// (two 16-byte logit loads and one Gumbel load per token half), at least.
constexpr int kStepLoads = 6;

// A request block's logits and chunk Gumbels for one lane: tokens
// 32 tb + 16 h .. + 15 of the wave's tile for tb = 0, 1.
struct PipeLane {
  u32x4 u[2][2];
  float G[2];
};

template <int KS16, bool VEC>
__global__ __launch_bounds__(kPipeThreads, 1) void sample_steps_pipe(
    int R, int gamma, int V, const uint16_t* __restrict__ U, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W2t, const int32_t* __restrict__ x0, const float* __restrict__ G,
    const float* __restrict__ g, SampleWs ws, const uint32_t* __restrict__ cancel) {
  static_assert(kGChunk == 16 && kChunk == 64, "one Gumbel chunk per lane of a 32x32 output block");
  constexpr int kRowB = KS16 * 32;   // bytes of a W1 row
  constexpr int KL = pipe_lds_ksteps<KS16>();
  constexpr int KR = KS16 - KL;
  __shared__ __attribute__((aligned(1024))) uint8_t eslot0[32 * kRowB];
  __shared__ __attribute__((aligned(1024))) uint8_t eslot1[32 * kRowB];
  __shared__ __attribute__((aligned(1024))) float gslot0[32][kGChunk];
  __shared__ __attribute__((aligned(1024))) float gslot1[32][kGChunk];
  __shared__ unsigned long long mkey0[kPipeWaves][32], mkey1[kPipeWaves][32];
  __shared__ float2 mlse0[kPipeWaves][32], mlse1[kPipeWaves][32];
  __shared__ __attribute__((aligned(1024))) bf16x8 alds[KL > 0 ? kPipeWaves : 1][2][KL > 0 ? KL : 1][kWave];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int j = lane & 31;
  const int h = lane >> 5;
  const int nTiles = (V + kChunk - 1) / kChunk;
  const int nG = (V + kGChunk - 1) / kGChunk;
  const int gx = static_cast<int>(gridDim.x), bx = static_cast<int>(blockIdx.x);
  const int base = nTiles / gx, rem = nTiles % gx;
  const int nT = base + (bx < rem ? 1 : 0);
  const int t0 = bx * base + min(bx, rem);
  const int tile = t0 + min(wave, nT - 1);
  const int v0 = tile * kChunk;
  const int nb = (R + 31) / 32;      // request blocks (kPipeMinBlocks .. kPipeMaxBlocks)
  const int s_end = gamma * nb;      // steps s = k * nb + rb
  unsigned int* const dom = ws.bar + kPipeBarBase;
  const int grp = bx % kBarGroups;

  // 1. W2t: the wave's tile as A fragments, the first KR k-steps into
  // registers, the rest straight into LDS
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

  // logits and chunk Gumbels of step (k, rb) for this lane
  auto load_step = [&](PipeLane& p, int k, int rb) {
    const int reqc = min(32 * rb + j, R - 1);
    const uint16_t* row = U + (static_cast<int64_t>(reqc) * gamma + k) * V;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      load_lane16<VEC>(p.u[tb], row, v0 + 32 * tb + 16 * h, V);
      p.G[tb] = G[(static_cast<int64_t>(k) * nG + min(4 * tile + 2 * tb + h, nG - 1)) * R + reqc];
    }
  };

  // --- the round trips of a block (see the head of the file) ---

  // producer, start of step t + 1: merge the waves' results of step t into
  // the requests' key slots (atomic max) and log-sum-exp partials
  auto merge_step = [&](int k, int rb, const unsigned long long (*mk)[32], const float2 (*ml)[32]) {
    // lane (h, j): request j over waves 4 h .. 4 h + 3, then the two halves
    unsigned long long key = 0ull;
    float M2[4], T[4], M = neg_inf();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int w = 4 * h + q;
      const unsigned long long ok = w < nT ? mk[w][j] : 0ull;
      const float2 o = w < nT ? ml[w][j] : make_float2(neg_inf(), 0.f);
      key = ok > key ? ok : key;
      M2[q] = o.x;
      T[q] = o.y;
      M = fmaxf(M, o.x);
    }
    float Ts = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) Ts += M2[q] == neg_inf() ? 0.f : T[q] * __builtin_amdgcn_exp2f(M2[q] - M);
    const unsigned long long ko = xor32(key);
    const float Mo = xor32(M), To = xor32(Ts);
    key = ko > key ? ko : key;
    const float Mn = fmaxf(M, Mo);
    Ts = (M == neg_inf() ? 0.f : Ts * __builtin_amdgcn_exp2f(M - Mn)) + (Mo == neg_inf() ? 0.f : To * __builtin_amdgcn_exp2f(Mo - Mn));
    const int i = 32 * rb + j;
    if (h == 0 && i < R) {
      ws.lsep[(static_cast<int64_t>(k) * R + i) * gx + bx] = make_float2(Mn * kLn2, Ts);
      if (key != 0ull)
        __hip_atomic_fetch_max(ws.keys + (static_cast<int64_t>(k) * kPipeKeySlots + bx % kPipeKeySlots) * R + i, key,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  };
  // producer, middle of step t + 1: the key atomics have completed, then
  // arrive at the block's group counter.  Vector memory operations complete
  // in issue order; the only ones this wave issued after the atomics are
  // the step's logit and Gumbel loads (kStepLoads or more of them, in the
  // next basic block), so waiting until at most kStepLoads are outstanding
  // waits for the atomics without waiting for those loads.
  auto arrive = [&](int rb) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kStepLoads) : "memory");
    if (lane == 0)
      __hip_atomic_fetch_add(dom + 256 * rb + 32 * grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  };
  // consumer, middle of step c - 2: the block's eight group counters (lanes
  // 0-7), the time-out flag (lane 8) and the caller's cancel word (lane 9)
  auto poll_issue = [&](int rb) {
    uint32_t v = 0u;
    if (lane < kBarGroups)
      v = __hip_atomic_load(dom + 256 * rb + 32 * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else if (lane == kBarGroups)
      v = __hip_atomic_load(ws.bar + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else if (lane == kBarGroups + 1 && cancel)
      v = __hip_atomic_load(cancel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return v;
  };
  // a set flag or cancel word in the polled values
  auto stopped = [&](uint32_t v) {
    return (__builtin_amdgcn_readlane(v, kBarGroups) | __builtin_amdgcn_readlane(v, kBarGroups + 1)) != 0u;
  };
  auto sum8 = [&](uint32_t v) {
    uint32_t t = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
    for (int l = 1; l < kBarGroups; ++l) t += __builtin_amdgcn_readlane(v, l);
    return t;
  };
  // consumer, start of step c - 1: every work group has arrived for the
  // block at position k - 1 (wait, bounded, only if not yet); then load the
  // block's key slots of that position.  False when the wait gave up.
  auto poll_finish = [&](int k, int rb, uint32_t pv, unsigned long long (&kr)[kHalfSlots]) {
    const uint32_t target = static_cast<uint32_t>(k) * static_cast<uint32_t>(gx);
    bool ok = false, stop = stopped(pv);
    if (!stop) {
      ok = sum8(pv) >= target;
      const unsigned long long tstart = __builtin_amdgcn_s_memrealtime();
      while (!ok) {
        const uint32_t v = poll_issue(rb);
        if (stopped(v) || __builtin_amdgcn_s_memrealtime() - tstart > kBarrierTicks) {
          stop = true;
          break;
        }
        ok = sum8(v) >= target;
      }
    }
    if (stop && lane == 0) __hip_atomic_fetch_or(ws.bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    // unconditional (requests past R read request R - 1's keys and are
    // dropped at the gather), so the wait for them can be counted exactly
    const unsigned long long* kp = ws.keys + (static_cast<int64_t>(k - 1) * kPipeKeySlots + h * kHalfSlots) * R +
                                   min(32 * rb + j, R - 1);
#pragma unroll
    for (int q = 0; q < kHalfSlots; ++q)
      kr[q] = __hip_atomic_load(kp + static_cast<int64_t>(q) * R, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return ok;
  };
  // consumer, middle of step c - 1 (the prologue, for the first two steps):
  // the block's previous tokens (the anchors at position 0), their W1 rows
  // and the block's in-chunk Gumbels, copied into the slot of step c
  auto gather_issue = [&](int k, int rb, const unsigned long long (&kr)[kHalfSlots], uint8_t* eslot,
                          float (*gslot)[kGChunk]) {
    int tok;
    if (k == 0) {
      const int i = 32 * rb + j;
      tok = i < R ? token_or_none(x0[i], V) : -1;
    } else {
      unsigned long long b = kr[0];
#pragma unroll
      for (int q = 1; q < kHalfSlots; ++q) b = kr[q] > b ? kr[q] : b;
      const unsigned long long o = xor32(b);
      b = o > b ? o : b;
      tok = 32 * rb + j < R ? token_or_none(key_token(b), V) : -1;
    }
    // copy q fills pieces 2 q and 2 q + 1 of all 32 rows: lane (h, j)
    // copies piece 2 q + h of row j, so every lane copies from its own
    // request's row
    const uint16_t* src = (tok >= 0 ? W1 + static_cast<int64_t>(tok) * (KS16 * 16) : kZeroRow) + h * 8;
#pragma unroll
    for (int q = 0; q < KS16; ++q) copy16_to_lds(src + q * 16, eslot + q * 1024);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = min(32 * rb + 16 * q + (lane >> 2), R - 1);
      copy16_to_lds(g + (static_cast<int64_t>(i) * gamma + k) * kGChunk + 4 * (lane & 3), &gslot[16 * q][0]);
    }
  };

  uint32_t pv = 0u;                          // consumer: the polled group counters
  unsigned long long kr[kHalfSlots] = {};    // consumer: the key slots read (half of them per lane)
  bool cok = true;                           // consumer: the wait did not give up

  // one step: the request block's logits plus bias for the wave's tile, the
  // fold of each lane's two chunks, and the draw inside the winning chunk;
  // the round trips of other blocks at the step's start, middle and end
  // (position, block) of steps s - 1, s + 1 and s + 2, advanced step by step
  struct Pos {
    int k, rb;
  };
  auto advance = [&](Pos p) { return p.rb + 1 == nb ? Pos{p.k + 1, 0} : Pos{p.k, p.rb + 1}; };
  const Pos last{gamma - 1, nb - 1};
  auto step = [&](int s, Pos pm1, Pos p1, Pos p2, PipeLane& cur, const uint8_t* ecur, const float (*gcur)[kGChunk],
                  unsigned long long (*mkcur)[32], float2 (*mlcur)[32], uint8_t* enxt,
                  float (*gnxt)[kGChunk], const unsigned long long (*mkprev)[32], const float2 (*mlprev)[32]) {
    const bool prod = s >= 1 && ((s - 1) & (kPipeWaves - 1)) == wave;              // producer of step s - 1
    const bool cons1 = s + 1 < s_end && s + 1 >= 2 && ((s + 1) & (kPipeWaves - 1)) == wave;   // copies for s + 1
    const bool cons2 = s + 2 < s_end && p2.k > 0 && ((s + 2) & (kPipeWaves - 1)) == wave;     // polls for s + 2
    if (prod) merge_step(pm1.k, pm1.rb, mkprev, mlprev);
    if (cons1) cok = p1.k > 0 ? poll_finish(p1.k, p1.rb, pv, kr) : true;

    f32x16 acc0, acc1;
    {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t w0 = cur.u[0][q >> 3][(q >> 1) & 3];
        const uint32_t w1 = cur.u[1][q >> 3][(q >> 1) & 3];
        acc0[q] = __uint_as_float((q & 1) ? (w0 & 0xFFFF0000u) : (w0 << 16));
        acc1[q] = __uint_as_float((q & 1) ? (w1 & 0xFFFF0000u) : (w1 << 16));
      }
    }
    const float G0 = cur.G[0], G1 = cur.G[1];
    {
      const Pos ld = s + 2 < s_end ? p2 : last;   // unconditional: no branch near the end
      load_step(cur, ld.k, ld.rb);
      const uint8_t* erow = ecur + h * (32 * 16) + j * 16;   // piece 2 ks + h of row j
      // interleave the products with the neighbouring vector work (at small
      // r the products are too few for the strategy)
      if constexpr (KS16 >= 8) __builtin_amdgcn_iglp_opt(1);
      bf16x8 bc = *reinterpret_cast<const bf16x8*>(erow);
      bf16x8 bn = KS16 > 1 ? *reinterpret_cast<const bf16x8*>(erow + 1024) : bc;
#pragma unroll
      for (int ks = 0; ks < KS16; ++ks) {
        const bf16x8 bnn = ks + 2 < KS16 ? *reinterpret_cast<const bf16x8*>(erow + (ks + 2) * 1024) : bn;
        if (ks < KR) {
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
    }

    // middle of the step
    if (prod && s - 1 + nb < s_end) arrive(pm1.rb);
    if (cons2) pv = poll_issue(p2.rb);
    if (cons1 && cok) gather_issue(p1.k, p1.rb, kr, enxt, gnxt);

    {
      LaneDraw dr;
      lane_draw_init(dr);
      f32x4 a[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = f32x4{acc0[4 * q], acc0[4 * q + 1], acc0[4 * q + 2], acc0[4 * q + 3]};
      fold_chunk(a, G0, v0 + 16 * h, dr);
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = f32x4{acc1[4 * q], acc1[4 * q + 1], acc1[4 * q + 2], acc1[4 * q + 3]};
      const bool take1 = fold_chunk(a, G1, v0 + 32 + 16 * h, dr);
      float bs = neg_inf();
      int bo = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(&gcur[j][4 * q]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = 4 * q + t;
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
        mkcur[wave][j] = key;
        mlcur[wave][j] = make_float2(M2, Ts);
      }
    }
    // end of the step: the consumer's copies have landed before anyone reads
    // the slot
    if (cons1) __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
  };

  PipeLane pa, pb;   // steps s and s + 1 in flight (nb >= 3: both at position 0)
  load_step(pa, 0, 0);
  load_step(pb, 0, 1);
  // the first two steps' W1 rows and Gumbels (position 0: the anchors)
  if (wave == 0) gather_issue(0, 0, kr, eslot0, gslot0);
  if (wave == 1) gather_issue(0, 1, kr, eslot1, gslot1);
  __builtin_amdgcn_s_waitcnt(0);   // includes the A fragments copied into LDS
  __syncthreads();

  Pos pm1{-1, nb - 1}, p0{0, 0};
  Pos p1 = advance(p0), p2 = advance(p1);
  for (int s = 0; s < s_end; s += 2) {
    step(s, pm1, p1, p2, pa, eslot0, gslot0, mkey0, mlse0, eslot1, gslot1, mkey1, mlse1);
    pm1 = p0;
    p0 = p1;
    p1 = p2;
    p2 = advance(p2);
    if (s + 1 < s_end) step(s + 1, pm1, p1, p2, pb, eslot1, gslot1, mkey1, mlse1, eslot0, gslot0, mkey0, mlse0);
    pm1 = p0;
    p0 = p1;
    p1 = p2;
    p2 = advance(p2);
  }
  // the last step's merge
  const int tl = s_end - 1;
  if ((tl & (kPipeWaves - 1)) == wave) {
    if (tl & 1)
      merge_step(last.k, last.rb, mkey1, mlse1);
    else
      merge_step(last.k, last.rb, mkey0, mlse0);
  }
}

// ------------------------------------------------------------------ host side

int compute_units();   // abi.hip

// Work groups of the launch: one per compute unit (at most one per tile and
// max_wgs), or 0 when some group would get more than kPipeMaxTiles tiles.
static int pipe_grid_x(int V, int max_wgs) {
  const int nTiles = (V + kChunk - 1) / kChunk;
  int gx = compute_units();
  if (gx > nTiles) gx = nTiles;
  if (gx > max_wgs) gx = max_wgs;
  if (gx < 1) return 0;
  return (nTiles + gx - 1) / gx <= kPipeMaxTiles ? gx : 0;
}

template <int KS16, bool VEC>
static bool pipe_fits_one() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, reinterpret_cast<const void*>(&sample_steps_pipe<KS16, VEC>), kPipeThreads, 0);
    v = (e == hipSuccess && n >= 1) ? 1 : 2;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1;
}

// Whether the per-block-barrier kernel takes a bf16 Markov-head launch of
// this shape: 3 to kPipeMaxBlocks request blocks of 32, r in {32, 64, 128,
// 256}, at most kPipeMaxTiles tiles per work group, and the work group fits
// on a compute unit.  Returns its grid width, or 0.
int pipe_grid(int R, int V, int r, int max_wgs) {
  const int nb = (R + 31) / 32;
  if (nb < kPipeMinBlocks || nb > kPipeMaxBlocks) return 0;
  const int gx = pipe_grid_x(V, max_wgs);
  if (gx == 0) return 0;
  const bool vec = (V % kGChunk) == 0;
  bool fits = false;
  switch (r) {
    case 32: fits = vec ? pipe_fits_one<2, true>() : pipe_fits_one<2, false>(); break;
    case 64: fits = vec ? pipe_fits_one<4, true>() : pipe_fits_one<4, false>(); break;
    case 128: fits = vec ? pipe_fits_one<8, true>() : pipe_fits_one<8, false>(); break;
    case 256: fits = vec ? pipe_fits_one<16, true>() : pipe_fits_one<16, false>(); break;
    default: break;
  }
  return fits ? gx : 0;
}

template <int KS16, bool VEC>
static void launch_pipe(int R, int gamma, int V, const void* U, const void* W1, const void* W2t, const int32_t* x0,
                        const float* G, const float* g, const SampleWs& w, int gx, const uint32_t* cancel,
                        hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
  hipExtLaunchKernelGGL((sample_steps_pipe<KS16, VEC>), dim3(gx), dim3(kPipeThreads), 0, s, ev0, ev1, 0, R, gamma, V,
                        static_cast<const uint16_t*>(U), static_cast<const uint16_t*>(W1),
                        static_cast<const uint16_t*>(W2t), x0, G, g, w, cancel);
}

// Launches all gamma positions (the caller checked pipe_grid).
hipError_t pipe_launch(int R, int gamma, int V, int r, const void* U, const void* W1, const void* W2t,
                       const int32_t* x0, const float* G, const float* g, const SampleWs& w, int gx,
                       const uint32_t* cancel, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
  const bool vec = (V % kGChunk) == 0;
#define DSPARK_PIPE(KS)                                                                      \
  (vec ? launch_pipe<KS, true>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, cancel, ev0, ev1, s) \
       : launch_pipe<KS, false>(R, gamma, V, U, W1, W2t, x0, G, g, w, gx, cancel, ev0, ev1, s))
  switch (r) {
    case 32: DSPARK_PIPE(2); break;
    case 64: DSPARK_PIPE(4); break;
    case 128: DSPARK_PIPE(8); break;
    default: DSPARK_PIPE(16); break;
  }
#undef DSPARK_PIPE
  return hipGetLastError();
}

}  // namespace dspark
