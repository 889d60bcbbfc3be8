// Pieces shared by the sampling kernels: the workspace layout (argmax key
// slots, grid-barrier words, log-sum-exp partials), the grid barrier's time
// bound and the per-lane fold of one 16-token Gumbel chunk.
#pragma once

#include "common.hpp"
#include "sample_keys.hpp"

namespace dspark {

struct SampleWs {
  unsigned long long* keys;   // [gamma][slots][R]
  unsigned int* bar;          // barrier words (below)
  float2* lsep;               // [gamma][R][nPart]  (M, S) log-sum-exp partials
  int slots;                  // argmax key slots per (position, request)
};

// Barrier words (32-bit), cleared on every call: bar[0] is the top counter
// of the persistent kernel's grid barrier and bar[1] its time-out flag; the
// group counters sit at bar[64 + 32 g], 128 bytes apart.
constexpr int kBarGroups = 8;              // arrival groups of the two-level barrier
// The per-block barriers of sample_steps_pipe: block d's group counter g at
// bar[kPipeBarBase + 256 d + 32 g], for at most kPipeMaxBlocks blocks of 32
// requests.
constexpr int kPipeBarBase = 512;
constexpr int kPipeMaxBlocks = 32;
constexpr int kBarWords = (kPipeBarBase + 256 * kPipeMaxBlocks) / 2;   // as 64-bit words

// The wait at a grid barrier is bounded: after this many ticks of the 100 MHz
// real-time clock a work group gives up (0.5 s).
constexpr unsigned long long kBarrierTicks = 50000000ull;

// The confidence head's inputs when a sampling call computes it too (h null:
// not asked for).
struct SampleConf {
  const void* h;   // [R][gamma][d]
  const void* w;   // [d + r]
  int d;
  const float* T;  // [gamma] or null
  float* c;        // [R][gamma]
  float* z;        // [R][gamma] or null
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// A 16-byte copy from global memory straight into LDS: lane l writes
// dst + 16 l (dst the same for the whole wave).
__device__ __forceinline__ void copy16_to_lds(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
}

// Token offset (within a 64-token tile) of the 32x32x16 A-operand row `row`
// (0..63) of the sampling kernels: the rows are permuted so that a lane's
// sixteen accumulators are sixteen consecutive tokens (one Gumbel chunk);
// the inverse of row32_of_token.
__host__ __device__ constexpr int token_of_row32(int row) {
  return (row & 32) | (((row >> 2) & 1) << 4) | (((row >> 3) & 3) << 2) | (row & 3);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
// score of -inf and add nothing: their base is a finite stand-in far below
// any logit (kEmptyBase), so merging them never lifts the running maximum
// (which would flush the real partial sum to zero for very negative logits)
// and never forms -inf - (-inf).
constexpr float kEmptyBase = -1e30f;
__device__ __forceinline__ bool fold_chunk(const f32x4 (&acc)[4], float G, int first, LaneDraw& d) {
  float l[kGChunk];
#pragma unroll
  for (int c = 0; c < kGChunk; ++c) l[c] = acc[c >> 2][c & 3];
  float m = l[0];
#pragma unroll
  for (int c = 1; c < kGChunk; ++c) m = fmaxf(m, l[c]);
  const float m2 = m == neg_inf() ? kEmptyBase : m * kLog2e;
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

// Grid-wide barrier between positions of the persistent kernel: every work
// group of the launch is resident (one per compute unit, at most as many as
// the device has), so a counter of arrivals suffices.  The key slots and the
// counter are updated with system-scope atomics, which are performed in
// memory rather than in the issuing die's L2, so no cache write-back is
// needed to publish them; each wave waits for its own atomics to complete
// before the work group arrives.  The wait is bounded: after kBarrierTicks of
// the 100 MHz real-time clock the work group raises the time-out flag and
// the launch ends early (sample_finalize then reports every token as -1 and
// the call's status word, if any, as DSPARK_ETIMEOUT), so a grid that is not
// resident as a whole cannot hang.  A caller's cancel word, when given and
// non-zero, ends the wait the same way.

__device__ __forceinline__ bool grid_barrier(unsigned int* bar, unsigned int round, int* flag,
                                             const uint32_t* cancel) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's key atomics have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    // two levels: work group b arrives at group counter b mod kBarGroups; the
    // last arrival of a group arrives at the top counter, which everyone polls
    const unsigned int nWG = gridDim.x * gridDim.y;
    const unsigned int id = blockIdx.y * gridDim.x + blockIdx.x;
    const unsigned int groups = nWG < kBarGroups ? nWG : kBarGroups;
    const unsigned int grp = id % groups;
    const unsigned int per = (nWG - grp + groups - 1) / groups;
    const unsigned int old =
        __hip_atomic_fetch_add(bar + 64 + 32 * grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (old + 1 == round * per) __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    int ok = 1;
    while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) < round * groups) {
      if (__hip_atomic_load(bar + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0u ||
          __builtin_amdgcn_s_memrealtime() - t0 > kBarrierTicks ||
          (cancel && __hip_atomic_load(cancel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0u)) {
        __hip_atomic_fetch_or(bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        ok = 0;
        break;
      }
      // no sleep between polls: the next load goes out as soon as this one
      // returns (a sleep of one measured about 2 % slower per launch)
    }
    *flag = ok;
  }
  __syncthreads();
  return *flag != 0;
}

}  // namespace dspark
