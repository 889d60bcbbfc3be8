// The RNN head's recurrent step (DSpark reading notes, "implementation two:
// the RNN head", eq (6)): for every request,
//   z = [s_{k-1}; W1[x_{k-1}]; h_k],  y = W z  (W = [W_g; W_c; W_o]),
//   s_k = sigma(y_g) * s_{k-1} + (1 - sigma(y_g)) * tanh(y_c),  o_k = tanh(y_o),
// with s_{-1} = 0.  o_k is the r-vector the sampler's bias product takes in
// W1[x_{k-1}]'s place.  The previous token comes from the sampler's argmax
// keys of position k - 1 (the anchor at k = 0).
//
// bf16 storage: the projection runs on the matrix cores (32x32x16 MFMA,
// fp32 accumulation) with z in bf16 -- its state part rounded from fp32 to
// nearest, ties to even -- split along the inner dimension over kRnnSplits
// work groups; a second kernel adds the partials in order and applies the
// gates in fp32.  fp32 storage: one thread per output with fp32 FMAs.
#include "bias_tile.hpp"
#include "wide_tile.hpp"
#include "rnn_head.hpp"
#include "sample_keys.hpp"

namespace dspark {

typedef float f32x16_r __attribute__((ext_vector_type(16)));

constexpr int kRnnThreads = 256;   // four waves split each work group's inner range

// Round-to-nearest-even of an fp32 value to its bf16 bit pattern.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Work group (jb, ib, sp): columns 32 jb .. 32 jb + 31 of each of the three
// parts (gate, candidate, output), requests 32 ib .. 32 ib + 31, inner steps
// of 16 in [sp * per, (sp + 1) * per), dealt out over the four waves.  Lane
// (hh, j) brings weight row 32 jb + j of each part (the A operands) and z of
// request 32 ib + j (the B operand), eight inner indices each.
__global__ __launch_bounds__(kRnnThreads) void rnn_proj_bf16(int R, int gamma, int V, int r, int d, int k,
                                                             const uint16_t* __restrict__ W,
                                                             const uint16_t* __restrict__ h,
                                                             const uint16_t* __restrict__ W1,
                                                             const int32_t* __restrict__ x0,
                                                             const unsigned long long* __restrict__ keys,
                                                             const float* __restrict__ s, float* __restrict__ part,
                                                             int per) {
  __shared__ float red[3][kRnnThreads / kWave][16][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int j = lane & 31;
  const int hh = lane >> 5;
  const int jb = blockIdx.x, ib = blockIdx.y, sp = blockIdx.z;
  const int K = 2 * r + d;
  const int i = ib * 32 + j;
  const int ic = min(i, R - 1);
  const int st1 = min(K / 16, (sp + 1) * per);
  const int prev = previous_token(keys, kKeySlots, x0, R, V, k, ic);
  const float* srow = s + (static_cast<int64_t>(ic) * gamma + (k > 0 ? k - 1 : 0)) * r;   // read when k > 0
  const uint16_t* erow = prev >= 0 ? W1 + static_cast<int64_t>(prev) * r : kZeroRow;
  const uint16_t* hrow = h + (static_cast<int64_t>(ic) * gamma + k) * d;
  const uint16_t* wrow[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) wrow[g] = W + static_cast<int64_t>(g * r + jb * 32 + j) * K;
  f32x16_r acc[3] = {};
  constexpr int kW = kRnnThreads / kWave;   // waves; the wave takes every kW-th step of the range
  constexpr int kU = 4;                     // steps whose operands are in flight together
  // the wave's steps of [lo, hi) within this work group's range, kU at a time:
  // every load of a batch is issued before its products; a step past the
  // range reloads a valid one and multiplies a zero B operand
  auto run = [&](int lo, int hi, auto&& zfrag) {
    lo = max(lo, sp * per);
    hi = min(hi, st1);
    int st = sp * per + wave;
    if (st < lo) st += ceil_div(lo - st, kW) * kW;
    for (; st < hi; st += kU * kW) {
      bf16x8 a[kU][3], bz[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int su = st + u * kW < hi ? st + u * kW : st;
        const int kk = su * 16 + 8 * hh;
        bz[u] = zfrag(kk);
#pragma unroll
        for (int g = 0; g < 3; ++g) a[u][g] = load_bf16x8_global(wrow[g] + kk);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const bf16x8 bu = st + u * kW < hi ? bz[u] : bf16x8{};
#pragma unroll
        for (int g = 0; g < 3; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u][g], bu, acc[g], 0, 0, 0);
      }
    }
  };
  // the hidden state first, then z's state part (zero at the first
  // position; rounded from fp32 to bf16), then the previous token's W1 row
  // (a row of zeros when there is none), whose address waits on the keys
  run(2 * r / 16, K / 16, [&](int kk) { return load_bf16x8_global(hrow + kk - 2 * r); });
  if (k > 0)
    run(0, r / 16, [&](int kk) {
      const float4 lo = *reinterpret_cast<const float4*>(srow + kk);
      const float4 hi = *reinterpret_cast<const float4*>(srow + kk + 4);
      const uint32_t w0 = bf16_bits_rne(lo.x) | (bf16_bits_rne(lo.y) << 16);
      const uint32_t w1 = bf16_bits_rne(lo.z) | (bf16_bits_rne(lo.w) << 16);
      const uint32_t w2 = bf16_bits_rne(hi.x) | (bf16_bits_rne(hi.y) << 16);
      const uint32_t w3 = bf16_bits_rne(hi.z) | (bf16_bits_rne(hi.w) << 16);
      return __builtin_bit_cast(bf16x8, (uint4{w0, w1, w2, w3}));
    });
  run(r / 16, 2 * r / 16, [&](int kk) { return load_bf16x8_global(erow + kk - r); });
#pragma unroll
  for (int g = 0; g < 3; ++g)
#pragma unroll
    for (int q = 0; q < 16; ++q) red[g][wave][q][lane] = acc[g][q];
  __syncthreads();
  // output element (g, q, lane): part row 32 jb + 8 (q / 4) + 4 (lane / 32) + q % 4 of part g, request
  // 32 ib + lane % 32
  for (int e = threadIdx.x; e < 3 * 16 * kWave; e += kRnnThreads) {
    const int g = e / (16 * kWave), q = (e / kWave) % 16, l = e % kWave;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kRnnThreads / kWave; ++w) t += red[g][w][q][l];
    const int req = ib * 32 + (l & 31);
    const int col = jb * 32 + 8 * (q >> 2) + 4 * (l >> 5) + (q & 3);
    if (req < R) part[(static_cast<int64_t>(sp) * R + req) * 3 * r + g * r + col] = t;
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

hipError_t rnn_step_launch(dspark_dtype dt, const RnnHead& hd, int R, int gamma, int V, int r, int k,
                           const void* W1, const int32_t* x0, const unsigned long long* keys, hipStream_t s) {
  const int K = 2 * r + hd.d;
  const int nthreads = ceil_div(static_cast<int64_t>(R) * r, 256);
  if (dt == DSPARK_BF16) {
    const int per = ceil_div(K / 16, kRnnSplits);
    hipLaunchKernelGGL(rnn_proj_bf16, dim3(r / 32, ceil_div(R, 32), kRnnSplits), dim3(kRnnThreads), 0, s, R, gamma,
                       V, r, hd.d, k, static_cast<const uint16_t*>(hd.W), static_cast<const uint16_t*>(hd.h),
                       static_cast<const uint16_t*>(W1), x0, keys, hd.s, hd.part, per);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(rnn_gate<BF16>, dim3(nthreads), dim3(256), 0, s, R, gamma, r, k, kRnnSplits, hd.part, hd.s,
                       static_cast<uint16_t*>(hd.o));
  } else {
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

size_t rnn_workspace_bytes(int R, int r) {
  return (sizeof(float) * static_cast<size_t>(kRnnSplits) * R * 3 * r + 255) & ~static_cast<size_t>(255);
}

}  // namespace dspark
