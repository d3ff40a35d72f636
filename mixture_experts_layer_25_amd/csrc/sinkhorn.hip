// Sinkhorn routing: the per-expert selection bias of the balanced router.
//
// Megatron-LM part 6, load-balancing table, row sinkhorn: Sinkhorn
// iterations rescale the routing matrix until it is doubly stochastic, which
// evens out the expert load without an auxiliary loss.  The matrix is
// exp(l) [T,E]; one iteration scales every row to sum 1 and then every
// column to sum T/E.  Only the product col[e] of the column factors matters
// for the selection: within row t the balanced matrix ranks experts as
// l[t,e] + ln col[e] (the row factor is common).  This file computes
// bias[e] = ln col[e] after n iterations; the top-k kernel then takes it as
// a selection-only bias, so the gates still come from the logits.
//
// Log domain, with b = ln col (b = 0 before the first iteration):
//   rho[t] = -LSE_e(l[t,e] + b[e])              row scaling
//   b[e]   = ln(T/E) - LSE_t(l[t,e] + rho[t])   column scaling
// where LSE is log-sum-exp taken as a (max, sum of exp(v - max)) pair, so no
// exponent is positive whatever the logits.
//
// One launch per iteration.  Block j owns a contiguous range of tokens: it
// computes rho for them and writes, for every column, the (max, sum) pair
// over its tokens.  The next launch starts by merging the B pairs of every
// column, all threads of the block at once and in a fixed order, so every
// block gets the same b, bit for bit.  A last one-block launch merges the
// final pairs into bias[e] the same way.  Inside a block a token is
// handled by a segment of G lanes (G = the next power of two >= E, at most
// 64; lane s holds experts s, s+G, ...), as in the top-k kernel; the loads
// of several tokens go out before any is used; segment partials are merged
// by a butterfly over the wave, then across the 16 waves in wave order.
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kSkThreads = 1024;
constexpr int kSkWaves = kSkThreads / kWave;

// (m, s) <- the pair of the union: max and the sum of exp(v - max).
// Symmetric in its two arguments (fp32 addition commutes).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;   // both empty
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}

// (m, s) <- the pair with one more value v.
__device__ __forceinline__ void lse_add(float& m, float& s, float v) {
  if (v > m) {
    s = s * expf(m - v) + 1.f;
    m = v;
  } else {
    s += expf(v - m);
  }
}

// out[e] = ln_cols - LSE of column e, from the B pairs per column in part
// [B][E].  Every thread of the block takes part: columns go to groups of
// tpc consecutive lanes (tpc = 1024 / the next power of two >= E, between 1
// and 64); lane r of a group merges pairs r, r + tpc, ... eight loads at a
// time, then the group merges by a butterfly.  The order is fixed, so every
// block and the finishing launch get the same values, bit for bit.
__device__ void merge_columns(const float2* __restrict__ part, int B, int E, float ln_cols,
                              float* __restrict__ out) {
  int ep = 1;
  while (ep < E) ep <<= 1;
  int tpc = kSkThreads / ep;
  tpc = tpc < 1 ? 1 : (tpc > kWave ? kWave : tpc);
  const int cpp = kSkThreads / tpc;                 // columns per pass
  const int r = threadIdx.x % tpc;
  for (int c0 = 0; c0 < E; c0 += cpp) {             // uniform over the block
    const int e = c0 + threadIdx.x / tpc;
    float m = -INFINITY, s = 0.f;
    if (e < E) {
      int j = r;
      for (; j + 7 * tpc < B; j += 8 * tpc) {
        float2 p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) p[u] = part[(int64_t)(j + u * tpc) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) lse_merge(m, s, p[u].x, p[u].y);
      }
      for (; j < B; j += tpc) {
        const float2 p = part[(int64_t)j * E + e];
        lse_merge(m, s, p.x, p.y);
      }
    }
    for (int msk = 1; msk < tpc; msk <<= 1) {
      const float om = __shfl_xor(m, msk);
      const float os = __shfl_xor(s, msk);
      lse_merge(m, s, om, os);
    }
    if (e < E && r == 0) out[e] = ln_cols - (m + logf(s));
  }
}

template <int G, int NPL>
__global__ __launch_bounds__(kSkThreads) void sinkhorn_step_kernel(
    const float* __restrict__ logits, const float2* __restrict__ prev, float2* __restrict__ part,
    int64_t T, int E, int64_t tpb, float ln_cols) {
  constexpr int kSegs = kWave / G;            // tokens per wave at a time
  constexpr int U = NPL >= 8 ? 2 : 4;         // token steps whose loads go out together
  // b [E] floats, then the waves' column pairs [kSkWaves][E] float2
  extern __shared__ float sk_lds[];
  float* b = sk_lds;
  float2* wpart = reinterpret_cast<float2*>(sk_lds + ((E + 1) & ~1));
  const int tid = threadIdx.x;
  if (prev) {
    merge_columns(prev, gridDim.x, E, ln_cols, b);
  } else {
    for (int e = tid; e < E; e += kSkThreads) b[e] = 0.f;
  }
  __syncthreads();

  const int lane = tid % kWave, wave = tid / kWave;
  const int seg = lane / G, s = lane % G;
  float cm[NPL], cs[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    cm[i] = -INFINITY;
    cs[i] = 0.f;
  }
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  const int64_t t1 = t0 + tpb < T ? t0 + tpb : T;
  constexpr int kStep = kSkWaves * kSegs;
  // the loop bound depends on the wave only, so segments stay converged
  for (int64_t base = t0 + (int64_t)wave * kSegs; base < t1; base += U * kStep) {
    float lv[U][NPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = base + u * kStep + seg;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = s + G * i;
        lv[u][i] = (t < t1 && e < E) ? logits[t * E + e] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = base + u * kStep + seg < t1;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = s + G * i;
        if (valid && e < E) mx = fmaxf(mx, lv[u][i] + b[e]);
      }
      mx = seg_max_f32<G>(mx);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = s + G * i;
        if (valid && e < E) sum += expf(lv[u][i] + b[e] - mx);
      }
      sum = seg_sum_f32<G>(sum);
      const float rho = -(mx + logf(sum));
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = s + G * i;
        if (valid && e < E) lse_add(cm[i], cs[i], lv[u][i] + rho);
      }
    }
  }
  // segments of the wave -> one pair per column (lanes of a column agree)
#pragma unroll
  for (int m = G; m < kWave; m <<= 1) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const float om = __shfl_xor(cm[i], m);
      const float os = __shfl_xor(cs[i], m);
      lse_merge(cm[i], cs[i], om, os);
    }
  }
  if (seg == 0) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = s + G * i;
      if (e < E) wpart[wave * E + e] = float2{cm[i], cs[i]};
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kSkThreads) {
    float m = -INFINITY, sm = 0.f;
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) lse_merge(m, sm, wpart[w * E + e].x, wpart[w * E + e].y);
    part[(int64_t)blockIdx.x * E + e] = float2{m, sm};
  }
}

__global__ __launch_bounds__(kSkThreads) void sinkhorn_finish_kernel(
    const float2* __restrict__ part, int B, int E, float ln_cols, float* __restrict__ bias) {
  merge_columns(part, B, E, ln_cols, bias);
}

template <int G, int NPL>
hipError_t launch_steps(const float* logits, int64_t T, int E, int iters, float2* parts,
                        float* bias, hipStream_t st) {
  const int B = sinkhorn_blocks(T, E);
  const int64_t tpb = (T + B - 1) / B;
  const float ln_cols = (float)log((double)T / (double)E);
  float2* buf[2] = {parts, parts + (int64_t)B * E};
  const size_t lds = (size_t)((E + 1) & ~1) * 4 + (size_t)kSkWaves * E * 8;   // <= 132 KiB
  for (int it = 0; it < iters; ++it) {
    MOE_LAUNCH((sinkhorn_step_kernel<G, NPL>), dim3(B), dim3(kSkThreads), lds, st, logits,
                       it ? (const float2*)buf[(it - 1) & 1] : nullptr, buf[it & 1], T, E, tpb,
                       ln_cols);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  MOE_LAUNCH(sinkhorn_finish_kernel, dim3(1), dim3(kSkThreads), 0, st,
                     (const float2*)buf[(iters - 1) & 1], B, E, ln_cols, bias);
  return hipGetLastError();
}

}  // namespace

int sinkhorn_blocks(int64_t T, int E) {
  // at least 16 tokens a block, at most 256 blocks, and B*E <= 2^13 pairs so
  // that each of a block's 1024 threads merges at most 8 of them (one round
  // of loads)
  int64_t cap = (int64_t)(8192 / E);
  if (cap > 256) cap = 256;
  int64_t B = (T + 15) / 16;
  if (B > cap) B = cap;
  return B < 1 ? 1 : (int)B;
}

hipError_t launch_sinkhorn(const float* logits, int64_t T, int E, int iters, float2* parts,
                           float* bias, hipStream_t s) {
  if (E <= 8) return launch_steps<8, 1>(logits, T, E, iters, parts, bias, s);
  if (E <= 16) return launch_steps<16, 1>(logits, T, E, iters, parts, bias, s);
  if (E <= 32) return launch_steps<32, 1>(logits, T, E, iters, parts, bias, s);
  if (E <= 64) return launch_steps<64, 1>(logits, T, E, iters, parts, bias, s);
  if (E <= 128) return launch_steps<64, 2>(logits, T, E, iters, parts, bias, s);
  if (E <= 256) return launch_steps<64, 4>(logits, T, E, iters, parts, bias, s);
  if (E <= 512) return launch_steps<64, 8>(logits, T, E, iters, parts, bias, s);
  return launch_steps<64, 16>(logits, T, E, iters, parts, bias, s);
}

}  // namespace moe
