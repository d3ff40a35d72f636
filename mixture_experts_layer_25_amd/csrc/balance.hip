// Load-balance statistics of a routing.
//
// infra-l7, "NVIDIA 原题" notes on the load balancing loss: Switch
// Transformer adds alpha*E*sum_i f_i*P_i, f_i the share of tokens sent to
// expert i and P_i the router's mean probability for i, smallest when the
// load is even.  Megatron-LM part 6, "负载均衡": the aux loss penalises the
// gap between where tokens go and how likely the router makes each expert.
//
//   probsum  (also writes the distribution itself for expert-choice
//            routing) a workgroup covers the same token group as a top-k workgroup
//            (4 passes of 256/G tokens, G lanes per token): each token's
//            distribution over all E experts (softmax of the logits, or the
//            sigmoids normalised over E), summed per expert in a fixed
//            order (tokens of a pass in order, passes in order);
//   final    one workgroup: per expert the group sums in group order (in
//            parallel slices, combined in slice order), f = counts/(T*k),
//            P = sum/T, loss = alpha*E*sum f*P by a fixed tree.
// Every sum has a fixed order, so the results are the same on every run.
//
// The aux-loss-free selection-bias step moves each expert's bias one fixed
// step against its load (below).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

// partial (the group sums) and probs_et (the distribution itself, [E,T])
// are each optional.
template <int G, int NPL>
__global__ __launch_bounds__(256) void probsum_kernel(const float* __restrict__ logits,
                                                      int gate_mode, int64_t T, int E,
                                                      float* __restrict__ partial,
                                                      float* __restrict__ probs_et) {
  constexpr int kTokPerPass = 256 / G;
  constexpr int kPasses = 4;
  constexpr int kTok = kPasses * kTokPerPass;
  __shared__ float pl[kTokPerPass][G * NPL];   // one pass's probabilities
  __shared__ float acc[1024];

  const int tid = threadIdx.x;
  const int seg = tid / G;           // token slot within a pass
  const int s = tid % G;             // lane within the segment
  for (int e = tid; e < E; e += 256) acc[e] = 0.f;

  for (int pass = 0; pass < kPasses; ++pass) {
    const int64_t t = (int64_t)blockIdx.x * kTok + pass * kTokPerPass + seg;
    const bool valid = t < T;
    float v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = s + G * i;
      v[i] = (valid && e < E) ? logits[t * E + e] : -INFINITY;
    }
    float p[NPL];
    if (gate_mode == 2) {             // sigmoids normalised over all E
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        v[i] = (s + G * i < E && valid) ? 1.f / (1.f + expf(-v[i])) : 0.f;
        part += v[i];
      }
      const float den = seg_sum_f32<G>(part);
#pragma unroll
      for (int i = 0; i < NPL; ++i) p[i] = valid ? v[i] / den : 0.f;
    } else {                          // softmax over all E
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPL; ++i) m = fmaxf(m, v[i]);
      m = seg_max_f32<G>(m);
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        v[i] = (s + G * i < E && valid) ? expf(v[i] - m) : 0.f;
        part += v[i];
      }
      const float den = seg_sum_f32<G>(part);
#pragma unroll
      for (int i = 0; i < NPL; ++i) p[i] = valid ? v[i] / den : 0.f;
    }
    if (probs_et && valid) {
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (s + G * i < E) probs_et[(int64_t)(s + G * i) * T + t] = p[i];
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) pl[seg][s + G * i] = p[i];
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      float a = acc[e];
#pragma unroll
      for (int q = 0; q < kTokPerPass; ++q) a += pl[q][e];
      acc[e] = a;
    }
    __syncthreads();
  }
  if (partial)
    for (int e = tid; e < E; e += 256) partial[blockIdx.x * (int64_t)E + e] = acc[e];
}

template <int G, int NPL>
void launch_probsum_t(const float* logits, int gate, int64_t T, int E, float* partial,
                      float* probs_et, hipStream_t st) {
  const int64_t nwg = (T + 4 * (256 / G) - 1) / (4 * (256 / G));
  MOE_LAUNCH((probsum_kernel<G, NPL>), dim3((unsigned)nwg), dim3(256), 0, st, logits,
                     gate, T, E, partial, probs_et);
}

void launch_probsum(const float* logits, int gate, int64_t T, int E, float* partial,
                    float* probs_et, hipStream_t st) {
  const int G = seg_lanes(E);
  if (G == 8)
    launch_probsum_t<8, 1>(logits, gate, T, E, partial, probs_et, st);
  else if (G == 16)
    launch_probsum_t<16, 1>(logits, gate, T, E, partial, probs_et, st);
  else if (G == 32)
    launch_probsum_t<32, 1>(logits, gate, T, E, partial, probs_et, st);
  else if (E <= 64)
    launch_probsum_t<64, 1>(logits, gate, T, E, partial, probs_et, st);
  else if (E <= 128)
    launch_probsum_t<64, 2>(logits, gate, T, E, partial, probs_et, st);
  else if (E <= 256)
    launch_probsum_t<64, 4>(logits, gate, T, E, partial, probs_et, st);
  else if (E <= 512)
    launch_probsum_t<64, 8>(logits, gate, T, E, partial, probs_et, st);
  else
    launch_probsum_t<64, 16>(logits, gate, T, E, partial, probs_et, st);
}

// One workgroup of 1024 threads.  Thread (sl, e) = (tid / E, tid % E) sums
// the sl-th of S contiguous slices of the groups of expert e.
__global__ __launch_bounds__(1024) void balance_final_kernel(
    const float* __restrict__ partial, int64_t ngroups, const int32_t* __restrict__ counts,
    int64_t T, int E, int k, float alpha, float* __restrict__ f_out,
    float* __restrict__ P_out, float* __restrict__ loss_out) {
  __shared__ float slice_sum[1024];
  __shared__ float red[1024];
  int S = 1;
  while (2 * S * E <= 1024) S *= 2;
  const int tid = threadIdx.x;
  const int sl = tid / E, es = tid % E;
  if (sl < S) {
    const int64_t L = (ngroups + S - 1) / S;
    const int64_t g0 = sl * L, g1 = min(ngroups, g0 + L);
    float sum = 0.f;
    int64_t g = g0;
    for (; g + 8 <= g1; g += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = partial[(g + i) * E + es];
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[i];
    }
    for (; g < g1; ++g) sum += partial[g * E + es];
    slice_sum[tid] = sum;
  }
  __syncthreads();
  const int e = tid;
  float fp = 0.f;
  if (e < E) {
    float sum = 0.f;
    for (int q = 0; q < S; ++q) sum += slice_sum[q * E + e];
    const float P = sum / (float)T;
    const float f = (float)counts[e] / (float)(T * k);
    f_out[e] = f;
    P_out[e] = P;
    fp = f * P;
  }
  red[tid] = fp;
  for (int w = 512; w > 0; w >>= 1) {
    __syncthreads();
    if (tid < w) red[tid] += red[tid + w];
  }
  if (tid == 0) loss_out[0] = alpha * (float)E * red[0];
}

// One aux-loss-free balancing step (DeepSeek-V3 in the same notes: a
// per-expert bias that enters only the top-k selection).  Expert e's load is
// compared with the mean T*k/E in exact integers (T*k against E*count): an
// over-loaded expert's bias drops by gamma, an under-loaded one's rises by
// gamma, one at the mean is left untouched.  One thread per expert.
__global__ __launch_bounds__(256) void select_bias_update_kernel(const int32_t* __restrict__ counts,
                                                                 int64_t T, int E, int k,
                                                                 float gamma,
                                                                 float* __restrict__ bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t under = T * k - (int64_t)E * counts[e];
  if (under > 0)
    bias[e] = bias[e] + gamma;
  else if (under < 0)
    bias[e] = bias[e] - gamma;
}

}  // namespace

hipError_t launch_select_bias_update(const int32_t* counts, int64_t T, int E, int k, float gamma,
                                     float* bias, hipStream_t st) {
  MOE_LAUNCH(select_bias_update_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0,
                     st, counts, T, E, k, gamma, bias);
  return hipGetLastError();
}

hipError_t launch_load_balance(const float* logits, const int32_t* counts, int gate, int64_t T,
                               int E, int k, float alpha, float* partial, float* f, float* P,
                               float* loss, hipStream_t st) {
  launch_probsum(logits, gate, T, E, partial, nullptr, st);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t ngroups = (T + topk_tokens_per_wg(E) - 1) / topk_tokens_per_wg(E);
  MOE_LAUNCH(balance_final_kernel, dim3(1), dim3(1024), 0, st, partial, ngroups, counts,
                     T, E, k, alpha, f, P, loss);
  return hipGetLastError();
}

hipError_t launch_router_probs(const float* logits, int gate, int64_t T, int E, float* probs_et,
                               hipStream_t st) {
  launch_probsum(logits, gate, T, E, nullptr, probs_et, st);
  return hipGetLastError();
}

}  // namespace moe
