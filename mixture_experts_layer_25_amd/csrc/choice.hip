// Routing variants: a per-expert top-C selection shared by expert-choice
// routing and by the score-priority capacity drop.
//
// 10.5 序列并行与专家并行, section 10.5.6: expert-choice routing turns the
// direction round, every expert taking the fixed number of tokens that
// score highest for it.  专家并行 page, "EP+TP+DP": MoE theory drops the
// lower-priority tokens by their gate score.
//
// Candidates of expert e are ranked by a 64-bit key: the ordered bits of
// the fp32 score above ~position, so a larger score wins and equal scores
// go to the earlier candidate (token order).  One workgroup (1024 threads)
// per expert:
//   radix select  8 passes of 8 bits: a 256-bin histogram of the next
//                 digit among the candidates that match the prefix found
//                 so far (per-wave LDS histograms; counts do not depend on
//                 the order of the atomics), a suffix scan over the bins
//                 picks the digit of the C-th largest key;
//   compaction    candidates in order, selected iff key >= that key; a
//                 block scan gives each its row e*C + rank.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ uint64_t sel_key(float score, uint32_t pos) {
  return ((uint64_t)ordered_bits(score) << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}

constexpr int kSelThreads = 1024;            // 16 waves per expert
constexpr int kSelWaves = kSelThreads / 64;

// Exclusive scan over the kSelThreads threads of a workgroup; `tmp` holds
// kSelWaves + 1 ints.  Returns the prefix and the total in *tot.
__device__ int block_exclusive_scan_sel(int v, int* tmp, int* tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < kSelWaves; ++i) {
      const int c = tmp[i];
      tmp[i] = run;
      run += c;
    }
    tmp[kSelWaves] = run;
  }
  __syncthreads();
  const int res = tmp[w] + incl - v;
  *tot = tmp[kSelWaves];
  __syncthreads();
  return res;
}

// Key of candidate i of expert e: expert choice reads the score row
// probs_et[e][*] (position = token), the score drop reads the precomputed
// keys of the expert's assignments in token order.
struct CandEC {
  const float* p;   // probs_et + e*T
  __device__ uint64_t key(int64_t i) const { return sel_key(p[i], (uint32_t)i); }
};
struct CandSD {
  const uint64_t* k;   // key_dl + offsets_dl[e]
  __device__ uint64_t key(int64_t i) const { return k[i]; }
};

// Key of the C-th largest of the n candidates (n > C >= 1).  Each wave
// counts into its own histogram (scores that share their top bits would
// otherwise pile LDS atomics onto one bin); four keys are loaded per
// thread before their digits are counted.
template <class Cand>
__device__ uint64_t topc_threshold(const Cand& cand, int64_t n, int C) {
  __shared__ int hist[kSelWaves][256];
  __shared__ int tmp[kSelWaves + 1];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_rem;
  const int tid = threadIdx.x, w = tid >> 6;
  uint64_t prefix = 0, mask = 0;
  int rem = C;
  if (tid == 0) {
    s_prefix = 0;
    s_rem = C;
  }
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int q = tid; q < kSelWaves * 256; q += kSelThreads) (&hist[0][0])[q] = 0;
    __syncthreads();
    for (int64_t i0 = tid; i0 < n; i0 += 4 * kSelThreads) {
      uint64_t key[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * kSelThreads;
        key[u] = i < n ? cand.key(i) : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * kSelThreads < n && (key[u] & mask) == prefix)
          atomicAdd(&hist[w][(key[u] >> shift) & 255], 1);
    }
    __syncthreads();
    // thread b < 256 owns digit 255 - b, so the exclusive scan counts the
    // keys with a larger digit
    const int d = 255 - tid;
    int cnt = 0;
    if (tid < 256)
      for (int ww = 0; ww < kSelWaves; ++ww) cnt += hist[ww][d];
    int tot;
    const int above = block_exclusive_scan_sel(cnt, tmp, &tot);
    if (tid < 256 && cnt > 0 && above < rem && rem <= above + cnt) {
      s_prefix = prefix | ((uint64_t)d << shift);
      s_rem = rem - above;
    }
    __syncthreads();
    prefix = s_prefix;
    rem = s_rem;
    mask |= (uint64_t)0xFF << shift;
  }
  return prefix;
}

// Expert choice: expert e = blockIdx.x picks its C tokens.
__global__ __launch_bounds__(kSelThreads) void expert_choice_kernel(
    const float* __restrict__ probs_et, int64_t T, int E, int C,
    int32_t* __restrict__ sel_row, float* __restrict__ gate_te, int32_t* __restrict__ row_token) {
  __shared__ int tmp[kSelWaves + 1];
  const int e = blockIdx.x;
  const CandEC cand{probs_et + (int64_t)e * T};
  const uint64_t thr = (T > C) ? topc_threshold(cand, T, C) : 0;
  int base = 0;
  for (int64_t i0 = 0; i0 < T; i0 += kSelThreads) {
    const int64_t t = i0 + threadIdx.x;
    const bool valid = t < T;
    const float p = valid ? cand.p[t] : 0.f;
    const bool sel = valid && sel_key(p, (uint32_t)t) >= thr;
    int tot;
    const int r = block_exclusive_scan_sel(sel ? 1 : 0, tmp, &tot);
    // exactly C keys reach the threshold; the bound keeps every write inside
    // the expert's C rows regardless
    const bool keep = sel && base + r < C;
    if (valid) {
      const int64_t row = (int64_t)e * C + base + r;
      sel_row[t * E + e] = keep ? (int32_t)row : -1;
      gate_te[t * E + e] = keep ? p : 0.f;
      if (keep) row_token[row] = (int32_t)t;
    }
    base += tot;
  }
}

// Score drop, keys: every routed assignment a = t*k + j at its dropless row
// r (token order within its expert) gets key(gate, r - offsets_dl[e]).
__global__ __launch_bounds__(256) void score_keys_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const int32_t* __restrict__ assign_dl, const int32_t* __restrict__ offsets_dl, int64_t n_assign,
    int E, uint64_t* __restrict__ key_dl, int32_t* __restrict__ aid_dl) {
  const int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a >= n_assign) return;
  const int e = idx[a];
  const int r = assign_dl[a];
  if ((unsigned)e >= (unsigned)E || r < 0) return;
  key_dl[r] = sel_key(gate[a], (uint32_t)(r - offsets_dl[e]));
  aid_dl[r] = (int32_t)a;
}

// Score drop: expert e = blockIdx.x keeps its C largest-gate assignments.
__global__ __launch_bounds__(kSelThreads) void score_drop_kernel(
    const uint64_t* __restrict__ key_dl, const int32_t* __restrict__ aid_dl,
    const int32_t* __restrict__ offsets_dl, int k, int C, int32_t* __restrict__ assign_row,
    int32_t* __restrict__ row_token) {
  __shared__ int tmp[kSelWaves + 1];
  const int e = blockIdx.x;
  const int64_t off = offsets_dl[e];
  const int64_t n = offsets_dl[e + 1] - off;
  const CandSD cand{key_dl + off};
  const uint64_t thr = (n > C) ? topc_threshold(cand, n, C) : 0;
  int base = 0;
  for (int64_t i0 = 0; i0 < n; i0 += kSelThreads) {
    const int64_t i = i0 + threadIdx.x;
    const bool valid = i < n;
    const bool sel = valid && cand.key(i) >= thr;
    int tot;
    const int r = block_exclusive_scan_sel(sel ? 1 : 0, tmp, &tot);
    const bool keep = sel && base + r < C;
    if (valid) {
      const int32_t a = aid_dl[off + i];
      const int64_t row = (int64_t)e * C + base + r;
      assign_row[a] = keep ? (int32_t)row : -1;
      if (keep) row_token[row] = a / k;
    }
    base += tot;
  }
}

}  // namespace

hipError_t launch_expert_choice(const float* probs_et, int64_t T, int E, int C, int32_t* sel_row,
                                float* gate_te, int32_t* row_token, hipStream_t s) {
  MOE_LAUNCH(expert_choice_kernel, dim3((unsigned)E), dim3(kSelThreads), 0, s, probs_et, T, E, C,
                     sel_row, gate_te, row_token);
  return hipGetLastError();
}

hipError_t launch_score_drop(const int32_t* idx, const float* gate, const int32_t* assign_dl,
                             const int32_t* offsets_dl, int64_t T, int E, int k, int C,
                             uint64_t* key_dl, int32_t* aid_dl, int32_t* assign_row,
                             int32_t* row_token, hipStream_t s) {
  const int64_t n = T * k;
  MOE_LAUNCH(score_keys_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx,
                     gate, assign_dl, offsets_dl, n, E, key_dl, aid_dl);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  MOE_LAUNCH(score_drop_kernel, dim3((unsigned)E), dim3(kSelThreads), 0, s, key_dl, aid_dl,
                     offsets_dl, k, C, assign_row, row_token);
  return hipGetLastError();
}

}  // namespace moe
