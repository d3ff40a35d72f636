// Combine / unpermute: y[t] = sum_j gate[t,j] * y_perm[assign_row[t,j]]
//                             (+ shared_y[t]).
//
// 专家并行, "EP+DP" forward: the results of a token's top-k experts are
// gathered back and summed with their weights; infra-l7, "NVIDIA 原题" row
// combine (back to the original place, k outputs weighted by the gates);
// "自测": a slot dropped past capacity contributes nothing.
//
// kCombTok tokens per workgroup; each thread gathers 16-byte vectors of the
// k expert rows, sums in fp32 in slot order (shared expert last) and stores
// one 16-byte vector of y.  With expert-choice routing the slots of a token
// are the E experts (row -1 where an expert did not choose it).  A slot
// whose row is outside [0, nrows) (-1: dropped) contributes nothing, so a
// caller's map can never send a read past the expert outputs.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kCombTok = 2;

template <int KMAX>
__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const uint4* __restrict__ yp, int64_t pv, const int32_t* __restrict__ assign_row,
    const float* __restrict__ gate, const uint4* __restrict__ shared_y,
    uint4* __restrict__ y, int64_t T, int nv, int k, int nrows) {
  for (int tt = 0; tt < kCombTok; ++tt) {
    const int64_t t = (int64_t)blockIdx.x * kCombTok + tt;
    if (t >= T) return;
    int rows[KMAX];
    float g[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      rows[j] = j < k ? assign_row[t * k + j] : -1;
      g[j] = j < k ? gate[t * k + j] : 0.f;
    }
    for (int v = threadIdx.x; v < nv; v += 256) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if ((uint32_t)rows[j] < (uint32_t)nrows) {
          const uint4 q = yp[(int64_t)rows[j] * pv + v];
          const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            acc[2 * p] = fmaf(g[j], bf16_bits_to_f32(u[p] & 0xFFFFu), acc[2 * p]);
            acc[2 * p + 1] = fmaf(g[j], bf16_bits_to_f32(u[p] >> 16), acc[2 * p + 1]);
          }
        }
      }
      if (shared_y) {
        const uint4 q = shared_y[t * pv + v];
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          acc[2 * p] += bf16_bits_to_f32(u[p] & 0xFFFFu);
          acc[2 * p + 1] += bf16_bits_to_f32(u[p] >> 16);
        }
      }
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      y[t * nv + v] = o;
    }
  }
}

template <int KMAX>
__global__ __launch_bounds__(256) void combine_f32_kernel(
    const float4* __restrict__ yp, int64_t pv, const int32_t* __restrict__ assign_row,
    const float* __restrict__ gate, const float4* __restrict__ shared_y,
    float4* __restrict__ y, int64_t T, int nv, int k, int nrows) {
  for (int tt = 0; tt < kCombTok; ++tt) {
    const int64_t t = (int64_t)blockIdx.x * kCombTok + tt;
    if (t >= T) return;
    int rows[KMAX];
    float g[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      rows[j] = j < k ? assign_row[t * k + j] : -1;
      g[j] = j < k ? gate[t * k + j] : 0.f;
    }
    for (int v = threadIdx.x; v < nv; v += 256) {
      float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if ((uint32_t)rows[j] < (uint32_t)nrows) {
          const float4 q = yp[(int64_t)rows[j] * pv + v];
          acc.x = fmaf(g[j], q.x, acc.x);
          acc.y = fmaf(g[j], q.y, acc.y);
          acc.z = fmaf(g[j], q.z, acc.z);
          acc.w = fmaf(g[j], q.w, acc.w);
        }
      }
      if (shared_y) {
        const float4 q = shared_y[t * pv + v];
        acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
      }
      y[t * nv + v] = acc;
    }
  }
}

// More than 16 slots per token (expert-choice routing over many experts,
// where most slots are empty): the workgroup first compacts the token's
// kept (row, gate) pairs into LDS in slot order (a block scan of the
// flags), then sums only those, still in slot order.
__device__ int block_exclusive_scan_256c(int v, int* tmp, int* tot) {
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
    for (int i = 0; i < 4; ++i) {
      const int c = tmp[i];
      tmp[i] = run;
      run += c;
    }
    tmp[4] = run;
  }
  __syncthreads();
  const int res = tmp[w] + incl - v;
  *tot = tmp[4];
  __syncthreads();
  return res;
}

template <bool BF16>
__global__ __launch_bounds__(256) void combine_sparse_kernel(
    const void* __restrict__ yp_, int64_t pv, const int32_t* __restrict__ assign_row,
    const float* __restrict__ gate, const void* __restrict__ shared_y_, void* __restrict__ y_,
    int64_t T, int nv, int k, int nrows) {
  __shared__ int32_t lrow[1024];
  __shared__ float lgate[1024];
  __shared__ int tmp[8];
  const int64_t t = blockIdx.x;
  int n = 0;
  for (int j0 = 0; j0 < k; j0 += 256) {
    const int j = j0 + threadIdx.x;
    const int r = j < k ? assign_row[t * k + j] : -1;
    const bool kept = (uint32_t)r < (uint32_t)nrows;
    int tot;
    const int pos = block_exclusive_scan_256c(kept ? 1 : 0, tmp, &tot);
    if (kept) {
      lrow[n + pos] = r;
      lgate[n + pos] = gate[t * k + j];
    }
    n += tot;
  }
  __syncthreads();
  if (BF16) {
    const uint4* yp = (const uint4*)yp_;
    const uint4* shared_y = (const uint4*)shared_y_;
    uint4* y = (uint4*)y_;
    for (int v = threadIdx.x; v < nv; v += 256) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
      for (int q = 0; q < n; ++q) {
        const uint4 u4 = yp[(int64_t)lrow[q] * pv + v];
        const float g = lgate[q];
        const uint32_t u[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          acc[2 * p] = fmaf(g, bf16_bits_to_f32(u[p] & 0xFFFFu), acc[2 * p]);
          acc[2 * p + 1] = fmaf(g, bf16_bits_to_f32(u[p] >> 16), acc[2 * p + 1]);
        }
      }
      if (shared_y) {
        const uint4 q4 = shared_y[t * pv + v];
        const uint32_t u[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          acc[2 * p] += bf16_bits_to_f32(u[p] & 0xFFFFu);
          acc[2 * p + 1] += bf16_bits_to_f32(u[p] >> 16);
        }
      }
      y[t * nv + v] = uint4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                            pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    }
  } else {
    const float4* yp = (const float4*)yp_;
    const float4* shared_y = (const float4*)shared_y_;
    float4* y = (float4*)y_;
    for (int v = threadIdx.x; v < nv; v += 256) {
      float4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < n; ++q) {
        const float4 u = yp[(int64_t)lrow[q] * pv + v];
        const float g = lgate[q];
        acc.x = fmaf(g, u.x, acc.x);
        acc.y = fmaf(g, u.y, acc.y);
        acc.z = fmaf(g, u.z, acc.z);
        acc.w = fmaf(g, u.w, acc.w);
      }
      if (shared_y) {
        const float4 u = shared_y[t * pv + v];
        acc.x += u.x; acc.y += u.y; acc.z += u.z; acc.w += u.w;
      }
      y[t * nv + v] = acc;
    }
  }
}

template <int KMAX>
void launch_combine_t(int dtype, const void* yp, int ld, const int32_t* ar, const float* g,
                      const void* sy, void* y, int64_t T, int h, int k, int nrows,
                      hipStream_t s) {
  const int64_t nb = (T + kCombTok - 1) / kCombTok;
  if (dtype == 1)
    MOE_LAUNCH((combine_bf16_kernel<KMAX>), dim3((unsigned)nb), dim3(256), 0, s,
                       (const uint4*)yp, (int64_t)ld / 8, ar, g, (const uint4*)sy, (uint4*)y, T,
                       h / 8, k, nrows);
  else
    MOE_LAUNCH((combine_f32_kernel<KMAX>), dim3((unsigned)nb), dim3(256), 0, s,
                       (const float4*)yp, (int64_t)ld / 4, ar, g, (const float4*)sy, (float4*)y,
                       T, h / 4, k, nrows);
}

}  // namespace

hipError_t launch_combine(int dtype, const void* y_perm, int ld_perm,
                          const int32_t* assign_row, const float* gate,
                          const void* shared_y, void* y, int64_t T, int h, int k,
                          int64_t nrows, hipStream_t s) {
  if (k <= 1)
    launch_combine_t<1>(dtype, y_perm, ld_perm, assign_row, gate, shared_y, y, T, h, k, (int)nrows, s);
  else if (k <= 2)
    launch_combine_t<2>(dtype, y_perm, ld_perm, assign_row, gate, shared_y, y, T, h, k, (int)nrows, s);
  else if (k <= 4)
    launch_combine_t<4>(dtype, y_perm, ld_perm, assign_row, gate, shared_y, y, T, h, k, (int)nrows, s);
  else if (k <= 8)
    launch_combine_t<8>(dtype, y_perm, ld_perm, assign_row, gate, shared_y, y, T, h, k, (int)nrows, s);
  else if (k <= 16)
    launch_combine_t<16>(dtype, y_perm, ld_perm, assign_row, gate, shared_y, y, T, h, k, (int)nrows, s);
  else if (dtype == 1)
    MOE_LAUNCH(combine_sparse_kernel<true>, dim3((unsigned)T), dim3(256), 0, s, y_perm,
                       (int64_t)ld_perm / 8, assign_row, gate, shared_y, y, T, h / 8, k, (int)nrows);
  else
    MOE_LAUNCH(combine_sparse_kernel<false>, dim3((unsigned)T), dim3(256), 0, s, y_perm,
                       (int64_t)ld_perm / 4, assign_row, gate, shared_y, y, T, h / 4, k, (int)nrows);
  return hipGetLastError();
}

}  // namespace moe
