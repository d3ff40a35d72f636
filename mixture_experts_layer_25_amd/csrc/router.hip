// Router GEMM: logits[t,e] = sum_i x[t,i] * w_router[e,i] (+ logit_bias[e]).
//
// Megatron-LM part 6, section "Router": the gating step multiplies the
// hidden states by the router weight; infra-l7, "NVIDIA 原题" table row
// "router" ([T,h] x [h,E] -> [T,E]).  Logits are fp32.
//
// bf16 layers use MFMA v_mfma_f32_16x16x32_bf16: one workgroup takes 16
// tokens, its 4 waves split the reduction over h into quarters and the
// experts are walked 16 at a time (up to 256 per pass), so x is read from
// HBM once; the four partial sums meet in LDS.  bf16 x bf16 products are
// exact in fp32 and accumulate in fp32.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kRouterTok = 16;       // tokens per workgroup
constexpr int kRouterChunks = 16;    // 16-expert chunks per pass

__global__ __launch_bounds__(256) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int64_t T,
    int h, int E) {
  __shared__ float red[4][kRouterTok][kRouterChunks * 16];  // 64 KiB
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kRouterTok;
  const int kq = h >> 2;                  // h % 128 == 0: kq % 32 == 0
  const int kbeg = w * kq;
  int64_t trow = t0 + (lane & 15);
  if (trow > T - 1) trow = T - 1;
  // MFMA 16x16x32 operands: lane l holds row (l & 15) and 8 consecutive k
  // values at k-group (l >> 4); A and B use the same k placement.
  const uint16_t* xp = x + trow * h + kbeg + (lane >> 4) * 8;
  const int nch = (E + 15) >> 4;

  for (int cg = 0; cg < nch; cg += kRouterChunks) {
    floatx4 acc[kRouterChunks];
#pragma unroll
    for (int c = 0; c < kRouterChunks; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int kk = 0; kk < kq; kk += 32) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(xp + kk));
#pragma unroll
      for (int c = 0; c < kRouterChunks; ++c) {
        if (cg + c < nch) {
          const int e = (cg + c) * 16 + (lane & 15);
          const int ec = e < E ? e : E - 1;
          uint4 braw = ld16(wr + (int64_t)ec * h + kbeg + (lane >> 4) * 8 + kk);
          if (e >= E) braw = uint4{0u, 0u, 0u, 0u};
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, __builtin_bit_cast(bf16x8, braw), acc[c], 0, 0, 0);
        }
      }
    }
    // C layout: lane l holds expert column (l & 15), token rows 4*(l>>4)+i.
#pragma unroll
    for (int c = 0; c < kRouterChunks; ++c) {
      if (cg + c < nch) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[w][4 * (lane >> 4) + i][c * 16 + (lane & 15)] = acc[c][i];
      }
    }
    __syncthreads();
    const int ne = min(kRouterChunks * 16, E - cg * 16);
    for (int p = threadIdx.x; p < kRouterTok * ne; p += 256) {
      const int tk = p / ne, ee = p - tk * ne;
      float s = red[0][tk][ee] + red[1][tk][ee];
      s += red[2][tk][ee];
      s += red[3][tk][ee];
      const int e = cg * 16 + ee;
      if (bias) s += bias[e];
      const int64_t t = t0 + tk;
      if (t < T) logits[t * E + e] = s;
    }
    __syncthreads();
  }
}

// fp32 layers: one thread per (token, expert), fp32 FMA over h.
__global__ __launch_bounds__(256) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int64_t T,
    int h, int E) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= T * E) return;
  const int64_t t = p / E;
  const int e = (int)(p - t * E);
  const float* xr = x + t * h;
  const float* wrow = wr + (int64_t)e * h;
  float s = 0.f;
  for (int i = 0; i < h; ++i) s = fmaf(xr[i], wrow[i], s);
  if (bias) s += bias[e];
  logits[p] = s;
}

}  // namespace

hipError_t launch_router(int dtype, const void* x, const void* w_router,
                         const float* logit_bias, float* logits, int64_t T,
                         int h, int E, hipStream_t s) {
  if (dtype == 1) {
    const int64_t nb = (T + kRouterTok - 1) / kRouterTok;
    hipLaunchKernelGGL(router_bf16_kernel, dim3((unsigned)nb), dim3(256), 0, s,
                       (const uint16_t*)x, (const uint16_t*)w_router,
                       logit_bias, logits, T, h, E);
  } else {
    const int64_t nb = (T * E + 255) / 256;
    hipLaunchKernelGGL(router_f32_kernel, dim3((unsigned)nb), dim3(256), 0, s,
                       (const float*)x, (const float*)w_router, logit_bias,
                       logits, T, h, E);
  }
  return hipGetLastError();
}

}  // namespace moe
