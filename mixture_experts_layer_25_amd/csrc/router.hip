// Router GEMM: logits[t,e] = sum_i x[t,i] * w_router[e,i] (+ logit_bias[e]).
//
// Megatron-LM part 6, section "Router": the gating step multiplies the
// hidden states by the router weight; infra-l7, "NVIDIA 原题" table row
// "router" ([T,h] x [h,E] -> [T,E]).  Logits are fp32.
//
// bf16 layers use MFMA v_mfma_f32_16x16x32_bf16, and in both kernels the
// waves of a workgroup split the reduction over h into equal parts whose
// partial sums meet in LDS in a fixed order.  Up to 16 experts: one
// workgroup takes 16 tokens and every expert, so x and the small w_router
// are each read once; its 16 (or 8, or 4) waves each take an equal share
// of h, so that a workgroup's whole slice of x is in flight at once.  More experts: one workgroup per tile of 64 tokens x
// 64 experts (4x4 MFMA tiles per wave), which bounds the re-reads of
// w_router to one per 64 tokens and keeps the grid wide.  bf16 x bf16
// products are exact in fp32 and accumulate in fp32.
//
// Up to 64 experts, the router kernel also runs the top-k, the gates and the
// expert histogram (the tile then holds every expert's logit of its tokens),
// so the logits do not make a round trip through memory before the
// selection and no separate top-k kernel runs.
#include "moe_device.h"
#include "moe_internal.h"
#include "topk_device.h"

namespace moe {

namespace {

constexpr int kRouterTok = 16;       // tokens per workgroup (up to 16 experts)
constexpr int kRouterBatch = 8;      // 32-deep steps whose loads are issued together

constexpr int kRouterMaxWaves = 16;

// Waves per workgroup of the small-E router: the most (16, 8 or 4) whose
// share of h is a multiple of 32 (h % 128 == 0, so 4 always is).
inline int router_waves(int h) { return h % (16 * 32) == 0 ? 16 : (h % (8 * 32) == 0 ? 8 : 4); }

__global__ __launch_bounds__(64 * kRouterMaxWaves) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int64_t T,
    int h, int E) {
  __shared__ float red[kRouterMaxWaves][kRouterTok][16];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;         // waves: 16, 8 or 4
  const int64_t t0 = (int64_t)blockIdx.x * kRouterTok;
  const int kq = h / nw;                  // a multiple of 32
  const int koff = w * kq + (lane >> 4) * 8;
  // MFMA 16x16x32 operands: lane l holds row (l & 15) and 8 consecutive k
  // values at k-group (l >> 4); A and B use the same k placement.  Rows
  // past T or E are clamped; their sums are dropped (experts past E are
  // zeroed so every lane's MFMA input is defined).
  int64_t trow = t0 + (lane & 15);
  trow = trow < T ? trow : T - 1;
  const int e = lane & 15;
  const bool ez = e >= E;
  const uint16_t* xp = x + trow * h + koff;
  const uint16_t* wp = wr + (int64_t)(ez ? E - 1 : e) * h + koff;

  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  int kk = 0;
  for (; kk + 32 * kRouterBatch <= kq; kk += 32 * kRouterBatch) {
    uint4 a[kRouterBatch], b[kRouterBatch];
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
      a[u] = ld16(xp + kk + 32 * u);
      b[u] = ld16(wp + kk + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
      if (ez) b[u] = uint4{0u, 0u, 0u, 0u};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                    __builtin_bit_cast(bf16x8, b[u]), acc,
                                                    0, 0, 0);
    }
  }
  for (; kk < kq; kk += 32) {
    const uint4 a = ld16(xp + kk);
    uint4 b = ld16(wp + kk);
    if (ez) b = uint4{0u, 0u, 0u, 0u};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
  // C layout: lane l holds expert column (l & 15), token rows 4*(l>>4)+i.
#pragma unroll
  for (int i = 0; i < 4; ++i) red[w][4 * (lane >> 4) + i][lane & 15] = acc[i];
  __syncthreads();
  const int tk = threadIdx.x >> 4, ee = threadIdx.x & 15;
  const int64_t t = t0 + tk;
  if (threadIdx.x < 256 && ee < E && t < T) {
    float s = red[0][tk][ee];             // wave partials in wave order
    for (int q = 1; q < nw; ++q) s += red[q][tk][ee];
    if (bias) s += bias[ee];
    logits[t * E + ee] = s;
  }
}

// The router GEMM of up to 16 experts fused with the top-k, the gates and
// the histogram of the selected experts: the workgroup's 16 tokens are 16
// top-k segments of 16 lanes (one expert per lane), so the logits never
// leave the workgroup before the selection (they are still written out).
// chunk_hist, if given, gets one row of E counts per workgroup (16 tokens).
__global__ __launch_bounds__(64 * kRouterMaxWaves) void router_topk_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits,
    const float* __restrict__ sbias, int gate_mode, int64_t T, int h, int E, int k,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out,
    int32_t* __restrict__ chunk_hist) {
  __shared__ float red[kRouterMaxWaves][kRouterTok][16];
  __shared__ int32_t sel_e[kRouterTok][16];
  __shared__ float sel_l[kRouterTok][16];
  __shared__ int32_t hist[16];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;         // waves: 16, 8 or 4
  const int64_t t0 = (int64_t)blockIdx.x * kRouterTok;
  const int kq = h / nw;                  // a multiple of 32
  const int koff = w * kq + (lane >> 4) * 8;
  // MFMA operands as in router_bf16_kernel
  int64_t trow = t0 + (lane & 15);
  trow = trow < T ? trow : T - 1;
  const int e = lane & 15;
  const bool ez = e >= E;
  const uint16_t* xp = x + trow * h + koff;
  const uint16_t* wp = wr + (int64_t)(ez ? E - 1 : e) * h + koff;

  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  int kk = 0;
  for (; kk + 32 * kRouterBatch <= kq; kk += 32 * kRouterBatch) {
    uint4 a[kRouterBatch], b[kRouterBatch];
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
      a[u] = ld16(xp + kk + 32 * u);
      b[u] = ld16(wp + kk + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
      if (ez) b[u] = uint4{0u, 0u, 0u, 0u};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                    __builtin_bit_cast(bf16x8, b[u]), acc,
                                                    0, 0, 0);
    }
  }
  for (; kk < kq; kk += 32) {
    const uint4 a = ld16(xp + kk);
    uint4 b = ld16(wp + kk);
    if (ez) b = uint4{0u, 0u, 0u, 0u};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[w][4 * (lane >> 4) + i][lane & 15] = acc[i];
  if (threadIdx.x < 16) hist[threadIdx.x] = 0;
  __syncthreads();
  if (threadIdx.x < 256) {
    // thread (tk, ee): token tk's logit of expert ee, wave partials summed
    // in wave order; then the token's 16 lanes select its top k
    const int tk = threadIdx.x >> 4, ee = threadIdx.x & 15;
    const int64_t t = t0 + tk;
    const bool valid = t < T;
    float lg[1] = {-INFINITY};
    uint64_t key[1] = {0};
    if (valid && ee < E) {
      float sum = red[0][tk][ee];
      for (int q = 1; q < nw; ++q) sum += red[q][tk][ee];
      if (bias) sum += bias[ee];
      logits[t * E + ee] = sum;
      lg[0] = sum;
      key[0] = topk_key(sbias ? sum + sbias[ee] : sum, ee);
    }
    topk_segment<16, 1>(valid, ee, E, k, gate_mode, lg, key, sel_e[tk], sel_l[tk],
                        chunk_hist ? hist : nullptr, idx_out + t * k, gate_out + t * k);
  }
  if (chunk_hist) {
    __syncthreads();
    if ((int)threadIdx.x < E) chunk_hist[blockIdx.x * (int64_t)E + threadIdx.x] = hist[threadIdx.x];
  }
}

constexpr int kTileT = 64;           // tokens per tile

// The K loop of a 64x64 router tile (4x4 MFMA 16x16x32 tiles per wave):
// U 32-deep steps per iteration, all of their loads (32 * U bytes per lane
// and row) issued before the MFMAs, then single 32-deep steps for the rest
// of kq (a multiple of 32).
template <int U>
__device__ __forceinline__ void tile_mfma_loop(const uint16_t* const (&ap)[4],
                                               const uint16_t* const (&bp)[4], int kq,
                                               floatx4 (&acc)[4][4]) {
  int kk = 0;
  for (; kk + 32 * U <= kq; kk += 32 * U) {
    bf16x8 a[U][4], b[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[u][i] = __builtin_bit_cast(bf16x8, ld16(ap[i] + kk + 32 * u));
        b[u][i] = __builtin_bit_cast(bf16x8, ld16(bp[i] + kk + 32 * u));
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][i], b[u][j], acc[i][j], 0, 0, 0);
  }
  for (; kk < kq; kk += 32) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = __builtin_bit_cast(bf16x8, ld16(ap[i] + kk));
      b[i] = __builtin_bit_cast(bf16x8, ld16(bp[i] + kk));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}
constexpr int kTileE = 64;           // experts per tile
constexpr int kRedLd = kTileE + 4;   // LDS row stride of the partial sums

// NW waves (8 when h is a multiple of 256, else 4) each take an equal share
// of h, their partial sums meeting in LDS in wave order.
template <int NW>
__global__ __launch_bounds__(64 * NW) void router_bf16_tile_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int64_t T,
    int h, int E) {
  __shared__ float red[NW][kTileT][kRedLd];  // 68 KiB per 4 waves
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTileT;
  const int e0 = blockIdx.y * kTileE;
  const int kq = h / NW;                  // a multiple of 32
  const int koff = w * kq + (lane >> 4) * 8;
  // Rows past T or E are clamped to the last one; their sums are dropped.
  const uint16_t* ap[4];
  const uint16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t t = t0 + 16 * i + (lane & 15);
    t = t < T ? t : T - 1;
    ap[i] = x + t * h + koff;
    int e = e0 + 16 * i + (lane & 15);
    e = e < E ? e : E - 1;
    bp[i] = wr + (int64_t)e * h + koff;
  }
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Two 32-deep steps per iteration so 16 loads are in flight; a 32-deep
  // tail when kq is an odd multiple of 32.
  tile_mfma_loop<2>(ap, bp, kq, acc);
  // C layout: lane l holds expert column (l & 15), token rows 4*(l>>4)+r.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[w][16 * i + 4 * (lane >> 4) + r][16 * j + (lane & 15)] = acc[i][j][r];
  __syncthreads();
  for (int p = threadIdx.x; p < kTileT * kTileE; p += 64 * NW) {
    const int tk = p / kTileE, ee = p % kTileE;
    const int64_t t = t0 + tk;
    const int e = e0 + ee;
    if (t < T && e < E) {
      float s = red[0][tk][ee];
#pragma unroll
      for (int q = 1; q < NW; ++q) s += red[q][tk][ee];
      if (bias) s += bias[e];
      logits[t * E + e] = s;
    }
  }
}

// The tile router of up to 64 experts fused with the top-k, the gates and
// the histogram.  The MFMA tile covers the workgroup's 64 tokens and every
// expert; its NW waves (8 when h is a multiple of 256, else 4) each take an
// equal share of h, so twice the loads of router_bf16_tile_kernel are in
// flight per compute unit.  The partial sums meet in LDS in wave order; then
// the tokens go through the top-k in segments of 16 lanes, lane s holding
// experts s, s + 16, ... (NPL of them), 16 * NW / 4 tokens at a time.  The
// logits are still written out.  chunk_hist, if given, gets one row of E
// counts per workgroup (64 tokens).
template <int NW, int NPL>
__global__ __launch_bounds__(64 * NW) void router_topk_tile_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits,
    const float* __restrict__ sbias, int gate_mode, int64_t T, int h, int E, int k,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out,
    int32_t* __restrict__ chunk_hist) {
  static_assert(NPL * 16 <= kTileE, "up to 64 experts");
  __shared__ float red[NW][kTileT][kRedLd];  // 68 KiB per 4 waves
  __shared__ int32_t sel_e[kTileT][16];
  __shared__ float sel_l[kTileT][16];
  __shared__ int32_t hist[kTileE];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTileT;
  const int kq = h / NW;                  // a multiple of 32
  const int koff = w * kq + (lane >> 4) * 8;
  // MFMA operands as in router_bf16_tile_kernel (one tile of 64 experts)
  const uint16_t* ap[4];
  const uint16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t t = t0 + 16 * i + (lane & 15);
    t = t < T ? t : T - 1;
    ap[i] = x + t * h + koff;
    int e = 16 * i + (lane & 15);
    e = e < E ? e : E - 1;
    bp[i] = wr + (int64_t)e * h + koff;
  }
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  tile_mfma_loop<2>(ap, bp, kq, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[w][16 * i + 4 * (lane >> 4) + r][16 * j + (lane & 15)] = acc[i][j][r];
  if (threadIdx.x < kTileE) hist[threadIdx.x] = 0;
  __syncthreads();
  constexpr int kPerPass = 4 * NW;         // 16-lane segments per pass
  const int seg = threadIdx.x >> 4, sl = threadIdx.x & 15;
  for (int p = 0; p < kTileT / kPerPass; ++p) {
    const int tk = p * kPerPass + seg;
    const int64_t t = t0 + tk;
    const bool valid = t < T;
    float lg[NPL];
    uint64_t key[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int ee = sl + 16 * i;
      lg[i] = -INFINITY;
      key[i] = 0;
      if (valid && ee < E) {
        float sum = red[0][tk][ee];
#pragma unroll
        for (int q = 1; q < NW; ++q) sum += red[q][tk][ee];
        if (bias) sum += bias[ee];
        logits[t * E + ee] = sum;
        lg[i] = sum;
        key[i] = topk_key(sbias ? sum + sbias[ee] : sum, ee);
      }
    }
    topk_segment<16, NPL>(valid, sl, E, k, gate_mode, lg, key, sel_e[tk], sel_l[tk],
                          chunk_hist ? hist : nullptr, idx_out + t * k, gate_out + t * k);
  }
  if (chunk_hist) {
    __syncthreads();
    if ((int)threadIdx.x < E) chunk_hist[blockIdx.x * (int64_t)E + threadIdx.x] = hist[threadIdx.x];
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

bool router_topk_fused(int dtype, int E) { return dtype == 1 && E <= 64; }

int router_topk_tokens(int E) { return E <= 16 ? kRouterTok : kTileT; }

hipError_t launch_router_topk(const void* x, const void* w_router, const float* logit_bias,
                              float* logits, const float* select_bias, int gate, int64_t T,
                              int h, int E, int k, int32_t* idx, float* gate_out,
                              int32_t* chunk_hist, hipStream_t s) {
  const int tok = router_topk_tokens(E);
  const int64_t nb = (T + tok - 1) / tok;
  if (E <= 16)
    MOE_LAUNCH(router_topk_bf16_kernel, dim3((unsigned)nb), dim3(64 * router_waves(h)), 0, s,
               (const uint16_t*)x, (const uint16_t*)w_router, logit_bias, logits, select_bias,
               gate, T, h, E, k, idx, gate_out, chunk_hist);
  else if (h % 256 == 0 && E <= 32)
    MOE_LAUNCH((router_topk_tile_bf16_kernel<8, 2>), dim3((unsigned)nb), dim3(512), 0, s,
               (const uint16_t*)x, (const uint16_t*)w_router, logit_bias, logits, select_bias,
               gate, T, h, E, k, idx, gate_out, chunk_hist);
  else if (h % 256 == 0)
    MOE_LAUNCH((router_topk_tile_bf16_kernel<8, 4>), dim3((unsigned)nb), dim3(512), 0, s,
               (const uint16_t*)x, (const uint16_t*)w_router, logit_bias, logits, select_bias,
               gate, T, h, E, k, idx, gate_out, chunk_hist);
  else if (E <= 32)
    MOE_LAUNCH((router_topk_tile_bf16_kernel<4, 2>), dim3((unsigned)nb), dim3(256), 0, s,
               (const uint16_t*)x, (const uint16_t*)w_router, logit_bias, logits, select_bias,
               gate, T, h, E, k, idx, gate_out, chunk_hist);
  else
    MOE_LAUNCH((router_topk_tile_bf16_kernel<4, 4>), dim3((unsigned)nb), dim3(256), 0, s,
               (const uint16_t*)x, (const uint16_t*)w_router, logit_bias, logits, select_bias,
               gate, T, h, E, k, idx, gate_out, chunk_hist);
  return hipGetLastError();
}

hipError_t launch_router(int dtype, const void* x, const void* w_router,
                         const float* logit_bias, float* logits, int64_t T,
                         int h, int E, hipStream_t s) {
  if (dtype == 1 && E > 16) {
    const dim3 grid((unsigned)((T + kTileT - 1) / kTileT), (unsigned)((E + kTileE - 1) / kTileE));
    if (h % 256 == 0)
      MOE_LAUNCH(router_bf16_tile_kernel<8>, grid, dim3(512), 0, s, (const uint16_t*)x,
                 (const uint16_t*)w_router, logit_bias, logits, T, h, E);
    else
      MOE_LAUNCH(router_bf16_tile_kernel<4>, grid, dim3(256), 0, s, (const uint16_t*)x,
                 (const uint16_t*)w_router, logit_bias, logits, T, h, E);
  } else if (dtype == 1) {
    const int64_t nb = (T + kRouterTok - 1) / kRouterTok;
    MOE_LAUNCH(router_bf16_kernel, dim3((unsigned)nb), dim3(64 * router_waves(h)), 0, s,
                       (const uint16_t*)x, (const uint16_t*)w_router,
                       logit_bias, logits, T, h, E);
  } else {
    const int64_t nb = (T * E + 255) / 256;
    MOE_LAUNCH(router_f32_kernel, dim3((unsigned)nb), dim3(256), 0, s,
                       (const float*)x, (const float*)w_router, logit_bias,
                       logits, T, h, E);
  }
  return hipGetLastError();
}

}  // namespace moe
