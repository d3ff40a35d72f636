// Backward of the MoE layer (bf16): the kernels around the grouped GEMMs.
//
// 专家并行 page, "EP+DP" BWD: every GPU computes the gradients of its
// experts' weights and the gradients go back along the routing path (the
// reverse all-to-all) to the layers before.  With L = sum(y * dy) and the
// routing held fixed, for a kept slot (t, j) of expert e at row r:
//   dO[r] = g[t,j] dy[t],  dg[t,j] = dy[t] . o[r],  dU = dO W2,
//   dA1 = dU a3 s (1 + a1 (1 - s)), dA3 = dU a1 s  (s = sigmoid(a1)),
//   dx_perm = dA1 W1 + dA3 W3,  dW2 += dO^T u,  dW1 += dA1^T x,  dW3 += dA3^T x,
// the gate modes' Jacobians give dl[t,:] from dg[t,:], and
//   dW_router = dl^T x,  dlogit_bias = sum_t dl,  dx = sum_j dx_perm + dl W_router.
// Every sum here runs in a fixed order: the same bits on every run.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

// ---------------------------------------------------------------- transposes
// 64 x 64 bf16 tiles through LDS (rows padded by one 4-byte word against
// bank conflicts); 16-byte loads and stores.
constexpr int kTr = 64;

// dst[b][c][col0 + r] = src[b][r][c] for r < R, c < Cc (R, Cc multiples of
// 64; dense src rows of Cc).
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src,
                                                        int64_t src_bs, int R, int Cc,
                                                        uint16_t* __restrict__ dst,
                                                        int64_t dst_bs, int dld, int col0) {
  __shared__ uint16_t tile[kTr][kTr + 2];
  const int b = blockIdx.z;
  const int c0 = blockIdx.x * kTr, r0 = blockIdx.y * kTr;
  const uint16_t* s = src + b * src_bs;
  uint16_t* d = dst + b * dst_bs;
  for (int q = threadIdx.x; q < kTr * 8; q += 256) {
    const int rr = q >> 3, cv = (q & 7) * 8;
    const uint4 v = ld16(s + (int64_t)(r0 + rr) * Cc + c0 + cv);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      tile[rr][cv + 2 * p] = (uint16_t)(u[p] & 0xFFFFu);
      tile[rr][cv + 2 * p + 1] = (uint16_t)(u[p] >> 16);
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kTr * 8; q += 256) {
    const int cc = q >> 3, rv = (q & 7) * 8;
    uint32_t u[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      u[p] = (uint32_t)tile[rv + 2 * p][cc] | ((uint32_t)tile[rv + 2 * p + 1][cc] << 16);
    st16(d + (int64_t)(c0 + cc) * dld + col0 + r0 + rv, uint4{u[0], u[1], u[2], u[3]});
  }
}

// K table of the weight gradients from the tile table gtab of G groups:
// kt[g] = first K column of group g (prefix of kpad), kt[G+g] = kpad =
// rows rounded up to 64, kt[2G+g] = first source row, kt[3G+g] = rows.
// use_a_rows: source rows are gtab's A rows (x_perm, or x for the shared
// group), else its output rows.  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void ktab_kernel(const int32_t* __restrict__ gtab, int G,
                                                    int use_a_rows, int32_t* __restrict__ kt) {
  __shared__ int tmp[32];
  const int g = threadIdx.x;
  const int n = g < G ? gtab[2 * G + 1 + g] : 0;
  const int kpad = (n + 63) & ~63;
  // exclusive scan of kpad over the workgroup
  const int lane = g & 63, w = g >> 6;
  int incl = kpad;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  if (g == 0) {
    int run = 0;
    for (int i = 0; i < 16; ++i) {
      const int c = tmp[i];
      tmp[i] = run;
      run += c;
    }
  }
  __syncthreads();
  if (g < G) {
    kt[g] = tmp[w] + incl - kpad;
    kt[G + g] = kpad;
    kt[2 * G + g] = use_a_rows ? gtab[G + 1 + g] : gtab[3 * G + 1 + g];
    kt[3 * G + g] = n;
  }
}

// Per-group transpose into the K layout of the weight gradients: for the
// 64 K columns of tile (blockIdx.y) in group g, dst[c][k] = src_g[r0 + k -
// koff][c] while k - koff < n, else 0.  Groups >= E_routed read src_shared.
__global__ __launch_bounds__(256) void transpose_groups_kernel(
    const uint16_t* __restrict__ src, int sld, const uint16_t* __restrict__ src_shared,
    int sld_shared, int E_routed, const int32_t* __restrict__ kt, int G, int Cc,
    uint16_t* __restrict__ dst, int dld) {
  __shared__ uint16_t tile[kTr][kTr + 2];
  const int64_t k0 = (int64_t)blockIdx.y * kTr;
  const int ktot = kt[G - 1] + kt[2 * G - 1];
  if (k0 >= ktot) return;
  int lo = 0, hi = G;               // last group with koff <= k0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (kt[mid] <= k0) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int64_t koff = kt[g], n = kt[3 * G + g], r0 = kt[2 * G + g];
  const bool sh = g >= E_routed;
  const uint16_t* s = sh ? src_shared : src;
  const int ld = sh ? sld_shared : sld;
  const int c0 = blockIdx.x * kTr;
  for (int q = threadIdx.x; q < kTr * 8; q += 256) {
    const int rr = q >> 3, cv = (q & 7) * 8;
    const int64_t kr = k0 + rr - koff;          // row within the group
    uint4 v = uint4{0u, 0u, 0u, 0u};
    if (kr < n) v = ld16(s + (r0 + kr) * ld + c0 + cv);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      tile[rr][cv + 2 * p] = (uint16_t)(u[p] & 0xFFFFu);
      tile[rr][cv + 2 * p + 1] = (uint16_t)(u[p] >> 16);
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kTr * 8; q += 256) {
    const int cc = q >> 3, rv = (q & 7) * 8;
    uint32_t u[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      u[p] = (uint32_t)tile[rv + 2 * p][cc] | ((uint32_t)tile[rv + 2 * p + 1][cc] << 16);
    st16(dst + (int64_t)(c0 + cc) * dld + k0 + rv, uint4{u[0], u[1], u[2], u[3]});
  }
}

// ------------------------------------------------------------ row kernels
constexpr int kRowTok = 2;

// dO rows: routed row assign_row[t,j] = bf16(g[t,j] dy[t]); shared row
// rows + t = dy[t]; then (capacity) padding rows zero, like the permute.
__global__ __launch_bounds__(256) void scatter_dy_kernel(
    const uint4* __restrict__ dy, const int32_t* __restrict__ assign_row,
    const float* __restrict__ gate, const int32_t* __restrict__ counts, int64_t T, int nv, int E,
    int k, int64_t C, int64_t rows, int has_shared, int64_t ntb, uint4* __restrict__ dO,
    int64_t pv) {
  const int64_t b = blockIdx.x;
  if (b < ntb) {
    for (int tt = 0; tt < kRowTok; ++tt) {
      const int64_t t = b * kRowTok + tt;
      if (t >= T) return;
      for (int v = threadIdx.x; v < nv; v += 256) {
        const uint4 q = dy[t * nv + v];
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
        for (int j = 0; j < k; ++j) {
          const int r = assign_row[t * k + j];
          if (r < 0) continue;
          const float g = gate[t * k + j];
          uint32_t o[4];
#pragma unroll
          for (int p = 0; p < 4; ++p)
            o[p] = pack_bf16x2(g * bf16_bits_to_f32(u[p] & 0xFFFFu),
                               g * bf16_bits_to_f32(u[p] >> 16));
          dO[(int64_t)r * pv + v] = uint4{o[0], o[1], o[2], o[3]};
        }
        if (has_shared) dO[(rows + t) * pv + v] = q;
      }
    }
    return;
  }
  const int64_t pb = b - ntb;
  for (int e = 0; e < E; ++e) {
    const int64_t kept = min((int64_t)counts[e], C);
    for (int64_t r = e * C + kept + pb; r < (e + 1) * C; r += 256) {
      for (int v = threadIdx.x; v < nv; v += 256) dO[r * pv + v] = uint4{0u, 0u, 0u, 0u};
    }
  }
}

// dg[t,j] = dy[t] . o[assign_row[t,j]] (0 for a dropped slot): one
// workgroup per token, per-thread fp32 partial sums, then a fixed tree.
__global__ __launch_bounds__(256) void gate_grad_kernel(const uint4* __restrict__ dy,
                                                        const uint4* __restrict__ o, int64_t pv,
                                                        const int32_t* __restrict__ assign_row,
                                                        int nv, int k, float* __restrict__ dg) {
  __shared__ float red[256];
  const int64_t t = blockIdx.x;
  for (int j = 0; j < k; ++j) {
    const int r = assign_row[t * k + j];
    float acc = 0.f;
    if (r >= 0) {
      for (int v = threadIdx.x; v < nv; v += 256) {
        const uint4 a = dy[t * nv + v], b = o[(int64_t)r * pv + v];
        const uint32_t ua[4] = {a.x, a.y, a.z, a.w}, ub[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          acc = fmaf(bf16_bits_to_f32(ua[p] & 0xFFFFu), bf16_bits_to_f32(ub[p] & 0xFFFFu), acc);
          acc = fmaf(bf16_bits_to_f32(ua[p] >> 16), bf16_bits_to_f32(ub[p] >> 16), acc);
        }
      }
    }
    red[threadIdx.x] = acc;
    for (int w = 128; w > 0; w >>= 1) {
      __syncthreads();
      if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    }
    __syncthreads();
    if (threadIdx.x == 0) dg[t * k + j] = red[0];
    __syncthreads();
  }
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.f / (1.f + __expf(-z)); }

// u = silu(a1) * a3 from a13 = [a1 | a3] (rows x 2F), 8 columns per thread.
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint4* __restrict__ a13,
                                                         int64_t lda13, int64_t rows, int fv,
                                                         uint4* __restrict__ u, int64_t ldu) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= rows * fv) return;
  const int64_t r = q / fv;
  const int v = (int)(q - r * fv);
  const uint4 x1 = a13[r * lda13 + v], x3 = a13[r * lda13 + fv + v];
  const uint32_t p1[4] = {x1.x, x1.y, x1.z, x1.w}, p3[4] = {x3.x, x3.y, x3.z, x3.w};
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float a[2] = {bf16_bits_to_f32(p1[p] & 0xFFFFu), bf16_bits_to_f32(p1[p] >> 16)};
    float c[2] = {bf16_bits_to_f32(p3[p] & 0xFFFFu), bf16_bits_to_f32(p3[p] >> 16)};
    o[p] = pack_bf16x2(a[0] * sigmoidf_(a[0]) * c[0], a[1] * sigmoidf_(a[1]) * c[1]);
  }
  u[r * ldu + v] = uint4{o[0], o[1], o[2], o[3]};
}

// dA = [dU a3 s (1 + a1 (1 - s)) | dU a1 s], s = sigmoid(a1).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint4* __restrict__ a13,
                                                         int64_t lda13,
                                                         const uint4* __restrict__ dU,
                                                         int64_t ldu, int64_t rows, int fv,
                                                         uint4* __restrict__ dA, int64_t ldda) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= rows * fv) return;
  const int64_t r = q / fv;
  const int v = (int)(q - r * fv);
  const uint4 x1 = a13[r * lda13 + v], x3 = a13[r * lda13 + fv + v], du = dU[r * ldu + v];
  const uint32_t p1[4] = {x1.x, x1.y, x1.z, x1.w}, p3[4] = {x3.x, x3.y, x3.z, x3.w},
                 pd[4] = {du.x, du.y, du.z, du.w};
  uint32_t o1[4], o3[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float r1[2], r3[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float a = bf16_bits_to_f32(e ? p1[p] >> 16 : p1[p] & 0xFFFFu);
      const float c = bf16_bits_to_f32(e ? p3[p] >> 16 : p3[p] & 0xFFFFu);
      const float d = bf16_bits_to_f32(e ? pd[p] >> 16 : pd[p] & 0xFFFFu);
      const float s = sigmoidf_(a);
      r1[e] = d * c * s * (1.f + a * (1.f - s));
      r3[e] = d * a * s;
    }
    o1[p] = pack_bf16x2(r1[0], r1[1]);
    o3[p] = pack_bf16x2(r3[0], r3[1]);
  }
  dA[r * ldda + v] = uint4{o1[0], o1[1], o1[2], o1[3]};
  dA[r * ldda + fv + v] = uint4{o3[0], o3[1], o3[2], o3[3]};
}

// dl[t,:] from dg[t,:] for the gate modes (one thread per token; fp32).
__global__ __launch_bounds__(256) void gates_bwd_kernel(const float* __restrict__ logits,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ gate,
                                                        const float* __restrict__ dg,
                                                        int gate_mode, int64_t T, int E, int k,
                                                        float* __restrict__ dl) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const float* l = logits + t * E;
  float* d = dl + t * E;
  for (int e = 0; e < E; ++e) d[e] = 0.f;
  float gd = 0.f;                     // sum_j g_j dg_j
  for (int j = 0; j < k; ++j) gd += gate[t * k + j] * dg[t * k + j];
  if (gate_mode == 0) {               // softmax over the selected
    for (int j = 0; j < k; ++j) {
      const float g = gate[t * k + j];
      d[idx[t * k + j]] += g * (dg[t * k + j] - gd);
    }
  } else if (gate_mode == 1) {        // softmax over all E, selected values
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmaxf(m, l[e]);
    float den = 0.f;
    for (int e = 0; e < E; ++e) den += expf(l[e] - m);
    for (int e = 0; e < E; ++e) d[e] = -(expf(l[e] - m) / den) * gd;
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      d[e] += (expf(l[e] - m) / den) * dg[t * k + j];
    }
  } else {                            // sigmoid normalised over the selected
    float S = 0.f;
    for (int j = 0; j < k; ++j) S += 1.f / (1.f + expf(-l[idx[t * k + j]]));
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      const float s = 1.f / (1.f + expf(-l[e]));
      d[e] += (dg[t * k + j] - gd) / S * s * (1.f - s);
    }
  }
}

// dW_router[e, i] = sum_t dl[t,e] x[t,i]: workgroup (column tile, 32
// experts, token slice z) sums its slice of tokens in order (64 at a time
// through LDS) into part[z][e][i] (fp32); router_wgrad_sum adds the
// slices in order and rounds to bf16.
constexpr int kRbE = 32;
constexpr int kRbSlices = 32;
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float* __restrict__ dl,
                                                           const uint16_t* __restrict__ x,
                                                           int64_t T, int h, int E, int64_t tc,
                                                           float* __restrict__ part) {
  __shared__ float sdl[64][kRbE];
  __shared__ float sx[64][64];
  const int i0 = blockIdx.x * 64, e0 = blockIdx.y * kRbE;
  const int64_t tb = (int64_t)blockIdx.z * tc, te = min(T, tb + tc);
  const int ii = threadIdx.x & 63, eg = threadIdx.x >> 6;   // experts eg, eg+4, ...
  float acc[kRbE / 4];
#pragma unroll
  for (int q = 0; q < kRbE / 4; ++q) acc[q] = 0.f;
  for (int64_t t0 = tb; t0 < te; t0 += 64) {
    for (int q = threadIdx.x; q < 64 * kRbE; q += 256) {
      const int tt = q / kRbE, ee = q % kRbE;
      sdl[tt][ee] = (t0 + tt < te && e0 + ee < E) ? dl[(t0 + tt) * E + e0 + ee] : 0.f;
    }
    for (int q = threadIdx.x; q < 64 * 64; q += 256) {
      const int tt = q >> 6, c = q & 63;
      sx[tt][c] = t0 + tt < te ? bf16_bits_to_f32(x[(t0 + tt) * h + i0 + c]) : 0.f;
    }
    __syncthreads();
    for (int tt = 0; tt < 64; ++tt) {
      const float xv = sx[tt][ii];
#pragma unroll
      for (int q = 0; q < kRbE / 4; ++q) acc[q] = fmaf(sdl[tt][eg + 4 * q], xv, acc[q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < kRbE / 4; ++q) {
    const int e = e0 + eg + 4 * q;
    if (e < E) part[((int64_t)blockIdx.z * E + e) * h + i0 + ii] = acc[q];
  }
}

__global__ __launch_bounds__(256) void router_wgrad_sum_kernel(const float* __restrict__ part,
                                                               int slices, int64_t n,
                                                               uint16_t* __restrict__ dwr) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n) return;
  float s = 0.f;
  for (int z = 0; z < slices; ++z) s += part[z * n + q];
  dwr[q] = f32_to_bf16_bits(s);
}

// dlogit_bias[e] = sum_t dl[t,e]: one workgroup per expert, fixed tree.
__global__ __launch_bounds__(256) void bias_grad_kernel(const float* __restrict__ dl, int64_t T,
                                                        int E, float* __restrict__ db) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float acc = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += 256) acc += dl[t * E + e];
  red[threadIdx.x] = acc;
  for (int w = 128; w > 0; w >>= 1) {
    __syncthreads();
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
  }
  if (threadIdx.x == 0) db[e] = red[0];
}

// dx[t] = bf16( sum_j dxp[assign_row[t,j]] (slot order) + dxp[rows + t]
// (shared) + sum_e dl[t,e] W_router[e] ); 64 columns x 32 tokens per
// workgroup (8 tokens per thread), the router term over experts in order
// through LDS, so W_router is read once per 32 tokens.
constexpr int kDxTok = 32;
__global__ __launch_bounds__(256) void dx_final_kernel(
    const uint16_t* __restrict__ dxp, int64_t ldp, const int32_t* __restrict__ assign_row,
    int k, int64_t rows, int has_shared, const float* __restrict__ dl,
    const uint16_t* __restrict__ wr, int64_t T, int h, int E, uint16_t* __restrict__ dx) {
  __shared__ float sw[kRbE][64];
  __shared__ float sdl[kDxTok][kRbE];
  const int i0 = blockIdx.x * 64;
  const int64_t t0 = (int64_t)blockIdx.y * kDxTok;
  const int ii = threadIdx.x & 63, tg = threadIdx.x >> 6;    // tokens tg + 4m
  float racc[kDxTok / 4];
#pragma unroll
  for (int m = 0; m < kDxTok / 4; ++m) racc[m] = 0.f;
  for (int e0 = 0; e0 < E; e0 += kRbE) {
    for (int q = threadIdx.x; q < kRbE * 64; q += 256) {
      const int ee = q >> 6, c = q & 63;
      sw[ee][c] = e0 + ee < E ? bf16_bits_to_f32(wr[(int64_t)(e0 + ee) * h + i0 + c]) : 0.f;
    }
    for (int q = threadIdx.x; q < kDxTok * kRbE; q += 256) {
      const int tq = q / kRbE, ee = q % kRbE;
      sdl[tq][ee] = (t0 + tq < T && e0 + ee < E) ? dl[(t0 + tq) * E + e0 + ee] : 0.f;
    }
    __syncthreads();
    for (int ee = 0; ee < kRbE; ++ee) {
      const float w = sw[ee][ii];
#pragma unroll
      for (int m = 0; m < kDxTok / 4; ++m) racc[m] = fmaf(sdl[tg + 4 * m][ee], w, racc[m]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < kDxTok / 4; ++m) {
    const int64_t t = t0 + tg + 4 * m;
    if (t >= T) continue;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = assign_row[t * k + j];
      if (r >= 0) acc += bf16_bits_to_f32(dxp[(int64_t)r * ldp + i0 + ii]);
    }
    if (has_shared) acc += bf16_bits_to_f32(dxp[(rows + t) * ldp + i0 + ii]);
    dx[t * h + i0 + ii] = f32_to_bf16_bits(acc + racc[m]);
  }
}

}  // namespace

hipError_t launch_transpose(const void* src, int64_t src_bs, int R, int Cc, void* dst,
                            int64_t dst_bs, int dld, int col0, int batches, hipStream_t s) {
  hipLaunchKernelGGL(transpose_kernel, dim3(Cc / kTr, R / kTr, batches), dim3(256), 0, s,
                     (const uint16_t*)src, src_bs, R, Cc, (uint16_t*)dst, dst_bs, dld, col0);
  return hipGetLastError();
}

hipError_t launch_ktab(const int32_t* gtab, int G, int use_a_rows, int32_t* kt, hipStream_t s) {
  hipLaunchKernelGGL(ktab_kernel, dim3(1), dim3(1024), 0, s, gtab, G, use_a_rows, kt);
  return hipGetLastError();
}

hipError_t launch_transpose_groups(const void* src, int sld, const void* src_shared,
                                   int sld_shared, int E_routed, const int32_t* kt, int G,
                                   int Cc, int64_t ktot_bound, void* dst, int dld,
                                   hipStream_t s) {
  const dim3 grid(Cc / kTr, (unsigned)((ktot_bound + kTr - 1) / kTr));
  hipLaunchKernelGGL(transpose_groups_kernel, grid, dim3(256), 0, s, (const uint16_t*)src, sld,
                     (const uint16_t*)src_shared, sld_shared, E_routed, kt, G, Cc,
                     (uint16_t*)dst, dld);
  return hipGetLastError();
}

hipError_t launch_scatter_dy(const void* dy, const int32_t* assign_row, const float* gate,
                             const int32_t* counts, int64_t T, int h, int E, int k, int64_t C,
                             int64_t rows, int has_shared, void* dO, int ld, hipStream_t s) {
  const int64_t ntb = (T + kRowTok - 1) / kRowTok;
  const int64_t nb = ntb + (C > 0 ? 256 : 0);
  hipLaunchKernelGGL(scatter_dy_kernel, dim3((unsigned)nb), dim3(256), 0, s, (const uint4*)dy,
                     assign_row, gate, counts, T, h / 8, E, k, C, rows, has_shared, ntb,
                     (uint4*)dO, (int64_t)ld / 8);
  return hipGetLastError();
}

hipError_t launch_gate_grad(const void* dy, const void* o, int ld, const int32_t* assign_row,
                            int64_t T, int h, int k, float* dg, hipStream_t s) {
  hipLaunchKernelGGL(gate_grad_kernel, dim3((unsigned)T), dim3(256), 0, s, (const uint4*)dy,
                     (const uint4*)o, (int64_t)ld / 8, assign_row, h / 8, k, dg);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const void* a13, int lda13, int64_t rows, int F, void* u, int ldu,
                             hipStream_t s) {
  const int64_t n = rows * (F / 8);
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const uint4*)a13, (int64_t)lda13 / 8, rows, F / 8, (uint4*)u,
                     (int64_t)ldu / 8);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* a13, int lda13, const void* dU, int ldu, int64_t rows,
                             int F, void* dA, int ldda, hipStream_t s) {
  const int64_t n = rows * (F / 8);
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const uint4*)a13, (int64_t)lda13 / 8, (const uint4*)dU, (int64_t)ldu / 8,
                     rows, F / 8, (uint4*)dA, (int64_t)ldda / 8);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* logits, const int32_t* idx, const float* gate,
                             const float* dg, int gate_mode, int64_t T, int E, int k,
                             const void* x, int h, float* dl, float* rpart, void* dw_router,
                             float* dlogit_bias, hipStream_t s) {
  hipLaunchKernelGGL(gates_bwd_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s,
                     logits, idx, gate, dg, gate_mode, T, E, k, dl);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (dw_router) {
    const int64_t tc = ((T + kRbSlices - 1) / kRbSlices + 63) / 64 * 64;   // tokens per slice
    const int slices = (int)((T + tc - 1) / tc);
    hipLaunchKernelGGL(router_wgrad_kernel, dim3(h / 64, (E + kRbE - 1) / kRbE, slices),
                       dim3(256), 0, s, dl, (const uint16_t*)x, T, h, E, tc, rpart);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t n = (int64_t)E * h;
    hipLaunchKernelGGL(router_wgrad_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       s, rpart, slices, n, (uint16_t*)dw_router);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (dlogit_bias) {
    hipLaunchKernelGGL(bias_grad_kernel, dim3(E), dim3(256), 0, s, dl, T, E, dlogit_bias);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_dx_final(const void* dxp, int ldp, const int32_t* assign_row, int k,
                           int64_t rows, int has_shared, const float* dl, const void* w_router,
                           int64_t T, int h, int E, void* dx, hipStream_t s) {
  hipLaunchKernelGGL(dx_final_kernel, dim3(h / 64, (unsigned)((T + kDxTok - 1) / kDxTok)),
                     dim3(256), 0, s,
                     (const uint16_t*)dxp, (int64_t)ldp, assign_row, k, rows, has_shared, dl,
                     (const uint16_t*)w_router, T, h, E, (uint16_t*)dx);
  return hipGetLastError();
}

}  // namespace moe
