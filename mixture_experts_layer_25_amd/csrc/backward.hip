// Backward of the MoE layer: the kernels around the grouped GEMMs.  Every
// row kernel is a template over the element type T of the layer's tensors
// (uint16_t bf16 bits or float), 16-byte vectors of Elt<T>::kVec elements;
// the arithmetic is fp32 in both cases.
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
// 64 x 64 element tiles through LDS (rows padded by one 4-byte word against
// bank conflicts); 16-byte loads and stores.
constexpr int kTr = 64;

// dst[b][c][col0 + r] = src[b][r][c] for r < R, c < Cc (R, Cc multiples of
// 64; dense src rows of Cc).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int64_t src_bs,
                                                        int R, int Cc, T* __restrict__ dst,
                                                        int64_t dst_bs, int dld, int col0) {
  constexpr int V = Elt<T>::kVec, NV = kTr / V;
  __shared__ T tile[kTr][kTr + 4 / sizeof(T)];
  const int b = blockIdx.z;
  const int c0 = blockIdx.x * kTr, r0 = blockIdx.y * kTr;
  const T* s = src + b * src_bs;
  T* d = dst + b * dst_bs;
  for (int q = threadIdx.x; q < kTr * NV; q += 256) {
    const int rr = q / NV, cv = (q % NV) * V;
    const uint4 v = ld16(s + (int64_t)(r0 + rr) * Cc + c0 + cv);
    T el[V];
    __builtin_memcpy(el, &v, 16);
#pragma unroll
    for (int e = 0; e < V; ++e) tile[rr][cv + e] = el[e];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kTr * NV; q += 256) {
    const int cc = q / NV, rv = (q % NV) * V;
    T el[V];
#pragma unroll
    for (int e = 0; e < V; ++e) el[e] = tile[rv + e][cc];
    uint4 v;
    __builtin_memcpy(&v, el, 16);
    st16(d + (int64_t)(c0 + cc) * dld + col0 + r0 + rv, v);
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
template <typename T>
__global__ __launch_bounds__(256) void transpose_groups_kernel(
    const T* __restrict__ src, int sld, const T* __restrict__ src_shared, int sld_shared,
    int E_routed, const int32_t* __restrict__ kt, int G, int Cc, T* __restrict__ dst, int dld) {
  constexpr int V = Elt<T>::kVec, NV = kTr / V;
  __shared__ T tile[kTr][kTr + 4 / sizeof(T)];
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
  const T* s = sh ? src_shared : src;
  const int ld = sh ? sld_shared : sld;
  const int c0 = blockIdx.x * kTr;
  for (int q = threadIdx.x; q < kTr * NV; q += 256) {
    const int rr = q / NV, cv = (q % NV) * V;
    const int64_t kr = k0 + rr - koff;          // row within the group
    uint4 v = uint4{0u, 0u, 0u, 0u};
    if (kr < n) v = ld16(s + (r0 + kr) * ld + c0 + cv);
    T el[V];
    __builtin_memcpy(el, &v, 16);
#pragma unroll
    for (int e = 0; e < V; ++e) tile[rr][cv + e] = el[e];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kTr * NV; q += 256) {
    const int cc = q / NV, rv = (q % NV) * V;
    T el[V];
#pragma unroll
    for (int e = 0; e < V; ++e) el[e] = tile[rv + e][cc];
    uint4 v;
    __builtin_memcpy(&v, el, 16);
    st16(dst + (int64_t)(c0 + cc) * dld + k0 + rv, v);
  }
}

// ------------------------------------------------------------ row kernels
constexpr int kRowTok = 2;

// dO rows: routed row assign_row[t,j] = g[t,j] dy[t] (rounded to T); shared
// row rows + t = dy[t]; then (capacity) padding rows zero, like the permute.
// nv, pv: 16-byte vectors per row of dy and of dO.
template <typename T>
__global__ __launch_bounds__(256) void scatter_dy_kernel(
    const uint4* __restrict__ dy, const int32_t* __restrict__ assign_row,
    const float* __restrict__ gate, const int32_t* __restrict__ counts, int64_t T_, int nv, int E,
    int k, int64_t C, int64_t rows, int has_shared, int64_t ntb, uint4* __restrict__ dO,
    int64_t pv) {
  constexpr int V = Elt<T>::kVec;
  const int64_t b = blockIdx.x;
  if (b < ntb) {
    for (int tt = 0; tt < kRowTok; ++tt) {
      const int64_t t = b * kRowTok + tt;
      if (t >= T_) return;
      for (int v = threadIdx.x; v < nv; v += 256) {
        const uint4 q = dy[t * nv + v];
        float f[V];
        Elt<T>::unpack(q, f);
        for (int j = 0; j < k; ++j) {
          const int r = assign_row[t * k + j];
          if (r < 0 || r >= rows) continue;   // dropped (or outside the rows)
          const float g = gate[t * k + j];
          float o[V];
#pragma unroll
          for (int e = 0; e < V; ++e) o[e] = g * f[e];
          dO[(int64_t)r * pv + v] = Elt<T>::pack(o);
        }
        if (has_shared) dO[(rows + t) * pv + v] = q;
      }
    }
    return;
  }
  const int64_t pb = b - ntb;
  for (int e = 0; e < E; ++e) {
    const int64_t kept = max(min((int64_t)counts[e], C), (int64_t)0);
    for (int64_t r = e * C + kept + pb; r < (e + 1) * C; r += 256) {
      for (int v = threadIdx.x; v < nv; v += 256) dO[r * pv + v] = uint4{0u, 0u, 0u, 0u};
    }
  }
}

// dg[t,j] = dy[t] . o[assign_row[t,j]] (0 for a dropped slot): one
// workgroup per token, per-thread fp32 partial sums, then a fixed tree.
template <typename T>
__global__ __launch_bounds__(256) void gate_grad_kernel(const uint4* __restrict__ dy,
                                                        const uint4* __restrict__ o, int64_t pv,
                                                        const int32_t* __restrict__ assign_row,
                                                        int64_t rows, int nv, int k,
                                                        float* __restrict__ dg) {
  constexpr int V = Elt<T>::kVec;
  __shared__ float red[256];
  const int64_t t = blockIdx.x;
  for (int j = 0; j < k; ++j) {
    const int r = assign_row[t * k + j];
    float acc = 0.f;
    if (r >= 0 && r < rows) {
      for (int v = threadIdx.x; v < nv; v += 256) {
        float fa[V], fb[V];
        Elt<T>::unpack(dy[t * nv + v], fa);
        Elt<T>::unpack(o[(int64_t)r * pv + v], fb);
#pragma unroll
        for (int e = 0; e < V; ++e) acc = fmaf(fa[e], fb[e], acc);
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

// u = silu(a1) * a3 from a13 = [a1 | a3] (rows x 2F), one 16-byte vector
// per thread; fv = vectors per F columns, strides in vectors.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint4* __restrict__ a13,
                                                         int64_t lda13, int64_t rows, int fv,
                                                         uint4* __restrict__ u, int64_t ldu) {
  constexpr int V = Elt<T>::kVec;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= rows * fv) return;
  const int64_t r = q / fv;
  const int v = (int)(q - r * fv);
  float a[V], c[V], o[V];
  Elt<T>::unpack(a13[r * lda13 + v], a);
  Elt<T>::unpack(a13[r * lda13 + fv + v], c);
#pragma unroll
  for (int e = 0; e < V; ++e) o[e] = a[e] * sigmoidf_(a[e]) * c[e];
  u[r * ldu + v] = Elt<T>::pack(o);
}

// dA = [dU a3 s (1 + a1 (1 - s)) | dU a1 s], s = sigmoid(a1).
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint4* __restrict__ a13,
                                                         int64_t lda13,
                                                         const uint4* __restrict__ dU,
                                                         int64_t ldu, int64_t rows, int fv,
                                                         uint4* __restrict__ dA, int64_t ldda) {
  constexpr int V = Elt<T>::kVec;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= rows * fv) return;
  const int64_t r = q / fv;
  const int v = (int)(q - r * fv);
  float a[V], c[V], d[V], r1[V], r3[V];
  Elt<T>::unpack(a13[r * lda13 + v], a);
  Elt<T>::unpack(a13[r * lda13 + fv + v], c);
  Elt<T>::unpack(dU[r * ldu + v], d);
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const float s = sigmoidf_(a[e]);
    r1[e] = d[e] * c[e] * s * (1.f + a[e] * (1.f - s));
    r3[e] = d[e] * a[e] * s;
  }
  dA[r * ldda + v] = Elt<T>::pack(r1);
  dA[r * ldda + fv + v] = Elt<T>::pack(r3);
}

// dl[t,:] from dg[t,:] for the gate modes (one thread per token; fp32).
// idx NULL: slot j is expert j (expert choice, k = E slots, the gate of an
// unchosen slot 0), with mode 1 for the softmax over all E and mode 2 for
// the sigmoids normalised over all E.
//
// With dl_hl, dl also as bf16 parts: hi = bf16(dl), lo = bf16(dl - hi), in
// dl_hl[t][e] / dl_hl[t][Ep + e] and dlT_hl[e][t] / dlT_hl[e][Tp + t], zero
// for e >= E and (dlT_hl) T <= t < Tp.
__global__ __launch_bounds__(256) void gates_bwd_kernel(const float* __restrict__ logits,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ gate,
                                                        const float* __restrict__ dg,
                                                        int gate_mode, int64_t T, int E, int k,
                                                        float* __restrict__ dl,
                                                        uint16_t* __restrict__ dl_hl, int Ep,
                                                        uint16_t* __restrict__ dlT_hl,
                                                        int64_t Tp) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) {
    if (dl_hl && t < Tp)
      for (int e = 0; e < Ep; ++e) {
        dlT_hl[(int64_t)e * 2 * Tp + t] = 0;
        dlT_hl[(int64_t)e * 2 * Tp + Tp + t] = 0;
      }
    return;
  }
  const float* l = logits + t * E;
  float* d = dl + t * E;
  // a slot whose expert id is outside [0, E) (a caller's map) is ignored
  auto ex = [&](int j) { return idx ? idx[t * k + j] : j; };
  auto ok = [&](int j) { return (unsigned)ex(j) < (unsigned)E; };
  for (int e = 0; e < E; ++e) d[e] = 0.f;
  float gd = 0.f;                     // sum_j g_j dg_j
  for (int j = 0; j < k; ++j)
    if (ok(j)) gd += gate[t * k + j] * dg[t * k + j];
  if (gate_mode == 0) {               // softmax over the selected
    for (int j = 0; j < k; ++j) {
      if (!ok(j)) continue;
      const float g = gate[t * k + j];
      d[ex(j)] += g * (dg[t * k + j] - gd);
    }
  } else if (gate_mode == 1) {        // softmax over all E, selected values
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmaxf(m, l[e]);
    float den = 0.f;
    for (int e = 0; e < E; ++e) den += expf(l[e] - m);
    for (int e = 0; e < E; ++e) d[e] = -(expf(l[e] - m) / den) * gd;
    for (int j = 0; j < k; ++j) {
      if (!ok(j)) continue;
      const int e = ex(j);
      d[e] += (expf(l[e] - m) / den) * dg[t * k + j];
    }
  } else {                            // sigmoid normalised over the selected
    float S = 0.f;
    for (int j = 0; j < k; ++j)
      if (ok(j)) S += 1.f / (1.f + expf(-l[ex(j)]));
    for (int j = 0; j < k; ++j) {
      if (!ok(j)) continue;
      const int e = ex(j);
      const float s = 1.f / (1.f + expf(-l[e]));
      d[e] += (dg[t * k + j] - gd) / S * s * (1.f - s);
    }
  }
  if (dl_hl) {
    for (int e = 0; e < Ep; ++e) {
      const float v = e < E ? d[e] : 0.f;
      const uint16_t hi = f32_to_bf16_bits(v);
      const uint16_t lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
      dl_hl[t * 2 * Ep + e] = hi;
      dl_hl[t * 2 * Ep + Ep + e] = lo;
      dlT_hl[(int64_t)e * 2 * Tp + t] = hi;
      dlT_hl[(int64_t)e * 2 * Tp + Tp + t] = lo;
    }
  }
}

// dl[t,:] from dg[t,:] as gates_bwd_kernel computes it, with the bf16 parts
// dl_hl / dlT_hl, for up to 256 experts: 16 tokens per workgroup, one wave
// per token at a time.  A token's slots sit in lanes (lane j: slot j's
// expert, gate and gate gradient; expert choice: lane e's experts), its sums
// are wave reductions, and the lanes then run over the experts, so dl and
// dl_hl rows are written by consecutive lanes; the parts are staged in LDS
// so that dlT_hl's token-contiguous rows are written 32 bytes at a time.
constexpr int kGbTok = 16, kGbMaxE = 256;
__global__ __launch_bounds__(256) void gates_bwd_split_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const float* __restrict__ dg, int gate_mode, int64_t T, int E,
    int k, float* __restrict__ dl, uint16_t* __restrict__ dl_hl, int Ep,
    uint16_t* __restrict__ dlT_hl, int64_t Tp) {
  __shared__ uint32_t sh[kGbMaxE][kGbTok + 1];   // hi | lo << 16
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kGbTok;
  for (int tt = w; tt < kGbTok; tt += 4) {
    const int64_t t = t0 + tt;
    if (t >= T) {
      for (int e = lane; e < Ep; e += 64) sh[e][tt] = 0u;
      continue;
    }
    const float* l = logits + t * E;
    // top-k: lane j < k holds slot j (an expert id outside [0, E) is
    // ignored); expert choice (idx NULL): slot j is expert j
    int exl = -1;
    float gl = 0.f, dgl = 0.f;
    if (idx && lane < k) {
      exl = idx[t * k + lane];
      gl = gate[t * k + lane];
      dgl = dg[t * k + lane];
      if ((unsigned)exl >= (unsigned)E) exl = -1;
    }
    float gd = 0.f, S = 0.f;   // sum_j g_j dg_j; sigmoid mode: sum_j s(l[ex(j)])
    if (idx) {
      gd = exl >= 0 ? gl * dgl : 0.f;
      if (gate_mode == 2 && exl >= 0) S = 1.f / (1.f + expf(-l[exl]));
    } else {
      for (int e = lane; e < E; e += 64) {
        gd += gate[t * k + e] * dg[t * k + e];
        if (gate_mode == 2) S += 1.f / (1.f + expf(-l[e]));
      }
    }
    gd = seg_sum_f32<64>(gd);
    if (gate_mode == 2) S = seg_sum_f32<64>(S);
    float m = -INFINITY, den = 0.f;
    if (gate_mode == 1) {
      for (int e = lane; e < E; e += 64) m = fmaxf(m, l[e]);
      m = seg_max_f32<64>(m);
      for (int e = lane; e < E; e += 64) den += expf(l[e] - m);
      den = seg_sum_f32<64>(den);
    }
    auto term = [&](int e, float g, float dgj) {
      if (gate_mode == 0) return g * (dgj - gd);
      if (gate_mode == 1) return (expf(l[e] - m) / den) * dgj;
      const float sg = 1.f / (1.f + expf(-l[e]));
      return (dgj - gd) / S * sg * (1.f - sg);
    };
    for (int e0 = 0; e0 < Ep; e0 += 64) {
      const int e = e0 + lane;
      float d = 0.f;
      if (e < E && gate_mode == 1) d = -(expf(l[e] - m) / den) * gd;
      if (idx) {
        for (int j = 0; j < k; ++j) {   // slots in order
          const int ej = __shfl(exl, j, 64);
          const float gj = __shfl(gl, j, 64), dj = __shfl(dgl, j, 64);
          if (ej == e) d += term(e, gj, dj);
        }
      } else if (e < E) {
        d += term(e, gate[t * k + e], dg[t * k + e]);
      }
      if (e < E) dl[t * E + e] = d;
      if (e < Ep) {
        const uint16_t hi = f32_to_bf16_bits(d);
        const uint16_t lo = f32_to_bf16_bits(d - bf16_bits_to_f32(hi));
        dl_hl[t * 2 * Ep + e] = hi;
        dl_hl[t * 2 * Ep + Ep + e] = lo;
        sh[e][tt] = (uint32_t)hi | ((uint32_t)lo << 16);
      }
    }
  }
  __syncthreads();
  // 16 lanes per expert row (its 16 tokens), 16 rows at a time
  const int tl = threadIdx.x & 15, er = threadIdx.x >> 4;
  const int64_t t = t0 + tl;
  if (t < Tp)
    for (int e = er; e < Ep; e += 16) {
      const uint32_t v = sh[e][tl];
      dlT_hl[(int64_t)e * 2 * Tp + t] = (uint16_t)(v & 0xFFFFu);
      dlT_hl[(int64_t)e * 2 * Tp + Tp + t] = (uint16_t)(v >> 16);
    }
}

// Tile table (4G + 1 ints, G = 1) of one group of `rows` rows: its row
// tiles, first A row 0, its rows, first output row 0; its claim blocks
// zeroed.  One workgroup of 256 threads.
__global__ void single_group_gtab_kernel(int32_t* gt, int64_t rows, int BM) {
  for (int i = threadIdx.x; i < kClaimBlocks * kClaimBlockInts; i += 256)
    gt[gtab_claims_off(1) + i] = 0;
  if (threadIdx.x == 0) {
    gt[0] = 0;
    gt[1] = (int32_t)((rows + BM - 1) / BM);
    gt[2] = 0;
    gt[3] = (int32_t)rows;
    gt[4] = 0;
  }
}

// dW_router[e, i] = sum_t dl[t,e] x[t,i]: workgroup (column tile, 32
// experts, token slice z) sums its slice of tokens in order (64 at a time
// through LDS) into part[z][e][i] (fp32); router_wgrad_sum adds the
// slices in order and rounds to the element type.
constexpr int kRbE = 32;
constexpr int kRbSlices = 32;
template <typename T>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float* __restrict__ dl,
                                                           const T* __restrict__ x,
                                                           int64_t T_, int h, int E, int64_t tc,
                                                           float* __restrict__ part) {
  __shared__ float sdl[64][kRbE];
  __shared__ float sx[64][64];
  const int i0 = blockIdx.x * 64, e0 = blockIdx.y * kRbE;
  const int64_t tb = (int64_t)blockIdx.z * tc, te = min(T_, tb + tc);
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
      sx[tt][c] = t0 + tt < te ? Elt<T>::ld(x + (t0 + tt) * h + i0 + c) : 0.f;
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

template <typename T>
__global__ __launch_bounds__(256) void router_wgrad_sum_kernel(const float* __restrict__ part,
                                                               int slices, int64_t n,
                                                               T* __restrict__ dwr) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n) return;
  float s = 0.f;
  for (int z = 0; z < slices; ++z) s += part[z * n + q];
  Elt<T>::st(dwr + q, s);
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

// dx[t] = round( sum_j dxp[assign_row[t,j]] (slot order) + dxp[rows + t]
// (shared) + sum_e dl[t,e] W_router[e] ); 64 columns x 32 tokens per
// workgroup (8 tokens per thread), the router term over experts in order
// through LDS, so W_router is read once per 32 tokens.
constexpr int kDxTok = 32;
template <typename T>
__global__ __launch_bounds__(256) void dx_final_kernel(
    const T* __restrict__ dxp, int64_t ldp, const int32_t* __restrict__ assign_row, int k,
    int64_t rows, int has_shared, const float* __restrict__ dl, const T* __restrict__ wr,
    int64_t T_, int h, int E, T* __restrict__ dx) {
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
      sw[ee][c] = e0 + ee < E ? Elt<T>::ld(wr + (int64_t)(e0 + ee) * h + i0 + c) : 0.f;
    }
    for (int q = threadIdx.x; q < kDxTok * kRbE; q += 256) {
      const int tq = q / kRbE, ee = q % kRbE;
      sdl[tq][ee] = (t0 + tq < T_ && e0 + ee < E) ? dl[(t0 + tq) * E + e0 + ee] : 0.f;
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
    if (t >= T_) continue;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = assign_row[t * k + j];
      if (r >= 0 && r < rows) acc += Elt<T>::ld(dxp + (int64_t)r * ldp + i0 + ii);
    }
    if (has_shared) acc += Elt<T>::ld(dxp + (rows + t) * ldp + i0 + ii);
    Elt<T>::st(dx + t * h + i0 + ii, acc + racc[m]);
  }
}

}  // namespace

namespace {
// 16-byte vectors per element of dtype (1: bf16, else fp32).
inline int vec_of(int dtype) { return dtype == 1 ? 8 : 4; }
}  // namespace

// Launches KERNEL<uint16_t> for bf16 (dtype 1), KERNEL<float> otherwise.
#define MOE_BY_DTYPE(DT, KERNEL, GRID, ...)                                         \
  do {                                                                              \
    if ((DT) == 1)                                                                  \
      MOE_LAUNCH(KERNEL<uint16_t>, GRID, dim3(256), 0, s, __VA_ARGS__);     \
    else                                                                            \
      MOE_LAUNCH(KERNEL<float>, GRID, dim3(256), 0, s, __VA_ARGS__);        \
  } while (0)

hipError_t launch_transpose(int dtype, const void* src, int64_t src_bs, int R, int Cc, void* dst,
                            int64_t dst_bs, int dld, int col0, int batches, hipStream_t s) {
  const dim3 grid(Cc / kTr, R / kTr, batches);
  if (dtype == 1)
    MOE_LAUNCH(transpose_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)src,
                       src_bs, R, Cc, (uint16_t*)dst, dst_bs, dld, col0);
  else
    MOE_LAUNCH(transpose_kernel<float>, grid, dim3(256), 0, s, (const float*)src, src_bs,
                       R, Cc, (float*)dst, dst_bs, dld, col0);
  return hipGetLastError();
}

hipError_t launch_ktab(const int32_t* gtab, int G, int use_a_rows, int32_t* kt, hipStream_t s) {
  MOE_LAUNCH(ktab_kernel, dim3(1), dim3(1024), 0, s, gtab, G, use_a_rows, kt);
  return hipGetLastError();
}

hipError_t launch_transpose_groups(int dtype, const void* src, int sld, const void* src_shared,
                                   int sld_shared, int E_routed, const int32_t* kt, int G,
                                   int Cc, int64_t ktot_bound, void* dst, int dld,
                                   hipStream_t s) {
  const dim3 grid(Cc / kTr, (unsigned)((ktot_bound + kTr - 1) / kTr));
  if (dtype == 1)
    MOE_LAUNCH(transpose_groups_kernel<uint16_t>, grid, dim3(256), 0, s,
                       (const uint16_t*)src, sld, (const uint16_t*)src_shared, sld_shared,
                       E_routed, kt, G, Cc, (uint16_t*)dst, dld);
  else
    MOE_LAUNCH(transpose_groups_kernel<float>, grid, dim3(256), 0, s, (const float*)src,
                       sld, (const float*)src_shared, sld_shared, E_routed, kt, G, Cc,
                       (float*)dst, dld);
  return hipGetLastError();
}

hipError_t launch_scatter_dy(int dtype, const void* dy, const int32_t* assign_row,
                             const float* gate, const int32_t* counts, int64_t T, int h, int E,
                             int k, int64_t C, int64_t rows, int has_shared, void* dO, int ld,
                             hipStream_t s) {
  const int64_t ntb = (T + kRowTok - 1) / kRowTok;
  const int64_t nb = ntb + (C > 0 ? 256 : 0);
  const int V = vec_of(dtype);
  MOE_BY_DTYPE(dtype, scatter_dy_kernel, dim3((unsigned)nb), (const uint4*)dy, assign_row, gate,
               counts, T, h / V, E, k, C, rows, has_shared, ntb, (uint4*)dO, (int64_t)ld / V);
  return hipGetLastError();
}

hipError_t launch_gate_grad(int dtype, const void* dy, const void* o, int ld,
                            const int32_t* assign_row, int64_t rows, int64_t T, int h, int k,
                            float* dg, hipStream_t s) {
  const int V = vec_of(dtype);
  MOE_BY_DTYPE(dtype, gate_grad_kernel, dim3((unsigned)T), (const uint4*)dy, (const uint4*)o,
               (int64_t)ld / V, assign_row, rows, h / V, k, dg);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(int dtype, const void* a13, int lda13, int64_t rows, int F, void* u,
                             int ldu, hipStream_t s) {
  const int V = vec_of(dtype);
  const int64_t n = rows * (F / V);
  MOE_BY_DTYPE(dtype, swiglu_fwd_kernel, dim3((unsigned)((n + 255) / 256)), (const uint4*)a13,
               (int64_t)lda13 / V, rows, F / V, (uint4*)u, (int64_t)ldu / V);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int dtype, const void* a13, int lda13, const void* dU, int ldu,
                             int64_t rows, int F, void* dA, int ldda, hipStream_t s) {
  const int V = vec_of(dtype);
  const int64_t n = rows * (F / V);
  MOE_BY_DTYPE(dtype, swiglu_bwd_kernel, dim3((unsigned)((n + 255) / 256)), (const uint4*)a13,
               (int64_t)lda13 / V, (const uint4*)dU, (int64_t)ldu / V, rows, F / V, (uint4*)dA,
               (int64_t)ldda / V);
  return hipGetLastError();
}

hipError_t launch_router_bwd(int dtype, const float* logits, const int32_t* idx,
                             const float* gate, const float* dg, int gate_mode, int64_t T, int E,
                             int k, const void* x, int h, float* dl, float* rpart,
                             void* dw_router, float* dlogit_bias, hipStream_t s) {
  MOE_LAUNCH(gates_bwd_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s,
                     logits, idx, gate, dg, gate_mode, T, E, k, dl, (uint16_t*)nullptr, 0,
                     (uint16_t*)nullptr, (int64_t)0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (dw_router) {
    const int64_t tc = ((T + kRbSlices - 1) / kRbSlices + 63) / 64 * 64;   // tokens per slice
    const int slices = (int)((T + tc - 1) / tc);
    const dim3 grid(h / 64, (E + kRbE - 1) / kRbE, slices);
    if (dtype == 1)
      MOE_LAUNCH(router_wgrad_kernel<uint16_t>, grid, dim3(256), 0, s, dl,
                         (const uint16_t*)x, T, h, E, tc, rpart);
    else
      MOE_LAUNCH(router_wgrad_kernel<float>, grid, dim3(256), 0, s, dl, (const float*)x,
                         T, h, E, tc, rpart);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t n = (int64_t)E * h;
    const dim3 g2((unsigned)((n + 255) / 256));
    if (dtype == 1)
      MOE_LAUNCH(router_wgrad_sum_kernel<uint16_t>, g2, dim3(256), 0, s, rpart, slices, n,
                         (uint16_t*)dw_router);
    else
      MOE_LAUNCH(router_wgrad_sum_kernel<float>, g2, dim3(256), 0, s, rpart, slices, n,
                         (float*)dw_router);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (dlogit_bias) {
    MOE_LAUNCH(bias_grad_kernel, dim3(E), dim3(256), 0, s, dl, T, E, dlogit_bias);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_gates_bwd(const float* logits, const int32_t* idx, const float* gate,
                            const float* dg, int gate_mode, int64_t T, int E, int k, float* dl,
                            uint16_t* dl_hl, int Ep, uint16_t* dlT_hl, int64_t Tp,
                            hipStream_t s) {
  if (dl_hl && Ep <= kGbMaxE) {
    MOE_LAUNCH(gates_bwd_split_kernel, dim3((unsigned)(Tp / kGbTok)), dim3(256), 0, s, logits,
               idx, gate, dg, gate_mode, T, E, k, dl, dl_hl, Ep, dlT_hl, Tp);
    return hipGetLastError();
  }
  const int64_t n = dl_hl ? (T > Tp ? T : Tp) : T;
  MOE_LAUNCH(gates_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, logits, idx,
             gate, dg, gate_mode, T, E, k, dl, dl_hl, Ep, dlT_hl, Tp);
  return hipGetLastError();
}

hipError_t launch_bias_grad(const float* dl, int64_t T, int E, float* dlogit_bias,
                            hipStream_t s) {
  MOE_LAUNCH(bias_grad_kernel, dim3(E), dim3(256), 0, s, dl, T, E, dlogit_bias);
  return hipGetLastError();
}

hipError_t launch_single_group_gtab(int32_t* gtab, int64_t rows, int BM, hipStream_t s) {
  MOE_LAUNCH(single_group_gtab_kernel, dim3(1), dim3(256), 0, s, gtab, rows, BM);
  return hipGetLastError();
}

hipError_t launch_dx_final(int dtype, const void* dxp, int ldp, const int32_t* assign_row, int k,
                           int64_t rows, int has_shared, const float* dl, const void* w_router,
                           int64_t T, int h, int E, void* dx, hipStream_t s) {
  const dim3 grid(h / 64, (unsigned)((T + kDxTok - 1) / kDxTok));
  if (dtype == 1)
    MOE_LAUNCH(dx_final_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)dxp,
                       (int64_t)ldp, assign_row, k, rows, has_shared, dl,
                       (const uint16_t*)w_router, T, h, E, (uint16_t*)dx);
  else
    MOE_LAUNCH(dx_final_kernel<float>, grid, dim3(256), 0, s, (const float*)dxp,
                       (int64_t)ldp, assign_row, k, rows, has_shared, dl, (const float*)w_router,
                       T, h, E, (float*)dx);
  return hipGetLastError();
}

#undef MOE_BY_DTYPE

}  // namespace moe
