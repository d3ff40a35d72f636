// Grouped GEMMs of the expert SwiGLU FFN.
//
// infra-l7, section "MoE:参数很多": every expert is the SwiGLU FFN h -> F -> h
// with three matrices; "自测": tokens sorted by expert go through one grouped
// GEMM.  Megatron-LM part 6, "MoE 层的数据流": experts run as a GroupedGEMM.
//
//   GEMM 1 (+SwiGLU): act[r,f]  = silu(A[r]·w1[e,f]) * (A[r]·w3[e,f])
//   GEMM 2:           out[r,i]  = act[r]·w2[e,i]
//
// Every operand is K-contiguous (weights stored [out,in]), so both GEMMs are
// C = A · B^T with 16-byte loads along K for A and B alike.
//
// bf16 kernel (gfx950): 256 threads = 4 waves in a 2x2 grid, a 256x256
// output tile per workgroup (BK = 64), each wave a 128x128 sub-tile held as
// 4x4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per lane).  A and B
// tiles are staged through LDS in two 64 KiB stages (double buffering):
// while the MFMAs consume one stage, the next K slice is loaded into
// registers and written to the other stage.  Rows are 128 B; the 16-byte
// chunk c of row r is stored at chunk c ^ (r & 7), so the 8 lanes that an
// LDS access services together touch 8 different bank groups, for both the
// row-wise stores and the column-of-rows MFMA operand reads.
//
// For GEMM 1 the 256 B rows of a tile are [w1 f0..f0+63 | w3 f0..f0+63 |
// w1 f0+64..f0+127 | w3 f0+64..f0+127]: each wave's 128 columns hold 64 w1
// columns and the matching 64 w3 columns, so silu(a1) * a3 is formed in
// registers and a tile writes 128 activation columns.
//
// Tiles: each group (expert) has ceil(rows/256) row tiles; the scan kernel
// writes their prefix.  Logical tile L walks (group, column tile, row tile)
// with the row tile fastest, so the workgroups running together share the
// same few weight column tiles and token row tiles.  Workgroup b runs on
// XCD b % 8; consecutive logical tiles are handed to the same XCD so that
// they share its L2.  Workgroups past the real tile count exit at once.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM_bf16, BN = 256, BK = 64;
constexpr int kHalf = BM * BK * 2;         // bytes of the A (or B) stage part
constexpr int kStage = 2 * kHalf;          // 64 KiB

// Largest g with mtp[g] * NT <= L (mtp non-decreasing, mtp[0] = 0,
// mtp[G] * NT > L).
__device__ __forceinline__ int find_group(const int32_t* mtp, int G, int64_t L,
                                          int NT) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)mtp[mid] * NT <= L)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

struct Tile {
  int g, mt, nt, m_valid;
  int64_t a_row, o_row;
};

__device__ __forceinline__ bool map_tile(const GroupedGemmArgs& a, int NT,
                                         int64_t b, bool xcd_remap, int BMx,
                                         Tile& t) {
  const int G = a.G;
  const int32_t* gt = a.gtab;
  const int64_t V = (int64_t)gt[G] * NT;
  if (b >= V) return false;
  int64_t L = b;
  if (xcd_remap) {
    const int64_t x = b & 7, q = V >> 3, r = V & 7;
    L = x * q + (x < r ? x : r) + (b >> 3);
  }
  const int g = find_group(gt, G, L, NT);
  const int me = gt[g + 1] - gt[g];
  const int64_t local = L - (int64_t)gt[g] * NT;
  t.g = g;
  t.nt = (int)(local / me);
  t.mt = (int)(local - (int64_t)t.nt * me);
  const int valid = gt[2 * G + 1 + g];
  t.m_valid = min(BMx, valid - t.mt * BMx);
  t.o_row = (int64_t)gt[3 * G + 1 + g] + (int64_t)t.mt * BMx;
  t.a_row = a.a_from_out_rows ? t.o_row : (int64_t)gt[G + 1 + g] + (int64_t)t.mt * BMx;
  return true;
}

template <bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GroupedGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  const int NT = SWIGLU ? a.N / 128 : (a.N + BN - 1) / BN;
  Tile tl;
  if (!map_tile(a, NT, blockIdx.x, true, BM, tl)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int K = a.K, N = a.N;
  const bool shared = tl.g >= a.E_routed;
  const uint16_t* A = (const uint16_t*)((shared && !a.a_from_out_rows) ? a.A_shared : a.A);
  const uint16_t* B0 = (const uint16_t*)(shared ? a.B0s : a.B0);
  const uint16_t* B1 = (const uint16_t*)(shared ? a.B1s : a.B1);
  if (!shared) {
    B0 += (int64_t)tl.g * a.b_stride;
    if (SWIGLU) B1 += (int64_t)tl.g * a.b_stride;
  }

  // Global -> register -> LDS copy: thread covers chunk (tid & 7) of rows
  // j*32 + (tid >> 3), j = 0..7, of both the A and the B tile.
  const int lrow = tid >> 3, lch = tid & 7;
  const uint16_t* asrc[8];
  const uint16_t* bsrc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = j * 32 + lrow;
    const int ar = row < tl.m_valid ? row : tl.m_valid - 1;
    asrc[j] = A + (tl.a_row + ar) * K + lch * 8;
    if (SWIGLU) {
      const int blk = j >> 1;  // 64-row blocks: w1, w3, w1, w3
      const uint16_t* W = (blk & 1) ? B1 : B0;
      const int64_t wrow = (int64_t)tl.nt * 128 + (blk >> 1) * 64 + (row & 63);
      bsrc[j] = W + wrow * K + lch * 8;
    } else {
      int64_t wrow = (int64_t)tl.nt * BN + row;
      if (wrow > N - 1) wrow = N - 1;
      bsrc[j] = B0 + wrow * K + lch * 8;
    }
  }
  const int st_off = lrow * 128 + ((lch ^ (lrow & 7)) << 4);

  // MFMA operand reads: lane l reads row (l & 31) of a 32-row fragment and
  // the 16-byte chunk 2*s + (l >> 5) of K sub-step s.
  const int rA = wm * (128 * 128) + (lane & 31) * 128;
  const int rB = kHalf + wn * (128 * 128) + (lane & 31) * 128;
  int cx[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) cx[s] = ((2 * s + (lane >> 5)) ^ (lane & 7)) << 4;

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[8], rb[8];
  const int nk = K / BK;

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ra[j] = ld16(asrc[j]);
    rb[j] = ld16(bsrc[j]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    *reinterpret_cast<uint4*>(smem + j * 4096 + st_off) = ra[j];
    *reinterpret_cast<uint4*>(smem + kHalf + j * 4096 + st_off) = rb[j];
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = (kt + 1) * BK;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ra[j] = ld16(asrc[j] + k0);
        rb[j] = ld16(bsrc[j] + k0);
      }
    }
    const uint8_t* sb = smem + cur * kStage;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(sb + rA + i * 4096 + cx[s]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(sb + rB + j * 4096 + cx[s]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      uint8_t* sn = smem + (cur ^ 1) * kStage;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        *reinterpret_cast<uint4*>(sn + j * 4096 + st_off) = ra[j];
        *reinterpret_cast<uint4*>(sn + kHalf + j * 4096 + st_off) = rb[j];
      }
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: lane l holds column (l & 31); register r of a
  // fragment is row 8*(r/4) + 4*(l/32) + r%4.
  uint16_t* out = (uint16_t*)a.out;
  const int col_l = lane & 31;
  const int row_l = 4 * (lane >> 5);
  if (SWIGLU) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = (int64_t)tl.nt * 128 + wn * 64 + j * 32 + col_l;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 128 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
          if (row < tl.m_valid) {
            const float z = acc[i][j][r];
            const float v = z / (1.f + __expf(-z)) * acc[i][j + 2][r];
            out[(tl.o_row + row) * N + col] = f32_to_bf16_bits(v);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = (int64_t)tl.nt * BN + wn * 128 + j * 32 + col_l;
        if (col < N) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wm * 128 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
            if (row < tl.m_valid)
              out[(tl.o_row + row) * N + col] = f32_to_bf16_bits(acc[i][j][r]);
          }
        }
      }
  }
}

// fp32 layers: 64x64 tiles, BK = 16, fp32 FMA, each thread 4 rows x 4
// columns (columns strided by 16 for conflict-free LDS reads).
constexpr int FBM = kGemmBM_f32, FBN = 64, FBK = 16;

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GroupedGemmArgs a) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];
  __shared__ float B3s[SWIGLU ? FBK : 1][FBN + 4];

  const int NT = a.N / FBN;
  Tile tl;
  if (!map_tile(a, NT, blockIdx.x, false, FBM, tl)) return;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int K = a.K, N = a.N;
  const bool shared = tl.g >= a.E_routed;
  const float* A = (const float*)((shared && !a.a_from_out_rows) ? a.A_shared : a.A);
  const float* B0 = (const float*)(shared ? a.B0s : a.B0);
  const float* B1 = (const float*)(shared ? a.B1s : a.B1);
  if (!shared) {
    B0 += (int64_t)tl.g * a.b_stride;
    if (SWIGLU) B1 += (int64_t)tl.g * a.b_stride;
  }
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int ar = lr < tl.m_valid ? lr : tl.m_valid - 1;
  const float* ap = A + (tl.a_row + ar) * K + lk;
  const int64_t n0 = (int64_t)tl.nt * FBN;
  const float* bp = B0 + (n0 + lr) * K + lk;
  const float* b3p = SWIGLU ? B1 + (n0 + lr) * K + lk : nullptr;

  float acc[4][4], acc3[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = acc3[i][c] = 0.f;

  for (int k0 = 0; k0 < K; k0 += FBK) {
    const float4 av = *reinterpret_cast<const float4*>(ap + k0);
    const float4 bv = *reinterpret_cast<const float4*>(bp + k0);
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    if (SWIGLU) {
      const float4 cv = *reinterpret_cast<const float4*>(b3p + k0);
      B3s[lk + 0][lr] = cv.x; B3s[lk + 1][lr] = cv.y; B3s[lk + 2][lr] = cv.z; B3s[lk + 3][lr] = cv.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float av4[4], bv4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av4[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv4[c] = Bs[kk][tx + 16 * c];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = fmaf(av4[i], bv4[c], acc[i][c]);
      if (SWIGLU) {
#pragma unroll
        for (int c = 0; c < 4; ++c) bv4[c] = B3s[kk][tx + 16 * c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc3[i][c] = fmaf(av4[i], bv4[c], acc3[i][c]);
      }
    }
    __syncthreads();
  }
  float* out = (float*)a.out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= tl.m_valid) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t col = n0 + tx + 16 * c;
      float v = acc[i][c];
      if (SWIGLU) v = v / (1.f + expf(-v)) * acc3[i][c];
      out[(tl.o_row + row) * N + col] = v;
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm(int dtype, bool swiglu, const GroupedGemmArgs& a,
                               hipStream_t s) {
  if (dtype == 1) {
    const int NT = swiglu ? a.N / 128 : (a.N + BN - 1) / BN;
    const int64_t nb = a.max_m_tiles * NT;
    if (nb <= 0) return hipSuccess;
    if (swiglu)
      hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, a);
  } else {
    const int NT = a.N / FBN;
    const int64_t nb = a.max_m_tiles * NT;
    if (nb <= 0) return hipSuccess;
    if (swiglu)
      hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
