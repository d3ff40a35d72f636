// Dispatch bookkeeping and the permute copy.
//
// infra-l7, "NVIDIA 原题": dispatch groups the tokens by expert, at most C
// per group (C = cf*k*T/E, excess dropped), unused places padded, giving
// [E,C,h]; without a capacity (Megatron's default) nothing is dropped.
// "自测": a token past capacity is dropped on that expert only; sorting the
// tokens by expert lets one grouped GEMM run every expert.
//
// rank(t,j) = number of tokens t' < t that chose the same expert.  Ranks
// come from counts, never from the order atomics happen to run in:
//   hist    per group of tokens (256 here; the top-k workgroup's tokens
//           on the fused path, where the top-k kernel writes it), the
//           assignments per expert as order-free LDS counts
//   scan    one workgroup: per-expert exclusive prefix over chunks, the
//           counts, group offsets, and the grouped-GEMM tile table
//   assign  per chunk: per-wave counts, then within a wave the lanes below
//           with the same expert, found by ballots over the expert's bits
//   permute x_perm[assign_row[t,j]] = x[t], 16-byte vectors; padding rows
//           (capacity mode) are zeroed and get row_token = -1.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

// Exclusive scan over one value per thread of a 1024-thread workgroup.
// `tmp` holds at least 17 ints of LDS.  Returns the prefix, total in *tot.
__device__ int block_exclusive_scan_1024(int v, int* tmp, int* tot) {
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
    for (int i = 0; i < 16; ++i) {
      const int c = tmp[i];
      tmp[i] = run;
      run += c;
    }
    tmp[16] = run;
  }
  __syncthreads();
  const int res = tmp[w] + incl - v;
  *tot = tmp[16];
  __syncthreads();
  return res;
}

// Tile table of G groups (rows computed per group `valid`, first rows
// a_row0 / o_row0) for row tiles of BM, and its claim blocks zeroed.
// Called by all 1024 threads of the scan workgroups with g = threadIdx.x
// (G <= 1024).
__device__ void write_gtab(int g, int G, int valid, int a_row0, int o_row0,
                           int BM, int* tmp, int32_t* gtab) {
  for (int i = g; i < kClaimBlocks * kClaimBlockInts; i += 1024) gtab[gtab_claims_off(G) + i] = 0;
  const int mt = (g < G) ? (valid + BM - 1) / BM : 0;
  int tot;
  const int pre = block_exclusive_scan_1024(mt, tmp, &tot);
  if (g < G) {
    gtab[g] = pre;
    gtab[G + 1 + g] = a_row0;
    gtab[2 * G + 1 + g] = valid;
    gtab[3 * G + 1 + g] = o_row0;
  }
  if (g == 0) gtab[G] = tot;
}

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx,
                                                   int64_t T, int E, int k,
                                                   int32_t* __restrict__ chunk_hist) {
  __shared__ int32_t hist[1024];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kChunkTokens + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_hist[blockIdx.x * (int64_t)E + e] = hist[e];
}

// One workgroup of 1024 threads; hist has one row of E counts per group of
// tokens (nch groups, in token order).  Thread (sl, e) = (tid / E, tid % E)
// owns the sl-th of S contiguous slices of the groups of expert e: it sums
// its slice, the slice totals are scanned in LDS, and it writes the bases
// of its groups from its slice's prefix.
__global__ __launch_bounds__(1024) void scan_kernel(
    const int32_t* __restrict__ chunk_hist, int64_t nch, int E, int64_t C,
    int64_t T, int k, int has_shared, int BM, int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ gtab, int32_t* __restrict__ pad_row_token) {
  __shared__ int tmp[32];
  __shared__ int slice_sum[1024];
  __shared__ int kept_s[1024];
  int S = 1;
  while (2 * S * E <= 1024) S *= 2;
  const int tid = threadIdx.x;
  const int sl = tid / E, es = tid % E;
  const int64_t L = (nch + S - 1) / S;
  const int64_t g0 = sl * L, g1 = min(nch, g0 + L);
  // 16 loads in flight per thread: with many experts a slice spans dozens
  // of groups, and each batch costs one memory round trip
  if (sl < S) {
    int sum = 0;
    int64_t c = g0;
    for (; c + 16 <= g1; c += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = chunk_hist[(c + i) * E + es];
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += v[i];
    }
    for (; c < g1; ++c) sum += chunk_hist[c * E + es];
    slice_sum[tid] = sum;
  }
  __syncthreads();
  if (sl < S) {
    int run = 0;
    for (int q = 0; q < sl; ++q) run += slice_sum[q * E + es];
    int64_t c = g0;
    for (; c + 16 <= g1; c += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = chunk_hist[(c + i) * E + es];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        chunk_base[(c + i) * E + es] = run;
        run += v[i];
      }
    }
    for (; c < g1; ++c) {
      chunk_base[c * E + es] = run;
      run += chunk_hist[c * E + es];
    }
  }
  const int e = tid;
  int cnt = 0;
  if (e < E)
    for (int q = 0; q < S; ++q) cnt += slice_sum[q * E + e];
  if (e < E) counts[e] = cnt;
  int rows_routed;
  int off;
  if (C == 0) {
    int tot;
    off = block_exclusive_scan_1024(e < E ? cnt : 0, tmp, &tot);
    rows_routed = tot;  // == T*k
  } else {
    off = e * (int)C;
    rows_routed = E * (int)C;
  }
  if (e < E) offsets[e] = off;
  if (e == 0) offsets[E] = rows_routed;
  const int G = E + (has_shared ? 1 : 0);
  int valid = 0, a0 = 0, o0 = 0;
  if (e < E) {
    valid = (C == 0) ? cnt : min(cnt, (int)C);
    a0 = off;
    o0 = off;
  } else if (e == E && has_shared) {
    valid = (int)T;
    a0 = 0;                 // the shared group reads the tokens x directly
    o0 = rows_routed;       // and writes after the routed rows
  }
  write_gtab(e, G, valid, a0, o0, BM, tmp, gtab);
  // capacity layout, when no permute runs after it: the padding rows
  // e*C + kept_e .. e*C + C - 1 get row_token -1
  if (C > 0 && pad_row_token) {
    if (e < E) kept_s[e] = valid;
    __syncthreads();
    const int64_t nrow = (int64_t)E * C;
    for (int64_t r = tid; r < nrow; r += 1024) {
      const int64_t ex = r / C;
      if (r - ex * C >= kept_s[ex]) pad_row_token[r] = -1;
    }
  }
}

// Standalone grouped GEMM: groups straight from counts and offsets, each
// clamped to the rows [0, rows) of the caller's buffers.
__global__ __launch_bounds__(1024) void gtab_kernel(const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets,
                                                    int E, int BM, int rows,
                                                    int32_t* __restrict__ gtab) {
  __shared__ int tmp[32];
  const int e = threadIdx.x;
  int valid = 0, off = 0;
  if (e < E) {
    off = min(max(offsets[e], 0), rows);
    valid = min(counts[e], offsets[e + 1] - off);
    valid = max(min(valid, rows - off), 0);
  }
  write_gtab(e, E, valid, off, off, BM, tmp, gtab);
}

// One workgroup of NW waves per chunk of 64 * NW tokens; lane = token.
// chunk_base rows are per group of hg tokens; chunk c starts at group
// c * gpc, gpc = 64 * NW / hg (one wave per chunk when hg <= 64, so that
// small T still spreads over many compute units).
template <int KMAX, int NW>
__global__ __launch_bounds__(64 * NW) void assign_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ chunk_base, int gpc,
    const int32_t* __restrict__ offsets, int64_t T, int E, int k, int nbits,
    int64_t C, int32_t* __restrict__ assign_row, int32_t* __restrict__ row_token) {
  __shared__ int32_t cnt[NW][1024];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t chunk = blockIdx.x;
  const int64_t t = chunk * (64 * NW) + tid;
  const bool valid = t < T;

  // Expert ids outside [0, E) (possible only through the standalone permute
  // call) take no row and do not count.
  int ex[KMAX];
  bool ok[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ex[j] = (valid && j < k) ? idx[t * k + j] : 0;
    ok[j] = valid && j < k && (unsigned)ex[j] < (unsigned)E;
    if (!ok[j]) ex[j] = 0;
  }

  for (int i = tid; i < NW * E; i += 64 * NW) cnt[i / E][i % E] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (ok[j]) atomicAdd(&cnt[w][ex[j]], 1);
  __syncthreads();
  // wave bases: chunk base of the expert plus the counts of earlier waves
  for (int e = tid; e < E; e += 64 * NW) {
    int run = chunk_base[chunk * gpc * E + e];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const int c = cnt[ww][e];
      cnt[ww][e] = run;
      run += c;
    }
  }
  __syncthreads();

  // local[j]: lanes below this one (earlier tokens of the wave) whose slot
  // jp holds the same expert as slot j here, summed over jp.  Equality is
  // tested bit by bit against one ballot per (slot, bit).
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int local[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) local[j] = 0;
#pragma unroll
  for (int jp = 0; jp < KMAX; ++jp) {
    if (jp < k) {
      const uint64_t vmask = __ballot(ok[jp]);
      uint64_t bits[10];
#pragma unroll
      for (int b = 0; b < 10; ++b) bits[b] = (b < nbits) ? __ballot((ex[jp] >> b) & 1) : 0ull;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          uint64_t m = vmask & below;
#pragma unroll
          for (int b = 0; b < 10; ++b)
            if (b < nbits) m &= ((ex[j] >> b) & 1) ? bits[b] : ~bits[b];
          local[j] += __popcll(m);
        }
      }
    }
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const int e = ex[j];
        int row = -1;
        if (ok[j]) {
          const int rank = cnt[w][e] + local[j];
          if (C == 0)
            row = offsets[e] + rank;
          else
            row = (rank < C) ? e * (int)C + rank : -1;
        }
        assign_row[t * k + j] = row;
        if (row >= 0) row_token[row] = (int32_t)t;
      }
    }
  }
}

// The same ranks for k > 2 slots when the histogram groups hold at most 64
// tokens: one workgroup of KP waves per 64 tokens, lane = (token, slot):
// wave w takes the chunk's tokens [w * 64/KP, (w + 1) * 64/KP), lane l
// token l / KP and slot l % KP (KP a power of two >= k).  A slot's rank is
// the chunk's base for its expert, plus the slots of the earlier waves'
// tokens that hold that expert (LDS counts summed in wave order), plus
// those of the earlier tokens of its own wave (lanes below its token's
// first lane whose expert id agrees bit by bit, one ballot per bit), so
// the rows are those of assign_kernel with a handful of ballots per wave
// instead of k * k * bits per lane.
template <int KP>
__global__ __launch_bounds__(64 * KP) void assign_pairs_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ chunk_base, int gpc,
    const int32_t* __restrict__ offsets, int64_t T, int E, int k, int nbits,
    int64_t C, int32_t* __restrict__ assign_row, int32_t* __restrict__ row_token) {
  constexpr int TPW = 64 / KP;           // tokens per wave
  __shared__ int32_t cnt[KP][1024];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int tl = lane / KP, j = lane % KP;
  const int64_t chunk = blockIdx.x;
  const int64_t t = chunk * 64 + w * TPW + tl;
  const bool valid = t < T && j < k;
  int ex = valid ? idx[t * k + j] : 0;
  // expert ids outside [0, E) take no row and do not count
  const bool ok = valid && (unsigned)ex < (unsigned)E;
  if (!ok) ex = 0;
  for (int ww = 0; ww < KP; ++ww)
    for (int e = tid; e < E; e += 64 * KP) cnt[ww][e] = 0;
  __syncthreads();
  if (ok) atomicAdd(&cnt[w][ex], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 64 * KP) {
    int run = chunk_base[chunk * gpc * E + e];
#pragma unroll
    for (int ww = 0; ww < KP; ++ww) {
      const int c = cnt[ww][e];
      cnt[ww][e] = run;
      run += c;
    }
  }
  __syncthreads();
  const uint64_t below = tl == 0 ? 0ull : (~0ull >> (64 - KP * tl));
  uint64_t m = __ballot(ok) & below;
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    if (b < nbits) {
      const uint64_t bb = __ballot((ex >> b) & 1);
      m &= ((ex >> b) & 1) ? bb : ~bb;
    }
  }
  if (valid) {
    int row = -1;
    if (ok) {
      const int rank = cnt[w][ex] + __popcll(m);
      if (C == 0)
        row = offsets[ex] + rank;
      else
        row = (rank < C) ? ex * (int)C + rank : -1;
    }
    assign_row[t * k + j] = row;
    if (row >= 0) row_token[row] = (int32_t)t;
  }
}

template <int KMAX>
void launch_assign_t(const int32_t* idx, const int32_t* base, int hg, const int32_t* off,
                     int64_t T, int E, int k, int nbits, int64_t C, int32_t* ar,
                     int32_t* rt, hipStream_t s) {
  if (hg <= 64) {
    const int64_t nch = (T + 63) / 64;
    MOE_LAUNCH((assign_kernel<KMAX, 1>), dim3((unsigned)nch), dim3(64), 0, s,
               idx, base, 64 / hg, off, T, E, k, nbits, C, ar, rt);
  } else {
    const int64_t nch = (T + kChunkTokens - 1) / kChunkTokens;
    MOE_LAUNCH((assign_kernel<KMAX, 4>), dim3((unsigned)nch), dim3(256), 0, s,
               idx, base, kChunkTokens / hg, off, T, E, k, nbits, C, ar, rt);
  }
}

constexpr int kPermTok = 2;      // tokens per permute workgroup
constexpr int kPadBlocks = 256;  // workgroups that clear padding rows

// Token part: blocks [0, ntb) copy kPermTok tokens each.  Padding part
// (capacity mode): the remaining kPadBlocks blocks walk every expert's
// unused rows e*C + kept_e .. e*C + C - 1.
__global__ __launch_bounds__(256) void permute_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ assign_row,
    const int32_t* __restrict__ counts, int64_t T, int nv, int E, int k,
    int64_t C, int64_t ntb, uint4* __restrict__ x_perm, int64_t pv,
    int32_t* __restrict__ row_token) {
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  if (b < ntb) {
    for (int tt = 0; tt < kPermTok; ++tt) {
      const int64_t t = b * kPermTok + tt;
      if (t >= T) return;
      const uint4* src = x + t * nv;
      for (int v = tid; v < nv; v += 256) {
        const uint4 val = src[v];
        for (int j = 0; j < k; ++j) {
          const int r = assign_row[t * k + j];
          if (r >= 0) x_perm[(int64_t)r * pv + v] = val;
        }
      }
    }
    return;
  }
  const int64_t pb = b - ntb;
  for (int e = 0; e < E; ++e) {
    const int64_t kept = min((int64_t)counts[e], C);
    for (int64_t r = e * C + kept + pb; r < (e + 1) * C; r += kPadBlocks) {
      uint4* dst = x_perm + r * pv;
      for (int v = tid; v < nv; v += 256) dst[v] = uint4{0u, 0u, 0u, 0u};
      if (tid == 0) row_token[r] = -1;
    }
  }
}

// Expert choice: every routed group holds exactly C rows (e*C ..), plus
// the shared group (T rows, read from x) when there is one.  One workgroup
// of 1024 threads.
__global__ __launch_bounds__(1024) void fixed_groups_kernel(int E, int C, int64_t T,
                                                            int has_shared, int BM,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ gtab) {
  __shared__ int tmp[32];
  const int e = threadIdx.x;
  if (e < E) {
    counts[e] = C;
    offsets[e] = e * C;
  }
  if (e == 0) offsets[E] = E * C;
  const int G = E + (has_shared ? 1 : 0);
  int valid = 0, a0 = 0, o0 = 0;
  if (e < E) {
    valid = C;
    a0 = o0 = e * C;
  } else if (e == E && has_shared) {
    valid = (int)T;
    a0 = 0;
    o0 = E * C;
  }
  write_gtab(e, G, valid, a0, o0, BM, tmp, gtab);
}

// Backward: groups from the forward's counts and offsets, each clamped to
// the rows [0, rows) of the dispatch buffers.  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void groups_from_counts_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int E, int64_t C,
    int64_t T, int has_shared, int BM, int64_t rows, int32_t* __restrict__ gtab) {
  __shared__ int tmp[32];
  const int e = threadIdx.x;
  const int G = E + (has_shared ? 1 : 0);
  int valid = 0, a0 = 0, o0 = 0;
  if (e < E) {
    valid = C > 0 ? min(counts[e], (int)C) : counts[e];
    a0 = o0 = min(max(offsets[e], 0), (int)rows);
    valid = max(min(valid, (int)rows - a0), 0);
  } else if (e == E && has_shared) {
    valid = (int)T;
    a0 = 0;
    o0 = (int)rows;
  }
  write_gtab(e, G, valid, a0, o0, BM, tmp, gtab);
}

// x_perm[r] = x[row_token[r]] for every row (expert choice fills each
// expert's C rows), kPermTok rows per workgroup, 16-byte vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          int64_t rows, int64_t T, int nv,
                                                          uint4* __restrict__ x_perm, int64_t pv) {
  for (int rr = 0; rr < kPermTok; ++rr) {
    const int64_t r = (int64_t)blockIdx.x * kPermTok + rr;
    if (r >= rows) return;
    const int64_t t = row_token[r];
    uint4* dst = x_perm + r * pv;
    if ((uint64_t)t >= (uint64_t)T) {   // no token: a zero row
      for (int v = threadIdx.x; v < nv; v += 256) dst[v] = uint4{0u, 0u, 0u, 0u};
      continue;
    }
    const uint4* src = x + t * nv;
    for (int v = threadIdx.x; v < nv; v += 256) dst[v] = src[v];
  }
}

}  // namespace

hipError_t launch_fixed_groups(int E, int C, int64_t T, int has_shared, int BM, int32_t* counts,
                               int32_t* offsets, int32_t* gtab, hipStream_t s) {
  MOE_LAUNCH(fixed_groups_kernel, dim3(1), dim3(1024), 0, s, E, C, T, has_shared, BM,
                     counts, offsets, gtab);
  return hipGetLastError();
}

hipError_t launch_groups_from_counts(const int32_t* counts, const int32_t* offsets, int E,
                                     int64_t C, int64_t T, int has_shared, int BM,
                                     int64_t rows, int32_t* gtab, hipStream_t s) {
  MOE_LAUNCH(groups_from_counts_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, E,
                     C, T, has_shared, BM, rows, gtab);
  return hipGetLastError();
}

hipError_t launch_gather_rows(int dtype, const void* x, const int32_t* row_token, int64_t rows,
                              int64_t T, int h, void* x_perm, int ld_perm, hipStream_t s) {
  const int esz = dtype == 1 ? 2 : 4;
  const int64_t nb = (rows + kPermTok - 1) / kPermTok;
  MOE_LAUNCH(gather_rows_kernel, dim3((unsigned)nb), dim3(256), 0, s, (const uint4*)x,
                     row_token, rows, T, h * esz / 16, (uint4*)x_perm,
                     (int64_t)ld_perm * esz / 16);
  return hipGetLastError();
}

hipError_t launch_hist(const int32_t* idx, int64_t T, int E, int k,
                       int32_t* chunk_hist, hipStream_t s) {
  const int64_t nch = (T + kChunkTokens - 1) / kChunkTokens;
  MOE_LAUNCH(hist_kernel, dim3((unsigned)nch), dim3(256), 0, s, idx, T,
                     E, k, chunk_hist);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* chunk_hist, int64_t nch, int E, int64_t C,
                       int64_t T, int k, int has_shared, int BM,
                       int32_t* chunk_base, int32_t* counts, int32_t* offsets,
                       int32_t* gtab, hipStream_t s, int32_t* pad_row_token) {
  MOE_LAUNCH(scan_kernel, dim3(1), dim3(1024), 0, s, chunk_hist, nch, E,
                     C, T, k, has_shared, BM, chunk_base, counts, offsets, gtab, pad_row_token);
  return hipGetLastError();
}

hipError_t launch_gtab(const int32_t* counts, const int32_t* offsets, int E,
                       int BM, int rows, int32_t* gtab, hipStream_t s) {
  MOE_LAUNCH(gtab_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, E,
                     BM, rows, gtab);
  return hipGetLastError();
}

hipError_t launch_assign(const int32_t* idx, const int32_t* chunk_base, int hg,
                         const int32_t* offsets, int64_t T, int E, int k,
                         int64_t C, int32_t* assign_row, int32_t* row_token,
                         hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (k > 2 && hg <= 64) {
    const int64_t nch = (T + 63) / 64;
    if (k <= 4)
      MOE_LAUNCH(assign_pairs_kernel<4>, dim3((unsigned)nch), dim3(256), 0, s, idx, chunk_base,
                 64 / hg, offsets, T, E, k, nbits, C, assign_row, row_token);
    else if (k <= 8)
      MOE_LAUNCH(assign_pairs_kernel<8>, dim3((unsigned)nch), dim3(512), 0, s, idx, chunk_base,
                 64 / hg, offsets, T, E, k, nbits, C, assign_row, row_token);
    else
      MOE_LAUNCH(assign_pairs_kernel<16>, dim3((unsigned)nch), dim3(1024), 0, s, idx, chunk_base,
                 64 / hg, offsets, T, E, k, nbits, C, assign_row, row_token);
    return hipGetLastError();
  }
  if (k <= 1)
    launch_assign_t<1>(idx, chunk_base, hg, offsets, T, E, k, nbits, C, assign_row, row_token, s);
  else if (k <= 2)
    launch_assign_t<2>(idx, chunk_base, hg, offsets, T, E, k, nbits, C, assign_row, row_token, s);
  else if (k <= 4)
    launch_assign_t<4>(idx, chunk_base, hg, offsets, T, E, k, nbits, C, assign_row, row_token, s);
  else if (k <= 8)
    launch_assign_t<8>(idx, chunk_base, hg, offsets, T, E, k, nbits, C, assign_row, row_token, s);
  else
    launch_assign_t<16>(idx, chunk_base, hg, offsets, T, E, k, nbits, C, assign_row, row_token, s);
  return hipGetLastError();
}

hipError_t launch_permute(int dtype, const void* x, const int32_t* assign_row,
                          const int32_t* counts, int64_t T, int h, int E, int k,
                          int64_t C, void* x_perm, int ld_perm, int32_t* row_token,
                          hipStream_t s) {
  const int esz = dtype == 1 ? 2 : 4;
  const int nv = h * esz / 16;
  const int64_t pv = (int64_t)ld_perm * esz / 16;
  const int64_t ntb = (T + kPermTok - 1) / kPermTok;
  const int64_t nb = ntb + (C > 0 ? kPadBlocks : 0);
  MOE_LAUNCH(permute_kernel, dim3((unsigned)nb), dim3(256), 0, s,
                     (const uint4*)x, assign_row, counts, T, nv, E, k, C, ntb,
                     (uint4*)x_perm, pv, row_token);
  return hipGetLastError();
}

}  // namespace moe
