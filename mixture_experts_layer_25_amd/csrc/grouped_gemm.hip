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
// C = A · B^T with 16-byte loads along K for A and B alike.  The same kernel
// runs the backward's GEMMs (input gradients on transposed weights, and
// weight gradients whose groups split along K over K-major copies).
//
// bf16: the eight-wave ping-pong kernel (gemm_pp_kernel, described where it
// is defined), a 256x256 output tile per workgroup.  The last row tile of a
// group is cut to 64, 128 or 192 rows when that holds its rows, so a group's
// leftover rows cost a quarter, half or three quarters of a tile instead of
// a whole one.  Routed group g starts its K loop at slice g*nk/8: groups run
// on different XCDs, and staggered K offsets spread their weight reads over
// the memory channels (the row strides are powers of two).
//
// For GEMM 1 the 256 B-tile rows are [w1 f0..f0+31 | w3 f0..f0+31 |
// w1 f0+32..f0+63 | w3 f0+32..f0+63 | ...]: each wave's 64 columns hold 32
// w1 columns and the matching 32 w3 columns, so silu(a1) * a3 is formed in
// registers and a tile writes 128 activation columns.
//
// Tiles: each group (expert) has ceil(rows/256) row tiles; the scan kernel
// writes their prefix.  Logical tile L walks (group, column tile, row tile)
// with the row tile fastest, so the workgroups running together share the
// same few weight column tiles and token row tiles.  Workgroup b runs on
// XCD b % 8; consecutive logical tiles are handed to the same XCD so that
// they share its L2.  Workgroups past the real tile count exit at once.
// The tiles of the last, partial round of workgroups are split along K and
// summed by a reduce kernel in part order.
//
// fp32 layers: a 64x64-tile FMA kernel (gemm_f32_kernel).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM_bf16, BN = 256, BK = 64;
constexpr int kPart = BM * BK * 2;          // 32 KiB: one K slice of the A (or B) tile

// Largest g with mtp[g] * NT <= L (mtp non-decreasing, mtp[0] = 0,
// mtp[G] * NT > L).
template <typename GT>
__device__ __forceinline__ int find_group(const GT* mtp, int G, int64_t L, int NT) {
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

// Tile of logical index L (row tile fastest within (group, column tile)).
template <typename GT>
__device__ __forceinline__ Tile tile_of(const GroupedGemmArgs& a, const GT* gt, int NT, int64_t L,
                                        int BMx) {
  const int G = a.G;
  Tile t;
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
  return t;
}

// Logical index of the tile workgroup b computes when every tile is whole
// (fp32 kernel), or -1.
__device__ __forceinline__ int64_t plain_tile(const GroupedGemmArgs& a, int NT, int64_t b) {
  const int64_t V = (int64_t)a.gtab[a.G] * NT;
  return b < V ? b : -1;
}

// Work of a bf16 workgroup.  With V tiles on P compute units the first
// V - r tiles (r = V mod P) run whole, in rounds of P; if r > 0 the last r
// tiles would leave most units idle in a final round, so each is split
// along K into s = min(P / r, nk / 8) parts (when s >= 2), computed by r*s
// workgroups that write fp32 partial tiles; a reduce kernel sums them.
// Whole tiles: workgroup b runs on XCD b % 8, and XCD x owns the x-th of
// eight contiguous runs of logical tiles, so that the workgroups sharing a
// weight column tile and a token row tile share its L2.  Without claim
// counters, workgroup 8j + x computes tile j of run x and the split parts
// follow the whole tiles in workgroup order.  With them (a.claims), every
// workgroup claims its work: the next tile of its own run, or, once that
// run is empty, the last unclaimed tile of the fullest other run (an XCD
// that finishes early takes over the end of a slower one's run), or, once
// every run is empty, the next split part.
struct Work {
  int64_t L;        // logical tile, -1: nothing to do
  int part, parts;  // K part of a split tile (parts == 1: whole tile)
  int64_t slot;     // split tiles: index among the split tiles
};
static_assert(sizeof(Work) <= 32, "a claimed Work fits the last 32 bytes of LDS");

// Workgroups per XCD beyond the bound on the tiles and split parts, which
// find work only in the runs of other XCDs.
constexpr int kClaimSlack = 32;
// Distance between two claim counters in uint64.
constexpr int kClaimU64 = kClaimStride / 8;

// Workgroups of a bf16 launch that is not split along groups' K: a bound on
// the whole tiles and split parts (all row tiles times the column tiles,
// plus one compute unit's worth of parts), and with claim counters the
// slack of every XCD.
__host__ __device__ inline int64_t pp_workgroups(const GroupedGemmArgs& a, int NT) {
  return a.max_m_tiles * NT + (a.partials ? a.num_cu : 0) + (a.claims ? 8 * kClaimSlack : 0);
}

__device__ __forceinline__ void split_shape(const GroupedGemmArgs& a, int32_t tiles, int NT,
                                            int nk, int64_t& V, int64_t& whole, int& s) {
  V = (int64_t)tiles * NT;
  const int64_t P = a.num_cu > 0 ? a.num_cu : 1;
  const int64_t r = V % P;
  s = 1;
  if (r > 0 && a.partials) {
    const int64_t byu = P / r, byk = nk / 8;
    s = (int)min(min(byu, byk), (int64_t)16);
  }
  whole = s >= 2 ? V - r : V;
}

// Run x of the whole tiles: [start, start + n).
__device__ __forceinline__ void xcd_run(int64_t whole, int x, int64_t& start, int64_t& n) {
  const int64_t q = whole >> 3, r8 = whole & 7;
  start = x * q + (x < r8 ? x : r8);
  n = q + (x < r8 ? 1 : 0);
}

// A whole tile for a workgroup of XCD run x whose claim on its own run
// returned `own` (counter value before its increment), or -1 when every
// run is empty.  A counter holds the tiles taken from the front of its run
// (low 32 bits) and from the back (high 32 bits); an increment claims a
// tile exactly when the two together were below the run's length, so each
// tile is claimed once.  Every failed claim marks a run as empty: at most
// eight rounds.
__device__ int64_t claim_whole_tile(unsigned long long* cl, unsigned long long own, int x,
                                    int64_t whole) {
  int64_t st, n;
  xcd_run(whole, x, st, n);
  {
    const int64_t h = (uint32_t)own, t = (int64_t)(own >> 32);
    if (h + t < n) return st + h;
  }
  unsigned empty = 1u << x;
  for (int it = 0; it < 8; ++it) {
    unsigned long long v[8];
#pragma unroll
    for (int y = 0; y < 8; ++y)
      v[y] = ((empty >> y) & 1) ? 0ull
                                : __hip_atomic_load(cl + y * kClaimU64, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
    int best = -1;
    int64_t brem = 0;
#pragma unroll
    for (int y = 0; y < 8; ++y) {
      if ((empty >> y) & 1) continue;
      int64_t sy, ny;
      xcd_run(whole, y, sy, ny);
      const int64_t rem = ny - ((int64_t)(uint32_t)v[y] + (int64_t)(v[y] >> 32));
      if (rem <= 0)
        empty |= 1u << y;
      else if (rem > brem) {
        brem = rem;
        best = y;
      }
    }
    if (best < 0) return -1;
    const unsigned long long o = atomicAdd(cl + best * kClaimU64, 1ull << 32);
    int64_t sb, nb;
    xcd_run(whole, best, sb, nb);
    const int64_t h = (uint32_t)o, t = (int64_t)(o >> 32);
    if (h + t < nb) return sb + nb - 1 - t;
    empty |= 1u << best;
  }
  return -1;
}

// Split part q of the split tiles (s parts each).
__device__ __forceinline__ Work split_part(int64_t whole, int s, int64_t q) {
  Work wk{-1, 0, 1, 0};
  wk.slot = q / s;
  wk.L = whole + wk.slot;
  wk.part = (int)(q - wk.slot * s);
  wk.parts = s;
  return wk;
}

// Work of workgroup b with claim counters `cl` (8 run counters, then the
// split-part counter), its claim on its own run having returned `own`:
// that tile, else (workgroups below the number of tiles and parts plus the
// slack) another run's tile or the next split part, else nothing.  Every
// workgroup of that number ends with work or after seeing all work
// claimed, and there are more of them than pieces of work, so all of it is
// claimed.
__device__ Work claim_work(unsigned long long* cl, unsigned long long own, int64_t b, int64_t V,
                           int64_t whole, int s) {
  Work wk{-1, 0, 1, 0};
  const int x = (int)(b & 7);
  {
    int64_t st, n;
    xcd_run(whole, x, st, n);
    const int64_t h = (uint32_t)own, t = (int64_t)(own >> 32);
    if (h + t < n) {
      wk.L = st + h;
      return wk;
    }
  }
  const int64_t parts = s >= 2 ? (V - whole) * s : 0;
  if (b >= whole + parts + 8 * kClaimSlack) return wk;
  wk.L = claim_whole_tile(cl, own, x, whole);
  if (wk.L < 0 && parts > 0) {
    const int64_t q = (int64_t)atomicAdd(cl + 8 * kClaimU64, 1ull);
    if (q < parts) wk = split_part(whole, s, q);
  }
  return wk;
}

// Work of workgroup b without claim counters: its whole tile by index, or
// its split part (split workgroups follow the whole tiles).
__device__ __forceinline__ Work plan_work(const GroupedGemmArgs& a, int32_t tiles, int NT, int nk,
                                          int64_t b) {
  int64_t V, whole;
  int s;
  split_shape(a, tiles, NT, nk, V, whole, s);
  Work wk{-1, 0, 1, 0};
  if (b < whole) {
    int64_t st, n;
    xcd_run(whole, (int)(b & 7), st, n);
    wk.L = st + (b >> 3);
  } else if (s >= 2 && b - whole < (V - whole) * s) {
    const int64_t qd = b - whole;
    wk.slot = qd / s;
    wk.L = whole + wk.slot;
    wk.part = (int)(qd - wk.slot * s);
    wk.parts = s;
  }
  return wk;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
#define LDS_AS(p) ((__attribute__((address_space(3))) void*)(p))

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero, which is how rows beyond a ragged group's end enter the MFMAs.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ bf16x8 lds_frag(const uint8_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// A K-major B fragment: rows +0..3 at p and +4..7 at p + 4 rows (2 KiB),
// through transposing reads (lane i of a 16-lane group gets column i).
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 lds_frag_tr(const uint8_t* p) {
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(p));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(p + 2048));
  const shortx8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Row fragments (32 rows) per wave for a tile of m_valid rows.  The last
// row tile of a group is only as tall as its rows need (64, 128, 192 or
// 256), so a group's few leftover rows do not cost a whole 256-row tile.
__device__ __forceinline__ int frags_of(int m_valid) {
  return m_valid > 192 ? 4 : (m_valid > 128 ? 3 : (m_valid > 64 ? 2 : 1));
}

// Epilogues of the plain product: store it (rounded to bf16), turn dU into
// the SwiGLU backward's dA, or add the gathered dx_perm rows of the layer's
// dx to the router term.
constexpr int kEpiPlain = 0, kEpiDSwiglu = 1, kEpiDxGather = 2;

// Where output row r (within the tile's group) lives: out0 + r*ldo, or
// out1 + (r - split)*ldo from row `split` on (weight gradients of w1 and w3
// computed as one [2F, h] product).
struct OutMap {
  uint16_t* out0;
  uint16_t* out1;
  int64_t split;
  int64_t ldo;
  uint16_t* a13;   // SwiGLU: pre-activations [a1 | a3] too, or NULL
  int64_t ld13;
  const uint16_t* dsw;   // plain: [a1 | a3] of the SwiGLU backward, or NULL
  int64_t ldsw;
  const uint16_t* dxg;   // plain: dx_perm rows gathered into dx, or NULL
  const int32_t* dxg_assign;
  int dxg_k, dxg_shared;
  int64_t dxg_rows, dxg_ld;
  __device__ __forceinline__ uint16_t* row(int64_t r) const {
    return r < split ? out0 + r * ldo : out1 + (r - split) * ldo;
  }
};

__device__ __forceinline__ OutMap out_map(const GroupedGemmArgs& a, int g) {
  OutMap m;
  const int64_t go = a.kgroup ? (int64_t)(g - a.kg0) * a.out_stride : 0;
  m.out0 = (uint16_t*)a.out + go;
  m.out1 = a.out1 ? (uint16_t*)a.out1 + go : nullptr;
  m.split = (a.out1 && a.split_rows > 0) ? a.split_rows : INT64_MAX;
  m.ldo = a.ldo;
  m.a13 = (uint16_t*)a.out13;
  m.ld13 = a.ld13;
  m.dsw = (const uint16_t*)a.dsw_a13;
  m.ldsw = a.dsw_ld13;
  m.dxg = (const uint16_t*)a.dxg;
  m.dxg_assign = a.dxg_assign;
  m.dxg_k = a.dxg_k;
  m.dxg_shared = a.dxg_shared;
  m.dxg_rows = a.dxg_rows;
  m.dxg_ld = a.dxg_ld;
  return m;
}

// ---------------------------------------------------------------------------
// Eight-wave ping-pong kernel (bf16, every mode).
//
// 512 threads in two groups of four waves, one wave of each group on every
// SIMD.  For a tile of 64*FI rows x 256 columns, group g owns rows
// [32*FI*g, 32*FI*(g+1)) and its wave q the 64 columns [64q, 64q + 64): FI x 2
// fragments of v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane, so
// two waves share a SIMD's registers).  K advances in slices of 64, copied
// global -> LDS directly (buffer_load_dwordx4 ... lds, 8 rows of 128 bytes
// per instruction, no registers in between; buffer bounds return zeros for
// rows past a ragged group's end) through three A slots and two B slots of
// 32 KiB (all 160 KiB of LDS).  The two groups take turns, a barrier ending
// every phase: while one group runs the 8*FI MFMAs of a slice from its
// registers at raised priority, the other reads its fragments of its next
// slice from LDS into registers and issues global -> LDS copies: group 0
// the B slice t + 1 while it reads slice t, group 1 the A slice t + 2.  A
// wave's copies and LDS reads thus never sit between its own MFMAs (in a
// wave's in-order stream they held the MFMAs up), and the MFMA pipe of every
// SIMD is fed by one wave or the other.  Slice t is read by group 0 in phase
// 2t - 1 and by group 1 in phase 2t; B slice t + 1 goes into the slot of
// slice t - 1 (free after phase 2t - 2) and is first read in phase 2t + 1,
// A slice t + 2 into the slot of slice t - 1 and first read in phase 2t + 3;
// each wave waits for its copies at the end of its next (MFMA) phase.
//
// LDS rows are 128 bytes (8 chunks of 16 B); chunk c of row r is stored at
// c ^ ((r ^ (r >> 3)) & 7).  An MFMA operand read has 16 lanes on 16
// consecutive rows and one chunk: with this swizzle they fall in 16
// distinct 16-byte slots of 256 bytes (64 banks).
//
// Epilogue: the MFMAs take the weight fragment first, so fragment (i, j)
// holds C^T: lane l has output row (l & 31) of row fragment i and, in
// registers 4b..4b+3, the 4 consecutive columns 8b + 4*(l >> 5) + 0..3 of
// column fragment j.  Lanes l and l ^ 32 (same row) trade one 4-column run
// so that each ends up with 8 consecutive columns: 16-byte stores.
constexpr int kPPLds = 5 * kPart;            // 160 KiB
// slot counts of the 192- and 256-row tiles (A, B)
constexpr int kTallNA = 3, kTallNB = 2;
// The tile table is staged at [128 KiB, 144.4 KiB) and a claimed tile's
// work passed on in the last 32 bytes: in every slot layout the copies
// issued before a tile's first barrier stay below 128 KiB.
constexpr int kTableOff = 4 * kPart;

// Where split-K partial register group c (= (i*2 + j)*4 + r4) of wave w goes
// within its 256x256 fp32 tile.
template <int FI>
__device__ __forceinline__ int64_t part_off_pp(int w, int c, int lane) {
  return ((int64_t)(w * 8 * FI + c) * 64 + lane) * 4;
}

// Epilogue: wave (grp, q) holds rows 32*FI*grp + 32i + (lane & 31) and, per
// fragment j, C^T runs of 4 columns (see above).
template <bool SWIGLU, int FI, int EPI = 0>
__device__ __forceinline__ void store_tile_pp(const floatx16 (&acc)[FI][2], const Tile& tl,
                                              int lane, int grp, int q, const OutMap& om, int N) {
  const int hi = lane >> 5;
  auto emit = [&](const uint32_t (&v)[4][2], uint16_t* rowp, int64_t col0, bool ok) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t lo[2], up[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const auto r = __builtin_amdgcn_permlane32_swap(v[2 * c][p], v[2 * c + 1][p], false, false);
        lo[p] = r[0];
        up[p] = r[1];
      }
      if (ok)
        *reinterpret_cast<uint4*>(rowp + col0 + 16 * c + 8 * hi) = uint4{lo[0], lo[1], up[0], up[1]};
    }
  };
  auto pack_runs = [&](const floatx16& f, uint32_t (&v)[4][2]) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int p = 0; p < 2; ++p) v[b][p] = pack_bf16x2(f[4 * b + 2 * p], f[4 * b + 2 * p + 1]);
  };
  if constexpr (EPI == kEpiDxGather) {
    // dx of the layer: the tile's rows are tokens and the product is the
    // router term dl W_router.  After the exchange with lane l ^ 32 a lane
    // holds 8 consecutive columns of it (fp32); it adds the token's dx_perm
    // rows (its slots in order, then the shared expert's row) to that sum
    // and rounds once.  The row ids of the first 8 slots are loaded once per
    // row fragment.
    const uint16_t* src = om.dxg;
    const int kk = om.dxg_k;
    const int64_t rows = om.dxg_rows, ldp = om.dxg_ld;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int row = grp * 32 * FI + i * 32 + (lane & 31);
      const bool ok = row < tl.m_valid;
      const int64_t t = tl.o_row + row;
      int ids[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) ids[u] = (ok && u < kk) ? om.dxg_assign[t * kk + u] : -1;
      uint16_t* orow = om.row(t);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col0 = (int64_t)tl.nt * BN + 64 * q + 32 * j;
        if (col0 >= N) continue;
        float rt[2][8];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // (the elements go through values: a bit cast of a vector
            // element designator reads element 0)
            const float x0 = acc[i][j][8 * c + e], x1 = acc[i][j][8 * c + 4 + e];
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0),
                                                            __float_as_uint(x1), false, false);
            rt[c][e] = __uint_as_float((uint32_t)r[0]);
            rt[c][4 + e] = __uint_as_float((uint32_t)r[1]);
          }
        if (!ok) continue;
        const int64_t cl[2] = {col0 + 8 * hi, col0 + 16 + 8 * hi};
        float sum[2][8];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) sum[c][e] = 0.f;
        auto add_rows = [&](const int (&rr)[4]) {
          uint4 v[4][2];
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 2; ++c)
              v[u][c] = (rr[u] >= 0 && rr[u] < rows)
                            ? *reinterpret_cast<const uint4*>(src + rr[u] * ldp + cl[c])
                            : uint4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (rr[u] < 0 || rr[u] >= rows) continue;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const uint32_t w[4] = {v[u][c].x, v[u][c].y, v[u][c].z, v[u][c].w};
#pragma unroll
              for (int p = 0; p < 4; ++p) {
                sum[c][2 * p] += __uint_as_float(w[p] << 16);
                sum[c][2 * p + 1] += __uint_as_float(w[p] & 0xFFFF0000u);
              }
            }
          }
        };
        {
          const int r0[4] = {ids[0], ids[1], ids[2], ids[3]};
          add_rows(r0);
        }
        if (kk > 4) {
          const int r1[4] = {ids[4], ids[5], ids[6], ids[7]};
          add_rows(r1);
        }
        for (int s0 = 8; s0 < kk; s0 += 4) {
          int rr[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) rr[u] = s0 + u < kk ? om.dxg_assign[t * kk + s0 + u] : -1;
          add_rows(rr);
        }
        if (om.dxg_shared) {   // the shared expert's row rows + t
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint4 q4 = *reinterpret_cast<const uint4*>(src + (rows + t) * ldp + cl[c]);
            const uint32_t w[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              sum[c][2 * p] += __uint_as_float(w[p] << 16);
              sum[c][2 * p + 1] += __uint_as_float(w[p] & 0xFFFF0000u);
            }
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          uint32_t o[4];
#pragma unroll
          for (int p = 0; p < 4; ++p)
            o[p] = pack_bf16x2(sum[c][2 * p] + rt[c][2 * p], sum[c][2 * p + 1] + rt[c][2 * p + 1]);
          *reinterpret_cast<uint4*>(orow + cl[c]) = uint4{o[0], o[1], o[2], o[3]};
        }
      }
    }
    return;
  }
  if constexpr (EPI == kEpiDSwiglu) {
    // SwiGLU backward: after the exchange with lane l ^ 32 a lane holds dU
    // (fp32) of 8 consecutive columns; with a1 and a3 of the same columns
    // it writes dA1 and dA3 (N columns apart).  The a1/a3 loads of row
    // fragment i + 1 are issued before fragment i is computed and stored.
    uint4 ld[2][2][2];   // [j][c][a1, a3] of the current row fragment
    auto issue = [&](int i, uint4 (&dst)[2][2][2]) {
      const int row = grp * 32 * FI + i * 32 + (lane & 31);
      if (row >= tl.m_valid) return;
      const uint16_t* r13 = om.dsw + (tl.o_row + row) * om.ldsw;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col0 = (int64_t)tl.nt * BN + 64 * q + 32 * j;
        if (col0 >= N) continue;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int64_t col = col0 + 16 * c + 8 * hi;
          dst[j][c][0] = *reinterpret_cast<const uint4*>(r13 + col);
          dst[j][c][1] = *reinterpret_cast<const uint4*>(r13 + N + col);
        }
      }
    };
    issue(0, ld);
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      uint4 cur[2][2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          cur[j][c][0] = ld[j][c][0];
          cur[j][c][1] = ld[j][c][1];
        }
      if (i + 1 < FI) issue(i + 1, ld);
      const int row = grp * 32 * FI + i * 32 + (lane & 31);
      const bool ok = row < tl.m_valid;
      uint16_t* orow = om.row(tl.o_row + row);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col0 = (int64_t)tl.nt * BN + 64 * q + 32 * j;
        if (col0 >= N) continue;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float d[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // (the elements go through values: a bit cast of a vector
            // element designator reads element 0)
            const float x0 = acc[i][j][8 * c + e], x1 = acc[i][j][8 * c + 4 + e];
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0),
                                                            __float_as_uint(x1), false, false);
            d[e] = __uint_as_float((uint32_t)r[0]);
            d[4 + e] = __uint_as_float((uint32_t)r[1]);
          }
          if (!ok) continue;
          const int64_t col = col0 + 16 * c + 8 * hi;
          const uint4 q1 = cur[j][c][0], q3 = cur[j][c][1];
          const uint32_t w1[4] = {q1.x, q1.y, q1.z, q1.w}, w3[4] = {q3.x, q3.y, q3.z, q3.w};
          uint32_t o1[4], o3[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            float g1[2], g3[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const float a1 = __uint_as_float(e ? w1[p] & 0xFFFF0000u : w1[p] << 16);
              const float a3 = __uint_as_float(e ? w3[p] & 0xFFFF0000u : w3[p] << 16);
              const float du = d[2 * p + e];
              const float sg = 1.f / (1.f + __expf(-a1));
              g1[e] = du * a3 * sg * (1.f + a1 * (1.f - sg));
              g3[e] = du * a1 * sg;
            }
            o1[p] = pack_bf16x2(g1[0], g1[1]);
            o3[p] = pack_bf16x2(g3[0], g3[1]);
          }
          *reinterpret_cast<uint4*>(orow + col) = uint4{o1[0], o1[1], o1[2], o1[3]};
          *reinterpret_cast<uint4*>(orow + N + col) = uint4{o3[0], o3[1], o3[2], o3[3]};
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const int row = grp * 32 * FI + i * 32 + (lane & 31);
    const bool ok = row < tl.m_valid;
    uint16_t* orow = om.row(tl.o_row + row);
    if constexpr (SWIGLU) {
      // fragment 0 holds a1 = x.w1 and fragment 1 a3 = x.w3 of the same 32
      // activation columns
      const int64_t col0 = (int64_t)tl.nt * 128 + 32 * q;
      uint32_t v[4][2];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float u[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 4 * b + 2 * p + e;
            const float z = acc[i][0][r];
            u[e] = z * acc[i][1][r] *
                   __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
          }
          v[b][p] = pack_bf16x2(u[0], u[1]);
        }
      emit(v, orow, col0, ok);
      if (om.a13) {
        uint16_t* r13 = om.a13 + (tl.o_row + row) * om.ld13;
        uint32_t v1[4][2], v3[4][2];
        pack_runs(acc[i][0], v1);
        pack_runs(acc[i][1], v3);
        emit(v1, r13, col0, ok);
        emit(v3, r13, col0 + N, ok);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col0 = (int64_t)tl.nt * BN + 64 * q + 32 * j;
        if (col0 >= N) continue;
        uint32_t v[4][2];
        pack_runs(acc[i][j], v);
        emit(v, orow, col0, ok);
      }
    }
  }
}

// One tile, or one K part of it: K slices [kbeg, kbeg + nsteps) starting at
// slice kbeg + krot and wrapping around.
//
// NA A slots and NB B slots: an operand with n slots is copied n - 1 slices
// ahead of its reads.  With three A slots group 1 copies A and group 0 B;
// with two A slots (and three B slots) the roles swap, so that the weight
// operand B always has the longer lead.
//
// GATHER: the A-copying waves read routed rows through a.a_map (one source
// row per lane and 8-row block, out of range for rows past the tile's).
// BKM: B is K-major (a.b_kmajor).  Its slice is 64 K rows of 256 columns
// (512 bytes) in LDS, 16-byte chunk c of row r stored at c ^ 4*(r & 3), and
// the fragments come out of it through transposing reads (two
// ds_read_b64_tr_b16 per fragment: in a 16-lane group, lane 4*j + r
// addresses row j, columns 4r .. 4r + 3, and lane i receives column i of
// rows 0 .. 3).
template <bool SWIGLU, int FI, int NA, int NB, bool GATHER, bool BKM, int EPI>
__device__ __forceinline__ void tile_body_pp(const GroupedGemmArgs& a, const Tile& tl, int kbeg,
                                             int nsteps, int krot, int part, int parts,
                                             int64_t slot, uint8_t* smem) {
  constexpr int AB = 2 * FI;    // A blocks of 8 rows each wave copies per slice
  // LDS: NA A slots of kAS bytes, then NB B slots of kPart bytes
  constexpr int kAS = (NA == 3 && NB == 2) ? kPart : FI * 8192;
  constexpr int kBO = NA * kAS;
  static_assert((NA == 3 && (NB == 2 || NB == 3)) || (NA == 2 && NB == 3), "slot counts");
  static_assert(kBO + NB * kPart <= kPPLds, "LDS");
  constexpr int gA = NA == 3 ? 1 : 0;   // the group that copies A; the other copies B
  constexpr int dA = NA - 1, dB = NB - 1;   // slices a copy runs ahead of its reads
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, q = w & 3;
  const int K = a.K, N = a.N;
  const bool shared = !a.kgroup && tl.g >= a.E_routed;
  const bool a_shared = shared && !a.a_from_out_rows;
  const uint16_t* A = (const uint16_t*)(a_shared ? a.A_shared : a.A);
  const int lda = a_shared ? a.lda_shared : a.lda;
  const int ldb = a.ldb ? a.ldb : K;
  const uint32_t browbytes = (uint32_t)ldb * 2;
  const uint32_t arowbytes = (uint32_t)lda * 2;
  const uint16_t* B0 = (const uint16_t*)(shared ? a.B0s : a.B0);
  const uint16_t* B1 = (const uint16_t*)(shared ? a.B1s : a.B1);
  if (!shared && !a.kgroup) {
    B0 += (int64_t)tl.g * a.b_stride;
    if (SWIGLU || a.b_split || a.b_ksplit) B1 += (int64_t)tl.g * a.b_stride;
  }

  // Copies, 8 rows (1 KiB) per instruction; lane l lands at byte 16*l of the
  // block: row l >> 3, stored chunk l & 7, which holds logical chunk
  // (l & 7) ^ (row ^ (row >> 3)) & 7 = (l & 7) ^ (l >> 3) ^ (m & 7) for the 8-row
  // block m.  In the A-copying group wave q copies A rows q*16*FI ..
  // (blocks m = 2*FI*q + b), in the other wave q the B rows 64q .. 64q + 63
  // (blocks m = 8q + b).
  rsrc_t rs0, rs1;
  uint32_t rowb;
  uint32_t gofs[GATHER ? AB : 1];   // GATHER: byte offset of this lane's row, per block
  uint32_t bofs[BKM ? 8 : 1];       // BKM: byte offset of this lane's chunk, per copy
  if (grp == gA) {
    const int a_rows = __builtin_amdgcn_readfirstlane(min(max(tl.m_valid - q * 16 * FI, 0), 16 * FI));
    if (GATHER && !a_shared) {
      rs0 = make_rsrc(A, (uint32_t)(a.a_rows * arowbytes));
#pragma unroll
      for (int b = 0; b < AB; ++b) {
        const int lr = b * 8 + (lane >> 3);
        gofs[b] = lr < a_rows ? (uint32_t)a.a_map[tl.a_row + q * 16 * FI + lr] * arowbytes
                              : 0x80000000u;
      }
    } else {
      rs0 = make_rsrc(A + (tl.a_row + q * 16 * FI) * (int64_t)lda, (uint32_t)a_rows * arowbytes);
      if (GATHER) {
#pragma unroll
        for (int b = 0; b < AB; ++b) gofs[b] = (uint32_t)(b * 8 + (lane >> 3)) * arowbytes;
      }
    }
    rs1 = rs0;
    rowb = arowbytes;
  } else if (SWIGLU) {
    // B rows 64q .. 64q + 63 of the tile: w1 then w3 rows f0 + 32q .. + 31
    const int64_t f = (int64_t)tl.nt * 128 + 32 * q;
    rs0 = make_rsrc(B0 + f * K, 32u * browbytes);
    rs1 = make_rsrc(B1 + f * K, 32u * browbytes);
    rowb = browbytes;
  } else if (BKM) {
    // K-major B: wave q copies slice rows 16q .. 16q + 15, two per copy (lane
    // l: row 16q + 2b + (l >> 5), stored chunk l & 31 = logical chunk
    // (l & 31) ^ 4*(row & 3), columns n0 + 8*chunk .. + 7; chunks past N out
    // of range)
    const int64_t n0 = (int64_t)tl.nt * BN;
    const int64_t krows0 = a.b_ksplit > 0 ? a.b_ksplit : K;
    const int64_t kv0 = a.b_krows > 0 ? a.b_krows : krows0;
    const int64_t kv1 = a.b_krows > 0 ? a.b_krows : K - krows0;
    rs0 = make_rsrc(B0 + n0, (uint32_t)((kv0 * ldb - n0) * 2));
    rs1 = a.b_ksplit > 0 ? make_rsrc(B1 + n0, (uint32_t)((kv1 * ldb - n0) * 2)) : rs0;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int row = 16 * q + 2 * b + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (row & 3));
      bofs[b] = n0 + 8 * c < N ? (uint32_t)((row * ldb + 8 * c) * 2) : 0x80000000u;
    }
    rowb = 0;
  } else {
    // b_split: rows [0, N/2) of B come from B0, [N/2, N) from B1 (64-row
    // blocks never straddle N/2, a multiple of 64)
    int64_t brow = (int64_t)tl.nt * BN + 64 * q;
    int64_t nrows = N;
    const uint16_t* Bb = B0;
    if (a.b_split) {
      nrows = N / 2;
      if (brow >= nrows) {
        Bb = B1;
        brow -= nrows;
      }
    }
    const int nb = __builtin_amdgcn_readfirstlane(
        (int)min(max(nrows - brow, (int64_t)0), (int64_t)64));
    rs0 = make_rsrc(Bb + min(brow, nrows - 1) * ldb, (uint32_t)nb * browbytes);
    rs1 = rs0;
    rowb = browbytes;
  }
  const uint32_t vrow = (uint32_t)(lane >> 3) * rowb;
  const uint32_t vx = (uint32_t)((lane & 7) ^ (lane >> 3));
  const int mbase = grp == gA ? 2 * FI * q : 8 * q;

  // Fragment reads: lane l reads row (l & 31) of a 32-row fragment and
  // logical chunk 2*k + (l >> 5) of sub-step k; a fragment starting at row
  // 32*r has swz = (l & 7) ^ (4*(r & 1) + ((l >> 3) & 3)): A fragment i has
  // r = FI*grp + i, B fragment j has r = 2q + j.
  const int rA = (grp * 32 * FI + (lane & 31)) * (BK * 2);
  const int rB = kBO + (64 * q + (lane & 31)) * (BK * 2);
  // BKM fragment reads: lane l = 16G + 4jj + r4 addresses row
  // 16k + 8(G >> 1) + 4h + jj and columns 64q + 32j + 16(G & 1) + 4r4 .. + 3
  int tbr = 0, tbc[2] = {0, 0};
  if (BKM) {
    const int G = lane >> 4, jj = (lane >> 2) & 3, r4 = lane & 3;
    tbr = kBO + (8 * (G >> 1) + jj) * 512;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      tbc[j] = (((8 * q + 4 * j + 2 * (G & 1) + (r4 >> 1)) ^ (4 * jj)) << 4) + (r4 & 1) * 8;
  }
  const int fe = (lane & 7) ^ ((lane >> 3) & 3);
  const int fo = (lane & 7) ^ (4 | ((lane >> 3) & 3));
  const bool aflip = (FI * grp) & 1;   // A fragment i has parity (i & 1) ^ aflip
  int cx[4][2], cxa[4][2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    cx[k][0] = ((2 * k + (lane >> 5)) ^ fe) << 4;
    cx[k][1] = ((2 * k + (lane >> 5)) ^ fo) << 4;
    cxa[k][0] = aflip ? cx[k][1] : cx[k][0];
    cxa[k][1] = aflip ? cx[k][0] : cx[k][1];
  }

  floatx16 acc[FI][2];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8 fa[4][FI], fb[4][2];

#define PP_SB() __builtin_amdgcn_sched_barrier(0)
// K byte offset of slice T within a row (out of the buffer past the last one)
#define PP_KOFF(T)                                                                             \
  ((T) < nsteps ? (uint32_t)(kbeg + ((T) + krot >= nsteps ? (T) + krot - nsteps : (T) + krot)) * \
                      (BK * 2)                                                                 \
                : 0x7FFFFFF0u)
// Copy block b of slice T: a B block into B slot T % NB, or an A block into
// A slot T % NA (the caller's group decides which)
// K-major B: slice T's first K row (-1 past the last slice)
#define PP_KSL(T)                                                                              \
  ((T) < nsteps ? (kbeg + ((T) + krot >= nsteps ? (T) + krot - nsteps : (T) + krot)) * BK : -1)
#define PP_COPY_B(T, B)                                                                        \
  if (BKM) {                                                                                   \
    const int kr_ = PP_KSL(T);                                                                 \
    const bool hi_ = a.b_ksplit > 0 && kr_ >= a.b_ksplit;                                      \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                  \
        hi_ ? rs1 : rs0, LDS_AS(smem + kBO + ((T) % NB) * kPart + (8 * q + (B)) * 1024), 16,   \
        bofs[(B)],                                                                             \
        kr_ < 0 ? 0x7FFFFFF0u : (uint32_t)((kr_ - (hi_ ? a.b_ksplit : 0)) * ldb * 2), 0, 0);   \
  } else {                                                                                     \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                  \
        (SWIGLU && (B) >= 4) ? rs1 : rs0,                                                      \
        LDS_AS(smem + kBO + ((T) % NB) * kPart + (8 * q + (B)) * 1024), 16,                    \
        vrow + ((vx ^ (uint32_t)(((B)) & 7)) << 4),                                            \
        (T) < nsteps ? (uint32_t)(SWIGLU ? ((B) & 3) : (B)) * 8u * browbytes + PP_KOFF(T)      \
                     : PP_KOFF(T),                                                             \
        0, 0);                                                                                 \
  }
#define PP_COPY_A(T, B)                                                                        \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                    \
      rs0, LDS_AS(smem + ((T) % NA) * kAS + (mbase + (B)) * 1024), 16,                         \
      (GATHER ? gofs[(B)] : vrow) + ((vx ^ (uint32_t)((mbase + (B)) & 7)) << 4),               \
      (T) < nsteps && !GATHER ? (uint32_t)(B) * 8u * arowbytes + PP_KOFF(T) : PP_KOFF(T), 0, 0)
// Memory phase: the group's copies (B slice T + dB, 8 blocks, or A slice
// T + dA, 2*FI blocks), then this wave's fragments of slice T.
#define PP_READS(T)                                                                            \
  {                                                                                            \
    if (grp != gA) {                                                                           \
      _Pragma("unroll") for (int c = 0; c < 8; ++c) PP_COPY_B((T) + dB, c);                    \
    } else {                                                                                   \
      _Pragma("unroll") for (int c = 0; c < AB; ++c) PP_COPY_A((T) + dA, c);                   \
    }                                                                                          \
    const uint8_t* SA = smem + ((T) % NA) * kAS;                                               \
    const uint8_t* SB = smem + ((T) % NB) * kPart;                                             \
    _Pragma("unroll") for (int k = 0; k < 4; ++k) {                                            \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) fb[k][j] =                                 \
          BKM ? lds_frag_tr(SB + tbr + k * 8192 + tbc[j])                                      \
              : lds_frag(SB + rB + j * 4096 + cx[k][j]);                                       \
      _Pragma("unroll") for (int i = 0; i < FI; ++i) fa[k][i] =                                \
          lds_frag(SA + rA + i * 4096 + cxa[k][i & 1]);                                        \
    }                                                                                          \
  }
#define PP_MFMAS()                                                                             \
  {                                                                                            \
    __builtin_amdgcn_s_setprio(1);                                                             \
    _Pragma("unroll") for (int k = 0; k < 4; ++k)                                              \
        _Pragma("unroll") for (int i = 0; i < FI; ++i)                                         \
            _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] =                          \
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[k][j], fa[k][i], acc[i][j], 0, 0, 0); \
    __builtin_amdgcn_s_setprio(0);                                                             \
  }
#define PP_VMCNT(n) (0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
#define PP_BARRIER()                       \
  PP_SB();                                 \
  asm volatile("s_barrier" ::: "memory");  \
  PP_SB()
// Copies in flight a group may leave at the end of its memory phase
// (kMemLeft) and of its MFMA phase (kMfmaLeft, group 0 only): its copies
// per slice times the slices after the one that must have landed (see
// below).
  constexpr int kCopies0 = gA == 0 ? AB : 8, kCopies1 = gA == 1 ? AB : 8;
  constexpr int kLead0 = gA == 0 ? dA : dB, kLead1 = gA == 1 ? dA : dB;
  constexpr int kMemLeft0 = kLead0 * kCopies0, kMfmaLeft0 = (kLead0 - 1) * kCopies0;
  constexpr int kMemLeft1 = (kLead1 - 1) * kCopies1;
// end of a memory phase: fragments in registers, copies waited as above
#define PP_END_MEM()                                                \
  PP_SB();                                                          \
  if (grp == 0)                                                     \
    __builtin_amdgcn_s_waitcnt(PP_VMCNT(kMemLeft0) & ~0x0F00);      \
  else                                                              \
    __builtin_amdgcn_s_waitcnt(PP_VMCNT(kMemLeft1) & ~0x0F00);      \
  PP_BARRIER()
  constexpr int kWaitAll = PP_VMCNT(0) & ~0x0F00;          // vmcnt(0) lgkmcnt(0)

  // Every wave runs the same sequence, group 1 one barrier behind group 0:
  //   prologue copies | barrier | (group 1: barrier) |
  //   [reads of slice t (+ copies) | barrier | MFMAs of slice t | barrier] ...
  // so that group 0's MFMAs of slice t run beside group 1's reads of slice t,
  // and group 1's MFMAs of slice t beside group 0's reads of slice t + 1.
  // Prologue: each group copies the first d slices of its operand (d its
  // lead); slice 0 has landed at the first barrier.
  //
  // A copy must land before the barrier that precedes its first reader,
  // group 0's memory phase for that slice (after barrier 2s for slice s).
  // A group copies slice t + d in its memory phase for slice t into the slot
  // of slice t - 1, whose last reader (group 1, before barrier 2t) is done.
  // Group 0 waits for slice t + 1 at the end of its MFMA phase for slice t
  // (the copies of the d - 1 later slices may stay in flight); group 1 at
  // the end of its memory phase for slice t.  A lead of d gives a copy about
  // 2d - 1 phases (group 0) or 2d - 2 phases (group 1) to land.
  if (grp == gA) {
#pragma unroll
    for (int b = 0; b < AB; ++b) PP_COPY_A(0, b);
    if (dA == 2) {
#pragma unroll
      for (int b = 0; b < AB; ++b) PP_COPY_A(1, b);
    }
  } else {
#pragma unroll
    for (int b = 0; b < 8; ++b) PP_COPY_B(0, b);
    if (dB == 2) {
#pragma unroll
      for (int b = 0; b < 8; ++b) PP_COPY_B(1, b);
    }
  }
  PP_SB();
  if (grp == 0) {
    __builtin_amdgcn_s_waitcnt(PP_VMCNT(kMfmaLeft0) & ~0x0F00);
    PP_BARRIER();
  } else {
    __builtin_amdgcn_s_waitcnt(PP_VMCNT(kMemLeft1) & ~0x0F00);
    PP_BARRIER();
    PP_BARRIER();
  }
  for (int t = 0; t < nsteps; ++t) {
    PP_READS(t);
    PP_END_MEM();
    PP_MFMAS();
    // the last barrier of group 1 is left out, which keeps the two groups'
    // barrier counts equal (group 1 had one more at the start)
    PP_SB();
    if (grp == 0) __builtin_amdgcn_s_waitcnt(PP_VMCNT(kMfmaLeft0) & ~0x0F00);
    if (grp == 0 || t + 1 < nsteps) asm volatile("s_barrier" ::: "memory");
    PP_SB();
  }
  // the copies past the last slice (zeros from out-of-range offsets) land
  // before the workgroup ends and its LDS is handed to another
  __builtin_amdgcn_s_waitcnt(kWaitAll);
#undef PP_SB
#undef PP_KOFF
#undef PP_COPY_A
#undef PP_COPY_B
#undef PP_READS
#undef PP_MFMAS
#undef PP_VMCNT
#undef PP_BARRIER
#undef PP_END_MEM

  if (parts > 1) {
    float* P = a.partials + (slot * parts + part) * (int64_t)(256 * 256);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int c = (i * 2 + j) * 4 + r4;
          *reinterpret_cast<floatx4*>(P + part_off_pp<FI>(w, c, lane)) =
              floatx4{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2],
                      acc[i][j][4 * r4 + 3]};
        }
    return;
  }
  store_tile_pp<SWIGLU, FI, EPI>(acc, tl, lane, grp, q, out_map(a, tl.g), N);
}

template <bool SWIGLU, bool GATHER, bool BKM, int EPI>
__device__ __forceinline__ void tile_dispatch_pp(const GroupedGemmArgs& a, const Tile& tl, int fi,
                                                 int kbeg, int nsteps, int krot, int part,
                                                 int parts, int64_t slot, uint8_t* smem) {
  if (fi == 4)
    tile_body_pp<SWIGLU, 4, kTallNA, kTallNB, GATHER, BKM, EPI>(a, tl, kbeg, nsteps, krot, part, parts, slot, smem);
  else if (fi == 3)
    tile_body_pp<SWIGLU, 3, kTallNA, kTallNB, GATHER, BKM, EPI>(a, tl, kbeg, nsteps, krot, part, parts, slot, smem);
  else if (fi == 2)
    tile_body_pp<SWIGLU, 2, 3, 3, GATHER, BKM, EPI>(a, tl, kbeg, nsteps, krot, part, parts, slot, smem);
  else
    tile_body_pp<SWIGLU, 1, 3, 3, GATHER, BKM, EPI>(a, tl, kbeg, nsteps, krot, part, parts, slot, smem);
}

// EPI: the epilogue of a plain product (kEpiPlain, kEpiDSwiglu with
// a.dsw_a13, kEpiDxGather with a.dxg), each a kernel of its own so that the
// others keep their register allocation.
template <bool SWIGLU, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(GroupedGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kPPLds];   // 160 KiB
  const int NT = SWIGLU ? a.N / 128 : (a.N + BN - 1) / BN;
  const int nk = a.K / BK;
  Work wk{-1, 0, 1, 0};
  Tile tl;
  int kbeg, nsteps, krot = 0;
  if (a.kgroup) {
    // every group: MT x NT tiles of its m_fixed x N output, row tile
    // fastest, reduced over the group's own K range
    const int MT = (a.m_fixed + BM - 1) / BM;
    const int64_t L = blockIdx.x;
    if (L >= (int64_t)a.G * MT * NT) return;
    const int64_t per = (int64_t)MT * NT;
    const int gl = (int)(L / per);
    tl.g = a.kg0 + gl;
    const int64_t rem = L - (int64_t)gl * per;
    tl.nt = (int)(rem / MT);
    tl.mt = (int)(rem - (int64_t)tl.nt * MT);
    tl.m_valid = min(BM, a.m_fixed - tl.mt * BM);
    tl.a_row = (int64_t)tl.mt * BM;
    tl.o_row = tl.a_row;
    kbeg = __builtin_amdgcn_readfirstlane(a.ktab[tl.g] / BK);
    nsteps = __builtin_amdgcn_readfirstlane(a.ktab[a.kt_size + tl.g] / BK);
    wk.L = L;
  } else {
    // The tile table (4G + 1 ints, at most 16.4 KiB) is staged in LDS by
    // one parallel load, at kTableOff, which no copy touches before the
    // first barrier; the group search then runs on LDS instead of a chain
    // of dependent global loads.
    // With claim counters, the claim on the workgroup's own run is issued
    // with the table load, so that its latency hides behind the load's;
    // the work then reaches the other waves through the last 32 bytes of
    // LDS, which no copy touches before the tile's first barrier.
    int32_t* gt = reinterpret_cast<int32_t*>(smem + kTableOff);
    unsigned long long own = 0;
    if (a.claims && threadIdx.x == 0) own = atomicAdd(a.claims + (blockIdx.x & 7) * kClaimU64, 1ull);
    for (int i = threadIdx.x; i < 4 * a.G + 1; i += 512) gt[i] = a.gtab[i];
    __syncthreads();
    if (a.claims) {
      Work* slot_w = reinterpret_cast<Work*>(smem + kPPLds - 32);
      if (threadIdx.x == 0) {
        int64_t V, whole;
        int s;
        split_shape(a, gt[a.G], NT, nk, V, whole, s);
        *slot_w = claim_work(a.claims, own, blockIdx.x, V, whole, s);
      }
      __syncthreads();
      wk = *slot_w;
    } else {
      wk = plan_work(a, gt[a.G], NT, nk, blockIdx.x);
    }
    if (wk.L < 0) return;
    tl = tile_of(a, gt, NT, wk.L, BM);
    // part `part` of K; a whole tile of a routed group starts at slice
    // g*nk/8 and wraps around
    kbeg = (int)((int64_t)wk.part * nk / wk.parts);
    nsteps = (int)((int64_t)(wk.part + 1) * nk / wk.parts) - kbeg;
    if (wk.parts == 1 && a.rotate_k && tl.g < a.E_routed) krot = (int)(((int64_t)tl.g * nk / 8) % nk);
  }
  // Tile fields are workgroup-uniform; saying so keeps the buffer
  // descriptors in scalar registers.
  tl.g = __builtin_amdgcn_readfirstlane(tl.g);
  tl.nt = __builtin_amdgcn_readfirstlane(tl.nt);
  tl.m_valid = __builtin_amdgcn_readfirstlane(tl.m_valid);
  tl.a_row = ((int64_t)__builtin_amdgcn_readfirstlane((int)(tl.a_row >> 32)) << 32) |
             (uint32_t)__builtin_amdgcn_readfirstlane((int)tl.a_row);
  tl.o_row = ((int64_t)__builtin_amdgcn_readfirstlane((int)(tl.o_row >> 32)) << 32) |
             (uint32_t)__builtin_amdgcn_readfirstlane((int)tl.o_row);
  const int part = __builtin_amdgcn_readfirstlane(wk.part);
  const int parts = __builtin_amdgcn_readfirstlane(wk.parts);
  kbeg = __builtin_amdgcn_readfirstlane(kbeg);
  nsteps = __builtin_amdgcn_readfirstlane(nsteps);
  krot = __builtin_amdgcn_readfirstlane(krot);
  // tiles of at most 128 rows have A slices small enough for three A and
  // three B slots; taller tiles take three A and two B slots (two A and
  // three B, the weights given the longer lead, measured the same)
  const int fi = frags_of(tl.m_valid);
  // gathered A rows: SwiGLU mode only; K-major B: plain mode only (the
  // dx-gathering epilogue always reads W_router K-major)
  if constexpr (SWIGLU) {
    if (a.a_map)
      tile_dispatch_pp<SWIGLU, true, false, EPI>(a, tl, fi, kbeg, nsteps, krot, part, parts, wk.slot, smem);
    else
      tile_dispatch_pp<SWIGLU, false, false, EPI>(a, tl, fi, kbeg, nsteps, krot, part, parts, wk.slot, smem);
  } else if constexpr (EPI == kEpiDxGather) {
    tile_dispatch_pp<SWIGLU, false, true, EPI>(a, tl, fi, kbeg, nsteps, krot, part, parts, wk.slot, smem);
  } else {
    if (a.b_kmajor)
      tile_dispatch_pp<SWIGLU, false, true, EPI>(a, tl, fi, kbeg, nsteps, krot, part, parts, wk.slot, smem);
    else
      tile_dispatch_pp<SWIGLU, false, false, EPI>(a, tl, fi, kbeg, nsteps, krot, part, parts, wk.slot, smem);
  }
}

template <bool SWIGLU, int FI, int EPI>
__device__ __forceinline__ void reduce_body_pp(const GroupedGemmArgs& a, const Tile& tl, int s,
                                               int64_t slot, int w) {
  const int lane = threadIdx.x & 63;
  floatx16 acc[FI][2];
  const float* P0 = a.partials + slot * s * (int64_t)(256 * 256);
  // per row fragment: the 8 loads of a part issued together, parts added in
  // part order (the sum is the same for every launch)
#pragma unroll
  for (int i = 0; i < FI; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int p = 0; p < s; ++p) {
      const float* P = P0 + p * (int64_t)(256 * 256);
      floatx4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const floatx4*>(P + part_off_pp<FI>(w, i * 8 + u, lane));
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * r4 + e] += v[j * 4 + r4][e];
    }
  }
  store_tile_pp<SWIGLU, FI, EPI>(acc, tl, lane, w >> 2, w & 3, out_map(a, tl.g), a.N);
}

template <bool SWIGLU, int EPI>
__device__ __forceinline__ void reduce_dispatch_pp(const GroupedGemmArgs& a, const Tile& tl, int fi,
                                                   int s, int64_t slot, int w) {
  if (fi == 4)
    reduce_body_pp<SWIGLU, 4, EPI>(a, tl, s, slot, w);
  else if (fi == 3)
    reduce_body_pp<SWIGLU, 3, EPI>(a, tl, s, slot, w);
  else if (fi == 2)
    reduce_body_pp<SWIGLU, 2, EPI>(a, tl, s, slot, w);
  else
    reduce_body_pp<SWIGLU, 1, EPI>(a, tl, s, slot, w);
}

// One wave per workgroup: workgroup 8 * slot + w sums and stores the part
// of split tile `slot` that wave w of the product computed (the epilogue
// is per wave), so the r split tiles occupy 8r compute units, not r.
template <bool SWIGLU, int EPI>
__global__ __launch_bounds__(64) void gemm_pp_reduce_kernel(GroupedGemmArgs a) {
  const int NT = SWIGLU ? a.N / 128 : (a.N + BN - 1) / BN;
  const int nk = a.K / BK;
  int64_t V, whole;
  int s;
  split_shape(a, a.gtab[a.G], NT, nk, V, whole, s);
  const int64_t slot = blockIdx.x >> 3;
  if (s < 2 || whole + slot >= V) return;
  const Tile tl = tile_of(a, a.gtab, NT, whole + slot, BM);
  reduce_dispatch_pp<SWIGLU, EPI>(a, tl, frags_of(tl.m_valid), s, slot, (int)(blockIdx.x & 7));
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
  int kbeg = 0, klen = a.K;
  if (a.kgroup) {
    // every group: MT x NT tiles of its m_fixed x N output, row tile
    // fastest, reduced over the group's own K range
    const int MT = (a.m_fixed + FBM - 1) / FBM;
    const int64_t L = blockIdx.x;
    if (L >= (int64_t)a.G * MT * NT) return;
    const int64_t per = (int64_t)MT * NT;
    const int gl = (int)(L / per);
    tl.g = a.kg0 + gl;
    const int64_t rem = L - (int64_t)gl * per;
    tl.nt = (int)(rem / MT);
    tl.mt = (int)(rem - (int64_t)tl.nt * MT);
    tl.m_valid = min(FBM, a.m_fixed - tl.mt * FBM);
    tl.a_row = (int64_t)tl.mt * FBM;
    tl.o_row = tl.a_row;
    kbeg = a.ktab[tl.g];
    klen = a.ktab[a.kt_size + tl.g];
  } else {
    const int64_t L = plain_tile(a, NT, blockIdx.x);
    if (L < 0) return;
    tl = tile_of(a, a.gtab, NT, L, FBM);
  }
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int N = a.N;
  const bool shared = !a.kgroup && tl.g >= a.E_routed;
  const bool a_shared = shared && !a.a_from_out_rows;
  const float* A = (const float*)(a_shared ? a.A_shared : a.A);
  const int lda = a_shared ? a.lda_shared : a.lda;
  const int64_t ldb = a.ldb ? a.ldb : a.K;
  const float* B0 = (const float*)(shared ? a.B0s : a.B0);
  const float* B1 = (const float*)(shared ? a.B1s : a.B1);
  if (!shared && !a.kgroup) {
    B0 += (int64_t)tl.g * a.b_stride;
    if (SWIGLU || a.b_split) B1 += (int64_t)tl.g * a.b_stride;
  }
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int ar = lr < tl.m_valid ? lr : tl.m_valid - 1;
  const float* ap = A + (tl.a_row + ar) * lda + lk;
  const int64_t n0 = (int64_t)tl.nt * FBN;
  // b_split: B rows [0, N/2) from B0, [N/2, N) from B1 (64-row tiles never
  // straddle N/2, a multiple of 64)
  const float* bp;
  if (!SWIGLU && a.b_split && n0 >= N / 2)
    bp = B1 + (n0 - N / 2 + lr) * ldb + lk;
  else
    bp = B0 + (n0 + lr) * ldb + lk;
  const float* b3p = SWIGLU ? B1 + (n0 + lr) * ldb + lk : nullptr;

  float acc[4][4], acc3[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = acc3[i][c] = 0.f;

  for (int k0 = kbeg; k0 < kbeg + klen; k0 += FBK) {
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
  // output row r of the group: out0 + r*ldo, or out1 + (r - split_rows)*ldo
  // from split_rows on; groups split along K write group g at
  // (g - kg0)*out_stride
  const int64_t go = a.kgroup ? (int64_t)(tl.g - a.kg0) * a.out_stride : 0;
  float* out0 = (float*)a.out + go;
  float* out1 = a.out1 ? (float*)a.out1 + go : nullptr;
  const int64_t split = (a.out1 && a.split_rows > 0) ? a.split_rows : INT64_MAX;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= tl.m_valid) continue;
    const int64_t r = tl.o_row + row;
    float* orow = r < split ? out0 + r * a.ldo : out1 + (r - split) * a.ldo;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t col = n0 + tx + 16 * c;
      float v = acc[i][c];
      if (SWIGLU) {
        if (a.out13) {             // the pre-activations a1 and a3 as well
          float* r13 = (float*)a.out13 + r * a.ld13;
          r13[col] = acc[i][c];
          r13[N + col] = acc3[i][c];
        }
        v = v / (1.f + expf(-v)) * acc3[i][c];
      }
      orow[col] = v;
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm(int dtype, bool swiglu, const GroupedGemmArgs& a,
                               hipStream_t s) {
  if (dtype == 1) {
    // the ping-pong kernel: whole tiles plus at most num_cu split-part
    // workgroups, then (with split tiles) the reduce; groups split along K:
    // exactly G x MT x NT tiles
    const int NT = swiglu ? a.N / 128 : (a.N + BN - 1) / BN;
    const int64_t nb = a.kgroup ? (int64_t)a.G * ((a.m_fixed + BM - 1) / BM) * NT
                                : pp_workgroups(a, NT);
    if (nb <= 0) return hipSuccess;
    if (swiglu)
      MOE_LAUNCH((gemm_pp_kernel<true, kEpiPlain>), dim3((unsigned)nb), dim3(512), 0, s, a);
    else if (a.dsw_a13)
      MOE_LAUNCH((gemm_pp_kernel<false, kEpiDSwiglu>), dim3((unsigned)nb), dim3(512), 0, s, a);
    else if (a.dxg)
      MOE_LAUNCH((gemm_pp_kernel<false, kEpiDxGather>), dim3((unsigned)nb), dim3(512), 0, s, a);
    else
      MOE_LAUNCH((gemm_pp_kernel<false, kEpiPlain>), dim3((unsigned)nb), dim3(512), 0, s, a);
    if (a.partials && !a.kgroup) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (swiglu)
        MOE_LAUNCH((gemm_pp_reduce_kernel<true, kEpiPlain>), dim3((unsigned)a.num_cu * 8), dim3(64), 0, s, a);
      else if (a.dsw_a13)
        MOE_LAUNCH((gemm_pp_reduce_kernel<false, kEpiDSwiglu>), dim3((unsigned)a.num_cu * 8), dim3(64), 0, s, a);
      else if (a.dxg)
        MOE_LAUNCH((gemm_pp_reduce_kernel<false, kEpiDxGather>), dim3((unsigned)a.num_cu * 8), dim3(64), 0, s, a);
      else
        MOE_LAUNCH((gemm_pp_reduce_kernel<false, kEpiPlain>), dim3((unsigned)a.num_cu * 8), dim3(64), 0, s, a);
    }
  } else {
    const int NT = a.N / FBN;
    const int64_t nb = a.kgroup ? (int64_t)a.G * ((a.m_fixed + FBM - 1) / FBM) * NT
                                : a.max_m_tiles * NT;
    if (nb <= 0) return hipSuccess;
    if (swiglu)
      MOE_LAUNCH(gemm_f32_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, a);
    else
      MOE_LAUNCH(gemm_f32_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
