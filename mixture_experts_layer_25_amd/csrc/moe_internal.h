// Internal launchers of the libmoe kernels (host side, not part of the ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

// Timing of one stage of a timed moe_forward call: the first kernel the
// stage launches takes `start` and every kernel takes `stop`, bound to the
// kernels themselves (hipExtLaunchKernel), so the pair spans the stage's
// kernels from the first one's start to the last one's end, without the
// gaps of separately recorded markers.  Set for the duration of one stage
// on the calling thread only; NULL otherwise.
struct StageEvents {
  hipEvent_t start, stop;
  int launched;   // kernels launched in the stage so far
};

inline StageEvents*& stage_events() {
  static thread_local StageEvents* cur = nullptr;
  return cur;
}

// Every kernel launch of the library goes through this: a plain launch, or
// one carrying the current stage's events.
#define MOE_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                \
  do {                                                                                   \
    ::moe::StageEvents* moe_ev_ = ::moe::stage_events();                                 \
    if (moe_ev_) {                                                                       \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM,                          \
                            moe_ev_->launched ? nullptr : moe_ev_->start, moe_ev_->stop, \
                            0u, __VA_ARGS__);                                            \
      ++moe_ev_->launched;                                                               \
    } else {                                                                             \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);               \
    }                                                                                    \
  } while (0)

// Tile table written by the scan kernels and read by the grouped GEMMs.
// For G groups it holds 4*G+1 int32:
//   [0 .. G]        exclusive prefix of row tiles per group (entry G = total)
//   [G+1 .. 2G]     first A row of each group
//   [2G+1 .. 3G]    rows computed in each group
//   [3G+1 .. 4G]    first output row of each group
// then, from int gtab_claims_off(G) (a multiple of 32), kClaimBlocks claim
// blocks: the work-claim counters of one bf16 grouped GEMM launch each,
// kClaimCounters uint64 kClaimStride bytes apart (each in a memory line of
// its own): one per XCD run of whole tiles, counting the tiles taken from
// its front in the low half and from its back in the high half, then the
// split parts taken.  Every kernel that writes a tile table zeroes its
// claim blocks; a launch uses a block of its own.
constexpr int kClaimBlocks = 4;
constexpr int kClaimCounters = 9;
constexpr int kClaimStride = 256;
constexpr int kClaimBlockInts = kClaimCounters * kClaimStride / 4;
constexpr int64_t gtab_claims_off(int G) { return (4 * (int64_t)G + 1 + 63) / 64 * 64; }
constexpr int64_t gtab_ints(int G) { return gtab_claims_off(G) + kClaimBlocks * kClaimBlockInts; }
// Claim block i of the tile table `gtab` of G groups; NULL (the launch
// then takes its work by workgroup index) for i outside [0, kClaimBlocks).
inline unsigned long long* claim_block(int32_t* gtab, int G, int i) {
  if (i < 0 || i >= kClaimBlocks) return nullptr;
  return reinterpret_cast<unsigned long long*>(gtab + gtab_claims_off(G) +
                                               (int64_t)i * kClaimBlockInts);
}

// Tiles of the last, partial round of a bf16 grouped GEMM are split along K
// into up to num_cu/r parts whose fp32 partial tiles go to this many floats
// of workspace (num_cu <= 256 parts of 256x256).
constexpr int64_t kSplitPartialFloats = (int64_t)256 * 256 * 256;

struct GroupedGemmArgs {
  const void* A;         // routed-group rows: x_perm (GEMM1) or act (GEMM2)
  const void* A_shared;  // GEMM1: the tokens x for the shared group; else unused
  const void* B0;        // GEMM1: w1 [E,F,h]; GEMM2: w2 [E,h,F]
  const void* B1;        // GEMM1: w3 [E,F,h]; GEMM2: unused
  const void* B0s;       // shared-expert weights (group index E_routed)
  const void* B1s;
  int64_t b_stride;      // elements between consecutive experts' matrices
  void* out;             // act [rows,F] (GEMM1) or y_perm [rows,h] (GEMM2)
  int K;                 // reduction length (h for GEMM1, F for GEMM2)
  int N;                 // output columns (F for GEMM1, h for GEMM2)
  int lda;               // row stride (elements) of A for the routed groups
  int lda_shared;        // row stride of A_shared
  int ldo;               // row stride of out
  int rotate_k;          // 1: routed group g starts its K loop at slice g*nk/8
  int num_cu;            // compute units of the device (tile rounds)
  float* partials;       // split-K partial tiles, kSplitPartialFloats floats
  const int32_t* gtab;
  int G;                 // groups in gtab
  int E_routed;          // groups 0..E_routed-1 use B0/B1, group E_routed B0s/B1s
  int a_from_out_rows;   // 1: A row of a tile = its output row (GEMM2)
  int64_t max_m_tiles;   // host-side bound on the total row tiles
  // Plain (non-SwiGLU) mode only:
  int b_split;           // 1: B rows [0, N/2) from B0, [N/2, N) from B1
  int ldb;               // B row stride in elements (0: K, dense)
  // Groups split along K (weight gradients): every group g has the same
  // m_fixed x N output out + g*out_stride, reduced over its own K range
  // ktab[g] .. ktab[g] + ktab[G+g] (elements, multiples of 64) of A [m_fixed,
  // lda] and B [N, ldb]; no split-K, no rotation; gtab unused.
  int kgroup;
  int m_fixed;
  const int32_t* ktab;   // ktab[g], ktab[kt_size + g] (ktab of kt_size groups)
  int kt_size;
  int kg0;               // first group of this launch (G groups from kg0)
  int64_t out_stride;
  // Output rows at or past split_rows (within a group) go to out1 + the
  // group's offset, row - split_rows (0: no split).
  void* out1;
  int split_rows;
  // SwiGLU mode: also store the pre-activations, a1 at columns [0, N) and
  // a3 at [N, 2N) of out13's output row (row stride ld13), or NULL.
  void* out13;
  int ld13;
  // bf16 plain mode, backward of the SwiGLU (N = F): if set, the product is
  // dU and the tile writes dA1 = dU a3 s (1 + a1 (1 - s)) at columns [0, N)
  // and dA3 = dU a1 s at [N, 2N) of its output row (s = sigmoid(a1); a1 and
  // a3 from row r of dsw_a13, columns [0, N) and [N, 2N), row stride
  // dsw_ld13) instead of dU.
  const void* dsw_a13;
  int dsw_ld13;
  // bf16 plain mode, dx of the layer: if dxg is set, the tile's rows are
  // tokens and output row t is, rounded once, the product plus the dx_perm
  // rows dxg[dxg_assign[t * dxg_k + j]] of its slots j in order (ids
  // outside [0, dxg_rows) skipped) plus, with dxg_shared, dxg[dxg_rows + t]
  // (row stride dxg_ld).
  const void* dxg;
  const int32_t* dxg_assign;
  int dxg_k;
  int dxg_shared;
  int64_t dxg_rows;
  int64_t dxg_ld;
  // bf16 SwiGLU mode: if set, routed row r is row a_map[r] of A (a_rows rows
  // of stride lda, a_rows * lda * 2 < 2^31 bytes): the tokens are gathered
  // by the copies themselves instead of from a dispatch buffer.
  const int32_t* a_map;
  int64_t a_rows;
  // bf16 plain mode: B is stored K-major, element (n, k) at B[k * ldb + n]
  // (a weight read in its own [K, N] layout, no transposed copy); with
  // b_ksplit > 0, K rows [0, b_ksplit) come from B0 and the rest from B1
  // (row k - b_ksplit).  Each operand's rows * ldb * 2 < 2^31 bytes.
  int b_kmajor;
  int b_ksplit;
  // K-major B: K rows each of B0 and B1 holds (0: all of its half); rows
  // past them read as zero.
  int b_krows;
  // bf16, not kgroup: if set, workgroups claim their work through these
  // zeroed counters (a claim block of gtab, used by no other launch since it
  // was zeroed) instead of taking it by workgroup index: workgroup b takes
  // the next tile of XCD run b & 7, once that run is empty the last
  // unclaimed tile of the fullest other run, then the next split part.
  unsigned long long* claims;
};

hipError_t launch_router(int dtype, const void* x, const void* w_router,
                         const float* logit_bias, float* logits, int64_t T,
                         int h, int E, hipStream_t s);

// The router fused with top-k, gates and histogram (bf16 layers of up to 64
// experts, router_topk_fused): writes logits, idx and gates like
// launch_router + launch_topk, and, if chunk_hist is given, one histogram
// row per router_topk_tokens(E) tokens (16 up to 16 experts, else 64; at
// least kRouteFusedTokens, a divisor of kChunkTokens).
constexpr int kRouteFusedTokens = 16;
bool router_topk_fused(int dtype, int E);
int router_topk_tokens(int E);
hipError_t launch_router_topk(const void* x, const void* w_router, const float* logit_bias,
                              float* logits, const float* select_bias, int gate, int64_t T,
                              int h, int E, int k, int32_t* idx, float* gate_out,
                              int32_t* chunk_hist, hipStream_t s);

// Tokens one probability-sum workgroup handles (4 passes of 256/G tokens,
// G = seg_lanes(E)).  Always a divisor of 256.
inline int topk_tokens_per_wg(int E) { return 4 * 256 / seg_lanes(E); }

// Lanes per token of the top-k kernel: one expert per lane up to 64
// experts; 65..256 experts in 16-lane segments (up to 16 experts per lane,
// 16 tokens per wave); more in 64-lane segments.
inline int topk_lanes(int E) { return E <= 64 ? seg_lanes(E) : (E <= 256 ? 16 : 64); }

// Tokens one top-k workgroup handles (4 passes of 256/G tokens, G =
// topk_lanes(E); one pass of 16 for 65..256 experts); its expert histogram
// covers that many tokens.  Always a divisor of 256.
inline int topk_kernel_tokens(int E) {
  return (E > 64 && E <= 256) ? 16 : 4 * 256 / topk_lanes(E);
}

// Routing variants (choice.hip, route_scan.hip).  Expert choice: expert e
// takes its C best tokens by probs_et[e][t]; sel_row/gate_te [T,E],
// row_token [E*C].  Score drop: from the dropless rows (assign_dl,
// offsets_dl) of a top-k routing, expert e keeps its C largest gates;
// key_dl/aid_dl [T*k] scratch, assign_row [T*k], row_token [E*C] (kept
// rows only).
hipError_t launch_expert_choice(const float* probs_et, int64_t T, int E, int C, int32_t* sel_row,
                                float* gate_te, int32_t* row_token, hipStream_t s);
hipError_t launch_score_drop(const int32_t* idx, const float* gate, const int32_t* assign_dl,
                             const int32_t* offsets_dl, int64_t T, int E, int k, int C,
                             uint64_t* key_dl, int32_t* aid_dl, int32_t* assign_row,
                             int32_t* row_token, hipStream_t s);
hipError_t launch_fixed_groups(int E, int C, int64_t T, int has_shared, int BM, int32_t* counts,
                               int32_t* offsets, int32_t* gtab, hipStream_t s);
// Tile table for the backward from the forward's counts and offsets:
// valid rows min(count, C) (C = 0: count) at offsets[e], plus the shared
// group (T rows read from x, written after the routed rows).
hipError_t launch_groups_from_counts(const int32_t* counts, const int32_t* offsets, int E,
                                     int64_t C, int64_t T, int has_shared, int BM,
                                     int64_t rows, int32_t* gtab, hipStream_t s);

// Backward kernels (backward.hip); dtype as in the ABI (1: bf16, 0: fp32)
// selects the element type of every tensor argument.
hipError_t launch_transpose(int dtype, const void* src, int64_t src_bs, int R, int Cc, void* dst,
                            int64_t dst_bs, int dld, int col0, int batches, hipStream_t s);
hipError_t launch_ktab(const int32_t* gtab, int G, int use_a_rows, int32_t* kt, hipStream_t s);
hipError_t launch_transpose_groups(int dtype, const void* src, int sld, const void* src_shared,
                                   int sld_shared, int E_routed, const int32_t* kt, int G,
                                   int Cc, int64_t ktot_bound, void* dst, int dld,
                                   hipStream_t s);
hipError_t launch_scatter_dy(int dtype, const void* dy, const int32_t* assign_row,
                             const float* gate, const int32_t* counts, int64_t T, int h, int E,
                             int k, int64_t C, int64_t rows, int has_shared, void* dO, int ld,
                             hipStream_t s);
hipError_t launch_gate_grad(int dtype, const void* dy, const void* o, int ld,
                            const int32_t* assign_row, int64_t rows, int64_t T, int h, int k,
                            float* dg, hipStream_t s);
hipError_t launch_swiglu_fwd(int dtype, const void* a13, int lda13, int64_t rows, int F, void* u,
                             int ldu, hipStream_t s);
hipError_t launch_swiglu_bwd(int dtype, const void* a13, int lda13, const void* dU, int ldu,
                             int64_t rows, int F, void* dA, int ldda, hipStream_t s);
// rpart: 32 * E * h floats of slice sums for dw_router.
hipError_t launch_router_bwd(int dtype, const float* logits, const int32_t* idx,
                             const float* gate, const float* dg, int gate_mode, int64_t T, int E,
                             int k, const void* x, int h, float* dl, float* rpart,
                             void* dw_router, float* dlogit_bias, hipStream_t s);
// dl from dg alone (the first step of launch_router_bwd), and with dl_hl
// also dl as bf16 parts hi + lo (hi = dl rounded, lo = the rest rounded):
// dl_hl [T][2Ep] holds [hi | lo] per token and dlT_hl [Ep][2Tp] [hi | lo]
// per expert (token-contiguous), zero past E experts and T tokens (Ep, Tp
// multiples of 64).
hipError_t launch_gates_bwd(const float* logits, const int32_t* idx, const float* gate,
                            const float* dg, int gate_mode, int64_t T, int E, int k, float* dl,
                            uint16_t* dl_hl, int Ep, uint16_t* dlT_hl, int64_t Tp,
                            hipStream_t s);
hipError_t launch_bias_grad(const float* dl, int64_t T, int E, float* dlogit_bias,
                            hipStream_t s);
// Tile table of a single group of `rows` rows (A and output rows from 0).
hipError_t launch_single_group_gtab(int32_t* gtab, int64_t rows, int BM, hipStream_t s);
hipError_t launch_dx_final(int dtype, const void* dxp, int ldp, const int32_t* assign_row, int k,
                           int64_t rows, int has_shared, const float* dl, const void* w_router,
                           int64_t T, int h, int E, void* dx, hipStream_t s);

hipError_t launch_gather_rows(int dtype, const void* x, const int32_t* row_token, int64_t rows,
                              int64_t T, int h, void* x_perm, int ld_perm, hipStream_t s);

// Router distribution summed per expert over token groups (partial:
// [ceil(T / topk_tokens_per_wg(E))][E] floats), then f, P and the Switch
// loss (one workgroup).
hipError_t launch_select_bias_update(const int32_t* counts, int64_t T, int E, int k, float gamma,
                                     float* bias, hipStream_t st);
hipError_t launch_load_balance(const float* logits, const int32_t* counts, int gate, int64_t T,
                               int E, int k, float alpha, float* partial, float* f, float* P,
                               float* loss, hipStream_t st);
// The router distribution itself, written transposed: probs_et [E,T].
hipError_t launch_router_probs(const float* logits, int gate, int64_t T, int E, float* probs_et,
                               hipStream_t st);

// Sinkhorn routing (sinkhorn.hip): bias[E] = ln of the column factors of
// iters row/column scalings of exp(logits).  parts: 2 * sinkhorn_blocks(T,
// E) * E float2 of scratch.
int sinkhorn_blocks(int64_t T, int E);
hipError_t launch_sinkhorn(const float* logits, int64_t T, int E, int iters, float2* parts,
                           float* bias, hipStream_t s);

hipError_t launch_topk(const float* logits, const float* select_bias,
                       int gate, int64_t T, int E, int k, int32_t* idx,
                       float* gate_out, int32_t* hist, hipStream_t s);

hipError_t launch_hist(const int32_t* idx, int64_t T, int E, int k,
                       int32_t* chunk_hist, hipStream_t s);

// hist/base: one row of E counts per group of hg tokens (hg divides 256).
// pad_row_token (capacity layout, or NULL): its padding rows are set to -1
// (for callers whose permute, which also does so, does not run).
hipError_t launch_scan(const int32_t* hist, int64_t ngroups, int E,
                       int64_t C, int64_t T, int k, int has_shared, int BM,
                       int32_t* base, int32_t* counts, int32_t* offsets,
                       int32_t* gtab, hipStream_t s, int32_t* pad_row_token = nullptr);

hipError_t launch_assign(const int32_t* idx, const int32_t* base, int hg,
                         const int32_t* offsets, int64_t T, int E, int k,
                         int64_t C, int32_t* assign_row, int32_t* row_token,
                         hipStream_t s);

// x_perm rows are ld_perm elements apart (>= h).
hipError_t launch_permute(int dtype, const void* x, const int32_t* assign_row,
                          const int32_t* counts, int64_t T, int h, int E,
                          int k, int64_t C, void* x_perm, int ld_perm,
                          int32_t* row_token, hipStream_t s);

// Groups from caller-provided counts/offsets, clamped to rows [0, rows).
hipError_t launch_gtab(const int32_t* counts, const int32_t* offsets, int E,
                       int BM, int rows, int32_t* gtab, hipStream_t s);

hipError_t launch_grouped_gemm(int dtype, bool swiglu,
                               const GroupedGemmArgs& a, hipStream_t s);

// y_perm and shared_y rows are ld_perm elements apart (>= h); slots whose
// row is outside [0, nrows) contribute nothing.
hipError_t launch_combine(int dtype, const void* y_perm, int ld_perm,
                          const int32_t* assign_row, const float* gate,
                          const void* shared_y, void* y, int64_t T, int h,
                          int k, int64_t nrows, hipStream_t s);

}  // namespace moe
