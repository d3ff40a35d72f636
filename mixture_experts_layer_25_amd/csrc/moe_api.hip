// libmoe C ABI: argument checks, workspace layout and launch sequencing.
// The operations themselves are documented in include/moe.h.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "moe_device.h"
#include "moe_internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

using moe::gtab_ints;

// Sizes are bounded so that every launch's grid stays below 2^32 work-items
// (the dispatch packet's grid size is 32-bit): some launches run one
// 256-thread workgroup per token, the permute and gather launches 128
// work-items per dispatch row; the grouped GEMMs are checked in grids_fit.
constexpr int64_t kMaxTokens = ((int64_t)1 << 24) - 1;
constexpr int64_t kMaxRows = ((int64_t)1 << 25) - 1;
constexpr uint64_t kMaxWorkItems = 0xFFFFFFFFull;
// Widest h and F: the bf16 GEMM addresses a 64-row block of a ragged group
// through a buffer descriptor with 32-bit extent and offsets.
constexpr int kMaxWidth = 65536;
// Backward: the weight-gradient GEMMs read K-major copies whose rows hold
// every group's rows (padded to 64); 64 of those rows must span < 4 GiB.
constexpr int64_t kMaxBwdKRows = (int64_t)1 << 25;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int esize(const moe_cfg_t& c) { return c.dtype == MOE_DTYPE_BF16 ? 2 : 4; }

int64_t rows_of(const moe_cfg_t& c) {
  return c.capacity > 0 ? (int64_t)c.E * c.capacity : c.T * c.k;
}

// Row strides (elements) of the workspace buffers x_perm / y_perm and act:
// 128 bytes of padding keep consecutive rows of these power-of-two widths
// off the same memory channels.
int ld_h(const moe_cfg_t& c) { return c.h + 128 / esize(c); }
int ld_f(const moe_cfg_t& c) { return c.F + 128 / esize(c); }

// Row stride of the kept pre-activations [a1 | a3] (2F elements + 128 B).
int ld_13(const moe_cfg_t& c) { return 2 * c.F + 128 / esize(c); }
bool saves(const moe_cfg_t& c) { return (c.flags & MOE_FLAG_SAVE_FOR_BACKWARD) != 0; }

int row_tile(const moe_cfg_t& c) {
  return c.dtype == MOE_DTYPE_BF16 ? moe::kGemmBM_bf16 : moe::kGemmBM_f32;
}

// Upper bounds on the work-items of the widest launches (grouped GEMMs,
// the fp32 router: one thread per logit, and for the backward the SwiGLU passes and the
// weight-gradient GEMMs) are below 2^32.  Column tiles are at least 128
// (bf16) or 64 (fp32) wide; the widest GEMM output is max(2F, h).
bool grids_fit(const moe_cfg_t& c, bool backward) {
  const uint64_t T = (uint64_t)c.T, G = (uint64_t)c.E + (uint64_t)c.has_shared;
  const uint64_t rows_all = (uint64_t)rows_of(c) + (c.has_shared ? T : 0);
  const uint64_t BM = (uint64_t)row_tile(c);
  const uint64_t ntile = c.dtype == MOE_DTYPE_BF16 ? 128 : 64;
  const uint64_t wmax = std::max<uint64_t>(2 * (uint64_t)c.F, (uint64_t)c.h);
  const uint64_t m_tiles = (rows_all + BM - 1) / BM + G + 1;
  if ((m_tiles * (wmax / ntile) + 256) * 256 > kMaxWorkItems) return false;
  if (c.dtype == MOE_DTYPE_F32 && T * (uint64_t)c.E > kMaxWorkItems) return false;  // fp32 router
  if (backward) {
    const uint64_t vec = c.dtype == MOE_DTYPE_BF16 ? 8 : 4;
    if (rows_all * ((uint64_t)c.F / vec) + 256 > kMaxWorkItems) return false;
    if (G * ((wmax + BM - 1) / BM) * (wmax / ntile) * 256 > kMaxWorkItems) return false;
  }
  return true;
}

int check_cfg(const moe_cfg_t* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->struct_size != (int32_t)sizeof(moe_cfg_t)) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->gate < MOE_GATE_SOFTMAX_TOPK || c->gate > MOE_GATE_SIGMOID_TOPK_NORM)
    return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->h <= 0 || c->F <= 0 || c->E <= 0 || c->k <= 0 || c->capacity < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->has_shared != 0 && c->has_shared != 1) return MOE_ERR_INVALID_ARG;
  if (c->routing < MOE_ROUTE_TOPK || c->routing > MOE_ROUTE_SINKHORN ||
      (c->flags & ~MOE_FLAG_SAVE_FOR_BACKWARD) != 0)
    return MOE_ERR_INVALID_ARG;
  if (c->sinkhorn_iters < 0 || c->sinkhorn_iters > MOE_MAX_SINKHORN_ITERS ||
      (c->routing == MOE_ROUTE_SINKHORN) != (c->sinkhorn_iters > 0))
    return MOE_ERR_INVALID_ARG;
  if (c->routing == MOE_ROUTE_TOPK_SCORE_DROP && c->capacity <= 0) return MOE_ERR_INVALID_ARG;
  if (c->routing == MOE_ROUTE_EXPERT_CHOICE && c->T > 0 &&
      (c->capacity <= 0 || c->capacity > c->T))
    return MOE_ERR_INVALID_ARG;
  if (c->k > c->E) return MOE_ERR_INVALID_ARG;
  if (c->h % 128 != 0 || c->F % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (c->h > kMaxWidth || c->F > kMaxWidth) return MOE_ERR_UNSUPPORTED;
  if (c->E > 1024 || c->k > 16 || c->E + c->has_shared > 1024) return MOE_ERR_UNSUPPORTED;
  if (c->T > kMaxTokens || c->capacity > kMaxRows) return MOE_ERR_UNSUPPORTED;
  const int64_t rows_all = rows_of(*c) + (c->has_shared ? c->T : 0);
  if (rows_all > kMaxRows) return MOE_ERR_UNSUPPORTED;
  if (!grids_fit(*c, false)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct Layout {
  size_t logits, idx, gate, hist, base, pbal, counts, offsets, assign, rowtok, gtab;
  // routing variants: expert choice (probs, selection rows and gates per
  // (token, expert)); score drop (the dropless maps it ranks within)
  size_t probs, selrow, gatete, offs_dl, gtab_dl, assign_dl, rowtok_dl, key_dl, aid_dl;
  // Sinkhorn routing: the per-block column pairs (two iterations' worth)
  // and the selection bias
  size_t skpart, skbias;
  size_t partials, xperm, act, yperm, a13, total;
};

Layout layout_of(const moe_cfg_t& c) {
  Layout L{};
  const int64_t T = c.T, E = c.E, k = c.k;
  // histogram rows: one per top-k workgroup (the finest grouping used)
  const int hg = moe::topk_tokens_per_wg(c.E);
  const int64_t nch = (T + hg - 1) / hg;
  const int64_t rows = rows_of(c);
  const int64_t rows_all = rows + (c.has_shared ? T : 0);
  const int64_t G = E + c.has_shared;
  const size_t es = (size_t)esize(c);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.logits = take((size_t)(T * E) * 4);
  L.idx = take((size_t)(T * k) * 4);
  L.gate = take((size_t)(T * k) * 4);
  // histogram rows: at most one per kRouteFusedTokens tokens (the fused
  // router's workgroups; the separate top-k kernel's groups are larger)
  const int64_t nrow = (T + moe::kRouteFusedTokens - 1) / moe::kRouteFusedTokens;
  L.hist = take((size_t)(nrow * E) * 4);
  L.base = take((size_t)(nrow * E) * 4);
  L.pbal = take((size_t)(nch * E) * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.assign = take((size_t)(T * k) * 4);
  L.rowtok = take((size_t)rows * 4);
  L.gtab = take((size_t)gtab_ints((int)G) * 4);
  const bool ec = c.routing == MOE_ROUTE_EXPERT_CHOICE;
  const bool sd = c.routing == MOE_ROUTE_TOPK_SCORE_DROP;
  L.probs = take(ec ? (size_t)(T * E) * 4 : 0);
  L.selrow = take(ec ? (size_t)(T * E) * 4 : 0);
  L.gatete = take(ec ? (size_t)(T * E) * 4 : 0);
  L.offs_dl = take(sd ? (size_t)(E + 1) * 4 : 0);
  L.gtab_dl = take(sd ? (size_t)gtab_ints((int)G) * 4 : 0);
  L.assign_dl = take(sd ? (size_t)(T * k) * 4 : 0);
  L.rowtok_dl = take(sd ? (size_t)(T * k) * 4 : 0);
  L.key_dl = take(sd ? (size_t)(T * k) * 8 : 0);
  L.aid_dl = take(sd ? (size_t)(T * k) * 4 : 0);
  const bool sk = c.routing == MOE_ROUTE_SINKHORN;
  L.skpart = take(sk ? (size_t)(2 * moe::sinkhorn_blocks(T, (int)E) * E) * 8 : 0);
  L.skbias = take(sk ? (size_t)E * 4 : 0);
  L.partials = take(c.dtype == MOE_DTYPE_BF16 ? (size_t)moe::kSplitPartialFloats * 4 : 0);
  L.xperm = take((size_t)rows * ld_h(c) * es);
  L.act = take((size_t)rows_all * ld_f(c) * es);
  L.yperm = take((size_t)rows_all * ld_h(c) * es);
  L.a13 = take(saves(c) ? (size_t)rows_all * ld_13(c) * es : 0);
  L.total = off;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int check_ws(const moe_cfg_t& c, void* ws, size_t ws_bytes) {
  const Layout L = layout_of(c);
  if (L.total > 0 && (ws == nullptr || ws_bytes < L.total)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// True if any non-null pointer breaks the 16-byte alignment every entry
// point requires (the kernels move 16-byte vectors).
template <typename... P>
bool misaligned(const P*... p) {
  return ((((uintptr_t)p & 15u) != 0) || ...);
}

#define MOE_TRY(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return MOE_ERR_HIP;       \
  } while (0)

int64_t max_m_tiles(int64_t rows, int64_t groups, int BM) {
  return (rows + BM - 1) / BM + groups;
}

// Compute units of the current device (at most 256: the split-K partial
// buffer holds 256 parts).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n < 256 ? n : 256;
}

void set_split(moe::GroupedGemmArgs& a, const moe_cfg_t& c, void* ws, const Layout& L) {
  a.num_cu = device_cus();
  a.partials = c.dtype == MOE_DTYPE_BF16 ? at<float>(ws, L.partials) : nullptr;
}

}  // namespace

MOE_API const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

MOE_API int moe_capacity(int64_t T, int32_t E, int32_t k, int64_t cf_num,
                         int64_t cf_den, int64_t* C) {
  if (!C || T <= 0 || E <= 0 || k <= 0 || cf_num <= 0 || cf_den <= 0)
    return MOE_ERR_INVALID_ARG;
  const __int128 num = (__int128)cf_num * k * T;
  const __int128 den = (__int128)cf_den * E;
  const __int128 q = (num + den - 1) / den;
  if (q > (__int128)INT64_MAX) return MOE_ERR_UNSUPPORTED;
  *C = (int64_t)q;
  return MOE_OK;
}

MOE_API int moe_num_rows(const moe_cfg_t* cfg, int64_t* rows) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!rows) return MOE_ERR_INVALID_ARG;
  *rows = rows_of(*cfg);
  return MOE_OK;
}

MOE_API int moe_workspace_bytes(const moe_cfg_t* cfg, size_t* bytes) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = layout_of(*cfg).total;
  return MOE_OK;
}

MOE_API int moe_router_topk(const moe_cfg_t* cfg, const void* x, const void* w_router,
                            const float* logit_bias, const float* select_bias,
                            float* logits, int32_t* topk_idx, float* topk_gate,
                            void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const moe_cfg_t& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (c.routing == MOE_ROUTE_EXPERT_CHOICE) return MOE_ERR_UNSUPPORTED;
  const bool sk = c.routing == MOE_ROUTE_SINKHORN;
  if (!x || !w_router || !topk_idx || !topk_gate || (sk && select_bias))
    return MOE_ERR_INVALID_ARG;
  if (misaligned(x, w_router, logit_bias, select_bias, logits, topk_idx, topk_gate, ws))
    return MOE_ERR_INVALID_ARG;
  if ((!logits || sk) && (st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  const Layout L = layout_of(c);
  float* lg = logits ? logits : at<float>(ws, L.logits);
  if (!sk && moe::router_topk_fused(c.dtype, c.E)) {
    MOE_TRY(moe::launch_router_topk(x, w_router, logit_bias, lg, select_bias, c.gate, c.T, c.h,
                                    c.E, c.k, topk_idx, topk_gate, nullptr, s));
    return MOE_OK;
  }
  MOE_TRY(moe::launch_router(c.dtype, x, w_router, logit_bias, lg, c.T, c.h, c.E, s));
  const float* sb = select_bias;
  if (sk) {
    float* bias = at<float>(ws, L.skbias);
    MOE_TRY(moe::launch_sinkhorn(lg, c.T, c.E, c.sinkhorn_iters, at<float2>(ws, L.skpart), bias,
                                 s));
    sb = bias;
  }
  MOE_TRY(moe::launch_topk(lg, sb, c.gate, c.T, c.E, c.k, topk_idx, topk_gate, nullptr, s));
  return MOE_OK;
}

MOE_API int moe_permute(const moe_cfg_t* cfg, const void* x, const int32_t* topk_idx,
                        int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* assign_row, int32_t* row_token, void* x_perm,
                        void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const moe_cfg_t& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (c.routing != MOE_ROUTE_TOPK && c.routing != MOE_ROUTE_SINKHORN) return MOE_ERR_UNSUPPORTED;
  if (!x || !topk_idx || !expert_counts || !expert_offsets || !assign_row || !row_token ||
      !x_perm)
    return MOE_ERR_INVALID_ARG;
  if (misaligned(x, topk_idx, expert_counts, expert_offsets, assign_row, row_token, x_perm, ws))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  const Layout L = layout_of(c);
  const int64_t nch = (c.T + moe::kChunkTokens - 1) / moe::kChunkTokens;
  int32_t* hist = at<int32_t>(ws, L.hist);
  int32_t* base = at<int32_t>(ws, L.base);
  MOE_TRY(moe::launch_hist(topk_idx, c.T, c.E, c.k, hist, s));
  MOE_TRY(moe::launch_scan(hist, nch, c.E, c.capacity, c.T, c.k, 0, row_tile(c), base,
                           expert_counts, expert_offsets, at<int32_t>(ws, L.gtab), s));
  MOE_TRY(moe::launch_assign(topk_idx, base, moe::kChunkTokens, expert_offsets, c.T, c.E,
                             c.k, c.capacity, assign_row, row_token, s));
  MOE_TRY(moe::launch_permute(c.dtype, x, assign_row, expert_counts, c.T, c.h, c.E, c.k,
                              c.capacity, x_perm, c.h, row_token, s));
  return MOE_OK;
}

MOE_API int moe_permute_rows(const moe_cfg_t* cfg, const void* x, const int32_t* assign_row,
                             const int32_t* expert_counts, int32_t* row_token, void* x_perm,
                             void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const moe_cfg_t& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (c.routing == MOE_ROUTE_EXPERT_CHOICE) return MOE_ERR_UNSUPPORTED;
  if (!x || !assign_row || !expert_counts || !row_token || !x_perm) return MOE_ERR_INVALID_ARG;
  if (misaligned(x, assign_row, expert_counts, row_token, x_perm)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(moe::launch_permute(c.dtype, x, assign_row, expert_counts, c.T, c.h, c.E, c.k,
                              c.capacity, x_perm, c.h, row_token, (hipStream_t)stream));
  return MOE_OK;
}

namespace {

// The standalone grouped GEMM (both entry points): groups from the caller's
// counts and offsets into the tile table `gtab` (gtab_ints(E) ints), split-K
// partial tiles (bf16) in `partials` (kSplitPartialFloats floats).
int grouped_gemm_impl(const moe_cfg_t& c, const void* x_perm, const int32_t* expert_counts,
                      const int32_t* expert_offsets, const void* w1, const void* w3,
                      const void* w2, void* act, void* y_perm, int32_t* gtab, float* partials,
                      hipStream_t s) {
  const int BM = row_tile(c);
  const int64_t rows = rows_of(c);
  MOE_TRY(moe::launch_gtab(expert_counts, expert_offsets, c.E, BM, (int)rows, gtab, s));
  moe::GroupedGemmArgs a{};
  a.A = x_perm;
  a.B0 = w1;
  a.B1 = w3;
  a.b_stride = (int64_t)c.F * c.h;
  a.out = act;
  a.K = c.h;
  a.N = c.F;
  a.lda = c.h;
  a.lda_shared = c.h;
  a.ldo = c.F;
  a.rotate_k = 1;
  a.gtab = gtab;
  a.G = c.E;
  a.E_routed = c.E;
  a.a_from_out_rows = 0;
  a.max_m_tiles = max_m_tiles(rows, c.E, BM);
  a.num_cu = device_cus();
  a.partials = c.dtype == MOE_DTYPE_BF16 ? partials : nullptr;
  a.claims = moe::claim_block(gtab, c.E, 0);
  MOE_TRY(moe::launch_grouped_gemm(c.dtype, true, a, s));
  a.claims = moe::claim_block(gtab, c.E, 1);
  a.A = act;
  a.B0 = w2;
  a.B1 = nullptr;
  a.out = y_perm;
  a.K = c.F;
  a.N = c.h;
  a.lda = c.F;
  a.ldo = c.h;
  a.a_from_out_rows = 1;
  MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, a, s));
  return MOE_OK;
}

int check_gemm_args(const moe_cfg_t* cfg, const void* x_perm, const int32_t* expert_counts,
                    const int32_t* expert_offsets, const void* w1, const void* w3,
                    const void* w2, const void* act, const void* y_perm) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!x_perm || !expert_counts || !expert_offsets || !w1 || !w3 || !w2 || !act || !y_perm)
    return MOE_ERR_INVALID_ARG;
  if (misaligned(x_perm, expert_counts, expert_offsets, w1, w3, w2, act, y_perm))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// ---- the grouped GEMM without a caller workspace ------------------------
// File-scope device scratch: the tile table with its claim blocks (room for
// 1024 routed groups + 1) and the split-K partial tiles (at most 256 parts
// of 256 x 256 fp32).
// In host code `scratch` names a host-side stand-in, never the device
// memory: its device address, one per GPU, comes from hipGetSymbolAddress
// (scratch_on_current_device) and only that address reaches a kernel.
constexpr size_t kScratchGtabBytes = (size_t)(moe::gtab_ints(1025) * 4 + 255) / 256 * 256;
constexpr size_t kScratchBytes = kScratchGtabBytes + (size_t)moe::kSplitPartialFloats * 4;
static_assert(kScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "scratch size as documented");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current; NULL if the lookup fails.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

MOE_API int moe_grouped_gemm_swiglu(const moe_cfg_t* cfg, const void* x_perm,
                                    const int32_t* expert_counts,
                                    const int32_t* expert_offsets, const void* w1,
                                    const void* w3, const void* w2, void* act,
                                    void* y_perm, void* ws, size_t ws_bytes,
                                    void* stream) {
  int st = check_gemm_args(cfg, x_perm, expert_counts, expert_offsets, w1, w3, w2, act, y_perm);
  if (st != MOE_OK || cfg->T == 0) return st;
  const moe_cfg_t& c = *cfg;
  if (misaligned(ws)) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  const Layout L = layout_of(c);
  return grouped_gemm_impl(c, x_perm, expert_counts, expert_offsets, w1, w3, w2, act, y_perm,
                           at<int32_t>(ws, L.gtab), at<float>(ws, L.partials),
                           (hipStream_t)stream);
}

MOE_API int moe_grouped_gemm_swiglu_noalloc(const moe_cfg_t* cfg, const void* x_perm,
                                            const int32_t* expert_counts,
                                            const int32_t* expert_offsets, const void* w1,
                                            const void* w3, const void* w2, void* act,
                                            void* y_perm, void* stream) {
  const int st = check_gemm_args(cfg, x_perm, expert_counts, expert_offsets, w1, w3, w2, act,
                                 y_perm);
  if (st != MOE_OK || cfg->T == 0) return st;
  const moe_cfg_t& c = *cfg;
  // the tile table of E groups and (bf16) the partials must fit the scratch
  const size_t need = (size_t)gtab_ints(c.E) * 4 <= kScratchGtabBytes
                          ? kScratchGtabBytes + (c.dtype == MOE_DTYPE_BF16
                                                     ? (size_t)moe::kSplitPartialFloats * 4
                                                     : 0)
                          : kScratchBytes + 1;
  if (need > kScratchBytes) return MOE_ERR_UNSUPPORTED;
  char* sp = static_cast<char*>(scratch_on_current_device());
  if (!sp) return MOE_ERR_HIP;
  return grouped_gemm_impl(c, x_perm, expert_counts, expert_offsets, w1, w3, w2, act, y_perm,
                           reinterpret_cast<int32_t*>(sp),
                           reinterpret_cast<float*>(sp + kScratchGtabBytes), (hipStream_t)stream);
}

MOE_API int moe_unpermute_combine(const moe_cfg_t* cfg, const void* y_perm,
                                  const int32_t* assign_row, const float* topk_gate,
                                  const void* shared_y, void* y, void* stream) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const moe_cfg_t& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (!y_perm || !assign_row || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (misaligned(y_perm, assign_row, topk_gate, shared_y, y)) return MOE_ERR_INVALID_ARG;
  const int slots = c.routing == MOE_ROUTE_EXPERT_CHOICE ? c.E : c.k;
  MOE_TRY(moe::launch_combine(c.dtype, y_perm, c.h, assign_row, topk_gate, shared_y, y,
                              c.T, c.h, slots, rows_of(c), (hipStream_t)stream));
  return MOE_OK;
}

MOE_API int moe_select_bias_update(const moe_cfg_t* cfg, const int32_t* expert_counts,
                                   float gamma, float* select_bias, void* stream) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const moe_cfg_t& c = *cfg;
  if (c.routing != MOE_ROUTE_TOPK && c.routing != MOE_ROUTE_TOPK_SCORE_DROP)
    return MOE_ERR_UNSUPPORTED;
  if (!(gamma - gamma == 0.f)) return MOE_ERR_INVALID_ARG;   // NaN or infinite
  if (c.T == 0) return MOE_OK;
  if (!expert_counts || !select_bias) return MOE_ERR_INVALID_ARG;
  if (misaligned(expert_counts, select_bias)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(moe::launch_select_bias_update(expert_counts, c.T, c.E, c.k, gamma, select_bias,
                                         (hipStream_t)stream));
  return MOE_OK;
}

MOE_API int moe_load_balance(const moe_cfg_t* cfg, const float* logits,
                             const int32_t* expert_counts, float alpha, float* f, float* P,
                             float* aux_loss, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const moe_cfg_t& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (!logits || !expert_counts || !f || !P || !aux_loss) return MOE_ERR_INVALID_ARG;
  if (misaligned(logits, expert_counts, f, P, aux_loss, ws)) return MOE_ERR_INVALID_ARG;
  if (!(alpha == alpha)) return MOE_ERR_INVALID_ARG;     // NaN
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  MOE_TRY(moe::launch_load_balance(logits, expert_counts, c.gate, c.T, c.E, c.k, alpha,
                                   at<float>(ws, layout_of(c).pbal), f, P, aux_loss,
                                   (hipStream_t)stream));
  return MOE_OK;
}

namespace {

// Workspace of moe_backward: tile and K tables, the recomputed and
// backward activations (rows padded like the forward's), the transposed
// weights, and the K-major copies the weight-gradient GEMMs read; tensors
// are in the layer's element type (2 or 4 bytes).
struct BwdLayout {
  size_t gtab, kta, kto, rowtok, dg, dl, rpart, partials, xp, a13, u, o, dO, dU, dA, dxp;
  size_t dl_hl, dlT_hl, gt_router, gt_tokens;
  int Ep;
  int64_t Tp;
  size_t w2t, w13t, dOT, uT, dAT, xpT, total;
  int ldh, ldf, ld13;
  int64_t ktb;
  size_t esz;
};

// bf16 backward: the input-gradient GEMMs may read w2 (for dU) and [w1; w3]
// (for dx_perm) in their own [K, N] layouts (K-major B operand) instead of
// transposed copies.  The transposing LDS reads cost GEMM time in proportion
// to the dispatch rows, the transposes in proportion to the weights, so each
// weight is read K-major up to a number of dispatch rows per expert.  With
// the transposes at ~5 TB/s, the GEMMs at ~1.1 PFLOP/s and the transposing
// reads adding ~43 % to dU's GEMM and ~31 % to dx_perm's, the two costs meet
// near 1000 rows per expert for w2 and 1400 for [w1; w3] (measured: [w1; w3]
// K-major saves 3 % of the backward at 1280 rows per expert and costs 2 %
// at 2048).
constexpr int64_t kKmajorRowsW2 = 512, kKmajorRowsW13 = 1536;
bool kmajor_ok(const moe_cfg_t& c) {
  return c.dtype == MOE_DTYPE_BF16 && (int64_t)c.F * c.h * 2 < ((int64_t)1 << 31);
}
bool kmajor_w2(const moe_cfg_t& c) {
  return kmajor_ok(c) && rows_of(c) <= kKmajorRowsW2 * c.E;
}
bool kmajor_w13(const moe_cfg_t& c) {
  return kmajor_ok(c) && rows_of(c) <= kKmajorRowsW13 * c.E;
}

// bf16 backward: the router's gradients (dl^T x and dl W_router, with dl
// as bf16 hi + lo parts) run on the grouped GEMM, x read K-major.
bool router_grads_on_gemm(const moe_cfg_t& c) {
  return c.dtype == MOE_DTYPE_BF16 && (int64_t)c.T * c.h * 2 < ((int64_t)1 << 31);
}

BwdLayout bwd_layout_of(const moe_cfg_t& c) {
  BwdLayout L{};
  const int64_t T = c.T, E = c.E, k = c.k, h = c.h, F = c.F;
  const int64_t G = E + c.has_shared;
  const int64_t rows = rows_of(c);
  const int64_t rows_all = rows + (c.has_shared ? T : 0);
  L.ldh = (int)h + 64;
  L.ldf = (int)F + 64;
  L.ld13 = 2 * (int)F + 64;
  L.ktb = (rows_all + 64 * G + 63) / 64 * 64;   // every group's rows rounded up to 64
  L.esz = c.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const size_t es = L.esz;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.gtab = take((size_t)gtab_ints((int)G) * 4);
  L.kta = take((size_t)(4 * G) * 4);
  L.kto = take((size_t)(4 * G) * 4);
  L.rowtok = take((size_t)rows * 4);
  const int64_t slots = c.routing == MOE_ROUTE_EXPERT_CHOICE ? E : k;   // gates per token
  L.dg = take((size_t)(T * slots) * 4);
  L.dl = take((size_t)(T * E) * 4);
  const bool rg = router_grads_on_gemm(c);
  L.rpart = take(rg ? 0 : (size_t)(32 * E * h) * 4);
  L.partials = take((size_t)moe::kSplitPartialFloats * 4);
  L.xp = take((size_t)rows * L.ldh * es);
  L.a13 = take((size_t)rows_all * L.ld13 * es);
  L.u = take((size_t)rows_all * L.ldf * es);
  L.o = take((size_t)rows_all * L.ldh * es);
  L.dO = take((size_t)rows_all * L.ldh * es);
  L.dU = take(c.dtype == MOE_DTYPE_BF16 ? 0 : (size_t)rows_all * L.ldf * es);
  L.dA = take((size_t)rows_all * L.ld13 * es);
  L.dxp = take((size_t)rows_all * L.ldh * es);
  L.w2t = take(kmajor_w2(c) ? 0 : (size_t)(G * F * h) * es);   // transposed copies
  L.w13t = take(kmajor_w13(c) ? 0 : (size_t)(G * h * 2 * F) * es);
  L.dOT = take((size_t)(h * L.ktb) * es);
  L.uT = take((size_t)(F * L.ktb) * es);
  L.dAT = take((size_t)(2 * F * L.ktb) * es);
  L.xpT = take((size_t)(h * L.ktb) * es);
  L.Ep = (int)((E + 63) / 64 * 64);
  L.Tp = (T + 63) / 64 * 64;
  L.dl_hl = take(rg ? (size_t)(T * 2 * L.Ep) * 2 : 0);
  L.dlT_hl = take(rg ? (size_t)(L.Ep * 2 * L.Tp) * 2 : 0);
  L.gt_router = take(rg ? (size_t)gtab_ints(1) * 4 : 0);
  L.gt_tokens = take(rg ? (size_t)gtab_ints(1) * 4 : 0);
  L.total = off;
  return L;
}

}  // namespace

MOE_API int moe_backward_workspace_bytes(const moe_cfg_t* cfg, size_t* bytes) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  if (cfg->T == 0) {
    *bytes = 0;
    return MOE_OK;
  }
  const BwdLayout L = bwd_layout_of(*cfg);
  if (L.ktb >= kMaxBwdKRows || !grids_fit(*cfg, true)) return MOE_ERR_UNSUPPORTED;
  *bytes = L.total;
  return MOE_OK;
}

namespace {

// Activations a forward call kept for the backward (pointers and row
// strides in elements): the dispatch buffer, [a1 | a3], the activations and
// the expert outputs.
struct Saved {
  const void* xp;
  int ldxp;
  const void* a13;
  int ld13;
  const void* u;
  int ldu;
  const void* o;
  int ldo;
};

// The backward; sv NULL: the activations are recomputed into ws.
int backward_impl(const moe_cfg_t& c, const moe_weights_t* w, const void* x, const void* dy,
                  const moe_route_out_t* route, const moe_grads_t* grads, void* ws,
                  size_t ws_bytes, void* stream, const Saved* sv) {
  if (c.T == 0) return MOE_OK;
  // expert choice: the E experts are each token's slots (assign_row and
  // topk_gate [T,E] as the forward wrote them; no topk_idx)
  const bool ec = c.routing == MOE_ROUTE_EXPERT_CHOICE;
  if (!w || !x || !dy || !route || !grads || !w->w_router || !w->w1 || !w->w3 || !w->w2)
    return MOE_ERR_INVALID_ARG;
  const moe_route_out_t& r = *route;
  const moe_grads_t& gr = *grads;
  if (!r.logits || (!ec && !r.topk_idx) || !r.topk_gate || !r.expert_counts ||
      !r.expert_offsets || !r.assign_row || !gr.dx || !gr.dw1 || !gr.dw3 || !gr.dw2)
    return MOE_ERR_INVALID_ARG;
  if (c.has_shared && (!w->ws1 || !w->ws3 || !w->ws2 || !gr.dws1 || !gr.dws3 || !gr.dws2))
    return MOE_ERR_INVALID_ARG;
  if (misaligned(x, dy, ws, w->w_router, w->w1, w->w3, w->w2, w->ws1, w->ws3) ||
      misaligned(w->ws2, r.logits, r.topk_idx, r.topk_gate, r.expert_counts, r.expert_offsets,
                 r.assign_row) ||
      misaligned(gr.dx, gr.dw_router, gr.dlogit_bias, gr.dw1, gr.dw3, gr.dw2, gr.dws1, gr.dws3,
                 gr.dws2) ||
      misaligned(gr.dgate))
    return MOE_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout_of(c);
  if (L.ktb >= kMaxBwdKRows || !grids_fit(c, true)) return MOE_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  const int E = c.E, h = c.h, F = c.F;
  const int k = ec ? c.E : c.k;        // gate slots per token
  const int G = E + c.has_shared;
  const int64_t T = c.T;
  const int64_t rows = rows_of(c);
  const int64_t rows_all = rows + (c.has_shared ? T : 0);
  const int BM = row_tile(c);
  int32_t* gtab = at<int32_t>(ws, L.gtab);
  int32_t* kta = at<int32_t>(ws, L.kta);
  int32_t* kto = at<int32_t>(ws, L.kto);
  float* dg = gr.dgate ? gr.dgate : at<float>(ws, L.dg);
  float* dl = at<float>(ws, L.dl);
  // recomputed (or kept) activations and their row strides
  const void* xp = at<char>(ws, L.xp);
  const void* a13 = at<char>(ws, L.a13);
  const void* u = at<char>(ws, L.u);
  const void* o = at<char>(ws, L.o);
  int ldxp = L.ldh, ld13 = L.ld13, ldu = L.ldf, ldo = L.ldh;
  if (sv) {
    xp = sv->xp; ldxp = sv->ldxp;
    a13 = sv->a13; ld13 = sv->ld13;
    u = sv->u; ldu = sv->ldu;
    o = sv->o; ldo = sv->ldo;
  }
  void* dO = at<char>(ws, L.dO);
  void* dU = at<char>(ws, L.dU);
  void* dA = at<char>(ws, L.dA);
  void* dxp = at<char>(ws, L.dxp);
  char* w2t = at<char>(ws, L.w2t);
  char* w13t = at<char>(ws, L.w13t);
  void* dOT = at<char>(ws, L.dOT);
  void* uT = at<char>(ws, L.uT);
  void* dAT = at<char>(ws, L.dAT);
  void* xpT = at<char>(ws, L.xpT);
  const int ktb = (int)L.ktb;

  // groups, K tables, the dispatch buffer
  MOE_TRY(moe::launch_groups_from_counts(r.expert_counts, r.expert_offsets, E, c.capacity, T,
                                         c.has_shared, BM, rows, gtab, s));
  MOE_TRY(moe::launch_ktab(gtab, G, 1, kta, s));
  MOE_TRY(moe::launch_ktab(gtab, G, 0, kto, s));
  if (!sv)
    MOE_TRY(moe::launch_permute(c.dtype, x, r.assign_row, r.expert_counts, T, h, E, k,
                                c.capacity, at<char>(ws, L.xp), L.ldh, at<int32_t>(ws, L.rowtok),
                                s));
  // transposed weights (unless the GEMMs read them K-major): w2t[g] =
  // w2[g]^T [F,h]; w13t[g] = [w1[g]^T | w3[g]^T] [h,2F]
  const bool km2 = kmajor_w2(c), km13 = kmajor_w13(c);
  if (!km2) {
    MOE_TRY(moe::launch_transpose(c.dtype, w->w2, (int64_t)h * F, h, F, w2t, (int64_t)F * h, h, 0,
                                  E, s));
    if (c.has_shared)
      MOE_TRY(moe::launch_transpose(c.dtype, w->ws2, 0, h, F, w2t + (size_t)E * F * h * L.esz, 0,
                                    h, 0, 1, s));
  }
  if (!km13) {
    MOE_TRY(moe::launch_transpose(c.dtype, w->w1, (int64_t)F * h, F, h, w13t, (int64_t)h * 2 * F,
                                  2 * F, 0, E, s));
    MOE_TRY(moe::launch_transpose(c.dtype, w->w3, (int64_t)F * h, F, h, w13t, (int64_t)h * 2 * F,
                                  2 * F, F, E, s));
    if (c.has_shared) {
      MOE_TRY(moe::launch_transpose(c.dtype, w->ws1, 0, F, h, w13t + (size_t)E * h * 2 * F * L.esz,
                                    0, 2 * F, 0, 1, s));
      MOE_TRY(moe::launch_transpose(c.dtype, w->ws3, 0, F, h, w13t + (size_t)E * h * 2 * F * L.esz,
                                    0, 2 * F, F, 1, s));
    }
  }

  moe::GroupedGemmArgs base{};
  base.gtab = gtab;
  base.G = G;
  base.E_routed = E;
  base.max_m_tiles = max_m_tiles(rows, E, BM) + (c.has_shared ? (T + BM - 1) / BM : 0);
  base.num_cu = device_cus();
  base.partials = at<float>(ws, L.partials);
  moe::GroupedGemmArgs a = base;
  if (!sv) {
    // [a1 | a3] = x_perm [w1; w3]^T (the shared group reads x)
    a.A = xp; a.lda = L.ldh; a.A_shared = x; a.lda_shared = h;
    a.B0 = w->w1; a.B1 = w->w3; a.B0s = w->ws1; a.B1s = w->ws3; a.b_split = 1;
    a.b_stride = (int64_t)F * h; a.K = h; a.N = 2 * F; a.out = at<char>(ws, L.a13);
    a.ldo = L.ld13; a.claims = moe::claim_block(gtab, G, 0);
    MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, a, s));
    MOE_TRY(moe::launch_swiglu_fwd(c.dtype, a13, L.ld13, rows_all, F, at<char>(ws, L.u), L.ldf,
                                   s));
    // expert outputs o = u w2^T (the forward's y_perm)
    a = base;
    a.A = u; a.lda = L.ldf; a.a_from_out_rows = 1;
    a.B0 = w->w2; a.B0s = w->ws2; a.b_stride = (int64_t)h * F; a.K = F; a.N = h;
    a.out = at<char>(ws, L.o); a.ldo = L.ldh; a.claims = moe::claim_block(gtab, G, 1);
    MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, a, s));
  }
  // dO rows, gate gradients
  MOE_TRY(moe::launch_scatter_dy(c.dtype, dy, r.assign_row, r.topk_gate, r.expert_counts, T, h, E, k,
                                 c.capacity, rows, c.has_shared, dO, L.ldh, s));
  MOE_TRY(moe::launch_gate_grad(c.dtype, dy, o, ldo, r.assign_row, rows, T, h, k, dg, s));
  // dU = dO w2, then dA, then dx_perm = dA [w1; w3]
  a = base;
  a.A = dO; a.lda = L.ldh; a.a_from_out_rows = 1; a.claims = moe::claim_block(gtab, G, 2);
  if (km2) {          // w2 [h,F] is K-major for dU
    a.B0 = w->w2; a.B0s = w->ws2; a.b_kmajor = 1; a.ldb = F;
  } else {
    a.B0 = w2t; a.B0s = w2t + (size_t)E * F * h * L.esz;
  }
  a.b_stride = (int64_t)F * h;
  a.K = h; a.N = F;
  if (c.dtype == MOE_DTYPE_BF16) {
    // the GEMM's epilogue turns dU into dA itself
    a.out = dA; a.ldo = L.ld13; a.dsw_a13 = a13; a.dsw_ld13 = ld13;
    MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, a, s));
  } else {
    a.out = dU; a.ldo = L.ldf;
    MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, a, s));
    MOE_TRY(moe::launch_swiglu_bwd(c.dtype, a13, ld13, dU, L.ldf, rows_all, F, dA, L.ld13, s));
  }
  a = base;
  a.A = dA; a.lda = L.ld13; a.a_from_out_rows = 1; a.claims = moe::claim_block(gtab, G, 3);
  if (km13) {         // w1, w3 [F,h] are the K-major rows [0,F) and [F,2F)
    a.B0 = w->w1; a.B1 = w->w3; a.B0s = w->ws1; a.B1s = w->ws3;
    a.b_kmajor = 1; a.b_ksplit = F; a.ldb = h; a.b_stride = (int64_t)F * h;
  } else {
    a.B0 = w13t; a.B0s = w13t + (size_t)E * h * 2 * F * L.esz; a.b_stride = (int64_t)h * 2 * F;
  }
  a.K = 2 * F; a.N = h; a.out = dxp; a.ldo = L.ldh;
  MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, a, s));
  // K-major copies of each group's rows, then the weight gradients
  MOE_TRY(moe::launch_transpose_groups(c.dtype, dO, L.ldh, dO, L.ldh, G, kto, G, h, L.ktb, dOT, ktb, s));
  MOE_TRY(moe::launch_transpose_groups(c.dtype, u, ldu, u, ldu, G, kto, G, F, L.ktb, uT, ktb, s));
  MOE_TRY(moe::launch_transpose_groups(c.dtype, dA, L.ld13, dA, L.ld13, G, kto, G, 2 * F, L.ktb, dAT, ktb,
                                       s));
  MOE_TRY(moe::launch_transpose_groups(c.dtype, xp, ldxp, x, h, E, kta, G, h, L.ktb, xpT, ktb, s));
  for (int pass = 0; pass < (c.has_shared ? 2 : 1); ++pass) {
    const bool sh = pass == 1;
    moe::GroupedGemmArgs wg{};
    wg.kgroup = 1; wg.ktab = kto; wg.kt_size = G; wg.kg0 = sh ? E : 0; wg.G = sh ? 1 : E;
    wg.E_routed = wg.G; wg.num_cu = device_cus();
    // dw2[g] [h,F] = dO_g^T u_g
    wg.A = dOT; wg.lda = ktb; wg.m_fixed = h; wg.B0 = uT; wg.ldb = ktb; wg.N = F; wg.K = 0;
    wg.out = sh ? gr.dws2 : gr.dw2; wg.ldo = F; wg.out_stride = (int64_t)h * F;
    MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, wg, s));
    // [dw1; dw3][g] [2F,h] = dA_g^T x_g
    wg.A = dAT; wg.m_fixed = 2 * F; wg.B0 = xpT; wg.N = h;
    wg.out = sh ? gr.dws1 : gr.dw1; wg.out1 = sh ? gr.dws3 : gr.dw3; wg.split_rows = F;
    wg.ldo = h; wg.out_stride = (int64_t)F * h;
    MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, wg, s));
  }
  // router: dl, dw_router, dlogit_bias; then dx
  // expert choice: the probabilities over all E, softmax (mode 1) or
  // normalised sigmoids (mode 2), slot j = expert j
  const int gmode = ec ? (c.gate == MOE_GATE_SIGMOID_TOPK_NORM ? 2 : 1) : c.gate;
  if (!router_grads_on_gemm(c)) {
    MOE_TRY(moe::launch_router_bwd(c.dtype, r.logits, ec ? nullptr : r.topk_idx, r.topk_gate, dg,
                                   gmode, T, E, k, x, h,
                                   dl, at<float>(ws, L.rpart), gr.dw_router, gr.dlogit_bias, s));
    MOE_TRY(moe::launch_dx_final(c.dtype, dxp, L.ldh, r.assign_row, k, rows, c.has_shared, dl,
                                 w->w_router, T, h, E, gr.dx, s));
    return MOE_OK;
  }
  // dl, and dl as bf16 hi + lo parts: [hi | lo] rows of 2*Ep per token and
  // of 2*Tp per expert, so that one bf16 product over K = 2*Ep (or 2*Tp)
  // against W_router (or x) read twice gives dl's products to ~2^-17
  uint16_t* dl_hl = at<uint16_t>(ws, L.dl_hl);
  uint16_t* dlT_hl = at<uint16_t>(ws, L.dlT_hl);
  int32_t* gt_router = at<int32_t>(ws, L.gt_router);
  int32_t* gt_tokens = at<int32_t>(ws, L.gt_tokens);
  const int Ep = L.Ep;
  const int64_t Tp = L.Tp;
  MOE_TRY(moe::launch_gates_bwd(r.logits, ec ? nullptr : r.topk_idx, r.topk_gate, dg, gmode, T, E,
                                k, dl, dl_hl, Ep, dlT_hl, Tp, s));
  moe::GroupedGemmArgs one{};
  one.G = 1;
  one.E_routed = 1;
  one.num_cu = device_cus();
  one.partials = at<float>(ws, L.partials);
  one.b_kmajor = 1;
  one.ldb = h;
  one.N = h;
  one.ldo = h;
  if (gr.dw_router) {
    // dw_router [E,h] = dl^T x: A = dlT_hl [E rows of 2*Tp], B = x (K-major)
    // for K rows [0, Tp) and again for [Tp, 2*Tp)
    MOE_TRY(moe::launch_single_group_gtab(gt_router, E, BM, s));
    moe::GroupedGemmArgs g = one;
    g.gtab = gt_router;
    g.max_m_tiles = (E + BM - 1) / BM;
    g.A = dlT_hl; g.lda = (int)(2 * Tp);
    g.B0 = x; g.B1 = x; g.b_ksplit = (int)Tp; g.b_krows = (int)T;
    g.K = (int)(2 * Tp);
    g.out = gr.dw_router;
    MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, g, s));
  }
  if (gr.dlogit_bias) MOE_TRY(moe::launch_bias_grad(dl, T, E, gr.dlogit_bias, s));
  // dx [T,h] = dl W_router (A = dl_hl [T rows of 2*Ep], B = W_router K-major
  // twice) plus, in the epilogue, each token's dx_perm rows
  MOE_TRY(moe::launch_single_group_gtab(gt_tokens, T, BM, s));
  moe::GroupedGemmArgs g = one;
  g.gtab = gt_tokens;
  g.max_m_tiles = (T + BM - 1) / BM;
  g.A = dl_hl; g.lda = 2 * Ep;
  g.B0 = w->w_router; g.B1 = w->w_router; g.b_ksplit = Ep; g.b_krows = E;
  g.K = 2 * Ep;
  g.out = gr.dx;
  g.dxg = dxp; g.dxg_assign = r.assign_row; g.dxg_k = k; g.dxg_shared = c.has_shared;
  g.dxg_rows = rows; g.dxg_ld = L.ldh;
  MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, g, s));
  return MOE_OK;
}

}  // namespace

MOE_API int moe_backward(const moe_cfg_t* cfg, const moe_weights_t* w, const void* x,
                         const void* dy, const moe_route_out_t* route, const moe_grads_t* grads,
                         void* ws, size_t ws_bytes, void* stream) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  return backward_impl(*cfg, w, x, dy, route, grads, ws, ws_bytes, stream, nullptr);
}

MOE_API int moe_backward_saved(const moe_cfg_t* cfg, const moe_weights_t* w, const void* x,
                               const void* dy, const moe_route_out_t* route, const void* fwd_ws,
                               size_t fwd_ws_bytes, const moe_grads_t* grads, void* ws,
                               size_t ws_bytes, void* stream) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const moe_cfg_t& c = *cfg;
  if (!saves(c) || misaligned(fwd_ws)) return MOE_ERR_INVALID_ARG;
  if (c.T == 0) return MOE_OK;
  const Layout F = layout_of(c);
  if (!fwd_ws || fwd_ws_bytes < F.total) return MOE_ERR_WORKSPACE;
  void* fw = const_cast<void*>(fwd_ws);
  const Saved sv{at<char>(fw, F.xperm), ld_h(c), at<char>(fw, F.a13), ld_13(c),
                 at<char>(fw, F.act), ld_f(c), at<char>(fw, F.yperm), ld_h(c)};
  return backward_impl(c, w, x, dy, route, grads, ws, ws_bytes, stream, &sv);
}

MOE_API int moe_forward(const moe_cfg_t* cfg, const moe_weights_t* w, const void* x,
                        void* y, const moe_route_out_t* route, void* ws,
                        size_t ws_bytes, void* const* events, void* stream) {
  int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const moe_cfg_t& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (!w || !x || !y || !w->w_router || !w->w1 || !w->w3 || !w->w2)
    return MOE_ERR_INVALID_ARG;
  if (c.has_shared && (!w->ws1 || !w->ws3 || !w->ws2)) return MOE_ERR_INVALID_ARG;
  // expert choice ranks by router probability; a selection-only bias has
  // no meaning there
  if (c.routing == MOE_ROUTE_EXPERT_CHOICE && w->select_bias) return MOE_ERR_INVALID_ARG;
  // Sinkhorn routing finds its own selection bias
  if (c.routing == MOE_ROUTE_SINKHORN && w->select_bias) return MOE_ERR_INVALID_ARG;
  if (misaligned(x, y, ws, w->w_router, w->w1, w->w3, w->w2, w->logit_bias, w->select_bias) ||
      misaligned(w->ws1, w->ws3, w->ws2))
    return MOE_ERR_INVALID_ARG;
  if (route && (misaligned(route->logits, route->topk_idx, route->topk_gate, route->expert_counts,
                           route->expert_offsets, route->assign_row, route->row_token) ||
                misaligned(route->probs, route->route_bias)))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(c, ws, ws_bytes)) != MOE_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  const Layout L = layout_of(c);
  const moe_route_out_t none{};
  const moe_route_out_t& r = route ? *route : none;
  float* logits = r.logits ? r.logits : at<float>(ws, L.logits);
  int32_t* idx = r.topk_idx ? r.topk_idx : at<int32_t>(ws, L.idx);
  float* gate = r.topk_gate ? r.topk_gate : at<float>(ws, L.gate);
  int32_t* counts = r.expert_counts ? r.expert_counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = r.expert_offsets ? r.expert_offsets : at<int32_t>(ws, L.offsets);
  int32_t* assign = r.assign_row ? r.assign_row : at<int32_t>(ws, L.assign);
  int32_t* rowtok = r.row_token ? r.row_token : at<int32_t>(ws, L.rowtok);
  int32_t* hist = at<int32_t>(ws, L.hist);
  int32_t* base = at<int32_t>(ws, L.base);
  int32_t* gtab = at<int32_t>(ws, L.gtab);
  void* xperm = at<char>(ws, L.xperm);
  void* act = at<char>(ws, L.act);
  void* yperm = at<char>(ws, L.yperm);
  // the router fused with the top-k (bf16, up to 64 experts, plain or
  // score-drop token choice): one histogram row per router workgroup
  const bool fused = moe::router_topk_fused(c.dtype, c.E) &&
                     (c.routing == MOE_ROUTE_TOPK || c.routing == MOE_ROUTE_TOPK_SCORE_DROP);
  const int hg = fused ? moe::router_topk_tokens(c.E) : moe::topk_kernel_tokens(c.E);
  const int64_t nch = (c.T + hg - 1) / hg;
  const int64_t rows = rows_of(c);
  const int BM = row_tile(c);
  // Stage timing: while stage i runs, its first kernel carries
  // events[2i] and every kernel events[2i+1] (bound to the kernels; see
  // moe::StageEvents).  A stage that launched nothing gets an empty interval.
  moe::StageEvents sev{};
  int stage = -1;
  struct ClearStage {
    ~ClearStage() { moe::stage_events() = nullptr; }
  } clear_stage_on_return;
  auto mark = [&](int i) -> hipError_t {   // stage i begins; i == MOE_NUM_STAGES: all done
    if (!events) return hipSuccess;
    moe::stage_events() = nullptr;
    if (stage >= 0 && sev.launched == 0) {
      hipError_t e = hipEventRecord((hipEvent_t)events[2 * stage], s);
      if (e == hipSuccess) e = hipEventRecord((hipEvent_t)events[2 * stage + 1], s);
      if (e != hipSuccess) return e;
    }
    if (i >= MOE_NUM_STAGES) return hipSuccess;
    stage = i;
    sev = moe::StageEvents{(hipEvent_t)events[2 * i], (hipEvent_t)events[2 * i + 1], 0};
    moe::stage_events() = &sev;
    return hipSuccess;
  };

  const bool ec = c.routing == MOE_ROUTE_EXPERT_CHOICE;
  // bf16 layers that keep no activations gather GEMM 1's token rows from x
  // through row_token: no dispatch buffer is written (the permute stage
  // launches nothing)
  const bool gather = c.dtype == MOE_DTYPE_BF16 && !saves(c) &&
                      (int64_t)c.T * c.h * 2 < ((int64_t)1 << 31);
  // expert choice: per-(token, expert) slots
  if (ec) {
    gate = r.topk_gate ? r.topk_gate : at<float>(ws, L.gatete);
    assign = r.assign_row ? r.assign_row : at<int32_t>(ws, L.selrow);
  }
  const int slots = ec ? c.E : c.k;

  MOE_TRY(mark(0));
  if (fused)
    MOE_TRY(moe::launch_router_topk(x, w->w_router, w->logit_bias, logits, w->select_bias,
                                    c.gate, c.T, c.h, c.E, c.k, idx, gate, hist, s));
  else
    MOE_TRY(moe::launch_router(c.dtype, x, w->w_router, w->logit_bias, logits, c.T, c.h,
                               c.E, s));
  MOE_TRY(mark(1));
  if (ec) {
    // probabilities -> each expert's C best tokens -> fixed groups -> gather
    float* probs = r.probs ? r.probs : at<float>(ws, L.probs);
    MOE_TRY(moe::launch_router_probs(logits, c.gate, c.T, c.E, probs, s));
    MOE_TRY(mark(2));
    MOE_TRY(moe::launch_expert_choice(probs, c.T, c.E, (int)c.capacity, assign, gate, rowtok, s));
    MOE_TRY(mark(3));
    MOE_TRY(moe::launch_fixed_groups(c.E, (int)c.capacity, c.T, c.has_shared, BM, counts, offsets,
                                     gtab, s));
    MOE_TRY(mark(4));
    if (!gather)
      MOE_TRY(moe::launch_gather_rows(c.dtype, x, rowtok, rows, c.T, c.h, xperm, ld_h(c), s));
  } else {
    const float* sb = w->select_bias;
    if (c.routing == MOE_ROUTE_SINKHORN) {
      float* bias = r.route_bias ? r.route_bias : at<float>(ws, L.skbias);
      MOE_TRY(moe::launch_sinkhorn(logits, c.T, c.E, c.sinkhorn_iters, at<float2>(ws, L.skpart),
                                   bias, s));
      sb = bias;
    }
    if (!fused) MOE_TRY(moe::launch_topk(logits, sb, c.gate, c.T, c.E, c.k, idx, gate, hist, s));
    MOE_TRY(mark(2));
    if (c.routing == MOE_ROUTE_TOPK_SCORE_DROP) {
      // dropless ranks first: each expert's assignments in token order
      int32_t* offs_dl = at<int32_t>(ws, L.offs_dl);
      int32_t* assign_dl = at<int32_t>(ws, L.assign_dl);
      MOE_TRY(moe::launch_scan(hist, nch, c.E, 0, c.T, c.k, c.has_shared, BM, base, counts,
                               offs_dl, at<int32_t>(ws, L.gtab_dl), s));
      MOE_TRY(mark(3));
      MOE_TRY(moe::launch_assign(idx, base, hg, offs_dl, c.T, c.E, c.k, 0, assign_dl,
                                 at<int32_t>(ws, L.rowtok_dl), s));
      MOE_TRY(moe::launch_score_drop(idx, gate, assign_dl, offs_dl, c.T, c.E, c.k,
                                     (int)c.capacity, at<uint64_t>(ws, L.key_dl),
                                     at<int32_t>(ws, L.aid_dl), assign, rowtok, s));
      // the capacity layout's counts, offsets and tile table
      MOE_TRY(moe::launch_scan(hist, nch, c.E, c.capacity, c.T, c.k, c.has_shared, BM, base,
                               counts, offsets, gtab, s, gather ? r.row_token : nullptr));
    } else {
      MOE_TRY(moe::launch_scan(hist, nch, c.E, c.capacity, c.T, c.k, c.has_shared, BM, base,
                               counts, offsets, gtab, s, gather ? r.row_token : nullptr));
      MOE_TRY(mark(3));
      MOE_TRY(moe::launch_assign(idx, base, hg, offsets, c.T, c.E, c.k, c.capacity, assign,
                                 rowtok, s));
    }
    MOE_TRY(mark(4));
    if (!gather)
      MOE_TRY(moe::launch_permute(c.dtype, x, assign, counts, c.T, c.h, c.E, c.k, c.capacity,
                                  xperm, ld_h(c), rowtok, s));
  }
  MOE_TRY(mark(5));
  moe::GroupedGemmArgs a{};
  a.A = gather ? x : xperm;
  if (gather) {
    a.a_map = rowtok;
    a.a_rows = c.T;
  }
  a.A_shared = x;
  a.B0 = w->w1;
  a.B1 = w->w3;
  a.B0s = w->ws1;
  a.B1s = w->ws3;
  a.b_stride = (int64_t)c.F * c.h;
  a.out = act;
  a.K = c.h;
  a.N = c.F;
  a.lda = gather ? c.h : ld_h(c);
  a.lda_shared = c.h;
  a.ldo = ld_f(c);
  a.rotate_k = 1;
  a.gtab = gtab;
  a.G = c.E + c.has_shared;
  a.E_routed = c.E;
  a.a_from_out_rows = 0;
  a.max_m_tiles = max_m_tiles(rows, c.E, BM) + (c.has_shared ? (c.T + BM - 1) / BM : 0);
  set_split(a, c, ws, L);
  if (saves(c)) {                     // [a1 | a3] kept for moe_backward_saved
    a.out13 = at<char>(ws, L.a13);
    a.ld13 = ld_13(c);
  }
  a.claims = moe::claim_block(gtab, a.G, 0);
  MOE_TRY(moe::launch_grouped_gemm(c.dtype, true, a, s));
  MOE_TRY(mark(6));
  a.claims = moe::claim_block(gtab, a.G, 1);
  a.out13 = nullptr;
  a.a_map = nullptr;
  a.A = act;
  a.A_shared = nullptr;
  a.B0 = w->w2;
  a.B1 = nullptr;
  a.B0s = w->ws2;
  a.B1s = nullptr;
  a.out = yperm;
  a.K = c.F;
  a.N = c.h;
  a.lda = ld_f(c);
  a.ldo = ld_h(c);
  a.a_from_out_rows = 1;
  MOE_TRY(moe::launch_grouped_gemm(c.dtype, false, a, s));
  MOE_TRY(mark(7));
  const void* shared_y =
      c.has_shared ? (const void*)(at<char>(yperm, (size_t)rows * ld_h(c) * esize(c))) : nullptr;
  MOE_TRY(moe::launch_combine(c.dtype, yperm, ld_h(c), assign, gate, shared_y, y, c.T, c.h,
                              slots, rows, s));
  MOE_TRY(mark(8));
  return MOE_OK;
}
