/*
 * moe.h - C ABI of libmoe: the forward pass of a top-k Mixture-of-Experts
 * SwiGLU FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages describe it:
 *   - "Megatron-LM 分布式训练（六）：MoE 专家并行 EP 与上下文并行 CP",
 *     section "MoE 层的数据流": router -> dispatch -> experts (one grouped
 *     GEMM) -> combine, plus optional shared experts added to the result;
 *     section "Router": logits = hidden states times the router weight,
 *     then top-k with softmax or sigmoid weights.
 *   - "v6:长序列和 MoE:Context Parallel 与 Expert Parallel" (infra-l7),
 *     section "NVIDIA 原题": the dimension chain [T,h] -> [T,E] -> [T,k] ->
 *     [E,C,h] -> [T,h], capacity C = cf*k*T/E with overflow dropped, or no
 *     capacity at all (dropless); section "MoE:参数很多": every expert is a
 *     SwiGLU FFN h -> F -> h.
 * One ABI entry point per stage of that chain, plus the fused layer.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Memory    All tensor pointers are DEVICE pointers owned by the caller.
 *             The library never allocates or frees device memory; scratch
 *             comes from a caller workspace of moe_workspace_bytes() bytes.
 *             Pointers must be 16-byte aligned (else MOE_ERR_INVALID_ARG,
 *             before any device work).  Tensors are dense,
 *             row-major, with the last dimension contiguous.
 *   Weights   Stored [out, in] (torch Linear layout): w_router [E,h],
 *             w1/w3 [E,F,h], w2 [E,h,F].  The page's router weight [h,E]
 *             is the transpose of w_router.
 *   Streams   `stream` is a hipStream_t passed as void* (NULL = default
 *             stream).  Calls only enqueue work; none synchronises.
 *   Errors    Arguments are checked on the host, synchronously, before any
 *             device work; on a bad argument nothing is enqueued and the
 *             call returns MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED.
 *             MOE_ERR_HIP reports a failed kernel launch.  Device faults
 *             surface at the caller's next synchronisation.  No C++
 *             exception crosses the ABI.
 *   Maps      Index arrays a call reads on the device (topk_idx,
 *             expert_counts, expert_offsets, assign_row) cannot be checked
 *             on the host without a synchronisation.  The kernels ignore a
 *             slot whose expert id is outside [0, E) or whose row is
 *             outside [0, rows), and clamp groups to [0, rows): values
 *             other than the ones the forward writes give unspecified
 *             results, but no access outside the caller's buffers.
 *   Threads   Stateless: concurrent calls are safe on different streams
 *             with different workspaces and outputs.
 *   Graphs    No call allocates, sets memory or synchronises, so a call can
 *             be captured in a HIP graph; each replay recomputes from the
 *             buffers' contents at replay time.
 *   Shapes    h % 128 == 0, F % 128 == 0, h <= 65536, F <= 65536,
 *             1 <= k <= min(E, 16), E <= 1024, T >= 0 (T == 0 enqueues
 *             nothing and reads no pointer), dispatch rows (T*k, or E*C
 *             with a capacity, + T with a shared expert) <= 2^30.  Otherwise
 *             MOE_ERR_UNSUPPORTED.
 *   Numerics  bf16 layers: bf16 inputs, fp32 accumulation, fp32 router
 *             logits and gates, bf16 round-to-nearest-even stores of the
 *             expert activation, expert outputs and the layer output.
 *             fp32 layers compute and store everything in fp32.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1  /* null pointer, bad enum, inconsistent sizes */
#define MOE_ERR_UNSUPPORTED 2  /* shape outside the supported set above */
#define MOE_ERR_WORKSPACE 3    /* workspace missing or too small */
#define MOE_ERR_HIP 4          /* a kernel launch failed */

/* ---- element types --------------------------------------------------- */
#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

/* ---- gate modes -------------------------------------------------------
 * Megatron-LM part 6, section "Router" (top-k over the logits, weights by
 * softmax or sigmoid); infra-l7, section "NVIDIA 原题" (softmax over all E
 * then the selected gate values; DeepSeek-V3's selection-only bias).
 *   SOFTMAX_TOPK        g_j = softmax over the k selected logits
 *   SOFTMAX_ALL_TOPK    g_j = softmax over all E logits, at the selected
 *                       experts, not renormalised
 *   SIGMOID_TOPK_NORM   g_j = sigmoid(l_j) / sum over the k selected
 * Selection always compares the fp32 key l[e] (+ select_bias[e]) and breaks
 * ties toward the lower expert index; select_bias never enters a gate.   */
#define MOE_GATE_SOFTMAX_TOPK 0
#define MOE_GATE_SOFTMAX_ALL_TOPK 1
#define MOE_GATE_SIGMOID_TOPK_NORM 2

/* ---- routing ----------------------------------------------------------
 *   TOPK              token choice: each token's top-k experts (gate modes
 *                     above); with a capacity C the first C assignments of
 *                     an expert in token order are kept, the rest dropped.
 *   TOPK_SCORE_DROP   token choice with a capacity C (> 0 required) where an
 *                     expert keeps the C assignments with the largest gate
 *                     (ties to the earlier token), laid out in token order:
 *                     专家并行 page, "EP+TP+DP" (MoE theory drops the
 *                     lower-priority tokens by gate score).
 *   EXPERT_CHOICE     every expert takes the C = capacity tokens (0 < C <= T)
 *                     with the largest router probability (softmax over E of
 *                     the logits, or for SIGMOID_TOPK_NORM the sigmoids
 *                     normalised over E; ties to the earlier token), in
 *                     token order at rows e*C ..; a token gets the sum over
 *                     the experts that chose it, in expert order, of
 *                     probability x expert output: 10.5 序列并行与专家并行,
 *                     section 10.5.6 (expert-choice routing).  k only enters
 *                     the caller's choice of C (moe_capacity); a
 *                     select_bias is rejected (MOE_ERR_INVALID_ARG).  Only
 *                     moe_forward, moe_grouped_gemm_swiglu,
 *                     moe_unpermute_combine and moe_load_balance accept it.
 *   SINKHORN          token choice on the Sinkhorn-balanced router
 *                     (Megatron-LM part 6, load-balancing table, row
 *                     sinkhorn: the routing matrix is rescaled until doubly
 *                     stochastic).  exp(logits) [T,E] is scaled
 *                     sinkhorn_iters times, rows to sum 1 then columns to sum
 *                     T/E; each token takes the k largest entries of its row
 *                     of the result, which is the top-k of the key
 *                     logit + bias[e] with bias = ln of the product of the
 *                     column factors (fp32, written to route_bias).  Gates
 *                     come from the logits (cfg.gate) as for TOPK, and a
 *                     capacity drops in token order as for TOPK.  A
 *                     select_bias is rejected (MOE_ERR_INVALID_ARG); every
 *                     later stage treats the selection as TOPK's.
 * Selection decisions are integer compares of fp32 keys on the device, so
 * every run routes the same.                                              */
/* Flags of moe_cfg_t.flags.
 *   SAVE_FOR_BACKWARD  moe_forward keeps in its workspace what the backward
 *                      needs (the dispatch buffer, the pre-activations
 *                      [a1 | a3], the activations and the expert outputs),
 *                      so that moe_backward_saved can skip recomputing them.
 *                      moe_workspace_bytes grows by rows x (2F + 128 bytes)
 *                      elements for [a1 | a3]; the layer's output is the
 *                      same bit for bit.  Other bits: MOE_ERR_INVALID_ARG. */
#define MOE_FLAG_SAVE_FOR_BACKWARD 1

#define MOE_ROUTE_TOPK 0
#define MOE_ROUTE_TOPK_SCORE_DROP 1
#define MOE_ROUTE_EXPERT_CHOICE 2
#define MOE_ROUTE_SINKHORN 3
#define MOE_MAX_SINKHORN_ITERS 1000

/* Stages of moe_forward, in launch order, each one timed on request:
 *   0 router GEMM, 1 top-k + gates + chunk histogram (after the Sinkhorn
 *   iterations with SINKHORN routing), 2 scan (counts,
 *   offsets, GEMM tile table), 3 assign (ranks, rows), 4 permute copy,
 *   5 grouped GEMM 1 + SwiGLU (+ its split-K reduce), 6 grouped GEMM 2
 *   (+ reduce), 7 combine.  (Routing variants launch their own kernels in
 *   stages 1-4.)  bf16 layers of up to 64 experts with TOPK or
 *   TOPK_SCORE_DROP routing run the router, the top-k, the gates and the
 *   histogram as one kernel in stage 0; their stage 1 launches no kernel.
 *   MOE_NUM_EVENTS events, a start and a stop per stage, time them (see
 *   moe_forward).                                                          */
#define MOE_NUM_STAGES 8
#define MOE_NUM_EVENTS (2 * MOE_NUM_STAGES)

typedef struct moe_cfg {
  int32_t struct_size; /* sizeof(moe_cfg_t) */
  int32_t dtype;       /* MOE_DTYPE_*: x, weights, activation and y */
  int64_t T;           /* tokens (batch x sequence flattened) */
  int32_t h;           /* model width */
  int32_t F;           /* expert FFN width */
  int32_t E;           /* routed experts */
  int32_t k;           /* experts per token */
  int32_t gate;        /* MOE_GATE_* */
  int32_t has_shared;  /* 1: one shared expert of shape (h, F) on every token */
  int64_t capacity;    /* 0: dropless; > 0: capacity C rows per expert */
  int32_t routing;     /* MOE_ROUTE_* */
  int32_t flags;       /* MOE_FLAG_* bits, 0 for none */
  int32_t sinkhorn_iters; /* SINKHORN: 1..MOE_MAX_SINKHORN_ITERS iterations;
                             0 for every other routing */
} moe_cfg_t;

typedef struct moe_weights {
  const void* w_router;     /* [E,h] dtype */
  const void* w1;           /* [E,F,h] dtype, SiLU branch */
  const void* w3;           /* [E,F,h] dtype, linear branch */
  const void* w2;           /* [E,h,F] dtype, down projection */
  const float* logit_bias;  /* [E] fp32 added to the logits, or NULL */
  const float* select_bias; /* [E] fp32 added for selection only, or NULL */
  const void* ws1;          /* shared expert [F,h], NULL unless has_shared */
  const void* ws3;          /* shared expert [F,h] */
  const void* ws2;          /* shared expert [h,F] */
} moe_weights_t;

/* Optional device outputs of moe_forward (each field may be NULL; a NULL
 * field is kept in the workspace instead).  Layouts as in the stage calls.
 * With MOE_ROUTE_EXPERT_CHOICE the per-token slots are the E experts:
 * topk_idx is not written, topk_gate and assign_row are [T,E] (the
 * probability and row of (t, e) if e chose t, else 0 and -1), and probs
 * holds the router probabilities the experts chose by, laid out [E,T].     */
typedef struct moe_route_out {
  float* logits;           /* [T,E] */
  int32_t* topk_idx;       /* [T,k] */
  float* topk_gate;        /* [T,k] ([T,E] for expert choice) */
  int32_t* expert_counts;  /* [E]   assignments per expert, before any drop */
  int32_t* expert_offsets; /* [E+1] first row of each expert's group */
  int32_t* assign_row;     /* [T*k] row of (t,j) in x_perm, -1 if dropped */
  int32_t* row_token;      /* [rows] token of each row, -1 for padding */
  float* probs;            /* [E,T] expert choice only */
  float* route_bias;       /* [E] Sinkhorn only: the selection bias found */
} moe_route_out_t;

/* Gradients written by moe_backward (device pointers in a host struct). */
typedef struct moe_grads {
  void* dx;            /* [T,h] dtype, required */
  void* dw_router;     /* [E,h] dtype, or NULL (not computed) */
  float* dlogit_bias;  /* [E] fp32, or NULL */
  void* dw1;           /* [E,F,h] dtype, required */
  void* dw3;           /* [E,F,h] dtype, required */
  void* dw2;           /* [E,h,F] dtype, required */
  void* dws1;          /* shared expert [F,h], required iff has_shared */
  void* dws3;          /* [F,h] */
  void* dws2;          /* [h,F] */
  float* dgate;        /* [T,k] ([T,E] expert choice) fp32 dL/dgate, or NULL */
} moe_grads_t;

/* Host-only helpers (no device work, callable without a GPU). ---------- */

/* Static string for a status code. */
const char* moe_strerror(int status);

/* Capacity C = ceil(cf_num * k * T / (cf_den * E)) in exact integer
 * arithmetic (infra-l7, "NVIDIA 原题", capacity bullet: 1280 at T=4096,
 * E=8, k=2, cf=5/4).  All arguments > 0, else MOE_ERR_INVALID_ARG.       */
int moe_capacity(int64_t T, int32_t E, int32_t k, int64_t cf_num,
                 int64_t cf_den, int64_t* C);

/* Rows of the dispatch buffer x_perm: T*k when dropless, E*C otherwise. */
int moe_num_rows(const moe_cfg_t* cfg, int64_t* rows);

/* Workspace bytes moe_forward needs for cfg (the stage calls need at most
 * this much too). */
int moe_workspace_bytes(const moe_cfg_t* cfg, size_t* bytes);

/* Stage 1: router GEMM, gating and top-k ----------------------------------
 * Megatron-LM part 6, "Router"; infra-l7, "NVIDIA 原题" rows router/top-k.
 *   x            [T,h] dtype
 *   w_router     [E,h] dtype
 *   logit_bias   [E] fp32 or NULL   (added to the logits)
 *   select_bias  [E] fp32 or NULL   (added to the selection key only)
 *   logits       [T,E] fp32 out, or NULL (then kept in the workspace)
 *   topk_idx     [T,k] int32 out: slot 0 = largest key
 *   topk_gate    [T,k] fp32 out: gate of each slot (cfg->gate)
 *   ws, ws_bytes workspace (moe_workspace_bytes); required with SINKHORN
 *                routing, whose selection bias is kept there
 * Expert choice: MOE_ERR_UNSUPPORTED (moe_forward routes it).             */
int moe_router_topk(const moe_cfg_t* cfg, const void* x, const void* w_router,
                    const float* logit_bias, const float* select_bias,
                    float* logits, int32_t* topk_idx, float* topk_gate,
                    void* ws, size_t ws_bytes, void* stream);

/* Stage 2: dispatch / permute ---------------------------------------------
 * infra-l7, "NVIDIA 原题" row dispatch and capacity bullet, "自测" (sort by
 * expert, drop past capacity on that expert only, pad unused places).
 *   x              [T,h] dtype
 *   topk_idx       [T,k] int32 (from stage 1, any valid selection)
 *   expert_counts  [E] int32 out: assignments per expert before dropping
 *   expert_offsets [E+1] int32 out: dropless = exclusive prefix of counts;
 *                  capacity = e*C
 *   assign_row     [T*k] int32 out: row of (t,j); rank = number of earlier
 *                  tokens that chose the same expert; dropless row =
 *                  offsets[e] + rank; capacity row = e*C + rank if rank < C,
 *                  else -1 (dropped)
 *   row_token      [rows] int32 out: token of each row, -1 for padding
 *   x_perm         [rows,h] dtype out: x_perm[assign_row[t,j]] = x[t];
 *                  padding rows are zero                                  */
int moe_permute(const moe_cfg_t* cfg, const void* x, const int32_t* topk_idx,
                int32_t* expert_counts, int32_t* expert_offsets,
                int32_t* assign_row, int32_t* row_token, void* x_perm,
                void* ws, size_t ws_bytes, void* stream);

/* Stage 2 with a routing already made: dispatch another [T,h] tensor by the
 * maps moe_permute or moe_forward wrote (infra-l7, "NVIDIA 原题" row
 * dispatch; "自测": rows sorted by expert, unused places padded).
 *   x              [T,h] dtype
 *   assign_row     [T*k] int32: row of (t,j), -1 if dropped
 *   expert_counts  [E] int32: assignments per expert before dropping
 *   row_token      [rows] int32 out: -1 written for the padding rows of the
 *                  capacity layout (kept rows are left as they are)
 *   x_perm         [rows,h] dtype out: x_perm[assign_row[t,j]] = x[t];
 *                  capacity layout: rows e*C + min(counts[e], C) ..
 *                  e*C + C - 1 are zero
 * Token-choice routings only (TOPK, TOPK_SCORE_DROP, SINKHORN); expert
 * choice gives MOE_ERR_UNSUPPORTED.  Needs no workspace.                  */
int moe_permute_rows(const moe_cfg_t* cfg, const void* x, const int32_t* assign_row,
                     const int32_t* expert_counts, int32_t* row_token, void* x_perm,
                     void* stream);

/* Stage 3: grouped GEMM running every expert's SwiGLU FFN ------------------
 * infra-l7, "MoE:参数很多" (SwiGLU FFN h->F->h) and "自测" (one grouped GEMM
 * over tokens sorted by expert); Megatron-LM part 6 (experts as GroupedGEMM).
 * Group e owns rows expert_offsets[e] .. and min(expert_counts[e],
 * expert_offsets[e+1]-expert_offsets[e]) of them are computed; other rows
 * of act/y_perm are left unspecified.
 *   act[r,f]    = bf16( silu(x_perm[r]·w1[e,f]) * (x_perm[r]·w3[e,f]) )
 *   y_perm[r,i] = bf16( act[r]·w2[e,i] )       silu(z) = z/(1+exp(-z))
 *   x_perm [rows,h], act [rows,F], y_perm [rows,h] dtype; rows =
 *   expert_offsets[E].  A shared expert is this call with E=1,
 *   counts=[T], offsets=[0,T].                                            */
int moe_grouped_gemm_swiglu(const moe_cfg_t* cfg, const void* x_perm,
                            const int32_t* expert_counts,
                            const int32_t* expert_offsets, const void* w1,
                            const void* w3, const void* w2, void* act,
                            void* y_perm, void* ws, size_t ws_bytes,
                            void* stream);

/* The same grouped GEMM without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, results and errors are those
 * of moe_grouped_gemm_swiglu (bit-identical outputs), without ws/ws_bytes:
 * its scratch (the tile table with its tile-claim counters and the split-K
 * partial tiles) is a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES
 * in the library, one per GPU, held from the library's load until the
 * process ends.  Limit:
 * every config the library accepts fits it (E <= 1024 groups, at most 256
 * split-K parts); a config needing more returns MOE_ERR_UNSUPPORTED before
 * any device work.  The call allocates and frees nothing and sets no
 * memory: every scratch byte a kernel reads was written earlier in the same
 * call.  All calls on one GPU share that GPU's scratch, so calls that
 * overlap on one GPU (different streams, or threads) race and give
 * unspecified results; calls in one stream are ordered and safe.
 * MOE_ERR_HIP if the scratch's device address cannot be obtained.          */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)25856 + (size_t)67108864)
int moe_grouped_gemm_swiglu_noalloc(const moe_cfg_t* cfg, const void* x_perm,
                                    const int32_t* expert_counts,
                                    const int32_t* expert_offsets, const void* w1,
                                    const void* w3, const void* w2, void* act,
                                    void* y_perm, void* stream);

/* Stage 4: combine / unpermute -----------------------------------------------
 * 专家并行, "EP+DP" forward (each token's top-k outputs summed with their
 * weights); infra-l7 "NVIDIA 原题" row combine.
 *   y[t] = sum over kept slots j in slot order of topk_gate[t,j] *
 *          y_perm[assign_row[t,j]]  (+ shared_y[t]), summed in fp32
 *   shared_y [T,h] dtype or NULL;  y [T,h] dtype out.                     */
int moe_unpermute_combine(const moe_cfg_t* cfg, const void* y_perm,
                          const int32_t* assign_row, const float* topk_gate,
                          const void* shared_y, void* y, void* stream);

/* Load-balance statistics of a routing --------------------------------------
 * infra-l7 "NVIDIA 原题" notes on the load balancing loss (Switch
 * Transformer's alpha*E*sum_i f_i*P_i, f_i the share of tokens sent to
 * expert i, P_i the router's mean probability for i); Megatron-LM part 6,
 * "负载均衡" (aux loss and the load_balancing_loss metric).
 *   logits [T,E] fp32 in (as written by moe_router_topk / moe_forward);
 *   expert_counts [E] int32 in (routed assignments per expert, before any
 *       capacity drop, as written by moe_permute / moe_forward);
 *   f [E] out: expert_counts[i] / (T*k);
 *   P [E] out: mean over the T tokens of the router's distribution over all
 *       E experts: softmax of the logits for the two softmax gate modes, the
 *       per-expert sigmoids normalised over E for SIGMOID_TOPK_NORM (the
 *       selection bias takes no part);
 *   aux_loss [1] out: alpha * E * sum_i f[i] * P[i] (alpha finite).
 * Sums are fp32 in a fixed order: identical results on every run.  Needs
 * the workspace of moe_workspace_bytes(cfg).                               */
int moe_load_balance(const moe_cfg_t* cfg, const float* logits,
                     const int32_t* expert_counts, float alpha, float* f, float* P,
                     float* aux_loss, void* ws, size_t ws_bytes, void* stream);

/* Aux-loss-free balancing step ----------------------------------------------
 * infra-l7, "NVIDIA 原题" notes on the load balancing loss: DeepSeek-V3
 * replaces the auxiliary loss with a per-expert bias that enters only the
 * top-k selection (select_bias of moe_router_topk / moe_forward) and is kept
 * out of the loss.  The pages do not say how the bias moves; this call takes
 * one fixed step per routing: for expert e, with c = expert_counts[e] (the
 * routed assignments before any drop, as moe_permute / moe_forward write
 * them), T*k > E*c (fewer than the mean) raises select_bias[e] by gamma,
 * T*k < E*c lowers it by gamma, T*k == E*c leaves it unchanged; one fp32
 * addition each, compared in exact integers.
 *   expert_counts [E] int32 in;  select_bias [E] fp32 in/out (in place);
 *   gamma: step, finite (else MOE_ERR_INVALID_ARG).
 * Top-k routing (with or without score drop) only; other routings:
 * MOE_ERR_UNSUPPORTED.  T == 0: nothing is enqueued.                       */
int moe_select_bias_update(const moe_cfg_t* cfg, const int32_t* expert_counts,
                           float gamma, float* select_bias, void* stream);

/* Backward of the layer -------------------------------------------------
 * 专家并行 page, "EP+DP" BWD (each GPU computes its experts' weight
 * gradients; the gradients go back along the routing path) and Megatron-LM
 * part 6, "MoE 层的数据流" (the same chain, reversed).  Gradients of
 * L = sum(y * dy) with the routing of a moe_forward call held fixed (the
 * top-k choice and capacity drops are not differentiated; a dropped slot
 * passes nothing back; select_bias gets no gradient):
 *   per kept slot (t, j) of expert e:  dO = g[t,j] dy[t],  dg[t,j] = dy[t].o,
 *   SwiGLU and expert weights by the chain rule, the gate mode's Jacobian
 *   from dg to the logits dl, dw_router = dl^T x, dlogit_bias = sum_t dl,
 *   dx = (sum over the kept slots of the expert's input gradient) + the
 *   shared expert's + dl w_router.
 * The expert activations are recomputed from x (one grouped GEMM for
 * [a1 | a3], one for the expert outputs), so nothing of the forward's
 * workspace is needed.
 *   route    the routing outputs of the forward: logits, topk_idx, topk_gate,
 *            expert_counts, expert_offsets, assign_row (all required)
 *   dy [T,h] dtype in;  grads  see moe_grads_t.
 * bf16 and fp32 layers, every routing.  With MOE_ROUTE_EXPERT_CHOICE the
 * experts' choices are held fixed, topk_idx is not read, topk_gate and
 * assign_row are the forward's [T,E] slots and dgate is [T,E]; the gate of
 * a chosen (t, e) is the router probability itself, so the logits get that
 * distribution's Jacobian over all E (10.5 section 10.5.6).  Gradient sums
 * in fp32; dx, weight gradients and the intermediates (a1, a3, u, dO, dA,
 * dx_perm; fp32 layers also dU) stored in the layer's dtype.  bf16 layers
 * form dA from dU in fp32 registers, and take dl^T x and dl w_router as
 * bf16 products of dl's parts hi = bf16(dl), lo = bf16(dl - hi), which
 * carry dl to about 2^-17 of its size.  Every sum has a fixed order:
 * the same bits on every run.  Size limit: the dispatch rows plus 64 per
 * group (E, + 1 with a shared expert), rounded up to 64, stay below 2^25;
 * beyond it both calls return MOE_ERR_UNSUPPORTED.                        */
int moe_backward_workspace_bytes(const moe_cfg_t* cfg, size_t* bytes);
int moe_backward(const moe_cfg_t* cfg, const moe_weights_t* w, const void* x,
                 const void* dy, const moe_route_out_t* route, const moe_grads_t* grads,
                 void* ws, size_t ws_bytes, void* stream);

/* The same backward from the activations a moe_forward call kept (cfg with
 * MOE_FLAG_SAVE_FOR_BACKWARD, the same cfg, weights and x): the dispatch
 * buffer, [a1 | a3], the activations and the expert outputs are read from
 * that call's workspace fwd_ws (fwd_ws_bytes >= moe_workspace_bytes(cfg),
 * untouched since) instead of being recomputed, which skips the permute,
 * two of the six grouped GEMMs and the SwiGLU pass.  The results equal
 * moe_backward's up to the rounding of the kept bf16 values (the forward
 * sums its K slices in another order).  cfg without the flag, or fwd_ws
 * NULL or too small: MOE_ERR_INVALID_ARG / MOE_ERR_WORKSPACE.             */
int moe_backward_saved(const moe_cfg_t* cfg, const moe_weights_t* w, const void* x,
                       const void* dy, const moe_route_out_t* route, const void* fwd_ws,
                       size_t fwd_ws_bytes, const moe_grads_t* grads, void* ws,
                       size_t ws_bytes, void* stream);

/* The fused layer: stages 1-4 (+ the shared expert as one more group of
 * the grouped GEMM) on one stream, no host synchronisation.
 *   w        weights (device pointers inside a host struct)
 *   x [T,h]  in;  y [T,h] out
 *   route    optional extra outputs (host struct of device pointers) or NULL
 *   events   NULL, or MOE_NUM_EVENTS hipEvent_t (as void*) created by the
 *            caller with timing enabled, for per-stage kernel timing:
 *            events[2i] is bound to the start of stage i's first kernel and
 *            events[2i+1] to the end of its last kernel (hipExtLaunchKernel
 *            start/stop events, taken from the kernels' own timestamps), so
 *            hipEventElapsedTime(events[2i], events[2i+1]) is the stage's
 *            kernel time and (events[0], events[2*MOE_NUM_STAGES-1]) spans
 *            the layer from its first kernel's start to its last kernel's
 *            end.  A stage that launches nothing records both events on
 *            `stream` at that point (an interval of two back-to-back
 *            markers, a few microseconds, not kernel time).                 */
int moe_forward(const moe_cfg_t* cfg, const moe_weights_t* w, const void* x,
                void* y, const moe_route_out_t* route, void* ws,
                size_t ws_bytes, void* const* events, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
