"""CPU oracle of the top-k Mixture-of-Experts SwiGLU FFN layer forward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never does; this code
shares nothing with it but the seeded inputs of ``moe_inputs``.

What it computes is the plain definition of the layer, token by token, with
no permutation buffer, no blocking and no fusion:

1. router logits, one dot product per (token, expert), accumulated in fp64
   and rounded once to fp32, plus an optional per-expert fp32 offset;
2. selection keys (logit plus an optional selection-only bias, in fp32) and
   top-k by (key descending, expert index ascending);
3. gate values in fp64 from the fp32 logits, rounded to fp32;
4. per-expert token counts and ranks in token order; with a capacity C an
   assignment whose rank is C or more is dropped;
5. for every kept (token, slot): the expert's SwiGLU FFN in fp64;
6. the gate-weighted sum of the kept expert outputs, in slot order, plus the
   shared expert's output when there is one;
7. (separately) the load-balance statistics of a routing: the share of
   assignments per expert, the router's mean probability per expert and the
   Switch auxiliary loss built from them; and one step of the aux-loss-free
   update of the per-expert selection bias;
8. three routing variants: capacity drops by gate score instead of token
   order, expert choice (every expert takes its C best-scoring tokens), and
   Sinkhorn balancing of the routing matrix before the top-k;
9. the backward of the layer: gradients of sum(y * dy) with respect to the
   input, the router and every expert weight, with the routing held fixed
   (token choice, and expert choice with the experts' choices held fixed).

Sources (pages and the part of each that is followed):

* "Megatron-LM 分布式训练（六）：MoE 专家并行 EP 与上下文并行 CP"
  (swordlidev.github.io): section "MoE 层的数据流" (router → dispatch →
  experts → combine, optional shared experts added) and section
  "Router：token 怎么选专家" (logits = hidden · W_router, then top-k with
  softmax or sigmoid weights), and its load-balancing table (the sinkhorn
  row: Sinkhorn iterations make the routing matrix doubly stochastic).
* "v6:长序列和 MoE:Context Parallel 与 Expert Parallel"
  (charliedreemur.github.io, infra-l7): section "MoE:参数很多,每个 token
  只算一点" (an expert is the SwiGLU FFN h → F → h with three matrices) and
  section "NVIDIA 原题" (dimension table [T,h] → [T,E] → [T,k] → [E,C,h] →
  [T,h]; capacity C = cf·k·T/E with overflow dropped; DeepSeek-V3's
  selection-only bias), and its "自测" answers (an overflowing token is
  dropped on that expert only; padding fills unused capacity slots; sorting
  tokens by expert before one grouped GEMM).
* "专家并行" (formulaic.cloudchewie.com, 7-expert-parallel): section "EP+DP",
  forward of the MoE layer (each token's expert outputs are gathered back and
  summed with the top-k weights).
* "10.5 序列并行与专家并行" (paper.xwysyy.cn): 10.5.5 (combine weights the
  expert outputs by the routing weights) and 10.5.6 (capacity factor, excess
  tokens dropped or passed on by the residual).

Readings where the pages are silent or disagree (all listed in the design doc):

* gate modes: "softmax_topk" = softmax over the k selected logits;
  "softmax_all_topk" = softmax over all E logits, the selected k values
  taken without renormalising (the worked example's order);
  "sigmoid_topk_norm" = per-expert sigmoid, normalised over the selected k;
* top-k always compares the fp32 selection key, ties to the lower index;
* C = ceil(cf·k·T/E) in exact integer arithmetic (cf given as num/den);
* overflow keeps the first C assignments in token order; a dropped slot adds
  nothing and the other gates are not renormalised;
* the expert FFN is W2 · (silu(W1 x) ⊙ (W3 x)) with silu(z) = z/(1+e^-z);
* the layer output excludes the residual; the shared expert has weight 1;
* Sinkhorn: exp(l) scaled alternately, rows to sum 1 then columns to sum
  T/E, a given number of times; top-k over the rows of the result; gates
  from the logits;
* load balance: f_i counts routed assignments over T*k (before capacity
  drops); P_i averages the router's distribution over all E (softmax of the
  logits, or the sigmoids normalised over E); the loss coefficient alpha is
  an input.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against hand-worked fixtures, closed forms and brute force; none is
"parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

GATE_MODES = ("softmax_topk", "softmax_all_topk", "sigmoid_topk_norm")


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# 1. Router logits.  Megatron-LM part 6, "Router：token 怎么选专家": the gating
# step multiplies the hidden states by the router weight; infra-l7,
# "NVIDIA 原题" table, row "router": x [T,h] times Wr [h,E] gives [T,E].
# The router weight is stored [E,h] here (its transpose).
# ---------------------------------------------------------------------------
def router_logits(x, w_router, logit_bias=None) -> np.ndarray:
    """fp32 [T,E]: l[t,e] = fp32(sum_i x[t,i] * w_router[e,i]) (+ bias[e] in fp32)."""
    l = (_f64(x) @ _f64(w_router).T).astype(np.float32)
    if logit_bias is not None:
        l = (l + np.asarray(logit_bias, dtype=np.float32)[None, :]).astype(np.float32)
    return l


def selection_keys(logits, select_bias=None) -> np.ndarray:
    """fp32 [T,E] key the top-k compares.

    infra-l7, "NVIDIA 原题", load-balancing bullet: the aux-loss-free scheme
    adds a per-expert bias that only takes part in choosing the top-k.
    """
    k = np.asarray(logits, dtype=np.float32)
    if select_bias is not None:
        k = (k + np.asarray(select_bias, dtype=np.float32)[None, :]).astype(np.float32)
    return k


# ---------------------------------------------------------------------------
# 2. Top-k.  Megatron-LM part 6, "Router": top-k over the logits picks each
# token's k experts; infra-l7 table row "top-k": [T,k].  Order: key
# descending, lower expert index first on equal keys.
# ---------------------------------------------------------------------------
def topk(keys, k: int) -> np.ndarray:
    """int32 [T,k]; slot 0 holds the largest key."""
    keys = np.asarray(keys, dtype=np.float32)
    E = keys.shape[1]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # A stable sort of the negated keys keeps equal keys in index order.
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def near_tie(keys, k: int, threshold: float = 1e-5) -> np.ndarray:
    """bool [T]: gap between the k-th and (k+1)-th largest key below threshold.

    Either choice is correct for such a token when two implementations round
    the logits differently; with k = E there is no (k+1)-th key.
    """
    keys = np.asarray(keys, dtype=np.float32)
    T, E = keys.shape
    if k >= E:
        return np.zeros(T, dtype=bool)
    s = -np.sort(-keys.astype(np.float64), axis=1)
    return (s[:, k - 1] - s[:, k]) < threshold


# ---------------------------------------------------------------------------
# 3. Gates.  Megatron-LM part 6, "Router": weights by softmax or sigmoid;
# infra-l7 table rows "router"/"top-k": softmax over E, then the top-k gate
# values.  Computed in fp64 from the fp32 logits, rounded to fp32.
# ---------------------------------------------------------------------------
def gates(logits, idx, mode: str) -> np.ndarray:
    """fp32 [T,k] gate of each selected slot."""
    l = _f64(logits)
    idx = np.asarray(idx)
    sel = np.take_along_axis(l, idx, axis=1)            # [T,k] selected logits
    if mode == "softmax_topk":
        m = sel.max(axis=1, keepdims=True)
        ex = np.exp(sel - m)
        g = ex / ex.sum(axis=1, keepdims=True)
    elif mode == "softmax_all_topk":
        m = l.max(axis=1, keepdims=True)
        ex = np.exp(l - m)
        p = ex / ex.sum(axis=1, keepdims=True)
        g = np.take_along_axis(p, idx, axis=1)
    elif mode == "sigmoid_topk_norm":
        s = 1.0 / (1.0 + np.exp(-sel))
        g = s / s.sum(axis=1, keepdims=True)
    else:
        raise ValueError(f"unknown gate mode {mode!r}")
    return g.astype(np.float32)


# ---------------------------------------------------------------------------
# 4. Capacity and routing maps.  infra-l7, "NVIDIA 原题": dispatch groups
# tokens by expert, at most C per group, unfilled places padded, giving
# [E,C,h]; C = cf·k·T/E (1280 at T=4096, E=8, k=2, cf=1.25) and tokens past
# it are dropped; Megatron's default has no capacity (dropless).  "自测": a
# token past capacity is dropped on that expert only; sorting the tokens by
# expert lets one grouped GEMM run all experts.
# ---------------------------------------------------------------------------
def capacity(T: int, E: int, k: int, cf_num: int, cf_den: int) -> int:
    """C = ceil(cf_num * k * T / (cf_den * E)), exact integers."""
    if min(T, E, k, cf_num, cf_den) <= 0:
        raise ValueError("capacity needs positive T, E, k and cf")
    num = cf_num * k * T
    den = cf_den * E
    return -(-num // den)


def route_maps(idx, E: int, C: Optional[int] = None) -> dict:
    """Per-expert counts, group offsets and the (token, slot) -> row map.

    rank(t, j): number of tokens t' < t that also chose expert idx[t, j]
    (a token picks an expert at most once).  Dropless: rows of expert e are
    offsets[e] .. offsets[e+1]-1, row = offsets[e] + rank.  With capacity C:
    expert e owns rows e*C .. e*C+C-1, kept iff rank < C, row = e*C + rank,
    else -1 (dropped).  row_token[row] = token, -1 for padding rows.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counter = [0] * E
    rank = np.empty((T, k), dtype=np.int64)
    for t in range(T):              # token order decides the ranks
        for j in range(k):
            e = int(idx[t, j])
            rank[t, j] = counter[e]
            counter[e] += 1
    counts = np.array(counter, dtype=np.int64)
    if C is None:
        offsets = np.zeros(E + 1, dtype=np.int64)
        offsets[1:] = np.cumsum(counts)
        rows = int(offsets[-1])
        assign_row = offsets[idx] + rank
    else:
        offsets = np.arange(E + 1, dtype=np.int64) * C
        rows = E * C
        assign_row = np.where(rank < C, idx.astype(np.int64) * C + rank, -1)
    row_token = np.full(rows, -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            r = int(assign_row[t, j])
            if r >= 0:
                row_token[r] = t
    kept = counts if C is None else np.minimum(counts, C)
    return {
        "counts": counts,
        "offsets": offsets,
        "kept": kept,
        "rank": rank,
        "assign_row": assign_row,
        "row_token": row_token,
        "rows": rows,
    }


# ---------------------------------------------------------------------------
# 5. Expert FFN.  infra-l7, "MoE:参数很多" section: each expert is the dense
# SwiGLU FFN h → F → h with three h×F matrices; "NVIDIA 原题" table row
# "expert".  Reading: W1 carries the SiLU, W3 the linear branch.
# ---------------------------------------------------------------------------
def silu(z):
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(xrows, w1, w3, w2) -> np.ndarray:
    """fp64 [n,h] = W2 · (silu(W1 x) ⊙ (W3 x)) for each row x of xrows."""
    xr = _f64(xrows)
    a1 = xr @ _f64(w1).T          # [n,F]
    a3 = xr @ _f64(w3).T          # [n,F]
    u = silu(a1) * a3
    return u @ _f64(w2).T         # [n,h]


# ---------------------------------------------------------------------------
# 6. Whole layer.  Megatron-LM part 6, "MoE 层的数据流": router, dispatch,
# experts, combine, plus shared experts every token passes through;
# 专家并行, "EP+DP" forward: the top-k outputs of a token are summed with
# their gate weights; infra-l7 table row "combine" and "自测" (a dropped slot
# contributes nothing; the rest of the token goes on by the residual, which
# this layer's output excludes).
# ---------------------------------------------------------------------------
def moe_forward(x, w_router, w1, w3, w2, *, k: int, gate: str,
                C: Optional[int] = None, logit_bias=None, select_bias=None,
                shared=None, tokens=None, idx=None, maps_only=False,
                drop: str = "token", priority=None,
                sinkhorn_iters: Optional[int] = None) -> dict:
    """Reference forward.

    x [T,h]; w_router [E,h]; w1, w3 [E,F,h]; w2 [E,h,F] (any array-likes of
    the exact values the device gets).  ``shared`` = (ws1, ws3, ws2) or None.
    ``tokens``: optional 1-D array of token ids whose outputs are computed
    (routing, ranks and drops still cover all T tokens).  ``idx``: optional
    externally chosen top-k (used to recompute maps from another selection);
    when given, gates still come from this oracle's logits.  ``drop``: with
    a capacity, "token" keeps the first C assignments of an expert in token
    order, "score" the C with the largest gate (route_maps_score_drop),
    deciding on ``priority`` [T,k] fp32 when given (e.g. the device's own
    gates) and on this oracle's gates otherwise.  ``sinkhorn_iters``: the
    selection takes the Sinkhorn-balanced top-k (``sinkhorn``; then no
    select_bias), returned as ``sinkhorn_bias``.
    Returns logits, keys, idx, gates, near_tie, maps, and ``y`` (fp64) for the
    requested tokens, in the order of ``tokens``.
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(w_router).shape[0]
    logits = router_logits(x, w_router, logit_bias)
    sk_bias = None
    if sinkhorn_iters is not None:
        if select_bias is not None:
            raise ValueError("Sinkhorn routing takes no select_bias")
        select_bias = sk_bias = sinkhorn(logits, sinkhorn_iters)["bias"]
    keys = selection_keys(logits, select_bias)
    if idx is None:
        idx = topk(keys, k)
    idx = np.asarray(idx).astype(np.int32)
    g = gates(logits, idx, gate)
    if drop == "score":
        if C is None:
            raise ValueError("the score drop needs a capacity")
        maps = route_maps_score_drop(idx, g if priority is None else priority, E, C)
    elif drop == "token":
        maps = route_maps(idx, E, C)
    else:
        raise ValueError(f"unknown drop rule {drop!r}")
    out = {"logits": logits, "keys": keys, "idx": idx, "gates": g,
           "near_tie": near_tie(keys, k), "maps": maps, "sinkhorn_bias": sk_bias}
    if maps_only:
        return out

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    h = x.shape[1]
    y = np.zeros((len(tok), h), dtype=np.float64)
    xs = _f64(x[tok])
    # Expert outputs of every kept (token, slot); experts are independent,
    # so each expert's rows are one matrix product.
    o = np.zeros((len(tok), k, h), dtype=np.float64)
    sel = idx[tok]                                  # [n,k]
    kept = maps["assign_row"][tok] >= 0             # [n,k]
    for e in range(E):
        mask = (sel == e) & kept
        if not mask.any():
            continue
        rows_n, slots = np.nonzero(mask)
        o[rows_n, slots] = swiglu_ffn(xs[rows_n], w1[e], w3[e], w2[e])
    gsel = _f64(g[tok])
    for j in range(k):                              # slot order
        y += np.where(kept[:, j:j + 1], gsel[:, j:j + 1] * o[:, j], 0.0)
    if shared is not None:
        ws1, ws3, ws2 = shared
        y += swiglu_ffn(xs, ws1, ws3, ws2)
    out["y"] = y
    out["tokens"] = tok
    return out


# ---------------------------------------------------------------------------
# 7. Load-balance statistics.  infra-l7, "NVIDIA 原题" notes on the load
# balancing loss: Switch Transformer adds alpha*E*sum_i f_i*P_i, with f_i the
# share of tokens sent to expert i and P_i the router's mean probability for
# i, smallest when the load is even.  Megatron-LM part 6, "负载均衡":
# aux_loss penalises the gap between where tokens go and how likely the
# router makes each expert (logged as load_balancing_loss).
# ---------------------------------------------------------------------------
def router_probs(logits, gate: str) -> np.ndarray:
    """fp64 [T,E]: the router's distribution over all E experts per token:
    softmax of the logits for the softmax gates, the per-expert sigmoids
    normalised over all E for the sigmoid gate.  The selection-only bias is
    not part of it."""
    l = _f64(logits)
    if gate in ("softmax_topk", "softmax_all_topk"):
        ex = np.exp(l - l.max(axis=1, keepdims=True))
        return ex / ex.sum(axis=1, keepdims=True)
    if gate == "sigmoid_topk_norm":
        s = 1.0 / (1.0 + np.exp(-l))
        return s / s.sum(axis=1, keepdims=True)
    raise ValueError(f"unknown gate mode {gate!r}")


def load_balance(logits, counts, k: int, gate: str, alpha: float) -> dict:
    """f [E] = counts / (T*k) (routed assignments, before any capacity drop),
    P [E] = mean over tokens of router_probs, loss = alpha*E*sum_i f_i*P_i.
    Sums in fp64; f, P and loss returned rounded to fp32."""
    l = _f64(logits)
    T, E = l.shape
    f = np.asarray(counts, dtype=np.float64) / float(T * k)
    P = router_probs(l, gate).mean(axis=0)
    loss = float(alpha) * E * float(np.dot(f, P))
    return {"f": f.astype(np.float32), "P": P.astype(np.float32),
            "loss": np.float32(loss)}


def select_bias_update(select_bias, counts, T: int, k: int, gamma: float) -> np.ndarray:
    """One step of aux-loss-free balancing.  infra-l7, "NVIDIA 原题" notes on
    the load balancing loss: DeepSeek-V3 drops the auxiliary loss and gives
    every expert a bias that only enters the top-k selection, kept outside
    the loss.  The pages name the bias but not how it moves; the reading
    taken: after a routing, an expert that received more than the mean
    T*k/E assignments has its bias lowered by gamma, one that received fewer
    has it raised by gamma, one exactly at the mean keeps it.  The
    comparison is T*k against E*count in exact integers; the step is one fp32
    addition, and an expert at the mean keeps its bias bit for bit."""
    b = np.asarray(select_bias, dtype=np.float32).copy()
    c = np.asarray(counts, dtype=np.int64)
    E = b.shape[0]
    under = T * k - E * c          # > 0: fewer than the mean, < 0: more
    step = np.float32(gamma)
    b[under > 0] = b[under > 0] + step
    b[under < 0] = b[under < 0] - step
    return b


# ---------------------------------------------------------------------------
# 8. Routing variants.  专家并行 page, "EP+TP+DP": MoE theory drops the
# lower-priority tokens by their gate score (as opposed to cutting along C
# for parallelism).  10.5 §10.5.6: expert-choice routing turns the direction
# round: every expert takes the fixed number of tokens that score highest
# for it, so the load is balanced by construction.
# ---------------------------------------------------------------------------
def route_maps_score_drop(idx, gates_fp32, E: int, C: int) -> dict:
    """Capacity C with score priority.  Of the assignments to expert e (a
    token picks e at most once), the C with the largest fp32 gate are kept,
    ties going to the earlier token; the kept ones take rows e*C, e*C+1, ...
    in token order and the rest are dropped (row -1)."""
    idx = np.asarray(idx)
    g = np.asarray(gates_fp32, dtype=np.float32)
    T, k = idx.shape
    assign_row = np.full((T, k), -1, dtype=np.int64)
    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        cand = [(t, j) for t in range(T) for j in range(k) if int(idx[t, j]) == e]
        counts[e] = len(cand)
        # position i in `cand` is token order; priority = (gate desc, i asc)
        order = sorted(range(len(cand)), key=lambda i: (-float(g[cand[i]]), i))
        for r, i in enumerate(sorted(order[:C])):
            t, j = cand[i]
            assign_row[t, j] = e * C + r
    row_token = np.full(E * C, -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if assign_row[t, j] >= 0:
                row_token[assign_row[t, j]] = t
    return {"counts": counts, "offsets": np.arange(E + 1, dtype=np.int64) * C,
            "kept": np.minimum(counts, C), "assign_row": assign_row,
            "row_token": row_token, "rows": E * C}


def expert_choice(logits, C: int, gate: str, scores=None) -> dict:
    """Every expert takes the C tokens with the largest router probability
    (router_probs rounded to fp32; ties to the earlier token) and lays them
    out in token order at rows e*C .. e*C+C-1.  ``scores``: optional fp32
    [T,E] to decide on instead (e.g. the device's own probabilities).

    sel_row [T,E]: row of (t, e) or -1; gate [T,E]: the chosen token's score
    (0 where not chosen); row_token [E*C]; counts [E] = C."""
    if scores is None:
        p = router_probs(logits, gate).astype(np.float32)
    else:
        p = np.asarray(scores, dtype=np.float32)
    T, E = p.shape
    if not 0 < C <= T:
        raise ValueError("expert choice needs 0 < C <= T")
    sel_row = np.full((T, E), -1, dtype=np.int64)
    g = np.zeros((T, E), dtype=np.float32)
    row_token = np.empty(E * C, dtype=np.int64)
    for e in range(E):
        top = np.argsort(-p[:, e].astype(np.float64), kind="stable")[:C]
        for r, t in enumerate(np.sort(top)):
            sel_row[t, e] = e * C + r
            g[t, e] = p[t, e]
            row_token[e * C + r] = t
    return {"scores": p, "sel_row": sel_row, "gate": g, "row_token": row_token,
            "counts": np.full(E, C, dtype=np.int64),
            "offsets": np.arange(E + 1, dtype=np.int64) * C, "rows": E * C}


def expert_choice_forward(x, w_router, w1, w3, w2, *, C: int, gate: str, logit_bias=None,
                          shared=None, tokens=None, scores=None) -> dict:
    """Layer forward with expert-choice routing: y[t] = sum over the experts
    that chose t, in expert order, of gate[t,e] * FFN_e(x[t]) (+ shared)."""
    logits = router_logits(x, w_router, logit_bias)
    m = expert_choice(logits, C, gate, scores)
    T, E = m["sel_row"].shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xs = _f64(x[tok])
    y = np.zeros((len(tok), x.shape[1]), dtype=np.float64)
    for e in range(E):                      # expert order
        chosen = m["sel_row"][tok, e] >= 0
        if chosen.any():
            o = swiglu_ffn(xs[chosen], w1[e], w3[e], w2[e])
            y[chosen] += _f64(m["gate"][tok[chosen], e])[:, None] * o
    if shared is not None:
        ws1, ws3, ws2 = shared
        y += swiglu_ffn(xs, ws1, ws3, ws2)
    m.update({"logits": logits, "y": y, "tokens": tok})
    return m


# ---------------------------------------------------------------------------
# 8b. Sinkhorn routing.  Megatron-LM part 6, "负载均衡" table, row sinkhorn:
# Sinkhorn iterations rescale the routing matrix until it is doubly
# stochastic, which evens out the load with no auxiliary loss.  The page
# gives nothing more; the reading taken: the matrix is exp(l) [T,E]; one
# iteration scales every row to sum 1 and then every column to sum T/E
# (the T x E form of a doubly stochastic matrix); the iteration count is an
# input; each token takes the k largest entries of its row of the balanced
# matrix, and its gates come from the logits as for plain top-k.
# ---------------------------------------------------------------------------
def sinkhorn(logits, iters: int) -> dict:
    """Sinkhorn-Knopp balancing of exp(logits), fp64.

    Returns ``P`` [T,E] after ``iters`` row-then-column scalings, ``col``
    [E], the product of every column factor applied (so that
    P = diag(r) exp(l) diag(col) for some row factors r), and ``bias`` =
    fp32(ln col).  Within row t the row factor is common and ln is
    increasing, so ranking P[t] is ranking l[t,e] + ln col[e]: the balanced
    top-k is topk(selection_keys(l, bias), k).  Each row is shifted by its
    maximum before exp (the first row scaling cancels any per-row factor).
    """
    if iters < 1:
        raise ValueError("need iters >= 1")
    l = _f64(logits)
    T, E = l.shape
    P = np.exp(l - l.max(axis=1, keepdims=True))
    col = np.ones(E)
    for _ in range(iters):
        P = P / P.sum(axis=1, keepdims=True)        # rows to 1
        f = (T / E) / P.sum(axis=0)                 # columns to T/E
        P = P * f[None, :]
        col = col * f
    return {"P": P, "col": col, "bias": np.log(col).astype(np.float32)}


# ---------------------------------------------------------------------------
# 9. Backward.  专家并行 page, "EP+DP" BWD: every GPU computes the gradients
# of its experts' weights, and the gradients go back along the routing path
# (the reverse all-to-all) into the layers before; Megatron-LM part 6, "MoE
# 层的数据流" (the same chain, reversed).  This is the gradient of the
# forward above by the chain rule, in fp64, with the top-k choice and the
# capacity drops held fixed (they are not differentiable): a dropped slot
# passes no gradient, the selection-only bias gets none.
# ---------------------------------------------------------------------------
def _gates_backward(l, idx, dg, mode: str) -> np.ndarray:
    """dL/dlogits [T,E] from dL/dgates [T,k] (fp64), for the gate modes of
    gates()."""
    T, E = l.shape
    dl = np.zeros((T, E))
    rows = np.arange(T)[:, None]
    if mode == "softmax_topk":
        sel = np.take_along_axis(l, idx, axis=1)
        ex = np.exp(sel - sel.max(axis=1, keepdims=True))
        g = ex / ex.sum(axis=1, keepdims=True)
        dsel = g * (dg - (g * dg).sum(axis=1, keepdims=True))
        np.add.at(dl, (rows, idx), dsel)
    elif mode == "softmax_all_topk":
        ex = np.exp(l - l.max(axis=1, keepdims=True))
        p = ex / ex.sum(axis=1, keepdims=True)
        dp = np.zeros((T, E))
        np.add.at(dp, (rows, idx), dg)
        dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    elif mode == "sigmoid_topk_norm":
        sel = np.take_along_axis(l, idx, axis=1)
        sg = 1.0 / (1.0 + np.exp(-sel))
        S = sg.sum(axis=1, keepdims=True)
        g = sg / S
        ds = (dg - (g * dg).sum(axis=1, keepdims=True)) / S
        np.add.at(dl, (rows, idx), ds * sg * (1.0 - sg))
    else:
        raise ValueError(f"unknown gate mode {mode!r}")
    return dl


def _ffn_backward(xr, dO, w1, w3, w2):
    """SwiGLU expert on rows xr with output gradient dO: returns the expert
    output o, dx, dw1, dw3, dw2 (fp64)."""
    W1, W3, W2 = _f64(w1), _f64(w3), _f64(w2)
    a1 = xr @ W1.T
    a3 = xr @ W3.T
    s = 1.0 / (1.0 + np.exp(-a1))
    u = a1 * s * a3
    o = u @ W2.T
    dW2 = dO.T @ u
    dU = dO @ W2
    dA1 = dU * a3 * (s + a1 * s * (1.0 - s))     # d silu(z)/dz = s + z s (1 - s)
    dA3 = dU * a1 * s
    return o, dA1 @ W1 + dA3 @ W3, dA1.T @ xr, dA3.T @ xr, dW2


def moe_backward(x, w_router, w1, w3, w2, dy, *, k: int, gate: str, C: Optional[int] = None,
                 logit_bias=None, select_bias=None, shared=None, idx=None,
                 drop: str = "token", priority=None, tokens=None) -> dict:
    """Gradients of L = sum(y * dy) for the layer forward (same arguments as
    moe_forward; ``idx``/``priority`` fix the routing to another choice).
    Returns fp64 dx [T,h], dw_router [E,h], dlogit_bias [E], dw1/dw3 [E,F,h],
    dw2 [E,h,F], dws1/dws3/dws2 (shared expert), dgate [T,k], dlogits [T,E].
    ``tokens``: only dx, dgate and dlogits of these tokens (rows in that
    order), token by token; the weight gradients are not computed."""
    if tokens is not None:
        return _backward_rows(x, w_router, w1, w3, w2, dy, k=k, gate=gate, C=C,
                              logit_bias=logit_bias, select_bias=select_bias, shared=shared,
                              idx=idx, drop=drop, priority=priority, tokens=tokens)
    x = np.asarray(x)
    T, h = x.shape
    E = np.asarray(w_router).shape[0]
    fwd = moe_forward(x, w_router, w1, w3, w2, k=k, gate=gate, C=C, logit_bias=logit_bias,
                      select_bias=select_bias, idx=idx, maps_only=True, drop=drop,
                      priority=priority)
    l = _f64(fwd["logits"])
    idx = fwd["idx"].astype(np.int64)
    kept = fwd["maps"]["assign_row"] >= 0
    g = _f64(fwd["gates"])
    xs = _f64(x)
    dY = _f64(dy)
    dx = np.zeros((T, h))
    dg = np.zeros((T, k))
    dw1 = [None] * E
    dw3 = [None] * E
    dw2 = [None] * E
    for e in range(E):
        tt, jj = np.nonzero((idx == e) & kept)
        if len(tt) == 0:
            F = np.asarray(w1[e]).shape[0]
            dw1[e] = np.zeros((F, h))
            dw3[e] = np.zeros((F, h))
            dw2[e] = np.zeros((h, F))
            continue
        dO = g[tt, jj][:, None] * dY[tt]
        o, dxe, dw1[e], dw3[e], dw2[e] = _ffn_backward(xs[tt], dO, w1[e], w3[e], w2[e])
        dg[tt, jj] = (dY[tt] * o).sum(axis=1)
        np.add.at(dx, tt, dxe)
    out = {"dw1": np.stack(dw1), "dw3": np.stack(dw3), "dw2": np.stack(dw2), "dgate": dg}
    if shared is not None:
        ws1, ws3, ws2 = shared
        _, dxs, out["dws1"], out["dws3"], out["dws2"] = _ffn_backward(xs, dY, ws1, ws3, ws2)
        dx += dxs
    dl = _gates_backward(l, idx, dg, gate)
    out["dlogits"] = dl
    out["dlogit_bias"] = dl.sum(axis=0)
    out["dw_router"] = dl.T @ xs
    out["dx"] = dx + dl @ _f64(w_router)
    out["idx"] = idx
    out["maps"] = fwd["maps"]
    return out


def expert_choice_backward(x, w_router, w1, w3, w2, dy, *, C: int, gate: str,
                           logit_bias=None, shared=None, scores=None) -> dict:
    """Gradients of L = sum(y * dy) for expert_choice_forward, the experts'
    choices held fixed.  The gate of a chosen (t, e) is router_probs[t, e]
    itself, not renormalised over the experts that chose t, so the logits
    get the Jacobian of router_probs applied to dgate [T,E] (zero where e did
    not choose t): the token-choice gate Jacobians with every expert as a
    slot (softmax over all E; sigmoids normalised over all E).  Returns fp64
    dx, dw_router, dlogit_bias, dw1/dw3/dw2, dws1/dws3/dws2 (shared expert),
    dgate [T,E], dlogits [T,E]."""
    x = np.asarray(x)
    T, h = x.shape
    logits = router_logits(x, w_router, logit_bias)
    m = expert_choice(logits, C, gate, scores)
    E = m["sel_row"].shape[1]
    chosen = m["sel_row"] >= 0
    g = _f64(m["gate"])
    xs = _f64(x)
    dY = _f64(dy)
    dx = np.zeros((T, h))
    dg = np.zeros((T, E))
    dw1, dw3, dw2 = [], [], []
    for e in range(E):                      # C >= 1: every expert has rows
        tt = np.nonzero(chosen[:, e])[0]
        dO = g[tt, e][:, None] * dY[tt]
        o, dxe, d1, d3, d2 = _ffn_backward(xs[tt], dO, w1[e], w3[e], w2[e])
        dw1.append(d1)
        dw3.append(d3)
        dw2.append(d2)
        dg[tt, e] = (dY[tt] * o).sum(axis=1)
        np.add.at(dx, tt, dxe)
    out = {"dw1": np.stack(dw1), "dw3": np.stack(dw3), "dw2": np.stack(dw2), "dgate": dg}
    if shared is not None:
        ws1, ws3, ws2 = shared
        _, dxs, out["dws1"], out["dws3"], out["dws2"] = _ffn_backward(xs, dY, ws1, ws3, ws2)
        dx += dxs
    every = np.tile(np.arange(E), (T, 1))
    mode = "sigmoid_topk_norm" if gate == "sigmoid_topk_norm" else "softmax_all_topk"
    dl = _gates_backward(_f64(logits), every, dg, mode)
    out["dlogits"] = dl
    out["dlogit_bias"] = dl.sum(axis=0)
    out["dw_router"] = dl.T @ xs
    out["dx"] = dx + dl @ _f64(w_router)
    out["maps"] = m
    return out


def _backward_rows(x, w_router, w1, w3, w2, dy, *, k, gate, C, logit_bias, select_bias, shared,
                   idx, drop, priority, tokens) -> dict:
    """dx, dgate and dlogits of the given tokens only (see moe_backward)."""
    fwd = moe_forward(x, w_router, w1, w3, w2, k=k, gate=gate, C=C, logit_bias=logit_bias,
                      select_bias=select_bias, idx=idx, maps_only=True, drop=drop,
                      priority=priority)
    tok = np.asarray(tokens, dtype=np.int64)
    l = _f64(fwd["logits"])[tok]
    sel = fwd["idx"].astype(np.int64)[tok]
    kept = fwd["maps"]["assign_row"][tok] >= 0
    g = _f64(fwd["gates"])[tok]
    xs = _f64(np.asarray(x)[tok])
    dY = _f64(np.asarray(dy)[tok])
    dx = np.zeros_like(xs)
    dg = np.zeros((len(tok), k))
    for n in range(len(tok)):
        for j in range(k):
            if not kept[n, j]:
                continue
            e = int(sel[n, j])
            W1, W3, W2 = _f64(w1[e]), _f64(w3[e]), _f64(w2[e])
            a1 = W1 @ xs[n]
            a3 = W3 @ xs[n]
            s = 1.0 / (1.0 + np.exp(-a1))
            u = a1 * s * a3
            dg[n, j] = float(dY[n] @ (W2 @ u))
            dU = (g[n, j] * dY[n]) @ W2
            dx[n] += (dU * a3 * (s + a1 * s * (1.0 - s))) @ W1 + (dU * a1 * s) @ W3
    if shared is not None:
        ws1, ws3, ws2 = (_f64(w) for w in shared)
        a1 = xs @ ws1.T
        a3 = xs @ ws3.T
        s = 1.0 / (1.0 + np.exp(-a1))
        dU = dY @ ws2
        dx += (dU * a3 * (s + a1 * s * (1.0 - s))) @ ws1 + (dU * a1 * s) @ ws3
    dl = _gates_backward(l, sel, dg, gate)
    return {"dx": dx + dl @ _f64(w_router), "dgate": dg, "dlogits": dl, "tokens": tok}
