"""Shared helpers of the GPU tests: run the HIP path, run the oracle on the
same inputs, compare.  (No tests in this module.)"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_layer_25_amd as moe
import oracle
from moe_inputs import MoEConfig, make_inputs

DEV = "cuda"


class LazyExperts:
    """Per-expert fp32 numpy view of a [E, ...] device tensor, fetched on use,
    so the oracle only pulls the experts it needs.  cache=False fetches on
    every use and keeps nothing (the oracle's forward touches each expert
    once; a 256-expert layer would otherwise hold tens of GB of fp32)."""

    def __init__(self, t: torch.Tensor, cache: bool = True):
        self.t = t
        self.keep = cache
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e in self.cache:
            return self.cache[e]
        v = self.t[e].float().cpu().numpy()
        if self.keep:
            self.cache[e] = v
        return v


def np32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def capacity_of(cfg: MoEConfig):
    """(C for the library, C for the oracle), each computed by its own side."""
    if cfg.cf is None:
        return 0, None
    c_lib = moe.moe_capacity(cfg.T, cfg.E, cfg.k, *cfg.cf)
    c_ref = oracle.capacity(cfg.T, cfg.E, cfg.k, *cfg.cf)
    assert c_lib == c_ref
    return c_lib, c_ref


def lib_cfg(cfg: MoEConfig, C: int, routing: str = "topk", save: bool = False,
            sinkhorn_iters: int = 0):
    return moe.make_cfg(cfg.T, cfg.h, cfg.F, cfg.E, cfg.k, cfg.dtype, cfg.gate,
                        capacity=C, has_shared=cfg.shared, routing=routing,
                        save_for_backward=save, sinkhorn_iters=sinkhorn_iters)


def run_forward(cfg: MoEConfig, inp: dict, C: int, routing: str = "topk",
                save: bool = False, sinkhorn_iters: int = 0) -> dict:
    """moe_forward with every routing output requested; tensors stay on GPU.
    With expert choice the per-token slots are the E experts.  save: the
    forward keeps its activations for moe_backward_saved (out["ws"])."""
    c = lib_cfg(cfg, C, routing, save, sinkhorn_iters)
    T, E, k, h = cfg.T, cfg.E, cfg.k, cfg.h
    slots = E if routing == "expert_choice" else k
    rows = moe.moe_num_rows(c)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    route = {
        "logits": torch.empty((T, E), dtype=torch.float32, device=DEV),
        "topk_idx": torch.empty((T, k), dtype=torch.int32, device=DEV),
        "topk_gate": torch.empty((T, slots), dtype=torch.float32, device=DEV),
        "expert_counts": torch.empty((E,), dtype=torch.int32, device=DEV),
        "expert_offsets": torch.empty((E + 1,), dtype=torch.int32, device=DEV),
        "assign_row": torch.empty((T * slots,), dtype=torch.int32, device=DEV),
        "row_token": torch.empty((rows,), dtype=torch.int32, device=DEV),
    }
    if routing == "expert_choice":
        route["probs"] = torch.empty((E, T), dtype=torch.float32, device=DEV)
    if routing == "sinkhorn":
        route["route_bias"] = torch.empty((E,), dtype=torch.float32, device=DEV)
    # fill outputs with garbage so that an unwritten entry shows up
    for v in route.values():
        v.fill_(-7)
    y = torch.full((T, h), float("nan"), dtype=tdt, device=DEV)
    ws = torch.empty(max(moe.moe_workspace_bytes(c), 1), dtype=torch.uint8, device=DEV)
    weights = {n: inp[n] for n in ("w_router", "w1", "w3", "w2", "logit_bias",
                                   "select_bias", "ws1", "ws3", "ws2")}
    moe.moe_forward(c, weights, inp["x"], y, route, ws)
    torch.cuda.synchronize()
    out = dict(route)
    out["y"] = y
    out["rows"] = rows
    out["ws"] = ws
    return out


def oracle_weights(cfg: MoEConfig, inp: dict):
    """(x, w_router, w1, w3, w2, logit_bias, shared) as the oracle takes them."""
    lb = None if inp["logit_bias"] is None else inp["logit_bias"].cpu().numpy()
    shared = None
    if cfg.shared:
        shared = (np32(inp["ws1"]), np32(inp["ws3"]), np32(inp["ws2"]))
    return (np32(inp["x"]), np32(inp["w_router"]), LazyExperts(inp["w1"]),
            LazyExperts(inp["w3"]), LazyExperts(inp["w2"]), lb, shared)


def oracle_forward(cfg: MoEConfig, inp: dict, C_ref, tokens=None, idx=None,
                   maps_only=False, drop="token", priority=None, sinkhorn_iters=None,
                   cache_experts=True):
    x = np32(inp["x"])
    wr = np32(inp["w_router"])
    lb = None if inp["logit_bias"] is None else inp["logit_bias"].cpu().numpy()
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    shared = None
    if cfg.shared and not maps_only:
        shared = (np32(inp["ws1"]), np32(inp["ws3"]), np32(inp["ws2"]))
    lz = lambda t: None if t is None else LazyExperts(t, cache_experts)  # noqa: E731
    w1, w3, w2 = lz(inp["w1"]), lz(inp["w3"]), lz(inp["w2"])
    return oracle.moe_forward(x, wr, w1, w3, w2, k=cfg.k, gate=cfg.gate, C=C_ref,
                              logit_bias=lb, select_bias=sb, shared=shared,
                              tokens=tokens, idx=idx, maps_only=maps_only, drop=drop,
                              priority=priority, sinkhorn_iters=sinkhorn_iters)


def check_routing(cfg: MoEConfig, gpu: dict, ref: dict, C_ref, inp: dict,
                  drop: str = "token", tie: float = 1e-5) -> dict:
    """Routing checks; returns a small report.  drop="score": the capacity
    maps are the score-priority ones, decided on the GPU's own gates.  With
    Sinkhorn routing the GPU's own keys add the GPU's route_bias, and tokens
    whose oracle key gap is below ``tie`` may choose either way."""
    g_logits = gpu["logits"].cpu().numpy()
    g_idx = gpu["topk_idx"].cpu().numpy()
    g_gate = gpu["topk_gate"].cpu().numpy()
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    if "route_bias" in gpu:
        assert sb is None
        sb = gpu["route_bias"].cpu().numpy()
    # logits: fp32-accumulated on the GPU vs fp64-accumulated then rounded
    dl = float(np.abs(g_logits - ref["logits"]).max())
    scale = max(1.0, float(np.abs(ref["logits"]).max()))
    assert dl <= 5e-5 * scale, f"logits differ by {dl}"
    # 1. selection on the GPU's own fp32 keys: bit-exact for every token
    keys_gpu = oracle.selection_keys(g_logits, sb)
    np.testing.assert_array_equal(oracle.topk(keys_gpu, cfg.k), g_idx)
    # 2. selection vs the oracle's logits: exact off near-ties, valid on them
    thr = tie
    tie = oracle.near_tie(ref["keys"], cfg.k, thr)
    same = (np.sort(g_idx, 1) == np.sort(ref["idx"], 1)).all(1)
    assert same[~tie].all(), f"{(~same & ~tie).sum()} non-tie tokens route differently"
    if tie.any():
        kth = -np.sort(-ref["keys"].astype(np.float64), 1)[:, cfg.k - 1]
        chosen = np.take_along_axis(ref["keys"].astype(np.float64), g_idx.astype(np.int64), 1)
        assert (chosen[tie] >= kth[tie, None] - thr).all()
    # 3. gates from the GPU's logits and selection
    g_ref = oracle.gates(g_logits, g_idx, cfg.gate)
    dg = float(np.abs(g_gate - g_ref).max())
    assert dg <= 2e-6, f"gates differ by {dg}"
    # 4. maps recomputed by the oracle from the GPU's selection: bit-exact
    if drop == "score":
        m = oracle.route_maps_score_drop(g_idx, g_gate, cfg.E, C_ref)
    else:
        m = oracle.route_maps(g_idx, cfg.E, C_ref)
    np.testing.assert_array_equal(gpu["expert_counts"].cpu().numpy(), m["counts"])
    np.testing.assert_array_equal(gpu["expert_offsets"].cpu().numpy(), m["offsets"])
    np.testing.assert_array_equal(gpu["assign_row"].cpu().numpy().reshape(-1, cfg.k),
                                  m["assign_row"])
    np.testing.assert_array_equal(gpu["row_token"].cpu().numpy(), m["row_token"])
    return {"max_dlogit": dl, "near_ties": int(tie.sum()), "max_dgate": dg,
            "dropped": int((m["assign_row"] < 0).sum())}


def rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    """max |y_gpu - y_ref| / max |y_ref| (normwise max relative error)."""
    return float(np.abs(y_gpu.astype(np.float64) - y_ref).max() / np.abs(y_ref).max())


def token_rel_err(y_gpu: np.ndarray, y_ref: np.ndarray):
    """Per-token normwise error: for each row t, max_i |y_gpu - y_ref| over
    max_i |y_ref| of that row alone.  Rows whose reference is exactly zero
    (every slot dropped, no shared expert) are returned separately: their
    output must be exactly zero, which ``assert_dropped_rows_zero`` checks.
    Returns (max over the non-zero rows, index of that row, zero-row mask)."""
    d = np.abs(y_gpu.astype(np.float64) - y_ref).max(1)
    m = np.abs(y_ref).max(1)
    zero = m == 0
    r = np.where(zero, 0.0, d / np.where(zero, 1.0, m))
    i = int(r.argmax()) if len(r) else 0
    return (float(r[i]) if len(r) else 0.0), i, zero


def assert_dropped_rows_zero(y_gpu: np.ndarray, zero_rows: np.ndarray) -> int:
    """Rows whose every slot was dropped (and no shared expert) carry no
    expert output at all: each element must be exactly +0.0 or -0.0."""
    if zero_rows.any():
        bad = np.count_nonzero(y_gpu[zero_rows] != 0)
        assert bad == 0, f"{bad} elements of fully dropped tokens are not zero"
    return int(zero_rows.sum())


def check_outputs(cfg: MoEConfig, y_gpu: np.ndarray, y_ref: np.ndarray, label: str) -> dict:
    """The output bars: normwise over all compared rows and per token, both
    within the layer's tolerance; fully dropped rows exactly zero."""
    tol = tol_of(cfg)
    err = rel_err(y_gpu, y_ref) if np.abs(y_ref).max() > 0 else float(np.abs(y_gpu).max())
    terr, worst, zero = token_rel_err(y_gpu, y_ref)
    nzero = assert_dropped_rows_zero(y_gpu, zero)
    assert err <= tol, f"{label}: normwise error {err:.3e} > {tol}"
    assert terr <= tol, f"{label}: token {worst} error {terr:.3e} > {tol}"
    return {"rel_err": f"{err:.2e}", "token_rel_err": f"{terr:.2e}", "zero_rows": nzero}


def tol_of(cfg: MoEConfig) -> float:
    return 2e-2 if cfg.dtype == "bf16" else 1e-5


def gen_inputs(cfg: MoEConfig, device=DEV) -> dict:
    return make_inputs(cfg, device=device)
