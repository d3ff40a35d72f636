"""Python binding of libmoe (MoE layer forward on MI355X / gfx950).

Argument marshalling only: every function passes torch tensors' device
pointers and the current HIP stream to the function of the same name in
libmoe.so (declared in include/moe.h) and raises on a non-zero status.  No
step of the layer runs here.  torch provides device memory and streams.

If libmoe.so has not been built, every call raises ``RuntimeError``: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1

MOE_GATE_SOFTMAX_TOPK = 0
MOE_GATE_SOFTMAX_ALL_TOPK = 1
MOE_GATE_SIGMOID_TOPK_NORM = 2

MOE_NUM_STAGES = 8
MOE_NUM_EVENTS = 2 * MOE_NUM_STAGES     # a start and a stop event per stage
STAGE_NAMES = ("router", "topk", "scan", "assign", "permute", "gemm1_swiglu",
               "gemm2", "combine")

GATE_BY_NAME = {
    "softmax_topk": MOE_GATE_SOFTMAX_TOPK,
    "softmax_all_topk": MOE_GATE_SOFTMAX_ALL_TOPK,
    "sigmoid_topk_norm": MOE_GATE_SIGMOID_TOPK_NORM,
}
DTYPE_BY_NAME = {"f32": MOE_DTYPE_F32, "bf16": MOE_DTYPE_BF16}
MOE_ROUTE_TOPK = 0
MOE_ROUTE_TOPK_SCORE_DROP = 1
MOE_ROUTE_EXPERT_CHOICE = 2
MOE_ROUTE_SINKHORN = 3
MOE_MAX_SINKHORN_ITERS = 1000
ROUTING_BY_NAME = {
    "topk": MOE_ROUTE_TOPK,
    "topk_score_drop": MOE_ROUTE_TOPK_SCORE_DROP,
    "expert_choice": MOE_ROUTE_EXPERT_CHOICE,
    "sinkhorn": MOE_ROUTE_SINKHORN,
}

# Every symbol include/moe.h declares.
ABI_SYMBOLS = (
    "moe_strerror", "moe_capacity", "moe_num_rows", "moe_workspace_bytes",
    "moe_router_topk", "moe_permute", "moe_permute_rows", "moe_grouped_gemm_swiglu",
    "moe_grouped_gemm_swiglu_noalloc", "moe_unpermute_combine", "moe_load_balance", "moe_select_bias_update",
    "moe_backward_workspace_bytes",
    "moe_backward", "moe_backward_saved", "moe_forward",
)


class MoECfg(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("T", ctypes.c_int64),
        ("h", ctypes.c_int32),
        ("F", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("gate", ctypes.c_int32),
        ("has_shared", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("routing", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("sinkhorn_iters", ctypes.c_int32),
    ]


class MoEWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "w1", "w3", "w2", "logit_bias", "select_bias", "ws1", "ws3", "ws2")]


class MoERouteOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "topk_idx", "topk_gate", "expert_counts", "expert_offsets",
        "assign_row", "row_token", "probs", "route_bias")]


class MoEGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dx", "dw_router", "dlogit_bias", "dw1", "dw3", "dw2", "dws1", "dws3", "dws2",
        "dgate")]


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({strerror(status)})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixture_experts_layer_25_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cfgp = ctypes.POINTER(MoECfg)
        sig = {
            "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_capacity": (ctypes.c_int, [I64, I32, I32, I64, I64, ctypes.POINTER(I64)]),
            "moe_num_rows": (ctypes.c_int, [cfgp, ctypes.POINTER(I64)]),
            "moe_workspace_bytes": (ctypes.c_int, [cfgp, ctypes.POINTER(SZ)]),
            "moe_router_topk": (ctypes.c_int, [cfgp, P, P, P, P, P, P, P, P, SZ, P]),
            "moe_permute": (ctypes.c_int, [cfgp, P, P, P, P, P, P, P, P, SZ, P]),
            "moe_permute_rows": (ctypes.c_int, [cfgp, P, P, P, P, P, P]),
            "moe_grouped_gemm_swiglu": (ctypes.c_int, [cfgp, P, P, P, P, P, P, P, P, P, SZ, P]),
            "moe_grouped_gemm_swiglu_noalloc": (ctypes.c_int, [cfgp, P, P, P, P, P, P, P, P, P]),
            "moe_unpermute_combine": (ctypes.c_int, [cfgp, P, P, P, P, P, P]),
            "moe_load_balance": (ctypes.c_int, [cfgp, P, P, ctypes.c_float, P, P, P, P, SZ,
                                                P]),
            "moe_select_bias_update": (ctypes.c_int, [cfgp, P, ctypes.c_float, P, P]),
            "moe_backward_workspace_bytes": (ctypes.c_int, [cfgp, ctypes.POINTER(SZ)]),
            "moe_backward": (ctypes.c_int, [cfgp, ctypes.POINTER(MoEWeights), P, P,
                                            ctypes.POINTER(MoERouteOut),
                                            ctypes.POINTER(MoEGrads), P, SZ, P]),
            "moe_backward_saved": (ctypes.c_int, [cfgp, ctypes.POINTER(MoEWeights), P, P,
                                                  ctypes.POINTER(MoERouteOut), P, SZ,
                                                  ctypes.POINTER(MoEGrads), P, SZ, P]),
            "moe_forward": (ctypes.c_int, [cfgp, ctypes.POINTER(MoEWeights), P, P,
                                           ctypes.POINTER(MoERouteOut), P, SZ, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().moe_strerror(status).decode()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status)


def _ptr(t, nbytes: int = 0, name: str = "tensor") -> Optional[int]:
    """Device pointer of a tensor (None stays NULL).  The kernels take the
    pointer as a device address and trust the sizes the config implies, so a
    host tensor or one smaller than ``nbytes`` is refused here."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"libmoe takes device tensors: {name} is on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"libmoe takes contiguous tensors: {name} is not")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the config needs {nbytes}")
    return t.data_ptr()


def _sizes(cfg) -> dict:
    """Bytes each named tensor of a call must hold for ``cfg`` (empty when
    the library refuses the config: the call itself then reports why)."""
    rows = ctypes.c_int64()
    if lib().moe_num_rows(ctypes.byref(cfg), ctypes.byref(rows)) != MOE_OK:
        return {}
    T, h, F, E, k = cfg.T, cfg.h, cfg.F, cfg.E, cfg.k
    R = rows.value
    es = 2 if cfg.dtype == MOE_DTYPE_BF16 else 4
    slots = E if cfg.routing == MOE_ROUTE_EXPERT_CHOICE else k
    return {
        "x": T * h * es, "y": T * h * es, "dy": T * h * es, "dx": T * h * es,
        "shared_y": T * h * es,
        "w_router": E * h * es, "dw_router": E * h * es,
        "w1": E * F * h * es, "w3": E * F * h * es, "w2": E * h * F * es,
        "dw1": E * F * h * es, "dw3": E * F * h * es, "dw2": E * h * F * es,
        "ws1": F * h * es, "ws3": F * h * es, "ws2": h * F * es,
        "dws1": F * h * es, "dws3": F * h * es, "dws2": h * F * es,
        "logit_bias": E * 4, "select_bias": E * 4, "dlogit_bias": E * 4, "route_bias": E * 4,
        "logits": T * E * 4, "probs": E * T * 4,
        "topk_idx": T * k * 4, "topk_gate": T * slots * 4, "assign_row": T * slots * 4,
        "dgate": T * slots * 4,
        "expert_counts": E * 4, "expert_offsets": (E + 1) * 4, "row_token": R * 4,
        "x_perm": R * h * es, "act": R * F * es, "y_perm": R * h * es,
        "f": E * 4, "P": E * 4, "aux_loss": 4,
    }


def _p(sizes: dict, name: str, t) -> Optional[int]:
    return _ptr(t, sizes.get(name, 0), name)


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


MOE_FLAG_SAVE_FOR_BACKWARD = 1


def make_cfg(T: int, h: int, F: int, E: int, k: int, dtype="bf16",
             gate="softmax_topk", capacity: int = 0, has_shared: bool = False,
             routing="topk", save_for_backward: bool = False,
             sinkhorn_iters: int = 0) -> MoECfg:
    c = MoECfg()
    c.struct_size = ctypes.sizeof(MoECfg)
    c.dtype = DTYPE_BY_NAME[dtype] if isinstance(dtype, str) else int(dtype)
    c.T, c.h, c.F, c.E, c.k = T, h, F, E, k
    c.gate = GATE_BY_NAME[gate] if isinstance(gate, str) else int(gate)
    c.has_shared = int(bool(has_shared))
    c.capacity = int(capacity)
    c.routing = ROUTING_BY_NAME[routing] if isinstance(routing, str) else int(routing)
    c.flags = MOE_FLAG_SAVE_FOR_BACKWARD if save_for_backward else 0
    c.sinkhorn_iters = int(sinkhorn_iters)
    return c


def moe_capacity(T: int, E: int, k: int, cf_num: int, cf_den: int) -> int:
    out = ctypes.c_int64()
    _check("moe_capacity", lib().moe_capacity(T, E, k, cf_num, cf_den, ctypes.byref(out)))
    return out.value


def moe_num_rows(cfg: MoECfg) -> int:
    out = ctypes.c_int64()
    _check("moe_num_rows", lib().moe_num_rows(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def moe_workspace_bytes(cfg: MoECfg) -> int:
    out = ctypes.c_size_t()
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def _ws(ws):
    """Workspace pointer and size (the library checks the size itself)."""
    if ws is None:
        return None, 0
    if not ws.is_cuda:
        raise ValueError(f"libmoe takes a device workspace: it is on {ws.device}")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def moe_router_topk(cfg, x, w_router, logit_bias, select_bias, logits, topk_idx,
                    topk_gate, ws=None, stream=None) -> None:
    wp, wb = _ws(ws)
    z = _sizes(cfg)
    _check("moe_router_topk", lib().moe_router_topk(
        ctypes.byref(cfg), _p(z, "x", x), _p(z, "w_router", w_router),
        _p(z, "logit_bias", logit_bias), _p(z, "select_bias", select_bias),
        _p(z, "logits", logits), _p(z, "topk_idx", topk_idx), _p(z, "topk_gate", topk_gate),
        wp, wb, _stream(stream)))


def moe_permute(cfg, x, topk_idx, expert_counts, expert_offsets, assign_row,
                row_token, x_perm, ws, stream=None) -> None:
    wp, wb = _ws(ws)
    z = _sizes(cfg)
    _check("moe_permute", lib().moe_permute(
        ctypes.byref(cfg), _p(z, "x", x), _p(z, "topk_idx", topk_idx),
        _p(z, "expert_counts", expert_counts), _p(z, "expert_offsets", expert_offsets),
        _p(z, "assign_row", assign_row), _p(z, "row_token", row_token),
        _p(z, "x_perm", x_perm), wp, wb, _stream(stream)))


def moe_permute_rows(cfg, x, assign_row, expert_counts, row_token, x_perm,
                     stream=None) -> None:
    """Dispatch x by a routing already made (assign_row, expert_counts from
    moe_permute or moe_forward)."""
    z = _sizes(cfg)
    _check("moe_permute_rows", lib().moe_permute_rows(
        ctypes.byref(cfg), _p(z, "x", x), _p(z, "assign_row", assign_row),
        _p(z, "expert_counts", expert_counts), _p(z, "row_token", row_token),
        _p(z, "x_perm", x_perm), _stream(stream)))


def moe_grouped_gemm_swiglu(cfg, x_perm, expert_counts, expert_offsets, w1, w3, w2,
                            act, y_perm, ws, stream=None) -> None:
    wp, wb = _ws(ws)
    z = _sizes(cfg)
    _check("moe_grouped_gemm_swiglu", lib().moe_grouped_gemm_swiglu(
        ctypes.byref(cfg), _p(z, "x_perm", x_perm), _p(z, "expert_counts", expert_counts),
        _p(z, "expert_offsets", expert_offsets), _p(z, "w1", w1), _p(z, "w3", w3),
        _p(z, "w2", w2), _p(z, "act", act), _p(z, "y_perm", y_perm), wp, wb,
        _stream(stream)))


def moe_grouped_gemm_swiglu_noalloc(cfg, x_perm, expert_counts, expert_offsets, w1, w3, w2,
                                    act, y_perm, stream=None) -> None:
    """moe_grouped_gemm_swiglu with the library's own per-GPU scratch instead
    of a workspace (allocates nothing; calls overlapping on one GPU race)."""
    z = _sizes(cfg)
    _check("moe_grouped_gemm_swiglu_noalloc", lib().moe_grouped_gemm_swiglu_noalloc(
        ctypes.byref(cfg), _p(z, "x_perm", x_perm), _p(z, "expert_counts", expert_counts),
        _p(z, "expert_offsets", expert_offsets), _p(z, "w1", w1), _p(z, "w3", w3),
        _p(z, "w2", w2), _p(z, "act", act), _p(z, "y_perm", y_perm), _stream(stream)))


def moe_unpermute_combine(cfg, y_perm, assign_row, topk_gate, shared_y, y,
                          stream=None) -> None:
    z = _sizes(cfg)
    _check("moe_unpermute_combine", lib().moe_unpermute_combine(
        ctypes.byref(cfg), _p(z, "y_perm", y_perm), _p(z, "assign_row", assign_row),
        _p(z, "topk_gate", topk_gate), _p(z, "shared_y", shared_y), _p(z, "y", y),
        _stream(stream)))


def moe_load_balance(cfg, logits, expert_counts, alpha: float, f, P, aux_loss, ws,
                     stream=None) -> None:
    """Share of assignments f [E], mean router probability P [E] and the
    Switch loss alpha*E*sum(f*P) [1] of a routing (fp32 device outputs)."""
    wp, wb = _ws(ws)
    z = _sizes(cfg)
    _check("moe_load_balance", lib().moe_load_balance(
        ctypes.byref(cfg), _p(z, "logits", logits), _p(z, "expert_counts", expert_counts),
        float(alpha), _p(z, "f", f), _p(z, "P", P), _p(z, "aux_loss", aux_loss), wp, wb,
        _stream(stream)))


def moe_select_bias_update(cfg, expert_counts, gamma: float, select_bias, stream=None) -> None:
    """One aux-loss-free balancing step, in place on select_bias [E] fp32: an
    expert with more than the mean T*k/E routed assignments (expert_counts
    [E] int32) loses gamma, one with fewer gains gamma."""
    z = _sizes(cfg)
    _check("moe_select_bias_update", lib().moe_select_bias_update(
        ctypes.byref(cfg), _p(z, "expert_counts", expert_counts), float(gamma),
        _p(z, "select_bias", select_bias), _stream(stream)))


def moe_backward_workspace_bytes(cfg: MoECfg) -> int:
    out = ctypes.c_size_t()
    _check("moe_backward_workspace_bytes",
           lib().moe_backward_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def moe_backward(cfg, weights: dict, x, dy, route: dict, grads: dict, ws, stream=None) -> None:
    """Gradients of sum(y * dy) with the routing of a forward call held
    fixed.  ``route``: that call's logits, topk_idx, topk_gate,
    expert_counts, expert_offsets and assign_row; ``grads``: dict of output
    tensors (dx, dw1, dw3, dw2 required; dw_router, dlogit_bias, dgate and
    the shared expert's dws1/dws3/dws2 as needed)."""
    wp, wb = _ws(ws)
    z = _sizes(cfg)
    g = _struct(MoEGrads, grads, z)
    _check("moe_backward", lib().moe_backward(
        ctypes.byref(cfg), ctypes.byref(weights_struct(weights, cfg)), _p(z, "x", x),
        _p(z, "dy", dy), ctypes.byref(route_struct(route, cfg)), ctypes.byref(g), wp, wb,
        _stream(stream)))


def moe_backward_saved(cfg, weights: dict, x, dy, route: dict, fwd_ws, grads: dict, ws,
                       stream=None) -> None:
    """moe_backward from the activations the moe_forward call kept in its
    workspace ``fwd_ws`` (cfg made with save_for_backward=True; the same
    cfg, weights, x and routing outputs)."""
    fp, fb = _ws(fwd_ws)
    wp, wb = _ws(ws)
    z = _sizes(cfg)
    g = _struct(MoEGrads, grads, z)
    _check("moe_backward_saved", lib().moe_backward_saved(
        ctypes.byref(cfg), ctypes.byref(weights_struct(weights, cfg)), _p(z, "x", x),
        _p(z, "dy", dy), ctypes.byref(route_struct(route, cfg)), fp, fb, ctypes.byref(g),
        wp, wb, _stream(stream)))


def _struct(kind, tensors: dict, sizes: dict):
    s = kind()
    for name, _ in kind._fields_:
        setattr(s, name, _p(sizes, name, tensors.get(name)))
    return s


def weights_struct(w: dict, cfg: Optional[MoECfg] = None) -> MoEWeights:
    return _struct(MoEWeights, w, _sizes(cfg) if cfg is not None else {})


def route_struct(r: Optional[dict], cfg: Optional[MoECfg] = None) -> Optional[MoERouteOut]:
    if r is None:
        return None
    return _struct(MoERouteOut, r, _sizes(cfg) if cfg is not None else {})


def moe_forward(cfg, weights: dict, x, y, route: Optional[dict] = None, ws=None,
                events=None, stream=None) -> None:
    """Fused layer.  ``weights``: dict with w_router, w1, w3, w2 and optional
    logit_bias, select_bias, ws1, ws3, ws2.  ``route``: optional dict of
    output tensors (logits, topk_idx, topk_gate, expert_counts,
    expert_offsets, assign_row, row_token; probs for expert choice,
    route_bias for Sinkhorn routing).  ``events``: None or
    MOE_NUM_EVENTS ``torch.cuda.Event(enable_timing=True)``: events[2i] and
    events[2i+1] are bound to the start of stage i's first kernel and the end
    of its last kernel (``events[2*i].elapsed_time(events[2*i+1])`` is the
    stage's kernel time in ms)."""
    wp, wb = _ws(ws)
    z = _sizes(cfg)
    ws_struct = weights_struct(weights, cfg)
    rs = route_struct(route, cfg)
    ev = None
    if events is not None:
        if len(events) != MOE_NUM_EVENTS:
            raise ValueError(f"need {MOE_NUM_EVENTS} events")
        handles = []
        for e in events:
            if not e.cuda_event:      # torch creates its events on first record
                e.record()
            handles.append(e.cuda_event)
        ev = (ctypes.c_void_p * MOE_NUM_EVENTS)(*handles)
    _check("moe_forward", lib().moe_forward(
        ctypes.byref(cfg), ctypes.byref(ws_struct), _p(z, "x", x), _p(z, "y", y),
        ctypes.byref(rs) if rs is not None else None, wp, wb, ev, _stream(stream)))
