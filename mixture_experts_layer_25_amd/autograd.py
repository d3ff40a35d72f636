"""torch.autograd wrapper of the layer.

Argument marshalling only: the forward is one ``moe_forward`` call made with
``save_for_backward`` (the library keeps the activations in the forward's
workspace), the backward one ``moe_backward_saved`` call on that workspace.
Every step of both runs in libmoe; nothing here computes.

    y = moe_layer(x, w_router, w1, w3, w2, k=2, gate="softmax_topk")
    (y * dy).sum().backward()      # x.grad, w_router.grad, w1.grad, ...

The routing (top-k choice, capacity drops, expert choice) is held fixed in
the backward, as ``moe_backward`` documents.  Tensors must be contiguous, on
one device, all bf16 or all fp32 (logit_bias fp32).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import (make_cfg, moe_backward_saved, moe_backward_workspace_bytes, moe_forward,
               moe_workspace_bytes)


def _route_buffers(T: int, E: int, k: int, expert_choice: bool, device) -> dict:
    slots = E if expert_choice else k
    i32, f32 = torch.int32, torch.float32
    r = {"logits": torch.empty((T, E), dtype=f32, device=device),
         "topk_idx": torch.empty((T, k), dtype=i32, device=device),
         "topk_gate": torch.empty((T, slots), dtype=f32, device=device),
         "expert_counts": torch.empty((E,), dtype=i32, device=device),
         "expert_offsets": torch.empty((E + 1,), dtype=i32, device=device),
         "assign_row": torch.empty((T * slots,), dtype=i32, device=device)}
    if expert_choice:
        r["probs"] = torch.empty((E, T), dtype=f32, device=device)
    return r


class _MoELayer(torch.autograd.Function):
    @staticmethod
    def forward(ctx, settings: dict, x, w_router, w1, w3, w2, logit_bias, select_bias,
                ws1, ws3, ws2):
        for t in (x, w_router, w1, w3, w2, logit_bias, select_bias, ws1, ws3, ws2):
            if t is not None and not t.is_contiguous():
                raise ValueError("moe_layer takes contiguous tensors")
        T, h = x.shape
        E, F = w1.shape[0], w1.shape[1]
        dtype = "bf16" if x.dtype == torch.bfloat16 else "f32"
        shared = ws1 is not None
        cfg = make_cfg(T, h, F, E, settings["k"], dtype, settings["gate"],
                       capacity=settings["capacity"], has_shared=shared,
                       routing=settings["routing"], save_for_backward=True,
                       sinkhorn_iters=settings["sinkhorn_iters"])
        ws = torch.empty(max(moe_workspace_bytes(cfg), 1), dtype=torch.uint8, device=x.device)
        route = _route_buffers(T, E, settings["k"], settings["routing"] == "expert_choice",
                               x.device)
        y = torch.empty_like(x)
        weights = {"w_router": w_router, "w1": w1, "w3": w3, "w2": w2, "logit_bias": logit_bias,
                   "select_bias": select_bias, "ws1": ws1, "ws3": ws3, "ws2": ws2}
        moe_forward(cfg, weights, x, y, route, ws)
        ctx.cfg, ctx.route, ctx.fwd_ws = cfg, route, ws
        ctx.has_bias = logit_bias is not None
        ctx.save_for_backward(x, w_router, w1, w3, w2, logit_bias, select_bias, ws1, ws3, ws2)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w_router, w1, w3, w2, logit_bias, select_bias, ws1, ws3, ws2 = ctx.saved_tensors
        dy = dy.contiguous().to(x.dtype)
        e = torch.empty_like
        grads = {"dx": e(x), "dw_router": e(w_router), "dw1": e(w1), "dw3": e(w3), "dw2": e(w2)}
        if ctx.has_bias:
            grads["dlogit_bias"] = torch.empty_like(logit_bias)
        if ws1 is not None:
            grads.update({"dws1": e(ws1), "dws3": e(ws3), "dws2": e(ws2)})
        wsb = torch.empty(max(moe_backward_workspace_bytes(ctx.cfg), 1), dtype=torch.uint8,
                          device=x.device)
        weights = {"w_router": w_router, "w1": w1, "w3": w3, "w2": w2, "logit_bias": logit_bias,
                   "select_bias": select_bias, "ws1": ws1, "ws3": ws3, "ws2": ws2}
        moe_backward_saved(ctx.cfg, weights, x, dy, ctx.route, ctx.fwd_ws, grads, wsb)
        ctx.fwd_ws = None
        return (None, grads["dx"], grads["dw_router"], grads["dw1"], grads["dw3"], grads["dw2"],
                grads.get("dlogit_bias"), None, grads.get("dws1"), grads.get("dws3"),
                grads.get("dws2"))


def moe_layer(x: torch.Tensor, w_router: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor,
              w2: torch.Tensor, *, k: int, gate: str = "softmax_topk", capacity: int = 0,
              routing: str = "topk", sinkhorn_iters: int = 0,
              logit_bias: Optional[torch.Tensor] = None,
              select_bias: Optional[torch.Tensor] = None,
              shared: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None
              ) -> torch.Tensor:
    """The MoE layer y [T,h] of x [T,h] with gradients for x, w_router, w1,
    w3, w2, logit_bias and the shared expert's (ws1, ws3, ws2); select_bias
    gets none (it only decides the top-k).  routing: "topk",
    "topk_score_drop", "expert_choice" or "sinkhorn" (with sinkhorn_iters)."""
    ws1, ws3, ws2 = shared if shared is not None else (None, None, None)
    settings = {"k": k, "gate": gate, "capacity": capacity, "routing": routing,
                "sinkhorn_iters": sinkhorn_iters}
    return _MoELayer.apply(settings, x, w_router, w1, w3, w2, logit_bias, select_bias,
                           ws1, ws3, ws2)
