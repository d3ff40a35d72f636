"""Seeded synthetic inputs for the MoE layer forward.

This module only draws numbers: it holds no step of the layer's arithmetic
(no routing, capacity, gating or FFN math).  Both the HIP path and the CPU
oracle take their inputs from here, and from nowhere else.

Generation
----------
Every tensor comes from ``torch.randn`` driven by a ``torch.Generator``
seeded with a value derived from (seed, tensor id, chunk).  Values are drawn
in fp32, scaled by the standard deviation, and then rounded to the layer's
storage dtype (bf16 round-to-nearest-even, or kept fp32).  Large weight
tensors are drawn one expert at a time so that peak memory stays at the
tensor's own size.

The generator runs on the device the caller asks for.  ``device="cpu"`` and
``device="cuda"`` draw different (but each deterministic) streams; a test
that compares the HIP path with the oracle draws once, on one device, and
hands the same values to both sides.

Distributions (the page workloads give shapes only; these are the usual
fan-in initialisations, variance 1/fan_in):

* ``x ~ N(0, 1)``
* ``w_router, w1, w3 ~ N(0, 1/h)``, ``w2 ~ N(0, 1/F)`` (shared expert alike)
* logit offsets per expert (``logit_bias``): ``N(0, var)`` or a Zipf(s)
  log-pmf ``-s * ln(e + 1)``
* selection-only bias per expert (``select_bias``): ``N(0, var)``
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import torch

# Fixed ids so that adding a tensor never changes the values of the others.
_TENSOR_ID = {
    "x": 1,
    "w_router": 2,
    "w1": 3,
    "w3": 4,
    "w2": 5,
    "ws1": 6,
    "ws3": 7,
    "ws2": 8,
    "logit_bias": 9,
    "select_bias": 10,
    "dy": 11,           # output gradient of the backward tests and benchmark
    "x_second": 12,     # a second token tensor dispatched by an existing routing
}


@dataclass(frozen=True)
class MoEConfig:
    """Shape and routing description of one MoE layer workload."""

    name: str
    T: int                      # tokens
    h: int                      # model width
    E: int                      # routed experts
    k: int                      # experts per token
    F: int                      # expert FFN width
    dtype: str = "bf16"         # "bf16" or "f32": x, weights, act, y storage
    gate: str = "softmax_topk"  # "softmax_topk" | "softmax_all_topk" | "sigmoid_topk_norm"
    cf: Optional[Tuple[int, int]] = None   # capacity factor as num/den; None = dropless
    shared: bool = False        # one shared expert of the same FFN shape
    logit_bias: Optional[Tuple[str, float]] = None   # ("normal", var) | ("zipf", s)
    select_bias: Optional[Tuple[str, float]] = None  # ("normal", var)
    seed: int = 0

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


# The five workloads.  The second is the dimension table of the worked
# example on the "v6: 长序列和 MoE" page (section "NVIDIA 原题"); the others
# take their shapes from the Mixtral and DeepSeek-V3 models the pages name,
# and from a skewed-routing stress case.
CONFIGS = {
    "tiny_fp32": MoEConfig("tiny_fp32", T=64, h=128, E=4, k=2, F=256,
                           dtype="f32", gate="softmax_topk"),
    "worked_example": MoEConfig("worked_example", T=4096, h=4096, E=8, k=2,
                                F=12288, gate="softmax_all_topk", cf=(5, 4)),
    "mixtral": MoEConfig("mixtral", T=8192, h=4096, E=8, k=2, F=14336,
                         gate="softmax_topk", logit_bias=("normal", 0.5)),
    "deepseek_v3": MoEConfig("deepseek_v3", T=4096, h=7168, E=256, k=8,
                             F=2048, gate="sigmoid_topk_norm",
                             select_bias=("normal", 0.1), shared=True),
    "skewed": MoEConfig("skewed", T=16384, h=2048, E=64, k=4, F=1024,
                        gate="softmax_topk", logit_bias=("zipf", 1.2)),
    "skewed_cf1": MoEConfig("skewed_cf1", T=16384, h=2048, E=64, k=4, F=1024,
                            gate="softmax_topk", logit_bias=("zipf", 1.2),
                            cf=(1, 1)),
}


def _seed_of(seed: int, tensor: str, chunk: int) -> int:
    return (seed * 1_000_003 + _TENSOR_ID[tensor] * 65_537 + chunk) & ((1 << 62) - 1)


def _torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(shape, std: float, seed: int, tensor: str, device="cpu",
           dtype: str = "bf16", chunk: int = 0) -> torch.Tensor:
    """Draw N(0, std^2) values of ``shape``, rounded to ``dtype`` (RNE)."""
    g = torch.Generator(device=device)
    g.manual_seed(_seed_of(seed, tensor, chunk))
    v = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(_torch_dtype(dtype))


def stacked_normal(E: int, shape, std: float, seed: int, tensor: str,
                   device="cpu", dtype: str = "bf16") -> torch.Tensor:
    """[E, *shape] tensor drawn one expert at a time (chunk id = expert)."""
    out = torch.empty((E, *shape), device=device, dtype=_torch_dtype(dtype))
    for e in range(E):
        out[e].copy_(normal(shape, std, seed, tensor, device, dtype, chunk=e))
    return out


def per_expert_bias(spec, E: int, seed: int, tensor: str, device="cpu"):
    """fp32 [E] per-expert offsets, or None."""
    if spec is None:
        return None
    kind, p = spec
    if kind == "normal":
        return normal((E,), math.sqrt(p), seed, tensor, device, "f32")
    if kind == "zipf":
        # log of a Zipf(s) pmf over experts 0..E-1 (expert 0 hottest); the
        # normalising constant is dropped because it shifts every logit alike.
        return torch.tensor([-p * math.log(e + 1.0) for e in range(E)],
                            dtype=torch.float32, device=device)
    raise ValueError(f"unknown bias spec {spec!r}")


def make_inputs(cfg: MoEConfig, device="cpu", with_experts: bool = True) -> dict:
    """All input tensors of ``cfg``.

    Keys: x [T,h], w_router [E,h], w1 [E,F,h], w3 [E,F,h], w2 [E,h,F],
    ws1/ws3 [F,h], ws2 [h,F] (shared expert, if any), logit_bias [E] fp32 or
    None, select_bias [E] fp32 or None.  Weights are stored [out, in].
    """
    s, dt = cfg.seed, cfg.dtype
    T, h, E, F = cfg.T, cfg.h, cfg.E, cfg.F
    inp = {
        "x": normal((T, h), 1.0, s, "x", device, dt),
        "w_router": normal((E, h), 1.0 / math.sqrt(h), s, "w_router", device, dt),
        "logit_bias": per_expert_bias(cfg.logit_bias, E, s, "logit_bias", device),
        "select_bias": per_expert_bias(cfg.select_bias, E, s, "select_bias", device),
        "w1": None, "w3": None, "w2": None, "ws1": None, "ws3": None, "ws2": None,
    }
    if with_experts:
        inp["w1"] = stacked_normal(E, (F, h), 1.0 / math.sqrt(h), s, "w1", device, dt)
        inp["w3"] = stacked_normal(E, (F, h), 1.0 / math.sqrt(h), s, "w3", device, dt)
        inp["w2"] = stacked_normal(E, (h, F), 1.0 / math.sqrt(F), s, "w2", device, dt)
        if cfg.shared:
            inp["ws1"] = normal((F, h), 1.0 / math.sqrt(h), s, "ws1", device, dt)
            inp["ws3"] = normal((F, h), 1.0 / math.sqrt(h), s, "ws3", device, dt)
            inp["ws2"] = normal((h, F), 1.0 / math.sqrt(F), s, "ws2", device, dt)
    return inp
