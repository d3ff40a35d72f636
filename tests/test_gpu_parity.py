"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars (written in each check):
* routing on the GPU's own fp32 keys: bit-exact for every token;
* routing vs the oracle's logits: identical expert sets except on tokens whose
  k-th / (k+1)-th key gap is below 1e-5, where the GPU choice must be valid;
* gates within 2e-6 of the oracle's fp64 gates from the same logits;
* counts, offsets, assign_row, row_token, drops: bit-exact;
* x_perm: bit-exact copies, padding rows exactly zero;
* y: max|y_gpu - y_ref| / max|y_ref| <= 2e-2 (bf16), <= 1e-5 (fp32), over all
  compared rows and for every token on its own (max over the token's
  elements of |y_gpu - y_ref| over the max of its |y_ref|);
* a token whose every slot was dropped: exactly zero without a shared expert,
  bit-equal to the shared expert's own output with one.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_25_amd as moe
import oracle
from helpers import (DEV, LazyExperts, capacity_of, check_outputs, check_routing, gen_inputs,
                     lib_cfg, np32, oracle_forward, oracle_weights, rel_err, run_forward, tol_of)
from moe_inputs import CONFIGS, MoEConfig, normal

pytestmark = pytest.mark.gpu

# Sizes the oracle finishes in seconds that still span several GEMM tiles
# (256-row and 256/128-column tiles, 64-deep K steps) with ragged tails.
MEDIUM = [
    CONFIGS["tiny_fp32"],
    MoEConfig("dropless_softmax", T=1000, h=512, E=4, k=2, F=640, gate="softmax_topk"),
    MoEConfig("capacity_heavy_drop", T=1000, h=384, E=8, k=2, F=384,
              gate="softmax_all_topk", cf=(1, 2)),
    MoEConfig("worked_example_small", T=512, h=256, E=8, k=2, F=384,
              gate="softmax_all_topk", cf=(5, 4)),
    MoEConfig("sigmoid_bias_shared", T=700, h=256, E=16, k=4, F=256,
              gate="sigmoid_topk_norm", select_bias=("normal", 0.1), shared=True),
    MoEConfig("zipf_dropless", T=2048, h=256, E=64, k=4, F=128,
              logit_bias=("zipf", 1.2)),
    MoEConfig("zipf_cf1", T=2048, h=256, E=64, k=4, F=128,
              logit_bias=("zipf", 1.2), cf=(1, 1)),
    MoEConfig("e256_k8_shared", T=300, h=256, E=256, k=8, F=128,
              gate="sigmoid_topk_norm", select_bias=("normal", 0.1), shared=True),
    MoEConfig("mixtral_bias", T=777, h=256, E=8, k=2, F=384, logit_bias=("normal", 0.5)),
    MoEConfig("e1_k1_dense", T=333, h=256, E=1, k=1, F=256),
    MoEConfig("k_equals_e", T=257, h=128, E=4, k=4, F=128),
    MoEConfig("one_token", T=1, h=128, E=8, k=2, F=128, cf=(5, 4)),
    MoEConfig("e1024_k16", T=70, h=128, E=1024, k=16, F=128, gate="softmax_all_topk"),
    # expert count that fills neither a 16- nor a 64-expert router tile, h an
    # odd multiple of 128 (router K loop tail)
    MoEConfig("e40_ragged", T=333, h=384, E=40, k=3, F=256, gate="softmax_all_topk",
              cf=(3, 2)),
    # 17..32 and 33..64 experts: the fused router tile with 4 waves (h an
    # odd multiple of 128) and with 8 (h a multiple of 256), two or four
    # experts per top-k lane
    MoEConfig("e24_sigmoid_bias", T=517, h=384, E=24, k=3, F=256, gate="sigmoid_topk_norm",
              select_bias=("normal", 0.1), cf=(5, 4)),
    MoEConfig("e20_wide", T=300, h=512, E=20, k=2, F=256, gate="softmax_all_topk", cf=(1, 1)),
    # 65..128 experts: the top-k kernel's 16-lane segments of 8 experts
    MoEConfig("e100_k6", T=400, h=256, E=100, k=6, F=128, gate="softmax_topk"),
    # the bf16 backward reads w2 through a transposed copy past 512 dispatch
    # rows per expert and [w1; w3] past 1536 (with fewer, K-major): 600 rows
    # per expert transpose w2 only, 1600 both
    MoEConfig("bwd_many_rows", T=1200, h=256, E=4, k=2, F=384, gate="sigmoid_topk_norm",
              shared=True),
    MoEConfig("bwd_more_rows", T=1600, h=256, E=2, k=2, F=256, gate="softmax_topk",
              shared=True),
    # few rows per expert and at most 256 tokens: every weight gradient,
    # the shared expert's too, on the 128x128 small-K tiles
    MoEConfig("bwd_few_rows_shared", T=200, h=384, E=8, k=2, F=256, gate="sigmoid_topk_norm",
              shared=True),
    # K long enough (>= 16 slices of 64) that the tiles of the last partial
    # round are split along K and reduced (GEMM 1 and GEMM 2)
    MoEConfig("split_k_tail", T=600, h=1024, E=4, k=2, F=1024, gate="softmax_topk"),
    MoEConfig("split_k_tail_capacity_shared", T=500, h=1024, E=4, k=2, F=1024,
              gate="sigmoid_topk_norm", cf=(1, 1), shared=True),
    MoEConfig("f32_capacity", T=300, h=256, E=8, k=2, F=256, dtype="f32",
              gate="softmax_all_topk", cf=(1, 1)),
    MoEConfig("f32_sigmoid_shared", T=200, h=128, E=16, k=4, F=256, dtype="f32",
              gate="sigmoid_topk_norm", select_bias=("normal", 0.1), shared=True),
    # capacity a quarter of the even share: most tokens lose every slot and
    # keep only the shared expert's output
    MoEConfig("drop_all_shared", T=600, h=256, E=8, k=2, F=256, gate="softmax_topk",
              cf=(1, 4), shared=True),
]


def _report(name, **kw):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


@pytest.mark.parametrize("cfg", MEDIUM, ids=lambda c: c.name)
def test_forward_matches_oracle(cfg):
    print(f"[case] forward {cfg.name} T={cfg.T} h={cfg.h} E={cfg.E} k={cfg.k} "
          f"F={cfg.F} {cfg.dtype} {cfg.gate} cf={cfg.cf}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib)
    ref = oracle_forward(cfg, inp, C_ref, maps_only=True)
    rep = check_routing(cfg, gpu, ref, C_ref, inp)
    g_idx = gpu["topk_idx"].cpu().numpy()
    ref_y = oracle_forward(cfg, inp, C_ref, idx=g_idx)["y"]
    y = np32(gpu["y"])
    assert np.isfinite(y).all()
    out = check_outputs(cfg, y, ref_y, cfg.name)
    _report(cfg.name, **out, **rep)


# ------------------------------------------------------------------ backward
# e1024_k16: more than 256 experts (the gates backward's per-thread kernel);
# drop_all_shared: most slots dropped, dx mostly the shared expert's rows
BACKWARD = ["dropless_softmax", "capacity_heavy_drop", "worked_example_small",
            "sigmoid_bias_shared", "zipf_dropless", "split_k_tail", "e40_ragged",
            "mixtral_bias", "e256_k8_shared", "k_equals_e", "bwd_many_rows",
            "bwd_more_rows", "bwd_few_rows_shared", "e1024_k16", "drop_all_shared",
            "tiny_fp32", "f32_capacity", "f32_sigmoid_shared"]


def run_backward(cfg, inp, C_lib, gpu, dy, routing="topk", saved=False):
    """moe_backward on the forward's routing outputs; saved: the forward ran
    with save_for_backward and moe_backward_saved reads its workspace."""
    return _backward_with_cfg(cfg, lib_cfg(cfg, C_lib, routing, saved), inp, gpu, dy,
                              routing, saved)


def _backward_with_cfg(cfg, c, inp, gpu, dy, routing="topk", saved=False):
    T, E, k, h, F = cfg.T, cfg.E, cfg.k, cfg.h, cfg.F
    slots = E if routing == "expert_choice" else k
    bf = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def nan(*shape, dtype=bf):
        return torch.full(shape, float("nan"), dtype=dtype, device=DEV)

    grads = {"dx": nan(T, h), "dw_router": nan(E, h), "dlogit_bias": nan(E, dtype=torch.float32),
             "dw1": nan(E, F, h), "dw3": nan(E, F, h), "dw2": nan(E, h, F),
             "dgate": nan(T, slots, dtype=torch.float32)}
    if cfg.shared:
        grads.update({"dws1": nan(F, h), "dws3": nan(F, h), "dws2": nan(h, F)})
    ws = torch.empty(moe.moe_backward_workspace_bytes(c), dtype=torch.uint8, device=DEV)
    weights = {n: inp[n] for n in ("w_router", "w1", "w3", "w2", "logit_bias", "select_bias",
                                   "ws1", "ws3", "ws2")}
    route = {n: gpu[n] for n in ("logits", "topk_idx", "topk_gate", "expert_counts",
                                 "expert_offsets", "assign_row")}
    if saved:
        moe.moe_backward_saved(c, weights, inp["x"], dy, route, gpu["ws"], grads, ws)
    else:
        moe.moe_backward(c, weights, inp["x"], dy, route, grads, ws)
    torch.cuda.synchronize()
    return grads


@pytest.mark.parametrize("name", BACKWARD)
def test_backward_matches_oracle(name):
    """Every gradient of sum(y * dy) against the oracle's chain rule on the
    GPU's own routing (top-k choice and drops held fixed); normwise max
    relative error within 2e-2 (bf16 tensors) or 1e-5 (fp32)."""
    cfg = next(c for c in MEDIUM if c.name == name)
    print(f"[case] backward {name}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib)
    dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=DEV, dtype=cfg.dtype)
    g = run_backward(cfg, inp, C_lib, gpu, dy)
    x, wr, w1, w3, w2, lb, shared = oracle_weights(cfg, inp)
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    ref = oracle.moe_backward(x, wr, w1, w3, w2, np32(dy), k=cfg.k, gate=cfg.gate, C=C_ref,
                              logit_bias=lb, select_bias=sb, shared=shared,
                              idx=gpu["topk_idx"].cpu().numpy())
    _check_grads(cfg, g, ref, f"backward_{name}")


def _check_grads(cfg, g, ref, label):
    """Every gradient the library wrote against the oracle's, normwise."""
    names = ["dx", "dw1", "dw3", "dw2", "dw_router", "dlogit_bias", "dgate"]
    if cfg.shared:
        names += ["dws1", "dws3", "dws2"]
    errs = {}
    for n in names:
        r = ref[n]
        if np.abs(r).max() == 0:
            assert float(np.abs(np32(g[n])).max()) == 0.0, n
            errs[n] = 0.0
            continue
        errs[n] = rel_err(np32(g[n]), r)
    _report(label, **{kk: f"{v:.2e}" for kk, v in errs.items()})
    for kk, v in errs.items():
        assert v <= tol_of(cfg), (kk, v)


def test_backward_is_deterministic():
    cfg = next(c for c in MEDIUM if c.name == "sigmoid_bias_shared")
    inp = gen_inputs(cfg)
    C_lib, _ = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib)
    dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=DEV)
    a = run_backward(cfg, inp, C_lib, gpu, dy)
    b = run_backward(cfg, inp, C_lib, gpu, dy)
    for key in a:
        assert torch.equal(a[key].view(torch.int16) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.int16) if b[key].dtype == torch.bfloat16 else b[key]), key


SAVED = ["worked_example_small", "sigmoid_bias_shared", "capacity_heavy_drop", "split_k_tail",
         "zipf_dropless", "e40_ragged", "bwd_many_rows", "bwd_more_rows", "bwd_few_rows_shared",
         "tiny_fp32",
         "f32_sigmoid_shared"]


@pytest.mark.parametrize("name", SAVED)
def test_backward_saved_matches_oracle(name):
    """Forward with save_for_backward (same output bits as without), then
    the backward from its kept activations: every gradient against the
    oracle's chain rule on the GPU's routing."""
    cfg = next(c for c in MEDIUM if c.name == name)
    print(f"[case] saved backward {name}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    plain = run_forward(cfg, inp, C_lib)
    gpu = run_forward(cfg, inp, C_lib, save=True)
    y0, y1 = plain["y"], gpu["y"]
    if y0.dtype == torch.bfloat16:
        y0, y1 = y0.view(torch.int16), y1.view(torch.int16)
    assert torch.equal(y0, y1), "the flag changed the layer output"
    dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=DEV, dtype=cfg.dtype)
    g = run_backward(cfg, inp, C_lib, gpu, dy, saved=True)
    x, wr, w1, w3, w2, lb, shared = oracle_weights(cfg, inp)
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    ref = oracle.moe_backward(x, wr, w1, w3, w2, np32(dy), k=cfg.k, gate=cfg.gate, C=C_ref,
                              logit_bias=lb, select_bias=sb, shared=shared,
                              idx=gpu["topk_idx"].cpu().numpy())
    _check_grads(cfg, g, ref, f"saved_backward_{name}")


@pytest.mark.parametrize("name", ["ec_sigmoid_shared", "ec_e40_ragged_f32"])
def test_expert_choice_backward_saved_matches_oracle(name):
    cfg = next(c for c in EXPERT_CHOICE if c.name == name)
    print(f"[case] expert choice saved backward {name}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib, routing="expert_choice", save=True)
    dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=DEV, dtype=cfg.dtype)
    g = run_backward(cfg, inp, C_lib, gpu, dy, routing="expert_choice", saved=True)
    x, wr, w1, w3, w2, lb, shared = oracle_weights(cfg, inp)
    ref = oracle.expert_choice_backward(x, wr, w1, w3, w2, np32(dy), C=C_ref, gate=cfg.gate,
                                        logit_bias=lb, shared=shared,
                                        scores=gpu["probs"].cpu().numpy().T)
    _check_grads(cfg, g, ref, f"expert_choice_saved_backward_{name}")


@pytest.mark.parametrize("name,routing,iters", [
    ("sigmoid_bias_shared", "topk", 0), ("mixtral_bias", "topk", 0), ("tiny_fp32", "topk", 0),
    ("mixtral_bias", "sinkhorn", 6), ("capacity_heavy_drop", "topk_score_drop", 0),
    ("ec_sigmoid_shared", "expert_choice", 0)])
def test_autograd_layer_matches_oracle(name, routing, iters):
    """The torch.autograd wrapper under each routing: its output is
    moe_forward's bit for bit, and the leaves' gradients of sum(y * dy) meet
    the oracle's bound (the routing held fixed as the forward chose it)."""
    from mixture_experts_layer_25_amd.autograd import moe_layer
    cfg = next(c for c in MEDIUM + EXPERT_CHOICE if c.name == name)
    print(f"[case] autograd layer {name} {routing}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib, routing=routing, sinkhorn_iters=iters)
    leaf = {n: inp[n].clone().requires_grad_(True) for n in ("x", "w_router", "w1", "w3", "w2")}
    lb = None if inp["logit_bias"] is None else inp["logit_bias"].clone().requires_grad_(True)
    sh = (tuple(inp[n].clone().requires_grad_(True) for n in ("ws1", "ws3", "ws2"))
          if cfg.shared else None)
    y = moe_layer(leaf["x"], leaf["w_router"], leaf["w1"], leaf["w3"], leaf["w2"], k=cfg.k,
                  gate=cfg.gate, capacity=C_lib, routing=routing, sinkhorn_iters=iters,
                  logit_bias=lb, select_bias=inp["select_bias"], shared=sh)
    y0, y1 = gpu["y"], y.detach()
    if y0.dtype == torch.bfloat16:
        y0, y1 = y0.view(torch.int16), y1.view(torch.int16)
    assert torch.equal(y0, y1)
    dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=DEV, dtype=cfg.dtype)
    (y.float() * dy.float()).sum().backward()
    torch.cuda.synchronize()
    x, wr, w1, w3, w2, lbn, shared = oracle_weights(cfg, inp)
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    if routing == "expert_choice":
        ref = oracle.expert_choice_backward(x, wr, w1, w3, w2, np32(dy), C=C_ref, gate=cfg.gate,
                                            logit_bias=lbn, shared=shared,
                                            scores=gpu["probs"].cpu().numpy().T)
    else:
        kw = ({"drop": "score", "priority": gpu["topk_gate"].cpu().numpy()}
              if routing == "topk_score_drop" else {})
        ref = oracle.moe_backward(x, wr, w1, w3, w2, np32(dy), k=cfg.k, gate=cfg.gate, C=C_ref,
                                  logit_bias=lbn, select_bias=sb, shared=shared,
                                  idx=gpu["topk_idx"].cpu().numpy(), **kw)
    got = {"dx": leaf["x"].grad, "dw_router": leaf["w_router"].grad, "dw1": leaf["w1"].grad,
           "dw3": leaf["w3"].grad, "dw2": leaf["w2"].grad}
    if lb is not None:
        got["dlogit_bias"] = lb.grad
    if sh is not None:
        got.update({"dws1": sh[0].grad, "dws3": sh[1].grad, "dws2": sh[2].grad})
    errs = {n: rel_err(np32(t), ref[n]) for n, t in got.items()}
    _report(f"autograd_{name}_{routing}", **{n: f"{v:.2e}" for n, v in errs.items()})
    for n, v in errs.items():
        assert v <= tol_of(cfg), (n, v)


def _random_configs(n=16, seed=2024):
    """Seeded draws over every axis of the layer (shape, gate, biases,
    capacity, shared expert, dtype), small enough for the oracle."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 24, 40, 64]))
        k = int(rng.integers(1, min(E, 8) + 1))
        gate = str(rng.choice(["softmax_topk", "softmax_all_topk", "sigmoid_topk_norm"]))
        cf = [None, (1, 2), (1, 1), (5, 4), (3, 1)][int(rng.integers(0, 5))]
        out.append(MoEConfig(
            f"rand{i}", T=int(rng.integers(1, 600)), h=int(rng.choice([128, 256, 384, 512])),
            E=E, k=k, F=int(rng.choice([128, 256, 384])),
            dtype="f32" if rng.random() < 0.2 else "bf16", gate=gate, cf=cf,
            shared=bool(rng.random() < 0.3),
            logit_bias=("normal", 0.5) if rng.random() < 0.3 else None,
            select_bias=("normal", 0.1) if gate == "sigmoid_topk_norm" and rng.random() < 0.5
            else None,
            seed=int(rng.integers(0, 1000))))
    return out


@pytest.mark.parametrize("cfg", _random_configs(), ids=lambda c: c.name)
def test_random_configs_forward_and_backward(cfg):
    """Forward (routing checks and output) and backward (every gradient)
    against the oracle on seeded random layers."""
    print(f"[case] random {cfg}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib)
    ref = oracle_forward(cfg, inp, C_ref, maps_only=True)
    rep = check_routing(cfg, gpu, ref, C_ref, inp)
    ref_y = oracle_forward(cfg, inp, C_ref, idx=gpu["topk_idx"].cpu().numpy())["y"]
    y = np32(gpu["y"])
    assert np.isfinite(y).all()
    err = check_outputs(cfg, y, ref_y, cfg.name)["token_rel_err"]
    dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=DEV, dtype=cfg.dtype)
    g = run_backward(cfg, inp, C_lib, gpu, dy)
    x, wr, w1, w3, w2, lb, shared = oracle_weights(cfg, inp)
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    refb = oracle.moe_backward(x, wr, w1, w3, w2, np32(dy), k=cfg.k, gate=cfg.gate, C=C_ref,
                               logit_bias=lb, select_bias=sb, shared=shared,
                               idx=gpu["topk_idx"].cpu().numpy())
    if lb is None:
        g.pop("dlogit_bias", None)
        refb.pop("dlogit_bias", None)
    names = [n for n in ("dx", "dw1", "dw3", "dw2", "dw_router", "dlogit_bias", "dgate",
                         "dws1", "dws3", "dws2") if n in g and n in refb]
    errs = {}
    for n in names:
        r = refb[n]
        errs[n] = (float(np.abs(np32(g[n])).max()) if np.abs(r).max() == 0
                   else rel_err(np32(g[n]), r))
    _report(cfg.name, fwd=err, **{n: f"{v:.2e}" for n, v in errs.items()}, **rep)
    for n, v in errs.items():
        assert v <= tol_of(cfg), (n, v)


# ------------------------------------------------------------ routing variants
SCORE_DROP = ["capacity_heavy_drop", "zipf_cf1", "worked_example_small",
              "split_k_tail_capacity_shared", "f32_capacity", "e24_sigmoid_bias"]


@pytest.mark.parametrize("name", SCORE_DROP)
def test_score_drop_matches_oracle(name):
    """Capacity drop by gate score: maps bit-exact against the oracle's
    score-priority maps decided on the GPU's own gates; every output row
    against the oracle's layer with those maps."""
    cfg = next(c for c in MEDIUM if c.name == name)
    print(f"[case] score drop {name}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib, routing="topk_score_drop")
    g_idx = gpu["topk_idx"].cpu().numpy()
    g_gate = gpu["topk_gate"].cpu().numpy()
    ref = oracle_forward(cfg, inp, C_ref, idx=g_idx, drop="score", priority=g_gate)
    rep = check_routing(cfg, gpu, ref, C_ref, inp, drop="score")
    token_order = oracle.route_maps(g_idx, cfg.E, C_ref)["assign_row"]
    changed = int((token_order != ref["maps"]["assign_row"]).sum())
    out = check_outputs(cfg, np32(gpu["y"]), ref["y"], f"score_drop_{name}")
    _report(f"score_drop_{name}", rows_moved=changed, **out, **rep)


def test_score_drop_with_equal_gates_is_token_order():
    """k = 1 with softmax over the selected expert: every gate is 1.0, so the
    score-priority drop keeps exactly the token-order assignments."""
    cfg = MoEConfig("k1_capacity", T=500, h=256, E=8, k=1, F=256, gate="softmax_topk",
                    cf=(1, 2))
    inp = gen_inputs(cfg)
    C_lib, _ = capacity_of(cfg)
    a = run_forward(cfg, inp, C_lib, routing="topk_score_drop")
    b = run_forward(cfg, inp, C_lib, routing="topk")
    for key in ("assign_row", "row_token", "expert_counts", "expert_offsets"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(a["y"].view(torch.int16), b["y"].view(torch.int16))


EXPERT_CHOICE = [
    MoEConfig("ec_softmax", T=1000, h=256, E=8, k=2, F=256, gate="softmax_topk", cf=(1, 1)),
    MoEConfig("ec_sigmoid_shared", T=700, h=256, E=16, k=4, F=256, gate="sigmoid_topk_norm",
              shared=True, cf=(1, 1)),
    MoEConfig("ec_e256", T=300, h=256, E=256, k=8, F=128, gate="softmax_all_topk", cf=(1, 1)),
    MoEConfig("ec_e40_ragged_f32", T=333, h=128, E=40, k=3, F=128, dtype="f32",
              gate="softmax_topk", cf=(1, 1)),
    MoEConfig("ec_all_tokens", T=200, h=128, E=4, k=4, F=128, gate="softmax_all_topk",
              cf=(1, 1)),
    MoEConfig("ec_zipf", T=2048, h=256, E=64, k=4, F=128, logit_bias=("zipf", 1.2), cf=(1, 1)),
]


@pytest.mark.parametrize("cfg", EXPERT_CHOICE, ids=lambda c: c.name)
def test_expert_choice_matches_oracle(cfg):
    """Expert-choice routing: probabilities against the oracle's on the GPU's
    logits; selection, rows and gates bit-exact against the oracle deciding on
    the GPU's own probabilities; the layer output against the oracle's."""
    print(f"[case] expert choice {cfg.name}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    assert 0 < C_lib <= cfg.T
    gpu = run_forward(cfg, inp, C_lib, routing="expert_choice")
    T, E = cfg.T, cfg.E
    g_logits = gpu["logits"].cpu().numpy()
    scores = gpu["probs"].cpu().numpy().T          # [T,E]
    dp = float(np.abs(scores - oracle.router_probs(g_logits, cfg.gate)).max())
    assert dp <= 1e-6, dp
    m = oracle.expert_choice(g_logits, C_ref, cfg.gate, scores=scores)
    np.testing.assert_array_equal(gpu["assign_row"].cpu().numpy().reshape(T, E), m["sel_row"])
    np.testing.assert_array_equal(gpu["topk_gate"].cpu().numpy(), m["gate"])
    np.testing.assert_array_equal(gpu["row_token"].cpu().numpy(), m["row_token"])
    np.testing.assert_array_equal(gpu["expert_counts"].cpu().numpy(), m["counts"])
    np.testing.assert_array_equal(gpu["expert_offsets"].cpu().numpy(), m["offsets"])
    x, wr, w1, w3, w2, lb, shared = oracle_weights(cfg, inp)
    ref = oracle.expert_choice_forward(x, wr, w1, w3, w2, C=C_ref, gate=cfg.gate, logit_bias=lb,
                                       shared=shared, scores=scores)
    out = check_outputs(cfg, np32(gpu["y"]), ref["y"], f"expert_choice_{cfg.name}")
    per_token = (m["sel_row"] >= 0).sum(1)
    _report(f"expert_choice_{cfg.name}", max_dprob=f"{dp:.1e}", C=C_lib,
            unrouted_tokens=int((per_token == 0).sum()), max_experts_per_token=int(per_token.max()),
            **out)


@pytest.mark.parametrize("cfg", EXPERT_CHOICE, ids=lambda c: c.name)
def test_expert_choice_backward_matches_oracle(cfg):
    """Backward with expert-choice routing: every gradient against the
    oracle's chain rule with the experts' choices held fixed (decided on the
    GPU's own probabilities)."""
    print(f"[case] expert choice backward {cfg.name}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib, routing="expert_choice")
    dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=DEV, dtype=cfg.dtype)
    g = run_backward(cfg, inp, C_lib, gpu, dy, routing="expert_choice")
    x, wr, w1, w3, w2, lb, shared = oracle_weights(cfg, inp)
    ref = oracle.expert_choice_backward(x, wr, w1, w3, w2, np32(dy), C=C_ref, gate=cfg.gate,
                                        logit_bias=lb, shared=shared,
                                        scores=gpu["probs"].cpu().numpy().T)
    _check_grads(cfg, g, ref, f"expert_choice_backward_{cfg.name}")


# Sinkhorn routing: (config, iterations).  Covers one- to 16-entry lanes
# (E = 8 .. 1024), one token, fp32, capacity drops and an uneven router.
SINKHORN = [("zipf_dropless", 8), ("zipf_cf1", 30), ("worked_example_small", 5),
            ("mixtral_bias", 1), ("e1024_k16", 3), ("e40_ragged", 4), ("tiny_fp32", 10),
            ("f32_capacity", 6), ("one_token", 3), ("k_equals_e", 2)]
# |bias_gpu - bias_oracle| on the same logits: fp32 log-sum-exp over at most
# T terms per column against fp64; keys near-tied within twice that (plus the
# logits' own rounding) may select either way.
SK_BIAS_TOL = 5e-5
SK_TIE = 2 * SK_BIAS_TOL + 1e-5


def _sinkhorn_case(cfg, iters, C_lib, C_ref):
    inp = gen_inputs(cfg)
    gpu = run_forward(cfg, inp, C_lib, routing="sinkhorn", sinkhorn_iters=iters)
    sk = oracle.sinkhorn(gpu["logits"].cpu().numpy(), iters)
    db = float(np.abs(gpu["route_bias"].cpu().numpy().astype(np.float64) -
                      np.log(sk["col"])).max())
    ref = oracle_forward(cfg, inp, C_ref, maps_only=True, sinkhorn_iters=iters)
    rep = check_routing(cfg, gpu, ref, C_ref, inp, tie=SK_TIE)
    return inp, gpu, ref, db, rep


@pytest.mark.parametrize("name,iters", SINKHORN)
def test_sinkhorn_matches_oracle(name, iters):
    """Sinkhorn routing: the GPU's selection bias within SK_BIAS_TOL of the
    oracle's balancing of the same logits; selection bit-exact on the GPU's
    own keys and equal to the oracle's off near-ties; maps bit-exact; every
    output row against the oracle's layer on the GPU's selection."""
    cfg = next(c for c in MEDIUM if c.name == name)
    print(f"[case] sinkhorn {name} iters={iters}", flush=True)
    C_lib, C_ref = capacity_of(cfg)
    inp, gpu, ref, db, rep = _sinkhorn_case(cfg, iters, C_lib, C_ref)
    ref_y = oracle_forward(cfg, inp, C_ref, idx=gpu["topk_idx"].cpu().numpy())["y"]
    out = check_outputs(cfg, np32(gpu["y"]), ref_y, f"sinkhorn_{name}")
    counts = gpu["expert_counts"].cpu().numpy()
    _report(f"sinkhorn_{name}", bias_err=f"{db:.1e}",
            max_over_mean=f"{counts.max() / counts.mean():.2f}", **out, **rep)
    assert db <= SK_BIAS_TOL


def test_sinkhorn_evens_out_zipf_load():
    """With the Zipf-biased router the hottest expert gets several times the
    mean under plain top-k; 30 Sinkhorn iterations bring every load within
    25 % of the mean (the balancing the routing exists for)."""
    cfg = next(c for c in MEDIUM if c.name == "zipf_dropless")
    inp = gen_inputs(cfg)
    plain = run_forward(cfg, inp, 0)["expert_counts"].cpu().numpy()
    bal = run_forward(cfg, inp, 0, routing="sinkhorn",
                      sinkhorn_iters=30)["expert_counts"].cpu().numpy()
    mean = cfg.T * cfg.k / cfg.E
    _report("sinkhorn_balance", plain_max=int(plain.max()), sinkhorn_max=int(bal.max()),
            sinkhorn_min=int(bal.min()), mean=mean)
    assert plain.max() > 3 * mean
    assert 0.75 * mean < bal.min() and bal.max() < 1.25 * mean


@pytest.mark.parametrize("name,iters", [("zipf_cf1", 10), ("tiny_fp32", 4)])
def test_sinkhorn_backward_matches_oracle(name, iters):
    """The backward with the Sinkhorn selection held fixed equals the top-k
    backward on that selection (the bias only chose the experts)."""
    cfg = next(c for c in MEDIUM if c.name == name)
    print(f"[case] sinkhorn backward {name}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib, routing="sinkhorn", sinkhorn_iters=iters)
    dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=DEV, dtype=cfg.dtype)
    c = lib_cfg(cfg, C_lib, "sinkhorn", sinkhorn_iters=iters)
    g = _backward_with_cfg(cfg, c, inp, gpu, dy)
    x, wr, w1, w3, w2, lb, shared = oracle_weights(cfg, inp)
    ref = oracle.moe_backward(x, wr, w1, w3, w2, np32(dy), k=cfg.k, gate=cfg.gate, C=C_ref,
                              logit_bias=lb, shared=shared, idx=gpu["topk_idx"].cpu().numpy())
    _check_grads(cfg, g, ref, f"sinkhorn_backward_{name}")


def test_sinkhorn_full_size_skewed_routing():
    """Sinkhorn routing on the skewed workload's full router (T=16384, E=64,
    k=4, 256 blocks of 64 tokens): bias, selection and maps as above, and the
    load evened out."""
    cfg = CONFIGS["skewed"]
    print("[case] sinkhorn full skewed", flush=True)
    torch.cuda.empty_cache()
    inp, gpu, ref, db, rep = _sinkhorn_case(cfg, 10, 0, None)
    counts = gpu["expert_counts"].cpu().numpy()
    _report("sinkhorn_full_skewed", bias_err=f"{db:.1e}",
            max_over_mean=f"{counts.max() / counts.mean():.2f}", **rep)
    assert db <= SK_BIAS_TOL
    assert counts.max() < 1.25 * counts.mean()
    del gpu, inp
    torch.cuda.empty_cache()


def _random_variant_cases(n=12, seed=4096):
    """Seeded (layer, routing, Sinkhorn iterations) draws for the three
    routing variants: score drop, expert choice and Sinkhorn."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        routing = ("topk_score_drop", "expert_choice", "sinkhorn")[i % 3]
        E = int(rng.choice([2, 3, 5, 8, 13, 16, 24, 40, 64, 100]))
        k = int(rng.integers(1, min(E, 8) + 1))
        gate = str(rng.choice(["softmax_topk", "softmax_all_topk", "sigmoid_topk_norm"]))
        cf = [(1, 2), (1, 1), (5, 4)][int(rng.integers(0, 3))]
        if routing == "sinkhorn" and rng.random() < 0.5:
            cf = None
        cfg = MoEConfig(
            f"rv{i}_{routing}", T=int(rng.integers(2, 500)), h=int(rng.choice([128, 256, 384])),
            E=E, k=k, F=int(rng.choice([128, 256])),
            dtype="f32" if rng.random() < 0.25 else "bf16", gate=gate, cf=cf,
            shared=bool(rng.random() < 0.3),
            logit_bias=("normal", 0.5) if rng.random() < 0.4 else None,
            select_bias=("normal", 0.1) if routing == "topk_score_drop" and rng.random() < 0.5
            else None,
            seed=int(rng.integers(0, 1000)))
        out.append((cfg, routing, int(rng.integers(1, 25)) if routing == "sinkhorn" else 0))
    return out


@pytest.mark.parametrize("case", _random_variant_cases(), ids=lambda c: c[0].name)
def test_random_routing_variants_forward_and_backward(case):
    """Seeded random layers under each routing variant: routing checked as
    in the variant's own test, the output and every gradient against the
    oracle with that routing held fixed."""
    cfg, routing, iters = case
    print(f"[case] random variant {cfg} iters={iters}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    T, E = cfg.T, cfg.E
    if routing == "expert_choice":
        C_lib, C_ref = min(C_lib, T), min(C_ref, T)
    gpu = run_forward(cfg, inp, C_lib, routing=routing, sinkhorn_iters=iters)
    x, wr, w1, w3, w2, lb, shared = oracle_weights(cfg, inp)
    dy = normal((T, cfg.h), 1.0, cfg.seed, "dy", device=DEV, dtype=cfg.dtype)
    c = lib_cfg(cfg, C_lib, routing, sinkhorn_iters=iters)
    g = _backward_with_cfg(cfg, c, inp, gpu, dy, routing)
    if routing == "expert_choice":
        scores = gpu["probs"].cpu().numpy().T
        m = oracle.expert_choice(gpu["logits"].cpu().numpy(), C_ref, cfg.gate, scores=scores)
        np.testing.assert_array_equal(gpu["assign_row"].cpu().numpy().reshape(T, E), m["sel_row"])
        np.testing.assert_array_equal(gpu["row_token"].cpu().numpy(), m["row_token"])
        ref_y = oracle.expert_choice_forward(x, wr, w1, w3, w2, C=C_ref, gate=cfg.gate,
                                             logit_bias=lb, shared=shared, scores=scores)["y"]
        refb = oracle.expert_choice_backward(x, wr, w1, w3, w2, np32(dy), C=C_ref, gate=cfg.gate,
                                             logit_bias=lb, shared=shared, scores=scores)
        rep = {}
    else:
        g_idx = gpu["topk_idx"].cpu().numpy()
        sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
        if routing == "sinkhorn":
            ref = oracle_forward(cfg, inp, C_ref, maps_only=True, sinkhorn_iters=iters)
            rep = check_routing(cfg, gpu, ref, C_ref, inp, tie=SK_TIE)
            kw = {}
        else:
            g_gate = gpu["topk_gate"].cpu().numpy()
            ref = oracle_forward(cfg, inp, C_ref, idx=g_idx, drop="score", priority=g_gate,
                                 maps_only=True)
            rep = check_routing(cfg, gpu, ref, C_ref, inp, drop="score")
            kw = {"drop": "score", "priority": g_gate}
        ref_y = oracle_forward(cfg, inp, C_ref, idx=g_idx, **kw)["y"]
        refb = oracle.moe_backward(x, wr, w1, w3, w2, np32(dy), k=cfg.k, gate=cfg.gate,
                                   C=C_ref, logit_bias=lb, select_bias=sb, shared=shared,
                                   idx=g_idx, **kw)
    y = np32(gpu["y"])
    assert np.isfinite(y).all()
    err = check_outputs(cfg, y, ref_y, cfg.name)["token_rel_err"]
    if lb is None:
        g.pop("dlogit_bias", None)
        refb.pop("dlogit_bias", None)
    errs = {}
    for n in ("dx", "dw1", "dw3", "dw2", "dw_router", "dlogit_bias", "dgate", "dws1", "dws3",
              "dws2"):
        if n in g and n in refb:
            r = refb[n]
            errs[n] = (float(np.abs(np32(g[n])).max()) if np.abs(r).max() == 0
                       else rel_err(np32(g[n]), r))
    _report(cfg.name, fwd=err, **{n: f"{v:.2e}" for n, v in errs.items()}, **rep)
    for n, v in errs.items():
        assert v <= tol_of(cfg), (n, v)


BALANCE = ["worked_example_small", "sigmoid_bias_shared", "zipf_dropless", "e256_k8_shared",
           "e1024_k16", "one_token", "e40_ragged", "k_equals_e", "f32_capacity"]


@pytest.mark.parametrize("name", BALANCE)
def test_load_balance_matches_oracle(name):
    """f, P and the Switch loss of the GPU's own routing (its logits and
    counts) against the oracle on the same values; a second call gives the
    same bits."""
    cfg = next(c for c in MEDIUM if c.name == name)
    print(f"[case] load balance {name}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, _ = capacity_of(cfg)
    out = run_forward(cfg, inp, C_lib)
    c = lib_cfg(cfg, C_lib)
    alpha = 0.01
    res = []
    for _ in range(2):
        f = torch.full((cfg.E,), float("nan"), dtype=torch.float32, device=DEV)
        P = torch.full((cfg.E,), float("nan"), dtype=torch.float32, device=DEV)
        loss = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
        moe.moe_load_balance(c, out["logits"], out["expert_counts"], alpha, f, P, loss, out["ws"])
        torch.cuda.synchronize()
        res.append((f.cpu().numpy(), P.cpu().numpy(), float(loss.item())))
    (f, P, loss), (f2, P2, loss2) = res
    assert np.array_equal(f, f2) and np.array_equal(P, P2) and loss == loss2
    ref = oracle.load_balance(np32(out["logits"]), out["expert_counts"].cpu().numpy(), cfg.k,
                              cfg.gate, alpha)
    # f: the same integer ratio on both sides (one rounding each)
    np.testing.assert_allclose(f, ref["f"], rtol=2.0 ** -23, atol=0)
    # P: fp32 sums in a fixed tree over T tokens vs fp64 sums
    dP = float(np.abs(P.astype(np.float64) - ref["P"].astype(np.float64)).max())
    assert dP <= 2e-5 * float(ref["P"].max()), dP
    dl = abs(loss - float(ref["loss"])) / max(abs(float(ref["loss"])), 1e-30)
    assert dl <= 2e-5, dl
    _report(f"load_balance_{name}", dP=f"{dP:.2e}", dloss=f"{dl:.2e}", loss=f"{loss:.6g}")


STAGED = ["dropless_softmax", "capacity_heavy_drop", "sigmoid_bias_shared", "split_k_tail",
          "f32_capacity", "f32_sigmoid_shared", "drop_all_shared", "e24_sigmoid_bias",
          "zipf_cf1"]


@pytest.mark.parametrize("hF", [(512, 512), (1024, 1024)], ids=["whole_tiles", "k_split"])
def test_grouped_gemm_tile_heights(hF):
    """Standalone grouped GEMM on groups whose last row tile falls in each
    height class (64, 128, 192 or 256 rows, the class boundaries included),
    plus an empty and a one-row group.  With K = 1024 every tile of both
    GEMMs is in the last partial round and is split along K; with K = 512
    none is."""
    h, F = hF
    counts = [300, 100, 1, 0, 256, 384, 320, 449, 192, 385, 160]
    E, T = len(counts), sum(counts)
    print(f"[case] tile heights h={h} F={F} counts={counts}", flush=True)
    cfg = MoEConfig("tile_heights", T=T, h=h, E=E, k=1, F=F, gate="softmax_topk")
    inp = gen_inputs(cfg)
    c = moe.make_cfg(T, h, F, E, 1, "bf16", "softmax_topk")
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    cnt_d = torch.tensor(counts, dtype=torch.int32, device=DEV)
    off_d = torch.tensor(off, dtype=torch.int32, device=DEV)
    act = torch.full((T, F), float("nan"), dtype=torch.bfloat16, device=DEV)
    yp = torch.full((T, h), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(moe.moe_workspace_bytes(c), dtype=torch.uint8, device=DEV)
    moe.moe_grouped_gemm_swiglu(c, inp["x"], cnt_d, off_d, inp["w1"], inp["w3"], inp["w2"],
                                act, yp, ws)
    torch.cuda.synchronize()
    y = np32(yp)
    assert np.isfinite(y).all(), "rows left unwritten"
    x = np32(inp["x"])
    w1, w3, w2 = LazyExperts(inp["w1"]), LazyExperts(inp["w3"]), LazyExperts(inp["w2"])
    worst = 0.0
    for e, n in enumerate(counts):
        if n == 0:
            continue
        r = slice(off[e], off[e] + n)
        ref = oracle.swiglu_ffn(x[r], w1[e], w3[e], w2[e])
        err = float(check_outputs(cfg, y[r], ref, f"tile_heights group {e}")["token_rel_err"])
        worst = max(worst, err)
    _report(f"tile_heights_{h}", rel_err=f"{worst:.2e}")


@pytest.mark.parametrize("name,routing,iters",
                         [(n, "topk", 0) for n in STAGED] +
                         [("dropless_softmax", "sinkhorn", 4), ("capacity_heavy_drop", "sinkhorn", 7)])
def test_stage_calls_equal_fused_call(name, routing, iters):
    """router_topk -> permute -> grouped_gemm_swiglu (+ the shared expert as
    its own E=1 call) -> combine gives bit-for-bit the fused layer's output
    (top-k or Sinkhorn routing); x_perm holds exact copies of token rows and
    zero padding rows."""
    cfg = next(c for c in MEDIUM if c.name == name)
    print(f"[case] staged {name} {routing}", flush=True)
    inp = gen_inputs(cfg)
    C_lib, _ = capacity_of(cfg)
    fused = run_forward(cfg, inp, C_lib, routing=routing, sinkhorn_iters=iters)
    c = lib_cfg(cfg, C_lib, routing, sinkhorn_iters=iters)
    T, E, k, h, F = cfg.T, cfg.E, cfg.k, cfg.h, cfg.F
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    rows = moe.moe_num_rows(c)
    ws = torch.empty(moe.moe_workspace_bytes(c), dtype=torch.uint8, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gate = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe.moe_router_topk(c, inp["x"], inp["w_router"], inp["logit_bias"], inp["select_bias"],
                        None, idx, gate, ws)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    assign = torch.empty(T * k, dtype=torch.int32, device=DEV)
    rowtok = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    xperm = torch.full((rows, h), 7.0, dtype=tdt, device=DEV)
    moe.moe_permute(c, inp["x"], idx, counts, offsets, assign, rowtok, xperm, ws)
    act = torch.empty((rows, F), dtype=tdt, device=DEV)
    yperm = torch.empty((rows, h), dtype=tdt, device=DEV)
    moe.moe_grouped_gemm_swiglu(c, xperm, counts, offsets, inp["w1"], inp["w3"], inp["w2"],
                                act, yperm, ws)
    shared_y = None
    if cfg.shared:
        cs = moe.make_cfg(T, h, F, 1, 1, cfg.dtype, cfg.gate)
        ws_s = torch.empty(moe.moe_workspace_bytes(cs), dtype=torch.uint8, device=DEV)
        cnt_s = torch.tensor([T], dtype=torch.int32, device=DEV)
        off_s = torch.tensor([0, T], dtype=torch.int32, device=DEV)
        act_s = torch.empty((T, F), dtype=tdt, device=DEV)
        shared_y = torch.empty((T, h), dtype=tdt, device=DEV)
        moe.moe_grouped_gemm_swiglu(cs, inp["x"], cnt_s, off_s, inp["ws1"].unsqueeze(0),
                                    inp["ws3"].unsqueeze(0), inp["ws2"].unsqueeze(0),
                                    act_s, shared_y, ws_s)
    y = torch.empty((T, h), dtype=tdt, device=DEV)
    moe.moe_unpermute_combine(c, yperm, assign, gate, shared_y, y)
    torch.cuda.synchronize()

    assert torch.equal(idx, fused["topk_idx"])
    assert torch.equal(gate, fused["topk_gate"])
    assert torch.equal(assign, fused["assign_row"])
    assert torch.equal(rowtok, fused["row_token"])
    assert torch.equal(counts, fused["expert_counts"])
    assert torch.equal(offsets, fused["expert_offsets"])
    assert torch.equal(y.view(torch.int16 if cfg.dtype == "bf16" else torch.int32),
                       fused["y"].view(torch.int16 if cfg.dtype == "bf16" else torch.int32))
    # a token whose every slot was dropped: the shared expert's output (own
    # E = 1 call) bit for bit, or exactly zero without one
    gone = (assign.view(T, k) < 0).all(1)
    if bool(gone.any()):
        got = fused["y"][gone].view(torch.int16 if cfg.dtype == "bf16" else torch.int32)
        if cfg.shared:
            want = shared_y[gone].view(torch.int16 if cfg.dtype == "bf16" else torch.int32)
            assert torch.equal(got, want)
        else:
            assert not bool(fused["y"][gone].ne(0).any())
    _report(f"staged_{name}_{routing}", tokens_all_dropped=int(gone.sum()))
    # dispatch buffer: row r holds token row_token[r] exactly; pads are zero
    rt = rowtok.long()
    kept = rt >= 0
    xb = inp["x"].view(torch.int16 if cfg.dtype == "bf16" else torch.int32)
    pb = xperm.view(torch.int16 if cfg.dtype == "bf16" else torch.int32)
    assert torch.equal(pb[kept], xb[rt[kept]])
    assert (pb[~kept] == 0).all()
    # unpermute of the dispatch buffer (k = 1 view of slot 0) is the identity
    a0 = assign.view(T, k)[:, 0].long()
    ok = a0 >= 0
    assert torch.equal(pb[a0[ok]], xb[ok])
    # the same routing applied to another tensor (moe_permute_rows): the
    # buffer moe_permute gives for that tensor, bit for bit, pads included
    x2 = normal((T, h), 1.0, cfg.seed, "x_second", device=DEV, dtype=cfg.dtype)
    want = torch.full((rows, h), 3.0, dtype=tdt, device=DEV)
    moe.moe_permute(c, x2, idx, counts, offsets, assign, rowtok, want, ws)
    got = torch.full((rows, h), 5.0, dtype=tdt, device=DEV)
    rowtok2 = rowtok.clone()
    moe.moe_permute_rows(c, x2, assign, counts, rowtok2, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(pb.dtype), want.view(pb.dtype))
    assert torch.equal(rowtok2, rowtok)


def test_deterministic():
    cfg = next(c for c in MEDIUM if c.name == "zipf_cf1")
    inp = gen_inputs(cfg)
    C_lib, _ = capacity_of(cfg)
    a = run_forward(cfg, inp, C_lib)
    b = run_forward(cfg, inp, C_lib)
    for key in ("topk_idx", "topk_gate", "expert_counts", "assign_row", "row_token"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(a["y"].view(torch.int16), b["y"].view(torch.int16))


def _layer_buffers(cfg, C, routing="topk"):
    """Library cfg, workspace, output and routing buffers of one layer."""
    c = lib_cfg(cfg, C, routing)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    ws = torch.empty(max(moe.moe_workspace_bytes(c), 1), dtype=torch.uint8, device=DEV)
    y = torch.empty((cfg.T, cfg.h), dtype=tdt, device=DEV)
    route = {"topk_idx": torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV),
             "assign_row": torch.empty((cfg.T * cfg.k,), dtype=torch.int32, device=DEV)}
    return c, ws, y, route


def _weights(inp):
    return {n: inp[n] for n in ("w_router", "w1", "w3", "w2", "logit_bias", "select_bias",
                                "ws1", "ws3", "ws2")}


def test_concurrent_calls_on_two_streams():
    """Two layers enqueued alternately on two streams (each with its own
    workspace and outputs), several times over: every output equals the
    same layer run alone, bit for bit (the library keeps no state)."""
    cfgs = [next(c for c in MEDIUM if c.name == n)
            for n in ("worked_example_small", "split_k_tail_capacity_shared")]
    inps = [gen_inputs(c) for c in cfgs]
    Cs = [capacity_of(c)[0] for c in cfgs]
    refs = [run_forward(c, i, C) for c, i, C in zip(cfgs, inps, Cs)]
    bufs = [_layer_buffers(c, C) for c, C in zip(cfgs, Cs)]
    streams = [torch.cuda.Stream() for _ in cfgs]
    torch.cuda.synchronize()
    for _ in range(3):
        for inp, (c, ws, y, route), st in zip(inps, bufs, streams):
            with torch.cuda.stream(st):
                moe.moe_forward(c, _weights(inp), inp["x"], y, route, ws)
    torch.cuda.synchronize()
    for ref, (c, ws, y, route) in zip(refs, bufs):
        assert torch.equal(route["topk_idx"], ref["topk_idx"])
        assert torch.equal(route["assign_row"], ref["assign_row"])
        assert torch.equal(y.view(torch.int16), ref["y"].view(torch.int16))


def test_forward_captured_in_a_graph():
    """moe_forward captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed with eager work and synchronisations in between, also after new
    token values are copied into the captured input: every replay equals an
    eager forward on the same values, bit for bit."""
    cfg = next(c for c in MEDIUM if c.name == "worked_example_small")
    inp = gen_inputs(cfg)
    C, _ = capacity_of(cfg)
    ref0 = run_forward(cfg, inp, C)
    x1 = normal((cfg.T, cfg.h), 1.0, cfg.seed + 1, "x", device=DEV, dtype=cfg.dtype)
    ref1 = run_forward(cfg, dict(inp, x=x1), C)
    c, ws, y, route = _layer_buffers(cfg, C)
    x = inp["x"].clone()
    w = _weights(inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_forward(c, w, x, y, route, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(c, w, x, y, route, ws)
    torch.cuda.synchronize()
    for rep, (xv, ref) in enumerate([(inp["x"], ref0), (x1, ref1), (inp["x"], ref0),
                                     (x1, ref1)]):
        x.copy_(xv)
        y.fill_(float("nan"))
        route["topk_idx"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(route["topk_idx"], ref["topk_idx"]), rep
        assert torch.equal(y.view(torch.int16), ref["y"].view(torch.int16)), rep
        run_forward(cfg, inp, C)          # eager work between the replays


def test_empty_input_is_a_no_op():
    cfg = MoEConfig("empty", T=0, h=128, E=4, k=2, F=128)
    c = lib_cfg(cfg, 0)
    inp = gen_inputs(cfg.with_(T=1))
    y = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(moe.moe_workspace_bytes(c), 1), dtype=torch.uint8, device=DEV)
    moe.moe_forward(c, {n: inp[n] for n in ("w_router", "w1", "w3", "w2")},
                    inp["x"], y, None, ws)
    torch.cuda.synchronize()


def test_errors_are_reported_before_launch():
    cfg = CONFIGS["tiny_fp32"]
    inp = gen_inputs(cfg)
    c = lib_cfg(cfg, 0)
    y = torch.empty((cfg.T, cfg.h), dtype=torch.float32, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    w = {n: inp[n] for n in ("w_router", "w1", "w3", "w2")}
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward(c, w, inp["x"], y, None, small)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    bad = lib_cfg(cfg.with_(k=5), 0)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward(bad, w, inp["x"], y, None, small)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_select_bias_update_matches_oracle():
    """Random loads and biases: the step equals the oracle's bit for bit,
    experts exactly at the mean load keep their bias (a -0.0 included)."""
    g = torch.Generator().manual_seed(5)
    for T, E, k in [(12, 4, 2), (4096, 8, 2), (4096, 256, 8), (1000, 1024, 16)]:
        print(f"[case] select-bias step T={T} E={E} k={k}", flush=True)
        c = moe.make_cfg(T, 128, 128, E, k, "bf16", "sigmoid_topk_norm")
        mean = T * k // E
        counts = torch.randint(max(0, mean - 3), mean + 4, (E,), generator=g, dtype=torch.int32)
        bias = (torch.randn(E, generator=g) * 0.3).float()
        bias[0] = -0.0
        counts[1] = mean
        gb = bias.to(DEV)
        moe.moe_select_bias_update(c, counts.to(DEV), 1e-3, gb)
        ref = oracle.select_bias_update(bias.numpy(), counts.numpy(), T, k, 1e-3)
        np.testing.assert_array_equal(gb.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_select_bias_update_evens_a_skewed_router():
    """Route with the bias, count, step the bias, 150 times on a Zipf-skewed
    router: every step equals the oracle's step from the GPU's own counts
    (which equal the counts of the GPU's selection), and the loads end near
    the mean."""
    cfg = MoEConfig("bias_loop", T=2048, h=128, E=16, k=2, F=128, gate="softmax_topk",
                    logit_bias=("zipf", 1.2))
    print(f"[case] select-bias loop T={cfg.T} E={cfg.E} k={cfg.k}", flush=True)
    inp = gen_inputs(cfg)
    c = lib_cfg(cfg, 0)
    T, E, k, h = cfg.T, cfg.E, cfg.k, cfg.h
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gate = torch.empty((T, k), dtype=torch.float32, device=DEV)
    counts = torch.empty((E,), dtype=torch.int32, device=DEV)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    assign = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    rowtok = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    xperm = torch.empty((T * k, h), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(moe.moe_workspace_bytes(c), dtype=torch.uint8, device=DEV)
    bias = torch.zeros((E,), dtype=torch.float32, device=DEV)
    mean = T * k / E
    first = None
    for _ in range(150):
        prev = bias.cpu().numpy()
        moe.moe_router_topk(c, inp["x"], inp["w_router"], inp["logit_bias"], bias, logits, idx,
                            gate, ws)
        moe.moe_permute(c, inp["x"], idx, counts, offs, assign, rowtok, xperm, ws)
        moe.moe_select_bias_update(c, counts, 0.02, bias)
        cnt = counts.cpu().numpy()
        np.testing.assert_array_equal(cnt, np.bincount(idx.cpu().numpy().ravel(), minlength=E))
        np.testing.assert_array_equal(bias.cpu().numpy(),
                                      oracle.select_bias_update(prev, cnt, T, k, 0.02))
        first = cnt if first is None else first
    assert first.max() > 2.5 * mean
    assert cnt.max() < 1.25 * mean and cnt.min() > 0.75 * mean


def test_binding_refuses_tensors_smaller_than_the_config():
    """A tensor smaller than the config implies would send the kernels past
    its end: the binding refuses it before any launch."""
    cfg = CONFIGS["tiny_fp32"]
    inp = gen_inputs(cfg)
    c = lib_cfg(cfg, 0)
    ws = torch.empty(moe.moe_workspace_bytes(c), dtype=torch.uint8, device=DEV)
    w = {n: inp[n] for n in ("w_router", "w1", "w3", "w2")}
    y_short = torch.empty((cfg.T - 1, cfg.h), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="y holds"):
        moe.moe_forward(c, w, inp["x"], y_short, None, ws)
    w_short = dict(w, w2=inp["w2"][:-1])
    y = torch.empty((cfg.T, cfg.h), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="w2 holds"):
        moe.moe_forward(c, w_short, inp["x"], y, None, ws)


@pytest.mark.parametrize("k", [2, 20])
def test_combine_ignores_rows_outside_the_expert_outputs(k):
    """A caller's map with rows outside [0, rows) (negative, rows, past it,
    INT32_MAX): those slots contribute nothing, exactly as dropped slots
    (-1) do, bit for bit; k = 20 takes the many-slot combine (expert choice
    over 20 experts)."""
    T, h, E = 64, 256, max(k, 4)
    print(f"[case] combine with out-of-range rows T={T} h={h} k={k}", flush=True)
    routing = "expert_choice" if k > 16 else "topk"
    c = moe.make_cfg(T, h, 128, E, k if k <= 16 else 2, "bf16", "softmax_topk",
                     capacity=(T if k > 16 else 0), routing=routing)
    rows = moe.moe_num_rows(c)
    slots = E if k > 16 else k
    g = torch.Generator().manual_seed(11)
    y_perm = torch.randn((rows, h), generator=g).to(torch.bfloat16).to(DEV)
    gate = torch.rand((T, slots), generator=g).to(DEV)
    good = torch.randint(0, rows, (T * slots,), generator=g, dtype=torch.int32)
    bad_vals = torch.tensor([-5, rows, rows + 100, 2 ** 31 - 1], dtype=torch.int32)
    pos = torch.randperm(T * slots, generator=g)[:T]          # one in `slots` slots
    bad = good.clone()
    bad[pos] = bad_vals[torch.arange(T) % 4]
    dropped = good.clone()
    dropped[pos] = -1
    y_bad = torch.empty((T, h), dtype=torch.bfloat16, device=DEV)
    y_drop = torch.empty_like(y_bad)
    moe.moe_unpermute_combine(c, y_perm, bad.to(DEV), gate, None, y_bad)
    moe.moe_unpermute_combine(c, y_perm, dropped.to(DEV), gate, None, y_drop)
    torch.cuda.synchronize()
    assert torch.equal(y_bad.view(torch.int16), y_drop.view(torch.int16))
    assert y_drop.abs().sum().item() > 0


# ------------------------------------------------------------ maximum sizes
def test_beyond_int32_element_counts():
    """x [2^19 + 77, 4096] bf16 holds more than 2^31 elements and the
    dispatch buffers x_perm and y_perm more than 2^32 (rows of 4096 + 64),
    so a 32-bit index or byte offset anywhere on the path would show: the
    routing on the GPU's own keys, gates and maps compared for every token,
    logits and outputs of sampled tokens (the first and last among them)
    against the oracle."""
    cfg = MoEConfig("beyond_int32", T=(1 << 19) + 77, h=4096, E=8, k=2, F=128,
                    gate="softmax_topk")
    print(f"[case] beyond int32 T={cfg.T} h={cfg.h}", flush=True)
    torch.cuda.empty_cache()
    inp = gen_inputs(cfg)
    assert inp["x"].numel() > 2 ** 31
    gpu = run_forward(cfg, inp, 0)
    assert gpu["rows"] * (cfg.h + 64) > 2 ** 32
    g_logits = gpu["logits"].cpu().numpy()
    g_idx = gpu["topk_idx"].cpu().numpy()
    np.testing.assert_array_equal(oracle.topk(g_logits, cfg.k), g_idx)
    dg = float(np.abs(gpu["topk_gate"].cpu().numpy() - oracle.gates(g_logits, g_idx, cfg.gate)).max())
    assert dg <= 2e-6
    m = oracle.route_maps(g_idx, cfg.E)
    np.testing.assert_array_equal(gpu["expert_counts"].cpu().numpy(), m["counts"])
    np.testing.assert_array_equal(gpu["expert_offsets"].cpu().numpy(), m["offsets"])
    np.testing.assert_array_equal(gpu["assign_row"].cpu().numpy().reshape(-1, cfg.k),
                                  m["assign_row"])
    np.testing.assert_array_equal(gpu["row_token"].cpu().numpy(), m["row_token"])
    # every 64th token, the last 256 (whose x rows start past element 2^31)
    # and the tokens on the last dispatch rows (byte offsets past 2^32)
    rt = gpu["row_token"][-512:].cpu().numpy()
    tok = np.unique(np.concatenate([np.arange(0, cfg.T, 64), np.arange(cfg.T - 256, cfg.T),
                                    rt[rt >= 0]]))
    tt = torch.as_tensor(tok, device=DEV)
    ref = oracle.moe_forward(np32(inp["x"][tt]), np32(inp["w_router"]), LazyExperts(inp["w1"]),
                             LazyExperts(inp["w3"]), LazyExperts(inp["w2"]), k=cfg.k,
                             gate=cfg.gate, idx=g_idx[tok])
    dl = float(np.abs(ref["logits"] - g_logits[tok]).max())
    assert dl <= 5e-5 * max(1.0, float(np.abs(ref["logits"]).max()))
    out = check_outputs(cfg, np32(gpu["y"][tt]), ref["y"], "beyond_int32")
    _report("beyond_int32", max_dlogit=dl, max_dgate=dg, rows=gpu["rows"], sampled=len(tok),
            **out)
    del gpu, inp
    torch.cuda.empty_cache()


# ------------------------------------------------------------ full sizes
FULL = ["worked_example", "mixtral", "deepseek_v3", "skewed", "skewed_cf1"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_routing_and_every_output(name):
    """The full workloads, launched exactly as the benchmark launches them:
    routing, counts, maps and drops compared in full, and the output of
    every token against the oracle (normwise over the layer and per token;
    tokens whose every slot was dropped exactly zero).  The oracle fetches
    one expert's weights at a time and drops them after use."""
    cfg = CONFIGS[name]
    print(f"[case] full {name} T={cfg.T} h={cfg.h} E={cfg.E} k={cfg.k} F={cfg.F}", flush=True)
    torch.cuda.empty_cache()
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    if name == "worked_example":
        assert C_lib == 1280
    gpu = run_forward(cfg, inp, C_lib)
    ref = oracle_forward(cfg, inp, C_ref, maps_only=True)
    rep = check_routing(cfg, gpu, ref, C_ref, inp)
    counts = gpu["expert_counts"].cpu().numpy()
    if cfg.logit_bias is not None and cfg.logit_bias[0] == "zipf":
        assert counts.max() > 10 * counts.mean()
    g_idx = gpu["topk_idx"].cpu().numpy()
    assign = gpu["assign_row"].cpu().numpy().reshape(cfg.T, cfg.k)
    all_dropped = int((assign < 0).all(1).sum())
    ref_y = oracle_forward(cfg, inp, C_ref, idx=g_idx, cache_experts=False)["y"]
    y = np32(gpu["y"])
    assert np.isfinite(y).all()
    out = check_outputs(cfg, y, ref_y, name)
    assert out["zero_rows"] == (0 if cfg.shared else all_dropped)
    del ref_y
    # load-balance statistics of this routing, against the oracle's own
    # logits and counts (so the whole chain router -> counts -> stats)
    c = lib_cfg(cfg, C_lib)
    lb = [torch.full((n_,), float("nan"), dtype=torch.float32, device=DEV)
          for n_ in (cfg.E, cfg.E, 1)]
    moe.moe_load_balance(c, gpu["logits"], gpu["expert_counts"], 0.01, *lb, gpu["ws"])
    torch.cuda.synchronize()
    ref_lb = oracle.load_balance(ref["logits"], np.bincount(ref["idx"].ravel(), minlength=cfg.E),
                                 cfg.k, cfg.gate, 0.01)
    lb_err = abs(float(lb[2].item()) - float(ref_lb["loss"])) / float(ref_lb["loss"])
    _report(name, tokens=cfg.T, max_count=int(counts.max()),
            mean_count=float(counts.mean()), aux_loss=f"{float(lb[2].item()):.6g}",
            aux_loss_rel_err=f"{lb_err:.1e}", **out, **rep)
    # near-tie tokens may route differently; each moves at most 1/(T*k) of f
    assert lb_err <= 1e-4
    del gpu, inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,saved", [("worked_example", False), ("deepseek_v3", False),
                                        ("worked_example", True)])
def test_full_size_backward_sampled(name, saved):
    """The backward at full size, launched as the benchmark launches it
    (saved: from the activations the forward kept): dx and the gate
    gradients of sampled tokens against the oracle's token-by-token rows;
    every gradient finite."""
    cfg = CONFIGS[name]
    print(f"[case] full backward {name} saved={saved} T={cfg.T} h={cfg.h} E={cfg.E} "
          f"k={cfg.k} F={cfg.F}", flush=True)
    torch.cuda.empty_cache()
    inp = gen_inputs(cfg)
    C_lib, C_ref = capacity_of(cfg)
    gpu = run_forward(cfg, inp, C_lib, save=saved)
    dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=DEV)
    g = run_backward(cfg, inp, C_lib, gpu, dy, saved=saved)
    for key, v in g.items():
        assert bool(torch.isfinite(v.float()).all()), key
    rng = np.random.default_rng(1)
    tok = np.array(sorted(set(rng.choice(cfg.T, 6, replace=False).tolist()) | {0, cfg.T - 1}))
    x, wr, w1, w3, w2, lb, shared = oracle_weights(cfg, inp)
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    ref = oracle.moe_backward(x, wr, w1, w3, w2, np32(dy), k=cfg.k, gate=cfg.gate, C=C_ref,
                              logit_bias=lb, select_bias=sb, shared=shared,
                              idx=gpu["topk_idx"].cpu().numpy(), tokens=tok)
    t = torch.as_tensor(tok, device=DEV)
    e_dx = rel_err(np32(g["dx"][t]), ref["dx"])
    e_dg = rel_err(np32(g["dgate"][t]), ref["dgate"])
    _report(f"full_backward_{name}{'_saved' if saved else ''}", sampled=len(tok),
            dx=f"{e_dx:.2e}", dgate=f"{e_dg:.2e}")
    assert e_dx <= 2e-2 and e_dg <= 2e-2
    del g, gpu, inp
    torch.cuda.empty_cache()
