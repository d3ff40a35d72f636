"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

A step is one fused moe_forward (router GEMM, top-k/gates, scan, assign,
permute, grouped GEMM 1 + SwiGLU, grouped GEMM 2, combine) over one batch of
seeded synthetic input already resident in HBM.  Default workload: the
worked example T=4096, h=4096, E=8, k=2, F=12288, capacity factor 5/4
(C = 1280), softmax over all E then the top-2 gate values.

Prints ONE JSON line: tokens/s over the K timed steps (no instrumentation),
per-stage kernel durations from K more steps whose stages carry HIP start/stop
events bound to their kernels (hipExtLaunchKernel: the kernels' own
timestamps, the figures rocprofv3's kernel trace reports), the grouped-GEMM
roofline (algorithmic FLOPs / GEMM 1's kernel time vs the bf16 dense MFMA
peak, or its compulsory bytes vs HBM when it streams weights),
permute/combine algorithmic bytes vs HBM, the same step timed from a cold
last-level cache (medians), and the CPU oracle timed on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

def metric_label(T: int, h: int, E: int, k: int) -> str:
    """The metric's name for a workload of T tokens, width h, E experts,
    top-k (the headline workload's is the T=4096 h=4096 E=8 k=2 one)."""
    return ("MoE-layer fwd tokens/s and grouped-GEMM TFLOPS (% MFMA peak), "
            f"T={T} h={h} E={E} k={k}")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


# ---------------------------------------------------------------- accounting
def gemm1_flops(kept_rows: int, h: int, F: int) -> int:
    """GEMM 1: two [rows,h] x [h,F] products (w1 and w3), 2 flops per MAC."""
    return 4 * kept_rows * h * F


def gemm2_flops(kept_rows: int, h: int, F: int) -> int:
    """GEMM 2: one [rows,F] x [F,h] product."""
    return 2 * kept_rows * h * F


def expert_flops(kept_rows: int, h: int, F: int) -> int:
    return gemm1_flops(kept_rows, h, F) + gemm2_flops(kept_rows, h, F)


def gemm1_bytes(kept_per_expert, T: int, h: int, F: int, esz: int, shared: bool,
                in_rows=None) -> int:
    """GEMM 1's compulsory HBM bytes: w1 and w3 of every expert with a row
    (and of the shared expert), the input rows read once, the activations
    written once.  The input rows are the dispatch rows, or `in_rows` token
    rows when the GEMM gathers them from the tokens (each distinct token
    once)."""
    active = sum(1 for n in kept_per_expert if n > 0) + (1 if shared else 0)
    rows = sum(kept_per_expert) + (T if shared else 0)
    a_rows = rows if in_rows is None else in_rows
    return (2 * active * F * h + a_rows * h + rows * F) * esz


def router_bytes(T: int, h: int, E: int, esz: int) -> int:
    """Read the tokens and the router weights once, write fp32 logits."""
    return (T + E) * h * esz + T * E * 4


def permute_bytes(T: int, h: int, rows: int, esz: int) -> int:
    """Read every token row once, write every row of the dispatch buffer
    (kept copies and zero padding)."""
    return (T + rows) * h * esz


def dispatch_payload_bytes(T: int, k: int, h: int, esz: int) -> int:
    """The T*k token copies of a dropless dispatch (the part of the permute's
    writes that the expert-parallel all-to-all would carry)."""
    return T * k * h * esz


def combine_bytes(kept_rows: int, T: int, h: int, esz: int, shared: bool) -> int:
    """Read every kept expert-output row (and the shared rows), write y."""
    return (kept_rows + T + (T if shared else 0)) * h * esz


# ------------------------------------------------------------ HBM traffic
GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_layer_25_amd", "csrc", "grouped_gemm.hip")


def traffic_file(workload: str) -> str:
    """The committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary of a workload."""
    return os.path.join(ROOT, "profiles", f"grouped_gemm_traffic_{workload.split(':')[0]}.txt")


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _machine_fields(path: str) -> dict:
    """The ``name: value`` lines of a committed profile summary."""
    kv = {}
    if os.path.exists(path):
        with open(path) as f:
            for line in f:
                m = re.match(r"^([a-z_0-9]+):\s*(\S+)", line)
                if m:
                    kv[m.group(1)] = m.group(2)
    return kv


def measured_traffic(workload: str):
    """HBM bytes per launch of GEMM 1 from the committed counter summary, or
    None when the summary is missing, is for another workload, or was taken
    on a different version of the kernel source."""
    kv = _machine_fields(traffic_file(workload))
    if not kv:
        return None
    if kv.get("kernel_source_sha256_16") != source_hash(GEMM_SOURCE):
        return None
    if kv.get("workload") != workload.split(":")[0]:
        return None
    try:
        return int(kv["gemm1_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gathered_dispatch(dtype: str, T: int, h: int) -> bool:
    """bf16 forwards that keep no activations read GEMM 1's token rows from x
    through row_token: no dispatch buffer is written and the permute stage
    launches nothing (its events hold two markers)."""
    return dtype == "bf16" and T * h * 2 < (1 << 31)


def fused_router_topk(dtype: str, E: int, routing: str) -> bool:
    """bf16 layers of up to 64 experts with plain or score-drop top-k run the
    router, top-k, gates and histogram as one kernel (stage "router"); the
    "topk" stage then launches nothing and its events hold two markers."""
    return dtype == "bf16" and E <= 64 and routing in ("topk", "topk_score_drop")


# --------------------------------------------------------------------- bench
def _workload_name(cfg, C, routing="topk"):
    s = (f"{cfg.name}: T={cfg.T} h={cfg.h} E={cfg.E} k={cfg.k} F={cfg.F} {cfg.dtype} "
         f"{cfg.gate}")
    if routing != "topk":
        s += f" {routing}"
    s += f" C={C}" if C else " dropless"
    if cfg.shared:
        s += " +1 shared expert"
    return s


def routing_stats(logits, select_bias, assign_row, k: int, tie: float = 1e-5) -> dict:
    """Counts of the step's routing, from the device's own outputs: tokens
    whose k-th and (k+1)-th fp32 selection keys are closer than `tie` (where
    another fp32 summation order of the logits could choose differently),
    dropped assignments and tokens that lost every slot."""
    import numpy as np
    keys = logits.astype(np.float32)
    if select_bias is not None:
        keys = keys + select_bias.astype(np.float32)[None, :]
    E = keys.shape[1]
    near = 0
    if k < E:
        srt = -np.sort(-keys.astype(np.float64), axis=1)
        near = int((srt[:, k - 1] - srt[:, k] < tie).sum())
    a = assign_row.reshape(-1, k)
    return {"near_ties": near, "dropped_assignments": int((a < 0).sum()),
            "tokens_all_dropped": int((a < 0).all(1).sum())}


def cpu_baseline(cfg, inp, C, sample_tokens: int, min_seconds: float) -> dict:
    """The oracle, as it stands, on the first `sample_tokens` tokens' outputs
    (routing, ranks and drops still over all T tokens), repeated until at
    least `min_seconds` of CPU work have been timed."""
    import numpy as np
    import oracle
    f32 = lambda t: t.float().cpu().numpy()  # noqa: E731
    x, wr = f32(inp["x"]), f32(inp["w_router"])
    w1, w3, w2 = f32(inp["w1"]), f32(inp["w3"]), f32(inp["w2"])
    lb = None if inp["logit_bias"] is None else inp["logit_bias"].cpu().numpy()
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    shared = (f32(inp["ws1"]), f32(inp["ws3"]), f32(inp["ws2"])) if cfg.shared else None
    tok = np.arange(min(sample_tokens, cfg.T))
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_forward(x, wr, w1, w3, w2, k=cfg.k, gate=cfg.gate, C=C or None,
                           logit_bias=lb, select_bias=sb, shared=shared, tokens=tok)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    try:
        import threadpoolctl
        cores = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        cores = os.cpu_count() or 1
    return {"value": passes * len(tok) / dt, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{passes} passes over the outputs of the first {len(tok)} of {cfg.T} "
                      f"tokens (routing of all {cfg.T} in each pass), fp64 numpy oracle"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="worked_example")
    ap.add_argument("--routing", default="topk",
                    choices=("topk", "topk_score_drop", "expert_choice", "sinkhorn"),
                    help="routing variant (the headline workload uses topk)")
    ap.add_argument("--sinkhorn-iters", type=int, default=10,
                    help="Sinkhorn iterations (--routing sinkhorn, and the Sinkhorn leg "
                         "of a topk run; 0 skips that leg)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--cpu-sample", type=int, default=1024)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle sample until this much time has been timed")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed one by one after a 512 MiB fill evicts the "
                         "last-level cache (medians reported; 0: skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this size before the timed steps "
                         "(reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the layer "
              "has no multi-GPU path in this library", file=sys.stderr)
        return 2

    import torch
    import mixture_experts_layer_25_amd as moe
    from moe_inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = make_inputs(cfg, device=dev)
    C = moe.moe_capacity(cfg.T, cfg.E, cfg.k, *cfg.cf) if cfg.cf else 0
    if args.routing not in ("topk", "sinkhorn") and C == 0:
        print(f"--routing {args.routing} needs a workload with a capacity", file=sys.stderr)
        return 2
    if args.routing == "expert_choice":
        C = min(C, cfg.T)
        inp["select_bias"] = None      # expert choice ranks by probability only
    sk_iters = args.sinkhorn_iters if args.routing == "sinkhorn" else 0
    if args.routing == "sinkhorn":
        inp["select_bias"] = None      # the balancing finds its own selection bias
    c = moe.make_cfg(cfg.T, cfg.h, cfg.F, cfg.E, cfg.k, cfg.dtype, cfg.gate, capacity=C,
                     has_shared=cfg.shared, routing=args.routing, sinkhorn_iters=sk_iters)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    esz = 2 if cfg.dtype == "bf16" else 4
    rows = moe.moe_num_rows(c)
    ws = torch.empty(moe.moe_workspace_bytes(c), dtype=torch.uint8, device=dev)
    y = torch.empty((cfg.T, cfg.h), dtype=tdt, device=dev)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    route = {"expert_counts": counts}
    weights = {n: inp[n] for n in ("w_router", "w1", "w3", "w2", "logit_bias",
                                   "select_bias", "ws1", "ws3", "ws2")}

    for _ in range(args.warmup):
        moe.moe_forward(c, weights, inp["x"], y, route, ws)
    torch.cuda.synchronize()
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # `value`: K steps with no instrumentation, host clock between two
    # synchronisations.
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        moe.moe_forward(c, weights, inp["x"], y, route, ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Kernel times: K more steps whose stages carry start/stop events bound
    # to their first and last kernels (the kernels' own timestamps).
    NS = moe.MOE_NUM_STAGES

    def new_events(n):
        out = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.MOE_NUM_EVENTS)]
               for _ in range(n)]
        for es in out:         # create the events outside the timed region
            for e in es:
                e.record()
        return out

    def stage_lists(ev_sets):
        return {name: [es[2 * st].elapsed_time(es[2 * st + 1]) for es in ev_sets]
                for st, name in enumerate(moe.STAGE_NAMES)}

    def median(v):
        v = sorted(v)
        return 0.5 * (v[(len(v) - 1) // 2] + v[len(v) // 2])

    evs = new_events(K)
    torch.cuda.synchronize()
    for i in range(K):
        moe.moe_forward(c, weights, inp["x"], y, route, ws, events=evs[i])
    torch.cuda.synchronize()
    kern = stage_lists(evs)
    stage_ms = {name: sum(v) / K for name, v in kern.items()}
    kernel_span_ms = sum(es[0].elapsed_time(es[2 * NS - 1]) for es in evs) / K

    # On-box HBM yardstick: a plain 1 GiB device-to-device copy (torch),
    # best of 5, read + write bytes over its event time.  Skipped in the
    # counter runs (--copy-calibration-mib), whose only large copy must be
    # the calibration copy.
    copy_gbs = None
    if args.copy_calibration_mib == 0:
        cp_src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        cp_dst = torch.empty_like(cp_src)
        cp_dst.copy_(cp_src)
        cp_best = None
        for _ in range(5):
            ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ce0.record()
            cp_dst.copy_(cp_src)
            ce1.record()
            torch.cuda.synchronize()
            ms = ce0.elapsed_time(ce1)
            cp_best = ms if cp_best is None else min(cp_best, ms)
        copy_gbs = 2 * cp_src.numel() * 4 / (cp_best * 1e-3) / 1e9
        del cp_src, cp_dst

    # The step's routing, read back once (not timed): counts of near-tied
    # selection keys and of drops, for the record.
    rs_route = {"logits": torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev),
                "expert_counts": counts}
    slots = cfg.E if args.routing == "expert_choice" else cfg.k
    rs_route["assign_row"] = torch.empty(cfg.T * slots, dtype=torch.int32, device=dev)
    rs_route["topk_gate"] = torch.empty((cfg.T, slots), dtype=torch.float32, device=dev)
    moe.moe_forward(c, weights, inp["x"], y, rs_route, ws)
    torch.cuda.synchronize()
    if args.routing == "expert_choice":
        a = rs_route["assign_row"].view(cfg.T, cfg.E).cpu().numpy()
        rstats = {"tokens_no_expert": int((a < 0).all(1).sum())}
    else:
        sb_np = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
        rstats = routing_stats(rs_route["logits"].cpu().numpy(), sb_np,
                               rs_route["assign_row"].cpu().numpy(), cfg.k)

    # The combine kernel alone (moe_unpermute_combine) on this step's
    # routing, cycling over enough buffer sets (expert outputs + y) that
    # each call's operands have left the 256 MB last-level cache; 10 rounds
    # over the sets between one pair of events.
    comb_alone = None
    comb_sets = 0
    if args.routing == "topk" and not cfg.shared:
        set_bytes = (rows + cfg.T) * cfg.h * esz
        comb_sets = max(2, min(8, -(-(512 << 20) // set_bytes)))
        sets = [(torch.empty((rows, cfg.h), dtype=tdt, device=dev).normal_(), torch.empty_like(y))
                for _ in range(comb_sets)]
        for yp, yc in sets:
            moe.moe_unpermute_combine(c, yp, rs_route["assign_row"], rs_route["topk_gate"], None, yc)
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ce[0].record()
        for _ in range(10):
            for yp, yc in sets:
                moe.moe_unpermute_combine(c, yp, rs_route["assign_row"], rs_route["topk_gate"],
                                          None, yc)
        ce[1].record()
        torch.cuda.synchronize()
        comb_alone = ce[0].elapsed_time(ce[1]) * 1e3 / (10 * comb_sets)
        del sets

    # The permute kernel alone (moe_permute_rows: the step's routing applied
    # to other token tensors), cycling over enough buffer sets (tokens +
    # dispatch buffer) that each call's operands have left the 256 MB
    # last-level cache; 10 rounds over the sets between one pair of events.
    perm_alone = None
    perm_sets = 0
    if args.routing != "expert_choice":
        set_bytes = (cfg.T + rows) * cfg.h * esz
        perm_sets = max(2, min(8, -(-(512 << 20) // set_bytes)))
        psets = [(torch.empty((cfg.T, cfg.h), dtype=tdt, device=dev).normal_(),
                  torch.empty((rows, cfg.h), dtype=tdt, device=dev)) for _ in range(perm_sets)]
        ptok = torch.empty(rows, dtype=torch.int32, device=dev)
        for xs, xp in psets:
            moe.moe_permute_rows(c, xs, rs_route["assign_row"], counts, ptok, xp)
        pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        pe[0].record()
        for _ in range(10):
            for xs, xp in psets:
                moe.moe_permute_rows(c, xs, rs_route["assign_row"], counts, ptok, xp)
        pe[1].record()
        torch.cuda.synchronize()
        perm_alone = pe[0].elapsed_time(pe[1]) * 1e3 / (10 * perm_sets)
        del psets, ptok

    # The same step from a cold last-level cache (256 MB on the MI355X): a
    # 512 MiB fill before each step, every step's kernels timed by their own
    # events, medians reported.  Not part of `value`.
    cold = None
    if args.cold_steps > 0:
        junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cev = new_events(args.cold_steps)
        torch.cuda.synchronize()
        for i in range(args.cold_steps):
            junk.fill_(i & 0xFF)
            moe.moe_forward(c, weights, inp["x"], y, route, ws, events=cev[i])
        torch.cuda.synchronize()
        del junk
        ck = stage_lists(cev)
        cold = {"steps": args.cold_steps,
                "kernel_span_ms": round(median([es[0].elapsed_time(es[2 * NS - 1])
                                                for es in cev]), 4)}
        cold["stage_ms"] = {name: round(median(v), 5) for name, v in ck.items()}
        if fused_router_topk(cfg.dtype, cfg.E, args.routing):
            cold["stage_ms"]["topk"] = None
        if gathered_dispatch(cfg.dtype, cfg.T, cfg.h):
            cold["stage_ms"]["permute"] = None

    # load-balance statistics of the last step's routing (not part of the
    # step): reads the logits once (T*E*4 bytes)
    logits = rs_route["logits"]
    lb_out = [torch.empty(cfg.E, dtype=torch.float32, device=dev) for _ in range(2)]
    lb_loss = torch.empty(1, dtype=torch.float32, device=dev)
    for _ in range(3):
        moe.moe_load_balance(c, logits, counts, 0.01, lb_out[0], lb_out[1], lb_loss, ws)
    lb_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    lb_ev[0].record()
    for _ in range(K):
        moe.moe_load_balance(c, logits, counts, 0.01, lb_out[0], lb_out[1], lb_loss, ws)
    lb_ev[1].record()
    torch.cuda.synchronize()
    lb_us = lb_ev[0].elapsed_time(lb_ev[1]) * 1e3 / K

    # backward of the same layer with this routing (not part of the step):
    # gradients of sum(y * dy) for x, the router and every expert weight
    bwd = None
    if not args.no_backward:
        from moe_inputs import normal
        dy = normal((cfg.T, cfg.h), 1.0, cfg.seed, "dy", device=dev, dtype=cfg.dtype)
        full_route = {"logits": logits,
                      "topk_idx": torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev),
                      "topk_gate": torch.empty((cfg.T, slots), dtype=torch.float32, device=dev),
                      "expert_counts": counts,
                      "expert_offsets": torch.empty(cfg.E + 1, dtype=torch.int32, device=dev),
                      "assign_row": torch.empty(cfg.T * slots, dtype=torch.int32, device=dev)}
        if args.routing == "expert_choice":
            full_route["probs"] = torch.empty((cfg.E, cfg.T), dtype=torch.float32, device=dev)
        moe.moe_forward(c, weights, inp["x"], y, full_route, ws)
        bf = tdt
        grads = {"dx": torch.empty((cfg.T, cfg.h), dtype=bf, device=dev),
                 "dw_router": torch.empty((cfg.E, cfg.h), dtype=bf, device=dev),
                 "dw1": torch.empty((cfg.E, cfg.F, cfg.h), dtype=bf, device=dev),
                 "dw3": torch.empty((cfg.E, cfg.F, cfg.h), dtype=bf, device=dev),
                 "dw2": torch.empty((cfg.E, cfg.h, cfg.F), dtype=bf, device=dev)}
        if cfg.shared:
            grads.update({"dws1": torch.empty((cfg.F, cfg.h), dtype=bf, device=dev),
                          "dws3": torch.empty((cfg.F, cfg.h), dtype=bf, device=dev),
                          "dws2": torch.empty((cfg.h, cfg.F), dtype=bf, device=dev)})
        wsb = torch.empty(moe.moe_backward_workspace_bytes(c), dtype=torch.uint8, device=dev)
        for _ in range(2):
            moe.moe_backward(c, weights, inp["x"], dy, full_route, grads, wsb)
        bw_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        nb = max(3, K // 4)
        bw_ev[0].record()
        for _ in range(nb):
            moe.moe_backward(c, weights, inp["x"], dy, full_route, grads, wsb)
        bw_ev[1].record()
        torch.cuda.synchronize()
        bwd = bw_ev[0].elapsed_time(bw_ev[1]) / nb
        # the same backward from activations the forward kept
        # (save_for_backward): the forward's cost with the flag, then the
        # saved backward
        cs = moe.make_cfg(cfg.T, cfg.h, cfg.F, cfg.E, cfg.k, cfg.dtype, cfg.gate, capacity=C,
                          has_shared=cfg.shared, routing=args.routing, save_for_backward=True,
                          sinkhorn_iters=sk_iters)
        wsf = torch.empty(moe.moe_workspace_bytes(cs), dtype=torch.uint8, device=dev)
        for _ in range(2):
            moe.moe_forward(cs, weights, inp["x"], y, full_route, wsf)
        sv_ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        sv_ev[0].record()
        for _ in range(nb):
            moe.moe_forward(cs, weights, inp["x"], y, full_route, wsf)
        sv_ev[1].record()
        for _ in range(2):
            moe.moe_backward_saved(cs, weights, inp["x"], dy, full_route, wsf, grads, wsb)
        sv_ev[2].record()
        for _ in range(nb):
            moe.moe_backward_saved(cs, weights, inp["x"], dy, full_route, wsf, grads, wsb)
        sv_ev[3].record()
        torch.cuda.synchronize()
        fwd_save_ms = sv_ev[0].elapsed_time(sv_ev[1]) / nb
        bwd_saved_ms = sv_ev[2].elapsed_time(sv_ev[3]) / nb
        del wsb, grads, wsf

    # Sinkhorn routing on the same workload (not part of the step): the
    # balancing runs inside the top-k stage; the per-expert load it gives
    # against the plain top-k's
    sk = None
    if args.routing == "topk" and inp["select_bias"] is None and args.sinkhorn_iters > 0:
        csk = moe.make_cfg(cfg.T, cfg.h, cfg.F, cfg.E, cfg.k, cfg.dtype, cfg.gate, capacity=C,
                           has_shared=cfg.shared, routing="sinkhorn",
                           sinkhorn_iters=args.sinkhorn_iters)
        wsk = torch.empty(moe.moe_workspace_bytes(csk), dtype=torch.uint8, device=dev)
        sk_counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
        for _ in range(2):
            moe.moe_forward(csk, weights, inp["x"], y, {"expert_counts": sk_counts}, wsk)
        nsk = max(3, K // 4)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(nsk):
            moe.moe_forward(csk, weights, inp["x"], y, {"expert_counts": sk_counts}, wsk)
        torch.cuda.synchronize()
        sk_ms = (time.perf_counter() - t1) * 1e3 / nsk
        skev = new_events(nsk)
        torch.cuda.synchronize()
        for i in range(nsk):
            moe.moe_forward(csk, weights, inp["x"], y, {"expert_counts": sk_counts}, wsk,
                            events=skev[i])
        torch.cuda.synchronize()
        skc = sk_counts.cpu().tolist()
        sk = {"iters": args.sinkhorn_iters,
              "ms_per_step": round(sk_ms, 4),
              "topk_stage_ms": round(sum(es[2].elapsed_time(es[3]) for es in skev) / nsk, 5),
              "max_over_mean_load": round(max(skc) * cfg.E / sum(skc), 3)}
        del wsk

    cnt = counts.cpu().tolist()
    kept = sum(min(n, C) for n in cnt) if C else sum(cnt)   # expert choice: E*C
    kept_all = kept + (cfg.T if cfg.shared else 0)
    ms_step = elapsed * 1e3 / K
    g1_ms, g2_ms = stage_ms["gemm1_swiglu"], stage_ms["gemm2"]
    g1 = gemm1_flops(kept_all, cfg.h, cfg.F) / (g1_ms * 1e-3) / 1e12
    g2 = gemm2_flops(kept_all, cfg.h, cfg.F) / (g2_ms * 1e-3) / 1e12
    gg = expert_flops(kept_all, cfg.h, cfg.F) / ((g1_ms + g2_ms) * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    # GEMM 1 is MFMA-bound when its flops per compulsory byte exceed the
    # ridge point peak / HBM bandwidth (312.5 flop/B for bf16), else bound by
    # streaming its weights (few rows per expert)
    kept_e = [min(n, C) for n in cnt] if C else cnt
    # a gathering GEMM 1 reads each token with a kept slot (all of them with
    # a shared expert) once
    in_rows = None
    if gathered_dispatch(cfg.dtype, cfg.T, cfg.h):
        lost = rstats.get("tokens_all_dropped", rstats.get("tokens_no_expert", 0))
        in_rows = cfg.T if cfg.shared else cfg.T - lost
    g1_bytes = gemm1_bytes(kept_e, cfg.T, cfg.h, cfg.F, esz, cfg.shared, in_rows)
    g1_intensity = gemm1_flops(kept_all, cfg.h, cfg.F) / g1_bytes
    hbm_bound = cfg.dtype == "bf16" and g1_intensity < peak / PEAK_HBM_GBS * 1e3
    g1_gbs = g1_bytes / (g1_ms * 1e-3) / 1e9
    pb = permute_bytes(cfg.T, cfg.h, rows, esz)
    if args.routing == "expert_choice":      # a row gather: every row read and written
        pb = 2 * rows * cfg.h * esz
    cb = combine_bytes(kept, cfg.T, cfg.h, esz, cfg.shared)
    rb = router_bytes(cfg.T, cfg.h, cfg.E, esz)
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9          # noqa: E731
    frac = lambda nbytes, ms: round(gbs(nbytes, ms) / PEAK_HBM_GBS, 4)  # noqa: E731
    fcopy = lambda nbytes, ms: (None if copy_gbs is None else    # noqa: E731
                                round(gbs(nbytes, ms) / copy_gbs, 4))

    def hbm_stage(name, nbytes, extra=None):
        if name == "permute" and gathered:
            # no permute kernel in the layer: only the standalone figures
            d = {"kernel_us": None, "in_layer": "gathered by GEMM 1's copies", "bytes": nbytes}
            d.update(extra or {})
            return d
        d = {"kernel_us": round(stage_ms[name] * 1e3, 2),
             "kernel_us_min": round(min(kern[name]) * 1e3, 2),
             "gbs": round(gbs(nbytes, stage_ms[name]), 1), "frac_hbm": frac(nbytes, stage_ms[name]),
             "frac_copy": fcopy(nbytes, stage_ms[name]), "bytes": nbytes}
        if cold is not None:
            cm = cold["stage_ms"][name]
            d.update({"cold_kernel_us": round(cm * 1e3, 2), "cold_frac_hbm": frac(nbytes, cm)})
        if extra:
            d.update(extra)
        return d

    fused_front = fused_router_topk(cfg.dtype, cfg.E, args.routing)
    gathered = gathered_dispatch(cfg.dtype, cfg.T, cfg.h)
    front = ["router", "scan", "assign"] + ([] if fused_front else ["topk"])
    out = {
        "metric": metric_label(cfg.T, cfg.h, cfg.E, cfg.k),
        "value": round(cfg.T * K / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, fan-in-scaled N(0,1/fan_in) random weights)",
        "config": {"workload": _workload_name(cfg, C, args.routing), "routing": args.routing,
                   "T": cfg.T, "h": cfg.h, "E": cfg.E, "k": cfg.k, "F": cfg.F, "capacity": C,
                   "gate": cfg.gate, "kept_rows": kept, "dispatch_rows": rows,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm" if hbm_bound else ("mfma" if cfg.dtype == "bf16" else "alu"),
                     "kernel": "gemm1_swiglu",
                     "achieved": round(g1_gbs if hbm_bound else g1, 1),
                     "peak": PEAK_HBM_GBS if hbm_bound else peak,
                     "unit": "GB/s" if hbm_bound else "TFLOP/s",
                     "frac": round(g1_gbs / PEAK_HBM_GBS if hbm_bound else g1 / peak, 4),
                     "traffic": (measured_traffic(_workload_name(cfg, C))
                                 if args.routing == "topk" else None),
                     "flop_per_byte": round(g1_intensity, 1),
                     "algorithmic_bytes": g1_bytes,
                     "algorithmic_flops": gemm1_flops(kept_all, cfg.h, cfg.F),
                     "kernel_ms": round(g1_ms, 5),
                     "pass": (f"{K} steps after the timed ones, GEMM 1's kernels (grouped GEMM "
                              "+ split-K reduce) timed by start/stop events bound to them")},
        "grouped_gemm": {"tflops": round(gg, 1), "frac_of_peak": round(gg / peak, 4),
                         "gemm1_tflops": round(g1, 1), "gemm2_tflops": round(g2, 1),
                         "gemm1_frac": round(g1 / peak, 4), "gemm2_frac": round(g2 / peak, 4)},
        "routing_stats": rstats,
        "hbm_copy_gbs": None if copy_gbs is None else round(copy_gbs, 1),
        "router": hbm_stage("router", rb),
        "permute": hbm_stage("permute", pb, {
            "standalone_us": None if perm_alone is None else round(perm_alone, 2),
            "standalone_frac_hbm": None if perm_alone is None else frac(pb, perm_alone * 1e-3),
            "standalone_buffer_sets": perm_sets}),
        "combine": hbm_stage("combine", cb, {
            "standalone_us": None if comb_alone is None else round(comb_alone, 2),
            "standalone_frac_hbm": None if comb_alone is None else frac(cb, comb_alone * 1e-3),
            "standalone_buffer_sets": comb_sets}),
        "stage_ms": {k: (None if (k == "topk" and fused_front) or (k == "permute" and gathered)
                         else round(v, 5))
                     for k, v in stage_ms.items()},
        "front_end_kernel_us": round(sum(stage_ms[n] for n in front) * 1e3, 2),
        "router_topk_fused": fused_front,
        "kernel_span_ms": round(kernel_span_ms, 4),
        "backward": (None if bwd is None else {
            "ms": round(bwd, 4),
            # 12*kept*h*F: dgrad and wgrad of both GEMMs; 18*kept*h*F counts
            # the recomputed [a1 | a3] and expert outputs as well
            "tflops": round(12 * kept_all * cfg.h * cfg.F / (bwd * 1e-3) / 1e12, 1),
            "tflops_with_recompute": round(18 * kept_all * cfg.h * cfg.F / (bwd * 1e-3) / 1e12, 1),
            "frac_of_peak": round(18 * kept_all * cfg.h * cfg.F / (bwd * 1e-3) / 1e12 / peak, 4),
            # forward with save_for_backward + moe_backward_saved: no recompute
            "forward_save_ms": round(fwd_save_ms, 4),
            "saved_ms": round(bwd_saved_ms, 4),
            "saved_tflops": round(12 * kept_all * cfg.h * cfg.F / (bwd_saved_ms * 1e-3) / 1e12, 1),
            "saved_frac_of_peak": round(12 * kept_all * cfg.h * cfg.F / (bwd_saved_ms * 1e-3)
                                        / 1e12 / peak, 4)}),
        "cold_cache": cold,
        "sinkhorn": sk,
        "load_balance": {"us": round(lb_us, 2),
                         "max_over_mean_load": round(max(cnt) * cfg.E / sum(cnt), 3),
                         "gbs": round(cfg.T * cfg.E * 4 / (lb_us * 1e-6) / 1e9, 1),
                         "aux_loss": round(float(lb_loss.item()), 6)},
    }
    if not args.no_cpu_baseline and args.routing == "topk":
        out["cpu_baseline"] = cpu_baseline(cfg, inp, C, args.cpu_sample, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
