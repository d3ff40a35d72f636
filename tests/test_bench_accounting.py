"""The benchmark's work accounting (the numerators of its roofline figures)
pinned to the numbers the worked example prints (infra-l7 page, "EP"
section: about 6.2 ms of expert compute at an assumed 400 TFLOPS, and a
64 MiB dispatch payload, for T=4096, h=4096, E=8, k=2 with the
Qwen3-8B-sized SwiGLU expert F=12288 of its "MoE:参数很多" section).
CPU only."""
import json
import os

import bench


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        return json.load(f)


def test_expert_flops_match_the_pages_estimate(golden_dir):
    g = _golden(golden_dir)
    T, h, k, F = g["T"], g["h"], g["k"], g["F"]
    flops = bench.expert_flops(T * k, h, F)
    assert flops == 6 * T * k * h * F == 2473901162496
    # 6.2 ms at 400 TFLOPS, to the two digits the page prints
    est = g["expert_compute_ms_at_400tflops_approx"] * 1e-3 * 400e12
    assert abs(flops - est) / est < 0.005
    assert round(flops / 400e12 * 1e3, 1) == g["expert_compute_ms_at_400tflops_approx"]
    # GEMM 1 (w1 and w3) is two thirds of it, GEMM 2 (w2) one third
    assert bench.gemm1_flops(T * k, h, F) == 2 * bench.gemm2_flops(T * k, h, F)


def test_dispatch_payload_is_64_mib(golden_dir):
    g = _golden(golden_dir)
    T, h, k = g["T"], g["h"], g["k"]
    payload = bench.dispatch_payload_bytes(T, k, h, 2)
    assert payload == g["dispatch_payload_mib"] << 20
    # the permute of a dropless dispatch reads x once and writes the payload
    assert bench.permute_bytes(T, h, T * k, 2) == T * h * 2 + payload
    # combine reads the payload back and writes y
    assert bench.combine_bytes(T * k, T, h, 2, shared=False) == payload + T * h * 2
    # the capacity layout writes E*C rows, padding included
    assert bench.permute_bytes(T, h, g["E"] * g["capacity"], 2) == (T + 10240) * h * 2


def test_gemm1_bytes_and_bound():
    # worked example: 8 experts of ~1024 rows are far above the ridge point
    # (2.5 PF / 8 TB/s = 312.5 flop/B); the DeepSeek-V3 shape (256 experts of
    # ~128 rows + a shared expert) is below it
    T, h, F = 4096, 4096, 12288
    rows = [1024] * 8
    b = bench.gemm1_bytes(rows, T, h, F, 2, shared=False)
    assert b == (2 * 8 * F * h + 8192 * h + 8192 * F) * 2
    assert bench.gemm1_flops(8192, h, F) / b > 312.5
    T, h, F = 4096, 7168, 2048
    rows = [128] * 256
    b = bench.gemm1_bytes(rows, T, h, F, 2, shared=True)
    assert b == (2 * 257 * F * h + (32768 + T) * h + (32768 + T) * F) * 2
    assert bench.gemm1_flops(32768 + T, h, F) / b < 312.5
    # gathering the rows from the tokens reads each token once
    bg = bench.gemm1_bytes(rows, T, h, F, 2, shared=True, in_rows=T)
    assert b - bg == 32768 * h * 2


def test_metric_label_follows_the_workload():
    assert bench.metric_label(4096, 4096, 8, 2) == (
        "MoE-layer fwd tokens/s and grouped-GEMM TFLOPS (% MFMA peak), T=4096 h=4096 E=8 k=2")
    assert bench.metric_label(4096, 7168, 256, 8).endswith("T=4096 h=7168 E=256 k=8")


def test_routing_stats_counts():
    import numpy as np
    # token 0: keys 3, 1, 1-5e-6 -> k=2 gap 5e-6: a near tie; token 1: clear
    logits = np.array([[3.0, 1.0, 1.0 - 5e-6], [0.0, 2.0, 5.0]], dtype=np.float32)
    assign = np.array([0, -1, -1, -1], dtype=np.int32)
    st = bench.routing_stats(logits, None, assign, 2)
    assert st == {"near_ties": 1, "dropped_assignments": 3, "tokens_all_dropped": 1}
    # a selection bias moves the keys apart
    st = bench.routing_stats(logits, np.array([0.0, 0.5, 0.0], dtype=np.float32), assign, 2)
    assert st["near_ties"] == 0


def test_committed_traffic_summaries_are_keyed_to_their_workload():
    # every committed FETCH_SIZE/WRITE_SIZE summary names its workload, the
    # kernel source it was taken on and plausible byte counts; bench.py
    # reports its traffic only for that workload and that source
    import glob
    files = glob.glob(os.path.join(bench.ROOT, "profiles", "grouped_gemm_traffic_*.txt"))
    assert files
    for f in files:
        w = os.path.basename(f)[len("grouped_gemm_traffic_"):-len(".txt")]
        assert bench.traffic_file(f"{w}: T=1") == f
        kv = bench._machine_fields(f)
        assert kv["workload"] == w
        assert len(kv["kernel_source_sha256_16"]) == 16
        comp, meas = int(kv["gemm1_compulsory_bytes"]), int(kv["gemm1_hbm_bytes_per_launch"])
        # the counters never read less than the compulsory bytes (within
        # the calibration's rounding)
        assert meas > 0.98 * comp > 0
        if kv["kernel_source_sha256_16"] == bench.source_hash(bench.GEMM_SOURCE):
            assert bench.measured_traffic(f"{w}: T=1") == meas
        else:
            assert bench.measured_traffic(f"{w}: T=1") is None
    assert bench.measured_traffic("no_such_workload: T=1") is None
