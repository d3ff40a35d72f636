"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Every pin is a hand-worked fixture under tests/golden/ (with its citation), a
closed form, a special case that reduces to something simpler, or brute
force on tiny inputs.  Each is chosen so that a plausible slip in the oracle
(a transposed operand, a wrong sign, the SiLU on the wrong branch, ranks in
slot order instead of token order, renormalised gates after a drop) fails.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from moe_inputs import CONFIGS, make_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# --------------------------------------------------------------- capacity
def test_capacity_worked_example(golden_dir):
    g = _load(golden_dir, "worked_example.json")
    C = oracle.capacity(g["T"], g["E"], g["k"], g["cf_num"], g["cf_den"])
    assert C == g["capacity"] == 1280


@pytest.mark.parametrize("T,E,k,num,den,C", [
    (10, 4, 1, 1, 1, 3),        # 2.5 rounds up
    (8, 4, 1, 1, 1, 2),         # exact
    (16384, 64, 4, 1, 1, 1024),
    (6, 4, 2, 1, 1, 3),
    (7, 3, 2, 5, 4, 6),         # 70/12 = 5.83 -> 6
])
def test_capacity_closed_form(T, E, k, num, den, C):
    assert oracle.capacity(T, E, k, num, den) == C


# ----------------------------------------------------------------- logits
def test_router_logits_orientation():
    rng = np.random.default_rng(1)
    E, h = 5, 7
    w = rng.standard_normal((E, h)).astype(np.float32)
    x = np.eye(h, dtype=np.float32)[[3, 0, 6]]          # one-hot tokens
    l = oracle.router_logits(x, w)
    assert l.dtype == np.float32 and l.shape == (3, E)
    np.testing.assert_array_equal(l[0], w[:, 3])
    np.testing.assert_array_equal(l[1], w[:, 0])
    np.testing.assert_array_equal(l[2], w[:, 6])
    b = np.arange(E, dtype=np.float32) * 0.5
    np.testing.assert_array_equal(oracle.router_logits(x, w, b)[0],
                                  (w[:, 3] + b).astype(np.float32))


def test_router_logits_rounding_once():
    # sum of 1 + 2^-30 * 4 terms: fp32 accumulation would lose the small
    # terms one by one; fp64 accumulation then one rounding keeps their sum.
    x = np.array([[1.0, 1.0, 1.0, 1.0, 1.0]], dtype=np.float32)
    w = np.array([[1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24]], dtype=np.float32)
    l = oracle.router_logits(x, w)
    assert l[0, 0] == np.float32(1.0 + 4 * 2.0 ** -24)


# ------------------------------------------------------------------ top-k
def _brute_rank(keys_row):
    """Position of each expert in the (key desc, index asc) order, by counting
    the experts that beat it pairwise."""
    E = len(keys_row)
    pos = []
    for a in range(E):
        beaten_by = sum(
            1 for b in range(E)
            if keys_row[b] > keys_row[a] or (keys_row[b] == keys_row[a] and b < a))
        pos.append(beaten_by)
    return pos


@pytest.mark.parametrize("E,k", [(6, 3), (4, 4), (5, 1), (8, 2)])
def test_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    # integer-valued keys from a small range: many exact ties
    keys = rng.integers(-3, 4, size=(300, E)).astype(np.float32)
    idx = oracle.topk(keys, k)
    for t in range(keys.shape[0]):
        pos = _brute_rank(list(keys[t]))
        expect = [pos.index(j) for j in range(k)]
        assert list(idx[t]) == expect
        # the chosen set dominates every subset of the same size
        best = max(itertools.combinations(range(E), k),
                   key=lambda s: (sorted([keys[t][e] for e in s], reverse=True),
                                  [-e for e in s]))
        assert set(idx[t]) == set(best)


def test_topk_ties_and_signed_zero():
    keys = np.array([[0.5, 0.5, 0.5, 0.5],
                     [-0.0, 0.0, -1.0, -0.0],
                     [1.0, 2.0, 2.0, 3.0]], dtype=np.float32)
    idx = oracle.topk(keys, 2)
    assert idx.tolist() == [[0, 1], [0, 1], [3, 1]]


def test_topk_hand_fixture(golden_dir):
    g = _load(golden_dir, "routing_hand.json")
    idx = oracle.topk(np.array(g["keys"], dtype=np.float32), g["k"])
    assert idx.tolist() == g["idx"]


def test_near_tie():
    keys = np.array([[3.0, 1.0, 1.0 + 5e-6, 0.0],
                     [3.0, 1.0, 1.0 + 2e-5, 0.0],
                     [3.0, 2.0, 1.0, 0.0]], dtype=np.float32)
    assert oracle.near_tie(keys, 2).tolist() == [True, False, False]
    assert oracle.near_tie(keys, 4).tolist() == [False, False, False]


# ------------------------------------------------------------------ gates
def test_gates_closed_forms(golden_dir):
    g = _load(golden_dir, "gates_closed_form.json")
    for case in g["cases"]:
        l = np.array([case["logits"]], dtype=np.float32)
        keys = oracle.selection_keys(l, case["select_bias"])
        idx = oracle.topk(keys, case["k"])
        assert idx[0].tolist() == case["idx"], case
        gv = oracle.gates(l, idx, case["mode"])
        np.testing.assert_allclose(gv[0], case["gates"], rtol=0, atol=2e-7, err_msg=str(case))


def test_gate_sums():
    rng = np.random.default_rng(7)
    l = rng.standard_normal((500, 8)).astype(np.float32)
    for k in (1, 2, 3, 8):
        idx = oracle.topk(l, k)
        for mode in ("softmax_topk", "sigmoid_topk_norm"):
            s = oracle.gates(l, idx, mode).astype(np.float64).sum(1)
            np.testing.assert_allclose(s, 1.0, atol=3e-7)
        s_all = oracle.gates(l, idx, "softmax_all_topk").astype(np.float64).sum(1)
        if k < 8:
            assert (s_all < 1.0).all()
        else:
            np.testing.assert_allclose(s_all, 1.0, atol=3e-7)
        if k == 1:
            assert (oracle.gates(l, idx, "softmax_topk") == 1.0).all()
            assert (oracle.gates(l, idx, "sigmoid_topk_norm") == 1.0).all()
        # gates follow slot order: non-increasing for softmax modes
        g = oracle.gates(l, idx, "softmax_topk")
        assert (np.diff(g, axis=1) <= 0).all()


# ----------------------------------------------------------- routing maps
def test_route_maps_hand_fixture(golden_dir):
    g = _load(golden_dir, "routing_hand.json")
    idx = np.array(g["idx"])
    m = oracle.route_maps(idx, g["E"], None)
    assert m["counts"].tolist() == g["counts"]
    assert m["rank"].tolist() == g["rank"]
    assert m["offsets"].tolist() == g["dropless"]["offsets"]
    assert m["assign_row"].tolist() == g["dropless"]["assign_row"]
    assert m["row_token"].tolist() == g["dropless"]["row_token"]
    c = g["capacity"]
    C = oracle.capacity(g["T"], g["E"], g["k"], c["cf_num"], c["cf_den"])
    assert C == c["C"]
    m = oracle.route_maps(idx, g["E"], C)
    assert m["offsets"].tolist() == c["offsets"]
    assert m["kept"].tolist() == c["kept"]
    assert m["assign_row"].tolist() == c["assign_row"]
    assert m["row_token"].tolist() == c["row_token"]


@pytest.mark.parametrize("C", [None, 1, 5, 40])
def test_route_maps_invariants(C):
    rng = np.random.default_rng(3)
    T, E, k = 257, 7, 3
    keys = rng.standard_normal((T, E)).astype(np.float32)
    keys[:, 2] += 1.5                       # one hot expert so drops happen
    idx = oracle.topk(keys, k)
    m = oracle.route_maps(idx, E, C)
    counts, ar, rt = m["counts"], m["assign_row"], m["row_token"]
    assert counts.sum() == T * k
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    kept = ar >= 0
    cap = C if C is not None else T
    assert kept.sum() == np.minimum(counts, cap).sum()
    for e in range(E):
        rows_e = np.sort(ar[(idx == e) & kept])
        lo = m["offsets"][e]
        # the kept rows of an expert are the first places of its group
        assert rows_e.tolist() == list(range(lo, lo + min(counts[e], cap)))
        # the kept tokens are the earliest ones that chose e
        toks = np.nonzero((idx == e).any(1))[0]
        kept_toks = np.nonzero(((idx == e) & kept).any(1))[0]
        assert kept_toks.tolist() == toks[:cap].tolist()
    tt = np.repeat(np.arange(T)[:, None], k, 1)
    assert np.array_equal(rt[ar[kept]], tt[kept])      # row -> token inverts
    assert (rt >= 0).sum() == kept.sum()


# -------------------------------------------------------------- SwiGLU FFN
def test_silu_closed_forms():
    ln3 = math.log(3.0)
    v = oracle.silu(np.array([0.0, ln3, -ln3, 40.0, -40.0]))
    np.testing.assert_allclose(v[:3], [0.0, 0.75 * ln3, -0.25 * ln3], rtol=1e-15, atol=0)
    assert abs(v[3] - 40.0) < 1e-15 * 40 + 1e-15
    assert abs(v[4]) < 1e-15


def test_swiglu_one_hot_weights():
    """Rows of W1, W3, W2 with a single non-zero: each product is a gather, so
    the FFN has a closed form that exposes operand orientation and which
    branch carries the SiLU."""
    h, F = 5, 7
    rng = np.random.default_rng(11)
    p1 = rng.integers(0, h, F)
    p3 = rng.integers(0, h, F)
    p2 = rng.integers(0, F, h)
    a, b, c = 0.7, -1.3, 2.1
    w1 = np.zeros((F, h)); w1[np.arange(F), p1] = a
    w3 = np.zeros((F, h)); w3[np.arange(F), p3] = b
    w2 = np.zeros((h, F)); w2[np.arange(h), p2] = c
    x = rng.standard_normal((3, h))
    y = oracle.swiglu_ffn(x, w1, w3, w2)
    for r in range(3):
        for i in range(h):
            f = p2[i]
            z = a * x[r, p1[f]]
            expect = c * (z / (1.0 + math.exp(-z))) * (b * x[r, p3[f]])
            assert abs(y[r, i] - expect) <= 1e-14 * (1 + abs(expect))


# ------------------------------------------------------------ whole layer
def _rand_layer(T, h, E, F, seed, shared=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, h)).astype(np.float32)
    wr = (rng.standard_normal((E, h)) / math.sqrt(h)).astype(np.float32)
    w1 = (rng.standard_normal((E, F, h)) / math.sqrt(h)).astype(np.float32)
    w3 = (rng.standard_normal((E, F, h)) / math.sqrt(h)).astype(np.float32)
    w2 = (rng.standard_normal((E, h, F)) / math.sqrt(F)).astype(np.float32)
    sh = None
    if shared:
        sh = ((rng.standard_normal((F, h)) / math.sqrt(h)).astype(np.float32),
              (rng.standard_normal((F, h)) / math.sqrt(h)).astype(np.float32),
              (rng.standard_normal((h, F)) / math.sqrt(F)).astype(np.float32))
    return x, wr, w1, w3, w2, sh


def test_e1_k1_is_dense_ffn():
    x, wr, w1, w3, w2, _ = _rand_layer(33, 16, 1, 24, 5)
    for gate in oracle.GATE_MODES:
        out = oracle.moe_forward(x, wr, w1, w3, w2, k=1, gate=gate)
        assert (out["gates"] == 1.0).all()
        np.testing.assert_array_equal(out["y"], oracle.swiglu_ffn(x, w1[0], w3[0], w2[0]))


def test_k_equals_e_is_dense_soft_mixture():
    T, h, E, F = 40, 12, 4, 20
    x, wr, w1, w3, w2, _ = _rand_layer(T, h, E, F, 6)
    out = oracle.moe_forward(x, wr, w1, w3, w2, k=E, gate="softmax_topk")
    # dense mixture: every expert on every token, softmax weights over all E
    l = (x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32).astype(np.float64)
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    dense = sum(p[:, e:e + 1] * oracle.swiglu_ffn(x, w1[e], w3[e], w2[e]) for e in range(E))
    np.testing.assert_allclose(out["y"], dense, rtol=0, atol=1e-6 * np.abs(dense).max())


@pytest.mark.parametrize("gate", ["softmax_topk", "sigmoid_topk_norm"])
def test_identical_experts_give_the_ffn(gate):
    T, h, E, F = 50, 16, 6, 24
    x, wr, w1, w3, w2, _ = _rand_layer(T, h, E, F, 8)
    w1[:] = w1[0]; w3[:] = w3[0]; w2[:] = w2[0]
    out = oracle.moe_forward(x, wr, w1, w3, w2, k=3, gate=gate)
    ffn = oracle.swiglu_ffn(x, w1[0], w3[0], w2[0])
    np.testing.assert_allclose(out["y"], ffn, rtol=0, atol=1e-6 * np.abs(ffn).max())


def test_large_capacity_equals_dropless():
    T, h, E, F, k = 64, 16, 4, 24, 2
    x, wr, w1, w3, w2, _ = _rand_layer(T, h, E, F, 9)
    C = oracle.capacity(T, E, k, E, k)           # cf = E/k  ->  C = T
    assert C == T
    a = oracle.moe_forward(x, wr, w1, w3, w2, k=k, gate="softmax_topk")
    b = oracle.moe_forward(x, wr, w1, w3, w2, k=k, gate="softmax_topk", C=C)
    assert (b["maps"]["assign_row"] >= 0).all()
    np.testing.assert_array_equal(a["y"], b["y"])


def test_dropped_slot_adds_nothing_and_no_renormalisation(golden_dir):
    g = _load(golden_dir, "routing_hand.json")
    T, E, k, h, F = g["T"], g["E"], g["k"], 8, 12
    x, wr, w1, w3, w2, _ = _rand_layer(T, h, E, F, 10)
    idx = np.array(g["idx"], dtype=np.int32)
    C = g["capacity"]["C"]
    out = oracle.moe_forward(x, wr, w1, w3, w2, k=k, gate="softmax_topk", C=C, idx=idx)
    gts = out["gates"].astype(np.float64)
    # token 4: slot 0 (expert 0) dropped, slot 1 (expert 1) kept
    e1 = oracle.swiglu_ffn(x[4:5], w1[1], w3[1], w2[1])[0]
    np.testing.assert_allclose(out["y"][4], gts[4, 1] * e1, rtol=1e-15, atol=0)
    assert gts[4, 1] < 1.0
    # token 5: slot 0 (expert 1, rank 3) dropped, slot 1 (expert 2) kept
    e2 = oracle.swiglu_ffn(x[5:6], w1[2], w3[2], w2[2])[0]
    np.testing.assert_allclose(out["y"][5], gts[5, 1] * e2, rtol=1e-15, atol=0)


def test_all_slots_dropped_gives_zero():
    x, wr, w1, w3, w2, _ = _rand_layer(12, 8, 2, 8, 12)
    out = oracle.moe_forward(x, wr, w1, w3, w2, k=2, gate="softmax_topk", C=3)
    # k = E = 2: every token picks both experts; tokens 3.. are dropped twice
    assert (out["maps"]["assign_row"][3:] == -1).all()
    assert (out["y"][3:] == 0.0).all()
    assert np.abs(out["y"][:3]).max() > 0


def test_shared_expert_is_added_with_weight_one():
    x, wr, w1, w3, w2, sh = _rand_layer(20, 8, 4, 12, 13, shared=True)
    a = oracle.moe_forward(x, wr, w1, w3, w2, k=2, gate="sigmoid_topk_norm")
    b = oracle.moe_forward(x, wr, w1, w3, w2, k=2, gate="sigmoid_topk_norm", shared=sh)
    np.testing.assert_allclose(b["y"] - a["y"], oracle.swiglu_ffn(x, *sh), rtol=0, atol=1e-12)


def test_token_subset_matches_full():
    x, wr, w1, w3, w2, sh = _rand_layer(30, 8, 4, 12, 14, shared=True)
    full = oracle.moe_forward(x, wr, w1, w3, w2, k=2, gate="softmax_topk", C=10, shared=sh)
    tok = np.array([29, 0, 7, 7])
    sub = oracle.moe_forward(x, wr, w1, w3, w2, k=2, gate="softmax_topk", C=10, shared=sh, tokens=tok)
    np.testing.assert_array_equal(sub["y"], full["y"][tok])


def test_permute_then_unpermute_is_identity():
    """k = 1, unit gates: scattering token rows to their group rows and
    gathering them back through the same map returns every token."""
    rng = np.random.default_rng(15)
    T, E, h = 90, 5, 6
    x = rng.standard_normal((T, h))
    idx = rng.integers(0, E, (T, 1))
    for C in (None, 100):
        m = oracle.route_maps(idx, E, C)
        perm = np.zeros((m["rows"], h))
        perm[m["assign_row"][:, 0]] = x
        back = perm[m["assign_row"][:, 0]]
        np.testing.assert_array_equal(back, x)
        pads = m["row_token"] < 0
        assert (perm[pads] == 0).all()


# ---------------------------------------------- worked example dimensions
def test_worked_example_dimension_chain(golden_dir):
    g = _load(golden_dir, "worked_example.json")
    cfg = CONFIGS["worked_example"]
    assert (cfg.T, cfg.h, cfg.E, cfg.k, cfg.F) == (g["T"], g["h"], g["E"], g["k"], g["F"])
    inp = make_inputs(cfg, device="cpu", with_experts=False)
    x = inp["x"].float().numpy()
    wr = inp["w_router"].float().numpy()
    assert list(x.shape) == g["shapes"]["x"]
    C = oracle.capacity(cfg.T, cfg.E, cfg.k, *cfg.cf)
    out = oracle.moe_forward(x, wr, None, None, None, k=cfg.k, gate=cfg.gate, C=C,
                             maps_only=True)
    assert list(out["logits"].shape) == g["shapes"]["router"]
    assert list(out["idx"].shape) == g["shapes"]["topk"]
    assert [cfg.E, out["maps"]["rows"] // cfg.E, cfg.h] == g["shapes"]["dispatch"]
    # each expert FFN: three h x F matrices (about 151M), E of them per layer
    per_expert = 3 * cfg.h * cfg.F
    assert abs(per_expert / g["params_per_expert_approx"] - 1) < 0.01
    assert abs(cfg.E * per_expert / g["params_per_layer_approx"] - 1) < 0.01


# ---------------------------------------------------------------- load balance
def test_load_balance_hand_cases(golden_dir):
    """Hand-worked Switch losses (closed-form probabilities)."""
    g = _load(golden_dir, "load_balance_hand.json")
    for c in g["cases"]:
        lg = np.asarray(c["logits"], dtype=np.float32)
        r = oracle.load_balance(lg, c["counts"], c["k"], c["gate"], c["alpha"])
        np.testing.assert_allclose(r["f"], c["f"], rtol=0, atol=1e-7)
        np.testing.assert_allclose(r["P"], c["P"], rtol=0, atol=1e-7)
        assert abs(float(r["loss"]) - c["loss"]) <= 2e-7 * max(1.0, c["loss"])


@pytest.mark.parametrize("gate", oracle.GATE_MODES)
def test_load_balance_even_load_gives_alpha(gate):
    """Equal logits and equal counts: f = P = 1/E, loss = alpha exactly."""
    T, E, k, alpha = 48, 6, 2, 0.37
    lg = np.full((T, E), 0.8125, dtype=np.float32)
    counts = [T * k // E] * E
    r = oracle.load_balance(lg, counts, k, gate, alpha)
    np.testing.assert_allclose(r["f"], 1.0 / E, rtol=1e-7)
    np.testing.assert_allclose(r["P"], 1.0 / E, rtol=1e-7)
    assert abs(float(r["loss"]) - alpha) <= 1e-7


def test_load_balance_collapse_gives_alpha_times_e():
    """Every token on expert 0 with the router near-certain of it: loss -> alpha*E."""
    T, E, alpha = 40, 8, 0.01
    lg = np.zeros((T, E), dtype=np.float32)
    lg[:, 0] = 60.0
    r = oracle.load_balance(lg, [T] + [0] * (E - 1), 1, "softmax_topk", alpha)
    assert abs(float(r["loss"]) - alpha * E) <= 1e-7 * alpha * E


@pytest.mark.parametrize("gate", oracle.GATE_MODES)
def test_load_balance_invariants(gate):
    """sum f = sum P = 1; for k = E every expert is selected by every token, so
    T*P_i equals the sum of the softmax-over-all gates of expert i."""
    rng = np.random.default_rng(5)
    T, E = 37, 5
    lg = rng.normal(0, 2, (T, E)).astype(np.float32)
    idx = oracle.topk(lg, E)
    counts = np.bincount(idx.ravel(), minlength=E)
    r = oracle.load_balance(lg, counts, E, gate, 1.0)
    assert abs(float(r["f"].astype(np.float64).sum()) - 1.0) <= 1e-6
    assert abs(float(r["P"].astype(np.float64).sum()) - 1.0) <= 1e-6
    if gate == "softmax_all_topk":
        g = oracle.gates(lg, idx, gate).astype(np.float64)
        per_e = np.zeros(E)
        np.add.at(per_e, idx.ravel(), g.ravel())
        np.testing.assert_allclose(r["P"], per_e / T, rtol=1e-6)


# ----------------------------------------------------------- routing variants
def test_routing_variants_hand_cases(golden_dir):
    g = _load(golden_dir, "routing_variants_hand.json")
    sd = g["score_drop"]
    m = oracle.route_maps_score_drop(np.array(sd["idx"]), np.array(sd["gates"], dtype=np.float32),
                                     sd["E"], sd["C"])
    assert m["assign_row"].tolist() == sd["assign_row"]
    assert m["row_token"].tolist() == sd["row_token"]
    assert m["counts"].tolist() == sd["counts"]
    ec = g["expert_choice"]
    m = oracle.expert_choice(np.array(ec["logits"], dtype=np.float32), ec["C"], ec["gate"])
    assert m["sel_row"].tolist() == ec["sel_row"]
    assert m["row_token"].tolist() == ec["row_token"]
    np.testing.assert_allclose(m["gate"], ec["gate_values"], rtol=0, atol=1e-7)


def _brute_keep(values, C):
    """Keep i iff fewer than C others beat it (larger value, or equal value
    and earlier position)."""
    n = len(values)
    return [sum(1 for i2 in range(n) if values[i2] > values[i] or
                (values[i2] == values[i] and i2 < i)) < C for i in range(n)]


@pytest.mark.parametrize("seed", range(4))
def test_score_drop_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E, k, C = 23, 4, 2, 4
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    g = np.round(rng.random((T, k)), 1).astype(np.float32)     # coarse: many ties
    m = oracle.route_maps_score_drop(idx, g, E, C)
    for e in range(E):
        cand = [(t, j) for t in range(T) for j in range(k) if idx[t, j] == e]
        keep = _brute_keep([float(g[c]) for c in cand], C)
        kept = [c for c, kp in zip(cand, keep) if kp]
        for r, (t, j) in enumerate(kept):          # token order
            assert m["assign_row"][t, j] == e * C + r
            assert m["row_token"][e * C + r] == t
        for c, kp in zip(cand, keep):
            if not kp:
                assert m["assign_row"][c] == -1


def test_score_drop_reduces_to_token_order():
    """Equal gates (k = 1 softmax over the selected one is always 1.0) and a
    capacity that nothing overflows both give the token-order maps."""
    rng = np.random.default_rng(9)
    T, E = 50, 5
    idx = rng.integers(0, E, (T, 1))
    ones = np.ones((T, 1), dtype=np.float32)
    for C in (3, 7, 50):
        a = oracle.route_maps_score_drop(idx, ones, E, C)
        b = oracle.route_maps(idx, E, C)
        assert np.array_equal(a["assign_row"], b["assign_row"])
        assert np.array_equal(a["row_token"], b["row_token"])
    g = rng.random((T, 1)).astype(np.float32)
    a = oracle.route_maps_score_drop(idx, g, E, T)
    b = oracle.route_maps(idx, E, T)
    assert np.array_equal(a["assign_row"], b["assign_row"])


@pytest.mark.parametrize("gate", oracle.GATE_MODES)
def test_expert_choice_matches_brute_force(gate):
    rng = np.random.default_rng(3)
    T, E, C = 19, 3, 5
    lg = np.round(rng.normal(0, 1, (T, E)), 1).astype(np.float32)
    m = oracle.expert_choice(lg, C, gate)
    p = m["scores"]
    for e in range(E):
        keep = _brute_keep([float(v) for v in p[:, e]], C)
        chosen = [t for t in range(T) if keep[t]]
        assert len(chosen) == C
        for r, t in enumerate(chosen):
            assert m["sel_row"][t, e] == e * C + r
            assert m["row_token"][e * C + r] == t
            assert m["gate"][t, e] == p[t, e]
        assert all(m["sel_row"][t, e] == -1 and m["gate"][t, e] == 0 for t in range(T)
                   if not keep[t])


def test_expert_choice_all_tokens_is_dense_soft_mixture():
    """C = T: every expert takes every token with its softmax probability,
    which is token choice with k = E and the softmax-over-all gates."""
    rng = np.random.default_rng(4)
    T, h, E, F = 9, 8, 3, 6
    x = rng.normal(0, 1, (T, h)).astype(np.float32)
    wr = rng.normal(0, 0.5, (E, h)).astype(np.float32)
    w1 = rng.normal(0, 0.3, (E, F, h)).astype(np.float32)
    w3 = rng.normal(0, 0.3, (E, F, h)).astype(np.float32)
    w2 = rng.normal(0, 0.3, (E, h, F)).astype(np.float32)
    ec = oracle.expert_choice_forward(x, wr, w1, w3, w2, C=T, gate="softmax_all_topk")
    tc = oracle.moe_forward(x, wr, w1, w3, w2, k=E, gate="softmax_all_topk")
    # the same gate values reach each expert output; sums differ only by order
    np.testing.assert_allclose(ec["y"], tc["y"], rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------------- backward
def _tiny_layer(seed, shared=False, T=6, h=5, E=3, F=4):
    rng = np.random.default_rng(seed)
    p = {"x": rng.normal(0, 1, (T, h)), "w_router": rng.normal(0, 1.0, (E, h)),
         "w1": rng.normal(0, 0.5, (E, F, h)), "w3": rng.normal(0, 0.5, (E, F, h)),
         "w2": rng.normal(0, 0.5, (E, h, F)), "logit_bias": rng.normal(0, 0.3, E)}
    if shared:
        p["ws1"] = rng.normal(0, 0.5, (F, h))
        p["ws3"] = rng.normal(0, 0.5, (F, h))
        p["ws2"] = rng.normal(0, 0.5, (h, F))
    dy = rng.normal(0, 1, (T, h))
    return p, dy


def _loss(p, dy, **kw):
    sh = (p["ws1"], p["ws3"], p["ws2"]) if "ws1" in p else None
    y = oracle.moe_forward(p["x"], p["w_router"], p["w1"], p["w3"], p["w2"],
                           logit_bias=p["logit_bias"], shared=sh, **kw)["y"]
    return float((y * dy).sum())


@pytest.mark.parametrize("gate,C,drop,shared", [
    ("softmax_topk", None, "token", False),
    ("softmax_all_topk", 3, "token", False),
    ("sigmoid_topk_norm", None, "token", True),
    ("softmax_topk", 3, "score", False),
])
def test_backward_matches_finite_differences(gate, C, drop, shared):
    """Every gradient of the oracle's backward against central differences
    of sum(y * dy) through the oracle's forward, on a tiny layer whose
    top-k choice and drops do not move under the perturbation."""
    kw = dict(k=2, gate=gate, C=C, drop=drop)
    for seed in range(11, 60):       # first layer whose top-2 keys are well apart
        p, dy = _tiny_layer(seed, shared)
        fwd = oracle.moe_forward(p["x"], p["w_router"], p["w1"], p["w3"], p["w2"],
                                 logit_bias=p["logit_bias"], maps_only=True, **kw)
        srt = -np.sort(-fwd["keys"].astype(np.float64), axis=1)
        if (srt[:, 1] - srt[:, 2]).min() > 0.02:          # routing stays put
            break
    else:
        raise AssertionError("no well-separated layer")
    sh = (p["ws1"], p["ws3"], p["ws2"]) if shared else None
    g = oracle.moe_backward(p["x"], p["w_router"], p["w1"], p["w3"], p["w2"], dy,
                            logit_bias=p["logit_bias"], shared=sh, **kw)
    if C is not None:
        assert (g["maps"]["assign_row"] < 0).any()          # the drop path is exercised
    names = {"x": "dx", "w_router": "dw_router", "w1": "dw1", "w3": "dw3", "w2": "dw2",
             "logit_bias": "dlogit_bias"}
    if shared:
        names.update({"ws1": "dws1", "ws3": "dws3", "ws2": "dws2"})
    eps = 1e-3
    for name, gname in names.items():
        grad = g[gname]
        fd = np.zeros_like(grad)
        for i in np.ndindex(grad.shape):
            old = p[name][i]
            p[name][i] = old + eps
            lp = _loss(p, dy, **kw)
            p[name][i] = old - eps
            lm = _loss(p, dy, **kw)
            p[name][i] = old
            fd[i] = (lp - lm) / (2 * eps)
        scale = max(1.0, float(np.abs(fd).max()))
        assert float(np.abs(fd - grad).max()) <= 2e-3 * scale, name


def _ec_loss(p, dy, C, gate):
    sh = (p["ws1"], p["ws3"], p["ws2"]) if "ws1" in p else None
    y = oracle.expert_choice_forward(p["x"], p["w_router"], p["w1"], p["w3"], p["w2"], C=C,
                                     gate=gate, logit_bias=p["logit_bias"], shared=sh)["y"]
    return float((y * dy).sum())


@pytest.mark.parametrize("gate,shared", [("softmax_all_topk", False),
                                         ("sigmoid_topk_norm", True)])
def test_expert_choice_backward_matches_finite_differences(gate, shared):
    """Every gradient of the oracle's expert-choice backward against central
    differences of sum(y * dy) through the oracle's expert-choice forward,
    on a tiny layer whose choices do not move under the perturbation (the
    C-th and (C+1)-th scores of every expert well apart)."""
    C = 2
    for seed in range(21, 200):
        p, dy = _tiny_layer(seed, shared)
        lg = oracle.router_logits(p["x"], p["w_router"], p["logit_bias"])
        sc = -np.sort(-oracle.router_probs(lg, gate), axis=0)
        if (sc[C - 1] - sc[C]).min() > 0.01:
            break
    else:
        raise AssertionError("no well-separated layer")
    sh = (p["ws1"], p["ws3"], p["ws2"]) if shared else None
    g = oracle.expert_choice_backward(p["x"], p["w_router"], p["w1"], p["w3"], p["w2"], dy, C=C,
                                      gate=gate, logit_bias=p["logit_bias"], shared=sh)
    # some token is chosen by several experts and some by none
    n_chosen = (g["maps"]["sel_row"] >= 0).sum(axis=1)
    assert n_chosen.max() >= 2 and n_chosen.min() == 0
    names = {"x": "dx", "w_router": "dw_router", "w1": "dw1", "w3": "dw3", "w2": "dw2",
             "logit_bias": "dlogit_bias"}
    if shared:
        names.update({"ws1": "dws1", "ws3": "dws3", "ws2": "dws2"})
    eps = 1e-3
    for name, gname in names.items():
        grad = g[gname]
        fd = np.zeros_like(grad)
        for i in np.ndindex(grad.shape):
            old = p[name][i]
            p[name][i] = old + eps
            lp = _ec_loss(p, dy, C, gate)
            p[name][i] = old - eps
            lm = _ec_loss(p, dy, C, gate)
            p[name][i] = old
            fd[i] = (lp - lm) / (2 * eps)
        scale = max(1.0, float(np.abs(fd).max()))
        assert float(np.abs(fd - grad).max()) <= 2e-3 * scale, name


def test_backward_gate_gradient_is_the_output_dot():
    """k = 1 with softmax over the selected expert: the gate is 1 whatever
    the logits, so the router gets no gradient at all."""
    p, dy = _tiny_layer(12)
    g = oracle.moe_backward(p["x"], p["w_router"], p["w1"], p["w3"], p["w2"], dy, k=1,
                            gate="softmax_topk", logit_bias=p["logit_bias"])
    assert np.abs(g["dlogits"]).max() == 0.0
    assert np.abs(g["dw_router"]).max() == 0.0


def test_backward_rows_match_full_backward():
    """The token-by-token path gives the full backward's rows."""
    p, dy = _tiny_layer(13, shared=True, T=9)
    sh = (p["ws1"], p["ws3"], p["ws2"])
    kw = dict(k=2, gate="softmax_all_topk", C=4, logit_bias=p["logit_bias"], shared=sh)
    full = oracle.moe_backward(p["x"], p["w_router"], p["w1"], p["w3"], p["w2"], dy, **kw)
    tok = np.array([7, 0, 3])
    part = oracle.moe_backward(p["x"], p["w_router"], p["w1"], p["w3"], p["w2"], dy, tokens=tok,
                               **kw)
    for key in ("dx", "dgate", "dlogits"):
        np.testing.assert_allclose(part[key], full[key][tok], rtol=1e-12, atol=1e-12)


# ---- Sinkhorn routing (Megatron-LM part 6, load-balancing table, sinkhorn row)

def test_sinkhorn_two_by_two_limit():
    """Closed form: scaling rows and columns of [[p, q], [r, s]] keeps the
    cross ratio ps/(qr), so the doubly stochastic limit is [[x, 1-x],
    [1-x, x]] with x/(1-x) = sqrt(ps/(qr))."""
    p, q, r, s = 3.0, 0.5, 1.2, 2.0
    m = oracle.sinkhorn(np.log([[p, q], [r, s]]), 400)
    x = math.sqrt(p * s) / (math.sqrt(p * s) + math.sqrt(q * r))
    np.testing.assert_allclose(m["P"], [[x, 1 - x], [1 - x, x]], atol=1e-12)


def test_sinkhorn_rank_one_is_uniform_after_one_iteration():
    """l[t,e] = a_t + b_e: one row scaling leaves e^{b_e}/Z in every row; the
    column scaling then makes every entry 1/E, and its factors undo b."""
    rng = np.random.default_rng(5)
    a, b = rng.normal(size=7), 2 * rng.normal(size=3)
    m = oracle.sinkhorn(a[:, None] + b[None, :], 1)
    np.testing.assert_allclose(m["P"], np.full((7, 3), 1 / 3), rtol=1e-12)
    assert np.ptp(m["bias"].astype(np.float64) + b) < 1e-5


def test_sinkhorn_marginals_and_form():
    """Columns sum to T/E after every iteration, rows to 1 at convergence,
    and the result is diag(r) exp(l) diag(col)."""
    rng = np.random.default_rng(11)
    T, E = 40, 6
    l = 2 * rng.normal(size=(T, E))
    np.testing.assert_allclose(oracle.sinkhorn(l, 1)["P"].sum(0), np.full(E, T / E), rtol=1e-12)
    m = oracle.sinkhorn(l, 300)
    np.testing.assert_allclose(m["P"].sum(1), 1.0, atol=1e-9)
    np.testing.assert_allclose(m["P"].sum(0), T / E, rtol=1e-12)
    R = m["P"] / (np.exp(l) * m["col"][None, :])
    np.testing.assert_allclose(R, np.repeat(R[:, :1], E, axis=1), rtol=1e-12)


def test_sinkhorn_cancels_expert_offsets():
    """Adding c_e to column e of the logits leaves the balanced matrix, and
    so the selection, unchanged at convergence; the bias absorbs -c_e."""
    rng = np.random.default_rng(3)
    l, c = rng.normal(size=(64, 8)), 3 * rng.normal(size=8)
    m0, m1 = oracle.sinkhorn(l, 500), oracle.sinkhorn(l + c, 500)
    np.testing.assert_allclose(m1["P"], m0["P"], atol=1e-9)
    assert np.ptp(np.log(m1["col"]) - np.log(m0["col"]) + c) < 1e-9


def test_sinkhorn_topk_ranks_the_balanced_matrix():
    """The top-k of selection_keys(l, bias) is the top-k of the rows of P."""
    rng = np.random.default_rng(8)
    l = (rng.normal(size=(300, 16)) + np.linspace(0, 3, 16)).astype(np.float32)
    m = oracle.sinkhorn(l, 20)
    keys = oracle.selection_keys(l, m["bias"])
    k = 3
    ok = ~oracle.near_tie(keys, k, 1e-4)
    assert ok.mean() > 0.95
    via_p = np.argsort(-m["P"], axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(oracle.topk(keys, k)[ok], via_p[ok])


def test_sinkhorn_evens_out_a_skewed_router():
    """Zipf-biased logits send several times the mean load to the hottest
    expert under plain top-k; after balancing every load is near the mean."""
    rng = np.random.default_rng(1)
    T, E, k = 4096, 16, 2
    l = (rng.normal(size=(T, E)) - 1.2 * np.log(np.arange(E) + 1)).astype(np.float32)
    mean = T * k / E
    plain = np.bincount(oracle.topk(l, k).ravel(), minlength=E)
    assert plain.max() > 3 * mean
    m = oracle.sinkhorn(l, 50)
    bal = np.bincount(oracle.topk(oracle.selection_keys(l, m["bias"]), k).ravel(), minlength=E)
    assert 0.75 * mean < bal.min() and bal.max() < 1.25 * mean


def test_moe_forward_sinkhorn_route():
    """moe_forward with Sinkhorn routing selects on the balanced keys; the
    gates still come from the logits of the selected experts."""
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg, device="cpu")
    a = [inp[n].float().numpy() for n in ("x", "w_router", "w1", "w3", "w2")]
    out = oracle.moe_forward(*a, k=cfg.k, gate=cfg.gate, sinkhorn_iters=5, maps_only=True)
    bias = oracle.sinkhorn(out["logits"], 5)["bias"]
    np.testing.assert_array_equal(out["sinkhorn_bias"], bias)
    np.testing.assert_array_equal(out["idx"], oracle.topk(oracle.selection_keys(out["logits"], bias), cfg.k))
    np.testing.assert_array_equal(out["gates"], oracle.gates(out["logits"], out["idx"], cfg.gate))
    with pytest.raises(ValueError):
        oracle.moe_forward(*a, k=cfg.k, gate=cfg.gate, sinkhorn_iters=5,
                           select_bias=np.zeros(cfg.E, np.float32), maps_only=True)


# ------------------------------------------------------------ aux-loss-free selection bias
def test_select_bias_update_hand_case():
    """T*k = 12 assignments over E = 4 experts (mean 3): loads 5, 3, 2, 2 give
    the steps -1/8, 0, +1/8, +1/8, worked by hand."""
    b = np.array([0.5, -0.25, 0.0, 1.0], np.float32)
    out = oracle.select_bias_update(b, [5, 3, 2, 2], T=6, k=2, gamma=0.125)
    np.testing.assert_array_equal(out, np.array([0.375, -0.25, 0.125, 1.125], np.float32))
    np.testing.assert_array_equal(b, [0.5, -0.25, 0.0, 1.0])      # input untouched


def test_select_bias_update_fractional_mean_and_rounding():
    """Mean 10/4 = 2.5 is never hit, so every expert moves; the step is one fp32
    addition (1 + 2^-30 rounds back to 1 in fp32)."""
    out = oracle.select_bias_update(np.ones(4, np.float32), [3, 2, 3, 2], T=5, k=2,
                                    gamma=2.0 ** -30)
    np.testing.assert_array_equal(out, np.ones(4, np.float32))
    out = oracle.select_bias_update(np.zeros(4, np.float32), [3, 2, 3, 2], T=5, k=2, gamma=0.5)
    np.testing.assert_array_equal(out, [-0.5, 0.5, -0.5, 0.5])


def test_select_bias_update_even_load_keeps_every_bit():
    b = np.array([-0.0, 0.1, -3.5, 7.25e-8], np.float32)
    out = oracle.select_bias_update(b, [6, 6, 6, 6], T=8, k=3, gamma=0.01)
    np.testing.assert_array_equal(out.view(np.uint32), b.view(np.uint32))


def test_select_bias_update_evens_out_a_skewed_router():
    """The sign convention closes the loop: routing a Zipf-skewed router on
    its logits plus the bias, then updating the bias from that routing's
    loads, brings the hottest expert from several times the mean load to
    near it; a flipped sign would make the skew worse."""
    rng = np.random.default_rng(3)
    T, E, k, gamma = 2048, 16, 2, 0.02
    l = (rng.normal(size=(T, E)) - 1.2 * np.log(np.arange(E) + 1)).astype(np.float32)
    mean = T * k / E
    b = np.zeros(E, np.float32)
    first = None
    for _ in range(200):
        counts = np.bincount(oracle.topk(oracle.selection_keys(l, b), k).ravel(), minlength=E)
        first = counts if first is None else first
        b = oracle.select_bias_update(b, counts, T, k, gamma)
    assert first.max() > 3 * mean
    assert counts.max() < 1.25 * mean and counts.min() > 0.75 * mean
