"""Pins of the CPU oracle to things other than itself: hand-worked cases, closed forms,
brute force on tiny inputs, invariants and special cases. CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def logistic(z):
    return 1.0 / (1.0 + math.exp(-z))


# ------------------------------------------------------------------ hand-worked route
def test_hand_route_case():
    g = GOLD["route"]
    L = O.gate_logits(np.array(g["x"]), np.array(g["w_router"]))
    np.testing.assert_array_equal(L, np.array(g["expected_logits"]))
    idx, flags = O.select_experts(L, g["top_k"])
    assert flags == 0
    np.testing.assert_array_equal(idx, np.array(g["expected_idx"]))
    w = O.topk_weights(L, idx, renormalize=True)
    want = np.array([[logistic(z) for z in row] for row in g["weights_logistic_args"]])
    np.testing.assert_allclose(w, want, rtol=1e-15, atol=0)


def test_hand_capacity_case():
    g, c = GOLD["route"], GOLD["capacity"]
    L = O.gate_logits(np.array(g["x"]), np.array(g["w_router"]))
    idx, _ = O.select_experts(L, 2)
    cap = O.capacity(c["capacity_factor"], 2, 2, 3)
    assert cap == c["expected_capacity"]
    p = O.permute_indices(idx, 3, cap)
    for key in ("counts", "kept", "offsets", "row_token", "slot_row"):
        np.testing.assert_array_equal(p[key], np.array(c["expected_" + key]), err_msg=key)
    assert p["flags"] == 0


# ------------------------------------------------------------------ brute-force top-k
def _beats(a, b, ia, ib):
    """Does (value a, index ia) rank ahead of (b, ib)? NaN lowest, lower index wins ties."""
    na, nb = math.isnan(a), math.isnan(b)
    if na and nb:
        return ia < ib
    if na:
        return False
    if nb:
        return True
    if a == b:
        return ia < ib
    return a > b


def brute_topk(L, k):
    T, E = L.shape
    out = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for e in range(E):
            rank = sum(1 for f in range(E) if f != e and _beats(L[t, f], L[t, e], f, e))
            if rank < k:
                out[t, rank] = e
    return out


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E = 40, 9
    if seed % 2 == 0:
        L = rng.standard_normal((T, E))
    else:  # tie-heavy, with signed zeros, infinities and NaN
        pool = np.array([-1.0, -0.0, 0.0, 1.0, 2.0, np.inf, -np.inf, np.nan])
        L = pool[rng.integers(0, len(pool), (T, E))]
    for k in (1, 2, 3, E):
        idx, flags = O.select_experts(L, k)
        np.testing.assert_array_equal(idx, brute_topk(L, k))
        assert ((idx >= 0) & (idx < E)).all()
        assert bool(flags & O.FLAG_NONFINITE_LOGIT) == (not np.isfinite(L).all())


def test_signed_zero_ties_by_index():
    L = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]])
    idx, _ = O.select_experts(L, 1)
    np.testing.assert_array_equal(idx[:, 0], [0, 0])


def test_zero_router_selects_first_k_with_equal_weights():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 8))
    for E, k in ((4, 2), (8, 3), (5, 5)):
        L = O.gate_logits(x, np.zeros((8, E)))
        idx, _ = O.select_experts(L, k)
        np.testing.assert_array_equal(idx, np.tile(np.arange(k), (16, 1)))
        np.testing.assert_allclose(O.topk_weights(L, idx, True), 1.0 / k, rtol=1e-15)


# ------------------------------------------------------------------ weights
def test_weight_invariants():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((50, 7)) * 3
    for k in (1, 2, 4, 7):
        idx, _ = O.select_experts(L, k)
        w = O.topk_weights(L, idx, True)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
        assert (np.diff(w, axis=1) <= 0).all()          # slots are in descending weight
    idx, _ = O.select_experts(L, 1)
    np.testing.assert_array_equal(O.topk_weights(L, idx, True), 1.0)
    idx, _ = O.select_experts(L, 7)
    np.testing.assert_allclose(O.topk_weights(L, idx, False).sum(1), 1.0, atol=1e-15)
    # two experts without renormalisation: the softmax probability is logistic(L0 - L1)
    L2 = np.array([[0.7, -1.3]])
    idx, _ = O.select_experts(L2, 1)
    assert O.topk_weights(L2, idx, False)[0, 0] == pytest.approx(logistic(2.0), rel=1e-15)


def test_nonfinite_weights_are_nan():
    L = np.array([[np.nan, 1.0, 0.0], [np.inf, 1.0, 0.0], [-np.inf, -np.inf, -np.inf]])
    idx, flags = O.select_experts(L, 2)
    assert flags & O.FLAG_NONFINITE_LOGIT
    np.testing.assert_array_equal(idx, [[1, 2], [0, 1], [0, 1]])
    assert np.isnan(O.topk_weights(L, idx, True)).all()


# ------------------------------------------------------------------ capacity
def test_capacity_formula():
    assert O.capacity(1.2, 8192, 2, 32) == 615           # ceil(614.4)
    assert O.capacity(1.0, 8192, 2, 32) == 512           # exact: no spurious round-up
    assert O.capacity(0.0, 100, 2, 8) == 100
    assert O.capacity(-1.0, 100, 2, 8) == 100
    assert O.capacity(1.25, 10, 1, 4) == 4               # ceil(3.125)


def sequential_permute(idx, E, cap):
    """Walk tokens in order with one counter per expert (a second, independent algorithm)."""
    T, k = idx.shape
    lists = [[] for _ in range(E)]
    counts = [0] * E
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(idx[t, j])
            if e < 0 or e >= E or e in seen:
                continue
            seen.add(e)
            counts[e] += 1
            if len(lists[e]) < cap:
                lists[e].append((t, j))
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + len(lists[e]))
    slot_row = -np.ones((T, k), dtype=np.int64)
    row_token = []
    for e in range(E):
        for r, (t, j) in enumerate(lists[e]):
            slot_row[t, j] = offsets[e] + r
            row_token.append(t)
    return np.array(counts), np.array(offsets), slot_row, np.array(row_token, dtype=np.int64)


@pytest.mark.parametrize("seed", range(5))
def test_permute_matches_sequential_walk(seed):
    rng = np.random.default_rng(10 + seed)
    T, E, k = 200, 6, 2
    L = rng.standard_normal((T, E)) + np.array([2.0, 1.0, 0, 0, -1, -2])
    idx, _ = O.select_experts(L, k)
    for cap in (1, 7, 50, 67, T):
        p = O.permute_indices(idx, E, cap)
        counts, offsets, slot_row, row_token = sequential_permute(idx, E, cap)
        np.testing.assert_array_equal(p["counts"], counts)
        np.testing.assert_array_equal(p["offsets"], offsets)
        np.testing.assert_array_equal(p["slot_row"], slot_row)
        np.testing.assert_array_equal(p["row_token"], row_token)
        assert p["counts"].sum() == T * k
        np.testing.assert_array_equal(p["kept"], np.minimum(counts, cap))


def test_invalid_and_repeated_ids_are_dropped_and_flagged():
    idx = np.array([[0, 5], [1, 1], [-1, 2], [2, 0]])
    p = O.permute_indices(idx, 3, 10)
    assert p["flags"] & O.FLAG_BAD_INDEX
    counts, offsets, slot_row, row_token = sequential_permute(idx, 3, 10)
    np.testing.assert_array_equal(p["slot_row"], slot_row)
    np.testing.assert_array_equal(p["counts"], [2, 1, 2])
    assert (p["slot_row"][[0, 1, 2], [1, 1, 0]] == -1).all()


# ------------------------------------------------------------------ permutation
def test_permutation_invariants_and_unpermute_identity():
    rng = np.random.default_rng(3)
    T, H, E, k = 120, 5, 8, 3
    x = rng.standard_normal((T, H))
    L = rng.standard_normal((T, E))
    idx, _ = O.select_experts(L, k)
    for cap in (T, 20):
        p = O.permute_indices(idx, E, cap)
        sr, rt, off = p["slot_row"], p["row_token"], p["offsets"]
        t_of = np.repeat(np.arange(T)[:, None], k, 1)
        m = sr >= 0
        np.testing.assert_array_equal(rt[sr[m]], t_of[m])
        for e in range(E):
            seg = rt[off[e]:off[e + 1]]
            assert (np.diff(seg) > 0).all()
            assert (idx[seg] == e).any(axis=1).all()
        x_perm = O.gather_rows(x, rt)
        back = O.combine(x_perm, sr, np.ones((T, k)), H)
        np.testing.assert_array_equal(back, m.sum(1)[:, None] * x)


# ------------------------------------------------------------------ expert FFN
def test_scalar_ffn_closed_forms():
    ln3 = math.log(3.0)
    x = np.array([[1.0]])
    y = O.expert_ffn(x, np.array([[ln3]]), np.array([[2.0]]), np.array([[0.5]]), "swiglu")
    assert y[0, 0] == pytest.approx(0.75 * ln3, rel=1e-15)
    # gate and up are not interchangeable
    y2 = O.expert_ffn(x, np.array([[2.0]]), np.array([[ln3]]), np.array([[0.5]]), "swiglu")
    assert abs(y2[0, 0] - 0.75 * ln3) > 0.1
    assert O.gelu(np.array([1.0]))[0] == pytest.approx(GOLD["scalar_ffn"]["gelu_at_1"], rel=1e-15)
    z = np.linspace(-4, 4, 17)
    np.testing.assert_allclose(O.gelu(z) - O.gelu(-z), z, atol=1e-15)
    assert O.silu(np.array([0.0]))[0] == 0.0 and O.gelu(np.array([0.0]))[0] == 0.0
    zero = O.expert_ffn(np.zeros((1, 3)), np.ones((3, 2)), np.ones((3, 2)), np.ones((2, 3)), "swiglu")
    np.testing.assert_array_equal(zero, 0.0)


def _dense_ffn(x, wg, wu, wd, act):
    # written from the textbook definitions: silu(z) = z * logistic(z), gelu(z) = z * Phi(z)
    vlog = np.vectorize(logistic)
    vphi = np.vectorize(lambda z: 0.5 * math.erfc(-z / math.sqrt(2.0)))
    if act == "swiglu":
        a = x @ wg
        h = a * vlog(a) * (x @ wu)
    else:
        a = x @ wu
        h = a * vphi(a)
    return h @ wd


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_single_expert_k1_is_dense_ffn(act):
    rng = np.random.default_rng(4)
    T, H, I = 33, 6, 10
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((H, 1))
    wg = rng.standard_normal((1, H, I)) if act == "swiglu" else None
    wu = rng.standard_normal((1, H, I))
    wd = rng.standard_normal((1, I, H))
    r = O.forward(x, wr, None, wg, wu, wd, top_k=1, activation=act)
    want = _dense_ffn(x, None if wg is None else wg[0], wu[0], wd[0], act)
    np.testing.assert_allclose(r["out"], want, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(r["topk_w"], 1.0)
    # linear in the down projection
    r2 = O.forward(x, wr, None, wg, wu, 2.5 * wd, top_k=1, activation=act)
    np.testing.assert_allclose(r2["out"], 2.5 * r["out"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_k_equals_E_is_dense_mixture(act):
    rng = np.random.default_rng(5)
    T, H, I, E = 9, 4, 6, 5
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((H, E))
    bias = rng.standard_normal(E)
    wg = rng.standard_normal((E, H, I))
    wu = rng.standard_normal((E, H, I))
    wd = rng.standard_normal((E, I, H))
    r = O.forward(x, wr, bias, wg, wu, wd, top_k=E, activation=act)
    want = np.zeros((T, H))
    for t in range(T):
        logit = [sum(x[t, h] * wr[h, e] for h in range(H)) + bias[e] for e in range(E)]
        mx = max(logit)
        z = [math.exp(v - mx) for v in logit]
        s = sum(z)
        for e in range(E):
            want[t] += (z[e] / s) * _dense_ffn(x[t:t + 1], wg[e], wu[e], wd[e], act)[0]
    np.testing.assert_allclose(r["out"], want, rtol=1e-12, atol=1e-12)


def test_token_subset_matches_full_forward():
    rng = np.random.default_rng(6)
    T, H, I, E, k = 50, 8, 12, 6, 2
    args = [rng.standard_normal(s) for s in ((T, H), (H, E), (E,), (E, H, I), (E, H, I), (E, I, H))]
    full = O.forward(*args, top_k=k, activation="swiglu", capacity_factor=0.7)
    ts = np.array([0, 7, 31, 49])
    sub = O.forward(*args, top_k=k, activation="swiglu", capacity_factor=0.7, tokens=ts)
    np.testing.assert_allclose(sub["out"], full["out"][ts], rtol=1e-13, atol=1e-13)
    assert full["capacity"] == math.ceil(0.7 * T * k / E)


def test_all_slots_dropped_gives_zero():
    T, H, E = 6, 3, 2
    x = np.ones((T, H))
    wr = np.zeros((H, E))
    bias = np.array([1.0, 0.0])          # every token prefers expert 0, then 1
    w = np.ones((E, H, 4))
    r = O.forward(x, wr, bias, w, w, np.ones((E, 4, H)), top_k=2, activation="swiglu",
                  capacity_factor=0.5)   # C = ceil(0.5*12/2) = 3
    assert r["capacity"] == 3
    np.testing.assert_array_equal(r["kept"], [3, 3])
    assert (r["out"][3:] == 0).all() and (r["out"][:3] != 0).all()


# ------------------------------------------------------------------ threshold routing (R14)
def test_hand_threshold_case():
    g = GOLD["threshold"]
    L = np.array(g["logits"])
    idx, flags = O.threshold_select(L, 4)
    assert flags == 0
    np.testing.assert_array_equal(idx, g["default_delta_k4_idx"])
    np.testing.assert_allclose(O.threshold_weights(L, idx), g["default_delta_k4_weights"],
                               rtol=1e-15, atol=0)
    idx1, _ = O.threshold_select(L, 1)
    np.testing.assert_array_equal(idx1, g["default_delta_k1_idx"])
    np.testing.assert_array_equal(O.threshold_weights(L, idx1), [[1.0], [1.0], [0.0], [1.0]])
    idx2, _ = O.threshold_select(L, 4, delta=0.1)
    np.testing.assert_array_equal(idx2, g["delta_0.1_k4_idx"])
    w2 = O.threshold_weights(L, idx2)
    e = math.e
    want = [[e / (2 * e + 1), e / (2 * e + 1), 1 / (2 * e + 1), 0.0],
            [logistic(1.0), logistic(-1.0), 0.0, 0.0], [0.25] * 4, [0.5, 0.5, 0.0, 0.0]]
    np.testing.assert_allclose(w2, want, rtol=1e-15, atol=0)
    # raw probabilities when not renormalised: row 1 keeps p0 = e^2 / (e^2 + e + 1 + 1/e)
    raw = O.threshold_weights(L, idx, renormalize=False)
    assert raw[1, 0] == pytest.approx(e * e / (e * e + e + 1 + 1 / e), rel=1e-15)


@pytest.mark.parametrize("u", [0.3, -0.3])
def test_threshold_two_level_closed_form(u):
    # a experts at logit u, the rest at 0: p_u > 1/E exactly when u > 0, p_0 > 1/E exactly
    # when u < 0, so the kept set is one of the two groups, with equal weights
    E = 9
    for a in range(1, E):
        L = np.zeros((1, E))
        hot = np.random.default_rng(a).choice(E, a, replace=False)
        L[0, hot] = u
        idx, _ = O.threshold_select(L, E)
        want = np.sort(hot) if u > 0 else np.setdiff1d(np.arange(E), hot)
        np.testing.assert_array_equal(idx[0, :len(want)], want)
        assert (idx[0, len(want):] == -1).all()
        np.testing.assert_allclose(O.threshold_weights(L, idx)[0, :len(want)], 1 / len(want),
                                   rtol=1e-15)


def _brute_threshold(row, k, delta):
    """log-sum-exp form: keep e when l_e - lse > log(delta); order (-l, e); first k."""
    m = max(row)
    lse = m + math.log(math.fsum(math.exp(v - m) for v in row))
    gap = [v - lse - math.log(delta) for v in row]
    kept = sorted((e for e in range(len(row)) if gap[e] > 0), key=lambda e: (-row[e], e))
    return kept[:k], min(abs(x) for x in gap)


@pytest.mark.parametrize("E,k,delta", [(3, 3, None), (8, 8, None), (8, 2, None), (33, 5, 0.05),
                                       (16, 16, 0.01)])
def test_threshold_matches_brute_force(E, k, delta):
    rng = np.random.default_rng(E * 100 + k)
    L = rng.standard_normal((300, E)) * rng.uniform(0.2, 3.0, (300, 1))
    L[::7, 1] = L[::7, 0]                     # ties
    idx, _ = O.threshold_select(L, k, delta)
    d = O.threshold_delta(E, delta)
    checked = 0
    for t in range(L.shape[0]):
        want, gap = _brute_threshold(list(L[t]), k, d)
        if gap < 1e-9:
            continue
        checked += 1
        got = [int(e) for e in idx[t] if e >= 0]
        assert got == want, t
    assert checked > 250


def test_threshold_tiny_delta_keeps_every_expert_as_topk():
    rng = np.random.default_rng(12)
    L = rng.standard_normal((50, 7))
    idx, _ = O.threshold_select(L, 7, delta=1e-300)
    ref, _ = O.select_experts(L, 7)
    np.testing.assert_array_equal(idx, ref)
    np.testing.assert_allclose(O.threshold_weights(L, idx), O.topk_weights(L, ref),
                               rtol=1e-15, atol=0)


def test_threshold_default_delta_keeps_between_one_and_E_minus_one():
    rng = np.random.default_rng(13)
    for E in (2, 5, 8, 64):
        L = rng.standard_normal((400, E)) * 2.0
        idx, _ = O.threshold_select(L, E)
        n = (idx >= 0).sum(1)
        assert n.min() >= 1 and n.max() <= E - 1
        np.testing.assert_allclose(O.threshold_weights(L, idx).sum(1), 1.0, atol=1e-15)


def test_threshold_nonfinite_rows():
    L = np.array([[0.0, np.nan, 1.0], [np.inf, 0.0, 1.0], [-np.inf, 0.0, 2.0]])
    idx, flags = O.threshold_select(L, 3)
    assert flags & O.FLAG_NONFINITE_LOGIT
    assert (idx[:2] == -1).all()                # NaN / +inf rows keep nothing
    np.testing.assert_array_equal(idx[2], [2, -1, -1])   # -inf only scores zero
    assert (O.threshold_weights(L, idx)[:2] == 0).all()


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_threshold_forward_extremes(act):
    rng = np.random.default_rng(14)
    T, H, I, E = 11, 4, 6, 5
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((H, E))
    wg = rng.standard_normal((E, H, I)) if act == "swiglu" else None
    wu = rng.standard_normal((E, H, I))
    wd = rng.standard_normal((E, I, H))
    # delta above every score: no expert anywhere, the layer outputs zeros
    r0 = O.forward(x, wr, None, wg, wu, wd, top_k=E, activation=act, routing="threshold",
                   threshold=1.5)
    assert (r0["topk_idx"] == -1).all() and (r0["out"] == 0).all()
    assert r0["flags"] == 0 and r0["offsets"][-1] == 0
    # a vanishing delta with k = E keeps every expert: the dense mixture, as top-E routing
    r1 = O.forward(x, wr, None, wg, wu, wd, top_k=E, activation=act, routing="threshold",
                   threshold=1e-300)
    want = np.zeros((T, H))
    for t in range(T):
        logit = [sum(x[t, h] * wr[h, e] for h in range(H)) for e in range(E)]
        mx = max(logit)
        z = [math.exp(v - mx) for v in logit]
        for e in range(E):
            want[t] += (z[e] / sum(z)) * _dense_ffn(x[t:t + 1], None if wg is None else wg[e],
                                                    wu[e], wd[e], act)[0]
    np.testing.assert_allclose(r1["out"], want, rtol=1e-10, atol=1e-10)


def test_empty_slots_are_dropped_without_a_flag():
    idx = np.array([[0, -1], [1, 0], [-1, -1]])
    p = O.permute_indices(idx, 2, 10)
    assert p["flags"] == 0
    np.testing.assert_array_equal(p["counts"], [2, 1])
    assert p["slot_row"][0, 1] == -1 and (p["slot_row"][2] == -1).all()
    counts, offsets, slot_row, row_token = sequential_permute(idx, 2, 10)
    np.testing.assert_array_equal(p["slot_row"], slot_row)
    np.testing.assert_array_equal(p["row_token"], row_token)


# ------------------------------------------------------------------ backward (R15)
def _layer(seed, T, H, I, E, act, bias=True):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((T, H)), w_router=rng.standard_normal((H, E)),
                bias=rng.standard_normal(E) if bias else None,
                w_gate=rng.standard_normal((E, H, I)) / math.sqrt(H) if act == "swiglu" else None,
                w_up=rng.standard_normal((E, H, I)) / math.sqrt(H),
                w_down=rng.standard_normal((E, I, H)) / math.sqrt(I)), rng


def _loss(p, dout, **kw):
    r = O.forward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], **kw)
    return float((r["out"] * dout).sum()), r


BWD_CASES = [
    dict(top_k=2, activation="swiglu"),
    dict(top_k=3, activation="gelu", renormalize=False),
    dict(top_k=2, activation="swiglu", capacity_factor=0.6),
    dict(top_k=5, activation="swiglu", routing="threshold"),
    dict(top_k=2, activation="swiglu", routing="threshold", threshold=0.3),
]


@pytest.mark.parametrize("kw", BWD_CASES, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_backward_matches_central_differences(kw):
    """Every gradient against the central difference of sum(out * dout) along a random
    direction (eps = 1e-6, float64), on inputs whose routing decisions are at least 1e-3
    away from flipping, so the selection is fixed over +-eps."""
    T, H, I, E = 12, 5, 7, 5
    p, rng = _layer(31, T, H, I, E, kw["activation"])
    dout = rng.standard_normal((T, H))
    L = O.gate_logits(p["x"], p["w_router"], p["bias"])
    if kw.get("routing") == "threshold":
        assert O.threshold_margin(L, kw.get("threshold")).min() > 1e-3
    else:
        assert O.selection_margin(L, kw["top_k"]).min() > 1e-3
    g = O.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], dout,
                   **kw)
    if kw.get("capacity_factor"):
        assert (g["forward"]["slot_row"] < 0).any() and (g["forward"]["slot_row"] >= 0).any()
    grads = dict(x=g["dx"], w_router=g["dw_router"], bias=g["dbias"],
                 w_gate=None if g["dw_gate"] is None else np.stack(g["dw_gate"]),
                 w_up=np.stack(g["dw_up"]), w_down=np.stack(g["dw_down"]))
    eps = 1e-6
    for name, grad in grads.items():
        if grad is None:
            continue
        v = rng.standard_normal(p[name].shape)
        plus = {**p, name: p[name] + eps * v}
        minus = {**p, name: p[name] - eps * v}
        fd = (_loss(plus, dout, **kw)[0] - _loss(minus, dout, **kw)[0]) / (2 * eps)
        an = float((grad * v).sum())
        assert an == pytest.approx(fd, rel=1e-6, abs=1e-8), name


def test_backward_single_expert_is_dense_ffn_backward():
    """E = 1, k = 1: the weight is 1 and the logits get no gradient; the expert gradients are
    the textbook dense-FFN ones, written out separately."""
    T, H, I = 9, 4, 6
    p, rng = _layer(32, T, H, I, 1, "swiglu")
    dout = rng.standard_normal((T, H))
    g = O.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], dout,
                   top_k=1, activation="swiglu")
    x, wg, wu, wd = p["x"], p["w_gate"][0], p["w_up"][0], p["w_down"][0]
    a, b = x @ wg, x @ wu
    sig = 1.0 / (1.0 + np.exp(-a))
    h = a * sig * b
    dh = dout @ wd.T
    da = dh * b * (sig + a * sig * (1.0 - sig))
    db = dh * a * sig
    np.testing.assert_allclose(g["dw_down"][0], h.T @ dout, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw_gate"][0], x.T @ da, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw_up"][0], x.T @ db, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dx"], da @ wg.T + db @ wu.T, rtol=1e-12, atol=1e-12)
    assert np.abs(g["dw_router"]).max() == 0 and np.abs(g["dbias"]).max() == 0


def test_backward_renormalised_logit_gradient_sums_to_zero():
    """With renormalised weights the output depends on the selected logits only through
    their differences: each token's logit gradient sums to zero and vanishes outside the
    selected experts."""
    T, H, I, E = 20, 4, 6, 6
    p, rng = _layer(33, T, H, I, E, "swiglu")
    dout = rng.standard_normal((T, H))
    g = O.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], dout,
                   top_k=3, activation="swiglu")
    dL = g["dlogits"]
    np.testing.assert_allclose(dL.sum(axis=1), 0.0, atol=1e-12)
    idx = g["forward"]["topk_idx"]
    mask = np.zeros_like(dL, dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert np.abs(dL[~mask]).max() < 1e-15


# ------------------------------------------------- auxiliary load-balancing loss (R16)
def test_aux_loss_balanced_closed_forms():
    """Where every expert's mean probability is 1/E the loss is the coefficient itself:
    (a) all logits equal: p = 1/E everywhere, ties send every token to experts 0..k-1, so
    f = 1/k on those and the loss is coeff * E * k * (1/k)(1/E); (b) E tokens, token t
    one-hot at expert t (k = 1): f = 1/E and, by symmetry, P = 1/E."""
    for E, k, c in ((8, 2, 0.01), (5, 5, 0.1), (3, 1, 1.0)):
        L = np.zeros((7, E))
        idx, _ = O.select_experts(L, k)
        r = O.aux_loss(L, idx, c)
        assert r["loss"] == pytest.approx(c, rel=1e-14)
        np.testing.assert_allclose(r["P"], 1.0 / E, rtol=1e-15)
        # p = 1/E and g = c E f / T: experts 0..k-1 get (1/E)(c E / (k T) - c / T), the rest
        # -c / (E T) (zero when k = E)
        T = L.shape[0]
        np.testing.assert_allclose(r["dlogits"][:, :k], c / T * (1.0 / k - 1.0 / E), rtol=1e-13,
                                   atol=1e-18)
        np.testing.assert_allclose(r["dlogits"][:, k:], -c / (E * T), rtol=1e-13)
    E, a, c = 6, 2.5, 0.05
    L = a * np.eye(E)
    idx, _ = O.select_experts(L, 1)
    np.testing.assert_array_equal(idx[:, 0], np.arange(E))
    r = O.aux_loss(L, idx, c)
    np.testing.assert_allclose(r["P"], 1.0 / E, rtol=1e-14)
    assert r["loss"] == pytest.approx(c, rel=1e-14)


def test_aux_loss_collapsed_routing_closed_form():
    """Every token on expert 0 (k = 1) with the same logits [z, 0, .., 0]: f = (1, 0, ..),
    P_0 = e^z / (e^z + E - 1), so the loss is coeff * E * P_0; the gradient on logit j of
    each token is p_j (g_j - p_0 g_0) with only g_0 = coeff * E / T nonzero."""
    T, E, z, c = 9, 4, 1.7, 0.02
    L = np.zeros((T, E))
    L[:, 0] = z
    idx, _ = O.select_experts(L, 1)
    r = O.aux_loss(L, idx, c)
    p0 = math.exp(z) / (math.exp(z) + E - 1)
    pj = 1.0 / (math.exp(z) + E - 1)
    assert r["loss"] == pytest.approx(c * E * p0, rel=1e-14)
    g0 = c * E / T
    np.testing.assert_allclose(r["dlogits"][:, 0], p0 * (g0 - p0 * g0), rtol=1e-13)
    np.testing.assert_allclose(r["dlogits"][:, 1:], pj * (0.0 - p0 * g0), rtol=1e-13)


def test_aux_loss_gradient_matches_central_differences():
    """Gradient of the loss with the routing held fixed against central differences along
    random directions; each token's gradient sums to zero (softmax). Invalid ids and -1
    slots do not count."""
    rng = np.random.default_rng(41)
    T, E, k, c = 11, 7, 3, 0.03
    L = rng.standard_normal((T, E))
    idx, _ = O.select_experts(L, k)
    idx = idx.copy()
    idx[0, 2] = -1
    idx[1, 1] = E + 3
    r = O.aux_loss(L, idx, c)
    assert r["counts"].sum() == T * k - 2
    np.testing.assert_allclose(r["dlogits"].sum(axis=1), 0.0, atol=1e-16)
    eps = 1e-6
    for _ in range(3):
        v = rng.standard_normal(L.shape)
        fd = (O.aux_loss(L + eps * v, idx, c)["loss"] - O.aux_loss(L - eps * v, idx, c)["loss"]) / (2 * eps)
        assert float((r["dlogits"] * v).sum()) == pytest.approx(fd, rel=1e-7, abs=1e-12)


@pytest.mark.parametrize("kw", [dict(top_k=2, activation="swiglu"),
                                dict(top_k=2, activation="swiglu", capacity_factor=0.6),
                                dict(top_k=3, activation="gelu", renormalize=False)],
                         ids=["topk", "capacity", "gelu-raw"])
def test_backward_with_aux_loss_matches_central_differences(kw):
    """The objective sum(out * dout) + aux_loss(logits, ids): the gradients with respect to
    x, W_router and the gate bias against central differences (routing fixed over +-eps);
    the expert-weight gradients do not change."""
    T, H, I, E, c = 12, 5, 7, 5, 0.05
    p, rng = _layer(31, T, H, I, E, kw["activation"])
    dout = rng.standard_normal((T, H))
    L = O.gate_logits(p["x"], p["w_router"], p["bias"])
    assert O.selection_margin(L, kw["top_k"]).min() > 1e-3
    idx, _ = O.select_experts(L, kw["top_k"])

    def objective(q):
        val, r = _loss(q, dout, **kw)
        return val + O.aux_loss(r["logits"], r["topk_idx"], c)["loss"]

    g0 = O.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], dout,
                    **kw)
    g = O.backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], dout,
                   aux_loss_coeff=c, **kw)
    assert g["aux_loss"] == pytest.approx(O.aux_loss(L, idx, c)["loss"], rel=1e-14)
    np.testing.assert_allclose(np.stack(g["dw_up"]), np.stack(g0["dw_up"]), rtol=0, atol=0)
    eps = 1e-6
    for name, grad in dict(x=g["dx"], w_router=g["dw_router"], bias=g["dbias"]).items():
        v = rng.standard_normal(p[name].shape)
        fd = (objective({**p, name: p[name] + eps * v}) -
              objective({**p, name: p[name] - eps * v})) / (2 * eps)
        assert float((grad * v).sum()) == pytest.approx(fd, rel=1e-6, abs=1e-8), name
