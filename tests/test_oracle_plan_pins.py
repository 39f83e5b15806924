"""Pins of the oracle's verify planner: Appendix A, brute-force optimality on tiny batches,
the admission threshold, non-anticipation and the lagged capacity."""
import itertools

import numpy as np
import pytest

import oracle
from helpers import dense_offsets, first_emitted, golden

EARLY, FULL, PATH, LAG = oracle.EARLY_STOP, oracle.FULL_VERIFY, oracle.FULL_PATH, oracle.LAGGED_TOPK


def _appendix_sps(gd):
    return np.array([1.0, gd["sps"]["1"], gd["sps"]["2"], gd["sps"]["3"]], np.float64)


def test_appendix_a_theta_values_and_choices():
    gd = golden("appendix_a.json")
    sps = _appendix_sps(gd)
    for c2, key, choice in ((gd["c2_if_A"], "2_if_A", gd["retrospective_choice"]["A"]),
                            (gd["c2_if_B"], "2_if_B", gd["retrospective_choice"]["B"])):
        conf = np.array([[gd["a1"], c2]], np.float32)
        e = oracle.plan(conf, sps, EARLY)
        th = e["theta_path"]
        assert th[0] == pytest.approx(gd["theta"]["0"], abs=1e-7)
        assert th[1] == pytest.approx(gd["theta"]["1"], abs=1e-7)
        assert th[2] == pytest.approx(gd["theta"][key], abs=1e-7)
        assert e["draft_len"][0] == gd["early_stop_choice"]
        assert e["stats"][2] == pytest.approx(gd["theta"]["0"], abs=1e-12)
        f = oracle.plan(conf, sps, PATH)
        assert f["draft_len"][0] == choice
        assert list(f["row_offsets"]) == [0, 1 + choice]


def _appendix_round(mode_of_x1):
    """One request, two drafted positions, V = {A, B}; p_d = (0.5, 0.5), p_t = (0.7, 0.3) at
    position 1; c_2 depends on the drafted x_1 (0.9 after A, 0 after B). Exact grid over the
    uniforms; returns the distribution of the first emitted token."""
    gd = golden("appendix_a.json")
    sps = _appendix_sps(gd)
    n = 10
    mid = (np.arange(n) + 0.5) / n
    i, l = np.meshgrid(mid, mid, indexing="ij")
    B, g, V, r = n * n, 2, 2, 16
    u = np.zeros((B, g + 1, 3), np.float32)
    u[:, 0, 0] = i.ravel()
    u[:, 0, 2] = l.ravel()
    u[:, :, 1] = 0.5
    U = np.zeros((B, g, V), np.float32)
    W = np.zeros((V, r), np.uint16)
    anchor = np.zeros(B, np.int32)
    d = oracle.markov_draft(U, W, W, anchor, u)
    ell = np.zeros(B, np.int32)
    for b in range(B):
        c2 = gd["c2_if_A"] if d["tokens"][b, 0] == 0 else gd["c2_if_B"]
        p = oracle.plan(np.array([[gd["a1"], c2]], np.float32), sps, mode_of_x1)
        ell[b] = p["draft_len"][0]
    offs = np.concatenate([[0], np.cumsum(1 + ell)]).astype(np.int32)
    pt = np.log(np.array(gd["p_target_pos1"], np.float64)).astype(np.float32)
    rows = []
    for b in range(B):
        rows.append(pt)
        rows.extend([np.zeros(V, np.float32)] * ell[b])
    v = oracle.verify(np.stack(rows), offs, ell, U, W, W, anchor, d["tokens"], d["q"], u)
    y = first_emitted(d["tokens"], v["accept_len"], v["next_token"])
    return np.bincount(y, minlength=2) / B


def test_appendix_a_retrospective_search_is_biased_and_early_stop_is_not():
    gd = golden("appendix_a.json")
    assert np.allclose(_appendix_round(PATH), gd["retrospective_output"], atol=1e-12)
    assert np.allclose(_appendix_round(EARLY), gd["early_stop_output"], atol=1e-12)


def _theta(ell, a, sps, R):
    tau = R + sum(a[rq, :ell[rq]].sum() for rq in range(R))
    return tau * sps[R + sum(ell)], tau


def _random_sps(rng, n, kind):
    x = np.arange(n, dtype=np.float64)
    if kind == "hyper":
        return 1.0 / (1.0 + x / rng.uniform(1, 12))
    if kind == "decreasing":
        return np.sort(rng.uniform(0.2, 1.0, n))[::-1].copy()
    if kind == "saw":
        return 1.0 / (1.0 + np.floor(x / 3) * rng.uniform(0.2, 0.8)) * (1 + 0.15 * (x % 3 == 2))
    return np.ones(n)


def _random_conf(rng, R, g):
    c = rng.uniform(0.05, 1.0, (R, g))
    kind = rng.integers(0, 4)
    if kind == 1:
        c[rng.uniform(size=c.shape) < 0.3] = 1.0
    elif kind == 2:
        c[rng.uniform(size=c.shape) < 0.2] = 0.0
    elif kind == 3:
        c = np.round(c * 4) / 4
    return c.astype(np.float32)


def _sorted_order(a):
    R, g = a.shape
    rq, j = np.meshgrid(np.arange(R), np.arange(g), indexing="ij")
    order = np.lexsort((j.ravel(), rq.ravel(), -a.ravel()))
    return rq.ravel()[order], j.ravel()[order], a.ravel()[order]


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_planner_optimality(seed):
    """All (gamma+1)^R length vectors, R <= 4, gamma <= 3: the full-path choice reaches the
    global maximum of Theta; for every budget the greedy prefix reaches the maximum tau; early
    stop is globally optimal whenever Theta is unimodal along the path; admitted sets are the
    top candidates by survival and per-request prefixes."""
    rng = np.random.default_rng(seed)
    R, g = int(rng.integers(1, 5)), int(rng.integers(1, 4))
    conf = _random_conf(rng, R, g)
    sps = _random_sps(rng, R * (g + 1) + 1, ["hyper", "decreasing", "saw", "flat"][seed % 4])
    a = np.cumprod(conf.astype(np.float64), axis=1)
    best, best_tau = -np.inf, {}
    for ell in itertools.product(range(g + 1), repeat=R):
        th, tau = _theta(ell, a, sps, R)
        best = max(best, th)
        n = sum(ell)
        best_tau[n] = max(best_tau.get(n, -np.inf), tau)
    f = oracle.plan(conf, sps, PATH)
    assert f["stats"][2] == pytest.approx(best, rel=1e-12)
    assert _theta(f["draft_len"], a, sps, R)[0] == pytest.approx(best, rel=1e-12)
    path = f["theta_path"]
    for n in range(R * g + 1):
        assert path[n] / sps[R + n] == pytest.approx(best_tau[n], rel=1e-12)
    # admitted set = top-n candidates; prefixes
    rq, j, _ = _sorted_order(a)
    for mode in (EARLY, PATH):
        p = oracle.plan(conf, sps, mode)
        n = int(p["draft_len"].sum())
        for q in range(R):
            top = sorted(j[:n][rq[:n] == q])
            assert top == list(range(p["draft_len"][q]))
        assert np.array_equal(p["row_offsets"], np.concatenate([[0], np.cumsum(1 + p["draft_len"])]))
    # early stop optimal when unimodal (strict rise, then no rise)
    d = np.diff(path)
    peak = int(np.argmax(path))
    unimodal = np.all(d[:peak] > 0) and np.all(d[peak:] <= 0)
    e = oracle.plan(conf, sps, EARLY)
    if unimodal:
        assert e["stats"][2] == pytest.approx(best, rel=1e-12)
    assert e["stats"][2] <= best * (1 + 1e-12)


@pytest.mark.parametrize("seed", range(20))
def test_admission_threshold_identity(seed):
    """Early stop admits a candidate with survival a exactly when
    a > tau (SPS(B) / SPS(B+1) - 1) at the current tau and B (the threshold form)."""
    rng = np.random.default_rng(100 + seed)
    R, g = int(rng.integers(2, 9)), int(rng.integers(1, 6))
    conf = _random_conf(rng, R, g)
    sps = _random_sps(rng, R * (g + 1) + 1, ["hyper", "decreasing"][seed % 2])
    p = oracle.plan(conf, sps, EARLY)
    a = np.cumprod(conf.astype(np.float64), axis=1)
    _, _, a_sorted = _sorted_order(a)
    n_adm = int(p["draft_len"].sum())
    tau = float(R)
    for i in range(min(n_adm + 1, R * g)):
        Bt = R + i
        thr = tau * (sps[Bt] / sps[Bt + 1] - 1.0)
        if abs(a_sorted[i] - thr) < 1e-12:
            break
        assert (a_sorted[i] > thr) == (i < n_adm)
        tau += a_sorted[i]


def test_flat_sps_verifies_everything():
    rng = np.random.default_rng(1)
    conf = rng.uniform(0.01, 1.0, (7, 5)).astype(np.float32)
    p = oracle.plan(conf, np.ones(7 * 6 + 1), EARLY)
    assert np.all(p["draft_len"] == 5)
    assert p["stats"][0] == 7 * 6
    full = oracle.plan(None, np.ones(7 * 6 + 1), FULL, B=7, gamma=5)
    assert np.all(full["draft_len"] == 5)
    assert np.array_equal(full["row_offsets"], dense_offsets(7, 5))


@pytest.mark.parametrize("seed", range(15))
def test_non_anticipation(seed):
    """Whether (r, j) is admitted never depends on c_{r,j'} for j' > j under early stop or the
    lagged top-K (those confidences depend on tokens drafted at or after j)."""
    rng = np.random.default_rng(200 + seed)
    R, g = 6, 4
    conf = _random_conf(rng, R, g)
    sps = _random_sps(rng, R * (g + 1) + 1, ["hyper", "saw"][seed % 2])
    lag = _random_conf(rng, R, g)
    for mode in (EARLY, LAG):
        def run(c):
            ring = np.zeros((2, R, g), np.float32)
            ring[0] = lag
            return oracle.plan(c, sps, mode, ring=ring, round_index=2)["draft_len"]
        base = run(conf)
        for rq in range(R):
            for j in range(g - 1):
                c2 = conf.copy()
                c2[rq, j + 1:] = rng.uniform(0, 1, g - 1 - j).astype(np.float32)
                assert (run(c2)[rq] > j) == (base[rq] > j)


def test_full_path_is_anticipating_on_appendix_a():
    gd = golden("appendix_a.json")
    sps = _appendix_sps(gd)
    a = oracle.plan(np.array([[0.8, 0.9]], np.float32), sps, PATH)["draft_len"][0]
    b = oracle.plan(np.array([[0.8, 0.0]], np.float32), sps, PATH)["draft_len"][0]
    assert (a > 0) != (b > 0)


def test_lagged_topk_ring_and_capacity():
    """Rounds 0-1 plan with early stop; from round 2 the capacity K comes from the full-path
    search on the confidences of round t-2 (ring slot t % 2) and the admitted set is the top
    K - R of round t's own order; every round leaves its confidences in slot t % 2."""
    rng = np.random.default_rng(42)
    R, g = 12, 5
    sps = 1.0 / (1.0 + np.arange(R * (g + 1) + 1) / 20.0)
    ring = np.zeros((2, R, g), np.float32)
    confs = [_random_conf(rng, R, g) for _ in range(5)]
    for t, c in enumerate(confs):
        p = oracle.plan(c, sps, LAG, ring=ring, round_index=t)
        assert np.array_equal(ring[t % 2], c)
        if t < 2:
            e = oracle.plan(c, sps, EARLY)
            assert np.array_equal(p["draft_len"], e["draft_len"])
            continue
        k_lag = int(oracle.plan(confs[t - 2], sps, PATH)["draft_len"].sum())
        assert p["stats"][3] == R + k_lag
        a = np.cumprod(c.astype(np.float64), axis=1)
        rq, _, _ = _sorted_order(a)
        expect = np.bincount(rq[:k_lag], minlength=R)
        assert np.array_equal(p["draft_len"], expect)


def _first_argmax_count(c, sps):
    """Admissions at the first maximiser of Theta along the survival order, written out from the
    definition ([V41] "目标函数": Theta = tau * SPS(B_tot), tau = R + admitted survivals)."""
    R = c.shape[0]
    _, _, a_sorted = _sorted_order(np.cumprod(c.astype(np.float64), axis=1))
    tau = R + np.concatenate([[0.0], np.cumsum(a_sorted)])
    theta = tau * sps[R + np.arange(len(tau))]
    return int(np.argmax(theta)), theta


def test_lagged_capacity_is_a_full_path_search_on_a_two_peak_table():
    """The lagged planner's capacity comes from a search of the whole path, not from early stop
    ([V41] "阈值随负载变化", [CSDN] 8: the production planner drops early stop because the step
    time is not unimodal in B). Hand-worked two-peak case, R = 2, gamma = 2:
    round t-2 confidences [[0.9, 0.9], [0.5, 0.5]] give survivals 0.9, 0.81, 0.5, 0.25 in path
    order, tau = 2, 2.9, 3.71, 4.21, 4.46, and with SPS(2..6) = 1, 0.6, 0.58, 0.45, 0.44
    Theta = 2, 1.74, 2.1518, 1.8945, 1.9624: early stop admits 0, the full path 2, so K = 4.
    Round t's own order (survivals 0.3, 0.06 | 0.95, 0.855) then admits both of request 1."""
    R, g = 2, 2
    sps = np.array([1.0, 1.0, 1.0, 0.6, 0.58, 0.45, 0.44])
    c_lag = np.array([[0.9, 0.9], [0.5, 0.5]], np.float32)
    c_now = np.array([[0.3, 0.2], [0.95, 0.9]], np.float32)
    k_np, theta = _first_argmax_count(c_lag, sps)
    assert np.allclose(theta, [2.0, 1.74, 2.1518, 1.8945, 1.9624], atol=1e-6)
    assert k_np == 2
    assert oracle.plan(c_lag, sps, EARLY)["draft_len"].sum() == 0
    ring = np.zeros((2, R, g), np.float32)
    ring[0] = c_lag
    p = oracle.plan(c_now, sps, LAG, ring=ring, round_index=2)
    assert p["stats"][3] == R + 2
    assert list(p["draft_len"]) == [0, 2]
    assert list(p["row_offsets"]) == [0, 1, 4]
    assert p["stats"][0] == 4
    assert np.array_equal(ring[0], c_now)


def test_full_path_takes_the_first_maximiser_on_a_plateau():
    """Theta ties exactly along the path (c = 1, SPS(1..4) = 1, 1/2, 1/4, 1/4 gives
    Theta = 1, 1, 0.75, 1): the full-path search keeps the smallest batch reaching the maximum
    (the strict comparison of "stop once Theta no longer rises", [V41] "贪心就能解"), so it
    admits nothing, and so does the lagged capacity read from the same confidences."""
    c = np.ones((1, 3), np.float32)
    sps = np.array([1.0, 1.0, 0.5, 0.25, 0.25])
    k_np, theta = _first_argmax_count(c, sps)
    assert list(theta) == [1.0, 1.0, 0.75, 1.0] and k_np == 0
    f = oracle.plan(c, sps, PATH)
    assert f["draft_len"][0] == 0 and f["stats"][2] == 1.0
    ring = np.zeros((2, 1, 3), np.float32)
    ring[1] = c
    p = oracle.plan(c, sps, LAG, ring=ring, round_index=3)
    assert p["stats"][3] == 1 and p["draft_len"][0] == 0


@pytest.mark.parametrize("seed", range(30))
def test_lagged_capacity_matches_argmax_on_sawtooth_tables(seed):
    """Random sawtooth and bucketed SPS tables (not unimodal): the lagged capacity equals R plus
    the first argmax of Theta on the confidences of round t-2, computed here from the
    definition."""
    rng = np.random.default_rng(900 + seed)
    R, g = int(rng.integers(2, 9)), int(rng.integers(1, 6))
    n = R * (g + 1) + 1
    x = np.arange(n, dtype=np.float64)
    if seed % 2:
        sps = 1.0 / (1.0 + np.floor(x / 4) * rng.uniform(0.3, 1.5)) * (1 + 0.3 * (x % 4 == 3))
    else:
        sps = 1.0 / np.ceil((x + 1) / rng.integers(2, 6))
    c_lag, c_now = _random_conf(rng, R, g), _random_conf(rng, R, g)
    k_np, _ = _first_argmax_count(c_lag, sps)
    ring = np.zeros((2, R, g), np.float32)
    ring[seed % 2] = c_lag
    p = oracle.plan(c_now, sps, LAG, ring=ring, round_index=2 + seed % 2)
    assert p["stats"][3] == R + k_np
    rq, _, _ = _sorted_order(np.cumprod(c_now.astype(np.float64), axis=1))
    assert np.array_equal(p["draft_len"], np.bincount(rq[:k_np], minlength=R))
