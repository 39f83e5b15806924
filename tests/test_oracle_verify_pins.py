"""Pins of the oracle's lossless verify against what the pages and the mathematics fix."""
import numpy as np
import pytest

import oracle
from helpers import (bf16_round, chi2_pvalue, dense_offsets, first_emitted, golden, softmax64)

R16 = 16


def _zeros_w(V, r=R16):
    return np.zeros((V, r), np.uint16), np.zeros((V, r), np.uint16)


def _grid_uniforms(n):
    mid = (np.arange(n) + 0.5) / n
    i, j, l = np.meshgrid(mid, mid, mid, indexing="ij")
    B = n ** 3
    u = np.zeros((B, 2, 3), np.float32)
    u[:, 0, 0] = i.ravel()
    u[:, 0, 1] = j.ravel()
    u[:, 0, 2] = l.ravel()
    u[:, 1, 2] = l.ravel()
    return u


def test_ab_worked_example_exact_grid():
    """p_t = (0.7, 0.3), p_d = (0.5, 0.5): output (0.7, 0.3), B accepted w.p. 0.6, the
    correction puts all its mass on A, acceptance 0.8 (worked example, Appendix A)."""
    gd = golden("ab_worked_example.json")
    n = 10
    B, g, V = n ** 3, 1, 2
    U = np.zeros((B, g, V), np.float32)           # p_d = (0.5, 0.5)
    W1, W2t = _zeros_w(V)
    anchor = np.zeros(B, np.int32)
    u = _grid_uniforms(n)
    d = oracle.markov_draft(U, W1, W2t, anchor, u)
    assert np.allclose(d["q"], 0.5)
    tl = np.log(np.array(gd["p_target"], np.float64)).astype(np.float32)
    target = np.tile(tl, (B * (g + 1), 1))
    v = oracle.verify(target, dense_offsets(B, g), np.full(B, g, np.int32), U, W1, W2t, anchor,
                      d["tokens"], d["q"], u)
    y = first_emitted(d["tokens"], v["accept_len"], v["next_token"])
    counts = np.bincount(y, minlength=2)
    assert list(counts) == [int(round(p * B)) for p in gd["output"]]
    drew_b = d["tokens"][:, 0] == 1
    acc_b = (v["accept_len"][drew_b] == 1).mean()
    assert acc_b == pytest.approx(gd["accept_prob"][1], abs=1e-12)
    assert np.all(v["accept_len"][~drew_b] == 1)          # A always accepted
    rej = v["accept_len"] == 0
    assert rej.sum() > 0
    assert np.all(v["next_token"][rej] == 0)               # correction mass only on A
    res_total = sum(gd["residual_unnormalised"])
    assert np.allclose(v["resid_mass"][rej], res_total, atol=1e-7)
    assert np.allclose(v["beta_emit"][rej], gd["beta"], atol=1e-6)
    assert np.all(v["beta_emit"][~rej] == -1.0)


def test_of_course_acceptance_is_half():
    """p = (1, 0), q = (0.5, 0.5) gives acceptance 0.5; drawing the impossible token is always
    rejected and corrected to the certain one."""
    gd = golden("of_course.json")
    B, g, V = 2, 1, 2
    U = np.zeros((B, g, V), np.float32)
    W1, W2t = _zeros_w(V)
    anchor = np.zeros(B, np.int32)
    u = np.zeros((B, g + 1, 3), np.float32)
    u[0, 0, 0] = 0.75      # draws token 1 ("problem" after "of")
    u[1, 0, 0] = 0.25      # draws token 0
    u[:, 0, 1] = 0.5
    d = oracle.markov_draft(U, W1, W2t, anchor, u)
    assert list(d["tokens"][:, 0]) == [1, 0]
    target = np.tile(np.array([0.0, -1e30], np.float32), (B * (g + 1), 1))
    v = oracle.verify(target, dense_offsets(B, g), np.full(B, g, np.int32), U, W1, W2t, anchor,
                      d["tokens"], d["q"], u)
    assert v["accept_len"][0] == 0 and v["next_token"][0] == 0
    assert v["beta_emit"][0] == pytest.approx(gd["beta"], abs=1e-7)
    assert v["resid_mass"][0] == pytest.approx(1.0 - gd["beta"], abs=1e-12)
    assert v["accept_len"][1] == 1 and v["beta_emit"][1] == -1.0


def test_sum_min_identity_on_every_emission_row():
    """sum_v min(p, q) = 1 - |p - q|_1 / 2 and sum_v max(0, p - q) = 1 - beta, on residual rows
    of random rounds; p_t and p_d recomputed here with scipy's softmax."""
    rng = np.random.default_rng(7)
    B, g, V, r = 64, 3, 300, 16
    U = rng.normal(0, 2.0, (B, g, V)).astype(np.float32)
    W1 = bf16_round(rng.normal(0, 0.3, (V, r)))
    W2t = bf16_round(rng.normal(0, 0.3, (V, r)))
    anchor = rng.integers(0, V, B).astype(np.int32)
    u = (rng.integers(0, 1 << 24, (B, g + 1, 3)) * 2.0 ** -24).astype(np.float32)
    d = oracle.markov_draft(U, W1, W2t, anchor, u, want_logits=True)
    dense = np.concatenate([d["logits"], rng.normal(0, 2.0, (B, 1, V)).astype(np.float32)], 1)
    dense = (dense + rng.normal(0, 1.5, dense.shape)).astype(np.float32)
    v = oracle.verify(dense.reshape(-1, V), dense_offsets(B, g), np.full(B, g, np.int32), U, W1,
                      W2t, anchor, d["tokens"], d["q"], u)
    rej = np.nonzero(v["beta_emit"] >= 0)[0]
    assert len(rej) > 10
    for b in rej:
        k = v["accept_len"][b]                       # 0-based position of the reject
        pt = softmax64(dense[b, k])
        pd = softmax64(d["logits"][b, k])
        beta_ref = 1.0 - 0.5 * np.abs(pt - pd).sum()
        assert v["beta_emit"][b] == pytest.approx(beta_ref, abs=1e-6)
        assert v["resid_mass"][b] == pytest.approx(1.0 - beta_ref, abs=1e-12)
        assert pt[v["next_token"][b]] > pd[v["next_token"][b]]   # drawn from the correction


@pytest.mark.parametrize("gamma", [1, 2])
def test_chi2_output_marginal_equals_target(gamma):
    """Monte Carlo on V = 4: whatever the draft distribution (Markov-biased, anchor dependent),
    the first emitted token follows p_t (the losslessness derivation)."""
    rng = np.random.default_rng(11 + gamma)
    B, V, r = 1_000_000, 4, R16
    U = np.tile(np.array([1.0, -0.5, 0.3, 2.0], np.float32), (B, gamma, 1))
    W1 = bf16_round(rng.normal(0, 0.6, (V, r)))
    W2t = bf16_round(rng.normal(0, 0.6, (V, r)))
    anchor = rng.integers(0, V, B).astype(np.int32)
    u = (rng.integers(0, 1 << 24, (B, gamma + 1, 3)) * 2.0 ** -24).astype(np.float32)
    d = oracle.markov_draft(U, W1, W2t, anchor, u)
    tl = np.array([0.2, 1.1, -0.7, 0.5], np.float32)
    target = np.tile(tl, (B * (gamma + 1), 1))
    v = oracle.verify(target, dense_offsets(B, gamma), np.full(B, gamma, np.int32), U, W1, W2t,
                      anchor, d["tokens"], d["q"], u)
    y = first_emitted(d["tokens"], v["accept_len"], v["next_token"])
    p = chi2_pvalue(np.bincount(y, minlength=V), softmax64(tl))
    assert p > 1e-3
    # and the draft distribution really differs from the target
    assert abs(d["q"].mean() - 0.25) > 1e-3


def test_joint_two_tokens_follow_target_chain():
    """Two emitted tokens (over one or two rounds, the second round anchored at the first
    emitted token) jointly follow p(y1) p(y2 | y1) of a table target model: exercises anchors,
    the Markov bias conditioning and the rule that the emitted token is the next anchor."""
    rng = np.random.default_rng(5)
    B, V, g, r = 1_000_000, 4, 2, R16
    T1 = np.array([0.3, -0.2, 1.0, 0.1], np.float32)
    T2 = rng.normal(0, 1.0, (V, V)).astype(np.float32)
    T3 = rng.normal(0, 1.0, (V, V, V)).astype(np.float32)
    W1 = bf16_round(rng.normal(0, 0.7, (V, r)))
    W2t = bf16_round(rng.normal(0, 0.7, (V, r)))
    U = rng.normal(0, 0.8, (1, g, V)).astype(np.float32).repeat(B, 0)

    def one_round(anchor, row1_fn, row2_fn, row3_fn, seed):
        rg = np.random.default_rng(seed)
        u = (rg.integers(0, 1 << 24, (len(anchor), g + 1, 3)) * 2.0 ** -24).astype(np.float32)
        d = oracle.markov_draft(U[:len(anchor)], W1, W2t, anchor, u)
        x1, x2 = d["tokens"][:, 0], d["tokens"][:, 1]
        rows = np.stack([row1_fn(anchor), row2_fn(anchor, x1), row3_fn(anchor, x1, x2)], 1)
        v = oracle.verify(rows.reshape(-1, V), dense_offsets(len(anchor), g),
                          np.full(len(anchor), g, np.int32), U[:len(anchor)], W1, W2t, anchor,
                          d["tokens"], d["q"], u)
        emitted = [[d["tokens"][i, j] for j in range(v["accept_len"][i])] + [v["next_token"][i]]
                   for i in range(len(anchor))] if len(anchor) < 10 else None
        return d, v, emitted

    anchor = np.zeros(B, np.int32)
    d, v, _ = one_round(anchor, lambda a: np.tile(T1, (len(a), 1)), lambda a, x1: T2[x1],
                        lambda a, x1, x2: T3[x1, x2], 100)
    y1 = first_emitted(d["tokens"], v["accept_len"], v["next_token"])
    y2 = np.where(v["accept_len"] >= 2, d["tokens"][:, 1],
                  np.where(v["accept_len"] == 1, v["next_token"], -1))
    need = np.nonzero(y2 < 0)[0]
    # second round for requests that emitted one token: anchored at y1, position 1 ~ T2[y1]
    a2 = y1[need].astype(np.int32)
    d2, v2, _ = one_round(a2, lambda a: T2[a], lambda a, x1: T3[a, x1],
                          lambda a, x1, x2: np.tile(T1, (len(a), 1)), 200)
    y2[need] = first_emitted(d2["tokens"], v2["accept_len"], v2["next_token"])
    joint = np.bincount(y1 * V + y2, minlength=V * V)
    ref = (softmax64(T1)[:, None] * softmax64(T2, axis=1)).ravel()
    assert chi2_pvalue(joint, ref) > 1e-3


def test_expected_accepted_length_is_sum_of_survivals():
    """E[N] = sum_j P(N >= j) = sum_j prod_{i<=j} beta_i when positions are independent."""
    rng = np.random.default_rng(3)
    B, V, g, r = 200_000, 16, 3, R16
    Ub = rng.normal(0, 1.0, (g, V)).astype(np.float32)
    Tb = (Ub + rng.normal(0, 0.8, (g, V))).astype(np.float32)
    U = np.broadcast_to(Ub, (B, g, V)).copy()
    W1, W2t = _zeros_w(V)
    anchor = np.zeros(B, np.int32)
    u = (rng.integers(0, 1 << 24, (B, g + 1, 3)) * 2.0 ** -24).astype(np.float32)
    d = oracle.markov_draft(U, W1, W2t, anchor, u)
    rows = np.concatenate([Tb, Tb[:1]], 0)
    target = np.tile(rows, (B, 1))
    v = oracle.verify(target, dense_offsets(B, g), np.full(B, g, np.int32), U, W1, W2t, anchor,
                      d["tokens"], d["q"], u)
    beta = np.array([np.minimum(softmax64(Tb[k]), softmax64(Ub[k])).sum() for k in range(g)])
    expected = np.cumprod(beta).sum()
    n = v["accept_len"].astype(np.float64)
    assert abs(n.mean() - expected) < 5 * n.std() / np.sqrt(B)
    for j in range(1, g + 1):
        assert abs((n >= j).mean() - np.prod(beta[:j])) < 5 * np.sqrt(0.25 / B)


def test_bonus_only_when_all_accepted_and_flags():
    """All-accepted requests emit a bonus drawn from p_t of row l+1; a non-finite target row
    sets the non-finite flag and its token falls back to id 0."""
    B, g, V = 3, 2, 8
    U = np.zeros((B, g, V), np.float32)
    W1, W2t = _zeros_w(V)
    anchor = np.zeros(B, np.int32)
    u = np.zeros((B, g + 1, 3), np.float32)
    u[:, :, 0] = 0.0        # draft picks token 0 everywhere (p_d uniform)
    u[:, :, 1] = 0.0        # accept whenever p_t(x) > 0
    u[:, 2, 2] = 0.99       # bonus draw near the top of the CDF
    d = oracle.markov_draft(U, W1, W2t, anchor, u)
    target = np.zeros((B * (g + 1), V), np.float32)
    target[2 * (g + 1) + 0, 3] = np.nan
    v = oracle.verify(target, dense_offsets(B, g), np.full(B, g, np.int32), U, W1, W2t, anchor,
                      d["tokens"], d["q"], u)
    assert list(v["accept_len"][:2]) == [2, 2]
    assert list(v["next_token"][:2]) == [V - 1, V - 1]    # 0.99 of a uniform bonus row
    assert v["flags"][2] & oracle.FLAG_NONFINITE
    assert v["accept_len"][2] == 0 and v["next_token"][2] == 0


def test_bonus_is_drawn_from_the_row_after_the_last_verified_draft():
    """When every verified draft is accepted, the extra token comes from the target's
    distribution at position l+1 ([V41] "投机解码：让小的先猜，大的一次验一串"), i.e. row l of the
    request's packed rows. Every row is a near point mass on its own token, so reading any
    other row gives another token. Lengths 3, 1, 2, 0 of gamma = 3 (packed rows)."""
    B, g, V = 4, 3, 8
    ell = np.array([3, 1, 2, 0], np.int32)
    U = np.zeros((B, g, V), np.float32)            # uniform draft
    W1, W2t = _zeros_w(V)
    anchor = np.zeros(B, np.int32)
    u = np.zeros((B, g + 1, 3), np.float32)        # draft token 0; accept whenever p_t(0) > 0
    u[:, :, 2] = 0.5
    d = oracle.markov_draft(U, W1, W2t, anchor, u)
    assert np.all(d["tokens"] == 0)
    offs = np.concatenate([[0], np.cumsum(1 + ell)]).astype(np.int32)
    rows, mass_tok = [], []
    for b in range(B):
        for k in range(ell[b] + 1):
            m = 1 + (3 * b + k) % (V - 1)          # never token 0, differs between rows k, k+1
            row = np.full(V, -1e30, np.float32)
            row[0] = 0.0                           # p_t(0) = e^-60 > 0: accepted at u = 0
            row[m] = 60.0
            rows.append(row)
            mass_tok.append(m)
    v = oracle.verify(np.stack(rows), offs, ell, U, W1, W2t, anchor, d["tokens"], d["q"], u)
    assert list(v["accept_len"]) == list(ell)
    expect = [mass_tok[offs[b] + ell[b]] for b in range(B)]
    assert list(v["next_token"]) == expect
    assert all(mass_tok[offs[b] + ell[b]] != mass_tok[offs[b] + ell[b] - 1]
               for b in range(B) if ell[b] > 0)
    assert np.all(v["beta_emit"] == -1.0)


def test_two_token_output_exact_grid_with_position_dependent_rows():
    """gamma = 1, V = 3, exact grid over the four uniforms used (draft, accept, resample,
    bonus). Target rows differ by position: row 1 is p_1 = (0.2, 0.3, 0.5), the bonus row is
    T2[x_1] (a table target chain). P(y_1 = a, accepted, y_2 = b) = min(p_d(a), p_1(a)) T2[a][b]
    and P(y_1 = a, rejected) = max(0, p_1(a) - p_d(a)) ([V41] "投机解码…"; [AIL] 02), so the
    counts over the 10^4 grid points are exact integers."""
    n = 10
    mid = (np.arange(n) + 0.5) / n
    G = np.stack(np.meshgrid(mid, mid, mid, mid, indexing="ij"), -1).reshape(-1, 4)
    B, g, V = n ** 4, 1, 3
    p_d = np.array([0.5, 0.3, 0.2])
    p_1 = np.array([0.2, 0.3, 0.5])
    T2 = np.array([[0.6, 0.3, 0.1], [0.1, 0.1, 0.8], [0.3, 0.4, 0.3]])
    U = np.tile(np.log(p_d).astype(np.float32), (B, g, 1))
    W1, W2t = _zeros_w(V)
    anchor = np.zeros(B, np.int32)
    u = np.zeros((B, g + 1, 3), np.float32)
    u[:, 0, 0], u[:, 0, 1], u[:, 0, 2], u[:, 1, 2] = G[:, 0], G[:, 1], G[:, 2], G[:, 3]
    d = oracle.markov_draft(U, W1, W2t, anchor, u)
    x1 = d["tokens"][:, 0]
    rows = np.stack([np.tile(np.log(p_1), (B, 1)), np.log(T2[x1])], 1).astype(np.float32)
    v = oracle.verify(rows.reshape(-1, V), dense_offsets(B, g), np.full(B, g, np.int32), U, W1,
                      W2t, anchor, d["tokens"], d["q"], u)
    acc = v["accept_len"] == 1
    y1 = first_emitted(d["tokens"], v["accept_len"], v["next_token"])
    joint = np.bincount(y1[acc] * V + v["next_token"][acc], minlength=V * V).reshape(V, V)
    expect = np.round(B * np.minimum(p_d, p_1)[:, None] * T2).astype(int)
    assert np.array_equal(joint, expect)
    rej = np.bincount(y1[~acc], minlength=V)
    assert np.array_equal(rej, np.round(B * np.maximum(0.0, p_1 - p_d)).astype(int))
