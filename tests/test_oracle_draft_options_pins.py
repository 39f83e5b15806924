"""Pins of the oracle's draft options: the sampling temperature of the official draft loop
([V41] "Markov head", the serial loop samples with a temperature) and the greedy draft of the
deployed recipe ([V41] / [AIL], draft_sample_method "greedy"). Limits and closed forms of the
draft, and the lossless property of the verify for tempered and greedy drafts (the first
emitted token follows the target whatever the draft distribution)."""
import numpy as np
import pytest

import oracle
from helpers import dense_offsets, first_emitted
from test_oracle_draft_pins import _chain_tables


def _zeros_w(V, r=16):
    return np.zeros((V, r), np.uint16), np.zeros((V, r), np.uint16)


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _one_position(U_row, n):
    """n requests with the same base logits for one position, draw uniforms on a midpoint grid."""
    V = len(U_row)
    U = np.tile(np.asarray(U_row, np.float32), (n, 1)).reshape(n, 1, V)
    u = np.zeros((n, 2, 3), np.float32)
    u[:, 0, 0] = (np.arange(n) + 0.5) / n
    return U, u


def test_temperature_one_is_the_default_path():
    rng = np.random.default_rng(7)
    B, g, V, r = 3, 4, 50, 16
    U = rng.normal(0, 2, (B, g, V)).astype(np.float32)
    W1 = _bf16_bits(rng.normal(0, 0.1, (V, r)))
    W2t = _bf16_bits(rng.normal(0, 0.1, (V, r)))
    anchor = rng.integers(0, V, B).astype(np.int32)
    u = rng.uniform(0, 1, (B, g + 1, 3)).astype(np.float32)
    a = oracle.markov_draft(U, W1, W2t, anchor, u)
    b = oracle.markov_draft(U, W1, W2t, anchor, u, temperature=1.0)
    for k in ("tokens", "q", "lse", "margin"):
        assert np.array_equal(a[k], b[k]), k


def test_temperature_limits_uniform_and_argmax():
    """A very high temperature flattens the draft to uniform; a very low one puts every draw on
    the largest logit."""
    V = 5
    row = np.array([0.5, -1.0, 2.0, 1.0, 0.0], np.float32)
    U, u = _one_position(row, 200)
    W1, W2t = _zeros_w(V)
    anchor = np.zeros(len(U), np.int32)
    hot = oracle.markov_draft(U, W1, W2t, anchor, u, temperature=1e6)
    assert np.allclose(hot["q"], 1.0 / V, atol=1e-5)
    assert np.allclose(hot["lse"], np.log(V), atol=1e-5)
    assert np.array_equal(np.bincount(hot["tokens"][:, 0], minlength=V), np.full(V, 40))
    cold = oracle.markov_draft(U, W1, W2t, anchor, u, temperature=1e-3)
    assert np.all(cold["tokens"] == 2)
    assert np.allclose(cold["q"], 1.0)


@pytest.mark.parametrize("tau", [0.5, 2.0])
def test_tempered_draw_frequencies_exact_grid(tau):
    """On a midpoint grid of n uniforms, the count of each token is n p_v up to one, with
    p = softmax(L / tau): a sharper draft below tau = 1, a flatter one above."""
    V, n = 4, 4000
    row = np.array([0.0, 1.0, 2.0, 0.5], np.float32)
    U, u = _one_position(row, n)
    W1, W2t = _zeros_w(V)
    d = oracle.markov_draft(U, W1, W2t, np.zeros(n, np.int32), u, temperature=tau)
    x = row.astype(np.float64) / tau
    p = np.exp(x - x.max())
    p /= p.sum()
    counts = np.bincount(d["tokens"][:, 0], minlength=V)
    assert np.all(np.abs(counts - n * p) <= 1.0 + 1e-9), (counts, n * p)
    assert np.allclose(d["q"][:, 0], p[d["tokens"][:, 0]], rtol=1e-6)
    sharper = tau < 1.0
    assert (p.max() > np.exp(row.max()) / np.exp(row).sum()) == sharper


def test_greedy_draft_closed_form_and_ties():
    V = 6
    W1, W2t = _zeros_w(V)
    U = np.array([[[0.0, 1.5, -2.0, 3.0, 2.5, 0.0]], [[1.0, 4.0, 0.0, 0.5, 4.0, 3.5]]], np.float32)
    u = np.full((2, 2, 3), 0.37, np.float32)
    d = oracle.markov_draft(U, W1, W2t, np.zeros(2, np.int32), u, greedy=True)
    assert list(d["tokens"][:, 0]) == [3, 1]                 # first maximum on the tie
    assert np.all(d["q"] == 1.0)
    assert list(d["lse"][:, 0]) == [3.0, 4.0]
    assert d["margin"][0, 0] == pytest.approx(0.5) and d["margin"][1, 0] == 0.0
    forced = oracle.markov_draft(U, W1, W2t, np.zeros(2, np.int32), u, greedy=True,
                                 force_tokens=np.array([[3], [4]], np.int32))
    assert list(forced["q"][:, 0]) == [1.0, 0.0]             # point mass: other tokens have 0


def test_greedy_path_follows_the_most_likely_transitions():
    """With U = 0 and one-hot embeddings the draft logits are the log transition probabilities
    of a Markov chain, so the greedy draft is the chain's most-likely-next-token path."""
    V, g = 8, 6
    Tm, W1, W2t = _chain_tables(V)
    anchor = np.arange(V, dtype=np.int32)
    U = np.zeros((V, g, V), np.float32)
    u = np.full((V, g + 1, 3), 0.5, np.float32)
    d = oracle.markov_draft(U, W1, W2t, anchor, u, greedy=True)
    for b in range(V):
        prev = b
        for k in range(g):
            assert d["tokens"][b, k] == int(np.argmax(Tm[prev]))
            prev = d["tokens"][b, k]


def test_greedy_verify_is_lossless_exact_grid():
    """Greedy draft x (q = 1): accepted iff u < p_t(x); on a reject the correction draws from p_t
    without x; so the first emitted token follows p_t exactly. beta = p_t(x), residual mass
    1 - p_t(x)."""
    V, n = 4, 60
    pt = np.array([0.1, 0.2, 0.3, 0.4])
    row = np.array([0.0, 1.0, 3.0, 2.0], np.float32)        # greedy draft: token 2
    B = n * n
    U = np.tile(row, (B, 1)).reshape(B, 1, V)
    W1, W2t = _zeros_w(V)
    anchor = np.zeros(B, np.int32)
    mid = (np.arange(n) + 0.5) / n
    ua, ue = np.meshgrid(mid, mid, indexing="ij")
    u = np.zeros((B, 2, 3), np.float32)
    u[:, 0, 1] = ua.ravel()
    u[:, 0, 2] = ue.ravel()
    u[:, 1, 2] = ue.ravel()
    d = oracle.markov_draft(U, W1, W2t, anchor, u, greedy=True)
    assert np.all(d["tokens"] == 2) and np.all(d["q"] == 1.0)
    target = np.tile(np.log(pt).astype(np.float32), (2 * B, 1))
    v = oracle.verify(target, dense_offsets(B, 1), np.ones(B, np.int32), U, W1, W2t, anchor,
                      d["tokens"], d["q"], u, greedy=True)
    assert (v["accept_len"] == 1).mean() == pytest.approx(pt[2], abs=1.0 / n)
    rej = v["accept_len"] == 0
    assert np.all(v["next_token"][rej] != 2)
    assert np.allclose(v["beta_emit"][rej], pt[2], atol=1e-6)
    assert np.allclose(v["resid_mass"][rej], 1.0 - pt[2], atol=1e-6)
    y = first_emitted(d["tokens"], v["accept_len"], v["next_token"])
    assert np.allclose(np.bincount(y, minlength=V) / B, pt, atol=2.0 / n)


@pytest.mark.parametrize("tau", [0.5, 1.7])
def test_tempered_verify_is_lossless_exact_grid(tau):
    """Draft at temperature tau, verify against p_t: the first emitted token follows p_t, and
    beta on a reject is sum_v min(p_t, p_d) for the tempered p_d."""
    V, n = 3, 24
    pt = np.array([0.5, 0.2, 0.3])
    row = np.array([0.4, -0.3, 1.1], np.float32)
    x = row.astype(np.float64) / tau
    pd = np.exp(x - x.max())
    pd /= pd.sum()
    B = n ** 3
    U = np.tile(row, (B, 1)).reshape(B, 1, V)
    W1, W2t = _zeros_w(V)
    anchor = np.zeros(B, np.int32)
    mid = (np.arange(n) + 0.5) / n
    i, j, l = np.meshgrid(mid, mid, mid, indexing="ij")
    u = np.zeros((B, 2, 3), np.float32)
    u[:, 0, 0], u[:, 0, 1], u[:, 0, 2], u[:, 1, 2] = i.ravel(), j.ravel(), l.ravel(), l.ravel()
    d = oracle.markov_draft(U, W1, W2t, anchor, u, temperature=tau)
    target = np.tile(np.log(pt).astype(np.float32), (2 * B, 1))
    v = oracle.verify(target, dense_offsets(B, 1), np.ones(B, np.int32), U, W1, W2t, anchor,
                      d["tokens"], d["q"], u, temperature=tau)
    rej = v["accept_len"] == 0
    assert rej.any()
    assert np.allclose(v["beta_emit"][rej], np.minimum(pt, pd).sum(), atol=1e-6)
    y = first_emitted(d["tokens"], v["accept_len"], v["next_token"])
    assert np.allclose(np.bincount(y, minlength=V) / B, pt, atol=3.0 / n)
