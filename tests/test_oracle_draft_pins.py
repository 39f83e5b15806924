"""Pins of the oracle's Markov-head draft and confidence head."""
import numpy as np
import pytest
from scipy import special

import oracle
from helpers import bf16_exact, bf16_round, bf16_to_f64, chi2_pvalue, logsumexp64, softmax64


def _unif(rng, B, g):
    return (rng.integers(0, 1 << 24, (B, g + 1, 3)) * 2.0 ** -24).astype(np.float32)


def _chain_tables(V=8, r=16, seed=0):
    """W1 = one-hot rows, W2 = a log-transition table in bf16-exact eighths: the Markov bias of
    previous token a is exactly row a of the table."""
    rng = np.random.default_rng(seed)
    Tm = rng.integers(-16, 17, (V, V)).astype(np.float32) / 8.0
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V)] = 1.0
    W2t = np.zeros((V, r), np.float32)
    W2t[:, :V] = Tm.T                       # W2t[v][i] = W2[i][v] = Tm[i][v]
    return Tm, bf16_exact(W1), bf16_exact(W2t)


def test_markov_chain_probabilities_closed_form():
    """With W1 one-hot and U = 0, p_k(v | x_{k-1} = a) = softmax(Tm[a])[v] exactly: checks that
    position k is biased by x_{k-1} (the anchor at k = 1), the same tables serve every
    position, and q, lse and the logits are those of one plain softmax."""
    V, g = 8, 4
    Tm, W1, W2t = _chain_tables(V)
    rng = np.random.default_rng(1)
    B = 256
    U = np.zeros((B, g, V), np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    force = rng.integers(0, V, (B, g)).astype(np.int32)
    d = oracle.markov_draft(U, W1, W2t, anchor, _unif(rng, B, g), force_tokens=force,
                            want_logits=True)
    prev = np.concatenate([anchor[:, None], force[:, :-1]], 1)
    P = softmax64(Tm, axis=1)
    assert np.array_equal(d["logits"], Tm[prev])
    assert np.allclose(d["q"], P[prev, force], rtol=0, atol=1e-7)
    assert np.allclose(d["lse"], logsumexp64(Tm, axis=1)[prev], rtol=0, atol=1e-13)


def test_markov_chain_draws_follow_transitions():
    """Sampled (unforced) drafts: transition counts from x_{k-1} to x_k follow the table."""
    V, g = 8, 4
    Tm, W1, W2t = _chain_tables(V, seed=3)
    rng = np.random.default_rng(2)
    B = 100_000
    anchor = rng.integers(0, V, B).astype(np.int32)
    d = oracle.markov_draft(np.zeros((B, g, V), np.float32), W1, W2t, anchor, _unif(rng, B, g))
    prev = np.concatenate([anchor[:, None], d["tokens"][:, :-1]], 1)
    P = softmax64(Tm, axis=1)
    for k in (0, g - 1):
        for a in range(V):
            sel = prev[:, k] == a
            counts = np.bincount(d["tokens"][sel, k], minlength=V)
            assert chi2_pvalue(counts, P[a]) > 1e-4


def test_w2_zero_reduces_to_inverse_cdf_categorical():
    """W2 = 0: every position is a plain categorical draw from softmax(U_k) by inverse CDF
    (numpy cumsum + searchsorted), independent of the previous token."""
    rng = np.random.default_rng(4)
    B, g, V, r = 64, 3, 1000, 16
    U = rng.normal(0, 2.0, (B, g, V)).astype(np.float32)
    W1 = bf16_round(rng.normal(0, 1, (V, r)))
    W2t = np.zeros((V, r), np.uint16)
    u = _unif(rng, B, g)
    d = oracle.markov_draft(U, W1, W2t, rng.integers(0, V, B).astype(np.int32), u,
                            want_logits=True)
    assert np.array_equal(d["logits"], U)
    P = softmax64(U, axis=2)
    ref = np.array([[np.searchsorted(np.cumsum(P[b, k]), u[b, k, 0], side="right")
                     for k in range(g)] for b in range(B)])
    ok = (ref == d["tokens"]) | (d["margin"] < 1e-12)
    assert ok.all()
    assert (ref == d["tokens"]).mean() > 0.99
    assert np.allclose(d["q"], np.take_along_axis(P, d["tokens"][..., None], 2)[..., 0], atol=1e-7)
    assert np.allclose(d["lse"], logsumexp64(U, axis=2), atol=1e-12)


def test_one_hot_embedding_selects_projection_column_and_bias_is_position_free():
    """W1[a] = e_i(a): the bias is column i(a) of W2 exactly; L = fp32(U + that column). With
    the same previous token at every position the bias L_k - U_k is identical across k."""
    rng = np.random.default_rng(6)
    B, g, V, r = 8, 4, 200, 32
    W1f = np.zeros((V, r), np.float32)
    idx = rng.integers(0, r, V)
    W1f[np.arange(V), idx] = 1.0
    W2t = bf16_round(rng.normal(0, 0.5, (V, r)))
    W2f = bf16_to_f64(W2t).astype(np.float32)
    U = rng.normal(0, 2.0, (B, g, V)).astype(np.float32)
    a = rng.integers(0, V, B).astype(np.int32)
    force = np.repeat(a[:, None], g, 1)
    d = oracle.markov_draft(U, bf16_exact(W1f), W2t, a, _unif(rng, B, g), force_tokens=force,
                            want_logits=True)
    bias = W2f[:, idx[a]].T                     # [B][V]: W2[idx(a), v]
    assert np.array_equal(d["logits"], U + bias[:, None, :])
    dl = d["logits"].astype(np.float64) - U
    assert np.allclose(dl, dl[:, :1, :], atol=2e-6)


def test_tiny_joint_by_exact_grid():
    """V = 3, gamma = 2: frequencies of (x1, x2) over a fine uniform grid match
    p_1(x1 | anchor) p_2(x2 | x1) within the grid resolution."""
    rng = np.random.default_rng(8)
    V, g, r, n = 3, 2, 16, 1000
    W1 = bf16_round(rng.normal(0, 1.0, (V, r)))
    W2t = bf16_round(rng.normal(0, 1.0, (V, r)))
    Ub = rng.normal(0, 1.0, (g, V)).astype(np.float32)
    B = n * n
    mid = ((np.arange(n) + 0.5) / n).astype(np.float32)
    u = np.zeros((B, g + 1, 3), np.float32)
    u[:, 0, 0] = np.repeat(mid, n)
    u[:, 1, 0] = np.tile(mid, n)
    anchor = np.full(B, 1, np.int32)
    d = oracle.markov_draft(np.broadcast_to(Ub, (B, g, V)).copy(), W1, W2t, anchor, u)
    freq = np.bincount(d["tokens"][:, 0] * V + d["tokens"][:, 1], minlength=V * V) / B
    E = bf16_to_f64(W1).reshape(V, r)
    W2 = bf16_to_f64(W2t).reshape(V, r).T
    bias = (E @ W2).astype(np.float32)           # [prev][v]
    p1 = softmax64(Ub[0] + bias[1])
    p2 = softmax64(Ub[1][None, :] + bias, axis=1)
    ref = (p1[:, None] * p2).ravel()
    assert np.abs(freq - ref).max() < 2.5 / n


def test_confidence_closed_forms():
    """c_k = sigmoid(z / T_k), z = w . [h_k; W1[x_{k-1}]]: a one-hot w picks a single hidden
    entry or a single entry of the previous token's embedding (the anchor at k = 1, x_{k-1}
    after); w = 0 gives 0.5."""
    rng = np.random.default_rng(9)
    B, g, V, r, d_ = 16, 4, 16, 16, 24
    h = bf16_round(rng.normal(0, 1, (B, g, d_)))
    W1f = (np.arange(V)[:, None] / 4.0 + np.arange(r)[None, :] / 64.0).astype(np.float32)
    W1 = bf16_exact(W1f)
    T = np.array([0.8, 1.0, 1.25, 1.5], np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    tokens = rng.integers(0, V, (B, g)).astype(np.int32)
    prev = np.concatenate([anchor[:, None], tokens[:, :-1]], 1)
    hf = bf16_to_f64(h).reshape(B, g, d_)
    # one-hot on hidden entry 5
    w = np.zeros(d_ + r, np.float32); w[5] = 1.0
    c = oracle.confidence(h, W1, bf16_exact(w), T, anchor, tokens)
    assert np.array_equal(c["z"], hf[:, :, 5])
    assert np.allclose(c["conf"], special.expit(hf[:, :, 5] / T), atol=1e-7)
    # one-hot on embedding entry 3 of the previous token
    w = np.zeros(d_ + r, np.float32); w[d_ + 3] = 1.0
    c = oracle.confidence(h, W1, bf16_exact(w), T, anchor, tokens)
    assert np.array_equal(c["z"], W1f[prev, 3].astype(np.float64))
    assert np.allclose(c["conf"], special.expit(W1f[prev, 3] / T), atol=1e-7)
    # zero weights
    c = oracle.confidence(h, W1, np.zeros(d_ + r, np.uint16), T, anchor, tokens)
    assert np.all(c["conf"] == 0.5)
    # linearity in w: z(w_a + w_b) = z(w_a) + z(w_b) for bf16-exact small integers
    wa = np.zeros(d_ + r, np.float32); wa[:d_] = rng.integers(-3, 4, d_)
    wb = np.zeros(d_ + r, np.float32); wb[d_:] = rng.integers(-3, 4, r)
    za = oracle.confidence(h, W1, bf16_exact(wa), T, anchor, tokens)["z"]
    zb = oracle.confidence(h, W1, bf16_exact(wb), T, anchor, tokens)["z"]
    zab = oracle.confidence(h, W1, bf16_exact(wa + wb), T, anchor, tokens)["z"]
    assert np.allclose(zab, za + zb, atol=1e-12)
