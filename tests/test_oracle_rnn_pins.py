"""Pins of the oracle's RNN head, eq. (6) ([CSDN] 4.2 "两种串行头"; [AIL] "RNN 头（可选）"):
z_k = [s_{k-1}; W1[x_{k-1}]; h_k], s_k = sigma(W_g z) s_{k-1} + (1 - sigma(W_g z)) tanh(W_c z),
B_k = W2^T tanh(W_o z). Weight blocks chosen so that the head reduces to closed forms computed
here in numpy: the output path alone (e_k = tanh(W1[x_{k-1}]), a first-order chain), the state
path alone with a half-open gate (s_k = (s_{k-1} + c_k) / 2, e_k = tanh(s_{k-1})), the two
saturated gates, and the verify of such drafts (the draft distribution of a rejected position
recomputed along the drafted tokens; the first emitted token follows the target)."""
import numpy as np
import pytest

import oracle
from helpers import dense_offsets, first_emitted


def to_bits(x):
    """float -> bf16 bits (truncation; the float value used below is the bf16 one)."""
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def from_bits(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _setup(rng, B=6, g=4, V=40, r=16, d=8):
    W1 = to_bits(rng.normal(0, 0.8, (V, r)))
    W2t = to_bits(rng.normal(0, 0.5, (V, r)))
    h = to_bits(rng.normal(0, 1, (B, g, d)))
    U = rng.normal(0, 1, (B, g, V)).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    u = rng.uniform(0, 1, (B, g + 1, 3)).astype(np.float32)
    return W1, W2t, h, U, anchor, u


def _logits(U_row, W2t, e):
    bias = from_bits(W2t) @ e
    return (U_row.astype(np.float32) + bias.astype(np.float32)).astype(np.float32)


def _softmax(L):
    x = L.astype(np.float64)
    p = np.exp(x - x.max())
    return p / p.sum()


def _draw(p, u):
    c = np.cumsum(p)
    v = int(np.searchsorted(c, u, side="right"))
    margin = min(abs(u - (c[v - 1] if v else 0.0)), abs(c[v] - u)) if v < len(p) else 0.0
    return min(v, len(p) - 1), margin


def _check_chain(d, U, W2t, u, e_ref_fn):
    """e_ref_fn(b, k, x_prev) -> e_k (numpy, fp64). Checks e, logits, q and the draws."""
    B, g, V = U.shape
    for b in range(B):
        for k in range(g):
            x_prev = None if k == 0 else d["tokens"][b, k - 1]
            e = e_ref_fn(b, k, x_prev)
            assert np.allclose(d["e"][b, k], e, rtol=0, atol=1e-14), (b, k)
            L = _logits(U[b, k], W2t, e)
            assert np.abs(d["logits"][b, k] - L).max() <= 1e-6
            p = _softmax(d["logits"][b, k])
            x, margin = _draw(p, float(u[b, k, 0]))
            if margin > 1e-12:
                assert d["tokens"][b, k] == x, (b, k)
            assert d["q"][b, k] == pytest.approx(p[d["tokens"][b, k]], abs=1e-7)


def test_output_path_is_a_tanh_embedding_chain():
    """W_o reads only the embedding block (identity), all else zero: e_k = tanh(W1[x_{k-1}]),
    so the RNN head is a first-order chain with embedding tanh(W1) (x_0 = the anchor)."""
    rng = np.random.default_rng(1)
    W1, W2t, h, U, anchor, u = _setup(rng)
    r, dd = W1.shape[1], h.shape[2]
    Wg = np.zeros((3 * r, 2 * r + dd), np.float32)
    Wg[2 * r + np.arange(r), r + np.arange(r)] = 1.0
    d = oracle.rnn_draft(U, W1, W2t, to_bits(Wg), h, anchor, u, want_logits=True)
    W1f = from_bits(W1)
    _check_chain(d, U, W2t, u,
                 lambda b, k, xp: np.tanh(W1f[anchor[b] if xp is None else xp]))


def test_state_path_half_gate_closed_form():
    """W_g = 0 (gate 1/2), W_c reads only the hidden block (c_k = tanh(Mc h_k)), W_o reads only
    the state block (identity): s_k = (s_{k-1} + c_k) / 2 from s_0 = 0, e_k = tanh(s_{k-1})."""
    rng = np.random.default_rng(2)
    W1, W2t, h, U, anchor, u = _setup(rng)
    r, dd = W1.shape[1], h.shape[2]
    Mc = to_bits(rng.normal(0, 0.7, (r, dd)))
    Wg = np.zeros((3 * r, 2 * r + dd), np.float32)
    Wg[r:2 * r, 2 * r:] = from_bits(Mc)
    Wg[2 * r + np.arange(r), np.arange(r)] = 1.0
    d = oracle.rnn_draft(U, W1, W2t, to_bits(Wg), h, anchor, u, want_logits=True)
    hf, Mcf = from_bits(h), from_bits(Mc)
    states = {}
    for b in range(U.shape[0]):
        s = np.zeros(r)
        for k in range(U.shape[1]):
            states[b, k] = np.tanh(s)
            s = 0.5 * s + 0.5 * np.tanh(Mcf @ hf[b, k])
    _check_chain(d, U, W2t, u, lambda b, k, xp: states[b, k])


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_saturated_gates(sign):
    """h_k[0] = 1 and W_g = 40 sign on that column: the gate is 1 (fp64) for sign = +1, so the
    state never leaves 0 and e_k = tanh(0) = 0; for sign = -1 the gate is ~4e-18, so s_k = c_k
    and e_{k+1} = tanh(tanh(Mc h_k))."""
    rng = np.random.default_rng(3)
    W1, W2t, h, U, anchor, u = _setup(rng)
    r, dd = W1.shape[1], h.shape[2]
    hf = from_bits(h)
    hf[..., 0] = 1.0
    h = to_bits(hf)
    Mc = np.zeros((r, dd))
    Mc[:, 1:] = from_bits(to_bits(rng.normal(0, 0.7, (r, dd - 1))))
    Wg = np.zeros((3 * r, 2 * r + dd), np.float32)
    Wg[:r, 2 * r] = 40.0 * sign
    Wg[r:2 * r, 2 * r:] = Mc
    Wg[2 * r + np.arange(r), np.arange(r)] = 1.0
    d = oracle.rnn_draft(U, W1, W2t, to_bits(Wg), h, anchor, u, want_logits=True)
    hf = from_bits(h)
    for b in range(U.shape[0]):
        for k in range(U.shape[1]):
            if sign > 0 or k == 0:
                assert np.all(d["e"][b, k] == 0.0)
            else:
                ref = np.tanh(np.tanh(Mc @ hf[b, k - 1]))
                assert np.allclose(d["e"][b, k], ref, rtol=0, atol=1e-14)


def test_zero_weights_reduce_to_categorical_sampling():
    rng = np.random.default_rng(4)
    W1, W2t, h, U, anchor, u = _setup(rng)
    r, dd = W1.shape[1], h.shape[2]
    Wz = np.zeros((3 * r, 2 * r + dd), np.uint16)
    d = oracle.rnn_draft(U, W1, W2t, Wz, h, anchor, u, want_logits=True)
    assert np.all(d["e"] == 0.0)
    assert np.array_equal(d["logits"], U)
    _check_chain(d, U, W2t, u, lambda b, k, xp: np.zeros(r))


def test_greedy_and_temperature_follow_the_markov_rules():
    """The draft options act on the RNN logits as on the Markov ones: greedy takes the first
    maximum (q = 1, lse = that logit), a temperature scales the logits by fp32(1/tau)."""
    rng = np.random.default_rng(5)
    W1, W2t, h, U, anchor, u = _setup(rng)
    r, dd = W1.shape[1], h.shape[2]
    Wg = to_bits(rng.normal(0, 0.2, (3 * r, 2 * r + dd)))
    base = oracle.rnn_draft(U, W1, W2t, Wg, h, anchor, u, want_logits=True, greedy=True)
    assert np.array_equal(base["tokens"], base["logits"].argmax(axis=2))
    assert np.all(base["q"] == 1.0)
    assert np.array_equal(base["lse"], base["logits"].max(axis=2).astype(np.float64))
    hot = oracle.rnn_draft(U, W1, W2t, Wg, h, anchor, u, want_logits=True, temperature=0.5,
                           force_tokens=base["tokens"])
    for b in range(U.shape[0]):
        for k in range(U.shape[1]):
            L = hot["logits"][b, k] * np.float32(2.0)
            p = _softmax(L)
            assert hot["q"][b, k] == pytest.approx(p[base["tokens"][b, k]], abs=1e-7)


def _verify_case(kind, seed):
    """Position 1 always accepted (the target puts all its mass on x_1), position 2 tested
    against a random target: on a reject at 2, beta = sum min(p_t, p_d) with p_d of position 2
    from the state and embedding after x_1."""
    rng = np.random.default_rng(seed)
    B, g, V, r, dd = 64, 2, 12, 8, 6
    W1, W2t, h, U, anchor, u = _setup(rng, B, g, V, r, dd)
    Wg = np.zeros((3 * r, 2 * r + dd), np.float32)
    if kind == "embedding":
        Wg[2 * r + np.arange(r), r + np.arange(r)] = 1.0
    else:
        Mc = from_bits(to_bits(rng.normal(0, 1.0, (r, dd))))
        Mx = from_bits(to_bits(rng.normal(0, 1.0, (r, r))))
        Wg[r:2 * r, 2 * r:] = Mc
        Wg[r:2 * r, r:2 * r] = Mx
        Wg[2 * r + np.arange(r), np.arange(r)] = 1.0
    Wb = to_bits(Wg)
    d = oracle.rnn_draft(U, W1, W2t, Wb, h, anchor, u, want_logits=True)
    x1 = d["tokens"][:, 0]
    t1 = np.zeros((B, V), np.float32)
    t1[np.arange(B), x1] = 50.0
    t2 = rng.normal(0, 2, (B, V)).astype(np.float32)
    t3 = rng.normal(0, 2, (B, V)).astype(np.float32)
    target = np.stack([t1, t2, t3], 1).reshape(3 * B, V)
    v = oracle.rnn_verify(target, dense_offsets(B, 2), np.full(B, 2, np.int32), U, W1, W2t, Wb, h,
                          anchor, d["tokens"], d["q"], u)
    assert np.all(v["accept_len"] >= 1)
    rej = v["accept_len"] == 1
    assert rej.sum() >= 10
    for b in np.flatnonzero(rej):
        pd = _softmax(d["logits"][b, 1])   # the draft's own logits of position 2 (pinned above)
        pt = _softmax(t2[b])
        assert v["beta_emit"][b] == pytest.approx(np.minimum(pt, pd).sum(), abs=1e-6)
        assert v["resid_mass"][b] == pytest.approx(np.maximum(pt - pd, 0).sum(), abs=1e-12)
    return v


@pytest.mark.parametrize("kind", ["embedding", "state"])
def test_verify_recomputes_the_draft_distribution_along_the_drafted_tokens(kind):
    _verify_case(kind, 11 if kind == "embedding" else 12)


def test_rnn_verify_is_lossless_exact_grid():
    """One position, exact midpoint grid over (draw, accept, emission) uniforms: the first
    emitted token follows p_t whatever the RNN draft distribution."""
    V, n = 3, 30
    rng = np.random.default_rng(13)
    r, dd = 4, 3
    B = n ** 3
    W1 = to_bits(rng.normal(0, 1, (V, r)))
    W2t = to_bits(rng.normal(0, 1, (V, r)))
    Wg = to_bits(rng.normal(0, 0.8, (3 * r, 2 * r + dd)))
    h = np.tile(to_bits(rng.normal(0, 1, (1, 1, dd))), (B, 1, 1))
    U = np.tile(np.array([0.3, -0.2, 0.5], np.float32), (B, 1)).reshape(B, 1, V)
    anchor = np.zeros(B, np.int32)
    mid = (np.arange(n) + 0.5) / n
    i, j, l = np.meshgrid(mid, mid, mid, indexing="ij")
    u = np.zeros((B, 2, 3), np.float32)
    u[:, 0, 0], u[:, 0, 1], u[:, 0, 2], u[:, 1, 2] = i.ravel(), j.ravel(), l.ravel(), l.ravel()
    d = oracle.rnn_draft(U, W1, W2t, Wg, h, anchor, u)
    pt = np.array([0.2, 0.5, 0.3])
    target = np.tile(np.log(pt).astype(np.float32), (2 * B, 1))
    v = oracle.rnn_verify(target, dense_offsets(B, 1), np.ones(B, np.int32), U, W1, W2t, Wg, h,
                          anchor, d["tokens"], d["q"], u)
    y = first_emitted(d["tokens"], v["accept_len"], v["next_token"])
    assert np.allclose(np.bincount(y, minlength=V) / B, pt, atol=3.0 / n)
