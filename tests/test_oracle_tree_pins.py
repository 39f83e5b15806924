"""Pins of the oracle's PCTree draft (children scored by the Markov head, the most likely paths
kept within a verify budget; [ZDS] "后续工作") and of its lossless tree verify."""
import itertools

import numpy as np
import pytest

import oracle
from helpers import bf16_exact, bf16_round, chi2_pvalue, softmax64


def _chain_tables(V, r=16, seed=0):
    """W1 one-hot rows and W2 a log-transition table in bf16-exact eighths: the Markov bias
    under previous token a is exactly row a of the table (V <= r)."""
    rng = np.random.default_rng(seed)
    Tm = rng.integers(-24, 25, (V, V)).astype(np.float32) / 8.0
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V)] = 1.0
    W2t = np.zeros((V, r), np.float32)
    W2t[:, :V] = Tm.T
    return Tm, bf16_exact(W1), bf16_exact(W2t)


def _paths(t, b):
    """The kept nodes of request b as token sequences from the root, in rank order."""
    out = []
    for n in range(t["token"].shape[1]):
        seq, m = [], n
        while m >= 0:
            seq.append(int(t["token"][b, m]))
            m = int(t["parent"][b, m])
        out.append(tuple(reversed(seq)))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_kept_nodes_are_the_most_likely_paths_brute_force(seed):
    """Every child scored (c = V), every depth-1 node expanded (M = c), gamma = 2: the kept set
    must be the N most likely token sequences of length 1 and 2 under the Markov chain, found by
    enumerating all of them; each kept node's path probability is the product of the chain's
    transition probabilities (softmax of U_k plus the table row of the previous token)."""
    rng = np.random.default_rng(seed)
    V, g = 4, 2
    Tm, W1, W2t = _chain_tables(V, seed=seed)
    B = 6
    U = (rng.integers(-16, 17, (B, g, V)) / 8.0).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    N = int(rng.integers(1, V + V * V + 1))
    t = oracle.tree_draft(U, W1, W2t, anchor, V, V, N)
    for b in range(B):
        prob = {}
        p1 = softmax64(U[b, 0].astype(np.float64) + Tm[anchor[b]])
        for a in range(V):
            prob[(a,)] = p1[a]
            p2 = softmax64(U[b, 1].astype(np.float64) + Tm[a])
            for c in range(V):
                prob[(a, c)] = p1[a] * p2[c]
        ranked = sorted(prob.items(), key=lambda kv: (-kv[1], len(kv[0])))
        # ties at the budget's edge would leave the set undetermined: skip such draws
        if N < len(ranked) and abs(ranked[N - 1][1] - ranked[N][1]) < 1e-12:
            continue
        kept = _paths(t, b)
        assert set(kept) == {k for k, _ in ranked[:N]}
        for n, seq in enumerate(kept):
            assert t["path"][b, n] == pytest.approx(prob[seq], rel=1e-12)
            assert t["depth"][b, n] == len(seq)


def test_w2_zero_children_are_the_top_c_of_the_base_logits():
    """W2 = 0: the Markov bias vanishes, so every node of depth k has the same children, the c
    largest entries of U_k (the smaller id first on ties), with q = softmax(U_k) and P the
    product of q along the path."""
    rng = np.random.default_rng(3)
    B, g, V, r, c, M = 5, 3, 40, 16, 3, 2
    U = rng.normal(0, 2.0, (B, g, V)).astype(np.float32)
    U[0, 1, [7, 9]] = 9.0                                  # an exact tie inside the top c
    W1 = bf16_round(rng.normal(0, 0.5, (V, r)))
    W2t = np.zeros((V, r), np.uint16)
    anchor = rng.integers(0, V, B).astype(np.int32)
    total = oracle.tree_candidates(g, c, M)
    t = oracle.tree_draft(U, W1, W2t, anchor, c, M, total)
    for b in range(B):
        tops = [np.lexsort((np.arange(V), -U[b, k].astype(np.float64)))[:c] for k in range(g)]
        q = [softmax64(U[b, k]) for k in range(g)]
        for n in range(total):
            k = t["depth"][b, n] - 1
            assert t["token"][b, n] in tops[k]
            assert t["q"][b, n] == pytest.approx(q[k][t["token"][b, n]], rel=1e-13)
            par = t["parent"][b, n]
            parent_P = 1.0 if par < 0 else t["path"][b, par]
            assert t["path"][b, n] == pytest.approx(parent_P * t["q"][b, n], rel=1e-13)
        # children of every expanded node of a depth: the same c tokens, in rank order
        for par in [-1] + list(range(total)):
            kids = [t["token"][b, n] for n in range(total) if t["parent"][b, n] == par]
            if kids:
                k = 0 if par < 0 else t["depth"][b, par]
                assert kids == list(tops[k])
    assert list(np.lexsort((np.arange(V), -U[0, 1].astype(np.float64)))[:2]) == [7, 9]


@pytest.mark.parametrize("seed", range(10))
def test_tree_structure_beam_and_budget(seed):
    """Random Markov heads: parents rank before their children, depth = parent depth + 1,
    P = parent P times q, q is the Markov probability of the token under its parent (numpy
    softmax of the table row), the expanded nodes of each depth are its M most likely ones,
    and the kept nodes are the N most likely candidates (P non-increasing in rank order)."""
    rng = np.random.default_rng(50 + seed)
    V, g = 6, 4
    Tm, W1, W2t = _chain_tables(V, seed=seed + 7)
    c, M = int(rng.integers(2, 5)), int(rng.integers(1, 3))
    B = 4
    U = (rng.integers(-16, 17, (B, g, V)) / 8.0).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    total = oracle.tree_candidates(g, c, M)
    full = oracle.tree_draft(U, W1, W2t, anchor, c, M, total)
    N = int(rng.integers(1, total + 1))
    t = oracle.tree_draft(U, W1, W2t, anchor, c, M, N)
    for b in range(B):
        P = full["path"][b]
        assert np.all(np.diff(P) <= 0)
        for n in range(total):
            par = full["parent"][b, n]
            prev = anchor[b] if par < 0 else full["token"][b, par]
            k = full["depth"][b, n]
            assert par < n and (par < 0 or full["depth"][b, par] == k - 1)
            q = softmax64(U[b, k - 1].astype(np.float64) + Tm[prev])
            assert full["q"][b, n] == pytest.approx(q[full["token"][b, n]], rel=1e-12)
        for k in range(1, g):
            depth_k = [n for n in range(total) if full["depth"][b, n] == k]
            expanded = {full["parent"][b, n] for n in range(total) if full["depth"][b, n] == k + 1}
            assert expanded == set(depth_k[:min(M, len(depth_k))])
        assert _paths(t, b) == _paths(full, b)[:N]


def _walk_case(rows_of, V, tree, grid):
    """Exact grid over the draws at depths 0 and 1 for a fixed tree; rows_of(path) gives the
    target logits after a path. Returns the emitted sequences (accepted path + next token)."""
    tok, dep, par = tree
    N = len(tok)
    mid = (np.arange(grid) + 0.5) / grid
    u0, u1 = np.meshgrid(mid, mid, indexing="ij")
    B = grid * grid
    g = 2
    uni = np.zeros((B, g + 1, 3), np.float32)
    uni[:, 0, 2], uni[:, 1, 2] = u0.ravel(), u1.ravel()
    uni[:, 2, 2] = 0.5
    paths = []
    for n in range(N):
        seq, m = [], n
        while m >= 0:
            seq.append(tok[m])
            m = par[m]
        paths.append(tuple(reversed(seq)))
    rows = np.stack([rows_of(())] + [rows_of(p) for p in paths]).astype(np.float32)
    target = np.broadcast_to(rows, (B,) + rows.shape).copy()
    rep = lambda a: np.tile(np.asarray(a, np.int32), (B, 1))
    v = oracle.tree_verify(target, rep(tok), rep(dep), rep(par), uni)
    out = []
    for b in range(B):
        acc = v["path"][b, :v["accept_len"][b]].tolist()
        out.append(tuple(acc) + (int(v["next_token"][b]),))
    return out, v


def test_tree_verify_exact_grid_follows_the_target_chain():
    """A fixed tree on V = 4 (root children 2, 0; node 2 has children 1, 3; node 0 has child 2)
    and target rows that depend on the path. Over an exact grid of the two draws, the first
    emitted token follows p_t after the anchor, and the second (when the first was a tree node
    and the walk continued) follows p_t after it, exactly: the tree never changes the target's
    distribution, and a correction never re-emits a child it rejected."""
    V = 4
    T1 = np.array([0.3, 0.1, 0.4, 0.2])
    T2 = {0: np.array([0.1, 0.2, 0.5, 0.2]), 2: np.array([0.2, 0.3, 0.1, 0.4])}
    def rows_of(path):
        if len(path) == 0:
            return np.log(T1)
        if len(path) == 1:
            return np.log(T2[path[0]])
        return np.log(np.full(V, 0.25))
    tree = ([2, 0, 1, 3, 2], [1, 1, 2, 2, 2], [-1, -1, 0, 0, 1])
    grid = 20
    seqs, v = _walk_case(rows_of, V, tree, grid)
    B = grid * grid
    first = np.bincount([s[0] for s in seqs], minlength=V)
    assert list(first) == [int(round(B * p)) for p in T1]
    for a in (0, 2):
        second = np.bincount([s[1] for s in seqs if s[0] == a], minlength=V)
        n_a = int(round(B * T1[a]))
        assert list(second) == [int(round(n_a * p)) for p in T2[a]]
    # a walk stops at a token that is not a child of where it stands
    kids = {(): {2, 0}, (2,): {1, 3}, (0,): {2}}
    for s in seqs:
        assert s[-1] not in kids.get(s[:-1], set())
    assert np.all(v["accept_len"] == np.array([len(s) - 1 for s in seqs]))


def test_tree_verify_accept_probability_is_the_children_mass():
    """P(the walk accepts at the root) = sum of p_t over the root's children (exact grid)."""
    V = 4
    T1 = np.array([0.35, 0.15, 0.3, 0.2])
    rows_of = lambda path: np.log(T1) if not path else np.log(np.full(V, 0.25))
    tree = ([2, 3], [1, 1], [-1, -1])
    seqs, v = _walk_case(rows_of, V, tree, 20)
    assert (v["accept_len"] >= 1).mean() == pytest.approx(T1[2] + T1[3], abs=1e-12)


def test_single_child_chain_is_the_point_mass_rule():
    """c = M = 1, N = gamma: the tree is one chain of most likely tokens (a greedy draft). The walk
    accepts x_1 with probability p_t(x_1), and after a reject the emitted token is never x_1 and
    follows p_t without x_1, the point-mass rule of the greedy draft's verify."""
    V, g = 4, 2
    Tm, W1, W2t = _chain_tables(V, seed=4)
    U = np.zeros((1, g, V), np.float32)
    t = oracle.tree_draft(U, W1, W2t, np.array([1], np.int32), 1, 1, g)
    x1 = int(t["token"][0, 0])
    assert x1 == int(np.argmax(Tm[1])) and list(t["parent"][0]) == [-1, 0]
    T1 = np.array([0.1, 0.4, 0.2, 0.3])
    rows_of = lambda path: np.log(T1) if not path else np.log(np.full(V, 0.25))
    tree = (t["token"][0].tolist(), t["depth"][0].tolist(), t["parent"][0].tolist())
    seqs, v = _walk_case(rows_of, V, tree, 20)
    B = len(seqs)
    acc = v["accept_len"] >= 1
    assert acc.mean() == pytest.approx(T1[x1], abs=1e-12)
    rej = np.bincount([s[0] for s, a in zip(seqs, acc) if not a], minlength=V)
    expect = T1.copy()
    expect[x1] = 0.0
    assert list(rej) == [int(round(B * p)) for p in expect]


@pytest.mark.parametrize("N", [3, 9])
def test_tree_verify_chi2_random_trees(N):
    """Random Markov heads, trees and target rows on V = 4 (10^5 requests): the first emitted
    token follows p_t after the anchor, and, given the first two tokens came from the tree walk,
    the second follows p_t after the first."""
    rng = np.random.default_rng(N)
    B, g, V = 100_000, 3, 4
    Tm, W1, W2t = _chain_tables(V, seed=N)
    U0 = rng.normal(0, 1.0, (g, V)).astype(np.float32)
    U = np.broadcast_to(U0, (B, g, V)).copy()
    anchor = np.zeros(B, np.int32)
    t = oracle.tree_draft(U[:1], W1, W2t, anchor[:1], 2, 2, N)
    tree = [np.tile(t[k], (B, 1)) for k in ("token", "depth", "parent")]
    R1 = rng.normal(0, 1.0, V)
    R2 = rng.normal(0, 1.0, (V, V))
    rows = np.zeros((N + 1, V))
    rows[0] = R1
    for n in range(N):
        rows[1 + n] = R2[t["token"][0, n]] if t["depth"][0, n] == 1 else rng.normal(0, 1, V)
    target = np.broadcast_to(rows.astype(np.float32), (B, N + 1, V)).copy()
    uni = (rng.integers(0, 1 << 24, (B, g + 1, 3)) * 2.0 ** -24).astype(np.float32)
    v = oracle.tree_verify(target, *tree, uni)
    y1 = np.where(v["accept_len"] >= 1, v["path"][:, 0], v["next_token"])
    assert chi2_pvalue(np.bincount(y1, minlength=V), softmax64(R1)) > 1e-3
    for a in set(t["token"][0][t["depth"][0] == 1].tolist()):
        sel = (v["accept_len"] >= 1) & (v["path"][:, 0] == a)
        y2 = np.where(v["accept_len"][sel] >= 2, v["path"][sel, 1], v["next_token"][sel])
        assert chi2_pvalue(np.bincount(y2, minlength=V), softmax64(R2[a])) > 1e-3
