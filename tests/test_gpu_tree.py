"""PCTree on the GPU against the oracle ([ZDS] "后续工作"): the tree draft (children scored by
the Markov head, the most likely paths within a verify budget) and the lossless tree walk.

The draft is compared tree by tree: a tree whose deciding logit gap or path-probability gap
is below the flag threshold (R27: 1e-4, about 100x the GPU's logit error) may differ; every
other tree must match node for node, with q and P within the probability tolerance. The verify
gets the oracle's tree (so both sides walk the same tree) and target rows built from the base
logits along each node's path plus noise."""
import numpy as np
import pytest
import torch

import oracle
import lossless_draft_verify_amd as L
from lossless_draft_verify_amd import workloads as W
from parity import NEAR_TIE, PROB_TOL, MismatchCounter, bits, log, np_

pytestmark = pytest.mark.gpu

DEV = "cuda"
TREE_TIE = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs the GPU")
    L.load_library()


def _wl(name, **kw):
    return W.scaled(W.WORKLOADS["b128-v129280-g5"], name=name, **kw)


CASES = {
    # tiny: every tile path, a ragged vocabulary tail
    "b4-v1000-r16-g3-c2m2n6": (W.WORKLOADS["tiny-b4-v1000-g3"], L.TreeShape(2, 2, 6)),
    # V % 4 != 0 (the step's register-load kernel), r = 64
    "b7-v4099-r64-g3-c3m2n9": (_wl("t-b7-v4099", seed_id=61, B=7, V=4099, r=64, gamma=3, d=64),
                               L.TreeShape(3, 2, 9)),
    # 80 rows a depth (one group), r = 256, pipelined step kernel
    "b20-v8192-r256-g4-c4m4n16": (_wl("t-b20-v8192", seed_id=62, B=20, V=8192, gamma=4, d=64),
                                  L.TreeShape(4, 4, 16)),
    # the pages' PCTree batch at the production drafter's vocabulary
    "b16-v129280-g5-c4m4n16": (_wl("t-b16", seed_id=63, B=16, d=64), L.TreeShape(4, 4, 16)),
    # 512 expanded rows a depth (four 128-row groups), eight children, M = 8
    "b64-v32768-g3-c8m8n32": (_wl("t-b64", seed_id=64, B=64, V=32768, gamma=3, d=64),
                              L.TreeShape(8, 8, 32)),
    # peaked base logits (std 8) and a close target (noise 0.3): walks reach the leaves and
    # draw the bonus there; every candidate kept (N = T)
    "b256-v8192-g4-peaked-c4m2n28": (_wl("t-peaked", seed_id=65, B=256, V=8192, gamma=4, d=64,
                                         u_std=8.0), L.TreeShape(4, 2, 28)),
}
NOISE = {"b256-v8192-g4-peaked-c4m2n28": 0.3}


def _tree_target(wl, inp, wts, tok, dep, N, std=0.6, seed=0):
    """Target rows of a tree [B][N+1][V]: after the anchor, U_1 + W1[anchor] W2; after node n of
    depth d, U_{d+1} + W1[token] W2 (the bonus base logits when d = gamma); plus noise."""
    B, g, V = wl.B, wl.gamma, wl.V
    U, Ub = inp["U"], inp["U_bonus"]
    tok_t = torch.as_tensor(tok, device=DEV).long()
    dep_t = torch.as_tensor(dep, device=DEV).long()
    prev = torch.cat([inp["anchor"].long()[:, None], tok_t], 1)              # [B][N+1]
    pos = torch.cat([torch.zeros((B, 1), dtype=torch.long, device=DEV), dep_t], 1)
    W1f, W2f = wts["W1"].float(), wts["W2t"].float()
    rows = torch.empty((B, N + 1, V), dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1000 + seed)
    for b in range(B):
        base = torch.where((pos[b] < g)[:, None], U[b, pos[b].clamp(max=g - 1)], Ub[b][None, :])
        rows[b] = base + W1f[prev[b]] @ W2f.T
    rows += torch.randn(rows.shape, generator=gen, device=DEV) * std
    return rows


@pytest.mark.parametrize("name", list(CASES))
def test_tree_draft_and_verify_match_the_oracle(name):
    wl, shape = CASES[name]
    B, g, V, N = wl.B, wl.gamma, wl.V, shape.N
    log(f"[tree] {name}")
    d = L.Dims(B, g, V, wl.r, wl.d)
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False, with_noise=False)
    o = oracle.tree_draft(np_(inp["U"]), bits(wts["W1"]), bits(wts["W2t"]), np_(inp["anchor"]),
                          shape.c, shape.M, N)
    tok, dep, par, q, P = (np_(t) for t in L.tree_draft(d, shape, inp["U"], wts["W1"],
                                                         wts["W2t"], inp["anchor"]))
    flagged = (o["logit_margin"] < TREE_TIE) | (o["path_margin"] < TREE_TIE)
    same = ((tok == o["token"]).all(1) & (dep == o["depth"]).all(1) & (par == o["parent"]).all(1))
    bad = ~same & ~flagged
    assert not bad.any(), f"unflagged tree mismatches in requests {np.nonzero(bad)[0][:8]}"
    assert (o["depth"][:, 0] == 1).all() and (par[:, 0] == -1).all()
    if same.any():
        assert np.abs(q[same] - o["q"][same]).max() <= PROB_TOL
        assert (np.abs(P[same] - o["path"][same]) <= PROB_TOL * o["depth"][same]).all()
    log(f"  draft: {int(same.sum())}/{B} trees equal, {int(flagged.sum())} flagged, "
        f"q err {np.abs(q[same] - o['q'][same]).max() if same.any() else 0:.1e}")
    # verify on the oracle's tree
    target = _tree_target(wl, inp, wts, o["token"], o["depth"], N, std=NOISE.get(name, 0.6))
    ov = oracle.tree_verify(np_(target), o["token"], o["depth"], o["parent"], np_(inp["uniforms"]))
    T = lambda a: torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32, device=DEV)
    al, path, nt, fl = (np_(t) for t in L.tree_verify(d, shape, target, T(o["token"]),
                                                      T(o["parent"]), inp["uniforms"]))
    c = MismatchCounter(f"tree walk {name}")
    walk_same = (al == ov["accept_len"]) & (path == ov["path"]).all(1) & (nt == ov["next_token"])
    c.add(walk_same, np.ones(B, bool), ov["margin"])
    assert np.array_equal(fl.astype(np.uint32), ov["flags"])
    assert ((al >= 0) & (al <= g)).all()
    log(f"  verify: mean accepted {al.mean():.2f} (max {al.max()}); {c.report()}")
    c.check_rate()
    if name in NOISE:
        assert (al == g).mean() > 0.2, "the peaked case should reach the leaves"


def test_tree_draft_is_deterministic_and_rows_share_base_logits():
    """Two identical calls give identical trees; with M = c the expanded rows of one request
    at a depth read the same U row (a shift of the row index), which the oracle comparison of
    the headline case covers; here the run-to-run bits."""
    wl, shape = CASES["b20-v8192-r256-g4-c4m4n16"]
    d = L.Dims(wl.B, wl.gamma, wl.V, wl.r, wl.d)
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 1, DEV, with_hidden=False, with_noise=False)
    a = [np_(t) for t in L.tree_draft(d, shape, inp["U"], wts["W1"], wts["W2t"], inp["anchor"])]
    b = [np_(t) for t in L.tree_draft(d, shape, inp["U"], wts["W1"], wts["W2t"], inp["anchor"])]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_tree_full_size_sampled_requests():
    """The PCTree round in the launch configuration the benchmark times (B = 128, V = 129280,
    r = 256, gamma = 5, c = 4, M = 4, N = 16; depths 2-5 expand 512 rows, four 128-row groups),
    checked against the oracle on six requests spread over those groups: a request's tree and
    walk depend only on its own rows. The verify walks the oracle's tree for those requests (the
    GPU's own tree for the rest), over target rows built along each tree's paths."""
    wl, shape = W.WORKLOADS["b128-v129280-g5"], L.TreeShape(4, 4, 16)
    B, g, V, N = wl.B, wl.gamma, wl.V, shape.N
    idx = np.array([0, 31, 45, 64, 101, 127])
    log(f"[tree full size] B {B} V {V} c4 m4 n16, oracle on requests {idx.tolist()}")
    d = L.Dims(B, g, V, wl.r, wl.d)
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False, with_noise=False)
    tok, dep, par, q, P = (np_(t) for t in L.tree_draft(d, shape, inp["U"], wts["W1"],
                                                         wts["W2t"], inp["anchor"]))
    o = oracle.tree_draft(np_(inp["U"])[idx], bits(wts["W1"]), bits(wts["W2t"]),
                          np_(inp["anchor"])[idx], shape.c, shape.M, N)
    flagged = (o["logit_margin"] < TREE_TIE) | (o["path_margin"] < TREE_TIE)
    same = ((tok[idx] == o["token"]).all(1) & (dep[idx] == o["depth"]).all(1)
            & (par[idx] == o["parent"]).all(1))
    assert not (~same & ~flagged).any(), f"unflagged mismatches at {idx[~same & ~flagged]}"
    if same.any():
        assert np.abs(q[idx][same] - o["q"][same]).max() <= PROB_TOL
        assert (np.abs(P[idx][same] - o["path"][same]) <= PROB_TOL * o["depth"][same]).all()
    log(f"  draft: {int(same.sum())}/{len(idx)} sampled trees equal, {int(flagged.sum())} flagged")
    tok_v, dep_v, par_v = tok.copy(), dep.copy(), par.copy()
    tok_v[idx], dep_v[idx], par_v[idx] = o["token"], o["depth"], o["parent"]
    target = _tree_target(wl, inp, wts, tok_v, dep_v, N)
    T = lambda a: torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32, device=DEV)
    al, path, nt, fl = (np_(t) for t in L.tree_verify(d, shape, target, T(tok_v), T(par_v),
                                                      inp["uniforms"]))
    ov = oracle.tree_verify(np_(target[torch.as_tensor(idx, device=DEV)]), o["token"], o["depth"],
                            o["parent"], np_(inp["uniforms"])[idx])
    del target
    c = MismatchCounter("tree walk full size")
    walk_same = ((al[idx] == ov["accept_len"]) & (path[idx] == ov["path"]).all(1)
                 & (nt[idx] == ov["next_token"]))
    c.add(walk_same, np.ones(len(idx), bool), ov["margin"])
    assert np.array_equal(fl[idx].astype(np.uint32), ov["flags"])
    assert ((al >= 0) & (al <= g)).all() and ((nt >= 0) & (nt < V)).all()
    log(f"  verify: accepted {al[idx].tolist()}; {c.report()}")
    c.check_rate()
