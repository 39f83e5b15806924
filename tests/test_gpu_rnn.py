"""GPU <-> oracle parity of the RNN draft head (eq. (6); [CSDN] 4.2, [AIL] "RNN 头（可选）")
through the C ABI: the draft (tokens, q, lse, logits and the bias vectors e_k) and the verify of
an RNN draft, on the same seeded inputs (Wgco from the workload generator's RNN weights).

Tolerances as for the Markov head (logits 2e-3, probabilities 1e-6, lse 1e-5, tokens exact except
flagged near ties), and e_k within 1e-5 absolute: the GPU sums the hidden block of a
pre-activation as fp32 MFMA chunks of 128 products (relative error about 1e-7 each) in fp64 and
rounds e_k once to fp32, while the oracle sums every term in fp64."""
import numpy as np
import pytest
import torch

import oracle
import lossless_draft_verify_amd as L
from lossless_draft_verify_amd import workloads as W
from parity import (LOGIT_TOL, LSE_TOL, PROB_TOL, MismatchCounter, bits, dims_of, log, np_)

pytestmark = pytest.mark.gpu

DEV = "cuda"
E_TOL = 1e-5
GREEDY_TIE = 2 * LOGIT_TOL


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs the GPU")
    L.load_library()


def _custom(name, **kw):
    return W.scaled(W.WORKLOADS["tiny-b4-v1000-g3"], name=name, **kw)


CASES = {
    # register-prefetch step (r = 16), register-load residual
    "tiny-b4-v1000-g3": W.WORKLOADS["tiny-b4-v1000-g3"],
    # pipelined step at r = 64, 4-token tail tile
    "b33-v2052-r64-g4": _custom("b33-v2052-r64-g4-rnn", seed_id=52, B=33, V=2052, r=64, gamma=4),
    # register-prefetch step at r = 256 (two request groups of 64), V % 4 != 0
    "b130-v4099-r256-g3": _custom("b130-v4099-r256-g3-rnn", seed_id=51, B=130, V=4099, r=256,
                                  d=64, u_std=3.0, w_std=0.05),
    # pipelined step and pipelined residual at r = 256, d = 320
    "b32-v32000-g7": W.scaled(W.WORKLOADS["b32-v32000-g7"], name="b32-v32000-g7-rnn", seed_id=53,
                              d=320),
    # pipelined step and residual at r = 128 over two request groups: the groups of one
    # vocabulary range placed on one XCD, with the three-term bias rows
    "b130-v4100-r128-g3": _custom("b130-v4100-r128-g3-rnn", seed_id=54, B=130, V=4100, r=128,
                                  d=64, u_std=3.0, w_std=0.05),
    # the four-stage one-tile step at r = 256 over two request groups, the second ragged (two
    # requests: one wave of four active), and a 4-token tail tile
    "b130-v4100-r256-g3": _custom("b130-v4100-r256-g3-rnn", seed_id=55, B=130, V=4100, r=256,
                                  d=64, u_std=3.0, w_std=0.05),
    # the four-stage step over three request groups (the third ragged) and the 512-thread
    # sampler of batches past 256, with the three-term bias rows
    "b300-v4100-r256-g3": _custom("b300-v4100-r256-g3-rnn", seed_id=56, B=300, V=4100, r=256,
                                  d=64, u_std=3.0, w_std=0.05),
}


def _inputs(wl, rnd=0):
    wts = W.weights(wl, DEV)
    wts["Wgco"] = W.rnn_weights(wl, DEV)
    inp = W.round_inputs(wl, rnd, DEV, with_hidden=True)
    return wts, inp


def gpu_rnn(wl, inp, wts, force=None, dbg=False, **kw):
    d = dims_of(wl)
    logits = torch.empty_like(inp["U"]) if dbg else None
    f = None if force is None else torch.as_tensor(force, dtype=torch.int32, device=DEV).contiguous()
    t, q, lse, e = L.rnn_draft(d, inp["U"], wts["W1"], wts["W2t"], wts["Wgco"], inp["h"],
                               inp["anchor"], inp["uniforms"], logits_dbg=logits, force_tokens=f,
                               **kw)
    torch.cuda.synchronize()
    return dict(tokens=np_(t), q=np_(q), lse=np_(lse), e=np_(e), logits=logits, tokens_t=t, q_t=q,
                lse_t=lse, e_t=e)


def oracle_rnn(inp, wts, force=None, want_logits=False, **kw):
    return oracle.rnn_draft(np_(inp["U"]), bits(wts["W1"]), bits(wts["W2t"]), bits(wts["Wgco"]),
                            bits(inp["h"]), np_(inp["anchor"]), np_(inp["uniforms"]),
                            force_tokens=force, want_logits=want_logits, **kw)


def _compare(g, o, counter, greedy=False):
    tie = GREEDY_TIE if greedy else 1e-5
    counter.add(g["tokens"], o["tokens"], o["margin"], tie=tie)
    if greedy:
        assert np.array_equal(g["q"], (g["tokens"] == o["tokens"]).astype(np.float32))
        assert np.abs(g["lse"] - o["lse"]).max() <= LOGIT_TOL
    else:
        assert np.abs(g["q"] - o["q"]).max() <= PROB_TOL, np.abs(g["q"] - o["q"]).max()
        assert np.abs(g["lse"] - o["lse"]).max() <= LSE_TOL, np.abs(g["lse"] - o["lse"]).max()
    e_err = np.abs(g["e"] - o["e"]).max()
    assert e_err <= E_TOL, e_err
    err = np.abs(np_(g["logits"]) - o["logits"]).max()
    assert err <= LOGIT_TOL, err
    return float(err), float(e_err)


OPTIONS = {"plain": {}, "greedy": dict(greedy=True), "tau0.6": dict(temperature=0.6)}


@pytest.mark.parametrize("opt", list(OPTIONS))
@pytest.mark.parametrize("name", list(CASES))
def test_rnn_draft_parity(name, opt):
    wl, kw = CASES[name], OPTIONS[opt]
    log(f"[rnn draft] {name} {opt}")
    wts, inp = _inputs(wl)
    o = oracle_rnn(inp, wts, want_logits=True, **kw)
    g = gpu_rnn(wl, inp, wts, force=o["tokens"], dbg=True, **kw)
    c = MismatchCounter(f"rnn draft {name} {opt}")
    err, e_err = _compare(g, o, c, greedy=bool(kw.get("greedy")))
    log(f"  logits max err {err:.2e}, e max err {e_err:.2e}; {c.report()}")
    # the step kernel without a debug output (the pipelined one where it applies): same draws
    gn = gpu_rnn(wl, inp, wts, force=o["tokens"], **kw)
    for k in ("tokens", "q", "lse", "e"):
        assert np.array_equal(gn[k], g[k]), k
    c.check_rate()


def test_rnn_draft_unforced_runs_its_own_chain():
    """Unforced: every position is conditioned on the GPU's own previous draw, and the oracle
    forced with those draws reproduces q, lse and e."""
    wl = CASES["b33-v2052-r64-g4"]
    wts, inp = _inputs(wl, 1)
    g = gpu_rnn(wl, inp, wts)
    o = oracle_rnn(inp, wts, force=g["tokens"])
    assert np.abs(g["q"] - o["q"]).max() <= PROB_TOL
    assert np.abs(g["lse"] - o["lse"]).max() <= LSE_TOL
    assert np.abs(g["e"] - o["e"]).max() <= E_TOL
    c = MismatchCounter("rnn unforced")
    c.add(g["tokens"], o["tokens"], o["margin"])


def _T(a, dt=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device=DEV)


def _target(wl, inp, o, draft_len):
    dense = np.concatenate([o["logits"], np_(inp["U_bonus"])[:, None, :]], 1) + np_(inp["noise"])
    keep = np.arange(wl.gamma + 1)[None, :] <= draft_len[:, None]
    return np.ascontiguousarray(dense[keep], dtype=np.float32)


@pytest.mark.parametrize("opt", list(OPTIONS))
@pytest.mark.parametrize("name", ["tiny-b4-v1000-g3", "b130-v4099-r256-g3", "b32-v32000-g7",
                                  "b130-v4100-r128-g3"])
def test_rnn_verify_parity(name, opt):
    """Verify of an RNN draft with ragged lengths: accept lengths and emitted tokens exact
    except flagged near ties, flags exact, beta within the probability tolerance."""
    wl, kw = CASES[name], OPTIONS[opt]
    log(f"[rnn verify] {name} {opt}")
    wts, inp = _inputs(wl)
    o = oracle_rnn(inp, wts, want_logits=True, **kw)
    rng = np.random.default_rng(wl.seed_id + 200)
    draft_len = rng.integers(0, wl.gamma + 1, wl.B).astype(np.int32)
    draft_len[0] = wl.gamma
    offs = np.concatenate([[0], np.cumsum(draft_len + 1)]).astype(np.int32)
    target = _target(wl, inp, o, draft_len)
    ov = oracle.rnn_verify(target, offs, draft_len, np_(inp["U"]), bits(wts["W1"]),
                           bits(wts["W2t"]), bits(wts["Wgco"]), bits(inp["h"]),
                           np_(inp["anchor"]), o["tokens"], o["q"], np_(inp["uniforms"]), **kw)
    g = gpu_rnn(wl, inp, wts, force=o["tokens"], **kw)
    al, nt, be, fl = L.rnn_verify(dims_of(wl), _T(target, torch.float32), _T(offs), _T(draft_len),
                                  inp["U"], wts["W2t"], g["e_t"], _T(o["tokens"]),
                                  _T(o["q"], torch.float32), g["lse_t"], inp["uniforms"], **kw)
    torch.cuda.synchronize()
    al, nt, be, fl = np_(al), np_(nt), np_(be), np_(fl)
    k = np.minimum(np.minimum(al, ov["accept_len"]), wl.gamma - 1)
    acc = MismatchCounter(f"rnn accept {name} {opt}")
    acc.add(al, ov["accept_len"], ov["accept_margin"][np.arange(wl.B), k])
    same = al == ov["accept_len"]
    emit = MismatchCounter(f"rnn emit {name} {opt}")
    emit.add(nt[same], ov["next_token"][same], ov["emit_margin"][same])
    assert np.array_equal(fl[same].astype(np.uint32), ov["flags"][same])
    assert np.abs(be[same] - ov["beta_emit"][same]).max() <= PROB_TOL
    rejected = same & (ov["beta_emit"] >= 0)
    log(f"  {acc.report()}; {emit.report()}; residual rows {int(rejected.sum())}")
    assert rejected.sum() >= 1


@pytest.mark.parametrize("opt", ["plain", "greedy"])
def test_rnn_round_full_size(opt):
    """A whole RNN-head round at the production-drafter shape (B 128, V 129280, r 256,
    gamma 5, d 5120, early stop), every request checked against the oracle."""
    wl, kw = W.WORKLOADS["b128-v129280-g5"], OPTIONS[opt]
    log(f"[rnn round] {wl.name} {opt}: oracle")
    wts, inp = _inputs(wl)
    d = dims_of(wl)
    o = oracle_rnn(inp, wts, want_logits=True, **kw)
    T = W.temperatures(wl).numpy()
    conf = oracle.confidence(bits(inp["h"]), bits(wts["W1"]), bits(wts["w"]), T,
                             np_(inp["anchor"]), o["tokens"])["conf"]
    p = oracle.plan(conf, W.sps_table(wl), wl.mode)
    target = _target(wl, inp, o, p["draft_len"])
    ov = oracle.rnn_verify(target, p["row_offsets"], p["draft_len"], np_(inp["U"]),
                           bits(wts["W1"]), bits(wts["W2t"]), bits(wts["Wgco"]), bits(inp["h"]),
                           np_(inp["anchor"]), o["tokens"], o["q"], np_(inp["uniforms"]), **kw)
    log("  gpu")
    g = gpu_rnn(wl, inp, wts, force=o["tokens"], dbg=True, **kw)
    c = MismatchCounter(f"rnn round draft {opt}")
    err, e_err = _compare(g, o, c, greedy=bool(kw.get("greedy")))
    gn = gpu_rnn(wl, inp, wts, force=o["tokens"], **kw)
    for k in ("tokens", "q", "lse", "e"):
        assert np.array_equal(gn[k], g[k]), k
    dl, ro, st = L.plan(d, _T(conf, torch.float32), _T(W.sps_table(wl), torch.float64), wl.mode)
    if p["margin"] > 1e-12:
        assert np.array_equal(np_(dl), p["draft_len"])
        assert np.array_equal(np_(ro), p["row_offsets"])
    al, nt, be, fl = L.rnn_verify(d, _T(target, torch.float32), ro, dl, inp["U"], wts["W2t"],
                                  g["e_t"], _T(o["tokens"]), _T(o["q"], torch.float32),
                                  g["lse_t"], inp["uniforms"], **kw)
    torch.cuda.synchronize()
    al, nt, be = np_(al), np_(nt), np_(be)
    k = np.minimum(np.minimum(al, ov["accept_len"]), wl.gamma - 1)
    acc = MismatchCounter(f"rnn accept {opt}")
    acc.add(al, ov["accept_len"], ov["accept_margin"][np.arange(wl.B), k])
    same = al == ov["accept_len"]
    emit = MismatchCounter(f"rnn emit {opt}")
    emit.add(nt[same], ov["next_token"][same], ov["emit_margin"][same])
    assert np.abs(be[same] - ov["beta_emit"][same]).max() <= PROB_TOL
    log(f"  logits err {err:.2e}, e err {e_err:.2e}; {c.report()}; mean accepted {al.mean():.2f}; "
        f"{acc.report()}; {emit.report()}")


def _rnn_round_setup(seed_id):
    wl = W.scaled(W.WORKLOADS["b128-v129280-g5"], name="rnn-graph", seed_id=seed_id, B=64,
                  V=8192, d=256, sps_scale=64.0)
    wts, inp = _inputs(wl)
    d = dims_of(wl)
    temps = W.temperatures(wl).to(DEV)
    sps = _T(W.sps_table(wl), torch.float64)
    logits = torch.empty_like(inp["U"])
    t0, _, _, _ = L.rnn_draft(d, inp["U"], wts["W1"], wts["W2t"], wts["Wgco"], inp["h"],
                              inp["anchor"], inp["uniforms"], logits_dbg=logits)
    c0 = L.confidence(d, inp["h"], wts["W1"], wts["w"], temps, inp["anchor"], t0)
    dl0, _, _ = L.plan(d, c0, sps, wl.mode)
    target = W.pack_rows(W.target_dense(logits, inp["U_bonus"], inp["noise"]), dl0)
    del logits
    B, g = wl.B, wl.gamma
    out = dict(tok=torch.empty((B, g), dtype=torch.int32, device=DEV),
               q=torch.empty((B, g), dtype=torch.float32, device=DEV),
               lse=torch.empty((B, g), dtype=torch.float64, device=DEV),
               e=torch.empty((B, g, wl.r), dtype=torch.float32, device=DEV),
               conf=torch.empty((B, g), dtype=torch.float32, device=DEV),
               dl=torch.empty(B, dtype=torch.int32, device=DEV),
               ro=torch.empty(B + 1, dtype=torch.int32, device=DEV),
               st=torch.empty(4, dtype=torch.float64, device=DEV),
               al=torch.empty(B, dtype=torch.int32, device=DEV),
               nt=torch.empty(B, dtype=torch.int32, device=DEV),
               be=torch.empty(B, dtype=torch.float32, device=DEV),
               fl=torch.empty(B, dtype=torch.int32, device=DEV))
    ws_d, ws_v = L.workspace(d, L.OP_RNN_DRAFT, DEV), L.workspace(d, L.OP_RNN_VERIFY, DEV)

    def round_():
        o = out
        L.rnn_draft(d, inp["U"], wts["W1"], wts["W2t"], wts["Wgco"], inp["h"], inp["anchor"],
                    inp["uniforms"], tokens=o["tok"], q=o["q"], lse=o["lse"], e_rows=o["e"],
                    ws=ws_d)
        L.confidence(d, inp["h"], wts["W1"], wts["w"], temps, inp["anchor"], o["tok"],
                     conf=o["conf"])
        L.plan(d, o["conf"], sps, wl.mode, draft_len=o["dl"], row_offsets=o["ro"],
               stats=o["st"])
        L.rnn_verify(d, target, o["ro"], o["dl"], inp["U"], wts["W2t"], o["e"], o["tok"],
                     o["q"], o["lse"], inp["uniforms"], accept_len=o["al"], next_token=o["nt"],
                     beta_emit=o["be"], flags=o["fl"], ws=ws_v)

    return out, round_, dl0


def test_rnn_round_graph_replays_and_determinism():
    """An RNN-head round (its pre-GEMM, state steps and three-term bias rows included) gives the
    same bits on a second eager run, and captured once as a hipGraph reproduces them on every
    replay, with eager work between the replays and the outputs overwritten before each."""
    out, round_, dl0 = _rnn_round_setup(91)
    round_()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    assert torch.equal(eager["dl"], dl0)
    round_()
    torch.cuda.synchronize()
    for k, v in out.items():
        assert torch.equal(v, eager[k]), ("second eager run", k)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_()
    torch.cuda.synchronize()
    for rep in range(4):
        junk = torch.randn(1 << 20, device=DEV)
        _ = float(junk.square().sum().item())
        for v in out.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, eager[k]), (rep, k)
    log(f"  rnn round: eager runs and four graph replays equal (B_tot {eager['st'][0].item():.0f})")
