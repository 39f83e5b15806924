"""GPU <-> oracle parity of the draft options through the C ABI: a sampling temperature (the
official draft loop samples each position with one: [V41] "Markov head", the serial loop) and
the greedy draft of the deployed recipe ([V41] / [AIL], draft_sample_method "greedy"), for the
draft and for the verify of such a draft (the residual max(0, p_t - p_d) with the tempered p_d,
or p_t without the drafted token for a greedy draft; [V41] "投机解码…").

Tolerances as for the plain draft, with one addition: a greedy token is decided by the largest
logit, so the GPU may pick another token only where the oracle's gap between the two largest
logits is below twice the logit tolerance (a flagged near tie); the greedy lse is a logit and is
held to the logit tolerance."""
import numpy as np
import pytest
import torch

import oracle
import lossless_draft_verify_amd as L
from lossless_draft_verify_amd import workloads as W
from parity import (LOGIT_TOL, PROB_TOL, MismatchCounter, bits, compare_draft, dims_of,
                    gpu_draft, log, np_, oracle_draft)

pytestmark = pytest.mark.gpu

DEV = "cuda"
GREEDY_TIE = 2 * LOGIT_TOL


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs the GPU")
    L.load_library()


def _custom(name, **kw):
    return W.scaled(W.WORKLOADS["tiny-b4-v1000-g3"], name=name, **kw)


CASES = {
    # register-load step kernel, scalar tail (V % 4 != 0), two request groups
    "b130-v4099-r256-g3": _custom("b130-v4099-r256-g3", seed_id=41, B=130, V=4099, r=256, d=64,
                                  u_std=3.0, w_std=0.05),
    # pipelined (LDS-copy) step kernel, 4-token tail tile
    "b33-v2052-r64-g4": _custom("b33-v2052-r64-g4", seed_id=42, B=33, V=2052, r=64, gamma=4),
    # W2-dominated, pipelined step and pipelined residual (V % 4 == 0, r = 256)
    "b32-v32000-g7": W.scaled(W.WORKLOADS["b32-v32000-g7"], name="b32-v32000-g7-opts", seed_id=43),
}
OPTIONS = {"tau0.6": dict(temperature=0.6), "tau1.8": dict(temperature=1.8),
           "greedy": dict(greedy=True)}


def _compare_greedy(g, o, counter):
    """g: GPU greedy draft forced with the oracle's tokens; o: oracle greedy draft."""
    counter.add(g["tokens"], o["tokens"], o["margin"], tie=GREEDY_TIE)
    same = g["tokens"] == o["tokens"]
    # the forced token is the GPU's own greedy choice exactly where the two agree
    assert np.array_equal(g["q"], same.astype(np.float32))
    assert np.abs(g["lse"] - o["lse"]).max() <= LOGIT_TOL
    err = np.abs(np_(g["logits"]) - o["logits"]).max()
    assert err <= LOGIT_TOL, err
    return float(err)


@pytest.mark.parametrize("opt", list(OPTIONS))
@pytest.mark.parametrize("name", list(CASES))
def test_draft_options_parity(name, opt):
    wl, kw = CASES[name], OPTIONS[opt]
    log(f"[draft options] {name} {opt}")
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False, with_noise=False)
    o = oracle_draft(inp, wts, want_logits=True, **kw)
    g = gpu_draft(wl, inp, wts, force=o["tokens"], dbg=True, **kw)
    c = MismatchCounter(f"draft {name} {opt}")
    if kw.get("greedy"):
        err = _compare_greedy(g, o, c)
    else:
        err = compare_draft(g, o, c)
    log(f"  logits max err {err:.2e}; {c.report()}")
    # the run without the debug output (the pipelined step where it applies) is bit-identical
    gn = gpu_draft(wl, inp, wts, force=o["tokens"], **kw)
    for k in ("tokens", "q", "lse"):
        assert np.array_equal(gn[k], g[k]), k
    c.check_rate()


def test_greedy_draft_unforced_is_the_chain_of_argmaxes():
    """Unforced greedy draft on the GPU: every token is the first maximal logit of its own
    position's logits (read back from the debug output), q = 1 and lse = that logit."""
    wl = CASES["b33-v2052-r64-g4"]
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 1, DEV, with_hidden=False, with_noise=False)
    g = gpu_draft(wl, inp, wts, dbg=True, greedy=True)
    Lg = np_(g["logits"])
    assert np.array_equal(g["tokens"], Lg.argmax(axis=2).astype(np.int32))
    assert np.all(g["q"] == 1.0)
    assert np.array_equal(g["lse"], Lg.max(axis=2).astype(np.float64))
    # the oracle forced with the GPU's tokens conditions every step on the same prefix
    o = oracle_draft(inp, wts, force=g["tokens"], want_logits=True, greedy=True)
    assert np.abs(Lg - o["logits"]).max() <= LOGIT_TOL


def test_greedy_ignores_temperature_and_tau_one_is_default():
    wl = CASES["b130-v4099-r256-g3"]
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False, with_noise=False)
    a = gpu_draft(wl, inp, wts, greedy=True)
    b = gpu_draft(wl, inp, wts, greedy=True, temperature=0.25)
    for k in ("tokens", "q", "lse"):
        assert np.array_equal(a[k], b[k]), k
    # an explicit options struct at temperature 1 takes the same path as no options
    d = dims_of(wl)
    import ctypes
    from lossless_draft_verify_amd import binding as Bd
    lib = L.load_library()
    t = torch.empty((wl.B, wl.gamma), dtype=torch.int32, device=DEV)
    q = torch.empty((wl.B, wl.gamma), dtype=torch.float32, device=DEV)
    lse = torch.empty((wl.B, wl.gamma), dtype=torch.float64, device=DEV)
    ws = L.workspace(d, L.OP_DRAFT, DEV)
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    st = lib.dspark_markov_draft_opts(d.c(), P(inp["U"]), P(wts["W1"]), P(wts["W2t"]),
                                      P(inp["anchor"]), P(inp["uniforms"]), P(t), P(q), P(lse),
                                      None, None, P(ws), ws.numel(),
                                      ctypes.byref(Bd._CDraftOpts(1.0, 0)),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    ref = gpu_draft(wl, inp, wts)
    assert np.array_equal(np_(t), ref["tokens"]) and np.array_equal(np_(q), ref["q"])
    assert np.array_equal(np_(lse), ref["lse"])


def _target(wl, inp, o, draft_len):
    dense = np.concatenate([o["logits"], np_(inp["U_bonus"])[:, None, :]], 1) + np_(inp["noise"])
    keep = np.arange(wl.gamma + 1)[None, :] <= draft_len[:, None]
    return np.ascontiguousarray(dense[keep], dtype=np.float32)


def _T(a, dt=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device=DEV)


@pytest.mark.parametrize("opt", list(OPTIONS))
@pytest.mark.parametrize("name", ["tiny-b4-v1000-g3", "b130-v4099-r256-g3", "b32-v32000-g7"])
def test_verify_options_parity(name, opt):
    """Verify of a tempered or greedy draft: accept lengths and emitted tokens exact except
    flagged near ties, flags exact and beta (sum_v min(p_t, p_d)) within the probability
    tolerance. Ragged verify lengths; the tiny and V % 4 != 0 cases take the register-load
    residual kernel, the r = 256, V % 4 == 0 case the pipelined one."""
    wl = CASES.get(name) or W.WORKLOADS[name]
    kw = OPTIONS[opt]
    log(f"[verify options] {name} {opt}")
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False)
    o = oracle_draft(inp, wts, want_logits=True, **kw)
    rng = np.random.default_rng(wl.seed_id + 100)
    draft_len = rng.integers(0, wl.gamma + 1, wl.B).astype(np.int32)
    draft_len[0] = wl.gamma
    offs = np.concatenate([[0], np.cumsum(draft_len + 1)]).astype(np.int32)
    target = _target(wl, inp, o, draft_len)
    U, uni = np_(inp["U"]), np_(inp["uniforms"])
    ov = oracle.verify(target, offs, draft_len, U, bits(wts["W1"]), bits(wts["W2t"]),
                       np_(inp["anchor"]), o["tokens"], o["q"], uni, **kw)
    g = gpu_draft(wl, inp, wts, force=o["tokens"], **kw)
    al, nt, be, fl = L.verify(dims_of(wl), _T(target, torch.float32), _T(offs), _T(draft_len),
                              inp["U"], wts["W1"], wts["W2t"], inp["anchor"], _T(o["tokens"]),
                              _T(o["q"], torch.float32), g["lse_t"], inp["uniforms"], **kw)
    torch.cuda.synchronize()
    al, nt, be, fl = np_(al), np_(nt), np_(be), np_(fl)
    k = np.minimum(np.minimum(al, ov["accept_len"]), wl.gamma - 1)
    acc = MismatchCounter(f"accept {name} {opt}")
    acc.add(al, ov["accept_len"], ov["accept_margin"][np.arange(wl.B), k])
    same = al == ov["accept_len"]
    emit = MismatchCounter(f"emit {name} {opt}")
    emit.add(nt[same], ov["next_token"][same], ov["emit_margin"][same])
    assert np.array_equal(fl[same].astype(np.uint32), ov["flags"][same])
    assert np.abs(be[same] - ov["beta_emit"][same]).max() <= PROB_TOL
    rejected = same & (ov["beta_emit"] >= 0)
    if kw.get("greedy"):
        # the correction never re-emits the drafted token it replaces
        pos = al[rejected]
        drafted = o["tokens"][np.flatnonzero(rejected), pos]
        assert np.all(nt[rejected] != drafted)
    log(f"  {acc.report()}; {emit.report()}; residual rows {int(rejected.sum())}")
    assert rejected.sum() >= 1


@pytest.mark.parametrize("opt", ["greedy", "tau0.6"])
def test_round_full_size_options(opt):
    """A whole round at the production-drafter shape (B 128, V 129280, r 256, gamma 5, early
    stop) with a greedy or tempered draft, every request checked against the oracle."""
    wl, kw = W.WORKLOADS["b128-v129280-g5"], OPTIONS[opt]
    log(f"[round options] {wl.name} {opt}")
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV)
    d = dims_of(wl)
    o = oracle_draft(inp, wts, want_logits=True, **kw)
    T = W.temperatures(wl).numpy()
    conf = oracle.confidence(bits(inp["h"]), bits(wts["W1"]), bits(wts["w"]), T,
                             np_(inp["anchor"]), o["tokens"])["conf"]
    p = oracle.plan(conf, W.sps_table(wl), wl.mode)
    target = _target(wl, inp, o, p["draft_len"])
    ov = oracle.verify(target, p["row_offsets"], p["draft_len"], np_(inp["U"]), bits(wts["W1"]),
                       bits(wts["W2t"]), np_(inp["anchor"]), o["tokens"], o["q"],
                       np_(inp["uniforms"]), **kw)
    g = gpu_draft(wl, inp, wts, force=o["tokens"], dbg=True, **kw)
    c = MismatchCounter(f"round draft {opt}")
    if kw.get("greedy"):
        _compare_greedy(g, o, c)
    else:
        compare_draft(g, o, c)
    dl, ro, st = L.plan(d, _T(conf, torch.float32), _T(W.sps_table(wl), torch.float64), wl.mode)
    if p["margin"] > 1e-12:
        assert np.array_equal(np_(dl), p["draft_len"])
        assert np.array_equal(np_(ro), p["row_offsets"])
    al, nt, be, fl = L.verify(d, _T(target, torch.float32), ro, dl, inp["U"], wts["W1"],
                              wts["W2t"], inp["anchor"], _T(o["tokens"]),
                              _T(o["q"], torch.float32), g["lse_t"], inp["uniforms"], **kw)
    torch.cuda.synchronize()
    al, nt, be = np_(al), np_(nt), np_(be)
    k = np.minimum(np.minimum(al, ov["accept_len"]), wl.gamma - 1)
    acc = MismatchCounter(f"accept {opt}")
    acc.add(al, ov["accept_len"], ov["accept_margin"][np.arange(wl.B), k])
    same = al == ov["accept_len"]
    emit = MismatchCounter(f"emit {opt}")
    emit.add(nt[same], ov["next_token"][same], ov["emit_margin"][same])
    assert np.abs(be[same] - ov["beta_emit"][same]).max() <= PROB_TOL
    log(f"  {c.report()}; mean accepted {al.mean():.2f}; {acc.report()}; {emit.report()}")
