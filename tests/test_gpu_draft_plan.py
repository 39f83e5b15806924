"""The draft-and-plan calls (dspark_markov_draft_plan, dspark_rnn_draft_plan) against the three
calls each stands for (the
draft, the confidence head and the planner, made one after the other), bit for bit: on the
shapes where the plan runs on one workgroup of the last draft step's launch (r in {64, 128, 256},
V % 4 == 0, B * gamma <= 4096) and on those that launch it on its own; in every plan mode, the
lag ring over consecutive rounds, and the draft options. The separate calls are checked against
the oracle in the other parity files; one oracle check of the plan at the production shape is
added here."""
import numpy as np
import pytest
import torch

import oracle
import lossless_draft_verify_amd as L
from lossless_draft_verify_amd import workloads as W
from parity import PLAN_TIE, dims_of, log, np_

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs the GPU")
    L.load_library()


def _custom(name, **kw):
    return W.scaled(W.WORKLOADS["tiny-b4-v1000-g3"], name=name, **kw)


# name -> (workload, whether the plan runs inside the last step's launch)
CASES = {
    "b128-v129280-g5": (W.WORKLOADS["b128-v129280-g5"], True),
    "b32-v32000-g7": (W.WORKLOADS["b32-v32000-g7"], True),
    # two request groups (the planner's workgroup ahead of both groups' step workgroups)
    "b130-v4100-r128-g3": (_custom("b130-v4100-r128-g3", seed_id=41, B=130, V=4100, r=128,
                                   u_std=3.0, w_std=0.05), True),
    "b33-v2052-r64-g4": (_custom("b33-v2052-r64-g4", seed_id=42, B=33, V=2052, r=64, gamma=4), True),
    # the fused planner's largest size: B * gamma = 4096 (eight candidates per thread)
    "b512-v2048-r64-g8": (_custom("b512-v2048-r64-g8", seed_id=43, B=512, V=2048, r=64, gamma=8),
                          True),
    # a single position: the confidences need only the anchors, and the fused step is the first
    "b9-v4096-r256-g1": (_custom("b9-v4096-r256-g1", seed_id=44, B=9, V=4096, r=256, gamma=1,
                                 u_std=3.0, w_std=0.05), True),
    # shapes that launch the planner on its own: r = 16, V % 4 != 0, B * gamma > 4096
    "tiny-b4-v1000-g3": (W.WORKLOADS["tiny-b4-v1000-g3"], False),
    "b130-v4099-r256-g3": (_custom("b130-v4099-r256-g3", seed_id=45, B=130, V=4099, r=256,
                                   u_std=3.0, w_std=0.05), False),
    "b1100-v1024-r64-g4": (_custom("b1100-v1024-r64-g4", seed_id=46, B=1100, V=1024, r=64,
                                   gamma=4), False),
}


def _bits(t):
    a = np_(t)
    return a.view(np.uint8) if a.dtype.kind == "f" else a


def _same(a, b, what):
    assert np.array_equal(_bits(a), _bits(b)), what


def _separate(wl, d, inp, wts, T, sps_t, mode, ring, t, temperature, greedy):
    tok, q, lse = L.markov_draft(d, inp["U"], wts["W1"], wts["W2t"], inp["anchor"],
                                 inp["uniforms"], temperature=temperature, greedy=greedy)
    conf = L.confidence(d, inp["h"], wts["W1"], wts["w"], T, inp["anchor"], tok)
    dl, ro, st = L.plan(d, conf, sps_t, mode, ring=ring, round_index=t)
    return tok, q, lse, conf, dl, ro, st


def _fused(d, inp, wts, T, sps_t, mode, ring, t, temperature, greedy):
    L.profile_begin()
    try:
        out = L.markov_draft_plan(d, inp["U"], wts["W1"], wts["W2t"], inp["anchor"],
                                  inp["uniforms"], inp["h"], wts["w"], T, sps_t, mode, ring=ring,
                                  round_index=t, temperature=temperature, greedy=greedy)
        torch.cuda.synchronize()
    finally:
        prof = L.profile_end()
    return out, prof


def _run_case(wl, fused_expected, modes, rounds=1, temperature=1.0, greedy=False):
    if wl.sps_kind == "flat":   # a table that makes the plans cut (a flat one admits nearly all)
        wl = W.scaled(wl, sps_kind="hyperbolic", sps_scale=max(1.0, wl.B * 1.5))
    d = dims_of(wl)
    wts = W.weights(wl, DEV)
    T = W.temperatures(wl).to(DEV)
    sps_t = torch.tensor(W.sps_table(wl), dtype=torch.float64, device=DEV)
    for mode in modes:
        ring_a = ring_b = None
        if mode == L.LAGGED_TOPK:
            ring_a = torch.zeros((2, wl.B, wl.gamma), dtype=torch.float32, device=DEV)
            ring_b = ring_a.clone()
        for t in range(rounds):
            inp = W.round_inputs(wl, t, DEV, with_hidden=True, with_noise=False)
            ref = _separate(wl, d, inp, wts, T, sps_t, mode, ring_a, t, temperature, greedy)
            got, prof = _fused(d, inp, wts, T, sps_t, mode, ring_b, t, temperature, greedy)
            for name, a, b in zip(("tokens", "q", "lse", "conf", "draft_len", "row_offsets",
                                   "stats"), got, ref):
                _same(a, b, f"{wl.name} mode {mode} round {t}: {name}")
            if ring_a is not None:
                _same(ring_b, ring_a, f"{wl.name} round {t}: ring")
            # the path taken: no launch of its own for the planner when it runs beside the step
            assert (prof["plan"][0] == 0) == fused_expected, (wl.name, prof["plan"])
            assert prof["markov_step"][0] == wl.gamma and prof["confidence"][0] == 1
    log(f"  {wl.name}: modes {list(modes)}, {rounds} round(s), fused {fused_expected}")


@pytest.mark.parametrize("name", list(CASES))
def test_draft_plan_matches_the_separate_calls(name):
    wl, fused = CASES[name]
    modes = (L.EARLY_STOP, L.FULL_PATH, L.FULL_VERIFY)
    if wl.B * wl.gamma > 4096 or wl.V > 32000:
        modes = (L.EARLY_STOP,)
    _run_case(wl, fused, modes)


def test_draft_plan_lagged_ring():
    """LAGGED_TOPK over five chained rounds: the ring the fused planner reads and rewrites
    matches the separate planner's after every round (rounds 0-1 plan synchronously)."""
    wl, fused = CASES["b130-v4100-r128-g3"]
    _run_case(wl, fused, (L.LAGGED_TOPK,), rounds=5)


@pytest.mark.parametrize("temperature,greedy", [(0.6, False), (1.8, False), (1.0, True)])
def test_draft_plan_options(temperature, greedy):
    wl, fused = CASES["b33-v2052-r64-g4"]
    _run_case(wl, fused, (L.EARLY_STOP,), temperature=temperature, greedy=greedy)


def test_draft_plan_against_the_oracle_planner():
    """At the production shape, the fused call's plan equals the oracle planner's on the
    confidences the call returned (exact, unless the oracle flags a Theta tie)."""
    wl, _ = CASES["b128-v129280-g5"]
    d = dims_of(wl)
    wts = W.weights(wl, DEV)
    T = W.temperatures(wl).to(DEV)
    sps = W.sps_table(wl)
    sps_t = torch.tensor(sps, dtype=torch.float64, device=DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=True, with_noise=False)
    for mode in (L.EARLY_STOP, L.FULL_PATH):
        (tok, q, lse, conf, dl, ro, st), _ = _fused(d, inp, wts, T, sps_t, mode, None, 0, 1.0,
                                                    False)
        o = oracle.plan(np_(conf), sps, mode)
        if o["margin"] > PLAN_TIE:
            assert np.array_equal(np_(dl), o["draft_len"]), mode
            assert np.array_equal(np_(ro), o["row_offsets"]), mode
            assert np.allclose(np_(st), o["stats"], rtol=1e-12, atol=0), mode
        else:
            log(f"  flagged planner tie (margin {o['margin']:.1e}), mode {mode}")


# The RNN head (eq. (6)): name -> (workload, whether the plan runs beside the last step)
RNN_CASES = {
    "rnn-b128-v129280-g5": (W.WORKLOADS["b128-v129280-g5"], True),      # four-stage step, r = 256
    "rnn-b130-v4100-r128-g3": (_custom("rnn-b130-v4100-r128-g3", seed_id=47, B=130, V=4100, r=128,
                                       d=64, u_std=3.0, w_std=0.05), True),
    "rnn-b33-v2052-r64-g4": (_custom("rnn-b33-v2052-r64-g4", seed_id=48, B=33, V=2052, r=64, d=64,
                                     gamma=4), True),
    "rnn-b20-v4099-r256-g3": (_custom("rnn-b20-v4099-r256-g3", seed_id=49, B=20, V=4099, r=256,
                                      d=64), False),                     # V % 4 != 0
}


def _run_rnn_case(wl, fused_expected, mode, temperature=1.0, greedy=False):
    if wl.sps_kind == "flat":
        wl = W.scaled(wl, sps_kind="hyperbolic", sps_scale=max(1.0, wl.B * 1.5))
    d = dims_of(wl)
    wts = W.weights(wl, DEV)
    Wgco = W.rnn_weights(wl, DEV)
    T = W.temperatures(wl).to(DEV)
    sps_t = torch.tensor(W.sps_table(wl), dtype=torch.float64, device=DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=True, with_noise=False)
    opts = dict(temperature=temperature, greedy=greedy)
    tok, q, lse, e = L.rnn_draft(d, inp["U"], wts["W1"], wts["W2t"], Wgco, inp["h"], inp["anchor"],
                                 inp["uniforms"], **opts)
    conf = L.confidence(d, inp["h"], wts["W1"], wts["w"], T, inp["anchor"], tok)
    dl, ro, st = L.plan(d, conf, sps_t, mode)
    ref = (tok, q, lse, e, conf, dl, ro, st)
    L.profile_begin()
    try:
        got = L.rnn_draft_plan(d, inp["U"], wts["W1"], wts["W2t"], Wgco, inp["h"], inp["anchor"],
                               inp["uniforms"], wts["w"], T, sps_t, mode, **opts)
        torch.cuda.synchronize()
    finally:
        prof = L.profile_end()
    for name, a, b in zip(("tokens", "q", "lse", "e_rows", "conf", "draft_len", "row_offsets",
                           "stats"), got, ref):
        _same(a, b, f"{wl.name} mode {mode}: {name}")
    assert (prof["plan"][0] == 0) == fused_expected, (wl.name, prof["plan"])
    log(f"  {wl.name}: mode {mode}, fused {fused_expected}")


@pytest.mark.parametrize("name", list(RNN_CASES))
def test_rnn_draft_plan_matches_the_separate_calls(name):
    wl, fused = RNN_CASES[name]
    modes = (L.EARLY_STOP,) if wl.V > 32000 else (L.EARLY_STOP, L.FULL_PATH)
    for mode in modes:
        _run_rnn_case(wl, fused, mode)


@pytest.mark.parametrize("temperature,greedy", [(0.6, False), (1.0, True)])
def test_rnn_draft_plan_options(temperature, greedy):
    wl, fused = RNN_CASES["rnn-b130-v4100-r128-g3"]
    _run_rnn_case(wl, fused, L.EARLY_STOP, temperature=temperature, greedy=greedy)
