"""GPU <-> oracle parity through the C ABI, per entry point and for whole rounds.

Inputs come from the seeded generators only; the oracle never receives anything the GPU
computed (GPU calls are fed oracle tokens / plans where a step needs the previous step's
output)."""
import numpy as np
import pytest
import torch

import oracle
import lossless_draft_verify_amd as L
from lossless_draft_verify_amd import workloads as W
from oracle_chain import OracleChain
from parity import (LSE_TOL, PLAN_TIE, PROB_TOL, MismatchCounter, bits, compare_draft, dims_of,
                    gpu_draft, log, np_, oracle_draft)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs the GPU")
    L.load_library()


def _custom(name, **kw):
    base = W.WORKLOADS["tiny-b4-v1000-g3"]
    return W.scaled(base, name=name, **kw)


DRAFT_CASES = {
    "tiny-b4-v1000-g3": W.WORKLOADS["tiny-b4-v1000-g3"],
    "b32-v32000-g7": W.WORKLOADS["b32-v32000-g7"],
    # two request groups (130 > 128), ragged 32-request tile, V % 4 != 0 (scalar path), tail tile
    "b130-v4099-r256-g3": _custom("b130-v4099-r256-g3", seed_id=11, B=130, V=4099, r=256, d=64,
                                  u_std=3.0, w_std=0.05),
    "b33-v2051-r64-g4": _custom("b33-v2051-r64-g4", seed_id=12, B=33, V=2051, r=64, gamma=4),
    "b7-v3000-r512-g2": _custom("b7-v3000-r512-g2", seed_id=13, B=7, V=3000, r=512, gamma=2,
                                w_std=0.03),
    "b5-v2-r16-g3": _custom("b5-v2-r16-g3", seed_id=14, B=5, V=2, r=16, gamma=3),
    # cases the pipelined (LDS-copy) step kernel takes (V % 4 == 0, r >= 64): two groups with a
    # ragged second one, a 4-token tail tile, r = 64 / 128, and a batch below one wave's 32
    "b130-v4100-r128-g3": _custom("b130-v4100-r128-g3", seed_id=15, B=130, V=4100, r=128,
                                  u_std=3.0, w_std=0.05),
    "b33-v2052-r64-g4": _custom("b33-v2052-r64-g4", seed_id=16, B=33, V=2052, r=64, gamma=4),
    "b20-v8192-r256-g2": _custom("b20-v8192-r256-g2", seed_id=17, B=20, V=8192, r=256, gamma=2,
                                 u_std=3.0, w_std=0.05),
    # three request groups (the third ragged) and the 512-thread sampler of batches past 256
    "b300-v4100-r256-g3": _custom("b300-v4100-r256-g3", seed_id=18, B=300, V=4100, r=256, d=64,
                                  u_std=3.0, w_std=0.05),
    # the 256-request one-tile step (B > 128, r = 256): a ragged second group whose second
    # wave is partly active, and three groups over the XCD-aware placement
    "b300-v4100-r256-g3": _custom("b300-v4100-r256-g3", seed_id=23, B=300, V=4100, r=256,
                                  u_std=3.0, w_std=0.05),
    "b520-v2052-r256-g2": _custom("b520-v2052-r256-g2", seed_id=24, B=520, V=2052, r=256,
                                  gamma=2, u_std=3.0, w_std=0.05),
    # three or four 64-token items per step workgroup: the partials flush with eight tile slots
    "b64-v57344-r256-g3": _custom("b64-v57344-r256-g3", seed_id=25, B=64, V=57344, r=256,
                                  gamma=3, u_std=3.0, w_std=0.05),
    # the largest vocabulary the library takes (2^19): 16 tiles per sampler thread, the
    # sampler's per-tile masses filling 128 KiB of LDS
    "b3-v524288-r64-g2": _custom("b3-v524288-r64-g2", seed_id=18, B=3, V=1 << 19, r=64, gamma=2),
}


def _forced_without_debug_matches(wl, inp, wts, g, force):
    """The step kernel without a debug output (the pipelined one wherever it applies) must give
    the same draws, q and lse, bit for bit, as the debug-output run g under the same forcing."""
    gn = gpu_draft(wl, inp, wts, force=force)
    for k in ("tokens", "q", "lse"):
        assert np.array_equal(gn[k], g[k]), k


@pytest.mark.parametrize("name", list(DRAFT_CASES))
def test_draft_parity(name):
    wl = DRAFT_CASES[name]
    log(f"[draft] {name}")
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False, with_noise=False)
    o = oracle_draft(inp, wts, want_logits=True)
    g = gpu_draft(wl, inp, wts, force=o["tokens"], dbg=True)
    c = MismatchCounter(f"draft {name}")
    err = compare_draft(g, o, c)
    log(f"  logits max err {err:.2e}; {c.report()}")
    _forced_without_debug_matches(wl, inp, wts, g, o["tokens"])
    # unforced GPU run: identical to the forced one wherever the draws agree
    gu = gpu_draft(wl, inp, wts)
    same = (gu["tokens"] == o["tokens"]).all(axis=1)
    assert np.array_equal(gu["q"][same], g["q"][same])
    c.check_rate()


def test_draft_logits_recompute_is_bit_exact():
    """The sampler recomputes one tile with the streaming pass's instruction sequence: forced
    q must equal exp(L - lse) from the debug logits exactly as recomputed in fp64 here."""
    wl = DRAFT_CASES["b130-v4099-r256-g3"]
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False, with_noise=False)
    g = gpu_draft(wl, inp, wts, dbg=True)
    Lg = np_(g["logits"]).astype(np.float64)
    x = g["tokens"]
    ref = np.exp(np.take_along_axis(Lg, x[..., None], 2)[..., 0] - g["lse"]).astype(np.float32)
    assert np.array_equal(ref, g["q"])


def test_draft_mismatch_rate_headline_shape():
    """2 x 10^4 draws at the production drafter's shape (V = 129280, r = 256, W std 0.05):
    every mismatch must be a flagged near tie, and mismatches must stay under 0.1 % of draws.
    The report gives how close to a CDF edge the mismatched draws were."""
    wl = W.scaled(W.WORKLOADS["b128-v129280-g5"], name="rate-r256", seed_id=22, B=1024, d=64)
    c = MismatchCounter("draft rate V=129280 r=256")
    wts = W.weights(wl, DEV)
    for rnd in range(4):
        inp = W.round_inputs(wl, rnd, DEV, with_hidden=False, with_noise=False)
        log(f"  round {rnd}: oracle")
        o = oracle_draft(inp, wts)
        g = gpu_draft(wl, inp, wts, force=o["tokens"])
        compare_draft(g, o, c, logits=False)
        log(f"  round {rnd}: {c.report()}")
        del inp
        torch.cuda.empty_cache()
    assert c.draws >= 20000
    c.check_rate()


def test_draft_mismatch_rate_headline_vocab():
    """2 x 10^4 draws at V = 129280 (r = 16 keeps the oracle fast): every mismatch must be a
    flagged near tie and mismatches must stay under 0.1 % of draws."""
    wl = W.scaled(W.WORKLOADS["b128-v129280-g5"], name="rate", seed_id=21, B=1024, r=16, d=64,
                  w_std=0.1)
    c = MismatchCounter("draft rate V=129280")
    wts = W.weights(wl, DEV)
    for rnd in range(4):
        inp = W.round_inputs(wl, rnd, DEV, with_hidden=False, with_noise=False)
        o = oracle_draft(inp, wts)
        g = gpu_draft(wl, inp, wts, force=o["tokens"])
        compare_draft(g, o, c, logits=False)
        log(f"  round {rnd}: {c.report()}")
        del inp
        torch.cuda.empty_cache()
    c.check_rate()


CONF_CASES = {
    "tiny-b4-v1000-g3": W.WORKLOADS["tiny-b4-v1000-g3"],
    "b128-v129280-g5": W.WORKLOADS["b128-v129280-g5"],
    # hidden sizes past one batch of loads (8192 elements): one piece in the second batch, and
    # two full batches; r = 512 puts an embedding-row piece on every lane of wave 0
    "b6-d8200-r512-g3": _custom("b6-d8200-r512-g3", seed_id=51, B=6, V=3000, r=512, d=8200,
                                gamma=3),
    "b5-d16384-r64-g2": _custom("b5-d16384-r64-g2", seed_id=52, B=5, V=2048, r=64, d=16384,
                                gamma=2),
    # the smallest hidden state: one piece, on thread 0 only
    "b7-d8-r16-g4": _custom("b7-d8-r16-g4", seed_id=53, B=7, V=1000, r=16, d=8, gamma=4),
}


@pytest.mark.parametrize("name", list(CONF_CASES))
def test_confidence_parity(name):
    wl = CONF_CASES[name]
    log(f"[confidence] {name}")
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=True)
    tokens = torch.randint(0, wl.V, (wl.B, wl.gamma), dtype=torch.int32, device=DEV)
    T = W.temperatures(wl).to(DEV)
    o = oracle.confidence(bits(inp["h"]), bits(wts["W1"]), bits(wts["w"]), np_(T), np_(inp["anchor"]),
                          np_(tokens))
    c = L.confidence(dims_of(wl), inp["h"], wts["W1"], wts["w"], T, inp["anchor"], tokens)
    err = np.abs(np_(c) - o["conf"]).max()
    log(f"  conf max err {err:.2e}")
    assert err <= PROB_TOL


def _plan_case(B, g, sps, seed):
    gen = torch.Generator().manual_seed(seed)
    conf = torch.rand((B, g), generator=gen, dtype=torch.float32)
    kind = seed % 4
    if kind == 1:
        conf[torch.rand((B, g), generator=gen) < 0.3] = 1.0
    elif kind == 2:
        conf = torch.round(conf * 4) / 4
    elif kind == 3:
        conf = 0.5 + 0.5 * conf
    return conf


@pytest.mark.parametrize("B,g,scale,seed", [(4, 3, 0.0, 1), (128, 5, 768.0, 2), (128, 5, 768.0, 3),
                                            (512, 5, 512.0, 4), (512, 5, 512.0, 5), (37, 7, 30.0, 6),
                                            (1, 2, 2.0, 7), (1024, 8, 2000.0, 8)])
def test_plan_parity(B, g, scale, seed):
    n = B * (g + 1) + 1
    sps = np.ones(n) if scale == 0 else 1.0 / (1.0 + np.arange(n) / scale)
    sps_t = torch.tensor(sps, dtype=torch.float64, device=DEV)
    d = L.Dims(B, g, 8, 16)
    for mode in (L.FULL_VERIFY, L.EARLY_STOP, L.FULL_PATH):
        conf = _plan_case(B, g, sps, seed)
        o = oracle.plan(conf.numpy(), sps, mode)
        dl, ro, st = L.plan(d, conf.to(DEV), sps_t, mode)
        if o["margin"] > PLAN_TIE:
            assert np.array_equal(np_(dl), o["draft_len"]), (mode, np_(dl), o["draft_len"])
            assert np.array_equal(np_(ro), o["row_offsets"])
            assert np.allclose(np_(st), o["stats"], rtol=1e-12, atol=0)
        else:
            log(f"  flagged planner tie (margin {o['margin']:.1e}), mode {mode}")
    # lagged capacity over rounds with the device ring
    ring_o = np.zeros((2, B, g), np.float32)
    ring_g = torch.zeros((2, B, g), dtype=torch.float32, device=DEV)
    for t in range(5):
        conf = _plan_case(B, g, sps, 100 * seed + t)
        o = oracle.plan(conf.numpy(), sps, L.LAGGED_TOPK, ring=ring_o, round_index=t)
        dl, ro, st = L.plan(d, conf.to(DEV), sps_t, L.LAGGED_TOPK, ring=ring_g, round_index=t)
        assert np.array_equal(np_(ring_g), ring_o)
        if o["margin"] > PLAN_TIE:
            assert np.array_equal(np_(dl), o["draft_len"]), t
            assert np.array_equal(np_(ro), o["row_offsets"])
            assert np.allclose(np_(st), o["stats"], rtol=1e-12, atol=0)


def _bucketed_sps(n, bucket, step, saw, rng):
    """Steps per second when the step time grows by `step` per bucket of verified tokens (a
    piecewise-constant, non-smooth table), optionally with a rise inside each bucket (sawtooth):
    Theta then has several local maxima along the admission path."""
    x = np.arange(n, dtype=np.float64)
    sps = 1.0 / (1.0 + np.floor(x / bucket) * step)
    if saw:
        sps = sps * (1.0 + rng.uniform(0.05, 0.3) * ((x % bucket) / bucket))
    return sps


@pytest.mark.parametrize("B,g,bucket,saw,seed", [(128, 5, 32, False, 61), (128, 5, 32, True, 62),
                                                 (512, 5, 64, True, 63), (37, 7, 8, True, 64)])
def test_plan_parity_bucketed_sps(B, g, bucket, saw, seed):
    """Planner parity under non-unimodal SPS tables (batch-bucketed step times, sawtooth): early
    stop halts at the first local maximum of Theta, full path finds the global one, and the
    lagged capacity takes the full-path count of the slot two rounds back."""
    rng = np.random.default_rng(seed)
    n = B * (g + 1) + 1
    sps = _bucketed_sps(n, bucket, rng.uniform(0.1, 0.5), saw, rng)
    sps_t = torch.tensor(sps, dtype=torch.float64, device=DEV)
    d = L.Dims(B, g, 8, 16)
    for mode in (L.EARLY_STOP, L.FULL_PATH):
        conf = _plan_case(B, g, sps, seed)
        o = oracle.plan(conf.numpy(), sps, mode)
        dl, ro, st = L.plan(d, conf.to(DEV), sps_t, mode)
        if o["margin"] > PLAN_TIE:
            assert np.array_equal(np_(dl), o["draft_len"]), mode
            assert np.array_equal(np_(ro), o["row_offsets"])
            assert np.allclose(np_(st), o["stats"], rtol=1e-12, atol=0)
    e = oracle.plan(_plan_case(B, g, sps, seed).numpy(), sps, L.EARLY_STOP)["draft_len"].sum()
    f = oracle.plan(_plan_case(B, g, sps, seed).numpy(), sps, L.FULL_PATH)["draft_len"].sum()
    ring_o = np.zeros((2, B, g), np.float32)
    ring_g = torch.zeros((2, B, g), dtype=torch.float32, device=DEV)
    for t in range(6):
        conf = _plan_case(B, g, sps, 100 * seed + t)
        o = oracle.plan(conf.numpy(), sps, L.LAGGED_TOPK, ring=ring_o, round_index=t)
        dl, ro, st = L.plan(d, conf.to(DEV), sps_t, L.LAGGED_TOPK, ring=ring_g, round_index=t)
        assert np.array_equal(np_(ring_g), ring_o)
        if o["margin"] > PLAN_TIE:
            assert np.array_equal(np_(dl), o["draft_len"]), t
            assert np.array_equal(np_(ro), o["row_offsets"])
            assert np.allclose(np_(st), o["stats"], rtol=1e-12, atol=0)
    log(f"  B={B} bucket={bucket} saw={saw}: early stop admits {e}, full path {f}")


def decisive_margin(ov, al_gpu, gamma):
    """Margin of the accept test that separates the two accept lengths (the first position
    where the GPU and the oracle could disagree)."""
    k = np.minimum(np.minimum(al_gpu, ov["accept_len"]), gamma - 1)
    return ov["accept_margin"][np.arange(len(k)), k]


def _oracle_round(wl, inp, wts, mode, conf=None):
    """Oracle draft (with logits) + plan + target rows; returns everything the round needs."""
    o = oracle_draft(inp, wts, want_logits=True)
    if conf is None and mode != W.FULL_VERIFY:
        T = W.temperatures(wl).numpy()
        conf = oracle.confidence(bits(inp["h"]), bits(wts["W1"]), bits(wts["w"]), T,
                                 np_(inp["anchor"]), o["tokens"])["conf"]
    sps = W.sps_table(wl)
    if mode == W.FULL_VERIFY and conf is None:
        p = oracle.plan(None, sps, mode, B=wl.B, gamma=wl.gamma)
    else:
        p = oracle.plan(conf, sps, mode)
    dense = np.concatenate([o["logits"], np_(inp["U_bonus"])[:, None, :]], 1) + np_(inp["noise"])
    keep = np.arange(wl.gamma + 1)[None, :] <= p["draft_len"][:, None]
    target = np.ascontiguousarray(dense[keep], dtype=np.float32)
    return o, conf, p, target


VERIFY_CASES = ["tiny-b4-v1000-g3", "b32-v32000-g7", "b130-v4099-r256-g3", "b33-v2051-r64-g4",
                "b5-v2-r16-g3"]


@pytest.mark.parametrize("name", VERIFY_CASES)
def test_verify_parity(name):
    wl = DRAFT_CASES.get(name) or W.WORKLOADS[name]
    log(f"[verify] {name}")
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False)
    # ragged verify lengths from a random confidence under a steep SPS
    rng = np.random.default_rng(wl.seed_id)
    conf = rng.uniform(0.3, 1.0, (wl.B, wl.gamma)).astype(np.float32)
    wl_p = W.scaled(wl, sps_kind="hyperbolic", sps_scale=max(1.0, wl.B * 1.5))
    o, conf, p, target = _oracle_round(wl_p, inp, wts, W.EARLY_STOP, conf=conf)
    ov = oracle.verify(target, p["row_offsets"], p["draft_len"], np_(inp["U"]), bits(wts["W1"]),
                       bits(wts["W2t"]), np_(inp["anchor"]), o["tokens"], o["q"], np_(inp["uniforms"]))
    g = gpu_draft(wl, inp, wts, force=o["tokens"])
    d = dims_of(wl)
    T = lambda a, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device=DEV)
    al, nt, be, fl = L.verify(d, T(target, torch.float32), T(p["row_offsets"]), T(p["draft_len"]),
                              inp["U"], wts["W1"], wts["W2t"], inp["anchor"], T(o["tokens"]),
                              T(o["q"], torch.float32), g["lse_t"], inp["uniforms"])
    torch.cuda.synchronize()
    al, nt, be, fl = np_(al), np_(nt), np_(be), np_(fl)
    acc = MismatchCounter(f"accept {name}")
    acc.add(al, ov["accept_len"], decisive_margin(ov, al, wl.gamma))
    same = al == ov["accept_len"]
    emit = MismatchCounter(f"emit {name}")
    emit.add(nt[same], ov["next_token"][same], ov["emit_margin"][same])
    assert np.array_equal(fl[same].astype(np.uint32), ov["flags"][same])
    assert np.abs(be[same] - ov["beta_emit"][same]).max() <= PROB_TOL
    log(f"  {acc.report()}; {emit.report()}; residual rows {int((ov['beta_emit'] >= 0).sum())}")


def test_verify_long_block():
    """Full verify of a 20-token block (21 rows a request, more than one batch of the accept
    scan's per-row reductions) at a vocabulary of fewer than 32 segments."""
    wl = _custom("b9-v3000-r64-g20", seed_id=19, B=9, V=3000, r=64, gamma=20, noise_std=lambda k: 0.05)
    log(f"[verify] {wl.name}")
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False)
    o, conf, p, target = _oracle_round(wl, inp, wts, W.FULL_VERIFY)
    assert (p["draft_len"] == wl.gamma).all()
    ov = oracle.verify(target, p["row_offsets"], p["draft_len"], np_(inp["U"]), bits(wts["W1"]),
                       bits(wts["W2t"]), np_(inp["anchor"]), o["tokens"], o["q"], np_(inp["uniforms"]))
    g = gpu_draft(wl, inp, wts, force=o["tokens"])
    al, nt, be, fl = L.verify(dims_of(wl), _T(target, torch.float32), _T(p["row_offsets"]),
                              _T(p["draft_len"]), inp["U"], wts["W1"], wts["W2t"], inp["anchor"],
                              _T(o["tokens"]), _T(o["q"], torch.float32), g["lse_t"],
                              inp["uniforms"])
    torch.cuda.synchronize()
    al, nt, be = np_(al), np_(nt), np_(be)
    acc = MismatchCounter("accept long block")
    acc.add(al, ov["accept_len"], decisive_margin(ov, al, wl.gamma))
    same = al == ov["accept_len"]
    emit = MismatchCounter("emit long block")
    emit.add(nt[same], ov["next_token"][same], ov["emit_margin"][same])
    assert np.abs(be[same] - ov["beta_emit"][same]).max() <= PROB_TOL
    assert ov["accept_len"].max() >= 16, "some request should accept into the second batch of rows"
    log(f"  accepted {ov['accept_len'].tolist()}; {acc.report()}")


@pytest.mark.parametrize("name", ["b128-v129280-g5", "b32-v32000-g7", "b128-v151936-g15"])
def test_round_full_size(name):
    """A whole round at the workload's full size, every request checked against the oracle."""
    wl = W.WORKLOADS[name]
    log(f"[round] {name}: generating")
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV)
    d = dims_of(wl)
    log("  oracle round")
    o, conf_o, p, target = _oracle_round(wl, inp, wts, wl.mode)
    ov = oracle.verify(target, p["row_offsets"], p["draft_len"], np_(inp["U"]), bits(wts["W1"]),
                       bits(wts["W2t"]), np_(inp["anchor"]), o["tokens"], o["q"], np_(inp["uniforms"]))
    log("  gpu round")
    gu = gpu_draft(wl, inp, wts)                          # the GPU's own draws
    c = MismatchCounter(f"round draft {name}")
    c.add(gu["tokens"][:, :1], o["tokens"][:, :1], o["margin"][:, :1])
    g = gpu_draft(wl, inp, wts, force=o["tokens"], dbg=True)
    err = compare_draft(g, o, c)
    _forced_without_debug_matches(wl, inp, wts, g, o["tokens"])
    log(f"  draft: logits err {err:.2e}; {c.report()}")
    T = lambda a, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device=DEV)
    tok_o = T(o["tokens"])
    if wl.mode != W.FULL_VERIFY:
        Tt = W.temperatures(wl).to(DEV)
        cg = L.confidence(d, inp["h"], wts["W1"], wts["w"], Tt, inp["anchor"], tok_o)
        assert np.abs(np_(cg) - conf_o).max() <= PROB_TOL
        # plan on the oracle's confidences (the GPU's agree within 1e-6 but a plan input must be
        # identical on both sides for an exact comparison)
        dl, ro, st = L.plan(d, T(conf_o, torch.float32), T(W.sps_table(wl), torch.float64), wl.mode)
    else:
        dl, ro, st = L.plan(d, None, T(W.sps_table(wl), torch.float64), wl.mode)
    if p["margin"] > PLAN_TIE:
        assert np.array_equal(np_(dl), p["draft_len"])
        assert np.array_equal(np_(ro), p["row_offsets"])
    log(f"  plan: B_tot {p['stats'][0]:.0f}, tau {p['stats'][1]:.2f}")
    al, nt, be, fl = L.verify(d, T(target, torch.float32), ro, dl, inp["U"], wts["W1"], wts["W2t"],
                              inp["anchor"], tok_o, T(o["q"], torch.float32), g["lse_t"],
                              inp["uniforms"])
    torch.cuda.synchronize()
    al, nt, be = np_(al), np_(nt), np_(be)
    acc = MismatchCounter("accept")
    acc.add(al, ov["accept_len"], decisive_margin(ov, al, wl.gamma))
    same = al == ov["accept_len"]
    emit = MismatchCounter("emit")
    emit.add(nt[same], ov["next_token"][same], ov["emit_margin"][same])
    assert np.abs(be[same] - ov["beta_emit"][same]).max() <= PROB_TOL
    log(f"  verify: mean accepted {al.mean():.2f}; {acc.report()}; {emit.report()}")


def _T(a, dt=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device=DEV)


def _compare_chain_round(wl, wts, rec, ring_g, sps_t, temps, cd, ca, ce):
    """One oracle-driven round of the lagged chain: each entry point gets the oracle's inputs
    (anchor, drafted tokens, confidences, plan) and is compared with it, the device ring
    included."""
    d = dims_of(wl)
    inp = {k: v.to(DEV) for k, v in rec["inp"].items()}
    inp["anchor"] = _T(rec["anchor"])
    o, p, ov = rec["draft"], rec["plan"], rec["verify"]
    gu = gpu_draft(wl, inp, wts)
    cd.add(gu["tokens"][:, :1], o["tokens"][:, :1], o["margin"][:, :1])
    del gu
    g = gpu_draft(wl, inp, wts, force=o["tokens"], dbg=True)
    compare_draft(g, o, cd)
    tok = _T(o["tokens"])
    cg = L.confidence(d, inp["h"], wts["W1"], wts["w"], temps, inp["anchor"], tok)
    assert np.abs(np_(cg) - rec["conf"]).max() <= PROB_TOL
    dl, ro, st = L.plan(d, _T(rec["conf"], torch.float32), sps_t, L.LAGGED_TOPK, ring=ring_g,
                        round_index=rec["t"])
    torch.cuda.synchronize()
    assert np.array_equal(np_(ring_g), rec["ring_after"]), rec["t"]
    if p["margin"] > PLAN_TIE:
        assert np.array_equal(np_(dl), p["draft_len"]), rec["t"]
        assert np.array_equal(np_(ro), p["row_offsets"]), rec["t"]
        assert np.allclose(np_(st), p["stats"], rtol=1e-12, atol=0), rec["t"]
    al, nt, be, fl = L.verify(d, _T(rec["target"], torch.float32), _T(p["row_offsets"]),
                              _T(p["draft_len"]), inp["U"], wts["W1"], wts["W2t"],
                              inp["anchor"], tok, _T(o["q"], torch.float32), g["lse_t"],
                              inp["uniforms"])
    torch.cuda.synchronize()
    al, nt, be, fl = np_(al), np_(nt), np_(be), np_(fl)
    ca.add(al, ov["accept_len"], decisive_margin(ov, al, wl.gamma))
    same = al == ov["accept_len"]
    ce.add(nt[same], ov["next_token"][same], ov["emit_margin"][same])
    assert np.array_equal(fl[same].astype(np.uint32), ov["flags"][same])
    assert np.abs(be[same] - ov["beta_emit"][same]).max() <= PROB_TOL
    log(f"  round {rec['t']}: B_tot {p['stats'][0]:.0f}, capacity {p['stats'][3]:.0f}, "
        f"mean accepted {al.mean():.2f}, rejected {int((be >= 0).sum())}")


def _oracle_chain(wl, rounds):
    log(f"[chain] {wl.name}: {rounds} rounds, oracle-driven")
    wts_cpu = W.weights(wl)
    wts = {k: v.to(DEV) for k, v in wts_cpu.items()}
    chain = OracleChain(wl, wts_cpu)
    state = chain.initial_state()
    ring_g = torch.zeros((2, wl.B, wl.gamma), dtype=torch.float32, device=DEV)
    sps_t = _T(W.sps_table(wl), torch.float64)
    temps = W.temperatures(wl).to(DEV)
    cd, ca, ce = (MismatchCounter("chain draft"), MismatchCounter("chain accept"),
                  MismatchCounter("chain emit"))
    for _ in range(rounds):
        rec, state = chain.step(state)      # one round at a time: the next needs its anchors
        _compare_chain_round(wl, wts, rec, ring_g, sps_t, temps, cd, ca, ce)
        del rec
        torch.cuda.empty_cache()
    log(f"  {cd.report()}; {ca.report()}; {ce.report()}")
    for c in (cd, ca, ce):
        c.check_rate()


def test_lagged_chain_parity():
    """Twenty chained rounds of the lagged planner at a scaled high-load shape (two request
    groups, the second ragged; a vocabulary tail): the oracle drives the chain (next anchor =
    its emitted token), and every round each entry point gets the oracle's inputs and is compared
    with it, the device confidence ring included."""
    wl = W.scaled(W.WORKLOADS["b512-v129280-g5-lagged"], name="chain-b160-v4100-g5", seed_id=32,
                  B=160, V=4100, d=256, sps_scale=160.0)
    _oracle_chain(wl, wl.rounds)


def test_lagged_chain_full_size_oracle():
    """The high-load workload at its full size (B = 512, V = 129280, r = 256, d = 5120, steep
    SPS, lag-2 ring): four chained rounds driven by the oracle, so rounds 2 and 3 plan from the
    device ring; every entry point is compared with the oracle element by element in the launch
    configuration the bench uses (four 128-request groups in the draft step with their XCD
    placement, several 64-request groups in the residual pass)."""
    _oracle_chain(W.WORKLOADS["b512-v129280-g5-lagged"], 4)


def _admission(conf, sps, B, gamma, mode):
    """Admission count along the survival order (numpy, from the definition): running fp64
    products per request, order by (-a, candidate index), tau_i = B + the first i survivals,
    Theta_i = tau_i * sps[B + i]; early stop at the first non-increase, full path at the first
    maximum. Returns (count, order, relative margin of the deciding comparison)."""
    a = np.cumprod(conf.astype(np.float64), axis=1).reshape(-1)
    n = a.size
    order = np.lexsort((np.arange(n), -a))
    tau = B + np.concatenate([[0.0], np.cumsum(a[order])])
    theta = tau * sps[B:B + n + 1]
    if mode == L.EARLY_STOP:
        stop = np.nonzero(~(theta[1:] > theta[:-1]))[0]
        count = int(stop[0]) if stop.size else n
        k = min(count, n - 1)   # comparisons 0 .. k decided the count
        gaps = np.abs(theta[1:k + 2] - theta[:k + 1]) / theta[:k + 1]
        return count, order, float(gaps.min()) if gaps.size else np.inf
    count = int(np.argmax(theta))
    rest = np.delete(theta, count)
    margin = (theta[count] - rest.max()) / theta[count] if rest.size else np.inf
    return count, order, float(margin)


def test_lagged_chain_full_size():
    """The high-load workload at full size (B = 512, V = 129280) for its 20 chained rounds, in
    the launch configuration the bench uses, driven by the GPU's own draws (next anchor = the
    emitted token). Checked by properties that hold at any size: the ring holds each round's
    confidences for the round two later; the lengths follow the lagged-capacity definition
    recomputed from the confidences (numpy); the packed offsets, the accept lengths, the emitted
    tokens and the beta values are consistent."""
    wl = W.WORKLOADS["b512-v129280-g5-lagged"]
    log(f"[chain] {wl.name}: {wl.rounds} rounds on the GPU")
    wts = W.weights(wl, DEV)
    d = dims_of(wl)
    B, g, V = wl.B, wl.gamma, wl.V
    sps = W.sps_table(wl)
    sps_t, temps = _T(sps, torch.float64), W.temperatures(wl).to(DEV)
    ring = torch.zeros((2, B, g), dtype=torch.float32, device=DEV)
    confs, anchor = [], None
    checked = 0
    for t in range(wl.rounds):
        inp = W.round_inputs(wl, t, DEV)
        if anchor is not None:
            inp["anchor"] = anchor
        logits = torch.empty_like(inp["U"])
        tok, q, lse = L.markov_draft(d, inp["U"], wts["W1"], wts["W2t"], inp["anchor"],
                                     inp["uniforms"], logits_dbg=logits)
        conf = L.confidence(d, inp["h"], wts["W1"], wts["w"], temps, inp["anchor"], tok)
        before = np_(ring).copy()
        dl, ro, st = L.plan(d, conf, sps_t, L.LAGGED_TOPK, ring=ring, round_index=t)
        torch.cuda.synchronize()
        c, dl_h, ro_h, st_h, after = np_(conf), np_(dl), np_(ro), np_(st), np_(ring)
        confs.append(c)
        assert np.array_equal(after[t % 2], c) and np.array_equal(after[1 - t % 2], before[1 - t % 2])
        if t >= 2:
            assert np.array_equal(before[t % 2], confs[t - 2])
            k_lag, _, m_lag = _admission(confs[t - 2], sps, B, g, L.FULL_PATH)
            _, order, _ = _admission(c, sps, B, g, L.FULL_PATH)
            n = min(k_lag, B * g)
            if m_lag > PLAN_TIE:
                assert st_h[3] == B + k_lag
                assert np.array_equal(dl_h, np.bincount(order[:n] // g, minlength=B)), t
                checked += 1
        else:
            n, order, m = _admission(c, sps, B, g, L.EARLY_STOP)
            if m > PLAN_TIE:
                assert np.array_equal(dl_h, np.bincount(order[:n] // g, minlength=B)), t
                checked += 1
        assert st_h[0] == B + dl_h.sum()
        assert np.array_equal(ro_h, np.concatenate([[0], np.cumsum(1 + dl_h)]))
        target = W.pack_rows(W.target_dense(logits, inp["U_bonus"], inp["noise"]), dl)
        del logits
        al, nt, be, fl = L.verify(d, target, ro, dl, inp["U"], wts["W1"], wts["W2t"],
                                  inp["anchor"], tok, q, lse, inp["uniforms"])
        torch.cuda.synchronize()
        al_h, nt_h, be_h, fl_h = np_(al), np_(nt), np_(be), np_(fl)
        assert ((al_h >= 0) & (al_h <= dl_h)).all()
        assert ((nt_h >= 0) & (nt_h < V)).all()
        assert (fl_h == 0).all()
        bonus = al_h == dl_h
        assert (be_h[bonus] == -1.0).all()
        assert ((be_h[~bonus] >= 0.0) & (be_h[~bonus] <= 1.0)).all()
        anchor = nt.to(torch.int32).contiguous()
        log(f"  round {t}: B_tot {st_h[0]:.0f}, capacity {st_h[3]:.0f}, mean accepted "
            f"{al_h.mean():.2f}, bonus {bonus.mean():.2f}")
        del inp, target
    assert checked >= wl.rounds - 2


def test_graph_replay_matches_eager():
    """A whole round (draft, confidence, plan, verify) captured once as a hipGraph and replayed
    several times, with unrelated eager work and synchronisations between the replays and the
    outputs overwritten before each one: every replay must reproduce the eager round bit for
    bit (all shapes the kernels need live on the device, and no call records a memset)."""
    wl = W.scaled(W.WORKLOADS["b128-v129280-g5"], name="graph-b64-v8192-g5", seed_id=40, B=64,
                  V=8192, d=256, sps_scale=64.0)
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV)
    d = dims_of(wl)
    B, g = wl.B, wl.gamma
    temps = W.temperatures(wl).to(DEV)
    sps = _T(W.sps_table(wl), torch.float64)
    logits = torch.empty_like(inp["U"])
    t0, _, _ = L.markov_draft(d, inp["U"], wts["W1"], wts["W2t"], inp["anchor"], inp["uniforms"],
                              logits_dbg=logits)
    c0 = L.confidence(d, inp["h"], wts["W1"], wts["w"], temps, inp["anchor"], t0)
    dl0, _, _ = L.plan(d, c0, sps, wl.mode)
    target = W.pack_rows(W.target_dense(logits, inp["U_bonus"], inp["noise"]), dl0)
    del logits
    ws_d, ws_v = L.workspace(d, L.OP_DRAFT, DEV), L.workspace(d, L.OP_VERIFY, DEV)
    out = dict(tok=torch.empty((B, g), dtype=torch.int32, device=DEV),
               q=torch.empty((B, g), dtype=torch.float32, device=DEV),
               lse=torch.empty((B, g), dtype=torch.float64, device=DEV),
               conf=torch.empty((B, g), dtype=torch.float32, device=DEV),
               dl=torch.empty(B, dtype=torch.int32, device=DEV),
               ro=torch.empty(B + 1, dtype=torch.int32, device=DEV),
               st=torch.empty(4, dtype=torch.float64, device=DEV),
               al=torch.empty(B, dtype=torch.int32, device=DEV),
               nt=torch.empty(B, dtype=torch.int32, device=DEV),
               be=torch.empty(B, dtype=torch.float32, device=DEV),
               fl=torch.empty(B, dtype=torch.int32, device=DEV))

    def round_():
        o = out
        L.markov_draft(d, inp["U"], wts["W1"], wts["W2t"], inp["anchor"], inp["uniforms"],
                       tokens=o["tok"], q=o["q"], lse=o["lse"], ws=ws_d)
        L.confidence(d, inp["h"], wts["W1"], wts["w"], temps, inp["anchor"], o["tok"], conf=o["conf"])
        L.plan(d, o["conf"], sps, wl.mode, draft_len=o["dl"], row_offsets=o["ro"], stats=o["st"])
        L.verify(d, target, o["ro"], o["dl"], inp["U"], wts["W1"], wts["W2t"], inp["anchor"],
                 o["tok"], o["q"], o["lse"], inp["uniforms"], accept_len=o["al"],
                 next_token=o["nt"], beta_emit=o["be"], flags=o["fl"], ws=ws_v)

    round_()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    assert torch.equal(eager["dl"], dl0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_()
    torch.cuda.synchronize()
    for rep in range(4):
        junk = torch.randn(1 << 20, device=DEV)
        _ = float(junk.square().sum().item())          # eager work between the replays
        for v in out.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, eager[k]), (rep, k)
    log(f"  graph replays match the eager round (B_tot {eager['st'][0].item():.0f})")


def test_determinism_bitwise():
    wl = W.WORKLOADS["b32-v32000-g7"]
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False, with_noise=False)
    a = gpu_draft(wl, inp, wts)
    b = gpu_draft(wl, inp, wts)
    for k in ("tokens", "q", "lse"):
        assert np.array_equal(a[k], b[k])


def test_nonfinite_flags_match_oracle():
    wl = DRAFT_CASES["tiny-b4-v1000-g3"]
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False)
    o = oracle_draft(inp, wts, want_logits=True)
    B, g, V = wl.B, wl.gamma, wl.V
    dense = np.concatenate([o["logits"], np_(inp["U_bonus"])[:, None, :]], 1) + np_(inp["noise"])
    dense = np.ascontiguousarray(dense.reshape(-1, V), dtype=np.float32)
    dense[0 * (g + 1) + 0, 5] = np.nan          # request 0: first verified row
    dense[1 * (g + 1) + g, :] = -np.inf          # request 1: bonus row all -inf
    offs = (np.arange(B + 1) * (g + 1)).astype(np.int32)
    dl = np.full(B, g, np.int32)
    ov = oracle.verify(dense, offs, dl, np_(inp["U"]), bits(wts["W1"]), bits(wts["W2t"]),
                       np_(inp["anchor"]), o["tokens"], o["q"], np_(inp["uniforms"]))
    gd = gpu_draft(wl, inp, wts, force=o["tokens"])
    T = lambda a, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device=DEV)
    al, nt, be, fl = L.verify(dims_of(wl), T(dense, torch.float32), T(offs), T(dl), inp["U"],
                              wts["W1"], wts["W2t"], inp["anchor"], T(o["tokens"]),
                              T(o["q"], torch.float32), gd["lse_t"], inp["uniforms"])
    torch.cuda.synchronize()
    assert np_(fl)[0] & L.FLAG_NONFINITE and ov["flags"][0] & L.FLAG_NONFINITE
    assert np.array_equal(np_(al)[:1], ov["accept_len"][:1])
    assert np.array_equal(np_(nt)[:1], ov["next_token"][:1])
    if ov["accept_len"][1] == g:
        assert np_(fl)[1] & L.FLAG_NONFINITE and ov["flags"][1] & L.FLAG_NONFINITE
        assert np_(nt)[1] == ov["next_token"][1] == 0


def _verify_against_oracle(wl, name, noise_scale=1.0):
    """Full verify of every drafted token against the oracle on the oracle's own draft; returns
    the oracle's and the GPU's accept lengths."""
    log(f"[verify edge] {name}")
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False)
    inp["noise"] = inp["noise"] * noise_scale
    o, conf, p, target = _oracle_round(wl, inp, wts, W.FULL_VERIFY)
    ov = oracle.verify(target, p["row_offsets"], p["draft_len"], np_(inp["U"]), bits(wts["W1"]),
                       bits(wts["W2t"]), np_(inp["anchor"]), o["tokens"], o["q"],
                       np_(inp["uniforms"]))
    g = gpu_draft(wl, inp, wts, force=o["tokens"])
    al, nt, be, fl = L.verify(dims_of(wl), _T(target, torch.float32), _T(p["row_offsets"]),
                              _T(p["draft_len"]), inp["U"], wts["W1"], wts["W2t"], inp["anchor"],
                              _T(o["tokens"]), _T(o["q"], torch.float32), g["lse_t"],
                              inp["uniforms"])
    torch.cuda.synchronize()
    al, nt, be, fl = np_(al), np_(nt), np_(be), np_(fl)
    acc = MismatchCounter(f"accept {name}")
    acc.add(al, ov["accept_len"], decisive_margin(ov, al, wl.gamma))
    same = al == ov["accept_len"]
    emit = MismatchCounter(f"emit {name}")
    emit.add(nt[same], ov["next_token"][same], ov["emit_margin"][same])
    assert np.array_equal(fl[same].astype(np.uint32), ov["flags"][same])
    assert np.abs(be[same] - ov["beta_emit"][same]).max() <= PROB_TOL
    log(f"  accepted {ov['accept_len'].tolist()[:8]}...; {acc.report()}; {emit.report()}")
    return ov["accept_len"], al


def test_verify_largest_vocabulary():
    """The largest vocabulary the library takes (2^19 tokens, 128 target segments a row)."""
    _verify_against_oracle(DRAFT_CASES["b3-v524288-r64-g2"], "b3-v524288-r64-g2")


def test_verify_longest_block():
    """The longest block (gamma 255: 256 rows a request, four 64-row batches of the accept
    scan), with a low-noise target so that long runs are accepted."""
    wl = _custom("b2-v1000-r16-g255", seed_id=92, B=2, V=1000, r=16, gamma=255,
                 noise_std=lambda k: 0.02)
    acc, _ = _verify_against_oracle(wl, "b2-v1000-g255")
    assert acc.max() >= 64, "a request should accept into the second batch of rows"


def test_verify_target_equal_to_draft():
    """Target = draft logits exactly (no noise): p_t = p_d, so every test passes unless the
    fp32 rounding of q puts u q at p_t (probability ~1e-7), and every request takes the bonus."""
    wl = _custom("b64-v4000-r64-g6-exact", seed_id=93, B=64, V=4000, r=64, gamma=6)
    acc, al = _verify_against_oracle(wl, "b64-v4000-g6 exact target", noise_scale=0.0)
    assert (acc == wl.gamma).mean() >= 0.99 and np.array_equal(acc, al)


@pytest.mark.parametrize("name", ["tiny-b4-v1000-g3", "b20-v8192-r256-g2"])
def test_out_of_range_token_ids_are_clamped(name):
    """Token ids a caller passes outside [0, V) (anchors, forced draft tokens, the drafted tokens
    given to the confidence head and the verify) and verify lengths past gamma are clamped on the
    device: every call gives the same bits as with the clamped values, and no access leaves the
    tensors."""
    wl = DRAFT_CASES[name]
    B, g, V = wl.B, wl.gamma, wl.V
    d = dims_of(wl)
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=False)
    raw = torch.tensor([-7, V, V + 100, 5] * ((B + 3) // 4), dtype=torch.int32, device=DEV)[:B]
    clamped = raw.clamp(0, V - 1).contiguous()
    run = lambda anc, **kw: [np_(t) for t in L.markov_draft(d, inp["U"], wts["W1"], wts["W2t"],
                                                             anc, inp["uniforms"], **kw)]
    for a, b_ in zip(run(raw), run(clamped)):
        assert np.array_equal(a, b_)
    force = torch.full((B, g), V + 3, dtype=torch.int32, device=DEV)
    force[:, ::2] = -2
    fc = force.clamp(0, V - 1).contiguous()
    for a, b_ in zip(run(clamped, force_tokens=force), run(clamped, force_tokens=fc)):
        assert np.array_equal(a, b_)
    tok, q, lse = L.markov_draft(d, inp["U"], wts["W1"], wts["W2t"], clamped, inp["uniforms"])
    bad_tok = tok.clone()
    bad_tok[:, 0] = -1
    bad_tok[:, -1] = V + 9
    h = torch.randn((B, g, wl.d), device=DEV).to(torch.bfloat16)
    temps = W.temperatures(wl).to(DEV)
    c_raw = L.confidence(d, h, wts["W1"], wts["w"], temps, raw, bad_tok)
    c_cl = L.confidence(d, h, wts["W1"], wts["w"], temps, clamped, bad_tok.clamp(0, V - 1).contiguous())
    assert torch.equal(c_raw, c_cl)
    offs = _T(np.arange(B + 1) * (g + 1))
    target = torch.randn((B * (g + 1), V), device=DEV)
    long_len = _T(np.full(B, g + 5))
    full_len = _T(np.full(B, g))
    out_raw = L.verify(d, target, offs, long_len, inp["U"], wts["W1"], wts["W2t"], raw, bad_tok,
                       q, lse, inp["uniforms"])
    out_cl = L.verify(d, target, offs, full_len, inp["U"], wts["W1"], wts["W2t"], clamped,
                      bad_tok.clamp(0, V - 1).contiguous(), q, lse, inp["uniforms"])
    torch.cuda.synchronize()
    for a, b_ in zip(out_raw, out_cl):
        assert torch.equal(a, b_)
    nt = np_(out_raw[1])
    assert ((nt >= 0) & (nt < V)).all()
    shape = L.TreeShape(2, 2, 4)
    ta = [np_(t) for t in L.tree_draft(d, shape, inp["U"], wts["W1"], wts["W2t"], raw)]
    tb = [np_(t) for t in L.tree_draft(d, shape, inp["U"], wts["W1"], wts["W2t"], clamped)]
    for a, b_ in zip(ta, tb):
        assert np.array_equal(a, b_)
