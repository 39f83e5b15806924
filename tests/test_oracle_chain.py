"""Chained rounds of the lagged planner on the oracle (CPU): the cross-round state is exactly
(anchors, confidence ring, round index), so resuming from a saved state reproduces the
uninterrupted run bit for bit; the ring holds the confidences of the round two back; and the
chain exercises both the warm-up rounds (no history: early stop) and the lagged capacity.
[V41] "阈值随负载变化", [CSDN] 8, [ZDS] "在 SGLang 里"."""
import numpy as np

from lossless_draft_verify_amd import workloads as W
from oracle_chain import OracleChain, save_state

WL = W.scaled(W.WORKLOADS["b512-v129280-g5-lagged"], name="chain-b16-v300-g5", seed_id=31, B=16,
              V=300, r=16, d=32, sps_scale=16.0)


def _same(a, b):
    return np.array_equal(np.asarray(a), np.asarray(b))


def _run():
    wts = W.weights(WL)
    full, _ = OracleChain(WL, wts).run(OracleChain(WL, wts).initial_state(), WL.rounds)
    return wts, full


def test_resume_from_saved_state_equals_uninterrupted_run():
    wts, full = _run()
    first, state = OracleChain(WL, wts).run(OracleChain(WL, wts).initial_state(), 10)
    saved = save_state(state)
    resumed, _ = OracleChain(WL, wts).run(saved, WL.rounds - 10)
    for a, b in zip(full[10:], resumed):
        assert a["t"] == b["t"]
        assert _same(a["anchor"], b["anchor"])
        assert _same(a["draft"]["tokens"], b["draft"]["tokens"])
        assert _same(a["conf"], b["conf"])
        for k in ("draft_len", "row_offsets", "stats"):
            assert _same(a["plan"][k], b["plan"][k]), k
        for k in ("accept_len", "next_token", "beta_emit", "flags"):
            assert _same(a["verify"][k], b["verify"][k]), k
        assert _same(a["ring_after"], b["ring_after"])


def test_chain_ring_lag_and_anchor_hand_off():
    _, recs = _run()
    for t, rec in enumerate(recs):
        # the round writes its confidences into slot t mod 2, which held those of round t - 2
        assert _same(rec["ring_after"][t % 2], rec["conf"])
        if t >= 2:
            assert _same(rec["ring_before"][t % 2], recs[t - 2]["conf"])
            # capacity = B + the full-path count on the lagged slot; admitted = min(that, B gamma)
            k_lag = rec["plan"]["stats"][3] - WL.B
            assert int(rec["plan"]["draft_len"].sum()) == min(int(k_lag), WL.B * WL.gamma)
        else:
            assert rec["plan"]["stats"][3] == rec["plan"]["stats"][0]
        if t > 0:
            assert _same(rec["anchor"], recs[t - 1]["verify"]["next_token"])
    lens = np.concatenate([r["plan"]["draft_len"] for r in recs])
    assert lens.min() < lens.max(), "the chain should plan ragged lengths"
