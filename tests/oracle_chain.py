"""Chained rounds of the lagged planner on the oracle.

Each round drafts from the previous round's emitted token (the first from the generated anchor),
plans with the lag-2 confidence ring, builds the target stand-in from the oracle's own draft
logits plus noise, and verifies. The state carried from round to round is exactly (anchors,
ring, round index): [V41] "阈值随负载变化" (the capacity read from confidences two steps back),
[CSDN] 8 (the asynchronous planner), [ZDS] "在 SGLang 里" (the relay ring, lag 2)."""
import copy

import numpy as np

import oracle
from lossless_draft_verify_amd import workloads as W


def bits(t):
    return W.bf16_bits(t)


class OracleChain:
    def __init__(self, wl, wts):
        self.wl = wl
        self.W1, self.W2t, self.w = bits(wts["W1"]), bits(wts["W2t"]), bits(wts["w"])
        self.sps = W.sps_table(wl)
        self.T = W.temperatures(wl).numpy()

    def initial_state(self):
        wl = self.wl
        return dict(anchor=None, ring=np.zeros((2, wl.B, wl.gamma), np.float32), t=0)

    def step(self, state):
        """One round from `state`; returns (record of the round, next state)."""
        wl, t = self.wl, state["t"]
        inp = W.round_inputs(wl, t, "cpu")
        anchor = inp["anchor"].numpy() if state["anchor"] is None else state["anchor"]
        anchor = np.ascontiguousarray(anchor, np.int32)
        U, uni = inp["U"].numpy(), inp["uniforms"].numpy()
        o = oracle.markov_draft(U, self.W1, self.W2t, anchor, uni, want_logits=True)
        conf = oracle.confidence(bits(inp["h"]), self.W1, self.w, self.T, anchor,
                                 o["tokens"])["conf"]
        ring = state["ring"].copy()
        p = oracle.plan(conf, self.sps, W.LAGGED_TOPK, ring=ring, round_index=t)
        dense = np.concatenate([o["logits"], inp["U_bonus"].numpy()[:, None, :]], 1)
        dense = dense + inp["noise"].numpy()
        keep = np.arange(wl.gamma + 1)[None, :] <= p["draft_len"][:, None]
        target = np.ascontiguousarray(dense[keep], dtype=np.float32)
        ov = oracle.verify(target, p["row_offsets"], p["draft_len"], U, self.W1, self.W2t, anchor,
                           o["tokens"], o["q"], uni)
        rec = dict(t=t, inp=inp, anchor=anchor, draft=o, conf=conf, plan=p, target=target,
                   verify=ov, ring_before=state["ring"].copy(), ring_after=ring.copy())
        nxt = dict(anchor=ov["next_token"].astype(np.int32), ring=ring, t=t + 1)
        return rec, nxt

    def run(self, state, rounds):
        recs = []
        for _ in range(rounds):
            rec, state = self.step(state)
            recs.append(rec)
        return recs, state


def save_state(state):
    return copy.deepcopy(state)
