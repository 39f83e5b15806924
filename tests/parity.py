"""Helpers for GPU <-> oracle parity tests: run one side or the other on identical inputs and
compare under the stated tolerances.

Tolerances (from the workload contract): logits 2e-3 absolute; probabilities (q, p_t(x),
confidence, beta) 1e-6 absolute; log-sum-exp 1e-5 absolute; tokens, accept lengths, planner
lengths and row offsets exact, except on flagged near-tie draws (the oracle's uniform lies
within 1e-5 of a CDF edge, or within 1e-5 of p_t/q for an accept test, or a planner Theta
comparison is within 1e-12 relative), and mismatches must stay under 0.1 % of draws.
"""
import sys

import numpy as np
import torch

import oracle
import lossless_draft_verify_amd as L
from lossless_draft_verify_amd import workloads as W

LOGIT_TOL = 2e-3
PROB_TOL = 1e-6
LSE_TOL = 1e-5
NEAR_TIE = 1e-5
PLAN_TIE = 1e-12
MAX_MISMATCH_RATE = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np_(t):
    return t.detach().cpu().numpy()


def bits(t):
    return W.bf16_bits(t)


def dims_of(wl, B=None):
    return L.Dims(B or wl.B, wl.gamma, wl.V, wl.r, wl.d)


class MismatchCounter:
    """Token draws of one kind compared with the oracle's.

    A draw is *flagged* when the GPU's token differs from the oracle's and the oracle's uniform
    lies within `tie` of a CDF edge (the edge the two tokens disagree about): the only draws on
    which a mismatch is allowed, and they must stay under 0.1 % of the draws. Draws whose
    uniform merely lies that close to some edge while both sides agree are counted apart as
    near-edge draws; how many there are is a property of the inputs (at V = 129280 the mean
    distance between edges is 7.7e-6, under the 1e-5 margin), not of either implementation."""

    def __init__(self, what):
        self.what = what
        self.draws = 0
        self.mismatches = 0
        self.near_edge = 0
        self.worst = 0.0      # largest edge distance of a mismatched draw

    def add(self, gpu, ref, margin, tie=NEAR_TIE):
        gpu, ref, margin = np.asarray(gpu), np.asarray(ref), np.asarray(margin)
        near = margin < tie
        bad = gpu != ref
        unflagged = bad & ~near
        assert not unflagged.any(), (
            f"{self.what}: {int(unflagged.sum())} mismatches on draws that are not near ties; "
            f"first at {np.argwhere(unflagged)[:5].tolist()}")
        self.draws += bad.size
        self.mismatches += int(bad.sum())   # every one of them flagged (asserted above)
        if bad.any():
            self.worst = max(self.worst, float(margin[bad].max()))
        self.near_edge += int(near.sum())

    @property
    def flagged(self):
        return self.mismatches

    def rate(self):
        return self.flagged / max(1, self.draws)

    def check_rate(self):
        """Flagged draws (the allowed mismatches) under 0.1 % of this counter's draws; a counter
        of fewer than 1000 draws therefore allows none."""
        assert self.flagged < MAX_MISMATCH_RATE * self.draws or self.flagged == 0, (
            f"{self.what}: flagged-draw rate {self.rate():.2e} ({self.flagged}/{self.draws})")

    def report(self):
        return (f"{self.what}: draws {self.draws}, flagged mismatches {self.flagged} "
                f"({100 * self.rate():.3f} %, within {self.worst:.1e} of an edge), "
                f"near-edge draws {100 * self.near_edge / max(1, self.draws):.1f} %")


def gpu_draft(wl, inp, wts, force=None, dbg=False, B=None, temperature=1.0, greedy=False):
    d = dims_of(wl, B)
    dev = inp["U"].device
    logits = torch.empty_like(inp["U"]) if dbg else None
    f = None if force is None else torch.as_tensor(force, dtype=torch.int32, device=dev).contiguous()
    t, q, lse = L.markov_draft(d, inp["U"], wts["W1"], wts["W2t"], inp["anchor"], inp["uniforms"],
                               logits_dbg=logits, force_tokens=f, temperature=temperature,
                               greedy=greedy)
    torch.cuda.synchronize()
    return dict(tokens=np_(t), q=np_(q), lse=np_(lse), logits=None if logits is None else logits,
                tokens_t=t, q_t=q, lse_t=lse)


def oracle_draft(inp, wts, force=None, want_logits=False, temperature=1.0, greedy=False):
    return oracle.markov_draft(np_(inp["U"]), bits(wts["W1"]), bits(wts["W2t"]), np_(inp["anchor"]),
                               np_(inp["uniforms"]), force_tokens=force, want_logits=want_logits,
                               temperature=temperature, greedy=greedy)


def compare_draft(g, o, counter, logits=True):
    """g: GPU draft forced with the oracle's tokens; o: oracle draft (with logits if asked)."""
    counter.add(g["tokens"], o["tokens"], o["margin"])
    assert np.abs(g["q"] - o["q"]).max() <= PROB_TOL, np.abs(g["q"] - o["q"]).max()
    assert np.abs(g["lse"] - o["lse"]).max() <= LSE_TOL, np.abs(g["lse"] - o["lse"]).max()
    if logits and g["logits"] is not None and "logits" in o:
        err = np.abs(np_(g["logits"]) - o["logits"]).max()
        assert err <= LOGIT_TOL, err
        return float(err)
    return None


def packed_target(dense, draft_len):
    return W.pack_rows(dense, draft_len)
