"""dspark_verify_noalloc (the verify on the library's fixed scratch array, for callers that
cannot allocate) against dspark_verify_opts on a caller workspace: two calls in a row on the
same GPU, the second with a smaller input, each bit for bit equal to the workspace path."""
import numpy as np
import pytest
import torch

import lossless_draft_verify_amd as L
from lossless_draft_verify_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _log(msg):
    print(msg, flush=True)


def _round(wl, opts):
    """Inputs of one verify: the GPU draft and plan, and a target stand-in (debug logits plus
    noise, packed by the plan)."""
    d = L.Dims(wl.B, wl.gamma, wl.V, wl.r, wl.d)
    wts = W.weights(wl, DEV)
    inp = W.round_inputs(wl, 0, DEV, with_hidden=True, with_noise=True)
    logits = torch.empty_like(inp["U"])
    tok, q, lse = L.markov_draft(d, inp["U"], wts["W1"], wts["W2t"], inp["anchor"],
                                 inp["uniforms"], logits_dbg=logits, **opts)
    sps = torch.tensor(W.sps_table(wl), dtype=torch.float64, device=DEV)
    if wl.mode == W.FULL_VERIFY:
        dl, ro, _ = L.plan(d, None, sps, wl.mode)
    else:
        conf = L.confidence(d, inp["h"], wts["W1"], wts["w"], W.temperatures(wl).to(DEV),
                            inp["anchor"], tok)
        dl, ro, _ = L.plan(d, conf, sps, wl.mode)
    target = W.pack_rows(W.target_dense(logits, inp["U_bonus"], inp["noise"]), dl)
    del logits
    return d, dict(target=target, row_offsets=ro, draft_len=dl, U=inp["U"], W1=wts["W1"],
                   W2t=wts["W2t"], anchor=inp["anchor"], tokens=tok, q=q, lse=lse,
                   uniforms=inp["uniforms"])


def _outputs(B):
    return dict(accept_len=torch.full((B,), -7, dtype=torch.int32, device=DEV),
                next_token=torch.full((B,), -7, dtype=torch.int32, device=DEV),
                beta_emit=torch.full((B,), -7.0, dtype=torch.float32, device=DEV),
                flags=torch.full((B,), -7, dtype=torch.int32, device=DEV))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs the GPU")
    L.load_library()


@pytest.mark.parametrize("opts", [{}, {"temperature": 0.6}, {"greedy": True}],
                         ids=["sampled", "tau0.6", "greedy"])
def test_noalloc_verify_matches_workspace_verify_on_two_calls(opts):
    for name in ("b128-v129280-g5", "b32-v32000-g7"):      # the second call is smaller
        wl = W.WORKLOADS[name]
        _log(f"[noalloc] {name} {opts}")
        d, a = _round(wl, opts)
        ref = _outputs(wl.B)
        got = _outputs(wl.B)
        L.verify(d, **a, **ref, **opts)
        torch.cuda.synchronize()
        L.verify_noalloc(d, **a, **got, **opts)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], got[k]), f"{name} {opts}: {k} differs"
        acc = ref["accept_len"].cpu().numpy()
        dl = a["draft_len"].cpu().numpy()
        assert (acc >= 0).all() and (acc <= dl).all()
        _log(f"  rows {int(a['row_offsets'][-1])}, rejected {(acc < dl).sum()}: equal")
        del a
        torch.cuda.empty_cache()
