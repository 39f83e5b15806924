"""Benchmark one DSpark draft-and-verify round on one MI355X.

A step is one whole round (Markov draft of gamma positions, confidence head, planner, verify)
over one batch of synthetic inputs already resident in HBM, for the headline workload
b128-v129280-g5 (B = 128 requests, V = 129280, gamma = 5, r = 256, d = 5120, early-stop planner,
SPS(n) = 1 / (1 + n / 768)). Three input sets rotate so the working set exceeds the 256 MB
Infinity Cache. Target logits (the out-of-scope target model) are prepared before timing from
each set's own draft logits plus noise, laid out in the planner's packed rows.

Prints one JSON line. `value` comes from K timed rounds with nothing recorded between launches;
per-kernel durations (and the roofline of the draft step kernel) come from a second pass of the
same K rounds with HIP events recorded around every library launch on the launch stream.

`--workload` runs another of the workloads instead (the full-verify ones as draft, plan and
verify; the lagged one with each input set's confidence ring in its steady state), reported
the same way under that workload's name.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import lossless_draft_verify_amd as L  # noqa: E402
from lossless_draft_verify_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, no sparsity
WORKLOAD = "b128-v129280-g5"
METRIC = "spec rounds/s at B=128,V=129280,γ=5; achieved HBM GB/s vs peak"
STEP_SOURCES = ["lossless_draft_verify_amd/csrc/kernels_draft.hip",
                "lossless_draft_verify_amd/csrc/tiles.h",
                "lossless_draft_verify_amd/csrc/device.h",
                "lossless_draft_verify_amd/csrc/dma.h"]


def step_source_sha():
    h = hashlib.sha256()
    for p in STEP_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(launch_units):
    """HBM bytes per markov_step launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "markov_step_b128-v129280-g5_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha:\s*([0-9a-f]+)", text)
    f = re.search(r"bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not f or m.group(1) != step_source_sha():
        return None
    return float(f.group(1))


# Round index given to the lagged planner in timed rounds: from round 2 on it reads the ring.
LAG_ROUND = 2


class InputSet:
    def __init__(self, wl, wts, round_index, dev, opts, head="markov"):
        d = L.Dims(wl.B, wl.gamma, wl.V, wl.r, wl.d)
        full = wl.mode == W.FULL_VERIFY
        inp = W.round_inputs(wl, round_index, dev, with_hidden=not full, with_noise=True)
        self.anchor, self.U, self.h, self.uniforms = (inp["anchor"], inp["U"], inp.get("h"),
                                                      inp["uniforms"])
        self.T = W.temperatures(wl).to(dev)
        self.sps = torch.tensor(W.sps_table(wl), dtype=torch.float64, device=dev)
        self.ring = None
        # Untimed pass: draft with debug logits -> target stand-in = logits + noise; the plan of
        # this pass fixes the packed row layout (the timed rounds recompute the same plan).
        logits = torch.empty_like(self.U)
        if head == "rnn":
            tok, q, lse, _ = L.rnn_draft(d, self.U, wts["W1"], wts["W2t"], wts["Wgco"], self.h,
                                         self.anchor, self.uniforms, logits_dbg=logits, **opts)
        else:
            tok, q, lse = L.markov_draft(d, self.U, wts["W1"], wts["W2t"], self.anchor,
                                         self.uniforms, logits_dbg=logits, **opts)
        if full:
            dl, ro, st = L.plan(d, None, self.sps, wl.mode)
        else:
            conf = L.confidence(d, self.h, wts["W1"], wts["w"], self.T, self.anchor, tok)
            if wl.mode == W.LAGGED_TOPK:
                # steady state of the lag ring: the slot a timed round reads holds this set's own
                # confidences (as two rounds earlier), and the round writes the same values back
                self.ring = torch.stack([conf, conf]).contiguous()
                dl, ro, st = L.plan(d, conf, self.sps, wl.mode, ring=self.ring,
                                    round_index=LAG_ROUND)
            else:
                dl, ro, st = L.plan(d, conf, self.sps, wl.mode)
        dense = W.target_dense(logits, inp["U_bonus"], inp["noise"])
        del logits, inp
        self.target = W.pack_rows(dense, dl)
        del dense
        torch.cuda.synchronize()
        self.rows = int(ro[-1].item())
        self.draft_len = dl.clone()


class TreeInputSet:
    """Inputs of a PCTree round: base logits, anchors, uniforms, and the target stand-in for
    the tree the GPU drafts from them (rows after the anchor and after every kept node: base
    logits of the next position plus the Markov bias of the node's token, plus noise)."""

    def __init__(self, wl, wts, shape, round_index, dev):
        d = L.Dims(wl.B, wl.gamma, wl.V, wl.r, wl.d)
        inp = W.round_inputs(wl, round_index, dev, with_hidden=False, with_noise=False)
        self.anchor, self.U, self.uniforms = inp["anchor"], inp["U"], inp["uniforms"]
        tok, dep, par, _, _ = L.tree_draft(d, shape, self.U, wts["W1"], wts["W2t"], self.anchor)
        B, g, N = wl.B, wl.gamma, shape.N
        prev = torch.cat([self.anchor.long()[:, None], tok.long()], 1)
        pos = torch.cat([torch.zeros((B, 1), dtype=torch.long, device=dev), dep.long()], 1)
        W1f, W2f = wts["W1"].float(), wts["W2t"].float()
        self.target = torch.empty((B, N + 1, wl.V), dtype=torch.float32, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(7000 + round_index)
        for b in range(B):
            base = torch.where((pos[b] < g)[:, None], self.U[b, pos[b].clamp(max=g - 1)],
                               inp["U_bonus"][b][None, :])
            self.target[b] = base + W1f[prev[b]] @ W2f.T
            self.target[b] += torch.randn((N + 1, wl.V), generator=gen, device=dev) * wl.noise_std(1)
        del inp
        torch.cuda.synchronize()


def tree_bytes(wl, shape):
    """Bytes a PCTree round must move: per depth the U slice and W2 (the expanded rows of a
    request share its U row), then every tree row of the target once."""
    return wl.gamma * step_bytes(wl) + 4 * wl.B * (shape.N + 1) * wl.V


def algorithmic_bytes(wl, rows, n_res, greedy=False, head="markov"):
    """Bytes the method must move in one round (no caching credit): per draft step the U slice
    and W2; the hidden states and confidence weights; every verified target row; for rejected
    requests one more W2 pass plus their U and target rows (a greedy draft's residual needs only
    the target rows: its draft distribution is a point mass). The RNN head adds the hidden
    states and the hidden block of Wgco once, the state and embedding blocks of Wgco per step,
    and the fp32 bias vectors written by the draft and read by the verify."""
    B, V, g, r, d = wl.B, wl.V, wl.gamma, wl.r, wl.d
    draft = g * step_bytes(wl)
    if head == "rnn":
        draft += 2 * B * g * d + 2 * 3 * r * d + g * 2 * 3 * r * 2 * r + 2 * 4 * B * g * r
    conf = 0 if wl.mode == W.FULL_VERIFY else 2 * B * g * d + 2 * (d + r)
    return draft + conf + stats_bytes(wl, rows) + residual_bytes(wl, n_res, greedy)


def step_bytes(wl):
    """One draft step: the U slice of the position and W2."""
    return 4 * wl.B * wl.V + 2 * wl.r * wl.V


def stats_bytes(wl, rows):
    """Target row statistics: every verified row once."""
    return 4 * rows * wl.V


def residual_bytes(wl, n_res, greedy=False):
    """Residual pass: W2 once plus the U and target rows of each rejected request (the target
    rows only for a greedy draft, whose draft distribution is a point mass)."""
    if greedy:
        return n_res * 4 * wl.V
    return (2 * wl.r * wl.V if n_res > 0 else 0) + n_res * 8 * wl.V


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family and model numbers (a virtual
    machine may report only a generic name: family 26 is AMD's Zen 5 generation, EPYC 9005)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                info.setdefault(k, v)
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    extra = [f"family {info['cpu family']} model {info['model']}"] if "cpu family" in info else []
    if "hypervisor" in info.get("flags", "").split():
        extra.append("virtual machine")
    extra.append(f"{os.cpu_count()} logical CPUs visible")
    return f"{name} ({', '.join(extra)})"


def cpu_baseline(wl, wts, s, threads, opts, head="markov", reps=3):
    """The oracle as it stands, timed on the host: `reps` full rounds of the same workload on
    the same inputs (the median is reported); building the target stand-in is not timed."""
    import oracle
    host = lambda t: t.detach().cpu().numpy()
    bits = W.bf16_bits
    U, W1b, W2b = host(s.U), bits(wts["W1"]), bits(wts["W2t"])
    anchor, unif = host(s.anchor), host(s.uniforms)
    h = bits(s.h) if s.h is not None else None
    Wg = bits(wts["Wgco"]) if head == "rnn" else None
    sps = W.sps_table(wl)
    full = wl.mode == W.FULL_VERIFY
    target = None
    secs = []
    for rep in range(reps):
        t0 = time.perf_counter()
        if head == "rnn":
            o = oracle.rnn_draft(U, W1b, W2b, Wg, h, anchor, unif, want_logits=rep == 0,
                                 threads=threads, **opts)
        else:
            o = oracle.markov_draft(U, W1b, W2b, anchor, unif, want_logits=rep == 0,
                                    threads=threads, **opts)
        if full:
            p = oracle.plan(None, sps, wl.mode, B=wl.B, gamma=wl.gamma)
        else:
            c = oracle.confidence(h, W1b, bits(wts["w"]), W.temperatures(wl).numpy(), anchor,
                                  o["tokens"], threads=threads)
            if wl.mode == W.LAGGED_TOPK:
                ring = np.stack([c["conf"], c["conf"]])
                p = oracle.plan(c["conf"], sps, wl.mode, ring=ring, round_index=LAG_ROUND)
            else:
                p = oracle.plan(c["conf"], sps, wl.mode)
        t1 = time.perf_counter()
        if target is None:
            # target stand-in (not timed): the oracle's own logits + noise, packed by its plan
            inp = W.round_inputs(wl, 0, "cuda", with_hidden=False)
            dense = np.concatenate([o["logits"], host(inp["U_bonus"])[:, None, :]], 1)
            dense += host(inp["noise"])
            del inp
            keep = np.arange(wl.gamma + 1)[None, :] <= p["draft_len"][:, None]
            target = np.ascontiguousarray(dense[keep], dtype=np.float32)
            del dense
        t2 = time.perf_counter()
        if head == "rnn":
            oracle.rnn_verify(target, p["row_offsets"], p["draft_len"], U, W1b, W2b, Wg, h,
                              anchor, o["tokens"], o["q"], unif, threads=threads, **opts)
        else:
            oracle.verify(target, p["row_offsets"], p["draft_len"], U, W1b, W2b, anchor,
                          o["tokens"], o["q"], unif, threads=threads, **opts)
        t3 = time.perf_counter()
        secs.append((t1 - t0) + (t3 - t2))
    sec = float(np.median(secs))
    return {"value": 1.0 / sec, "unit": "rounds/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{reps} full rounds of {wl.name} (all {wl.B} requests: {head}-head draft, "
                      f"{'' if full else 'confidence, '}plan, verify; target construction "
                      f"excluded), median {sec:.2f} s a round "
                      f"({', '.join(f'{x:.2f}' for x in secs)})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=sorted(W.WORKLOADS), default=WORKLOAD,
                    help="workload of the timed rounds (default: the headline one)")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="skip the kernel-timing pass (no per-kernel durations or roofline)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprof)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no hipGraph capture of the round)")
    ap.add_argument("--temperature", type=float, default=1.0,
                    help="draft sampling temperature (the drafted distribution softmax(L / tau))")
    ap.add_argument("--head", choices=["markov", "rnn"], default="markov",
                    help="serial draft head: the Markov head (eq. 5) or the RNN head (eq. 6)")
    ap.add_argument("--separate-plan", action="store_true",
                    help="launch the confidence head and the planner as calls of their own "
                         "after the draft (by default one call runs the plan beside the last "
                         "draft step)")
    ap.add_argument("--tree", default=None, metavar="c,M,N",
                    help="PCTree round instead of the chain: c children per node, M nodes "
                         "expanded per depth, N nodes kept (e.g. 4,4,16)")
    ap.add_argument("--greedy", action="store_true",
                    help="greedy draft (first maximal logit; the verify's residual is p_t "
                         "without the drafted token)")
    args = ap.parse_args()
    if not args.greedy and not (args.temperature > 0 and np.isfinite(args.temperature)):
        print("--temperature must be positive and finite", file=sys.stderr)
        sys.exit(2)
    opts = {"temperature": args.temperature, "greedy": args.greedy}
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    dev = "cuda"
    wl = W.WORKLOADS[args.workload]
    if args.tree:
        return tree_main(args, wl, dev)
    full = wl.mode == W.FULL_VERIFY
    if args.head == "rnn" and full:
        print("the RNN head reads hidden states, which the full-verify workloads do not have",
              file=sys.stderr)
        sys.exit(2)
    d = L.Dims(wl.B, wl.gamma, wl.V, wl.r, wl.d)
    L.load_library()
    wts = W.weights(wl, dev)
    if args.head == "rnn":
        wts["Wgco"] = W.rnn_weights(wl, dev)
    sets = [InputSet(wl, wts, i, dev, opts, args.head) for i in range(args.sets)]

    # output and workspace buffers, allocated once
    B, g = wl.B, wl.gamma
    rnn = args.head == "rnn"
    ws_d = L.workspace(d, L.OP_RNN_DRAFT if rnn else L.OP_DRAFT, dev)
    ws_v = L.workspace(d, L.OP_RNN_VERIFY if rnn else L.OP_VERIFY, dev)
    e_rows = torch.empty((wl.B, wl.gamma, wl.r), dtype=torch.float32, device=dev) if rnn else None
    tok = torch.empty((B, g), dtype=torch.int32, device=dev)
    q = torch.empty((B, g), dtype=torch.float32, device=dev)
    lse = torch.empty((B, g), dtype=torch.float64, device=dev)
    conf = torch.empty((B, g), dtype=torch.float32, device=dev)
    dl = torch.empty(B, dtype=torch.int32, device=dev)
    ro = torch.empty(B + 1, dtype=torch.int32, device=dev)
    st = torch.empty(4, dtype=torch.float64, device=dev)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    nt = torch.empty(B, dtype=torch.int32, device=dev)
    be = torch.empty(B, dtype=torch.float32, device=dev)
    fl = torch.empty(B, dtype=torch.int32, device=dev)

    lag = dict(ring=None, round_index=0)

    def plan_args(s):
        return dict(ring=s.ring, round_index=LAG_ROUND) if s.ring is not None else lag

    def round_markov(s):
        if full:
            L.markov_draft(d, s.U, wts["W1"], wts["W2t"], s.anchor, s.uniforms, tokens=tok, q=q,
                           lse=lse, ws=ws_d, **opts)
            L.plan(d, None, s.sps, wl.mode, draft_len=dl, row_offsets=ro, stats=st)
        elif args.separate_plan:
            L.markov_draft(d, s.U, wts["W1"], wts["W2t"], s.anchor, s.uniforms, tokens=tok, q=q,
                           lse=lse, ws=ws_d, **opts)
            L.confidence(d, s.h, wts["W1"], wts["w"], s.T, s.anchor, tok, conf=conf)
            L.plan(d, conf, s.sps, wl.mode, draft_len=dl, row_offsets=ro, stats=st,
                   **plan_args(s))
        else:
            L.markov_draft_plan(d, s.U, wts["W1"], wts["W2t"], s.anchor, s.uniforms, s.h,
                                wts["w"], s.T, s.sps, wl.mode, tokens=tok, q=q, lse=lse,
                                conf=conf, draft_len=dl, row_offsets=ro, stats=st, ws=ws_d,
                                **plan_args(s), **opts)
        L.verify(d, s.target, ro, dl, s.U, wts["W1"], wts["W2t"], s.anchor, tok, q, lse,
                 s.uniforms, accept_len=al, next_token=nt, beta_emit=be, flags=fl, ws=ws_v,
                 **opts)

    def round_rnn(s):
        if args.separate_plan:
            L.rnn_draft(d, s.U, wts["W1"], wts["W2t"], wts["Wgco"], s.h, s.anchor, s.uniforms,
                        tokens=tok, q=q, lse=lse, e_rows=e_rows, ws=ws_d, **opts)
            L.confidence(d, s.h, wts["W1"], wts["w"], s.T, s.anchor, tok, conf=conf)
            L.plan(d, conf, s.sps, wl.mode, draft_len=dl, row_offsets=ro, stats=st,
                   **plan_args(s))
        else:
            L.rnn_draft_plan(d, s.U, wts["W1"], wts["W2t"], wts["Wgco"], s.h, s.anchor, s.uniforms,
                             wts["w"], s.T, s.sps, wl.mode, tokens=tok, q=q, lse=lse,
                             e_rows=e_rows, conf=conf, draft_len=dl, row_offsets=ro, stats=st,
                             ws=ws_d, **plan_args(s), **opts)
        L.rnn_verify(d, s.target, ro, dl, s.U, wts["W2t"], e_rows, tok, q, lse, s.uniforms,
                     accept_len=al, next_token=nt, beta_emit=be, flags=fl, ws=ws_v, **opts)

    round_ = round_rnn if args.head == "rnn" else round_markov

    # per-set results (identical every time a set is replayed: deterministic)
    per_set = []
    for s in sets:
        round_(s)
        torch.cuda.synchronize()
        assert torch.equal(dl, s.draft_len), "the timed plan differs from the preparation pass"
        n_res = int((be >= 0).sum().item())
        per_set.append(dict(tokens=int((al + 1).sum().item()), rows=s.rows, n_res=n_res,
                            out=[t.clone() for t in (tok, dl, al, nt, be)]))

    for i in range(args.warmup):
        round_(sets[i % len(sets)])
    torch.cuda.synchronize()
    # Timed region: K rounds, nothing recorded between the launches.
    t0 = time.perf_counter()
    for i in range(args.steps):
        round_(sets[i % len(sets)])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Round-time distribution: the same K rounds with an event pair at each round boundary
    # only (no events between a round's launches).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for i in range(args.steps):
        round_(sets[i % len(sets)])
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_round_us = np.array([1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    round_us = {k: round(float(np.percentile(per_round_us, q)), 2)
                for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}
    # Graph region: each input set's round captured once as a hipGraph (every launch has its
    # shapes on the device, so one capture replays any planned lengths), every replay checked
    # against the eager results, then K replays timed the same way (reported beside `value`).
    elapsed_graph = None
    if not args.no_graph:
        graphs = []
        for s in sets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                round_(s)
            graphs.append(gr)
        for rep in range(2):
            for gr, ps in zip(graphs, per_set):
                gr.replay()
                torch.cuda.synchronize()
                for a, b in zip((tok, dl, al, nt, be), ps["out"]):
                    assert torch.equal(a, b), "a graph replay differs from the eager round"
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        elapsed_graph = time.perf_counter() - t0
    # Kernel-timing region: the same K rounds again, with a HIP event pair recorded around every
    # library launch on its stream (the events add gaps between kernels, so this region does not
    # set `value`; it gives each kernel's average duration).
    kern = {}
    elapsed_ev = None
    if not args.no_kernel_events:
        L.profile_begin(64 * args.steps)
        t1 = time.perf_counter()
        for i in range(args.steps):
            round_(sets[i % len(sets)])
        torch.cuda.synchronize()
        elapsed_ev = time.perf_counter() - t1
        kern = L.profile_end()

    # `value` is the eager rate: replaying the captured round measured slower than launching it
    # (the launches already run back to back), so the graph rate is reported beside it.
    timed = elapsed
    rounds_per_s = args.steps / timed
    used = [per_set[i % len(sets)] for i in range(args.steps)]
    tokens_per_round = float(np.mean([u["tokens"] for u in used]))
    bytes_per_round = float(np.mean([algorithmic_bytes(wl, u["rows"], u["n_res"], args.greedy,
                                                       args.head) for u in used]))

    roofline = None
    mfma = None
    kernels = {}
    for name, (cnt, ms) in kern.items():
        if cnt:
            kernels[name] = {"launches": cnt, "avg_us": 1e3 * ms / cnt}
    streaming = {}
    # algorithmic bytes per launch of each streaming kernel, averaged over the timed rounds
    per_launch = {
        "markov_step": step_bytes(wl),
        "target_stats": float(np.mean([stats_bytes(wl, u["rows"]) for u in used])),
        "residual_partials": float(np.mean([residual_bytes(wl, u["n_res"], args.greedy)
                                            for u in used])),
    }
    for name, nbytes in per_launch.items():
        if name in kernels and nbytes > 0:
            gbs = nbytes / (kernels[name]["avg_us"] * 1e-6) / 1e9
            streaming[name] = {"bytes_per_launch": round(nbytes), "avg_us": round(kernels[name]["avg_us"], 3),
                               "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if "markov_step" in kernels:
        sb = step_bytes(wl)                                     # U slice + W2 per launch
        avg_s = kernels["markov_step"]["avg_us"] * 1e-6
        achieved = sb / avg_s / 1e9
        # the committed counters were taken on the Markov head's step kernel at the headline
        # workload
        traffic = (traffic_from_profiles(1) if args.head == "markov" and wl.name == WORKLOAD
                   else None)
        roofline = {"kernel": "markov_step", "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "traffic_unit": "bytes per launch",
                    "algorithmic_bytes_per_launch": sb,
                    "avg_launch_us": round(kernels["markov_step"]["avg_us"], 3),
                    "timing": "HIP events recorded with each dispatch (dspark_profile_begin/end), "
                              "averaged over the K rounds of the kernel-timing pass",
                    "worst_streaming_kernel": (min(streaming, key=lambda k: streaming[k]["frac"])
                                               if streaming else None),
                    "worst_streaming_frac": (min(v["frac"] for v in streaming.values())
                                             if streaming else None)}
        # the W2 contraction per launch; the RNN head's bias vector enters it as three bf16 terms
        terms = 3 if args.head == "rnn" else 1
        flops = 2.0 * wl.B * wl.r * wl.V * terms
        mfma = {"kernel": "markov_step", "tflops": round(flops / avg_s / 1e12, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "frac": round(flops / avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "bias_terms": terms}

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    base = None
    if not args.no_cpu_baseline:
        # every host core this process may run on, up to the 16 one GPU's job gets on the box
        threads = min(16, len(os.sched_getaffinity(0)) or 1)
        base = cpu_baseline(wl, wts, sets[0], threads, opts, args.head)

    metric = (METRIC if wl.name == WORKLOAD else
              f"spec rounds/s at B={wl.B},V={wl.V},γ={wl.gamma}; achieved HBM GB/s vs peak")
    plan_name = {W.FULL_VERIFY: "full_verify", W.EARLY_STOP: "early_stop",
                 W.FULL_PATH: "full_path", W.LAGGED_TOPK: "lagged_topk"}[wl.mode]
    sps_name = "flat" if wl.sps_kind == "flat" else f"1/(1+n/{wl.sps_scale:g})"
    out = {
        "metric": metric,
        "value": round(rounds_per_s, 2),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * timed / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 mfma / f32 / f64",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "V": wl.V, "gamma": wl.gamma, "r": wl.r,
                   "d": wl.d, "plan": plan_name, "sps": sps_name, "input_sets": len(sets),
                   "parallelism": "1 GPU", "launch": "eager",
                   "draft": ("greedy" if args.greedy
                             else f"sampled at temperature {args.temperature:g}"),
                   "head": args.head,
                   "plan_launch": ("own call (full verify: no confidence head)" if full
                                   else "own call" if args.separate_plan
                                   else "beside the last draft step")},
        "round_us": round_us,
        "graph_rounds_per_s": (round(args.steps / elapsed_graph, 2)
                               if elapsed_graph is not None else None),
        "tokens_per_s": round(rounds_per_s * tokens_per_round, 1),
        "tokens_per_round": tokens_per_round,
        "round_algorithmic_gbs": round(bytes_per_round * rounds_per_s / 1e9, 1),
        "round_hbm_frac": round(bytes_per_round * rounds_per_s / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "streaming_kernels": streaming,
        "mfma": mfma,
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kernels.items()},
        "ms_per_step_with_kernel_events": (round(1e3 * elapsed_ev / args.steps, 4)
                                           if elapsed_ev else None),
        "cpu_baseline": base,
    }
    print(json.dumps(out), flush=True)


def tree_main(args, wl, dev):
    """A PCTree round (tree draft + tree verify) timed like the chain's round."""
    import oracle
    c, M, N = (int(x) for x in args.tree.split(","))
    shape = L.TreeShape(c, M, N)
    d = L.Dims(wl.B, wl.gamma, wl.V, wl.r, wl.d)
    L.load_library()
    wts = W.weights(wl, dev)
    sets = [TreeInputSet(wl, wts, shape, i, dev) for i in range(args.sets)]
    B, g = wl.B, wl.gamma
    ws_d = torch.empty(L.tree_workspace_bytes(d, shape, L.OP_TREE_DRAFT), dtype=torch.uint8, device=dev)
    ws_v = torch.empty(L.tree_workspace_bytes(d, shape, L.OP_TREE_VERIFY), dtype=torch.uint8, device=dev)
    tok, dep, par = (torch.empty((B, N), dtype=torch.int32, device=dev) for _ in range(3))
    q, P = (torch.empty((B, N), dtype=torch.float64, device=dev) for _ in range(2))
    al, nt, fl = (torch.empty(B, dtype=torch.int32, device=dev) for _ in range(3))
    path = torch.empty((B, g), dtype=torch.int32, device=dev)

    def round_(s):
        L.tree_draft(d, shape, s.U, wts["W1"], wts["W2t"], s.anchor, node_token=tok,
                     node_depth=dep, node_parent=par, node_q=q, node_path=P, ws=ws_d)
        L.tree_verify(d, shape, s.target, tok, par, s.uniforms, accept_len=al, path=path,
                      next_token=nt, flags=fl, ws=ws_v)

    tokens = []
    for s in sets:
        round_(s)
        torch.cuda.synchronize()
        tokens.append(int((al + 1).sum().item()))
    for i in range(args.warmup):
        round_(sets[i % len(sets)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        round_(sets[i % len(sets)])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern = {}
    if not args.no_kernel_events:
        L.profile_begin(64 * args.steps)
        for i in range(args.steps):
            round_(sets[i % len(sets)])
        torch.cuda.synchronize()
        kern = {k: round(1e3 * ms / n, 2) for k, (n, ms) in L.profile_end().items() if n}
    rps = args.steps / elapsed
    tpr = float(np.mean([tokens[i % len(sets)] for i in range(args.steps)]))
    nbytes = tree_bytes(wl, shape)
    base = None
    if not args.no_cpu_baseline:
        threads = min(16, len(os.sched_getaffinity(0)) or 1)
        s = sets[0]
        host = lambda t: t.detach().cpu().numpy()
        U, anc, uni, tgt = host(s.U), host(s.anchor), host(s.uniforms), host(s.target)
        W1b, W2b = W.bf16_bits(wts["W1"]), W.bf16_bits(wts["W2t"])
        secs = []
        for _ in range(3):
            t1 = time.perf_counter()
            o = oracle.tree_draft(U, W1b, W2b, anc, c, M, N, threads=threads)
            oracle.tree_verify(tgt, o["token"], o["depth"], o["parent"], uni, threads=threads)
            secs.append(time.perf_counter() - t1)
        sec = float(np.median(secs))
        base = {"value": 1.0 / sec, "unit": "rounds/s", "cores": threads, "kind": "oracle",
                "cpu": cpu_model(),
                "sample": f"3 PCTree rounds of {wl.name} (tree draft c={c} M={M} N={N}, tree "
                          f"verify; all {B} requests), median {sec:.2f} s a round"}
    out = {
        "metric": f"PCTree rounds/s at B={B},V={wl.V},γ={g}; achieved HBM GB/s vs peak",
        "value": round(rps, 2), "unit": "rounds/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 mfma / f32 / f64", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "V": wl.V, "gamma": g, "r": wl.r,
                   "tree": {"c": c, "M": M, "N": N}, "input_sets": len(sets),
                   "parallelism": "1 GPU", "launch": "eager"},
        "tokens_per_round": tpr, "tokens_per_s": round(rps * tpr, 1),
        "round_algorithmic_gbs": round(nbytes * rps / 1e9, 1),
        "round_hbm_frac": round(nbytes * rps / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_us": kern, "cpu_baseline": base,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
