"""Seeded synthetic inputs for the DSpark draft-and-verify round.

This module only draws random numbers and lays them out: it holds none of the method's
arithmetic (no softmax, sampling, survival products, planning or verify), so the GPU library
and the CPU oracle can both be fed from it without sharing any of the computation they are
compared on.

The drafter backbone and the target model are out of scope; their outputs are stood in for by
generated tensors with the shapes and distributions of the workloads below:
  - base logits U ~ N(0, s_U) per position (some rows with two raised tokens),
  - Markov tables W1, W2 ~ N(0, s_W) rounded to bf16 (W2 stored token-major, [V][r]),
  - hidden states h ~ N(0, 1) bf16, confidence weights w ~ N(0, 1/sqrt(d + r)) bf16,
  - per-position STS temperatures T_k = linspace(0.8, 1.5, gamma),
  - uniforms k * 2^-24 in [0, 1),
  - target logits = (draft logits of the drafted prefix) + N(0, s_t) noise; the caller adds the
    noise drawn here to draft logits it obtained itself (the bonus position gamma+1, which has no
    draft logits, uses freshly drawn base logits instead),
  - SPS tables: flat, or SPS(n) = 1 / (1 + n / scale).
N(0, s) means standard deviation s. Every tensor comes from its own torch.Generator seeded by
(workload id, round index, tensor id) through numpy's SeedSequence.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, Optional

import numpy as np
import torch

# tensor ids for seeding
_T_ANCHOR, _T_U, _T_PEAKS, _T_W1, _T_W2, _T_H, _T_W, _T_UNIF, _T_NOISE, _T_UBONUS, _T_WGCO = range(11)
_WEIGHTS_ROUND = 1 << 20

FULL_VERIFY, EARLY_STOP, FULL_PATH, LAGGED_TOPK = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int
    B: int
    gamma: int
    V: int
    r: int
    d: int
    u_std: float
    w_std: float
    peak_frac: float          # fraction of (request, position) rows with two raised tokens
    peak_height: float
    noise_std: Callable[[int], float]  # position k = 1..gamma+1 -> target noise std
    sps_kind: str             # "flat" | "hyperbolic"
    sps_scale: float
    mode: int
    rounds: int = 1

    @property
    def sps_len(self) -> int:
        return self.B * (self.gamma + 1) + 1


def _const(s):
    return lambda k: s


WORKLOADS: Dict[str, Workload] = {
    # Tiny case the oracle finishes instantly; V = 1000 leaves a ragged tail at every tile size.
    "tiny-b4-v1000-g3": Workload("tiny-b4-v1000-g3", 1, B=4, gamma=3, V=1000, r=16, d=64,
                                 u_std=2.0, w_std=0.1, peak_frac=0.0, peak_height=0.0,
                                 noise_std=_const(0.5), sps_kind="flat", sps_scale=0.0,
                                 mode=EARLY_STOP),
    # Small batch, W2-dominated; 5 % of rows two-peaked; full verify.
    "b32-v32000-g7": Workload("b32-v32000-g7", 2, B=32, gamma=7, V=32000, r=256, d=64,
                              u_std=3.0, w_std=0.05, peak_frac=0.05, peak_height=8.0,
                              noise_std=_const(0.7), sps_kind="flat", sps_scale=0.0,
                              mode=FULL_VERIFY),
    # Production-drafter shape (the headline workload).
    "b128-v129280-g5": Workload("b128-v129280-g5", 3, B=128, gamma=5, V=129280, r=256, d=5120,
                                u_std=3.0, w_std=0.05, peak_frac=0.0, peak_height=0.0,
                                noise_std=_const(0.6), sps_kind="hyperbolic", sps_scale=768.0,
                                mode=EARLY_STOP),
    # Long block with decaying acceptance: noise std 0.3 + 0.05 k at position k.
    "b128-v151936-g15": Workload("b128-v151936-g15", 4, B=128, gamma=15, V=151936, r=256, d=64,
                                 u_std=3.0, w_std=0.05, peak_frac=0.0, peak_height=0.0,
                                 noise_std=lambda k: 0.3 + 0.05 * k, sps_kind="flat",
                                 sps_scale=0.0, mode=FULL_VERIFY),
    # High load: steep SPS, lagged planner over 20 chained rounds.
    "b512-v129280-g5-lagged": Workload("b512-v129280-g5-lagged", 5, B=512, gamma=5, V=129280,
                                       r=256, d=5120, u_std=3.0, w_std=0.05, peak_frac=0.0,
                                       peak_height=0.0, noise_std=_const(0.6),
                                       sps_kind="hyperbolic", sps_scale=512.0, mode=LAGGED_TOPK,
                                       rounds=20),
}


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of a workload with some sizes changed (same distributions)."""
    return dataclasses.replace(wl, **changes)


def _gen(wl: Workload, round_index: int, tensor_id: int, device) -> torch.Generator:
    seed = np.random.SeedSequence([wl.seed_id, round_index, tensor_id]).generate_state(1, np.uint64)[0]
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & ((1 << 63) - 1))
    return g


def _normal(shape, std, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def weights(wl: Workload, device="cpu") -> Dict[str, torch.Tensor]:
    """W1 [V][r], W2t [V][r] (token-major W2), w [d+r], all bf16."""
    R = _WEIGHTS_ROUND
    W1 = _normal((wl.V, wl.r), wl.w_std, _gen(wl, R, _T_W1, device), device).to(torch.bfloat16)
    W2t = _normal((wl.V, wl.r), wl.w_std, _gen(wl, R, _T_W2, device), device).to(torch.bfloat16)
    w = _normal((wl.d + wl.r,), 1.0 / np.sqrt(wl.d + wl.r), _gen(wl, R, _T_W, device),
                device).to(torch.bfloat16)
    return dict(W1=W1, W2t=W2t, w=w)


def rnn_weights(wl: Workload, device="cpu") -> torch.Tensor:
    """RNN-head weights Wgco [3r][2r+d] bf16: rows W_g, W_c, W_o; columns in the order of
    z = [state; embedding; hidden]. Each column block is scaled so that it adds unit variance to
    a pre-activation: state block N(0, 1/sqrt(r)), embedding block N(0, 1/(w_std sqrt(r))),
    hidden block N(0, 1/sqrt(d))."""
    r, d = wl.r, wl.d
    W = _normal((3 * r, 2 * r + d), 1.0, _gen(wl, _WEIGHTS_ROUND, _T_WGCO, device), device)
    scale = torch.cat([torch.full((r,), 1.0 / np.sqrt(r)),
                       torch.full((r,), 1.0 / (wl.w_std * np.sqrt(r))),
                       torch.full((d,), 1.0 / np.sqrt(d))]).to(device)
    return (W * scale[None, :]).to(torch.bfloat16)


def sps_table(wl: Workload) -> np.ndarray:
    n = np.arange(wl.sps_len, dtype=np.float64)
    if wl.sps_kind == "flat":
        return np.ones(wl.sps_len, np.float64)
    return 1.0 / (1.0 + n / wl.sps_scale)


def temperatures(wl: Workload) -> torch.Tensor:
    return torch.linspace(0.8, 1.5, wl.gamma, dtype=torch.float32)


def round_inputs(wl: Workload, round_index: int = 0, device="cpu",
                 with_hidden: Optional[bool] = None, with_noise: bool = True) -> Dict[str, torch.Tensor]:
    """Per-round tensors: anchor [B], U [B][g][V], U_bonus [B][V], uniforms [B][g+1][3],
    noise [B][g+1][V] (target noise, std per position), and h [B][g][d] when with_hidden."""
    B, g, V = wl.B, wl.gamma, wl.V
    anchor = torch.randint(0, V, (B,), generator=_gen(wl, round_index, _T_ANCHOR, device),
                           device=device, dtype=torch.int64).to(torch.int32)
    U = _normal((B, g, V), wl.u_std, _gen(wl, round_index, _T_U, device), device)
    n_peak = int(round(wl.peak_frac * B * g))
    if n_peak > 0:
        gp = _gen(wl, round_index, _T_PEAKS, device)
        rows = torch.randperm(B * g, generator=gp, device=device)[:n_peak]
        Uf = U.view(B * g, V)
        for row in rows.tolist():
            toks = torch.randperm(V, generator=gp, device=device)[:2]
            Uf[row, toks] += wl.peak_height
    U_bonus = _normal((B, V), wl.u_std, _gen(wl, round_index, _T_UBONUS, device), device)
    kk = torch.randint(0, 1 << 24, (B, g + 1, 3), generator=_gen(wl, round_index, _T_UNIF, device),
                       device=device, dtype=torch.int64)
    uniforms = kk.to(torch.float32) * (2.0 ** -24)
    out = dict(anchor=anchor, U=U, U_bonus=U_bonus, uniforms=uniforms)
    if with_noise:
        std = torch.tensor([wl.noise_std(k) for k in range(1, g + 2)], dtype=torch.float32,
                           device=device).view(1, g + 1, 1)
        out["noise"] = torch.randn((B, g + 1, V), generator=_gen(wl, round_index, _T_NOISE, device),
                                   device=device, dtype=torch.float32) * std
    if with_hidden is None:
        with_hidden = wl.mode != FULL_VERIFY
    if with_hidden:
        out["h"] = _normal((B, g, wl.d), 1.0, _gen(wl, round_index, _T_H, device),
                           device).to(torch.bfloat16)
    return out


def target_dense(draft_logits: torch.Tensor, U_bonus: torch.Tensor,
                 noise: torch.Tensor) -> torch.Tensor:
    """Stand-in for the target model's logits over positions 1..gamma+1: the draft logits of the
    drafted prefix (positions 1..gamma) or fresh base logits (position gamma+1), plus noise."""
    B, g, V = draft_logits.shape
    dense = torch.empty((B, g + 1, V), dtype=torch.float32, device=draft_logits.device)
    dense[:, :g] = draft_logits
    dense[:, g] = U_bonus
    dense += noise
    return dense


def pack_rows(dense: torch.Tensor, draft_len) -> torch.Tensor:
    """Packed verify rows: for each request b, rows 0..draft_len[b] of dense[b], concatenated."""
    dl = torch.as_tensor(draft_len, device=dense.device).to(torch.int64)
    g1 = dense.shape[1]
    keep = torch.arange(g1, device=dense.device).view(1, g1) <= dl.view(-1, 1)
    return dense[keep].contiguous()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor, as numpy (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
