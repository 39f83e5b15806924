"""Thin ctypes binding of libdspark.so: argument marshalling only.

Every function takes torch tensors that live on the GPU, checks dtype / shape / contiguity,
and passes raw device pointers and the current HIP stream to the C ABI (include/dspark.h).
All computation happens in the library's HIP kernels; there is no CPU fallback, and a missing
library raises at the first call.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "Dims", "DsparkError", "FULL_VERIFY", "EARLY_STOP", "FULL_PATH", "LAGGED_TOPK",
    "OP_DRAFT", "OP_CONFIDENCE", "OP_PLAN", "OP_VERIFY", "OP_RNN_DRAFT", "OP_RNN_VERIFY",
    "FLAG_NONFINITE", "FLAG_ZERO_RESIDUAL", "library_path", "load_library", "workspace_bytes",
    "workspace", "markov_draft", "confidence", "plan", "markov_draft_plan", "verify",
    "rnn_draft", "rnn_verify", "rnn_draft_plan", "verify_noalloc", "NOALLOC_SCRATCH_BYTES",
    "TreeShape", "OP_TREE_DRAFT", "OP_TREE_VERIFY", "tree_workspace_bytes", "tree_draft",
    "tree_verify",
    "profile_begin", "profile_end", "version",
]

FULL_VERIFY, EARLY_STOP, FULL_PATH, LAGGED_TOPK = 0, 1, 2, 3
OP_DRAFT, OP_CONFIDENCE, OP_PLAN, OP_VERIFY, OP_RNN_DRAFT, OP_RNN_VERIFY = 0, 1, 2, 3, 4, 5
OP_TREE_DRAFT, OP_TREE_VERIFY = 6, 7
FLAG_NONFINITE, FLAG_ZERO_RESIDUAL = 1, 2
NOALLOC_SCRATCH_BYTES = 48 << 20     # DSPARK_NOALLOC_SCRATCH_BYTES

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libdspark.so")


class DsparkError(RuntimeError):
    pass


class _CDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("gamma", ctypes.c_int32), ("V", ctypes.c_int32),
                ("r", ctypes.c_int32), ("d", ctypes.c_int32)]


class _CDraftOpts(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("greedy", ctypes.c_int32)]


def _opts(temperature: float, greedy: bool):
    """Draft options for the *_opts entry points (None: temperature 1, sampling)."""
    if not greedy and float(temperature) == 1.0:
        return None
    return ctypes.byref(_CDraftOpts(float(temperature), 1 if greedy else 0))


class _CTreeShape(ctypes.Structure):
    _fields_ = [("c", ctypes.c_int32), ("M", ctypes.c_int32), ("N", ctypes.c_int32)]


@dataclass(frozen=True)
class TreeShape:
    """PCTree shape: c children expanded per node, M nodes expanded per depth, N nodes kept."""
    c: int
    M: int
    N: int

    def c_struct(self) -> _CTreeShape:
        return _CTreeShape(self.c, self.M, self.N)


@dataclass(frozen=True)
class Dims:
    B: int
    gamma: int
    V: int
    r: int
    d: int = 8

    def c(self) -> _CDims:
        return _CDims(self.B, self.gamma, self.V, self.r, self.d)


_P = ctypes.c_void_p


def load_library():
    """Load the in-tree libdspark.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise DsparkError(f"{path} is missing: build it with "
                              "`python -m lossless_draft_verify_amd.build`")
        lib = ctypes.CDLL(path)
        lib.dspark_status_string.restype = ctypes.c_char_p
        lib.dspark_status_string.argtypes = [ctypes.c_int32]
        lib.dspark_version.restype = ctypes.c_char_p
        lib.dspark_workspace_bytes.restype = ctypes.c_size_t
        lib.dspark_workspace_bytes.argtypes = [_CDims, ctypes.c_int32]
        lib.dspark_markov_draft.restype = ctypes.c_int32
        lib.dspark_markov_draft.argtypes = [_CDims] + [_P] * 10 + [_P, ctypes.c_size_t, _P]
        lib.dspark_markov_draft_opts.restype = ctypes.c_int32
        lib.dspark_markov_draft_opts.argtypes = ([_CDims] + [_P] * 10 +
                                                 [_P, ctypes.c_size_t, _P, _P])
        lib.dspark_confidence.restype = ctypes.c_int32
        lib.dspark_confidence.argtypes = [_CDims] + [_P] * 7 + [_P]
        lib.dspark_plan.restype = ctypes.c_int32
        lib.dspark_plan.argtypes = [_CDims, _P, _P, ctypes.c_int32, ctypes.c_int32, _P,
                                    ctypes.c_int32, _P, _P, _P, _P]
        lib.dspark_markov_draft_plan.restype = ctypes.c_int32
        lib.dspark_markov_draft_plan.argtypes = (
            [_CDims] + [_P] * 9 + [ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32] +
            [_P] * 7 + [_P, ctypes.c_size_t, _P, _P])
        lib.dspark_rnn_draft_plan.restype = ctypes.c_int32
        lib.dspark_rnn_draft_plan.argtypes = (
            [_CDims] + [_P] * 10 + [ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32] +
            [_P] * 8 + [_P, ctypes.c_size_t, _P, _P])
        lib.dspark_verify.restype = ctypes.c_int32
        lib.dspark_verify.argtypes = [_CDims] + [_P] * 15 + [_P, ctypes.c_size_t, _P]
        lib.dspark_verify_opts.restype = ctypes.c_int32
        lib.dspark_verify_opts.argtypes = [_CDims] + [_P] * 15 + [_P, ctypes.c_size_t, _P, _P]
        lib.dspark_verify_noalloc.restype = ctypes.c_int32
        lib.dspark_verify_noalloc.argtypes = [_CDims] + [_P] * 15 + [_P, _P]
        lib.dspark_tree_workspace_bytes.restype = ctypes.c_size_t
        lib.dspark_tree_workspace_bytes.argtypes = [_CDims, _CTreeShape, ctypes.c_int32]
        lib.dspark_tree_draft.restype = ctypes.c_int32
        lib.dspark_tree_draft.argtypes = [_CDims, _CTreeShape] + [_P] * 9 + [_P, ctypes.c_size_t, _P]
        lib.dspark_tree_verify.restype = ctypes.c_int32
        lib.dspark_tree_verify.argtypes = [_CDims, _CTreeShape] + [_P] * 8 + [_P, ctypes.c_size_t, _P]
        lib.dspark_rnn_draft.restype = ctypes.c_int32
        lib.dspark_rnn_draft.argtypes = [_CDims] + [_P] * 13 + [_P, ctypes.c_size_t, _P, _P]
        lib.dspark_rnn_verify.restype = ctypes.c_int32
        lib.dspark_rnn_verify.argtypes = [_CDims] + [_P] * 14 + [_P, ctypes.c_size_t, _P, _P]
        lib.dspark_profile_begin.restype = ctypes.c_int32
        lib.dspark_profile_begin.argtypes = [ctypes.c_int32]
        lib.dspark_profile_end.restype = ctypes.c_int32
        lib.dspark_profile_end.argtypes = [ctypes.POINTER(ctypes.c_char_p),
                                           ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_double), ctypes.c_int32]
        _LIB = lib
    return _LIB


def version() -> str:
    return load_library().dspark_version().decode()


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().dspark_status_string(status).decode()
        raise DsparkError(f"{what}: {msg} (status {status})")


def _ptr(t: Optional[torch.Tensor], dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise DsparkError(f"{name} must live on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(dims: Dims, op: int) -> int:
    n = load_library().dspark_workspace_bytes(dims.c(), op)
    if n == ctypes.c_size_t(-1).value:
        raise DsparkError(f"unsupported dims {dims} for op {op}")
    return int(n)


def workspace(dims: Dims, op: int, device="cuda") -> torch.Tensor:
    """A workspace tensor of the size an operation needs (uint8, 256-byte aligned)."""
    return torch.empty(max(1, workspace_bytes(dims, op)), dtype=torch.uint8, device=device)


def markov_draft(dims: Dims, U, W1, W2t, anchor, uniforms, *, tokens=None, q=None, lse=None,
                 logits_dbg=None, force_tokens=None, ws=None, temperature: float = 1.0,
                 greedy: bool = False, stream=None):
    """Markov-head draft (dspark_markov_draft_opts): sampled at `temperature`, or greedy.
    Returns (tokens, q, lse)."""
    B, g, V, r = dims.B, dims.gamma, dims.V, dims.r
    dev = U.device
    tokens = tokens if tokens is not None else torch.empty((B, g), dtype=torch.int32, device=dev)
    q = q if q is not None else torch.empty((B, g), dtype=torch.float32, device=dev)
    lse = lse if lse is not None else torch.empty((B, g), dtype=torch.float64, device=dev)
    ws = ws if ws is not None else workspace(dims, OP_DRAFT, dev)
    st = load_library().dspark_markov_draft_opts(
        dims.c(), _ptr(U, torch.float32, (B, g, V), "U"), _ptr(W1, torch.bfloat16, (V, r), "W1"),
        _ptr(W2t, torch.bfloat16, (V, r), "W2t"), _ptr(anchor, torch.int32, (B,), "anchor"),
        _ptr(uniforms, torch.float32, (B, g + 1, 3), "uniforms"),
        _ptr(tokens, torch.int32, (B, g), "tokens"), _ptr(q, torch.float32, (B, g), "q"),
        _ptr(lse, torch.float64, (B, g), "lse"),
        _ptr(logits_dbg, torch.float32, (B, g, V), "logits_dbg"),
        _ptr(force_tokens, torch.int32, (B, g), "force_tokens"), _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), _opts(temperature, greedy), _stream(stream))
    _check(st, "dspark_markov_draft_opts")
    return tokens, q, lse


def confidence(dims: Dims, h, W1, w, T, anchor, tokens, *, conf=None, stream=None):
    """Confidence head (dspark_confidence). Returns conf [B][gamma] fp32."""
    B, g, V, r, d = dims.B, dims.gamma, dims.V, dims.r, dims.d
    conf = conf if conf is not None else torch.empty((B, g), dtype=torch.float32, device=h.device)
    st = load_library().dspark_confidence(
        dims.c(), _ptr(h, torch.bfloat16, (B, g, d), "h"), _ptr(W1, torch.bfloat16, (V, r), "W1"),
        _ptr(w, torch.bfloat16, (d + r,), "w"), _ptr(T, torch.float32, (g,), "T"),
        _ptr(anchor, torch.int32, (B,), "anchor"), _ptr(tokens, torch.int32, (B, g), "tokens"),
        _ptr(conf, torch.float32, (B, g), "conf"), _stream(stream))
    _check(st, "dspark_confidence")
    return conf


def plan(dims: Dims, conf, sps, mode: int, *, ring=None, round_index: int = 0, draft_len=None,
         row_offsets=None, stats=None, stream=None):
    """Verify planner (dspark_plan). Returns (draft_len, row_offsets, stats)."""
    B, g = dims.B, dims.gamma
    dev = sps.device
    draft_len = draft_len if draft_len is not None else torch.empty(B, dtype=torch.int32, device=dev)
    row_offsets = (row_offsets if row_offsets is not None
                   else torch.empty(B + 1, dtype=torch.int32, device=dev))
    stats = stats if stats is not None else torch.empty(4, dtype=torch.float64, device=dev)
    st = load_library().dspark_plan(
        dims.c(), _ptr(conf, torch.float32, (B, g), "conf"), _ptr(sps, torch.float64, None, "sps"),
        int(sps.numel()), int(mode), _ptr(ring, torch.float32, (2, B, g), "ring"),
        int(round_index), _ptr(draft_len, torch.int32, (B,), "draft_len"),
        _ptr(row_offsets, torch.int32, (B + 1,), "row_offsets"),
        _ptr(stats, torch.float64, (4,), "stats"), _stream(stream))
    _check(st, "dspark_plan")
    return draft_len, row_offsets, stats


def markov_draft_plan(dims: Dims, U, W1, W2t, anchor, uniforms, h, w, T, sps, mode: int, *,
                      ring=None, round_index: int = 0, tokens=None, q=None, lse=None, conf=None,
                      draft_len=None, row_offsets=None, stats=None, ws=None,
                      temperature: float = 1.0, greedy: bool = False, stream=None):
    """Draft, confidence head and plan of a round in one call (dspark_markov_draft_plan).
    Returns (tokens, q, lse, conf, draft_len, row_offsets, stats)."""
    B, g, V, r, d = dims.B, dims.gamma, dims.V, dims.r, dims.d
    dev = U.device
    tokens = tokens if tokens is not None else torch.empty((B, g), dtype=torch.int32, device=dev)
    q = q if q is not None else torch.empty((B, g), dtype=torch.float32, device=dev)
    lse = lse if lse is not None else torch.empty((B, g), dtype=torch.float64, device=dev)
    conf = conf if conf is not None else torch.empty((B, g), dtype=torch.float32, device=dev)
    draft_len = draft_len if draft_len is not None else torch.empty(B, dtype=torch.int32, device=dev)
    row_offsets = (row_offsets if row_offsets is not None
                   else torch.empty(B + 1, dtype=torch.int32, device=dev))
    stats = stats if stats is not None else torch.empty(4, dtype=torch.float64, device=dev)
    ws = ws if ws is not None else workspace(dims, OP_DRAFT, dev)
    st = load_library().dspark_markov_draft_plan(
        dims.c(), _ptr(U, torch.float32, (B, g, V), "U"), _ptr(W1, torch.bfloat16, (V, r), "W1"),
        _ptr(W2t, torch.bfloat16, (V, r), "W2t"), _ptr(anchor, torch.int32, (B,), "anchor"),
        _ptr(uniforms, torch.float32, (B, g + 1, 3), "uniforms"),
        _ptr(h, torch.bfloat16, (B, g, d), "h"), _ptr(w, torch.bfloat16, (d + r,), "w"),
        _ptr(T, torch.float32, (g,), "T"), _ptr(sps, torch.float64, None, "sps"),
        int(sps.numel()), int(mode), _ptr(ring, torch.float32, (2, B, g), "ring"),
        int(round_index), _ptr(tokens, torch.int32, (B, g), "tokens"),
        _ptr(q, torch.float32, (B, g), "q"), _ptr(lse, torch.float64, (B, g), "lse"),
        _ptr(conf, torch.float32, (B, g), "conf"),
        _ptr(draft_len, torch.int32, (B,), "draft_len"),
        _ptr(row_offsets, torch.int32, (B + 1,), "row_offsets"),
        _ptr(stats, torch.float64, (4,), "stats"), _ptr(ws, torch.uint8, None, "ws"), ws.numel(),
        _opts(temperature, greedy), _stream(stream))
    _check(st, "dspark_markov_draft_plan")
    return tokens, q, lse, conf, draft_len, row_offsets, stats


def verify(dims: Dims, target, row_offsets, draft_len, U, W1, W2t, anchor, tokens, q, lse,
           uniforms, *, accept_len=None, next_token=None, beta_emit=None, flags=None, ws=None,
           temperature: float = 1.0, greedy: bool = False, stream=None):
    """Lossless verify (dspark_verify_opts) of a draft made at `temperature` (or greedy).
    `target` holds at least row_offsets[B] rows of V logits.
    Returns (accept_len, next_token, beta_emit, flags)."""
    B, g, V, r = dims.B, dims.gamma, dims.V, dims.r
    dev = U.device
    if target.dim() != 2 or target.shape[1] != V:
        raise ValueError("target must be [rows][V]")
    accept_len = accept_len if accept_len is not None else torch.empty(B, dtype=torch.int32, device=dev)
    next_token = next_token if next_token is not None else torch.empty(B, dtype=torch.int32, device=dev)
    beta_emit = beta_emit if beta_emit is not None else torch.empty(B, dtype=torch.float32, device=dev)
    flags = flags if flags is not None else torch.empty(B, dtype=torch.int32, device=dev)
    ws = ws if ws is not None else workspace(dims, OP_VERIFY, dev)
    st = load_library().dspark_verify_opts(
        dims.c(), _ptr(target, torch.float32, None, "target"),
        _ptr(row_offsets, torch.int32, (B + 1,), "row_offsets"),
        _ptr(draft_len, torch.int32, (B,), "draft_len"), _ptr(U, torch.float32, (B, g, V), "U"),
        _ptr(W1, torch.bfloat16, (V, r), "W1"), _ptr(W2t, torch.bfloat16, (V, r), "W2t"),
        _ptr(anchor, torch.int32, (B,), "anchor"), _ptr(tokens, torch.int32, (B, g), "tokens"),
        _ptr(q, torch.float32, (B, g), "q"), _ptr(lse, torch.float64, (B, g), "lse"),
        _ptr(uniforms, torch.float32, (B, g + 1, 3), "uniforms"),
        _ptr(accept_len, torch.int32, (B,), "accept_len"),
        _ptr(next_token, torch.int32, (B,), "next_token"),
        _ptr(beta_emit, torch.float32, (B,), "beta_emit"), _ptr(flags, torch.int32, (B,), "flags"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _opts(temperature, greedy), _stream(stream))
    _check(st, "dspark_verify_opts")
    return accept_len, next_token, beta_emit, flags


def verify_noalloc(dims: Dims, target, row_offsets, draft_len, U, W1, W2t, anchor, tokens, q,
                   lse, uniforms, *, accept_len, next_token, beta_emit=None, flags=None,
                   temperature: float = 1.0, greedy: bool = False, stream=None):
    """The verify on the library's own scratch array (dspark_verify_noalloc): no workspace, and
    every output is the caller's (nothing is allocated here either). Returns (accept_len,
    next_token, beta_emit, flags)."""
    B, g, V, r = dims.B, dims.gamma, dims.V, dims.r
    if target.dim() != 2 or target.shape[1] != V:
        raise ValueError("target must be [rows][V]")
    st = load_library().dspark_verify_noalloc(
        dims.c(), _ptr(target, torch.float32, None, "target"),
        _ptr(row_offsets, torch.int32, (B + 1,), "row_offsets"),
        _ptr(draft_len, torch.int32, (B,), "draft_len"), _ptr(U, torch.float32, (B, g, V), "U"),
        _ptr(W1, torch.bfloat16, (V, r), "W1"), _ptr(W2t, torch.bfloat16, (V, r), "W2t"),
        _ptr(anchor, torch.int32, (B,), "anchor"), _ptr(tokens, torch.int32, (B, g), "tokens"),
        _ptr(q, torch.float32, (B, g), "q"), _ptr(lse, torch.float64, (B, g), "lse"),
        _ptr(uniforms, torch.float32, (B, g + 1, 3), "uniforms"),
        _ptr(accept_len, torch.int32, (B,), "accept_len"),
        _ptr(next_token, torch.int32, (B,), "next_token"),
        _ptr(beta_emit, torch.float32, (B,), "beta_emit"), _ptr(flags, torch.int32, (B,), "flags"),
        _opts(temperature, greedy), _stream(stream))
    _check(st, "dspark_verify_noalloc")
    return accept_len, next_token, beta_emit, flags


def profile_begin(capacity: int = 4096):
    if load_library().dspark_profile_begin(int(capacity)) != 0:
        raise DsparkError("dspark_profile_begin failed")


def profile_end():
    """Returns {kernel name: (launches, total milliseconds)}."""
    n = 16
    names = (ctypes.c_char_p * n)()
    counts = (ctypes.c_int32 * n)()
    ms = (ctypes.c_double * n)()
    k = load_library().dspark_profile_end(names, counts, ms, n)
    if k < 0:
        raise DsparkError("dspark_profile_end failed")
    return {names[i].decode(): (counts[i], ms[i]) for i in range(k)}


def rnn_draft(dims: Dims, U, W1, W2t, Wgco, h, anchor, uniforms, *, tokens=None, q=None, lse=None,
              e_rows=None, logits_dbg=None, force_tokens=None, ws=None, temperature: float = 1.0,
              greedy: bool = False, stream=None):
    """Draft with the RNN head (dspark_rnn_draft). Wgco [3r][2r+d] bf16 (rows W_g, W_c, W_o),
    h [B][gamma][d] bf16. Returns (tokens, q, lse, e_rows) with e_rows [B][gamma][r] fp32."""
    B, g, V, r, d = dims.B, dims.gamma, dims.V, dims.r, dims.d
    dev = U.device
    tokens = tokens if tokens is not None else torch.empty((B, g), dtype=torch.int32, device=dev)
    q = q if q is not None else torch.empty((B, g), dtype=torch.float32, device=dev)
    lse = lse if lse is not None else torch.empty((B, g), dtype=torch.float64, device=dev)
    e_rows = e_rows if e_rows is not None else torch.empty((B, g, r), dtype=torch.float32, device=dev)
    ws = ws if ws is not None else workspace(dims, OP_RNN_DRAFT, dev)
    st = load_library().dspark_rnn_draft(
        dims.c(), _ptr(U, torch.float32, (B, g, V), "U"), _ptr(W1, torch.bfloat16, (V, r), "W1"),
        _ptr(W2t, torch.bfloat16, (V, r), "W2t"),
        _ptr(Wgco, torch.bfloat16, (3 * r, 2 * r + d), "Wgco"),
        _ptr(h, torch.bfloat16, (B, g, d), "h"), _ptr(anchor, torch.int32, (B,), "anchor"),
        _ptr(uniforms, torch.float32, (B, g + 1, 3), "uniforms"),
        _ptr(tokens, torch.int32, (B, g), "tokens"), _ptr(q, torch.float32, (B, g), "q"),
        _ptr(lse, torch.float64, (B, g), "lse"), _ptr(e_rows, torch.float32, (B, g, r), "e_rows"),
        _ptr(logits_dbg, torch.float32, (B, g, V), "logits_dbg"),
        _ptr(force_tokens, torch.int32, (B, g), "force_tokens"), _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), _opts(temperature, greedy), _stream(stream))
    _check(st, "dspark_rnn_draft")
    return tokens, q, lse, e_rows


def rnn_verify(dims: Dims, target, row_offsets, draft_len, U, W2t, e_rows, tokens, q, lse,
               uniforms, *, accept_len=None, next_token=None, beta_emit=None, flags=None, ws=None,
               temperature: float = 1.0, greedy: bool = False, stream=None):
    """Lossless verify of an RNN-head draft (dspark_rnn_verify): the draft distribution of a
    rejected position comes from its bias vector e_rows[b][j]. Returns (accept_len, next_token,
    beta_emit, flags)."""
    B, g, V, r = dims.B, dims.gamma, dims.V, dims.r
    dev = U.device
    if target.dim() != 2 or target.shape[1] != V:
        raise ValueError("target must be [rows][V]")
    accept_len = accept_len if accept_len is not None else torch.empty(B, dtype=torch.int32, device=dev)
    next_token = next_token if next_token is not None else torch.empty(B, dtype=torch.int32, device=dev)
    beta_emit = beta_emit if beta_emit is not None else torch.empty(B, dtype=torch.float32, device=dev)
    flags = flags if flags is not None else torch.empty(B, dtype=torch.int32, device=dev)
    ws = ws if ws is not None else workspace(dims, OP_RNN_VERIFY, dev)
    st = load_library().dspark_rnn_verify(
        dims.c(), _ptr(target, torch.float32, None, "target"),
        _ptr(row_offsets, torch.int32, (B + 1,), "row_offsets"),
        _ptr(draft_len, torch.int32, (B,), "draft_len"), _ptr(U, torch.float32, (B, g, V), "U"),
        _ptr(W2t, torch.bfloat16, (V, r), "W2t"), _ptr(e_rows, torch.float32, (B, g, r), "e_rows"),
        _ptr(tokens, torch.int32, (B, g), "tokens"), _ptr(q, torch.float32, (B, g), "q"),
        _ptr(lse, torch.float64, (B, g), "lse"),
        _ptr(uniforms, torch.float32, (B, g + 1, 3), "uniforms"),
        _ptr(accept_len, torch.int32, (B,), "accept_len"),
        _ptr(next_token, torch.int32, (B,), "next_token"),
        _ptr(beta_emit, torch.float32, (B,), "beta_emit"), _ptr(flags, torch.int32, (B,), "flags"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _opts(temperature, greedy), _stream(stream))
    _check(st, "dspark_rnn_verify")
    return accept_len, next_token, beta_emit, flags


def rnn_draft_plan(dims: Dims, U, W1, W2t, Wgco, h, anchor, uniforms, w, T, sps, mode: int, *,
                   ring=None, round_index: int = 0, tokens=None, q=None, lse=None, e_rows=None,
                   conf=None, draft_len=None, row_offsets=None, stats=None, ws=None,
                   temperature: float = 1.0, greedy: bool = False, stream=None):
    """RNN-head draft, confidence head and plan of a round in one call (dspark_rnn_draft_plan).
    Returns (tokens, q, lse, e_rows, conf, draft_len, row_offsets, stats)."""
    B, g, V, r, d = dims.B, dims.gamma, dims.V, dims.r, dims.d
    dev = U.device
    tokens = tokens if tokens is not None else torch.empty((B, g), dtype=torch.int32, device=dev)
    q = q if q is not None else torch.empty((B, g), dtype=torch.float32, device=dev)
    lse = lse if lse is not None else torch.empty((B, g), dtype=torch.float64, device=dev)
    e_rows = e_rows if e_rows is not None else torch.empty((B, g, r), dtype=torch.float32, device=dev)
    conf = conf if conf is not None else torch.empty((B, g), dtype=torch.float32, device=dev)
    draft_len = draft_len if draft_len is not None else torch.empty(B, dtype=torch.int32, device=dev)
    row_offsets = (row_offsets if row_offsets is not None
                   else torch.empty(B + 1, dtype=torch.int32, device=dev))
    stats = stats if stats is not None else torch.empty(4, dtype=torch.float64, device=dev)
    ws = ws if ws is not None else workspace(dims, OP_RNN_DRAFT, dev)
    st = load_library().dspark_rnn_draft_plan(
        dims.c(), _ptr(U, torch.float32, (B, g, V), "U"), _ptr(W1, torch.bfloat16, (V, r), "W1"),
        _ptr(W2t, torch.bfloat16, (V, r), "W2t"),
        _ptr(Wgco, torch.bfloat16, (3 * r, 2 * r + d), "Wgco"),
        _ptr(h, torch.bfloat16, (B, g, d), "h"), _ptr(anchor, torch.int32, (B,), "anchor"),
        _ptr(uniforms, torch.float32, (B, g + 1, 3), "uniforms"),
        _ptr(w, torch.bfloat16, (d + r,), "w"), _ptr(T, torch.float32, (g,), "T"),
        _ptr(sps, torch.float64, None, "sps"), int(sps.numel()), int(mode),
        _ptr(ring, torch.float32, (2, B, g), "ring"), int(round_index),
        _ptr(tokens, torch.int32, (B, g), "tokens"), _ptr(q, torch.float32, (B, g), "q"),
        _ptr(lse, torch.float64, (B, g), "lse"), _ptr(e_rows, torch.float32, (B, g, r), "e_rows"),
        _ptr(conf, torch.float32, (B, g), "conf"),
        _ptr(draft_len, torch.int32, (B,), "draft_len"),
        _ptr(row_offsets, torch.int32, (B + 1,), "row_offsets"),
        _ptr(stats, torch.float64, (4,), "stats"), _ptr(ws, torch.uint8, None, "ws"), ws.numel(),
        _opts(temperature, greedy), _stream(stream))
    _check(st, "dspark_rnn_draft_plan")
    return tokens, q, lse, e_rows, conf, draft_len, row_offsets, stats


def tree_workspace_bytes(dims: Dims, shape: TreeShape, op: int) -> int:
    n = load_library().dspark_tree_workspace_bytes(dims.c(), shape.c_struct(), op)
    if n == ctypes.c_size_t(-1).value:
        raise DsparkError(f"unsupported tree shape {shape} for dims {dims}")
    return int(n)


def tree_draft(dims: Dims, shape: TreeShape, U, W1, W2t, anchor, *, node_token=None,
               node_depth=None, node_parent=None, node_q=None, node_path=None, ws=None,
               stream=None):
    """PCTree draft (dspark_tree_draft). Returns (node_token, node_depth, node_parent, node_q,
    node_path), each [B][N], nodes in rank order."""
    B, g, V, r, N = dims.B, dims.gamma, dims.V, dims.r, shape.N
    dev = U.device
    i32 = lambda t: t if t is not None else torch.empty((B, N), dtype=torch.int32, device=dev)
    f64 = lambda t: t if t is not None else torch.empty((B, N), dtype=torch.float64, device=dev)
    node_token, node_depth, node_parent = i32(node_token), i32(node_depth), i32(node_parent)
    node_q, node_path = f64(node_q), f64(node_path)
    if ws is None:
        ws = torch.empty(tree_workspace_bytes(dims, shape, OP_TREE_DRAFT), dtype=torch.uint8,
                         device=dev)
    st = load_library().dspark_tree_draft(
        dims.c(), shape.c_struct(), _ptr(U, torch.float32, (B, g, V), "U"),
        _ptr(W1, torch.bfloat16, (V, r), "W1"), _ptr(W2t, torch.bfloat16, (V, r), "W2t"),
        _ptr(anchor, torch.int32, (B,), "anchor"),
        _ptr(node_token, torch.int32, (B, N), "node_token"),
        _ptr(node_depth, torch.int32, (B, N), "node_depth"),
        _ptr(node_parent, torch.int32, (B, N), "node_parent"),
        _ptr(node_q, torch.float64, (B, N), "node_q"),
        _ptr(node_path, torch.float64, (B, N), "node_path"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "dspark_tree_draft")
    return node_token, node_depth, node_parent, node_q, node_path


def tree_verify(dims: Dims, shape: TreeShape, target, node_token, node_parent, uniforms, *,
                accept_len=None, path=None, next_token=None, flags=None, ws=None, stream=None):
    """Lossless verify of a draft tree (dspark_tree_verify). target [B][N+1][V].
    Returns (accept_len, path, next_token, flags)."""
    B, g, V, N = dims.B, dims.gamma, dims.V, shape.N
    dev = target.device
    accept_len = accept_len if accept_len is not None else torch.empty(B, dtype=torch.int32, device=dev)
    path = path if path is not None else torch.empty((B, g), dtype=torch.int32, device=dev)
    next_token = next_token if next_token is not None else torch.empty(B, dtype=torch.int32, device=dev)
    flags = flags if flags is not None else torch.empty(B, dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(tree_workspace_bytes(dims, shape, OP_TREE_VERIFY), dtype=torch.uint8,
                         device=dev)
    st = load_library().dspark_tree_verify(
        dims.c(), shape.c_struct(), _ptr(target, torch.float32, (B, N + 1, V), "target"),
        _ptr(node_token, torch.int32, (B, N), "node_token"),
        _ptr(node_parent, torch.int32, (B, N), "node_parent"),
        _ptr(uniforms, torch.float32, (B, g + 1, 3), "uniforms"),
        _ptr(accept_len, torch.int32, (B,), "accept_len"), _ptr(path, torch.int32, (B, g), "path"),
        _ptr(next_token, torch.int32, (B,), "next_token"), _ptr(flags, torch.int32, (B,), "flags"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "dspark_tree_verify")
    return accept_len, path, next_token, flags
