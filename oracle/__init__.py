"""Plain fp64 CPU oracle of the DSpark draft-and-verify round (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. The GPU library (``lossless_draft_verify_amd``) never imports, links or calls it,
and the two share no code: the arithmetic lives in ``dspark_oracle.cpp`` (plain C++17, g++),
this module only marshals numpy arrays into it.

Sources cited in the C++ file: [V41] blog.javazero.top "DeepSeek-V4.1 模型结构（6）：解码，DSpark";
[ZDS] zdszero.github.io spec_dspark; [AIL] ailearn.mscapital.top "DSpark：不让大模型更聪明，而让它
「吐字更快」"; [CSDN] deepseek.csdn.net DSpark walk-through.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dspark_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FULL_VERIFY, EARLY_STOP, FULL_PATH, LAGGED_TOPK = 0, 1, 2, 3
FLAG_NONFINITE, FLAG_ZERO_RESIDUAL = 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (IEEE double, no contraction into FMAs)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
               "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", _LIB_PATH + ".tmp"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
        for name in ("oracle_markov_draft", "oracle_markov_draft_opts", "oracle_confidence",
                     "oracle_plan", "oracle_verify", "oracle_verify_opts", "oracle_rnn_draft",
                     "oracle_rnn_verify", "oracle_tree_draft", "oracle_tree_verify"):
            getattr(_lib, name).restype = ctypes.c_int
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _bits(a):
    """bf16 weights as uint16 bit patterns (accepts uint16/int16 numpy arrays)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("bf16 operands must be passed as uint16 bit patterns")
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} rejected its arguments (code {rc})")


def markov_draft(U, W1, W2t, anchor, uniforms, force_tokens=None, want_logits=False, threads=0,
                 temperature=1.0, greedy=False):
    """Markov-head draft. U [B][g][V] f32, W1/W2t [V][r] bf16 bits, anchor [B] i32,
    uniforms [B][g+1][3] f32; temperature > 0 (logits scaled by fp32(1/temperature)) or greedy.
    Returns dict(tokens, q, lse, margin[, logits]); for greedy, margin is the gap between the
    two largest logits."""
    lib = _load()
    U = _c(U, np.float32)
    B, g, V = U.shape
    W1, W2t = _bits(W1), _bits(W2t)
    r = W1.shape[1]
    anchor = _c(anchor, np.int32)
    uniforms = _c(uniforms, np.float32)
    assert W1.shape == (V, r) and W2t.shape == (V, r) and uniforms.shape == (B, g + 1, 3)
    force = None if force_tokens is None else _c(force_tokens, np.int32)
    out = dict(tokens=np.zeros((B, g), np.int32), q=np.zeros((B, g), np.float32),
               lse=np.zeros((B, g), np.float64), margin=np.zeros((B, g), np.float64))
    logits = np.zeros((B, g, V), np.float32) if want_logits else None
    rc = lib.oracle_markov_draft_opts(B, g, V, r, _ptr(U), _ptr(W1), _ptr(W2t), _ptr(anchor),
                                      _ptr(uniforms), _ptr(force), ctypes.c_float(temperature),
                                      int(bool(greedy)), _ptr(out["tokens"]), _ptr(out["q"]),
                                      _ptr(out["lse"]), _ptr(logits), _ptr(out["margin"]),
                                      int(threads))
    _check(rc, "oracle_markov_draft")
    if want_logits:
        out["logits"] = logits
    return out


def confidence(h, W1, w, T, anchor, tokens, threads=0):
    """Confidence head. h [B][g][d] bf16 bits, w [d+r] bf16 bits, T [g] f32.
    Returns dict(conf f32 [B][g], z f64 [B][g])."""
    lib = _load()
    h, W1, w = _bits(h), _bits(W1), _bits(w)
    B, g, d = h.shape
    V, r = W1.shape
    assert w.shape == (d + r,)
    T = _c(T, np.float32)
    anchor = _c(anchor, np.int32)
    tokens = _c(tokens, np.int32)
    conf = np.zeros((B, g), np.float32)
    z = np.zeros((B, g), np.float64)
    rc = lib.oracle_confidence(B, g, V, r, d, _ptr(h), _ptr(W1), _ptr(w), _ptr(T), _ptr(anchor),
                               _ptr(tokens), _ptr(conf), _ptr(z), int(threads))
    _check(rc, "oracle_confidence")
    return dict(conf=conf, z=z)


def plan(conf, sps, mode, B=None, gamma=None, ring=None, round_index=0):
    """Verify planner. conf [B][g] f32 (may be None for FULL_VERIFY with B, gamma given),
    sps f64 [n], ring f32 [2][B][g] updated in place for LAGGED_TOPK.
    Returns dict(draft_len, row_offsets, stats, margin, theta_path)."""
    lib = _load()
    if conf is not None:
        conf = _c(conf, np.float32)
        B, gamma = conf.shape
    sps = _c(sps, np.float64)
    if ring is not None:
        assert ring.dtype == np.float32 and ring.flags.c_contiguous and ring.shape == (2, B, gamma)
    draft_len = np.zeros(B, np.int32)
    row_offsets = np.zeros(B + 1, np.int32)
    stats = np.zeros(4, np.float64)
    margin = np.zeros(1, np.float64)
    theta = np.zeros(B * gamma + 1, np.float64)
    rc = lib.oracle_plan(B, gamma, _ptr(conf), _ptr(sps), int(sps.shape[0]), int(mode), _ptr(ring),
                         int(round_index), _ptr(draft_len), _ptr(row_offsets), _ptr(stats),
                         _ptr(margin), _ptr(theta))
    _check(rc, "oracle_plan")
    return dict(draft_len=draft_len, row_offsets=row_offsets, stats=stats, margin=float(margin[0]),
                theta_path=theta)


def verify(target, row_offsets, draft_len, U, W1, W2t, anchor, tokens, q, uniforms, threads=0,
           temperature=1.0, greedy=False):
    """Lossless verify. target [row_offsets[B]][V] f32 (packed rows); temperature / greedy
    describe the draft distribution (as for markov_draft).
    Returns dict(accept_len, next_token, beta_emit, flags, accept_margin, emit_margin,
    resid_mass)."""
    lib = _load()
    U = _c(U, np.float32)
    B, g, V = U.shape
    W1, W2t = _bits(W1), _bits(W2t)
    r = W1.shape[1]
    target = _c(target, np.float32)
    row_offsets = _c(row_offsets, np.int32)
    draft_len = _c(draft_len, np.int32)
    assert target.shape == (int(row_offsets[B]), V)
    out = dict(accept_len=np.zeros(B, np.int32), next_token=np.zeros(B, np.int32),
               beta_emit=np.zeros(B, np.float32), flags=np.zeros(B, np.uint32),
               accept_margin=np.zeros((B, g), np.float64), emit_margin=np.zeros(B, np.float64),
               resid_mass=np.zeros(B, np.float64))
    rc = lib.oracle_verify_opts(B, g, V, r, _ptr(target), _ptr(row_offsets), _ptr(draft_len),
                           _ptr(U), _ptr(W1), _ptr(W2t), _ptr(_c(anchor, np.int32)),
                           _ptr(_c(tokens, np.int32)), _ptr(_c(q, np.float32)),
                           _ptr(_c(uniforms, np.float32)), ctypes.c_float(temperature),
                           int(bool(greedy)), _ptr(out["accept_len"]),
                           _ptr(out["next_token"]), _ptr(out["beta_emit"]), _ptr(out["flags"]),
                           _ptr(out["accept_margin"]), _ptr(out["emit_margin"]),
                           _ptr(out["resid_mass"]), int(threads))
    _check(rc, "oracle_verify")
    return out


def rnn_draft(U, W1, W2t, Wgco, h, anchor, uniforms, force_tokens=None, want_logits=False,
              threads=0, temperature=1.0, greedy=False):
    """RNN-head draft, eq. (6). U [B][g][V] f32; W1/W2t [V][r], Wgco [3r][2r+d] (rows W_g, W_c,
    W_o) and h [B][g][d] as bf16 bits; anchor, uniforms, options as for markov_draft.
    Returns dict(tokens, q, lse, margin, e[, logits]) with e [B][g][r] f64 = tanh(W_o z_k)."""
    lib = _load()
    U = _c(U, np.float32)
    B, g, V = U.shape
    W1, W2t, Wgco, h = _bits(W1), _bits(W2t), _bits(Wgco), _bits(h)
    r = W1.shape[1]
    d = h.shape[2]
    assert W1.shape == (V, r) and W2t.shape == (V, r) and h.shape == (B, g, d)
    assert Wgco.shape == (3 * r, 2 * r + d)
    anchor = _c(anchor, np.int32)
    uniforms = _c(uniforms, np.float32)
    assert uniforms.shape == (B, g + 1, 3)
    force = None if force_tokens is None else _c(force_tokens, np.int32)
    out = dict(tokens=np.zeros((B, g), np.int32), q=np.zeros((B, g), np.float32),
               lse=np.zeros((B, g), np.float64), margin=np.zeros((B, g), np.float64),
               e=np.zeros((B, g, r), np.float64))
    logits = np.zeros((B, g, V), np.float32) if want_logits else None
    rc = lib.oracle_rnn_draft(B, g, V, r, d, _ptr(U), _ptr(W1), _ptr(W2t), _ptr(Wgco), _ptr(h),
                              _ptr(anchor), _ptr(uniforms), _ptr(force), ctypes.c_float(temperature),
                              int(bool(greedy)), _ptr(out["tokens"]), _ptr(out["q"]),
                              _ptr(out["lse"]), _ptr(logits), _ptr(out["margin"]), _ptr(out["e"]),
                              int(threads))
    _check(rc, "oracle_rnn_draft")
    if want_logits:
        out["logits"] = logits
    return out


def rnn_verify(target, row_offsets, draft_len, U, W1, W2t, Wgco, h, anchor, tokens, q, uniforms,
               threads=0, temperature=1.0, greedy=False):
    """Lossless verify of an RNN-head draft (p_d recomputed from eq. (6) along the drafted
    tokens). Arguments and result as for verify, plus Wgco and h as for rnn_draft."""
    lib = _load()
    U = _c(U, np.float32)
    B, g, V = U.shape
    W1, W2t, Wgco, h = _bits(W1), _bits(W2t), _bits(Wgco), _bits(h)
    r = W1.shape[1]
    d = h.shape[2]
    assert Wgco.shape == (3 * r, 2 * r + d) and h.shape == (B, g, d)
    target = _c(target, np.float32)
    row_offsets = _c(row_offsets, np.int32)
    draft_len = _c(draft_len, np.int32)
    assert target.shape == (int(row_offsets[B]), V)
    out = dict(accept_len=np.zeros(B, np.int32), next_token=np.zeros(B, np.int32),
               beta_emit=np.zeros(B, np.float32), flags=np.zeros(B, np.uint32),
               accept_margin=np.zeros((B, g), np.float64), emit_margin=np.zeros(B, np.float64),
               resid_mass=np.zeros(B, np.float64))
    rc = lib.oracle_rnn_verify(B, g, V, r, d, _ptr(target), _ptr(row_offsets), _ptr(draft_len),
                               _ptr(U), _ptr(W1), _ptr(W2t), _ptr(Wgco), _ptr(h),
                               _ptr(_c(anchor, np.int32)), _ptr(_c(tokens, np.int32)),
                               _ptr(_c(q, np.float32)), _ptr(_c(uniforms, np.float32)),
                               ctypes.c_float(temperature), int(bool(greedy)),
                               _ptr(out["accept_len"]), _ptr(out["next_token"]),
                               _ptr(out["beta_emit"]), _ptr(out["flags"]),
                               _ptr(out["accept_margin"]), _ptr(out["emit_margin"]),
                               _ptr(out["resid_mass"]), int(threads))
    _check(rc, "oracle_rnn_verify")
    return out


def tree_candidates(gamma, c, M):
    """Number of candidate nodes a tree draft expands: c at depth 1, min(M, previous) * c after."""
    total, width = c, c
    for _ in range(2, gamma + 1):
        width = min(M, width) * c
        total += width
    return total


def tree_draft(U, W1, W2t, anchor, c, M, N, threads=0):
    """PCTree draft: c children a node, M nodes expanded a depth, N nodes kept.
    Returns dict(token, depth, parent [B][N] int32, q, path [B][N] f64, logit_margin,
    path_margin [B] f64); nodes in rank order, parent = rank of the parent (-1: the root)."""
    lib = _load()
    U = _c(U, np.float32)
    B, g, V = U.shape
    W1, W2t = _bits(W1), _bits(W2t)
    r = W1.shape[1]
    out = dict(token=np.zeros((B, N), np.int32), depth=np.zeros((B, N), np.int32),
               parent=np.zeros((B, N), np.int32), q=np.zeros((B, N), np.float64),
               path=np.zeros((B, N), np.float64), logit_margin=np.zeros(B, np.float64),
               path_margin=np.zeros(B, np.float64))
    rc = lib.oracle_tree_draft(B, g, V, r, int(c), int(M), int(N), _ptr(U), _ptr(W1), _ptr(W2t),
                               _ptr(_c(anchor, np.int32)), _ptr(out["token"]), _ptr(out["depth"]),
                               _ptr(out["parent"]), _ptr(out["q"]), _ptr(out["path"]),
                               _ptr(out["logit_margin"]), _ptr(out["path_margin"]), int(threads))
    _check(rc, "oracle_tree_draft")
    return out


def tree_verify(target, token, depth, parent, uniforms, threads=0):
    """Lossless verify of a tree. target [B][N+1][V] f32 (row 0: after the anchor; row 1+n:
    after node n). Returns dict(accept_len, path [B][gamma], next_token, flags, margin)."""
    lib = _load()
    target = _c(target, np.float32)
    B, n1, V = target.shape
    N = n1 - 1
    uniforms = _c(uniforms, np.float32)
    g = uniforms.shape[1] - 1
    out = dict(accept_len=np.zeros(B, np.int32), path=np.zeros((B, g), np.int32),
               next_token=np.zeros(B, np.int32), flags=np.zeros(B, np.uint32),
               margin=np.zeros(B, np.float64))
    rc = lib.oracle_tree_verify(B, g, V, N, _ptr(target), _ptr(_c(token, np.int32)),
                                _ptr(_c(depth, np.int32)), _ptr(_c(parent, np.int32)),
                                _ptr(uniforms), _ptr(out["accept_len"]), _ptr(out["path"]),
                                _ptr(out["next_token"]), _ptr(out["flags"]), _ptr(out["margin"]),
                                int(threads))
    _check(rc, "oracle_tree_verify")
    return out
