"""Host-side checks of libdspark.so that need no GPU: every symbol the public header declares is
exported, workspace sizing, and the synchronous argument checks (a bad argument returns its
status before anything is enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

import lossless_draft_verify_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.library_path()):
        from lossless_draft_verify_amd import build
        build.build()
    return L.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"DSPARK_API\s+[\w\s\*]+?\b(dspark_\w+)\s*\(", text)))


def test_header_declares_the_four_round_operations():
    names = _declared()
    for n in ("dspark_markov_draft", "dspark_confidence", "dspark_plan", "dspark_verify"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(dspark_\w+)", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        getattr(lib, n)


def test_workspace_sizes(lib):
    d = L.Dims(128, 5, 129280, 256, 5120)
    draft = L.workspace_bytes(d, L.OP_DRAFT)
    assert draft >= 2 * 128 * (129280 // 32) * 4
    assert L.workspace_bytes(d, L.OP_CONFIDENCE) == 0
    assert L.workspace_bytes(d, L.OP_PLAN) == 0
    assert L.workspace_bytes(d, L.OP_VERIFY) > 0
    with pytest.raises(L.DsparkError):
        L.workspace_bytes(L.Dims(128, 5, 129280, 100, 5120), L.OP_DRAFT)   # unsupported rank


def _p(v=256):
    return ctypes.c_void_p(v)


def test_argument_checks_without_gpu(lib):
    d = L.Dims(4, 3, 1000, 16, 64).c()
    ws_ok = L.workspace_bytes(L.Dims(4, 3, 1000, 16, 64), L.OP_DRAFT)
    P = _p()
    # NULL
    assert lib.dspark_markov_draft(d, None, P, P, P, P, P, P, P, None, None, P, ws_ok, None) == 1
    # unsupported rank
    bad = L.Dims(4, 3, 1000, 24, 64).c()
    assert lib.dspark_markov_draft(bad, P, P, P, P, P, P, P, P, None, None, P, ws_ok, None) == 2
    # misaligned U
    assert lib.dspark_markov_draft(d, _p(260), P, P, P, P, P, P, P, None, None, P, ws_ok, None) == 3
    # workspace too small
    assert lib.dspark_markov_draft(d, P, P, P, P, P, P, P, P, None, None, P, ws_ok - 1, None) == 4
    # SPS table too short, bad mode, lagged without ring
    assert lib.dspark_plan(d, P, P, 4 * 4, 1, None, 0, P, P, None, None) == 5
    assert lib.dspark_plan(d, P, P, 4 * 4 + 1, 9, None, 0, P, P, None, None) == 7
    assert lib.dspark_plan(d, P, P, 4 * 4 + 1, 3, None, 0, P, P, None, None) == 7
    assert lib.dspark_plan(d, None, P, 4 * 4 + 1, 1, None, 0, P, P, None, None) == 1
    # planner size limit
    big = L.Dims(2000, 5, 1000, 16, 64).c()
    assert lib.dspark_plan(big, P, P, 2000 * 6 + 1, 1, None, 0, P, P, None, None) == 2
    # confidence: d must be a positive multiple of 8
    odd = L.Dims(4, 3, 1000, 16, 12).c()
    assert lib.dspark_confidence(odd, P, P, P, P, P, P, P, None) == 2
    # verify workspace
    vws = L.workspace_bytes(L.Dims(4, 3, 1000, 16, 64), L.OP_VERIFY)
    args = [P] * 13 + [None, None, P, vws - 1, None]
    assert lib.dspark_verify(d, *args) == 4
    assert lib.dspark_status_string(4) == b"workspace too small"


def test_draft_option_checks_without_gpu(lib):
    """A temperature that is not positive and finite is refused (status 8) by the draft and the
    verify; a greedy draft ignores the temperature, so its call goes on to the next check."""
    dims = L.Dims(4, 3, 1000, 16, 64)
    d, P = dims.c(), _p()
    ws_ok = L.workspace_bytes(dims, L.OP_DRAFT)
    vws = L.workspace_bytes(dims, L.OP_VERIFY)
    opts = L.binding._CDraftOpts
    for t in (0.0, -1.0, float("inf"), float("nan")):
        o = ctypes.byref(opts(t, 0))
        assert lib.dspark_markov_draft_opts(d, P, P, P, P, P, P, P, P, None, None, P, ws_ok, o,
                                            None) == 8
        assert lib.dspark_verify_opts(d, *([P] * 13), None, None, P, vws, o, None) == 8
    g = ctypes.byref(opts(0.0, 1))
    assert lib.dspark_markov_draft_opts(d, P, P, P, P, P, P, P, P, None, None, P, ws_ok - 1, g,
                                        None) == 4
    assert lib.dspark_verify_opts(d, *([P] * 13), None, None, P, vws - 1, g, None) == 4
    assert lib.dspark_status_string(8) == b"draft temperature not positive and finite"


def test_rnn_head_checks_without_gpu(lib):
    """The RNN head: workspace sizes, r <= 256 and d a positive multiple of 8, NULL checks."""
    dims = L.Dims(4, 3, 1000, 16, 64)
    d, P = dims.c(), _p()
    n = L.workspace_bytes(dims, L.OP_RNN_DRAFT)
    assert n >= L.workspace_bytes(dims, L.OP_DRAFT) + 8 * 12 * 48 * 4 + 2 * 4 * 16 * 8 + 12 * 48 * 2
    v = L.workspace_bytes(dims, L.OP_RNN_VERIFY)
    assert v >= L.workspace_bytes(dims, L.OP_VERIFY) + 12 * 48 * 2
    for bad in (L.Dims(4, 3, 1000, 512, 64), L.Dims(4, 3, 1000, 16, 12), L.Dims(4, 3, 1000, 16, 0)):
        with pytest.raises(L.DsparkError):
            L.workspace_bytes(bad, L.OP_RNN_DRAFT)
        assert lib.dspark_rnn_draft(bad.c(), *([P] * 11), None, None, P, n, None, None) == 2
    # NULL Wgco; a workspace one byte short
    assert lib.dspark_rnn_draft(d, P, P, P, None, *([P] * 7), None, None, P, n, None, None) == 1
    assert lib.dspark_rnn_draft(d, *([P] * 11), None, None, P, n - 1, None, None) == 4
    assert lib.dspark_rnn_verify(d, *([P] * 12), None, None, P, v - 1, None, None) == 4
    assert lib.dspark_rnn_verify(d, *([P] * 5), None, *([P] * 6), None, None, P, v, None,
                                 None) == 1


def test_binding_refuses_host_tensors(lib):
    import torch
    d = L.Dims(4, 3, 1000, 16, 64)
    with pytest.raises(L.DsparkError):
        L.confidence(d, torch.zeros((4, 3, 64), dtype=torch.bfloat16), None, None, None, None, None,
                     conf=torch.zeros((4, 3)))


def _c_kind(param):
    """The ctypes kind a C parameter needs: pointer, int32, size_t or the dims struct."""
    t = param.rsplit(" ", 1)[0] if not param.endswith("*") else param
    if "*" in param:
        return "ptr"
    if t.startswith("dspark_dims"):
        return "dims"
    if t.startswith("dspark_tree_shape"):
        return "tree_shape"
    if t.startswith("size_t"):
        return "size_t"
    if t.startswith("int32_t") or t.startswith("dspark_status"):
        return "int32"
    raise AssertionError(f"unmapped C parameter {param!r}")


def _py_kind(t):
    if t is L.binding._CDims:
        return "dims"
    if t is L.binding._CTreeShape:
        return "tree_shape"
    if t is ctypes.c_size_t:
        return "size_t"
    if t is ctypes.c_int32:
        return "int32"
    if t is ctypes.c_void_p or (isinstance(t, type) and issubclass(t, ctypes._Pointer)):
        return "ptr"
    raise AssertionError(f"unmapped ctypes type {t!r}")


def test_draft_plan_checks_without_gpu(lib):
    """dspark_markov_draft_plan refuses what the draft, confidence and plan calls refuse, with
    the same statuses, before anything is enqueued."""
    dims = L.Dims(4, 3, 1000, 16, 64)
    d, P = dims.c(), _p()
    ws = L.workspace_bytes(dims, L.OP_DRAFT)
    sl = 4 * 4 + 1

    def call(dd=d, U=P, h=P, sps_len=sl, mode=1, ring=None, conf=P, ws_bytes=ws, opts=None):
        return lib.dspark_markov_draft_plan(dd, U, P, P, P, P, h, P, P, P, sps_len, mode, ring, 0,
                                            P, P, P, conf, P, P, None, P, ws_bytes, opts, None)

    assert call(U=None) == 1                       # draft input
    assert call(h=None) == 1                       # confidence input
    assert call(conf=None) == 1                    # the confidences are an output here
    assert call(dd=L.Dims(4, 3, 1000, 16, 12).c()) == 2   # d not a multiple of 8
    assert call(dd=L.Dims(2000, 5, 1000, 16, 64).c(), sps_len=2000 * 6 + 1) == 2   # plan size
    assert call(sps_len=sl - 1) == 5
    assert call(mode=9) == 7
    assert call(mode=3) == 7                       # LAGGED_TOPK without a ring
    assert call(U=_p(260)) == 3
    assert call(ws_bytes=ws - 1) == 4
    bad_t = ctypes.byref(L.binding._CDraftOpts(0.0, 0))
    assert call(opts=bad_t) == 8


def test_rnn_draft_plan_checks_without_gpu(lib):
    """dspark_rnn_draft_plan refuses what the RNN draft, confidence and plan calls refuse."""
    dims = L.Dims(4, 3, 1000, 16, 64)
    d, P = dims.c(), _p()
    ws = L.workspace_bytes(dims, L.OP_RNN_DRAFT)
    sl = 4 * 4 + 1

    def call(dd=d, Wgco=P, e_rows=P, sps_len=sl, mode=1, ws_bytes=ws):
        return lib.dspark_rnn_draft_plan(dd, P, P, P, Wgco, P, P, P, P, P, P, sps_len, mode, None,
                                         0, P, P, P, e_rows, P, P, P, None, P, ws_bytes, None,
                                         None)

    assert call(Wgco=None) == 1
    assert call(e_rows=None) == 1
    assert call(dd=L.Dims(4, 3, 1000, 512, 64).c()) == 2     # the RNN head takes r <= 256
    assert call(sps_len=sl - 1) == 5
    assert call(mode=3) == 7                                  # LAGGED_TOPK without a ring
    assert call(ws_bytes=ws - 1) == 4


def test_binding_signatures_match_the_header(lib):
    """Every function the binding declares has the header's parameter count and kinds, so a
    marshalled call can never shift its arguments."""
    text = open(HEADER).read()
    decls = dict(re.findall(r"DSPARK_API\s+[\w\s\*]+?\b(dspark_\w+)\s*\(([^)]*)\)\s*;", text))
    checked = 0
    for name, params in decls.items():
        fn = getattr(lib, name)
        if getattr(fn, "argtypes", None) is None:
            continue
        c_params = [p.strip() for p in params.split(",") if p.strip() and p.strip() != "void"]
        assert len(fn.argtypes) == len(c_params), (name, len(fn.argtypes), len(c_params))
        for c, py in zip(c_params, fn.argtypes):
            assert _c_kind(c) == _py_kind(py), (name, c, py)
        checked += 1
    assert checked >= 12


def test_noalloc_verify_refuses_sizes_beyond_its_scratch(lib):
    """dspark_verify_noalloc checks the workspace its shape needs against its fixed scratch
    array on the host, before any HIP call: too large a shape returns DSPARK_ERR_WORKSPACE, a
    null output DSPARK_ERR_NULL, a bad shape DSPARK_ERR_SHAPE."""
    P = _p()
    big = L.Dims(1024, 5, 151936, 256, 8)
    assert L.workspace_bytes(big, L.OP_VERIFY) > L.NOALLOC_SCRATCH_BYTES
    args = [P] * 13 + [None, None, None, None]
    assert lib.dspark_verify_noalloc(big.c(), *args) == 4
    fits = L.Dims(512, 15, 151936, 256, 8)
    assert L.workspace_bytes(fits, L.OP_VERIFY) <= L.NOALLOC_SCRATCH_BYTES
    assert lib.dspark_verify_noalloc(fits.c(), *([P] * 12 + [None] + [None] * 4)) == 1
    assert lib.dspark_verify_noalloc(L.Dims(4, 3, 1000, 24, 8).c(), *args) == 2


def test_tree_shape_checks(lib):
    """PCTree shape limits are checked on the host: M <= c <= 8, M a power of two, the candidate
    count and the budget; an unsupported shape sizes no workspace and is refused."""
    d = L.Dims(16, 5, 129280, 256, 8)
    ok = L.TreeShape(4, 4, 16)
    assert L.tree_workspace_bytes(d, ok, L.OP_TREE_DRAFT) > 0
    assert L.tree_workspace_bytes(d, ok, L.OP_TREE_VERIFY) > 0
    for bad in (L.TreeShape(4, 8, 16), L.TreeShape(9, 1, 4), L.TreeShape(4, 3, 16),
                L.TreeShape(4, 4, 0), L.TreeShape(4, 4, 4 + 4 * 16 * 4 + 1)):
        with pytest.raises(L.DsparkError):
            L.tree_workspace_bytes(d, bad, L.OP_TREE_DRAFT)
    P = _p()
    ws = L.tree_workspace_bytes(d, ok, L.OP_TREE_DRAFT)
    assert lib.dspark_tree_draft(d.c(), ok.c_struct(), *([P] * 9), P, ws - 1, None) == 4
    assert lib.dspark_tree_draft(d.c(), L.TreeShape(4, 3, 16).c_struct(), *([P] * 9), P, ws,
                                 None) == 2
    assert lib.dspark_tree_verify(d.c(), ok.c_struct(), None, *([P] * 7), P, ws, None) == 1
