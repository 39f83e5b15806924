"""Small helpers shared by the tests (no method arithmetic beyond textbook library calls)."""
import json
import os

import numpy as np
from scipy import special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16_exact(x):
    """uint16 bf16 bit patterns of values that are exactly representable in bf16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bf16_round(x):
    """Round-to-nearest-even to bf16; returns uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def softmax64(x, axis=-1):
    return special.softmax(np.asarray(x, np.float64), axis=axis)


def logsumexp64(x, axis=-1):
    return special.logsumexp(np.asarray(x, np.float64), axis=axis)


def first_emitted(tokens, accept_len, next_token):
    """First token the round emits: the first drafted token if accepted, else the resample."""
    return np.where(accept_len >= 1, tokens[:, 0], next_token)


def chi2_pvalue(counts, probs):
    counts = np.asarray(counts, np.float64)
    n = counts.sum()
    exp = n * np.asarray(probs, np.float64)
    keep = exp > 0
    stat = ((counts[keep] - exp[keep]) ** 2 / exp[keep]).sum()
    dof = keep.sum() - 1
    from scipy import stats
    return stats.chi2.sf(stat, dof)


def dense_offsets(B, gamma):
    return (np.arange(B + 1) * (gamma + 1)).astype(np.int32)
