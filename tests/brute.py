"""Brute-force reference computations for tiny inputs, independent of the
oracle: exact rational arithmetic (fractions.Fraction) for the page bounds,
a rank-counting definition of top-k, and dense masked softmax attention in
numpy fp64.  They work on per-sequence logical token arrays, never on the
paged pool, so a page-table or layout mistake in the oracle shows up here.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


# ----------------------------------------------------------------------------
# bf16 helpers
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# summaries, bounds, selection
# ----------------------------------------------------------------------------

def _order_key(v: float):
    # numeric order, -0 before +0
    return (v, 0 if math.copysign(1.0, v) < 0 else 1)


def summary(keys):
    """keys: list of token key vectors (floats).  Returns (lo, hi) lists."""
    D = len(keys[0])
    lo = [min((k[d] for k in keys), key=_order_key) for d in range(D)]
    hi = [max((k[d] for k in keys), key=_order_key) for d in range(D)]
    return lo, hi


def page_bound(q, lo, hi) -> float:
    """Exact sum_d max(q_d lo_d, q_d hi_d), rounded once to the nearest double."""
    total = Fraction(0)
    for qd, a, b in zip(q, lo, hi):
        total += max(Fraction(qd) * Fraction(a), Fraction(qd) * Fraction(b))
    return float(total)  # Fraction -> float rounds correctly


def exact_dot(q, k) -> Fraction:
    return sum((Fraction(a) * Fraction(b) for a, b in zip(q, k)), Fraction(0))


def rank_select(keys: dict, k: int):
    """keys: {page id: score}.  Page j is kept iff fewer than k pages beat it,
    where i beats j when its score is larger, or equal with a smaller id."""
    chosen = []
    for j, sj in keys.items():
        beaten_by = sum(1 for i, si in keys.items() if si > sj or (si == sj and i < j))
        if beaten_by < k:
            chosen.append(j)
    return sorted(chosen)


# ----------------------------------------------------------------------------
# dense attention
# ----------------------------------------------------------------------------

def dense_attention(q, K, V, mask, scale):
    """q [Dk], K [L][Dk], V [L][Dv], mask [L] bool -> softmax(scale q.K) V over
    the masked-in tokens, fp64.  All tokens masked out -> zeros."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    mask = np.asarray(mask, bool)
    if not mask.any():
        return np.zeros(V.shape[1])
    s = scale * (K[mask] @ q)
    w = np.exp(s - s.max())
    return (w[:, None] * V[mask]).sum(0) / w.sum()


def ashape_mask(L, sink_tokens, window_tokens):
    t = np.arange(L)
    return (t < sink_tokens) | (t >= L - window_tokens)


def page_token_mask(L, ps, pages):
    m = np.zeros(L, bool)
    for j in pages:
        m[j * ps:min((j + 1) * ps, L)] = True
    return m
