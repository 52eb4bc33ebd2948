"""Brute-force checks used to pin the oracle (test infrastructure).

Everything here recomputes attention from scratch with the token(s) removed,
independently of the oracle's closed forms."""
from __future__ import annotations

import itertools

import numpy as np


def attn_row(q, k, v, scale, visible):
    """Plain softmax attention of one query over the keys where visible."""
    idx = np.nonzero(visible)[0]
    lg = scale * (k[idx] @ q)
    lg = lg - lg.max()
    p = np.exp(lg)
    p /= p.sum()
    return p @ v[idx]


def drop_one_perturbation(q, k, v, scale, pos):
    """||o_{-j} - o|| for every key j (NaN where j is hidden or the only key)."""
    n = k.shape[0]
    vis = np.arange(n) <= pos if pos is not None else np.ones(n, bool)
    o = attn_row(q, k, v, scale, vis)
    out = np.full(n, np.nan)
    for j in range(n):
        if not vis[j]:
            out[j] = 0.0
            continue
        vj = vis.copy()
        vj[j] = False
        if not vj.any():
            out[j] = np.nan
            continue
        out[j] = np.linalg.norm(attn_row(q, k, v, scale, vj) - o)
    return out


def drop_set_perturbation(q, k, v, scale, J):
    n = k.shape[0]
    vis = np.ones(n, bool)
    o = attn_row(q, k, v, scale, vis)
    vj = vis.copy()
    vj[list(J)] = False
    return np.linalg.norm(attn_row(q, k, v, scale, vj) - o)


def best_subset(q, k, v, scale, n_evict):
    """Exhaustive minimum of the output perturbation over all eviction sets of
    size n_evict (the exact combinatorial problem)."""
    n = k.shape[0]
    best, arg = np.inf, None
    for J in itertools.combinations(range(n), n_evict):
        f = drop_set_perturbation(q, k, v, scale, J)
        if f < best:
            best, arg = f, J
    return best, arg
