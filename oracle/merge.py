"""Partition-conserving merge of evicted entries (oracle; test
infrastructure only).

"Information-Theoretic Token Eviction and KV-Cache Compression for
Memory-Bounded Long-Context LLM Inference", §4.1 (Partition-Conserving
Key-Value Merge): an evicted entry e whose key has cosine similarity above
tau_merge with a retained entry r* is merged into r*, whose multiplicity
m_r* grows by one; later attention adds log m_r to that entry's logit, so an
exact duplicate leaves the softmax normaliser unchanged.

Readings (also in the design notes):
 * r* is the retained entry of the same sequence and KV head with the
   largest cosine similarity to e (the lowest kept position on ties); e is
   merged when that similarity is strictly above tau_merge;
 * every entry starts with multiplicity 1; the merged entry keeps its own key
   and value; its bias grows by log(m_r) = log(1 + number merged into it);
 * a zero key has similarity 0 with every key.

Pinned by: exact duplicates merge into their original and conserve the
normaliser; orthogonal keys never merge; a brute-force double loop.
"""
from __future__ import annotations

import numpy as np


def cosine(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Cosine similarities of the rows of a [p][d] with the rows of b [q][d]."""
    na = np.linalg.norm(a, axis=1)
    nb = np.linalg.norm(b, axis=1)
    ia = np.where(na > 0, 1.0 / np.where(na > 0, na, 1.0), 0.0)
    ib = np.where(nb > 0, 1.0 / np.where(nb > 0, nb, 1.0), 0.0)
    return (a @ b.T) * ia[:, None] * ib[None, :]


def merge_targets(k: np.ndarray, kept: np.ndarray, tau_merge: float):
    """k [n][d] keys of one (sequence, KV head); kept: ascending kept
    positions.  Returns (target [n]: kept-list position r* or -1, cos [n]:
    the best similarity, -inf for kept entries)."""
    n = k.shape[0]
    is_kept = np.zeros(n, dtype=bool)
    is_kept[kept] = True
    target = np.full(n, -1, dtype=np.int64)
    best = np.full(n, -np.inf)
    ev = np.nonzero(~is_kept)[0]
    if ev.size == 0 or kept.size == 0:
        return target, best
    c = cosine(k[ev], k[kept])
    r = np.argmax(c, axis=1)              # first maximum: lowest kept position on ties
    cm = c[np.arange(ev.size), r]
    best[ev] = cm
    target[ev] = np.where(cm > tau_merge, r, -1)
    return target, best


def merge_counts(k: np.ndarray, kept: np.ndarray, tau_merge: float) -> np.ndarray:
    """Number of evicted entries merged into each kept entry."""
    target, _ = merge_targets(k, kept, tau_merge)
    t = target[target >= 0]
    return np.bincount(t, minlength=kept.shape[0]).astype(np.int64)


def merged_bias(bias: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """Bias of the kept entries after the merge: bias + log(1 + count)."""
    return bias + np.log1p(counts.astype(np.float64))
