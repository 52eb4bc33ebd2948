"""Window attention in fp64 (oracle; test infrastructure only).

[PI] §2, Eq. 1-2: attention is softmax of query-key logits times V; with a
KV cache only the rows of the queries of interest are needed.
[DK] §2 (preliminaries): prefill attention carries a causal mask that hides
keys after the query position.
[DK] §3.4: the window's rows are scored against the full cache using their
row log-sum-exp LSE and output a (called o here).

Reading (logit scale): [PI] drops 1/sqrt(d), [DK] keeps it; the scale is an
explicit argument `sm_scale` (1/sqrt(d) in every workload).
Reading (window positions): window row i of a sequence of n tokens is prompt
position n - w + i; with causal=1 it sees keys 0..n-w+i.

Pinned by: rows of alpha sum to one; o against torch's fp64
scaled_dot_product_attention (a library routine); causal rows equal
non-causal attention restricted to the visible prefix.
"""
from __future__ import annotations

import numpy as np


def row_positions(n: int, w: int) -> np.ndarray:
    """Prompt position of each window row: n - w + i."""
    return np.arange(n - w, n, dtype=np.int64)


def window_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, pos: np.ndarray | None,
                     sm_scale: float):
    """Attention of R query rows against n keys.

    q   [R, d] float64 query rows
    k,v [n, d] float64
    pos [R] int positions (key j visible iff j <= pos[r]); None = no mask
    Returns dict(logits [R,n] with -inf for hidden keys, alpha [R,n],
    lse [R], o [R,d], e [R,n] = exp(logit - rowmax), z [R]).
    """
    n = k.shape[0]
    logits = sm_scale * (q @ k.T)
    if pos is not None:
        hidden = np.arange(n)[None, :] > np.asarray(pos)[:, None]
        logits = np.where(hidden, -np.inf, logits)
    mx = logits.max(axis=1)
    e = np.exp(logits - mx[:, None])
    z = e.sum(axis=1)
    alpha = e / z[:, None]
    o = alpha @ v
    lse = mx + np.log(z)
    return {"logits": logits, "alpha": alpha, "lse": lse, "o": o, "e": e, "z": z}
