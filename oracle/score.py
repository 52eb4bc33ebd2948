"""Output-aware eviction scores in fp64 (oracle; test infrastructure only).

[DK] §3.2 (proxy): dropping only token j from the cache moves the head
output by p_j / (1 - p_j) * ||a - v_j||, where p_j is j's softmax weight and
a the full output.
[DK] §3.3 (window score): a token's score is the sum over the observation
window's queries of the squared single-token perturbation.
[PI] §5 (grouped-query attention): all query heads of a GQA group share one
K/V cache, so eviction must be decided once per group.
[PI] App. D (SnapKV) / SnapKV-style 1-D pooling along the key axis.

Readings (listed in the design notes as well):
 * squared perturbation, summed over window rows and over the query heads of
   the group (sum of raw scores; a mean gives the same ranking);
 * 1 - alpha is formed as 1 - alpha except at each row's arg-max key, where
   it is the directly summed weight of all other keys (exact as alpha -> 1);
 * a row that sees a single key contributes 0 for it (o equals that value,
   the perturbation of removing the only key is undefined);
 * hidden (causally masked) pairs contribute 0;
 * pooling is a max filter of odd width along keys, stride 1, same length,
   out-of-range neighbours ignored; it is applied after the group sum.

Pinned by brute-force drop-one-token recomputation of the head output on
small inputs (each row's attention recomputed without token j), the
drop-set identity, and scipy's maximum filter for pooling.
"""
from __future__ import annotations

import numpy as np

from .attention import window_attention, row_positions


def perturbation_scores(q: np.ndarray, k: np.ndarray, v: np.ndarray, pos, sm_scale: float,
                        explicit: bool | None = None) -> np.ndarray:
    """Sum over rows r of (alpha_rj / (1 - alpha_rj))^2 * ||o_r - v_j||^2.

    q [R, d] rows (window rows of every q-head of one group), k/v [n, d],
    pos [R] or None.  explicit=True forms o - v_j directly (O(R n d)),
    False uses ||o||^2 + ||v||^2 - 2 <o, v> in fp64; default: explicit for
    n <= 4096.
    """
    n = k.shape[0]
    if explicit is None:
        explicit = n <= 4096
    att = window_attention(q, k, v, pos, sm_scale)
    alpha, e, z, o = att["alpha"], att["e"], att["z"], att["o"]
    R = q.shape[0]
    one_minus = 1.0 - alpha
    jstar = np.argmax(alpha, axis=1)
    for r in range(R):
        others = e[r].copy()
        others[jstar[r]] = 0.0
        one_minus[r, jstar[r]] = others.sum() / z[r]
    if explicit:
        dist2 = np.empty((R, n))
        for r in range(R):
            diff = o[r][None, :] - v
            dist2[r] = np.einsum("nd,nd->n", diff, diff)
    else:
        dist2 = (o * o).sum(1)[:, None] + (v * v).sum(1)[None, :] - 2.0 * (o @ v.T)
        dist2 = np.maximum(dist2, 0.0)
    # at the arg-max key, o - v_j* = sum_{k != j*} alpha_k (v_k - v_j*): no
    # cancellation when alpha_j* -> 1
    for r in range(R):
        js = jstar[r]
        wts = alpha[r].copy()
        wts[js] = 0.0
        diff = wts @ (v - v[js][None, :])
        dist2[r, js] = diff @ diff
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(alpha > 0.0, alpha / one_minus, 0.0)
        contrib = ratio * ratio * dist2
    # a row with a single visible key: alpha = 1, 1 - alpha = 0, o = v_j
    contrib = np.where((one_minus == 0.0), 0.0, contrib)
    return contrib.sum(axis=0)


def group_scores(q_win: np.ndarray, k: np.ndarray, v: np.ndarray, h: int, g: int,
                 sm_scale: float, causal: bool, row_chunk: int = 64) -> np.ndarray:
    """Score of every key of KV head h for one sequence.

    q_win [Hq][w][d] float64 window queries of the sequence; k, v [n][d].
    Rows are the w window rows of each q-head h*g .. h*g+g-1.
    """
    w, d = q_win.shape[1], q_win.shape[2]
    n = k.shape[0]
    rows = q_win[h * g:(h + 1) * g].reshape(g * w, d)
    pos_one = row_positions(n, w)
    pos = np.tile(pos_one, g) if causal else None
    total = np.zeros(n)
    for r0 in range(0, rows.shape[0], row_chunk):
        sl = slice(r0, r0 + row_chunk)
        total += perturbation_scores(rows[sl], k, v, None if pos is None else pos[sl], sm_scale)
    return total


def group_scores_at(q_win: np.ndarray, k: np.ndarray, v: np.ndarray, h: int, g: int,
                    sm_scale: float, causal: bool, keys: np.ndarray, row_chunk: int = 32) -> np.ndarray:
    """The same group score as group_scores, evaluated only at `keys`
    (sorted unique indices).  Every row's softmax still spans all n keys;
    only the per-key perturbation terms are restricted.  For large n."""
    w, d = q_win.shape[1], q_win.shape[2]
    n = k.shape[0]
    keys = np.asarray(keys, dtype=np.int64)
    rows = q_win[h * g:(h + 1) * g].reshape(g * w, d)
    pos_all = np.tile(row_positions(n, w), g)
    total = np.zeros(len(keys))
    vk = v[keys]
    for r0 in range(0, rows.shape[0], row_chunk):
        q = rows[r0:r0 + row_chunk]
        pos = pos_all[r0:r0 + row_chunk] if causal else None
        att = window_attention(q, k, v, pos, sm_scale)
        alpha, e, z, o = att["alpha"], att["e"], att["z"], att["o"]
        a = alpha[:, keys]
        one_minus = 1.0 - a
        dist2 = (o * o).sum(1)[:, None] + (vk * vk).sum(1)[None, :] - 2.0 * (o @ vk.T)
        dist2 = np.maximum(dist2, 0.0)
        jstar = np.argmax(alpha, axis=1)
        for r in range(q.shape[0]):
            hit = np.nonzero(keys == jstar[r])[0]
            if len(hit):
                c = hit[0]
                others = e[r].copy()
                others[jstar[r]] = 0.0
                one_minus[r, c] = others.sum() / z[r]
                wts = alpha[r].copy()
                wts[jstar[r]] = 0.0
                diff = wts @ (v - v[jstar[r]][None, :])
                dist2[r, c] = diff @ diff
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(a > 0.0, a / one_minus, 0.0)
            contrib = ratio * ratio * dist2
        contrib = np.where(one_minus == 0.0, 0.0, contrib)
        total += contrib.sum(axis=0)
    return total


def max_pool(s: np.ndarray, kernel: int) -> np.ndarray:
    """s'_j = max of s_k over |k - j| <= (kernel-1)/2, 0 <= k < n."""
    if kernel <= 1:
        return s.copy()
    r = (kernel - 1) // 2
    n = s.shape[0]
    out = np.empty_like(s)
    for j in range(n):
        out[j] = s[max(0, j - r):min(n, j + r + 1)].max()
    return out


def max_pool_fast(s: np.ndarray, kernel: int) -> np.ndarray:
    """Same as max_pool, vectorised over shifts (used at large n)."""
    if kernel <= 1:
        return s.copy()
    r = (kernel - 1) // 2
    out = s.copy()
    for sh in range(1, r + 1):
        out[sh:] = np.maximum(out[sh:], s[:-sh])
        out[:-sh] = np.maximum(out[:-sh], s[sh:])
    return out


def score_workload(q_win, k, v, seq_off, Hq: int, Hkv: int, sm_scale: float, causal: bool,
                   pool_kernel: int, heads=None, pooled: bool = True) -> np.ndarray:
    """Scores [Hkv][T] (float64) for a ragged batch laid out as the HIP path
    lays it out: q_win [S][Hq][w][d], k/v [Hkv][T][d], seq_off [S+1].
    heads: optional subset of KV heads (others left as NaN)."""
    g = Hq // Hkv
    T = k.shape[1]
    out = np.full((Hkv, T), np.nan)
    S = len(seq_off) - 1
    for h in (range(Hkv) if heads is None else heads):
        for s in range(S):
            a, b = int(seq_off[s]), int(seq_off[s + 1])
            sc = group_scores(q_win[s], k[h, a:b], v[h, a:b], h, g, sm_scale, causal)
            out[h, a:b] = max_pool_fast(sc, pool_kernel) if pooled else sc
    return out
