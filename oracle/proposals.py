"""Attention-weight eviction scores of the proposals compared on [PI]
(oracle; test infrastructure only).

[PI] App. D, Eq. 16-17 (H2O): a key's score is the sum of the attention
weights it receives over the observed query rows; the proposal normalises
the scores.
[PI] App. D, Eq. 19-20 (TOVA): the score is the last query's attention
weight (averaged over the layer's heads); the proposal normalises it.
[PI] App. H (pi_min, pi_min-h, pi_H2O-h): the minimum-variance proposal of
the last query weighs its attention by ||v_j||; the "-h" variants sum the
attention of every observed query row, row j of t weighted by the harmonic
prior h_j = 1 / ((t - j + 1) H_t), H_t the t-th harmonic number.
[PI] App. D (SnapKV): the column sums are smoothed by 1-D average pooling
along the key axis.
[PI] App. D, Eq. 18 (K-norm): a score from an L2 norm per entry and a
softmax proposal; [DK]'s related work describes the method as keeping the
entries whose KEYS have the smaller norms.

Readings (also in the design notes):
 * the observed query rows are the w observation-window rows; t = w and row
   i = 0 .. w-1 of the window is row j = i + 1 of the prior, so the last
   window row has h = 1 / H_w and the first 1 / (w H_w);
 * the GQA group's q-heads are summed (the layer average of TOVA and the
   group mean differ by a constant factor, which leaves both the ranking and
   the normalised proposal unchanged);
 * average pooling divides by the number of in-range keys in the window
   (out-of-range neighbours are ignored, as in the max pool);
 * K-norm (the two pages disagree on V versus K and on the sign): the
   negative norm of the key row, written as the positive score
   exp(KNORM_SHIFT - ||k_j||) so that the largest scores are the smallest
   norms and the tempered proposal s^(1/tau) is the softmax of -||k|| / tau
   (Eq. 18 with the prose's sign); the constant shift changes neither the
   ranking nor the normalised proposal and keeps norms up to about 167
   inside the fp32 normal range.

Pinned by closed forms: column sums of attention weights add up to the
number of rows (H2O), to the number of q-heads (TOVA, H2O-h), the harmonic
prior sums to one and has known values for small t, and with equal value
norms the value-weighted kinds are that norm times their unweighted
counterparts; average pooling is checked against a library box filter in
the interior.
"""
from __future__ import annotations

import numpy as np

from .attention import window_attention, row_positions

KINDS = ("h2o", "h2o_h", "tova", "min", "min_h")


def harmonic_prior(t: int) -> np.ndarray:
    """h_j = 1 / ((t - j + 1) H_t) for j = 1 .. t (returned for j - 1 = 0 .. t-1)."""
    Ht = sum(1.0 / k for k in range(1, t + 1))
    return np.array([1.0 / ((t - j + 1) * Ht) for j in range(1, t + 1)])


def row_weights(kind: str, w: int) -> np.ndarray:
    """Weight of window row i = 0 .. w-1 in the score sum."""
    if kind == "h2o":
        return np.ones(w)
    if kind in ("h2o_h", "min_h"):
        return harmonic_prior(w)
    if kind in ("tova", "min"):
        out = np.zeros(w)
        out[w - 1] = 1.0
        return out
    raise ValueError(kind)


def group_proposal_scores(kind: str, q_win: np.ndarray, k: np.ndarray, v: np.ndarray, h: int, g: int,
                          sm_scale: float, causal: bool) -> np.ndarray:
    """Score of every key of KV head h for one sequence: sum over the
    group's q-heads and window rows i of weight_i * alpha_ij, times ||v_j||
    for the "min" kinds.  q_win [Hq][w][d], k/v [n][d], float64."""
    w, d = q_win.shape[1], q_win.shape[2]
    n = k.shape[0]
    wt = row_weights(kind, w)
    pos = row_positions(n, w) if causal else None
    total = np.zeros(n)
    for qh in range(h * g, (h + 1) * g):
        att = window_attention(q_win[qh], k, v, pos, sm_scale)
        total += wt @ att["alpha"]
    if kind in ("min", "min_h"):
        total *= np.sqrt((v * v).sum(axis=1))
    return total


KNORM_SHIFT = 80.0


def knorm_scores(k: np.ndarray) -> np.ndarray:
    """exp(KNORM_SHIFT - ||k_j||) for every key row of k [n][d] (float64)."""
    return np.exp(KNORM_SHIFT - np.sqrt((k * k).sum(axis=1)))


def avg_pool(s: np.ndarray, kernel: int) -> np.ndarray:
    """s'_j = mean of s_k over |k - j| <= (kernel-1)/2, 0 <= k < n."""
    if kernel <= 1:
        return s.copy()
    r = (kernel - 1) // 2
    n = s.shape[0]
    out = np.empty_like(s)
    for j in range(n):
        lo, hi = max(0, j - r), min(n, j + r + 1)
        out[j] = s[lo:hi].sum() / (hi - lo)
    return out
