"""Budgeted selection in fp64 (oracle; test infrastructure only).

Deterministic mode -- [DK] §3.3: evict the tokens with the smallest scores,
i.e. keep the B largest.  [PI] §4: top-k is a zero-variance estimator.
Reading: ties keep the lower index; NaN ranks below every number (taken
last, lowest index first); kept indices are returned in ascending order.

Sampling mode -- [PI] §4: any score is an unnormalised proposal with full
support; [PI] App. D.1: proposals may be tempered; [PI] App. F, Problem 5 and
Algorithm 2: binary search over m in [0, 10^12] for an m whose expected
number of distinct draws, E[J(m)] = sum_i 1 - (1 - pi_i)^m (Eq. 24), is
within 0.5 of the target; [PI] §6, Eq. 10: importance weights tempered as
exp(log(w) / tau).
Readings:
 * proposal log pi~_j = log(max(s_j, 2^-126)) / tau (pi ~ s^(1/tau)); NaN
   scores are treated as 2^-126;
 * [PI] App. D.1 mixing with the uniform, pi' = alpha pi + (1 - alpha) / n,
   is applied to the tempered, normalised proposal (mix = alpha; 1 = none);
   with mixing the Gumbel keys use log pi'_j;
 * the target is the kept count, j* = B;
 * the kept set is B draws without replacement via Gumbel keys
   kappa_j = log pi~_j - log(-log u_j), u_j from Philox (see philox.py);
   ties in kappa keep the lower index;
 * q_j = 1 - (1 - pi_j)^m, the probability that j appears in m draws with
   replacement (Eq. 25), with m from Algorithm 2; the logit bias of a kept
   entry is -log(q_j) / tau_w (weight 1/q_j tempered as in Eq. 10);
 * B >= n keeps everything with bias 0 and reports m = 0;
 * if no m <= 10^12 reaches the band (E(10^12) < B - 0.5), m = 10^12 and the
   status is "not converged" (the Remark after Algorithm 2).
 * literal estimator ([PI] §4, Algorithm 1, Eq. 10): m draws with
   replacement by inverse CDF, draw k from u_k on the Philox counter
   (k, h, s, 1); kept = drawn at least once; bias log(c_j / (m pi_j)) / tau_w;
 * soft per-sequence budget ([PI] App. F.1): one m for all KV heads of a
   sequence, found by Algorithm 2 on the heads' mean E (Eq. 33); head h then
   keeps B_h = floor(E_h(m) + 0.5) entries (its expected number of distinct
   draws, clamped to the sequence length and the caller's capacity), chosen
   and weighted as above; a head that keeps every entry has bias 0.
E(m) is evaluated as sum(-expm1(m * log1p(-pi))), the same closed form
written to keep precision for tiny pi.

Pinned by: Monte-Carlo draws with replacement (E[J(m)]); monotonicity and
unit-bounded increments (Eq. 27-31); the worked example of [PI] App. F.1
(tests/golden); exact without-replacement inclusion probabilities on tiny
n (Gumbel keys); sum q_j = E[J(m)].
"""
from __future__ import annotations

import numpy as np

from .philox import uniform53, uniform53_draws

FLT_MIN = 2.0 ** -126
ALPHA_MAX = 10 ** 12
STATUS_OK = 0
STATUS_NOCONV = 5


def topk_select(s: np.ndarray, B: int) -> np.ndarray:
    """Indices of the B largest entries of s (ties -> lower index, NaN last),
    sorted ascending."""
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    B = min(int(B), n)
    if B <= 0:
        return np.zeros(0, dtype=np.int64)
    isnan = np.isnan(s)
    key = np.where(isnan, 0.0, s)
    order = np.lexsort((np.arange(n), -key, isnan))   # last key is primary
    return np.sort(order[:B])


def proposal_log(s: np.ndarray, tau: float) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    return np.log(np.fmax(s, FLT_MIN)) / tau


def proposal(s: np.ndarray, tau: float, mix: float = 1.0) -> np.ndarray:
    """Normalised tempered proposal, mixed with the uniform when mix < 1."""
    lp = proposal_log(s, tau)
    mx = lp.max()
    lse = mx + np.log(np.exp(lp - mx).sum())
    pi = np.exp(lp - lse)
    if mix < 1.0:
        pi = mix * pi + (1.0 - mix) / pi.shape[0]
    return pi


def expected_distinct(pi: np.ndarray, m) -> float:
    """E[J(m)] = sum_i 1 - (1 - pi_i)^m ([PI] App. F, Eq. 24)."""
    return float(np.sum(-np.expm1(float(m) * np.log1p(-pi))))


def expected_samples_search(pi: np.ndarray, target: float, eps: float = 0.5):
    """[PI] App. F, Algorithm 2: integer binary search over [0, 10^12].
    Returns (m, status)."""
    low, high = 0, ALPHA_MAX
    L = np.log1p(-pi)
    while low <= high:
        mid = (low + high) // 2
        e = float(np.sum(-np.expm1(float(mid) * L)))
        if abs(e - target) <= eps:
            return mid, STATUS_OK
        if e < target:
            low = mid + 1
        else:
            high = mid - 1
    return ALPHA_MAX, STATUS_NOCONV


def inclusion_prob(pi: np.ndarray, m) -> np.ndarray:
    """q_j = 1 - (1 - pi_j)^m ([PI] App. F, Eq. 25)."""
    return -np.expm1(float(m) * np.log1p(-pi))


def gumbel_keys(logp: np.ndarray, seed: int, s: int, h: int) -> np.ndarray:
    u = uniform53(seed, s, h, np.arange(logp.shape[0]))
    return logp - np.log(-np.log(u))


def sample_select(s: np.ndarray, B: int, tau: float, tau_w: float, seed: int, seq: int, head: int,
                  mix: float = 1.0):
    """Sampling-mode selection for one (sequence, KV head).
    Returns (idx ascending, bias fp64, m, status)."""
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    if B >= n:
        return np.arange(n), np.zeros(n), 0, STATUS_OK
    if B <= 0:
        return np.zeros(0, dtype=np.int64), np.zeros(0), 0, STATUS_OK
    pi = proposal(s, tau, mix)
    lp = proposal_log(s, tau) if mix >= 1.0 else np.log(pi)
    m, status = expected_samples_search(pi, float(B))
    kappa = gumbel_keys(lp, seed, seq, head)
    order = np.lexsort((np.arange(n), -kappa))
    idx = np.sort(order[:B])
    q = inclusion_prob(pi[idx], m)
    bias = -np.log(q) / tau_w
    return idx, bias, m, status


def global_search(pis, target: float, eps: float = 0.5):
    """[PI] App. F.1, Eq. 33: Algorithm 2 with E(m) replaced by the mean over
    the heads, (1/H) sum_h E_h(m), all heads sharing one m.  Returns (m, status)."""
    Ls = [np.log1p(-pi) for pi in pis]
    H = len(pis)
    low, high = 0, ALPHA_MAX
    while low <= high:
        mid = (low + high) // 2
        e = sum(float(np.sum(-np.expm1(float(mid) * L))) for L in Ls) / H
        if abs(e - target) <= eps:
            return mid, STATUS_OK
        if e < target:
            low = mid + 1
        else:
            high = mid - 1
    return ALPHA_MAX, STATUS_NOCONV


def global_kept_count(pi: np.ndarray, m, cap: int) -> int:
    """Kept entries of one head under the shared m: its expected number of
    distinct draws rounded half up, clamped to [0, min(n, cap)]."""
    e = expected_distinct(pi, m)
    return int(min(max(np.floor(e + 0.5), 0), min(pi.shape[0], cap)))


def global_sample_select(scores_heads, B: int, cap: int, tau: float, tau_w: float, seed: int, seq: int,
                         mix: float = 1.0, m=None):
    """Sampling selection of one sequence under a per-sequence soft budget
    ([PI] §7 and App. F.1): one m for all heads with mean expected kept count
    B (Eq. 33); head h keeps its own expected count B_h (global_kept_count)
    by the same Gumbel top-B_h and weights as sample_select.  With m given,
    the search is skipped (any m in the band is a valid result of it).
    Returns ([(idx, bias)] per head, [B_h], m, status)."""
    scores_heads = [np.asarray(sc, dtype=np.float64) for sc in scores_heads]
    n = scores_heads[0].shape[0]
    H = len(scores_heads)
    if B >= n:
        return [(np.arange(n), np.zeros(n)) for _ in range(H)], [n] * H, 0, STATUS_OK
    if B <= 0:
        return [(np.zeros(0, dtype=np.int64), np.zeros(0)) for _ in range(H)], [0] * H, 0, STATUS_OK
    pis = [proposal(sc, tau, mix) for sc in scores_heads]
    status = STATUS_OK
    if m is None:
        m, status = global_search(pis, float(B))
    out, kept = [], []
    for h, (sc, pi) in enumerate(zip(scores_heads, pis)):
        Bh = global_kept_count(pi, m, cap)
        kept.append(Bh)
        if Bh >= n:
            out.append((np.arange(n), np.zeros(n)))
            continue
        lp = proposal_log(sc, tau) if mix >= 1.0 else np.log(pi)
        kappa = gumbel_keys(lp, seed, seq, h)
        idx = np.sort(np.lexsort((np.arange(n), -kappa))[:Bh])
        q = inclusion_prob(pi[idx], m)
        out.append((idx, -np.log(q) / tau_w))
    return out, kept, m, status


def draw_counts(pi: np.ndarray, m: int, seed: int, seq: int, head: int) -> np.ndarray:
    """[PI] §4: m draws with replacement from pi; draw k takes u_k (Philox
    counter (k, head, seq, 1)) and lands on the first entry whose cumulative
    probability exceeds u_k times the total.  Returns the counts c_j."""
    cdf = np.cumsum(pi)
    u = uniform53_draws(seed, seq, head, np.arange(int(m)))
    j = np.minimum(np.searchsorted(cdf, u * cdf[-1], side="right"), pi.shape[0] - 1)
    return np.bincount(j, minlength=pi.shape[0])


def literal_select(s: np.ndarray, m: int, cap: int, tau: float, tau_w: float, seed: int, seq: int, head: int,
                   mix: float = 1.0):
    """[PI] §4-§6 as the pages state it: the kept set is the entries drawn at
    least once in m draws with replacement from pi, and entry j carries the
    tempered importance weight exp(log(c_j / (m pi_j)) / tau_w) (Algorithm 1
    step 4 and Eq. 10), i.e. the logit bias log(c_j / (m pi_j)) / tau_w.
    Returns (idx ascending, bias, J = number kept); at most cap are returned
    (the lowest indices) when J > cap."""
    pi = proposal(s, tau, mix)
    c = draw_counts(pi, m, seed, seq, head)
    idx = np.nonzero(c)[0]
    J = idx.shape[0]
    idx = idx[:cap]
    bias = (np.log(c[idx].astype(np.float64)) - np.log(float(m)) - np.log(pi[idx])) / tau_w
    return idx, bias, J


def select_workload(scores: np.ndarray, seq_off, budgets, mode: str, tau: float = 1.0,
                    tau_w: float = 1.0, seed: int = 0, heads=None, mix: float = 1.0):
    """Selection for a ragged batch: scores [Hkv][T] -> idx/bias [Hkv][sum B]
    (sequence-relative indices), m [S][Hkv], status [S][Hkv]."""
    Hkv = scores.shape[0]
    S = len(seq_off) - 1
    budgets = [int(b) for b in budgets]
    bud_off = np.concatenate([[0], np.cumsum(budgets)]).astype(np.int64)
    idx = np.full((Hkv, int(bud_off[-1])), -1, dtype=np.int64)
    bias = np.zeros((Hkv, int(bud_off[-1])))
    m_out = np.zeros((S, Hkv))
    st = np.zeros((S, Hkv), dtype=np.int64)
    for h in (range(Hkv) if heads is None else heads):
        for s in range(S):
            a, b = int(seq_off[s]), int(seq_off[s + 1])
            Bs = min(budgets[s], b - a)
            if mode == "topk":
                ii = topk_select(scores[h, a:b], Bs)
                bb = np.zeros(len(ii))
                m, status = 0, STATUS_OK
            else:
                ii, bb, m, status = sample_select(scores[h, a:b], Bs, tau, tau_w, seed, s, h, mix)
            idx[h, bud_off[s]:bud_off[s] + len(ii)] = ii
            bias[h, bud_off[s]:bud_off[s] + len(ii)] = bb
            m_out[s, h] = m
            st[s, h] = status
    return idx, bias, m_out, st
