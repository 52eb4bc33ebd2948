"""Compaction and decode-time corrected attention in fp64 (oracle; test
infrastructure only).

[PI] §2, Eq. 3: evicted attention keeps the rows of K and V indexed by the
kept set I; [PI] §5: an entry is evicted iff its count is zero, and evicted
entries are ignored.
[PI] §5, Definition 3-4 and Algorithm 1: self-normalised importance sampling
over the retained history with weights w_i, plus the exact contribution of
tokens generated after eviction (weight 1):
    o = (sum_hist w_i p~_i v_i + sum_new p~_i v_i) / (sum_hist w_i p~_i + sum_new p~_i)
which equals a softmax whose logits carry the additive bias log w_i.
[PI] §5 (GQA): one proposal (hence one bias per entry) per KV head, shared by
the query heads of the group.

Reading: the weight of a kept entry is exp(bias) with bias = -log(q)/tau_w
from the selection step; appended entries have bias 0; the same logit scale
as the scorer is used.

Pinned by: B = n with bias 0 reproduces exact attention over the full cache
plus appended tokens (torch fp64 SDPA), a literal transcription of
Algorithm 1 agrees with the biased softmax, bias 0 on an evicted cache is
the conditional expectation of [PI] Eq. 6, and with-replacement counts with
weights c/(m pi) converge to exact attention as m grows ([PI] §5,
Proposition).
"""
from __future__ import annotations

import numpy as np


def compact(k, v, idx, bias, seq_off, bud_off, cap_off):
    """k_c[h][cap_off[s] + r] = k[h][seq_off[s] + idx[h][bud_off[s] + r]] for
    r < B_s (same for v and bias).  Slots r >= B_s are returned as zeros."""
    Hkv, _, d = k.shape
    S = len(seq_off) - 1
    C = int(cap_off[-1])
    k_c = np.zeros((Hkv, C, d), dtype=k.dtype)
    v_c = np.zeros((Hkv, C, d), dtype=v.dtype)
    b_c = np.zeros((Hkv, C), dtype=np.float64)
    for h in range(Hkv):
        for s in range(S):
            B = int(bud_off[s + 1] - bud_off[s])
            rows = seq_off[s] + idx[h, bud_off[s]:bud_off[s] + B]
            k_c[h, cap_off[s]:cap_off[s] + B] = k[h, rows]
            v_c[h, cap_off[s]:cap_off[s] + B] = v[h, rows]
            b_c[h, cap_off[s]:cap_off[s] + B] = bias[h, bud_off[s]:bud_off[s] + B]
    return k_c, v_c, b_c


def decode_attention(q, k_c, v_c, bias_c, cap_off, cache_len, Hq: int, sm_scale: float):
    """o[s][qh] = sum_r softmax_r(sm_scale <q, k_r> + bias_r) v_r over the
    first cache_len[s] slots of sequence s of KV head qh // (Hq/Hkv).
    q [S][Hq][d] float64; k_c/v_c [Hkv][C][d]; bias_c [Hkv][C]."""
    S = q.shape[0]
    Hkv = k_c.shape[0]
    g = Hq // Hkv
    d = q.shape[2]
    out = np.zeros((S, Hq, d))
    for s in range(S):
        a = int(cap_off[s])
        L = int(cache_len[s])
        for qh in range(Hq):
            h = qh // g
            kk = k_c[h, a:a + L]
            vv = v_c[h, a:a + L]
            logit = sm_scale * (kk @ q[s, qh]) + bias_c[h, a:a + L]
            mx = logit.max()
            e = np.exp(logit - mx)
            out[s, qh] = (e / e.sum()) @ vv
    return out


def decode_alg1_literal(q, k_hist, v_hist, w_hist, k_new, v_new, sm_scale: float):
    """[PI] Algorithm 1 for one query: history entries with weights w_i,
    decode-time entries exact.  Returns the corrected attention vector."""
    p_hist = np.exp(sm_scale * (k_hist @ q))
    p_new = np.exp(sm_scale * (k_new @ q)) if len(k_new) else np.zeros(0)
    z_hat = np.sum(w_hist * p_hist)
    z_new = np.sum(p_new)
    mu_hat = (w_hist * p_hist) @ v_hist
    mu_new = p_new @ v_new if len(k_new) else np.zeros(q.shape[0])
    return (mu_hat + mu_new) / (z_hat + z_new)
