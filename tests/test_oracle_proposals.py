"""Pins of the attention-weight proposal scores ([PI] App. D and H)."""
import numpy as np
import pytest
from scipy.ndimage import uniform_filter1d

from oracle import proposals as P
from oracle.attention import window_attention, row_positions


def _case(seed, n=70, d=16, w=5, g=3, Hkv=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hkv * g, w, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    return q, k, v, g, w


def test_harmonic_prior_values():
    # H_3 = 11/6: h = [1/(3 H), 1/(2 H), 1/H] = [2/11, 3/11, 6/11]
    assert np.allclose(P.harmonic_prior(3), [2 / 11, 3 / 11, 6 / 11], rtol=0, atol=1e-15)
    assert P.harmonic_prior(1).tolist() == [1.0]
    for t in (2, 7, 32, 64):
        h = P.harmonic_prior(t)
        assert abs(h.sum() - 1.0) < 1e-14 and np.all(np.diff(h) > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_column_sums(causal):
    q, k, v, g, w = _case(1)
    for h in range(2):
        tot = {kind: P.group_proposal_scores(kind, q, k, v, h, g, 0.25, causal).sum() for kind in P.KINDS}
        assert abs(tot["h2o"] - g * w) < 1e-12       # each row's weights sum to 1
        assert abs(tot["tova"] - g) < 1e-12          # one last row per q-head
        assert abs(tot["h2o_h"] - g) < 1e-12         # prior sums to 1 per q-head


def test_value_norm_weighting():
    q, k, v, g, w = _case(2)
    v = v / np.linalg.norm(v, axis=1, keepdims=True) * 2.5   # all ||v_j|| = 2.5
    for a, b in (("min", "tova"), ("min_h", "h2o_h")):
        sa = P.group_proposal_scores(a, q, k, v, 0, g, 0.25, True)
        sb = P.group_proposal_scores(b, q, k, v, 0, g, 0.25, True)
        assert np.allclose(sa, 2.5 * sb, rtol=1e-13, atol=0)


def test_h2o_against_explicit_softmax():
    # brute force on a tiny case: plain per-row softmax loops
    q, k, v, g, w = _case(3, n=9, d=4, w=3, g=2, Hkv=1)
    n = k.shape[0]
    pos = row_positions(n, w)
    ref = np.zeros(n)
    hprior = P.harmonic_prior(w)
    for qh in range(g):
        for i in range(w):
            logits = [0.3 * float(np.dot(q[qh, i], k[j])) if j <= pos[i] else -np.inf for j in range(n)]
            m = max(logits)
            e = [np.exp(x - m) for x in logits]
            z = sum(e)
            for j in range(n):
                ref[j] += hprior[i] * e[j] / z
    got = P.group_proposal_scores("h2o_h", q, k, v, 0, g, 0.3, True)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_avg_pool():
    rng = np.random.default_rng(4)
    s = rng.random(50)
    for kern in (3, 7):
        r = kern // 2
        got = P.avg_pool(s, kern)
        assert np.allclose(got[r:-r], uniform_filter1d(s, kern, mode="constant")[r:-r], rtol=1e-13)
        assert abs(got[0] - s[:r + 1].mean()) < 1e-15 and abs(got[-1] - s[-r - 1:].mean()) < 1e-15
    assert np.array_equal(P.avg_pool(s, 1), s)


def test_knorm_closed_form_and_softmax_proposal():
    # keys r * e_1 have norm |r|: score exp(80 - |r|); rotation-invariant
    r = np.array([0.0, 1.0, -3.5, 10.0, 150.0])
    k = np.zeros((5, 8))
    k[:, 0] = r
    s = P.knorm_scores(k)
    assert np.allclose(s, np.exp(80.0 - np.abs(r)), rtol=1e-15, atol=0)
    rng = np.random.default_rng(7)
    kk = rng.standard_normal((40, 16))
    qmat, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    assert np.allclose(P.knorm_scores(kk @ qmat), P.knorm_scores(kk), rtol=1e-12, atol=0)
    # the largest scores are the smallest norms; s^(1/tau), normalised, is
    # the softmax of -||k|| / tau (Eq. 18 with the negative norm)
    from scipy.special import softmax
    from oracle.select import proposal, topk_select
    norms = np.linalg.norm(kk, axis=1)
    assert set(topk_select(P.knorm_scores(kk), 5)) == set(np.argsort(norms)[:5])
    for tau in (1.0, 0.5, 3.0):
        assert np.allclose(proposal(P.knorm_scores(kk), tau), softmax(-norms / tau), rtol=1e-12, atol=0)


def test_tova_is_the_last_row_brute_force():
    # TOVA: the last window row's softmax weights, summed over the group's
    # q-heads (a plain loop; the last row sees every key under the mask)
    q, k, v, g, w = _case(5, n=11, d=4, w=4, g=3, Hkv=1)
    n = k.shape[0]
    ref = np.zeros(n)
    for qh in range(g):
        logits = [0.7 * float(np.dot(q[qh, w - 1], k[j])) for j in range(n)]
        m = max(logits)
        e = [np.exp(x - m) for x in logits]
        for j in range(n):
            ref[j] += e[j] / sum(e)
    for causal in (True, False):
        got = P.group_proposal_scores("tova", q, k, v, 0, g, 0.7, causal)
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-16)
