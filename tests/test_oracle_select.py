"""Pins of oracle/select.py and oracle/philox.py."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import (topk_select, proposal, expected_distinct, expected_samples_search,
                    inclusion_prob, sample_select, philox4x64_10, uniform53)
from oracle.select import STATUS_NOCONV, select_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- top-k
def _topk_bruteforce(s, B):
    # pure-python ranking: larger value first, NaN after every number,
    # ties -> lower index
    def rank_key(j):
        x = s[j]
        return (1, 0.0, j) if np.isnan(x) else (0, -x, j)
    order = sorted(range(len(s)), key=rank_key)
    return sorted(order[:B])


@pytest.mark.parametrize("seed", range(5))
def test_topk_against_python_sort(seed):
    rng = np.random.default_rng(seed)
    s = np.round(rng.standard_normal(300), 1).astype(np.float32)   # many exact ties
    s[rng.choice(300, 5, replace=False)] = np.nan
    s[rng.choice(300, 3, replace=False)] = -np.inf
    for B in (0, 1, 17, 150, 295, 300):
        assert list(topk_select(s, B)) == _topk_bruteforce(list(s.astype(float)), B)


def test_topk_ties_lower_index():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0, 0.5])
    assert list(topk_select(s, 2)) == [1, 2]
    assert list(topk_select(s, 4)) == [1, 2, 3, 4]
    assert list(topk_select(np.array([np.nan, 1.0, np.nan]), 2)) == [0, 1]


# ---------------------------------------------------------------- E[J(m)]
@pytest.mark.parametrize("seed", range(3))
def test_expected_distinct_monte_carlo(seed):
    # [PI] App. F, Eq. 24 against direct simulation of m draws with replacement
    rng = np.random.default_rng(seed)
    n = 24
    pi = rng.dirichlet(np.full(n, 0.3))
    for m in (1, 5, 30, 200):
        trials = 100000
        draws = rng.choice(n, size=(trials, m), p=pi)
        distinct = np.array([len(np.unique(r)) for r in draws[:2000]])
        # full trial count via a vectorised membership count
        seen = np.zeros((trials, n), dtype=bool)
        seen[np.repeat(np.arange(trials), m), draws.ravel()] = True
        distinct = seen.sum(1)
        sigma = distinct.std() / np.sqrt(trials)
        assert abs(distinct.mean() - expected_distinct(pi, m)) < 4 * sigma + 1e-12


def test_expected_distinct_monotone_unit_increments():
    # [PI] App. F, Eq. 27-31: nondecreasing in m, increments at most 1, and
    # the increment equals sum_i (1 - pi_i)^m pi_i
    rng = np.random.default_rng(9)
    pi = rng.dirichlet(np.full(200, 0.2))
    e = np.array([expected_distinct(pi, m) for m in range(0, 400)])
    inc = np.diff(e)
    assert np.all(inc >= -1e-12) and np.all(inc <= 1 + 1e-12)
    closed = np.array([np.sum((1 - pi) ** m * pi) for m in range(0, 399)])
    assert np.allclose(inc, closed, atol=1e-10)


@pytest.mark.parametrize("target", [1, 10, 57, 150, 199])
def test_algorithm2_lands_in_band(target):
    rng = np.random.default_rng(target)
    pi = rng.dirichlet(np.full(200, 0.5))
    m, st = expected_samples_search(pi, float(target))
    assert st == 0
    assert abs(expected_distinct(pi, m) - target) <= 0.5


def test_algorithm2_not_converged_flag():
    pi = np.full(100, 1e-16)
    pi[0] = 1 - 99e-16
    m, st = expected_samples_search(pi, 90.0)
    assert st == STATUS_NOCONV and m == 10 ** 12


def test_worked_example_from_pages():
    # [PI] App. F.1 worked example, pi as printed
    ex = json.load(open(os.path.join(GOLDEN, "ccp_worked_example.json")))
    pi = np.array(ex["pi"])
    n = ex["n"]
    comp = 1 - expected_distinct(pi, ex["m_example"]) / n
    assert abs(comp - ex["compression_at_m_example"]) < ex["compression_tolerance"]
    for t in ex["targets"]:
        band = [m for m in range(0, 20000) if abs(expected_distinct(pi, m) - t["kept"]) <= 0.5]
        assert band, t
        lo, hi = min(band), max(band)
        assert lo <= t["m_page"] <= hi, (t, lo, hi)
        m, st = expected_samples_search(pi, float(t["kept"]))
        assert lo <= m <= hi and st == 0


# ---------------------------------------------------------------- Philox
def test_philox_matches_numpy_library():
    # numpy.random.Philox is Philox-4x64-10; it increments the counter before
    # producing a block, so counter c-1 yields the block of counter c.
    rng = np.random.default_rng(77)
    for _ in range(50):
        c = [int(x) for x in rng.integers(1, 2 ** 63, size=4, dtype=np.int64)]
        key = [int(x) for x in rng.integers(0, 2 ** 63, size=2, dtype=np.int64)]
        mine = philox4x64_10(*[np.uint64(x) for x in c], np.uint64(key[0]), np.uint64(key[1]))
        ref = np.random.Philox(counter=[c[0] - 1] + c[1:], key=key).random_raw(4)
        assert [int(a) for a in mine] == [int(b) for b in ref]
    # vectorised evaluation equals per-element evaluation
    js = np.arange(1000, dtype=np.uint64)
    vec = philox4x64_10(js, np.uint64(3), np.uint64(2), np.uint64(0), np.uint64(99), np.uint64(0))[0]
    one = [int(philox4x64_10(np.uint64(j), np.uint64(3), np.uint64(2), np.uint64(0),
                             np.uint64(99), np.uint64(0))[0]) for j in (0, 1, 999)]
    assert [int(vec[0]), int(vec[1]), int(vec[999])] == one


def test_uniform53_reads_the_philox_stream_in_order():
    # Token j takes word j mod 4 of counter block floor(j / 4): a head's
    # tokens read numpy's Philox output stream word after word.  numpy starts
    # at the block after its counter, so counter (0, h, s, 0) streams the
    # words of tokens 4, 5, 6, ...
    for seed, s, h in ((7, 0, 0), (2005, 3, 5), (2 ** 40 + 1, 7, 1)):
        K = 300
        raw = np.random.Philox(counter=[0, h, s, 0], key=[seed, 0]).random_raw(4 * K)
        ref = ((raw >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
        mine = uniform53(seed, s, h, np.arange(4, 4 * K + 4))
        assert np.array_equal(mine, ref)
        # the first block, word by word, from the block function
        words = philox4x64_10(np.uint64(0), np.uint64(h), np.uint64(s), np.uint64(0),
                              np.uint64(seed), np.uint64(0))
        first = [((int(w) >> 11) + 0.5) * 2.0 ** -53 for w in words]
        assert list(uniform53(seed, s, h, np.arange(4))) == first


def test_uniform_chi_square():
    u = uniform53(12345, 0, 0, np.arange(1 << 20))
    assert u.min() > 0 and u.max() < 1
    counts = np.bincount((u * 65536).astype(np.int64), minlength=65536)
    chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
    p = stats.chi2.sf(chi2, 65535)
    assert 1e-4 < p < 1 - 1e-4


# ---------------------------------------------------------------- Gumbel top-B
def _exact_inclusion(pi, B):
    """P(j among the first B draws of sequential sampling without
    replacement), by enumerating ordered prefixes."""
    n = len(pi)
    inc = np.zeros(n)
    for perm in itertools.permutations(range(n), B):
        p, rem = 1.0, 1.0
        for j in perm:
            p *= pi[j] / rem
            rem -= pi[j]
        for j in perm:
            inc[j] += p
    return inc


@pytest.mark.parametrize("n,B", [(4, 1), (5, 2), (6, 3)])
def test_gumbel_topB_is_sampling_without_replacement(n, B):
    # [PI] §4: the kept set is B draws without replacement from the tempered
    # proposal.  The oracle's own gumbel_keys, evaluated for 2e5 seeds at
    # once (its Philox counter takes the seed as a broadcast array), must
    # give inclusion frequencies of its top B equal to the exact inclusion
    # probabilities of sequential draws without replacement (enumerated).
    from oracle.select import gumbel_keys, proposal_log
    rng = np.random.default_rng(n * 10 + B)
    s = rng.uniform(0.05, 1.0, size=n)
    tau = 0.5
    pi = proposal(s, tau)
    exact = _exact_inclusion(pi, B)
    seeds = 200000
    kappa = gumbel_keys(proposal_log(s, tau), np.arange(seeds, dtype=np.uint64)[:, None], 0, 0)
    assert kappa.shape == (seeds, n)
    top = np.argsort(-kappa, axis=1, kind="stable")[:, :B]
    freq = np.bincount(top.ravel(), minlength=n) / seeds
    sigma = np.sqrt(exact * (1 - exact) / seeds)
    assert np.all(np.abs(freq - exact) <= 4 * sigma + 1e-9), (freq, exact)


def test_sample_select_kept_set_law():
    # The same law through sample_select itself (one call per seed): its
    # kept sets over 12000 seeds have the exact without-replacement
    # inclusion probabilities, and each one is the top B of that seed's keys.
    from oracle.select import gumbel_keys, proposal_log
    n, B, tau = 5, 2, 0.5
    s = np.random.default_rng(52).uniform(0.05, 1.0, size=n)
    exact = _exact_inclusion(proposal(s, tau), B)
    seeds = 12000
    freq = np.zeros(n)
    lp = proposal_log(s, tau)
    for sd in range(seeds):
        idx, _, _, st = sample_select(s, B, tau, 1.0, sd, 0, 0)
        assert st == 0 and len(idx) == B and np.all(np.diff(idx) > 0)
        freq[idx] += 1
        if sd < 200:
            kap = gumbel_keys(lp, sd, 0, 0)
            assert set(idx) == set(np.argsort(-kap, kind="stable")[:B])
    freq /= seeds
    sigma = np.sqrt(exact * (1 - exact) / seeds)
    assert np.all(np.abs(freq - exact) <= 4 * sigma + 1e-9), (freq, exact)


def test_sample_select_weight_temperature():
    # [PI] §6 Eq. 10: the importance weight w is tempered as exp(log(w) /
    # tau_w).  The weight of a kept entry is 1/q_j with q_j the chance that
    # j shows up in m draws with replacement; estimate q_j by simulating
    # those draws, and check bias * tau_w = -log q_j for several tau_w
    # (tau_w = inf would give every entry weight 1).
    rng = np.random.default_rng(17)
    n, B, tau = 12, 4, 0.8
    s = rng.uniform(0.01, 1.0, size=n)
    pi = proposal(s, tau)
    biases = {}
    for tw in (1.0, 0.5, 2.0, 3.0):
        idx, bias, m, st = sample_select(s, B, tau, tw, 9, 0, 0)
        assert st == 0
        biases[tw] = (idx, bias, m)
    idx1, b1, m1 = biases[1.0]
    for tw, (idx, bias, m) in biases.items():
        assert np.array_equal(idx, idx1) and m == m1   # tau_w changes weights only
        assert np.allclose(bias * tw, b1, rtol=1e-13, atol=0)
    trials = 200000
    draws = rng.choice(n, size=(trials, int(m1)), p=pi)
    seen = np.zeros((trials, n), dtype=bool)
    seen[np.arange(trials)[:, None], draws] = True
    q_mc = seen.mean(axis=0)[idx1]
    sig = np.sqrt(q_mc * (1 - q_mc) / trials)
    q_or = np.exp(-b1)
    assert np.all(np.abs(q_or - q_mc) <= 4 * sig + 1e-9), (q_or, q_mc)


# ---------------------------------------------------------------- weights
def test_inclusion_identity_and_full_budget():
    rng = np.random.default_rng(5)
    s = np.exp(rng.standard_normal(500) * 2).astype(np.float32)
    pi = proposal(s, 0.5)
    m, _ = expected_samples_search(pi, 50.0)
    assert np.isclose(inclusion_prob(pi, m).sum(), expected_distinct(pi, m), rtol=1e-13)
    idx, bias, m_all, st = sample_select(s, 500, 0.5, 1.0, 1, 0, 0)
    assert list(idx) == list(range(500)) and np.all(bias == 0.0)
    idx, bias, _, _ = sample_select(s, 50, 0.5, 1.0, 1, 0, 0)
    q = inclusion_prob(pi[idx], m)
    assert np.allclose(bias, -np.log(q))
    assert np.all(bias >= 0)


def test_select_workload_ragged_layout():
    rng = np.random.default_rng(8)
    lens = [30, 50]
    off = np.array([0, 30, 80])
    sc = rng.random((2, 80)).astype(np.float32)
    idx, bias, m, st = select_workload(sc, off, [3, 5], "topk")
    assert idx.shape == (2, 8)
    for h in range(2):
        assert list(idx[h, :3]) == list(topk_select(sc[h, :30], 3))
        assert list(idx[h, 3:]) == list(topk_select(sc[h, 30:], 5))


def test_uniform_mixing_of_the_proposal():
    from oracle import select as S
    # [PI] App. D.1: pi' = alpha pi + (1 - alpha) / n sums to one and has
    # full support; alpha = 0 is the uniform, where E[J(m)] = n (1 - (1 -
    # 1/n)^m) and every kept entry carries the same bias
    rng = np.random.default_rng(3)
    s = rng.exponential(size=300) ** 4
    n = s.shape[0]
    pi = S.proposal(s, 0.7)
    for a in (0.0, 0.3, 0.9):
        pm = S.proposal(s, 0.7, mix=a)
        assert abs(pm.sum() - 1.0) < 1e-12
        assert pm.min() >= (1 - a) / n * (1 - 1e-12)
        assert np.allclose(pm, a * pi + (1 - a) / n, rtol=1e-14, atol=0)
    u = S.proposal(s, 0.7, mix=0.0)
    for m in (10, 250, 4000):
        assert abs(S.expected_distinct(u, m) - n * (1 - (1 - 1 / n) ** m)) < 1e-9
    idx, bias, m, st = S.sample_select(s, 60, 0.7, 1.0, 11, 0, 0, mix=0.0)
    assert st == S.STATUS_OK and len(idx) == 60 and np.ptp(bias) < 1e-12
    # ... and the kept set ignores the scores: the B largest Gumbel noises
    g = S.gumbel_keys(np.zeros(n), 11, 0, 0)
    assert np.array_equal(idx, np.sort(np.argsort(-g, kind="stable")[:60]))
    # mix = 1 is the unmixed selection, bit for bit
    a = S.sample_select(s, 60, 0.7, 1.0, 11, 0, 0)
    b = S.sample_select(s, 60, 0.7, 1.0, 11, 0, 0, mix=1.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]
    # mixing raises the inclusion of the least likely entries
    idx1, bias1, m1, _ = S.sample_select(s, 60, 0.7, 1.0, 11, 0, 0, mix=0.5)
    q0 = S.inclusion_prob(pi, S.expected_samples_search(pi, 60)[0])
    q1 = S.inclusion_prob(S.proposal(s, 0.7, 0.5), m1)
    lo = np.argsort(pi)[:50]
    assert np.all(q1[lo] > q0[lo])


# ------------------------------------------------- soft per-sequence budget
def _heads(seed, n=400, H=4):
    rng = np.random.default_rng(seed)
    # head 0 peaked, head H-1 nearly flat, others in between
    return [rng.exponential(size=n) ** (6.0 - 1.5 * h) for h in range(H)]


def test_global_search_is_algorithm2_on_the_head_mean():
    from oracle import select as S
    heads = _heads(1)
    pis = [S.proposal(sc, 1.0) for sc in heads]
    for B in (20, 60, 150):
        m, st = S.global_search(pis, float(B))
        mean_e = np.mean([S.expected_distinct(pi, m) for pi in pis])
        assert st == S.STATUS_OK and abs(mean_e - B) <= 0.5
        # brute force: the band of integer m is non-empty and contains m
        ms = np.arange(max(0, m - 50), m + 51)
        e = np.array([np.mean([S.expected_distinct(pi, k) for pi in pis]) for k in ms])
        assert np.all(np.diff(e) >= 0) and np.all(np.diff(e) <= 1 + 1e-12)   # Eq. 27-31 per head
    # one head: the per-head search
    for B in (20, 60):
        assert S.global_search([pis[2]], float(B)) == S.expected_samples_search(pis[2], float(B))


def test_global_select_one_head_is_sample_select():
    from oracle import select as S
    sc = _heads(2)[1]
    out, kept, m, st = S.global_sample_select([sc], 50, 400, 0.7, 1.3, 9, 2)
    idx, bias, m1, st1 = S.sample_select(sc, 50, 0.7, 1.3, 9, 2, 0)
    assert m == m1 and kept == [50]
    assert np.array_equal(out[0][0], idx) and np.allclose(out[0][1], bias, rtol=1e-15, atol=0)


def test_global_select_adapts_per_head_budget():
    from oracle import select as S
    heads = _heads(3)
    H, B = len(heads), 60
    out, kept, m, st = S.global_sample_select(heads, B, 400, 1.0, 1.0, 4, 0)
    pis = [S.proposal(sc, 1.0) for sc in heads]
    # each head keeps its rounded expected count; they average to B
    for pi, k in zip(pis, kept):
        assert abs(k - S.expected_distinct(pi, m)) <= 0.5
    assert abs(np.mean(kept) - B) <= 0.5 + 0.5
    assert kept[0] < kept[-1]                       # the peaked head keeps fewer
    for (idx, bias), k, h in zip(out, kept, range(H)):
        assert len(idx) == k and np.all(np.diff(idx) > 0)
    # capacity clamps a head's count
    out2, kept2, m2, _ = S.global_sample_select(heads, B, 70, 1.0, 1.0, 4, 0)
    assert m2 == m and max(kept2) <= 70


def test_global_expected_count_monte_carlo():
    # draws with replacement under the shared m: the mean distinct count
    # over heads matches the target B (Eq. 33 by linearity)
    from oracle import select as S
    heads = _heads(5, n=200, H=3)
    pis = [S.proposal(sc, 1.0) for sc in heads]
    B = 40
    m, st = S.global_search(pis, float(B))
    rng = np.random.default_rng(0)
    trials = 400
    tot = 0.0
    for _ in range(trials):
        tot += np.mean([len(np.unique(rng.choice(len(pi), size=int(m), p=pi))) for pi in pis])
    assert abs(tot / trials - B) < 0.5 + 4 * 1.0 / np.sqrt(trials) * 3


# ------------------------------------------------------- literal estimator
def test_draw_counts_brute_force_and_frequencies():
    from oracle import select as S
    from oracle.philox import uniform53_draws
    rng = np.random.default_rng(8)
    pi = rng.exponential(size=7)
    pi /= pi.sum()
    m = 3000
    c = S.draw_counts(pi, m, 5, 1, 2)
    assert c.sum() == m
    # brute force: walk the cumulative sum for each draw
    u = uniform53_draws(5, 1, 2, np.arange(m))
    ref = np.zeros(7, dtype=np.int64)
    for x in u:
        acc, t = 0.0, x * np.cumsum(pi)[-1]
        for j in range(7):
            acc = np.cumsum(pi)[j]
            if acc > t:
                ref[j] += 1
                break
        else:
            ref[6] += 1
    assert np.array_equal(c, ref)
    # the frequencies follow pi (chi-square, 6 dof, far from the tail)
    big = S.draw_counts(pi, 200000, 6, 0, 0)
    chi2 = ((big - 200000 * pi) ** 2 / (200000 * pi)).sum()
    assert chi2 < 30.0


def test_literal_estimator_kept_count_and_unbiased_weights():
    # E[J] = E(m) (Eq. 24) and, with tau_w = 1, sum_j c_j/(m pi_j) f_j is an
    # unbiased estimate of sum_j f_j (importance sampling, Algorithm 1)
    from oracle import select as S
    rng = np.random.default_rng(9)
    s = rng.exponential(size=60) ** 3
    pi = S.proposal(s, 1.0)
    f = rng.standard_normal(60)
    m = 40
    Js, est = [], []
    for seed in range(600):
        idx, bias, J = S.literal_select(s, m, 60, 1.0, 1.0, seed, 0, 0)
        Js.append(J)
        est.append(np.sum(np.exp(bias) * f[idx]))
        assert np.allclose(np.exp(bias), S.draw_counts(pi, m, seed, 0, 0)[idx] / (m * pi[idx]), rtol=1e-12)
    E = S.expected_distinct(pi, m)
    assert abs(np.mean(Js) - E) < 4 * np.std(Js) / np.sqrt(len(Js)) + 1e-9
    assert abs(np.mean(est) - f.sum()) < 4 * np.std(est) / np.sqrt(len(est))
    # the weight temperature divides the log weight
    i1, b1, _ = S.literal_select(s, m, 60, 1.0, 2.0, 3, 0, 0)
    i2, b2, _ = S.literal_select(s, m, 60, 1.0, 1.0, 3, 0, 0)
    assert np.array_equal(i1, i2) and np.allclose(b1, b2 / 2.0, rtol=1e-14)
    # capacity keeps the lowest indices and reports the full count
    i3, b3, J3 = S.literal_select(s, m, 5, 1.0, 1.0, 3, 0, 0)
    assert J3 == len(i2) and np.array_equal(i3, i2[:5])
