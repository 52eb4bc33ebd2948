"""Pins of the partition-conserving merge oracle (§4.1 of the
information-theoretic eviction page)."""
import numpy as np

from oracle import merge as M


def test_duplicates_merge_and_conserve_the_normaliser():
    # evicted entries that duplicate retained keys merge into them, and the
    # merged cache's normaliser sum_r m_r exp(q.k_r) equals the full one
    rng = np.random.default_rng(1)
    d, nk = 16, 6
    base = rng.standard_normal((nk, d))
    dup_of = rng.integers(0, nk, size=20)
    k = np.concatenate([base, base[dup_of]])
    kept = np.arange(nk)
    cnt = M.merge_counts(k, kept, 0.99)
    assert np.array_equal(cnt, np.bincount(dup_of, minlength=nk))
    q = rng.standard_normal(d)
    full = np.exp(k @ q).sum()
    merged = np.sum(np.exp(M.merged_bias(np.zeros(nk), cnt)) * np.exp(base @ q))
    assert abs(merged - full) < 1e-12 * full


def test_orthogonal_keys_never_merge_and_threshold_is_strict():
    d = 8
    k = np.eye(d)                     # every pair orthogonal
    kept = np.array([0, 2, 4])
    t, c = M.merge_targets(k, kept, 0.0)
    assert np.all(t == -1)            # similarity 0 is not above 0
    ev = np.setdiff1d(np.arange(d), kept)
    assert np.all(c[ev] == 0.0) and np.all(np.isneginf(c[kept]))
    # scaled copies have similarity 1 (norms do not matter); equal
    # similarities go to the lowest kept position
    k2 = np.array([[1.0, 0], [2.0, 0], [0, 1.0], [5.0, 0]])
    t2, c2 = M.merge_targets(k2, np.array([0, 1]), 0.5)
    assert t2[3] == 0 and abs(c2[3] - 1.0) < 1e-15 and t2[2] == -1
    # a zero key is similar to nothing
    k3 = np.array([[1.0, 0], [0.0, 0]])
    t3, c3 = M.merge_targets(k3, np.array([0]), -0.5)
    assert c3[1] == 0.0 and t3[1] == 0


def test_brute_force_loop():
    rng = np.random.default_rng(4)
    n, d = 40, 6
    k = rng.standard_normal((n, d))
    k[7] = 0.0
    kept = np.sort(rng.choice(n, 9, replace=False))
    t, c = M.merge_targets(k, kept, 0.3)
    for e in range(n):
        if e in kept:
            assert t[e] == -1
            continue
        best, arg = -np.inf, -1
        for r, j in enumerate(kept):
            ne, nj = np.sqrt(np.dot(k[e], k[e])), np.sqrt(np.dot(k[j], k[j]))
            s = np.dot(k[e], k[j]) / (ne * nj) if ne > 0 and nj > 0 else 0.0
            if s > best:
                best, arg = s, r
        assert abs(best - c[e]) < 1e-12
        assert t[e] == (arg if best > 0.3 else -1)
    cnt = M.merge_counts(k, kept, 0.3)
    assert cnt.sum() == np.sum(t >= 0)
    assert np.allclose(M.merged_bias(np.full(9, -0.5), cnt), -0.5 + np.log(1 + cnt), rtol=0, atol=1e-15)
