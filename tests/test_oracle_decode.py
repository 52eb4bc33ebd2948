"""Pins of oracle/decode.py (compaction and SNIS decode)."""
import numpy as np
import torch

from oracle import compact, decode_attention, decode_alg1_literal


def _sdpa(q, k, v, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=scale)[0, 0].numpy()


def test_full_budget_equals_exact_attention():
    # [PI] §5, Proposition / Algorithm 1: keeping every entry with weight 1
    # (bias 0) plus the appended tokens is exact attention
    rng = np.random.default_rng(0)
    n, d, steps = 40, 16, 5
    k = rng.standard_normal((1, n, d))
    v = rng.standard_normal((1, n, d))
    idx = np.arange(n)[None]
    bias = np.zeros((1, n))
    off = np.array([0, n]); bud = np.array([0, n]); cap = np.array([0, n + steps])
    k_c, v_c, b_c = compact(k, v, idx, bias, off, bud, cap)
    kn = rng.standard_normal((steps, d)); vn = rng.standard_normal((steps, d))
    qn = rng.standard_normal((steps, d))
    for t in range(steps):
        k_c[0, n + t] = kn[t]; v_c[0, n + t] = vn[t]; b_c[0, n + t] = 0.0
        got = decode_attention(qn[t][None, None], k_c, v_c, b_c, cap, [n + t + 1], 1, 0.3)[0, 0]
        full_k = np.concatenate([k[0], kn[:t + 1]])
        full_v = np.concatenate([v[0], vn[:t + 1]])
        assert np.max(np.abs(got - _sdpa(qn[t][None], full_k, full_v, 0.3)[0])) < 1e-12


def test_literal_algorithm1_equals_biased_softmax():
    rng = np.random.default_rng(1)
    n, d, new = 30, 8, 4
    kh = rng.standard_normal((n, d)); vh = rng.standard_normal((n, d))
    kn = rng.standard_normal((new, d)); vn = rng.standard_normal((new, d))
    q = rng.standard_normal(d)
    q_incl = rng.uniform(0.05, 1.0, size=n)
    w = 1.0 / q_incl                     # Horvitz-Thompson style weights
    bias = np.concatenate([np.log(w), np.zeros(new)])
    k_c = np.concatenate([kh, kn])[None]; v_c = np.concatenate([vh, vn])[None]
    got = decode_attention(q[None, None], k_c, v_c, bias[None], [0, n + new], [n + new], 1, 0.5)[0, 0]
    ref = decode_alg1_literal(q, kh, vh, w, kn, vn, 0.5)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_zero_bias_is_conditional_expectation():
    # [PI] §5, Eq. 6: uncorrected attention over I = renormalised restriction
    # of the full distribution to I
    rng = np.random.default_rng(2)
    n, d = 50, 8
    k = rng.standard_normal((n, d)); v = rng.standard_normal((n, d)); q = rng.standard_normal(d)
    I = np.sort(rng.choice(n, 12, replace=False))
    lg = 0.4 * k @ q
    p = np.exp(lg - lg.max()); p /= p.sum()
    cond = (p[I] / p[I].sum()) @ v[I]
    got = decode_attention(q[None, None], k[I][None], v[I][None], np.zeros((1, 12)), [0, 12], [12], 1, 0.4)[0, 0]
    assert np.max(np.abs(got - cond)) < 1e-12


def test_with_replacement_weights_converge():
    # [PI] §5 Proposition: counts c from m draws of pi, weights c/(m pi) ->
    # exact attention as m grows; error shrinks roughly like m^-1/2
    rng = np.random.default_rng(3)
    n, d = 200, 8
    k = rng.standard_normal((n, d)); v = rng.standard_normal((n, d)); q = rng.standard_normal(d)
    exact = _sdpa(q[None], k, v, 0.5)[0]
    pi = rng.dirichlet(np.full(n, 1.0))
    errs = []
    for m in (100, 10000, 1000000):
        e = []
        for rep in range(20):
            c = rng.multinomial(m, pi)
            keep = c > 0
            w = c[keep] / (m * pi[keep])
            o = decode_alg1_literal(q, k[keep], v[keep], w, np.zeros((0, d)), np.zeros((0, d)), 0.5)
            e.append(np.linalg.norm(o - exact))
        errs.append(np.mean(e))
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 0.05 * errs[0]


def test_compact_gathers_rows():
    rng = np.random.default_rng(4)
    Hkv, d = 2, 4
    lens = [7, 9]
    off = np.array([0, 7, 16]); bud = np.array([0, 2, 5]); cap = np.array([0, 4, 9])
    k = rng.standard_normal((Hkv, 16, d)); v = rng.standard_normal((Hkv, 16, d))
    idx = np.array([[1, 5, 0, 2, 8], [0, 6, 3, 4, 5]])
    bias = rng.standard_normal((Hkv, 5))
    k_c, v_c, b_c = compact(k, v, idx, bias, off, bud, cap)
    assert np.array_equal(k_c[1, 4 + 2], k[1, 7 + idx[1, 2 + 2]])
    assert np.array_equal(v_c[0, 1], v[0, 5])
    assert b_c[0, 4] == bias[0, 2] and np.all(k_c[:, 2:4] == 0)
