"""Pins of oracle/attention.py against the mathematics, not against itself."""
import numpy as np
import pytest
import torch

from oracle import window_attention, row_positions


def _rand(seed, R, n, d):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((R, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))


@pytest.mark.parametrize("seed,R,n,d", [(0, 4, 17, 8), (1, 16, 300, 64), (2, 3, 5, 3)])
def test_rows_sum_to_one(seed, R, n, d):
    # [PI] §4, Eq. 5: every row of the softmax is a categorical distribution
    q, k, v = _rand(seed, R, n, d)
    att = window_attention(q, k, v, row_positions(n, R), 1 / np.sqrt(d))
    assert np.all(np.abs(att["alpha"].sum(1) - 1.0) < 1e-12)
    assert np.all(att["alpha"] >= 0)


@pytest.mark.parametrize("causal", [False, True])
def test_output_matches_torch_sdpa(causal):
    # library routine: torch's fp64 CPU scaled_dot_product_attention
    R, n, d = 16, 257, 64
    q, k, v = _rand(3, R, n, d)
    scale = 0.37
    pos = row_positions(n, R) if causal else None
    att = window_attention(q, k, v, pos, scale)
    mask = None
    if causal:
        mask = torch.from_numpy(np.arange(n)[None, :] <= pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=None if mask is None else mask[None], scale=scale)[0].numpy()
    assert np.max(np.abs(att["o"] - ref)) < 1e-12
    # LSE against torch.logsumexp over the visible logits
    lg = torch.from_numpy(scale * q @ k.T)
    if causal:
        lg = lg.masked_fill(~mask, float("-inf"))
    assert np.max(np.abs(att["lse"] - torch.logsumexp(lg, 1).numpy())) < 1e-12


def test_causal_row_is_prefix_attention():
    # a causal window row at position p equals unmasked attention over keys 0..p
    R, n, d = 8, 40, 16
    q, k, v = _rand(4, R, n, d)
    pos = row_positions(n, R)
    att_c = window_attention(q, k, v, pos, 0.25)
    for r in range(R):
        p = pos[r]
        att_u = window_attention(q[r:r + 1], k[:p + 1], v[:p + 1], None, 0.25)
        assert np.allclose(att_c["o"][r], att_u["o"][0], atol=1e-13, rtol=0)
    # the last window row sees every key: causal == non-causal for it
    att_n = window_attention(q, k, v, None, 0.25)
    assert np.allclose(att_c["o"][-1], att_n["o"][-1], atol=1e-14, rtol=0)
    assert not np.allclose(att_c["o"][0], att_n["o"][0])
