"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare with the oracle under the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

from long_context_attention_kvevict_amd import kvevict as K
from long_context_attention_kvevict_amd import synth

# tolerances (scores: 2e-2 relative above 1e-6 of the head's max, absolute
# 2e-8 x max below; select/compact exact; decode 1e-2 max-abs)
SCORE_RTOL = 2e-2
SCORE_FLOOR = 1e-6
SCORE_ATOL_REL_MAX = 2e-8
DECODE_ATOL = 1e-2


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def check_scores(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """Per-head score tolerance; returns (max rel err above floor, max abs err below / max)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite scores"
    mx = ref.max()
    big = ref >= SCORE_FLOOR * mx
    rel = np.abs(got[big] - ref[big]) / ref[big]
    small_err = np.abs(got[~big] - ref[~big]).max() / mx if (~big).any() else 0.0
    worst = rel.max() if rel.size else 0.0
    assert worst <= SCORE_RTOL, f"{what}: max rel err {worst:.3e} at {np.argmax(rel)}"
    assert small_err <= SCORE_ATOL_REL_MAX, f"{what}: abs err below floor {small_err:.3e} x max"
    return worst, small_err


class Run:
    """Inputs of one workload on the device plus the batch handle."""

    def __init__(self, wl, data=None):
        self.wl = wl
        self.data = synth.generate(wl) if data is None else data
        self.b = K.Batch(wl.lens, wl.Hq, wl.Hkv, wl.d, wl.w, wl.dtype)
        self.q = K.to_device(self.data["q_win"], wl.dtype)
        self.k = K.to_device(self.data["k"], wl.dtype)
        self.v = K.to_device(self.data["v"], wl.dtype)

    def f64(self, name):
        return synth.to_f64(self.data[name], self.wl.dtype)

    def score(self, causal=True):
        out = self.b.score(self.q, self.k, self.v, self.wl.sm_scale, causal=causal,
                           pool_kernel=self.wl.pool_kernel)
        torch.cuda.synchronize()
        return out

    def mode(self):
        return K.KVE_TOPK if self.wl.mode == "topk" else K.KVE_SAMPLE
