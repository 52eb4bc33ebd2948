"""Seeded synthetic inputs for the windowed KV-eviction path.

This module only draws inputs: window queries, cached keys/values and the
decode-time queries/keys/values.  It holds none of the method's arithmetic
(no softmax, no scores, no selection), so both the HIP path and the fp64
oracle can consume exactly the same bits from it.

Stand-ins for the long-context workloads the pages evaluate on (RULER /
LongBench at n = 128K with 5-10 % budgets).  Structure planted on purpose:

* sinks: the first 4 tokens of each KV head get a key aligned with the mean
  window query of that GQA group and a tiny value (norm 0.05), the
  "large weight, near-zero value" pattern discussed on the information-
  theoretic eviction page (sinks section);
* needles: keys aligned (cosine 0.9) with one random window query and values
  of norm 10, mimicking needle-in-a-haystack retrieval;
* outlier channels: 4 key channels per KV head scaled by 8 (Qwen-style).

Floating-point inputs are drawn in fp64, cast to fp32 and then, for bf16
workloads, rounded to bf16 with round-to-nearest-even.  Arrays are returned
as raw bit patterns (uint16 for bf16, float32 otherwise) plus helpers that
widen them exactly to float64.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    u = b.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored input bits (bf16 as uint16, or fp32) to float64 exactly."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    return x32


def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    u = rng.standard_normal(d)
    return u / np.linalg.norm(u)


@dataclass
class Workload:
    """Shape and structure of one synthetic eviction workload."""

    name: str
    S: int
    Hq: int
    Hkv: int
    d: int
    w: int
    dtype: str                      # "bf16" or "f32"
    lens: list                      # per-sequence token counts n_s
    budget_frac: float              # B_s = floor(budget_frac * n_s)
    mode: str                       # "topk" or "sample"
    pool_kernel: int = 7
    tau: float = 1.0                # proposal temperature (sample mode)
    tau_w: float = 1.0              # importance-weight temperature
    sinks: int = 0
    needles: int = 0                # per KV head
    outlier_channels: int = 0
    decode_steps: int = 0
    decode_headroom: int = 0
    data_seed: int = 0
    hash_seed: int = 0
    causal: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def T(self) -> int:
        return int(sum(self.lens))

    def seq_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int32)

    def budgets(self) -> np.ndarray:
        return np.array([int(np.floor(self.budget_frac * n)) for n in self.lens], dtype=np.int32)

    def bud_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.budgets())]).astype(np.int32)

    def caps(self) -> np.ndarray:
        return self.budgets() + np.int32(self.decode_headroom)

    def cap_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.caps())]).astype(np.int32)

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


def make_workload(name: str, **kw) -> Workload:
    return Workload(name=name, **kw)


def generate(wl: Workload) -> dict:
    """Draw the prefill tensors of a workload.

    Returns dict with
      q_win [S][Hq][w][d], k [Hkv][T][d], v [Hkv][T][d]   (stored dtype bits)
      plus metadata: seq_off, needle positions per (s, h).
    """
    rng = np.random.Generator(np.random.PCG64(wl.data_seed))
    S, Hq, Hkv, d, w, g = wl.S, wl.Hq, wl.Hkv, wl.d, wl.w, wl.g
    T = wl.T
    off = wl.seq_off()
    q = rng.standard_normal((S, Hq, w, d))
    k = np.empty((Hkv, T, d), dtype=np.float64)
    v = np.empty((Hkv, T, d), dtype=np.float64)
    needle_pos = {}
    for h in range(Hkv):
        k[h] = rng.standard_normal((T, d))
        v[h] = rng.standard_normal((T, d))
    # Planted structure is defined on the stored (rounded) query bits, so the
    # alignment is relative to what the kernels actually see.
    q_st = _store(q, wl.dtype)
    qf = to_f64(q_st, wl.dtype)
    for s in range(S):
        n = wl.lens[s]
        base = off[s]
        for h in range(Hkv):
            grp = qf[s, h * g:(h + 1) * g].reshape(g * w, d)
            if wl.sinks:
                mean = grp.mean(axis=0)
                qhat = mean / np.linalg.norm(mean)
                for t in range(min(wl.sinks, n)):
                    k[h, base + t] = 4.0 * np.sqrt(d) * qhat
                    v[h, base + t] = 0.05 * _unit(rng, d)
            if wl.needles:
                lo, hi = wl.sinks, n - w
                cnt = min(wl.needles, max(hi - lo, 0))
                pos = np.sort(rng.choice(np.arange(lo, hi), size=cnt, replace=False)) if cnt else np.zeros(0, np.int64)
                needle_pos[(s, h)] = pos
                for p in pos:
                    row = int(rng.integers(0, g * w))
                    qi = grp[row] / np.linalg.norm(grp[row])
                    e = rng.standard_normal(d)
                    e -= e.dot(qi) * qi
                    e /= np.linalg.norm(e)
                    k[h, base + p] = np.sqrt(d) * (0.9 * qi + np.sqrt(0.19) * e)
                    v[h, base + p] = 10.0 * _unit(rng, d)
    if wl.outlier_channels:
        for h in range(Hkv):
            ch = rng.choice(d, size=wl.outlier_channels, replace=False)
            k[h][:, ch] *= 8.0
    return {
        "q_win": q_st,
        "k": _store(k, wl.dtype),
        "v": _store(v, wl.dtype),
        "seq_off": off,
        "needle_pos": needle_pos,
    }


def generate_decode(wl: Workload, steps: int | None = None) -> dict:
    """Decode-time tensors: per step one query per q-head and one new key /
    value per KV head for every sequence, all N(0, 1)."""
    steps = wl.decode_steps if steps is None else steps
    rng = np.random.Generator(np.random.PCG64(wl.data_seed + 7919))
    S, Hq, Hkv, d = wl.S, wl.Hq, wl.Hkv, wl.d
    q = rng.standard_normal((steps, S, Hq, d))
    k = rng.standard_normal((steps, S, Hkv, d))
    v = rng.standard_normal((steps, S, Hkv, d))
    return {"q": _store(q, wl.dtype), "k": _store(k, wl.dtype), "v": _store(v, wl.dtype)}


def generate_cache(wl: Workload) -> dict:
    """A compacted cache of the workload's shape, for decode-only runs.

    Sequence s owns rows [cap_off[s], cap_off[s+1]) of every KV head; the
    first B_s rows hold N(0, 1) keys and values, the rest (decode headroom)
    are zero.  Biases of the kept rows are -log(q)/tau_w with q log-uniform
    on [1e-3, 1] in sample mode (the range inclusion probabilities of a
    10 % budget span), 0 in top-k mode.  Decode cost depends only on these
    shapes, not on which tokens a selection kept.
    """
    rng = np.random.Generator(np.random.PCG64(wl.data_seed + 104729))
    Hkv, d = wl.Hkv, wl.d
    budgets, coff = wl.budgets(), wl.cap_off()
    C = int(coff[-1])
    k = np.zeros((Hkv, C, d), dtype=np.float32)
    v = np.zeros((Hkv, C, d), dtype=np.float32)
    bias = np.zeros((Hkv, C), dtype=np.float32)
    for s, B in enumerate(budgets):
        a = int(coff[s])
        k[:, a:a + B] = rng.standard_normal((Hkv, B, d), dtype=np.float32)
        v[:, a:a + B] = rng.standard_normal((Hkv, B, d), dtype=np.float32)
        if wl.mode == "sample":
            q = np.exp(rng.uniform(np.log(1e-3), 0.0, size=(Hkv, B)))
            bias[:, a:a + B] = (-np.log(q) / wl.tau_w).astype(np.float32)
    return {"k": _store(k, wl.dtype), "v": _store(v, wl.dtype), "bias": bias,
            "cache_len": budgets.copy(), "cap_off": coff}


def random_scores(Hkv: int, lens, seed: int, ties: bool = True) -> np.ndarray:
    """Positive fp32 score arrays [Hkv][T] with a heavy tail and (optionally)
    runs of exactly equal values, like max-pooled eviction scores."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = int(sum(lens))
    s = np.exp(rng.standard_normal((Hkv, T)) * 3.0 - 12.0)
    if ties:
        # plateaus of equal values, as produced by a width-7 max filter
        for h in range(Hkv):
            starts = rng.integers(0, max(T - 7, 1), size=max(T // 50, 1))
            for st in starts:
                s[h, st:st + 7] = s[h, st]
    return s.astype(np.float32)
