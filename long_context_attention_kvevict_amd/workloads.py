"""The five synthetic workloads, named by what they are.

Shapes follow the model layers the DropKV page evaluates (Llama-3.1-8B,
Qwen2.5-7B-1M, MegaBeam-Mistral-7B-512K) at the RULER deployment length
n = 128K, plus one tiny fp32 single-head case for exact checks.
"""
from __future__ import annotations

import numpy as np

from .synth import Workload


def _ragged_lengths(seed: int, S: int) -> list:
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.integers(4096, 65536 + 1, size=S)]


def tiny_fp32() -> Workload:
    """1 q-head / 1 KV head, d=64, n=1024, w=16, fp32, 4 sinks, top-k B=102,
    no pooling, 8 decode steps."""
    return Workload(name="tiny_fp32_n1k", S=1, Hq=1, Hkv=1, d=64, w=16, dtype="f32",
                    lens=[1024], budget_frac=0.1, mode="topk", pool_kernel=1,
                    sinks=4, decode_steps=8, decode_headroom=8,
                    data_seed=1001, hash_seed=2001)


def llama8b_32k() -> Workload:
    """Llama-3.1-8B layer: 32 q-heads, 8 KV heads, d=128, n=32768, w=32,
    bf16, 4 sinks + 16 needles per KV head, top-k 10 %, max-pool 7."""
    return Workload(name="llama3.1-8b_layer_n32k", S=1, Hq=32, Hkv=8, d=128, w=32, dtype="bf16",
                    lens=[32768], budget_frac=0.1, mode="topk", pool_kernel=7,
                    sinks=4, needles=16, data_seed=1002, hash_seed=2002)


def llama8b_128k() -> Workload:
    """Same layer at n=131072, 5 % budget, 64 needles per KV head."""
    return Workload(name="llama3.1-8b_layer_n128k", S=1, Hq=32, Hkv=8, d=128, w=32, dtype="bf16",
                    lens=[131072], budget_frac=0.05, mode="topk", pool_kernel=7,
                    sinks=4, needles=64, data_seed=1003, hash_seed=2003)


def qwen7b_128k_sample() -> Workload:
    """Qwen2.5-7B layer: 28 q-heads, 4 KV heads, d=128, n=131072, w=64,
    bf16, 4 outlier key channels (x8); Gumbel sampling without replacement
    from a temperature-0.5 proposal, budget 10 %."""
    return Workload(name="qwen2.5-7b_layer_n128k_sample", S=1, Hq=28, Hkv=4, d=128, w=64,
                    dtype="bf16", lens=[131072], budget_frac=0.1, mode="sample",
                    pool_kernel=7, tau=0.5, tau_w=1.0, outlier_channels=4,
                    data_seed=1004, hash_seed=2004)


def mistral7b_ragged() -> Workload:
    """Mistral-7B-shaped ragged batch: 8 sequences of 4096..65536 tokens,
    32 q-heads, 8 KV heads, d=128, w=32, bf16, sinks + 16 needles, 10 %
    budget per sequence, 128 decode steps with 128 slots of headroom."""
    return Workload(name="mistral-7b_ragged8_decode", S=8, Hq=32, Hkv=8, d=128, w=32, dtype="bf16",
                    lens=_ragged_lengths(3005, 8), budget_frac=0.1, mode="sample",
                    pool_kernel=7, tau=0.5, tau_w=1.0, sinks=4, needles=16,
                    decode_steps=128, decode_headroom=128,
                    data_seed=1005, hash_seed=2005)


ALL = {
    "tiny": tiny_fp32,
    "llama32k": llama8b_32k,
    "llama128k": llama8b_128k,
    "qwen128k": qwen7b_128k_sample,
    "mistral_ragged": mistral7b_ragged,
}


def scaled(wl: Workload, n: int) -> Workload:
    """Same shape with every sequence cut to at most n tokens (for parity runs
    the oracle finishes in seconds)."""
    import dataclasses
    lens = [min(x, n) for x in wl.lens]
    return dataclasses.replace(wl, lens=lens, name=f"{wl.name}@n{n}")
