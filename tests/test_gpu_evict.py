"""GPU tier: kvevict_evict (score + select + compact in one call, the pooling
folded into the selection's first pass) against the three calls, bit for bit,
through the C ABI.  The three calls themselves are compared with the fp64
oracle in test_gpu_parity.py."""
import dataclasses

import numpy as np
import pytest
import torch

from long_context_attention_kvevict_amd import kvevict as K
from long_context_attention_kvevict_amd import synth, workloads
from tests.gpu_util import Run, say

pytestmark = pytest.mark.gpu


def _cases():
    ragged = dataclasses.replace(workloads.mistral7b_ragged(), name="ragged3", S=3, Hq=8, Hkv=2,
                                 lens=[300, 2049, 5000], needles=4)
    return {
        # top-k over several chunks: level 0 pools (one plane, radius 3)
        "llama_n4099_topk": (workloads.scaled(workloads.llama8b_32k(), 4099), K.KVE_TOPK, 7, None),
        # sampling chain: the key pass pools four row-group planes
        "qwen_n3001_sample": (workloads.scaled(workloads.qwen7b_128k_sample(), 3001), K.KVE_SAMPLE, 7, None),
        # top-k level 0 over four row-group planes
        "qwen_n3001_topk": (workloads.scaled(workloads.qwen7b_128k_sample(), 3001), K.KVE_TOPK, 7, None),
        # ragged batch, budgets 0 and n on two sequences (their scores are still written)
        "ragged3_topk_edges": (ragged, K.KVE_TOPK, 7, [0, 2049, 500]),
        "ragged3_sample_edges": (ragged, K.KVE_SAMPLE, 7, [30, 0, 5000]),
        # widest and narrowest pooling
        "ragged3_topk_pool31": (ragged, K.KVE_TOPK, 31, None),
        "llama_n4099_sample_pool1": (workloads.scaled(workloads.llama8b_32k(), 4099), K.KVE_SAMPLE, 1, None),
        # sequences exactly as long as the window (n = w = 32) and one longer by
        # a key, beside one that spans several chunks: pooling windows and
        # gathers that meet sequence ends
        "ragged_min_topk": (dataclasses.replace(ragged, name="ragged_min", lens=[32, 5000, 33], needles=0),
                            K.KVE_TOPK, 7, None),
        "ragged_min_sample": (dataclasses.replace(ragged, name="ragged_min", lens=[32, 5000, 33], needles=0),
                              K.KVE_SAMPLE, 31, [3, 500, 32]),
        # paths that run the three calls in turn: one chunk per head, fp32
        "ragged_short_topk": (dataclasses.replace(ragged, name="short", lens=[300, 1024, 777]), K.KVE_TOPK, 7, None),
        "tiny_fp32_topk": (workloads.tiny_fp32(), K.KVE_TOPK, 5, None),
    }


CASES = _cases()


@pytest.mark.parametrize("name", list(CASES))
def test_evict_equals_score_select_compact(name):
    wl, mode, pool, budgets = CASES[name]
    r = Run(wl)
    b = r.b
    budgets = np.asarray(wl.budgets() if budgets is None else budgets, dtype=np.int64)
    caps = budgets + 8
    say(f"[gpu] evict {name} lens={wl.lens} mode={mode} pool={pool} budgets={budgets.tolist()}")
    sc = b.score(r.q, r.k, r.v, wl.sm_scale, causal=True, pool_kernel=pool)
    idx, bias, m, st = b.select(sc, budgets, mode=mode, tau=wl.tau, tau_w=wl.tau_w, seed=wl.hash_seed)
    kc, vc, bc = b.compact(r.k, r.v, budgets, idx, bias, caps)
    ref = [x.clone() for x in (sc, idx, bias, m, st, kc, vc, bc)]
    torch.cuda.synchronize()
    for rep in range(2):   # the second call reuses the workspace the first one left
        got = b.evict(r.q, r.k, r.v, wl.sm_scale, budgets, caps, mode=mode, pool_kernel=pool, tau=wl.tau,
                      tau_w=wl.tau_w, seed=wl.hash_seed)
        torch.cuda.synchronize()
        for nm, x, y in zip(("scores", "idx", "bias", "m", "status", "k_c", "v_c", "bias_c"), got, ref):
            assert x.shape == y.shape, (nm, x.shape, y.shape)
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.float32 else x,
                               y.view(torch.uint8) if y.dtype == torch.float32 else y), f"{name}: {nm} differs"
    say(f"[gpu] evict {name} ok")


@pytest.mark.parametrize("name", ["llama128k", "qwen128k", "mistral_ragged"])
def test_evict_full_size_equals_three_calls(name):
    # the benchmark's step at its full size: the one call against the three
    wl = workloads.ALL[name]()
    r = Run(wl)
    b = r.b
    budgets, caps = wl.budgets(), wl.caps()
    mode = K.KVE_TOPK if wl.mode == "topk" else K.KVE_SAMPLE
    say(f"[gpu] evict full size {wl.name} T={wl.T} mode={mode}")
    sc = b.score(r.q, r.k, r.v, wl.sm_scale, causal=True, pool_kernel=wl.pool_kernel)
    idx, bias, m, st = b.select(sc, budgets, mode=mode, tau=wl.tau, tau_w=wl.tau_w, seed=wl.hash_seed)
    kc, vc, bc = b.compact(r.k, r.v, budgets, idx, bias, caps)
    ref = [x.clone() for x in (sc, idx, bias, m, st, kc, vc, bc)]
    del kc, vc, bc
    torch.cuda.synchronize()
    got = b.evict(r.q, r.k, r.v, wl.sm_scale, budgets, caps, mode=mode, pool_kernel=wl.pool_kernel, tau=wl.tau,
                  tau_w=wl.tau_w, seed=wl.hash_seed)
    torch.cuda.synchronize()
    for nm, x, y in zip(("scores", "idx", "bias", "m", "status", "k_c", "v_c", "bias_c"), got, ref):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.float32 else x,
                           y.view(torch.uint8) if y.dtype == torch.float32 else y), f"{name}: {nm} differs"
    say(f"[gpu] evict full size {wl.name} ok")
