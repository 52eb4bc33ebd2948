"""A step (score + select + compact, as three calls or as the one-call
eviction) captured in a HIP graph and replayed gives the eager results on
every replay, with eager work and synchronisations between replays (the
library records no memset nodes: every buffer it clears is cleared by a
kernel)."""
import numpy as np
import pytest
import torch

from long_context_attention_kvevict_amd import kvevict as K
from long_context_attention_kvevict_amd import workloads
from tests.gpu_util import Run, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["llama", "qwen_sample"])
def test_graph_replay_matches_eager(name):
    base = workloads.llama8b_32k() if name == "llama" else workloads.qwen7b_128k_sample()
    wl = workloads.scaled(base, 6000)
    say(f"graph replay {wl.name}")
    r = Run(wl)
    b = r.b
    dev = r.k.device
    budgets, caps = wl.budgets(), wl.caps()
    bud, cap = b.offsets(budgets, dev), b.offsets(caps, dev)
    mode = r.mode()
    tb, tc = int(budgets.sum()), int(caps.sum())
    scores = torch.empty((wl.Hkv, wl.T), dtype=torch.float32, device=dev)
    sel = (torch.empty((wl.Hkv, tb), dtype=torch.int32, device=dev),
           torch.empty((wl.Hkv, tb), dtype=torch.float32, device=dev),
           torch.empty((wl.S, wl.Hkv), dtype=torch.float64, device=dev),
           torch.empty((wl.S, wl.Hkv), dtype=torch.int32, device=dev))
    cmp = (torch.zeros((wl.Hkv, tc, wl.d), dtype=r.k.dtype, device=dev),
           torch.zeros((wl.Hkv, tc, wl.d), dtype=r.v.dtype, device=dev),
           torch.zeros((wl.Hkv, tc), dtype=torch.float32, device=dev))

    def step():
        b.score(r.q, r.k, r.v, wl.sm_scale, causal=True, pool_kernel=wl.pool_kernel, out=scores)
        idx, bias, _, _ = b.select(scores, budgets, mode=mode, tau=wl.tau, tau_w=wl.tau_w,
                                   seed=wl.hash_seed, out=sel, bud_offsets=bud)
        b.compact(r.k, r.v, budgets, idx, bias, caps, out=cmp, bud_offsets=bud, cap_offsets=cap)

    def snapshot():
        torch.cuda.synchronize()
        return [t.cpu().clone() for t in (scores, *sel, *cmp)]

    step()
    ref = snapshot()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (scores, *sel, *cmp):   # poison outputs between replays
            t.zero_()
        _ = (r.k.float().sum()).item()   # unrelated eager work
        graph.replay()
        got = snapshot()
        for a, e in zip(got, ref):
            assert torch.equal(a, e), f"replay {rep} differs from eager"


@pytest.mark.parametrize("name", ["llama", "qwen_sample"])
def test_graph_replay_one_call_eviction(name):
    # kvevict_evict: the scorer's merge launch clears the selection's counters
    # (top-k), the sampling key pass clears them itself, and the ordered write
    # gathers the kept rows; a captured call replays to the eager results
    base = workloads.llama8b_32k() if name == "llama" else workloads.qwen7b_128k_sample()
    wl = workloads.scaled(base, 6000)
    say(f"graph replay, one call {wl.name}")
    r = Run(wl)
    b = r.b
    dev = r.k.device
    budgets, caps = wl.budgets(), wl.caps()
    bud, cap = b.offsets(budgets, dev), b.offsets(caps, dev)
    mode = r.mode()

    def step(out=None):
        return b.evict(r.q, r.k, r.v, wl.sm_scale, budgets, caps, mode=mode, pool_kernel=wl.pool_kernel,
                       tau=wl.tau, tau_w=wl.tau_w, seed=wl.hash_seed, out=out, bud_offsets=bud, cap_offsets=cap)

    tb, tc = int(budgets.sum()), int(caps.sum())
    full = (torch.empty((wl.Hkv, wl.T), dtype=torch.float32, device=dev),
            torch.empty((wl.Hkv, tb), dtype=torch.int32, device=dev),
            torch.empty((wl.Hkv, tb), dtype=torch.float32, device=dev),
            torch.empty((wl.S, wl.Hkv), dtype=torch.float64, device=dev),
            torch.empty((wl.S, wl.Hkv), dtype=torch.int32, device=dev),
            torch.zeros((wl.Hkv, tc, wl.d), dtype=r.k.dtype, device=dev),
            torch.zeros((wl.Hkv, tc, wl.d), dtype=r.v.dtype, device=dev),
            torch.zeros((wl.Hkv, tc), dtype=torch.float32, device=dev))
    step(full)   # eager, which also allocates the workspace outside the capture
    torch.cuda.synchronize()
    ref = [t.cpu().clone() for t in full]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(full)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in full:   # poison outputs between replays
            t.zero_()
        _ = (r.k.float().sum()).item()   # unrelated eager work
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu().clone() for t in full]
        for nm, a, e in zip(("scores", "idx", "bias", "m", "status", "k_c", "v_c", "bias_c"), got, ref):
            assert torch.equal(a, e), f"replay {rep}: {nm} differs from eager"
