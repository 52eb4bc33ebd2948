"""The allocation-free decode entry point (kvevict_decode_snis_noalloc)
against kvevict_decode_snis: two calls in a row on the same GPU, the
second with a smaller batch, must give the workspace entry point's output
bit for bit (same kernels, partials in the library's device scratch)."""
import numpy as np
import pytest
import torch

from long_context_attention_kvevict_amd import kvevict as K
from long_context_attention_kvevict_amd import synth, workloads
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _case(lens, Hq, Hkv, headroom, seed):
    import dataclasses
    wl = dataclasses.replace(workloads.mistral7b_ragged(), name=f"noalloc{seed}", S=len(lens), Hq=Hq, Hkv=Hkv,
                             lens=lens, decode_headroom=headroom, data_seed=seed)
    cache = synth.generate_cache(wl)
    dev = torch.device("cuda:0")
    b = K.Batch(wl.lens, wl.Hq, wl.Hkv, wl.d, wl.w, wl.dtype, device=dev)
    caps, budgets = wl.caps(), wl.budgets()
    cap = b.offsets(caps, dev)
    k_c, v_c = K.to_device(cache["k"], wl.dtype, dev), K.to_device(cache["v"], wl.dtype, dev)
    b_c = torch.from_numpy(cache["bias"]).to(dev)
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((wl.S, wl.Hq, wl.d)).astype(np.float32)).to(torch.bfloat16).to(dev)
    cache_len = torch.from_numpy(budgets.astype(np.int32)).to(dev)
    return wl, b, cap, k_c, v_c, b_c, q, cache_len, int(budgets.max())


def test_noalloc_decode_matches_workspace_decode_twice():
    assert K.load_library().kvevict_decode_scratch_max() == 8 << 20
    outs = []
    # second call: fewer sequences, shorter caches (the scratch keeps the
    # first call's partials; only what the second writes may be read)
    for lens, Hq, Hkv, seed in (([9000, 41000, 23000, 60000], 32, 8, 71), ([5000, 700], 8, 2, 72)):
        wl, b, cap, k_c, v_c, b_c, q, cache_len, mx = _case(lens, Hq, Hkv, 16, seed)
        say(f"[gpu] noalloc decode S={wl.S} Hq={Hq} Hkv={Hkv} caches {cache_len.tolist()}")
        ref = b.decode(q, k_c, v_c, b_c, wl.caps(), cache_len, mx, wl.sm_scale, cap_offsets=cap)
        out = torch.full_like(ref, float("nan"))
        b.decode_noalloc(q, k_c, v_c, b_c, cap, cache_len, mx, wl.sm_scale, out)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert torch.equal(out, ref), float((out - ref).abs().max())
        outs.append(out)
    assert outs[1].shape != outs[0].shape
