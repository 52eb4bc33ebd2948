"""GPU tier at full workload sizes, in the launch configuration the benchmark
times.  The oracle scores every key of two KV heads per workload (all
window rows, all n keys), checks every head's selection given the GPU's
scores, and sampled decode steps.  One KV head at n = 2^20 (the longest
sequence tested) checks sampled keys and their pooling windows, each
against every row's full softmax."""
import numpy as np
import pytest
import torch

import oracle
from oracle.score import max_pool_fast
from oracle.select import select_workload, expected_distinct, proposal, inclusion_prob
from long_context_attention_kvevict_amd import kvevict as K
from long_context_attention_kvevict_amd import synth, workloads
from tests.gpu_util import Run, check_scores, say, DECODE_ATOL

pytestmark = pytest.mark.gpu


def _check_full_scores(r, got, s, h):
    """Every key of (sequence s, KV head h) against the oracle's pooled
    group score (all window rows of the group's q-heads, all n keys)."""
    wl = r.wl
    a, b = wl.seq_off()[s], wl.seq_off()[s + 1]
    raw = oracle.group_scores(r.f64_q()[s], r.f64_kv("k", h, a, b), r.f64_kv("v", h, a, b), h, wl.g,
                              wl.sm_scale, True)
    ref = max_pool_fast(raw, wl.pool_kernel)
    worst, small = check_scores(got[h, a:b], ref, f"{wl.name} s{s} h{h}")
    say(f"[gpu] full {wl.name} s{s} h{h}: all {b - a} keys, max rel err {worst:.2e}")
    return worst


class BigRun(Run):
    def f64_q(self):
        if not hasattr(self, "_q64"):
            self._q64 = synth.to_f64(self.data["q_win"], self.wl.dtype)
        return self._q64

    def f64_kv(self, name, h, a, b):
        return synth.to_f64(self.data[name][h, a:b], self.wl.dtype)


def _select_parity(r, scores_np):
    wl = r.wl
    mode = K.KVE_TOPK if wl.mode == "topk" else K.KVE_SAMPLE
    budgets = wl.budgets()
    idx, bias, m, st = r.b.select(torch.from_numpy(scores_np).cuda(), budgets, mode=mode, tau=wl.tau,
                                  tau_w=wl.tau_w, seed=wl.hash_seed)
    torch.cuda.synchronize()
    idx, bias, m, st = idx.cpu().numpy(), bias.cpu().numpy(), m.cpu().numpy(), st.cpu().numpy()
    ridx, rbias, rm, rst = select_workload(scores_np.astype(np.float64), wl.seq_off(), budgets, wl.mode,
                                           wl.tau, wl.tau_w, wl.hash_seed)
    assert np.array_equal(idx, ridx)
    assert np.array_equal(st, rst)
    if mode == K.KVE_SAMPLE:
        off, boff = wl.seq_off(), wl.bud_off()
        for h in range(wl.Hkv):
            for s in range(wl.S):
                a, b = off[s], off[s + 1]
                pi = proposal(scores_np[h, a:b].astype(np.float64), wl.tau)
                if st[s, h] == 0:
                    assert abs(expected_distinct(pi, m[s, h]) - budgets[s]) <= 0.5 + 1e-9 * (b - a)
                q = inclusion_prob(pi[idx[h, boff[s]:boff[s + 1]]], m[s, h])
                ref_b = -np.log(q) / wl.tau_w
                assert np.all(np.abs(bias[h, boff[s]:boff[s + 1]] - ref_b) <= 1e-6 * (1 + np.abs(ref_b)))
    return idx, bias, m, st


def test_llama_layer_n128k_topk():
    wl = workloads.llama8b_128k()
    say(f"[gpu] full {wl.name}: generating")
    r = BigRun(wl)
    say(f"[gpu] full {wl.name}: score")
    got = r.score().cpu().numpy()
    assert np.all(np.isfinite(got))
    for h in (0, 5):
        _check_full_scores(r, got, 0, h)
    say(f"[gpu] full {wl.name}: select")
    idx, bias, _, _ = _select_parity(r, got)
    # needle recall (context, not parity)
    npos = r.data["needle_pos"][(0, 0)]
    say(f"[gpu] needle recall head 0: {np.isin(npos, idx[0]).mean():.3f}")
    budgets = wl.budgets()
    k_c, v_c, b_c = r.b.compact(r.k, r.v, budgets, torch.from_numpy(idx).cuda(), torch.from_numpy(bias).cuda(),
                                budgets)
    torch.cuda.synchronize()
    kbits = r.data["k"].view(np.int16)
    for h in (0, 7):
        assert np.array_equal(k_c[h].cpu().view(torch.int16).numpy(), kbits[h, idx[h]])
    # partition-conserving merge at full size: sampled evicted tokens of head
    # 0 against all kept keys (fp64 cosines; near-ties within 1e-4 accepted)
    say(f"[gpu] full {wl.name}: merge")
    from oracle.merge import cosine
    tau = 0.3
    bias_d = torch.from_numpy(bias.copy()).cuda()
    _, merged, target = r.b.merge(r.k, budgets, torch.from_numpy(idx).cuda(), bias_d, tau, want_target=True)
    torch.cuda.synchronize()
    merged, target, bias1 = merged.cpu().numpy(), target.cpu().numpy(), bias_d.cpu().numpy()
    kept = idx[0].astype(np.int64)
    ev = np.setdiff1d(np.arange(wl.T), kept)
    smp = np.random.default_rng(3).choice(ev, 200, replace=False)
    kf = synth.to_f64(r.data["k"][0], wl.dtype)
    c = cosine(kf[smp], kf[kept])
    srt = np.sort(c, axis=1)
    for i, e in enumerate(smp):
        g = target[0, e]
        if g >= 0:
            assert c[i, g] >= srt[i, -1] - 1e-4 and c[i, g] > tau - 1e-4, (e, g)
        else:
            assert srt[i, -1] <= tau + 1e-4, e
    assert np.all(target[0, kept] == -1)
    cnt = np.bincount(target[0][target[0] >= 0], minlength=kept.size)
    assert np.array_equal(merged[0], cnt)
    assert np.allclose(bias1[0], (bias[0].astype(np.float64) + np.log1p(cnt)).astype(np.float32), rtol=1e-6,
                       atol=1e-6)


def test_llama_layer_n32k_topk():
    # the Llama layer at n = 32768 (10 % budget): the key chunk and grid the
    # benchmark runs at this length
    wl = workloads.llama8b_32k()
    say(f"[gpu] full {wl.name}: generating")
    r = BigRun(wl)
    got = r.score().cpu().numpy()
    assert np.all(np.isfinite(got))
    for h in (2, 7):
        _check_full_scores(r, got, 0, h)
    idx, bias, _, _ = _select_parity(r, got)
    budgets = wl.budgets()
    k_c, v_c, b_c = r.b.compact(r.k, r.v, budgets, torch.from_numpy(idx).cuda(), torch.from_numpy(bias).cuda(),
                                budgets)
    torch.cuda.synchronize()
    vbits = r.data["v"].view(np.int16)
    for h in range(wl.Hkv):
        assert np.array_equal(v_c[h].cpu().view(torch.int16).numpy(), vbits[h, idx[h]])


def test_qwen_layer_n128k_sample():
    wl = workloads.qwen7b_128k_sample()
    say(f"[gpu] full {wl.name}: generating")
    r = BigRun(wl)
    got = r.score().cpu().numpy()
    assert np.all(np.isfinite(got))
    for h in (0, 3):
        _check_full_scores(r, got, 0, h)
    say(f"[gpu] full {wl.name}: select")
    idx, bias, m, st = _select_parity(r, got)
    say(f"[gpu] full {wl.name}: per-head m {m[0].tolist()}")
    # one m for all heads (soft budget) at full size, capacity 2 B
    from oracle.select import global_sample_select
    budgets = wl.budgets()
    caps = [min(int(n), 2 * int(B)) for n, B in zip(wl.lens, budgets)]
    tau = float(np.float32(wl.tau))
    sidx, sbias, kept, sm, sst = r.b.select_soft(torch.from_numpy(got).cuda(), budgets, caps, tau=tau,
                                                 tau_w=wl.tau_w, seed=wl.hash_seed)
    torch.cuda.synchronize()
    sidx, sbias, kept, sm, sst = (x.cpu().numpy() for x in (sidx, sbias, kept, sm, sst))
    heads = [got[h].astype(np.float64) for h in range(wl.Hkv)]
    ms = float(sm[0, 0])
    assert np.all(sm[0] == ms) and np.all(sst[0] == 0)
    pis = [proposal(x, tau) for x in heads]
    assert abs(np.mean([expected_distinct(pi, ms) for pi in pis]) - budgets[0]) <= 0.5 + 1e-9 * wl.T
    say(f"[gpu] full {wl.name}: soft budget m {ms:.4g}, kept {kept[0].tolist()}")
    out, rkept, _, _ = global_sample_select(heads, int(budgets[0]), caps[0], tau, wl.tau_w, wl.hash_seed, 0, m=ms)
    assert list(kept[0]) == rkept
    for h in range(wl.Hkv):
        kk = kept[0, h]
        assert np.array_equal(sidx[h, :kk], out[h][0])
        assert np.all(np.abs(sbias[h, :kk] - out[h][1]) <= 1e-6 * (1 + np.abs(out[h][1])))
        assert np.all(sidx[h, kk:] == -1)
    # the literal estimator with head 0's searched m (about 1.5e7 draws)
    from oracle.select import literal_select
    say(f"[gpu] full {wl.name}: literal draws, m = {m[0, 0]:.4g}")
    mm = np.zeros_like(m)
    mm[0, 0] = m[0, 0]
    lcap = [int(wl.lens[0])]
    lidx, lbias, lkept, lst = r.b.select_literal(torch.from_numpy(got).cuda(), torch.from_numpy(mm), lcap, tau=tau,
                                                 tau_w=wl.tau_w, seed=wl.hash_seed)
    torch.cuda.synchronize()
    lidx, lbias, lkept, lst = (x.cpu().numpy() for x in (lidx, lbias, lkept, lst))
    ri, rb, J = literal_select(heads[0], int(m[0, 0]), lcap[0], tau, wl.tau_w, wl.hash_seed, 0, 0)
    assert lst[0, 0] == 0 and lkept[0, 0] == J
    assert np.array_equal(lidx[0, :J], ri)
    assert np.all(np.abs(lbias[0, :J] - rb) <= 1e-5 * (1 + np.abs(rb)))
    say(f"[gpu] full {wl.name}: literal kept {J}")


def test_mistral_ragged_batch_with_decode():
    wl = workloads.mistral7b_ragged()
    say(f"[gpu] full {wl.name}: generating lens={wl.lens}")
    r = BigRun(wl)
    got = r.score().cpu().numpy()
    for s, h in ((0, 0), (3, 3), (7, 6)):
        _check_full_scores(r, got, s, h)
    say(f"[gpu] full {wl.name}: select")
    idx, bias, m, st = _select_parity(r, got)
    budgets = wl.budgets()
    caps = wl.caps()
    k_c, v_c, b_c = r.b.compact(r.k, r.v, budgets, torch.from_numpy(idx).cuda(), torch.from_numpy(bias).cuda(),
                                caps)
    dec = synth.generate_decode(wl)
    cache_len = torch.tensor(budgets, dtype=torch.int32, device="cuda")
    cap_off = r.b.offsets(caps, "cuda")
    coff = wl.cap_off().astype(np.int64)
    lens = budgets.astype(np.int64)
    check_steps = {0, 63, wl.decode_steps - 1}
    say(f"[gpu] full {wl.name}: {wl.decode_steps} decode steps")
    for t in range(wl.decode_steps):
        rows = torch.from_numpy(coff[:-1] + lens).cuda()
        k_c[:, rows] = K.to_device(dec["k"][t], "bf16").transpose(0, 1)
        v_c[:, rows] = K.to_device(dec["v"][t], "bf16").transpose(0, 1)
        b_c[:, rows] = 0.0
        cache_len += 1
        lens += 1
        out = r.b.decode(K.to_device(dec["q"][t], "bf16"), k_c, v_c, b_c, caps, cache_len, int(lens.max()),
                         wl.sm_scale, cap_offsets=cap_off)
        if t in check_steps:
            torch.cuda.synchronize()
            kc = synth.to_f64(k_c.cpu().view(torch.int16).numpy().view(np.uint16), "bf16")
            vc = synth.to_f64(v_c.cpu().view(torch.int16).numpy().view(np.uint16), "bf16")
            ref = oracle.decode_attention(synth.to_f64(dec["q"][t], "bf16"), kc, vc,
                                          b_c.cpu().numpy().astype(np.float64), coff, lens, wl.Hq, wl.sm_scale)
            err = np.abs(out.cpu().numpy() - ref).max()
            say(f"[gpu] decode step {t}: max abs err {err:.2e}")
            assert err <= DECODE_ATOL



def _check_sampled_scores(r, got, s, h, keys):
    """Keys `keys` of (sequence s, KV head h) against the oracle's pooled
    group score: the raw score at every key of each pooling window (each
    row's softmax still over all n keys), then the pooling maximum."""
    from oracle.score import group_scores_at
    wl = r.wl
    a, b = wl.seq_off()[s], wl.seq_off()[s + 1]
    n, rad = b - a, (wl.pool_kernel - 1) // 2
    keys = np.unique(np.asarray(keys, dtype=np.int64))
    near = np.unique(np.clip(keys[:, None] + np.arange(-rad, rad + 1)[None, :], 0, n - 1))
    raw = group_scores_at(r.f64_q()[s], r.f64_kv("k", h, a, b), r.f64_kv("v", h, a, b), h, wl.g, wl.sm_scale,
                          True, near)
    at = dict(zip(near.tolist(), raw.tolist()))
    ref = np.array([max(at[j] for j in range(max(0, x - rad), min(n, x + rad + 1))) for x in keys.tolist()])
    worst, _ = check_scores(got[h, a + keys], ref, f"{wl.name} s{s} h{h} sampled")
    say(f"[gpu] full {wl.name} s{s} h{h}: {keys.size} sampled keys, max rel err {worst:.2e}")


def test_qwen_shape_one_head_n1m_sampling():
    # the largest single sequence here: 2^20 tokens (512 scorer chunks and
    # 1024 selection chunks), one KV head of the Qwen layer's shape (7
    # q-heads, 64 window rows each), through the one-call eviction: the three
    # calls bit for bit, sampled keys' scores against the oracle (the ten
    # largest, the first and last 64 and 1024 at random), the sampling
    # selection given the GPU's scores, and the compaction bit for bit
    import dataclasses
    wl = dataclasses.replace(workloads.qwen7b_128k_sample(), name="qwen_shape_n1m", Hq=7, Hkv=1, lens=[1 << 20])
    say(f"[gpu] full {wl.name}: generating")
    r = BigRun(wl)
    budgets, caps = wl.budgets(), wl.caps()
    say(f"[gpu] full {wl.name}: evict")
    sc, idx, bias, m, st, kc, vc, bc = r.b.evict(r.q, r.k, r.v, wl.sm_scale, budgets, caps, mode=K.KVE_SAMPLE,
                                                 pool_kernel=wl.pool_kernel, tau=wl.tau, tau_w=wl.tau_w,
                                                 seed=wl.hash_seed)
    sc3 = r.b.score(r.q, r.k, r.v, wl.sm_scale, pool_kernel=wl.pool_kernel)
    idx3, bias3, m3, st3 = r.b.select(sc3, budgets, mode=K.KVE_SAMPLE, tau=wl.tau, tau_w=wl.tau_w,
                                      seed=wl.hash_seed)
    torch.cuda.synchronize()
    assert torch.equal(sc.view(torch.uint8), sc3.view(torch.uint8))
    assert torch.equal(idx, idx3) and torch.equal(bias.view(torch.uint8), bias3.view(torch.uint8))
    assert torch.equal(m, m3) and torch.equal(st, st3)
    got = sc.cpu().numpy()
    assert np.all(np.isfinite(got))
    B = int(budgets[0])
    sel = idx.cpu().numpy()[0]
    assert np.array_equal(kc[0, :B].cpu().view(torch.int16).numpy(), r.data["k"].view(np.int16)[0, sel])
    assert np.array_equal(vc[0, :B].cpu().view(torch.int16).numpy(), r.data["v"].view(np.int16)[0, sel])
    n = wl.T
    keys = np.concatenate([np.argsort(got[0])[-10:], np.arange(64), np.arange(n - 64, n),
                           np.random.default_rng(7).choice(n, 1024, replace=False)])
    say(f"[gpu] full {wl.name}: oracle scores of sampled keys")
    _check_sampled_scores(r, got, 0, 0, keys)
    say(f"[gpu] full {wl.name}: selection")
    _, _, m, _ = _select_parity(r, got)
    say(f"[gpu] full {wl.name}: m {m[0, 0]:.6g}")
