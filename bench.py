#!/usr/bin/env python3
"""Eviction-time throughput of the HIP path on one MI355X.

One step = kvevict_score + kvevict_select + kvevict_compact over one layer of
the workload (inputs resident in HBM before timing starts).  The default
workload is the Llama-3.1-8B-shaped layer at n = 131072 (32 q-heads, 8 KV
heads, d = 128, w = 32, bf16, 5 % top-k budget, max-pool 7).

Every timed step starts with cold caches: a 1 GiB streaming read of an
unrelated buffer (clean lines, nothing left to write back) evicts the L2s
and the Infinity Cache first.  `value` and `ms_per_step` are the median
over K such steps; the back-to-back (warm) figures and those after a 512 MiB
device write (whose dirty lines are written back during the step) are extra
keys.

Prints one JSON line with the throughput (scored tokens / s per layer), a
roofline entry for the dominant kernel (per-launch HIP-event durations
recorded on the launch stream over K cold-cache steps), the HBM read
ceiling of the device for the same bytes (plain streaming read, and the
scorer's LDS ring with no arithmetic), the other four workloads timed the
same way, the SNIS decode loop (eager and as one HIP graph), the merge, and
the fp64 oracle timed on a bounded sample of the workload on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--configs all|none|a,b]
                    [--no-cpu-baseline]
    python bench.py --copy-probe MIB     # plain device copy of known size (counter calibration)

roofline.traffic is the HBM traffic per launch of the dominant kernel from
hardware counters (FETCH_SIZE + WRITE_SIZE, each scaled by what the same
counter reads for a plain copy of known size), taken from the committed
counter summary under profiles/; it is null when no summary exists for the
kernel and workload or when the kernel's source has changed since.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "long_context_attention_kvevict_amd", "csrc")
# dominant-kernel stage -> (kernel symbol, source file)
STAGE_KERNEL = {
    "score_pass1": ("score_p1_bf16", "score_bf16.hip"),
    "score_pass2": ("score_p2_bf16", "score_bf16.hip"),
    "score_merge": ("score_merge", "score_bf16.hip"),
    "select": ("sel_", "select.hip"),
    "compact": ("compact_rows", "compact.hip"),
    "decode_split": ("decode_split_mfma", "decode.hip"),
}

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of the MI355X


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama128k", help="headline workload (workloads.ALL)")
    ap.add_argument("--configs", default="all",
                    help="further workloads timed in the same line: 'all', 'none' or a comma list")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=4, help="KV heads the oracle baseline scores")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured in a HIP graph instead of eager launches")
    ap.add_argument("--no-decode", action="store_true", help="skip the SNIS decode measurement")
    ap.add_argument("--no-merge", action="store_true", help="skip the partition-conserving merge measurement")
    ap.add_argument("--score-kind", default="perturb", choices=["perturb", "h2o", "h2o_h", "tova", "min", "min_h"],
                    help="score of the step (the default is the output-perturbation score)")
    ap.add_argument("--pool-mode", default="max", choices=["max", "avg"])
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (5 times) and exit")
    ap.add_argument("--cold-only", action="store_true",
                    help="only the headline workload's K cold-cache steps, no events in the library "
                         "(for a kernel trace whose averages are those of the roofline)")
    return ap.parse_args()


def _source_sha(fname):
    with open(os.path.join(CSRC, fname), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic(stage, workload):
    """HBM bytes per launch of `stage` from the committed counter summary, or
    None if there is none for this workload or the kernel source changed."""
    if stage not in STAGE_KERNEL:
        return None
    kernel, src = STAGE_KERNEL[stage]
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != _source_sha(src):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _copy_probe(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)   # one elementwise kernel: reads and writes n*4 bytes
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 5}))


def _stage_bytes(wl, esize, score_kind="perturb"):
    """Algorithmic HBM bytes per launch of each stage (what the method has to
    move, not implementation scratch)."""
    T, Hkv, d = wl.T, wl.Hkv, wl.d
    kv = 2 * Hkv * T * d * esize            # K and V read once
    planes = ((wl.Hq // wl.Hkv) * wl.w + 127) // 128 if wl.dtype == "bf16" else 1
    B = int(sum(wl.budgets()))
    if score_kind == "perturb":
        p2 = kv + 4 * Hkv * T + 4 * Hkv * T * planes          # + ||v||^2 read, raw scores written
    else:                                                    # attention weights: K only (+ ||v||^2 for the min kinds)
        p2 = kv // 2 + 4 * Hkv * T * planes + (4 * Hkv * T if score_kind in ("min", "min_h") else 0)
    return {
        "score_pass1": kv + 4 * Hkv * T,                       # + ||v||^2 written
        "score_pass2": p2,
        "score_pool": 4 * Hkv * T * planes + 4 * Hkv * T,
        "select": 4 * Hkv * T + 8 * Hkv * B,
        "compact": 2 * (2 * Hkv * B * d * esize) + 12 * Hkv * B,
    }


def _stage_flops(wl, score_kind="perturb"):
    """Algorithmic matrix-core flops per launch of the two scorer passes: every
    window row of a KV head's group against every key, two contractions of
    length d per (row, key) pair (Q.K^T and P.V in pass 1; Q.K^T and O.V^T in
    pass 2, Q.K^T only for the attention-weight scores)."""
    pairs = (wl.Hq // wl.Hkv) * wl.w * wl.Hkv * wl.T
    return {"score_pass1": 4 * wl.d * pairs,
            "score_pass2": (4 if score_kind == "perturb" else 2) * wl.d * pairs}


def _cpu_baseline(wl, data, heads):
    """Oracle score + select + compact of `heads` KV heads, wall clock."""
    import numpy as np
    import oracle
    from oracle.score import max_pool_fast
    from long_context_attention_kvevict_amd import synth
    cores = len(os.sched_getaffinity(0))
    q = synth.to_f64(data["q_win"], wl.dtype)
    off = wl.seq_off()
    budgets = wl.budgets()
    t0 = time.perf_counter()
    for h in range(heads):
        k = synth.to_f64(data["k"][h], wl.dtype)
        v = synth.to_f64(data["v"][h], wl.dtype)
        for s in range(wl.S):
            a, b = off[s], off[s + 1]
            sc = max_pool_fast(oracle.group_scores(q[s], k[a:b], v[a:b], h, wl.g, wl.sm_scale, True),
                               wl.pool_kernel).astype(np.float32)
            if wl.mode == "topk":
                idx = oracle.topk_select(sc, budgets[s])
            else:
                idx, _, _, _ = oracle.sample_select(sc, budgets[s], wl.tau, wl.tau_w, wl.hash_seed, s, h)
            _ = k[a:b][idx], v[a:b][idx]
    dt = time.perf_counter() - t0
    tokens_per_s = wl.T / (dt * wl.Hkv / heads)
    # the same work on one head with the BLAS pool limited to one thread
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        k = synth.to_f64(data["k"][0], wl.dtype)
        v = synth.to_f64(data["v"][0], wl.dtype)
        for s in range(wl.S):
            a, b = off[s], off[s + 1]
            sc = max_pool_fast(oracle.group_scores(q[s], k[a:b], v[a:b], 0, wl.g, wl.sm_scale, True),
                               wl.pool_kernel).astype(np.float32)
            if wl.mode == "topk":
                idx = oracle.topk_select(sc, budgets[s])
            else:
                idx, _, _, _ = oracle.sample_select(sc, budgets[s], wl.tau, wl.tau_w, wl.hash_seed, s, 0)
            _ = k[a:b][idx], v[a:b][idx]
        dt1 = time.perf_counter() - t1
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of {wl.Hkv} KV heads (all {wl.T} tokens, {wl.g * wl.w} window rows), "
                      f"{dt:.1f} s, scaled by {wl.Hkv / heads:g}",
            "value_1thread": wl.T / (dt1 * wl.Hkv),
            "sample_1thread": f"1 of {wl.Hkv} KV heads, BLAS limited to 1 thread, {dt1:.1f} s, scaled by {wl.Hkv}"}


def _merge_cpu(data, wl, idx_np, budgets, tau_merge, sample=16384):
    """The oracle's merge (fp64 cosines, argmax, threshold) for a sample of the
    evicted tokens of KV head 0, scaled to all evicted tokens of all heads."""
    import numpy as np
    from oracle.merge import merge_targets
    from long_context_attention_kvevict_amd import synth
    n, B = int(wl.lens[0]), int(budgets[0])
    kept = idx_np[0, :B].astype(np.int64)
    ev = np.setdiff1d(np.arange(n), kept)
    pick = np.sort(np.random.default_rng(0).choice(ev, min(sample, ev.size), replace=False))
    k = synth.to_f64(data["k"][0], wl.dtype)
    rows = np.sort(np.concatenate([kept, pick]))
    pos = np.searchsorted(rows, kept)
    t0 = time.perf_counter()
    merge_targets(k[rows], pos, tau_merge)
    dt = time.perf_counter() - t0
    evicted = sum(int(x) - int(y) for x, y in zip(wl.lens, budgets)) * wl.Hkv
    flops = 2.0 * wl.d * B * pick.size
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{pick.size} evicted tokens of KV head 0 against its {B} kept keys, {dt:.2f} s "
                      f"(all {evicted} evicted tokens would take {dt * evicted / pick.size:.0f} s)"}


def _merge_leg(b, k, budgets, idx, bias, wl, tau_merge=0.33, reps=10):
    """kvevict_merge over the step's kept set: every evicted key against
    every kept key of its head (cosine), on bf16 MFMAs.  Algorithmic work:
    2 d B (n - B) flops per (sequence, KV head).  The keys are random
    N(0, 1) rows in 128 dimensions, whose best cosine against 6553 kept keys
    is about 0.34: tau_merge = 0.33 merges a part of the evicted tokens."""
    import torch
    flops = sum(2.0 * wl.d * int(B) * (int(n) - int(B)) for n, B in zip(wl.lens, budgets)) * wl.Hkv
    biases = [bias.clone() for _ in range(reps + 3)]
    torch.cuda.synchronize()
    for i in range(3):
        b.merge(k, budgets, idx, biases[i], tau_merge)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(reps):
        _, merged, _ = b.merge(k, budgets, idx, biases[3 + i], tau_merge)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    achieved = flops / (ms * 1e-3) / 1e12
    evicted = sum(int(n) - int(B) for n, B in zip(wl.lens, budgets)) * wl.Hkv
    return {"workload": wl.name, "tau_merge": tau_merge, "ms": ms,
            "merged_fraction_of_evicted": float(merged.sum().item()) / max(evicted, 1),
            "roofline": {"bound": "mfma", "kernel": "mrg_sim (with its prep/apply launches)",
                         "achieved": achieved, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_PEAK_TFLOPS,
                         "traffic": None, "algorithmic_flops": flops}}


def _decode_leg(steps_max, want_cpu):
    """SNIS decode over a compacted cache of the Mistral-7B-shaped ragged
    batch: every step appends one token per (sequence, KV head) with bias 0
    and runs kvevict_decode_snis for all 32 q-heads of the 8 sequences."""
    import numpy as np
    import torch
    from long_context_attention_kvevict_amd import kvevict as K
    from long_context_attention_kvevict_amd import synth, workloads

    wl = workloads.mistral7b_ragged()
    steps = min(wl.decode_steps, steps_max)
    dev = torch.device("cuda:0")
    cache = synth.generate_cache(wl)
    dec = synth.generate_decode(wl, steps)
    b = K.Batch(wl.lens, wl.Hq, wl.Hkv, wl.d, wl.w, wl.dtype, device=dev)
    caps, budgets = wl.caps(), wl.budgets()
    cap = b.offsets(caps, dev)
    k0, v0 = K.to_device(cache["k"], wl.dtype, dev), K.to_device(cache["v"], wl.dtype, dev)
    b0 = torch.from_numpy(cache["bias"]).to(dev)
    qd = K.to_device(dec["q"], wl.dtype, dev)
    kd = K.to_device(dec["k"], wl.dtype, dev).transpose(1, 2).contiguous()   # [t][Hkv][S][d]
    vd = K.to_device(dec["v"], wl.dtype, dev).transpose(1, 2).contiguous()
    coff = torch.from_numpy(wl.cap_off()[:-1].astype(np.int64)).to(dev)
    max_len = int(caps.max())
    out = torch.empty((wl.S, wl.Hq, wl.d), dtype=torch.float32, device=dev)

    k_c, v_c, b_c = k0.clone(), v0.clone(), b0.clone()
    cache_len = torch.from_numpy(budgets.copy()).to(dev)

    def reset():
        k_c.copy_(k0)
        v_c.copy_(v0)
        b_c.copy_(b0)
        cache_len.copy_(torch.from_numpy(budgets.copy()))

    def loop_host_append():
        # the caller appends each step's token (four small torch launches),
        # then kvevict_decode_snis
        for t in range(steps):
            rows = coff + cache_len
            k_c.index_copy_(1, rows, kd[t])
            v_c.index_copy_(1, rows, vd[t])
            b_c.index_fill_(1, rows, 0.0)
            cache_len.add_(1)
            b.decode(qd[t], k_c, v_c, b_c, caps, cache_len, max_len, wl.sm_scale, out=out, cap_offsets=cap)

    def loop():
        # kvevict_decode_snis_append: the decode attends to and stores the
        # step's token itself (two launches per step)
        for t in range(steps):
            b.decode_append(qd[t], kd[t], vd[t], k_c, v_c, b_c, caps, cache_len, max_len, wl.sm_scale, out=out,
                            cap_offsets=cap)

    def run(fn=loop):
        reset()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    run(loop_host_append)                    # warmup
    ms_host = run(loop_host_append)
    out_host = out.clone()
    run()                                    # warmup
    ms = run()
    out_eager = out.clone()
    append_equal = bool(torch.equal(out_eager, out_host))
    K.timing_enable(["decode_split", "decode_merge"])
    run()
    stages = K.timing_summary()
    K.timing_enable(False)
    # the same loop captured as one HIP graph (appends and decode calls of
    # every step) and replayed; the last step's output must equal the eager one
    reset()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()
    graph_ms = []
    for _ in range(3):
        reset()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms.append(g0.elapsed_time(g1) / steps)
    graph_equal = bool(torch.equal(out, out_eager))
    del graph
    esize = 2 if wl.dtype == "bf16" else 4
    # entries read per step, averaged over the steps: sum_s (B_s + t + 1)
    entries = float(budgets.sum()) * wl.Hkv + wl.S * wl.Hkv * (steps + 1) / 2.0
    kv_bytes = entries * (2 * wl.d * esize + 4) + wl.S * wl.Hq * wl.d * esize
    split_ms, merge_ms = stages["decode_split"][0], stages["decode_merge"][0]
    achieved = kv_bytes / (split_ms * 1e-3) / 1e9
    res = {
        "workload": wl.name, "S": wl.S, "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d,
        "cache_len": [int(x) for x in budgets], "steps": steps,
        "cache": "synthetic compacted cache of the batch's capacities (N(0,1) rows, sample-mode biases)",
        "ms_per_step": ms, "tokens_per_s": wl.S / (ms * 1e-3),
        "ms_per_step_graph": float(np.median(graph_ms)), "tokens_per_s_graph": wl.S / (np.median(graph_ms) * 1e-3),
        "graph_output_equals_eager": graph_equal,
        "ms_per_step_host_append": ms_host, "tokens_per_s_host_append": wl.S / (ms_host * 1e-3),
        "host_append_output_equal": append_equal,
        "launch": (f"eager: kvevict_decode_snis_append per step (the token appended by the decode); graph: the "
                   f"{steps} steps captured as one HIP graph; host_append: 4 torch appends + kvevict_decode_snis "
                   f"per step"),
        "kernel_ms": {"decode_split": split_ms, "decode_merge": merge_ms},
        "roofline": {"bound": "hbm", "kernel": "decode_split", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": _traffic("decode_split", wl.name),
                     "algorithmic_bytes": kv_bytes, "launch_ms": split_ms},
    }
    if want_cpu:
        import oracle
        t0 = time.perf_counter()
        kc = synth.to_f64(cache["k"], wl.dtype)
        vc = synth.to_f64(cache["v"], wl.dtype)
        bc = cache["bias"].astype(np.float64)
        lens = budgets.astype(np.int64)
        q0 = synth.to_f64(dec["q"][0], wl.dtype)
        t1 = time.perf_counter()
        reps = 3
        for _ in range(reps):
            oracle.decode_attention(q0, kc, vc, bc, wl.cap_off().astype(np.int64), lens, wl.Hq, wl.sm_scale)
        dt = (time.perf_counter() - t1) / reps
        res["cpu_baseline"] = {"value": wl.S / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
                               "kind": "oracle", "sample": f"{reps} decode steps over the step-0 cache "
                               f"(widening {t1 - t0:.1f} s not counted)"}
    return res


class Probe:
    """The memory-system probes of libkveprobe.so: a plain streaming read
    (the HBM read ceiling; also used to evict the caches with clean lines
    before each cold-cache step) and the scorer's ring structure with no
    arithmetic."""

    def __init__(self, dev):
        import torch
        path = os.path.join(ROOT, "long_context_attention_kvevict_amd", "lib", "libkveprobe.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} not found; build with `python -m long_context_attention_kvevict_amd.build`")
        self.lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        self.lib.kvp_read.argtypes = [P, ctypes.c_size_t, P, P]
        self.lib.kvp_read_ring.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
        self.sink = torch.zeros(self.lib.kvp_read_sink_words(), dtype=torch.int32, device=dev)
        # 1 GiB of clean lines, four times the Infinity Cache
        self.evict_buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev)

    def _st(self):
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def evict(self):
        rc = self.lib.kvp_read(self.evict_buf.data_ptr(), self.evict_buf.numel(), self.sink.data_ptr(), self._st())
        assert rc == 0, rc

    def read(self, ptr, nbytes):
        rc = self.lib.kvp_read(ptr, nbytes, self.sink.data_ptr(), self._st())
        assert rc == 0, rc

    def ring(self, k, v, Hkv, n, chunk):
        rc = self.lib.kvp_read_ring(k.data_ptr(), v.data_ptr(), Hkv, n, chunk, self.sink.data_ptr(), self._st())
        assert rc == 0, rc


def _cold_times(probe, fn, steps):
    """Per-call times (ms) of fn() with the caches evicted before each call:
    the eviction read, then events around fn, all on the current stream."""
    import torch
    stream = torch.cuda.current_stream()
    evs = []
    for _ in range(steps):
        probe.evict()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def _read_ceiling(probe, k, v, wl, chunk):
    """Cold-cache read rate of K and V of the workload: a plain streaming
    read, and the scorer's ring structure (its grid and tiles, no arithmetic)."""
    import numpy as np
    nbytes = k.numel() * k.element_size()
    assert v.numel() * v.element_size() == nbytes
    plain = np.median(_cold_times(probe, lambda: (probe.read(k.data_ptr(), nbytes), probe.read(v.data_ptr(), nbytes)), 7))
    n = int(wl.lens[0])
    ring = np.median(_cold_times(probe, lambda: probe.ring(k, v, wl.Hkv, n, chunk), 7))
    return {"plain_read_GBs": 2 * nbytes / (plain * 1e-3) / 1e9, "scorer_ring_GBs": 2 * nbytes / (ring * 1e-3) / 1e9,
            "bytes": 2 * nbytes, "ring_chunk_keys": chunk,
            "note": "K and V of the workload read once with the caches evicted by a 1 GiB read; plain: 16-byte "
                    "loads from 2048 workgroups; ring: the scorer's 2-stage LDS ring of 64-key tiles, one 4-wave "
                    "workgroup per (KV head, key chunk), no arithmetic"}


def _eviction_leg(wl, args, probe, headline=False):
    """Score + select + compact of one layer of `wl`, timed with the caches
    evicted before every step (the headline figures) and back to back."""
    import numpy as np
    import torch
    from long_context_attention_kvevict_amd import kvevict as K
    from long_context_attention_kvevict_amd import synth

    print(f"# generating {wl.name}", file=sys.stderr, flush=True)
    data = synth.generate(wl)
    dev = torch.device("cuda:0")
    b = K.Batch(wl.lens, wl.Hq, wl.Hkv, wl.d, wl.w, wl.dtype, device=dev)
    q = K.to_device(data["q_win"], wl.dtype, dev)
    k = K.to_device(data["k"], wl.dtype, dev)
    v = K.to_device(data["v"], wl.dtype, dev)
    budgets = wl.budgets()
    caps = wl.caps()
    bud = b.offsets(budgets, dev)
    cap = b.offsets(caps, dev)
    mode = K.KVE_TOPK if wl.mode == "topk" else K.KVE_SAMPLE
    total_B, total_C = int(budgets.sum()), int(caps.sum())
    scores = torch.empty((wl.Hkv, wl.T), dtype=torch.float32, device=dev)
    sel = (torch.empty((wl.Hkv, max(total_B, 1)), dtype=torch.int32, device=dev),
           torch.empty((wl.Hkv, max(total_B, 1)), dtype=torch.float32, device=dev),
           torch.empty((wl.S, wl.Hkv), dtype=torch.float64, device=dev),
           torch.empty((wl.S, wl.Hkv), dtype=torch.int32, device=dev))
    cmp = (torch.empty((wl.Hkv, total_C, wl.d), dtype=k.dtype, device=dev),
           torch.empty((wl.Hkv, total_C, wl.d), dtype=v.dtype, device=dev),
           torch.empty((wl.Hkv, total_C), dtype=torch.float32, device=dev))
    score_kind = args.score_kind if headline else "perturb"
    pool_mode = args.pool_mode if headline else "max"
    # the output-aware score with max pooling goes through the one-call
    # eviction (kvevict_evict: the same outputs as the three calls, fewer
    # launches); the other score kinds and mean pooling through the three
    one_call = score_kind == "perturb" and pool_mode == "max"
    evout = (scores, *sel, *cmp)

    def step3():
        b.score(q, k, v, wl.sm_scale, causal=True, pool_kernel=wl.pool_kernel, out=scores, score_kind=score_kind,
                pool_mode=pool_mode)
        idx, bias, _, _ = b.select(scores, budgets, mode=mode, tau=wl.tau, tau_w=wl.tau_w, seed=wl.hash_seed,
                                   out=sel, bud_offsets=bud)
        b.compact(k, v, budgets, idx, bias, caps, out=cmp, bud_offsets=bud, cap_offsets=cap)

    def step1():
        b.evict(q, k, v, wl.sm_scale, budgets, caps, mode=mode, pool_kernel=wl.pool_kernel, tau=wl.tau,
                tau_w=wl.tau_w, seed=wl.hash_seed, out=evout, bud_offsets=bud, cap_offsets=cap)

    step = step1 if one_call else step3

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.cold_only:
        cold = _cold_times(probe, step, args.steps)
        return {"workload": wl.name, "ms_per_step": float(np.median(cold)), "steps": args.steps,
                "timing": "cold caches (1 GiB read before each step), no library events"}, None
    run = step
    if args.graph and headline:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(2):
            run()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    esize = 2 if wl.dtype == "bf16" else 4
    sbytes = _stage_bytes(wl, esize, score_kind)
    K_ = args.steps

    def cold_stages(stages):
        """Mean per-launch time of `stages` over K cold steps (library events
        on its launch stream around those kernels only)."""
        K.timing_enable(stages)
        _cold_times(probe, step, K_)
        out = K.timing_summary()
        K.timing_enable(False)
        return out

    # 1. every stage, cold: names the dominant kernel, gives its launch time
    # for the roofline and the rows (events between all kernels; the kernel
    # trace of the same cold steps agrees within a few per cent)
    stages = cold_stages(list(K.STAGES))
    dominant = max((st for st in stages if st in sbytes), key=lambda st: stages[st][0])
    dom_ms = stages[dominant][0]
    # 2. the step, cold, no library events: the headline step time
    cold = _cold_times(probe, run, K_)
    ms = float(np.median(cold))
    # 3. events around the dominant kernel only (one event pair in the step)
    dom_only_ms = cold_stages([dominant])[dominant][0]
    # 4. back to back (warm caches; the next step re-reads what the last left)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K_):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_warm = e0.elapsed_time(e1) / K_
    # 5. the previous round's flush (a 512 MiB device write before each step):
    # its dirty lines are written back while the step runs
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    wf = []
    for i in range(K_):
        scratch.fill_(i & 0xff)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        run()
        a1.record(stream)
        wf.append((a0, a1))
    torch.cuda.synchronize()
    ms_write_flushed = float(np.median([x.elapsed_time(y) for x, y in wf]))
    del scratch
    # 6. the one call against the same step as three calls (score, select,
    # compact), cold, alternating step by step
    vs_three = None
    if one_call:
        step3()   # its workspaces
        t1, t3 = [], []
        for _ in range(K_):
            t1 += _cold_times(probe, step1, 1)
            t3 += _cold_times(probe, step3, 1)
        vs_three = {"one_call_ms": float(np.median(t1)), "three_calls_ms": float(np.median(t3)), "pairs": K_}
    print(f"# {wl.name}: {ms:.4f} ms/step cold (median of {K_}), {ms_warm:.4f} warm; dominant {dominant} "
          f"{dom_ms * 1e3:.1f} us cold; stages {stages}", file=sys.stderr, flush=True)

    achieved = sbytes[dominant] / (dom_ms * 1e-3) / 1e9
    flops = _stage_flops(wl, score_kind).get(dominant) if wl.dtype == "bf16" else None
    tflops = flops / (dom_ms * 1e-3) / 1e12 if flops else None
    if flops and flops / sbytes[dominant] > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "kernel": dominant, "achieved": tflops, "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": tflops / MFMA_PEAK_TFLOPS, "traffic": _traffic(dominant, wl.name),
                "algorithmic_flops": flops, "algorithmic_bytes": sbytes[dominant], "launch_ms": dom_ms,
                "hbm_frac": achieved / HBM_PEAK_GBS}
    else:
        roof = {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": _traffic(dominant, wl.name),
                "algorithmic_bytes": sbytes[dominant], "launch_ms": dom_ms}
        if flops:
            roof["algorithmic_flops"] = flops
            roof["mfma_frac"] = tflops / MFMA_PEAK_TFLOPS
    roof["timing"] = (f"mean per-launch time over {K_} cold-cache steps, HIP events on the launch stream around "
                      f"every kernel of the step")
    roof["launch_ms_events_around_it_only"] = dom_only_ms
    # the pooling's bytes count whether it runs as a launch or inside the selection's first pass
    step_bytes = sum(sbytes[st] for st in ("score_pass1", "score_pass2", "score_pool", "select", "compact"))
    rows = {}
    for st, rec in stages.items():
        if st in sbytes:
            gbs = sbytes[st] / (rec[0] * 1e-3) / 1e9
            rows[st] = {"ms": round(rec[0], 5), "algorithmic_bytes": sbytes[st], "GB/s": round(gbs, 1),
                        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
            f = _stage_flops(wl, score_kind).get(st) if wl.dtype == "bf16" else None
            if f:
                rows[st]["mfma_frac"] = round(f / (rec[0] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)
    res = {
        "workload": wl.name, "S": wl.S, "n": int(max(wl.lens)), "T": int(wl.T), "Hq": wl.Hq, "Hkv": wl.Hkv,
        "d": wl.d, "w": wl.w, "dtype": wl.dtype, "mode": wl.mode, "budget_frac": wl.budget_frac,
        "ms_per_step": ms, "tokens_per_s": wl.T / (ms * 1e-3),
        "ms_per_step_cold_min": float(np.min(cold)),
        "ms_per_step_warm": ms_warm, "tokens_per_s_warm": wl.T / (ms_warm * 1e-3),
        "ms_per_step_write_flushed_median": ms_write_flushed,
        "step_call": "kvevict_evict" if one_call else "kvevict_score + kvevict_select + kvevict_compact",
        "one_call_vs_three_calls": vs_three,
        "roofline": roof,
        "step_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "stage_ms": {name: round(rec[0], 5) for name, rec in stages.items()},
        "rows": rows,
    }
    extra = {"b": b, "k": k, "v": v, "q": q, "sel": sel, "budgets": budgets, "data": data,
             "score_ws": int(b._lib.kvevict_score_workspace(ctypes.byref(b.layout)))}
    return res, extra


def _decode_graph(b, run_once, steps):
    """The decode loop of `steps` steps captured as one HIP graph; returns ms
    per step of its replay (appends + decode, every kernel of every step)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_once()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps / steps


def main():
    args = _parse()
    if args.copy_probe:
        _copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from long_context_attention_kvevict_amd import workloads

    dev = torch.device("cuda:0")
    probe = Probe(dev)
    wl = workloads.ALL[args.workload]()
    head, ex = _eviction_leg(wl, args, probe, headline=True)
    if args.cold_only:
        print(json.dumps(head), flush=True)
        return
    b, k, v = ex["b"], ex["k"], ex["v"]
    roof = head["roofline"]
    result = {
        "metric": "scored KV tokens/sec per layer (score+select+compact) at n=128K; % HBM peak",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "S": wl.S, "n": int(max(wl.lens)), "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "d": wl.d, "w": wl.w, "budget_frac": wl.budget_frac, "mode": wl.mode,
                   "pool_kernel": wl.pool_kernel, "score_kind": args.score_kind, "pool_mode": args.pool_mode,
                   "parallelism": "none (1 GPU)",
                   "launch": "hip graph replay" if args.graph else "eager",
                   "timing": f"median of {args.steps} steps, caches evicted before each step by a 1 GiB read"},
        "roofline": roof,
    }
    for key in ("ms_per_step_cold_min", "ms_per_step_warm", "tokens_per_s_warm", "ms_per_step_write_flushed_median",
                "step_call", "one_call_vs_three_calls", "step_hbm_frac", "stage_ms", "rows"):
        result[key] = head[key]
    # device scratch of the scorer (the pages quote the scoring path's
    # intermediate memory at n = 128K); caller-owned, reused every step
    result["score_workspace_bytes"] = ex["score_ws"]
    if wl.dtype == "bf16" and wl.S == 1 and wl.lens[0] % 2048 == 0:
        result["read_ceiling"] = _read_ceiling(probe, k, v, wl, 2048)
        result["read_ceiling"]["dominant_frac_of_plain_read"] = (
            roof["algorithmic_bytes"] / (roof["launch_ms"] * 1e-3) / 1e9 / result["read_ceiling"]["plain_read_GBs"])
    # needles planted by the generator that the selection kept (context only)
    data = ex["data"]
    if data.get("needle_pos"):
        idx_h = ex["sel"][0].cpu().numpy()
        boff = wl.bud_off()
        kept = tot = 0
        for (s_, h_), pos in data["needle_pos"].items():
            chosen = set(idx_h[h_, boff[s_]:boff[s_ + 1]].tolist())
            kept += sum(int(p_) in chosen for p_ in pos)
            tot += len(pos)
        result["needle_recall"] = kept / max(tot, 1)
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = _cpu_baseline(wl, data, max(1, min(args.cpu_heads, wl.Hkv)))
    merge_data = {"k": data["k"][:1].copy()}   # KV head 0 for the merge leg's oracle sample
    del data, ex["data"]
    if not args.no_merge:
        print("# merge leg", file=sys.stderr, flush=True)
        sel, budgets = ex["sel"], ex["budgets"]
        total_B = int(budgets.sum())
        result["merge"] = _merge_leg(b, k, budgets, sel[0][:, :total_B], sel[1][:, :total_B], wl)
        if not args.no_cpu_baseline:
            result["merge"]["cpu_baseline"] = _merge_cpu(merge_data, wl, sel[0][:, :total_B].cpu().numpy(), budgets,
                                                         result["merge"]["tau_merge"])
    del ex, b, k, v
    torch.cuda.empty_cache()
    # the other workloads, each timed the same way (cold-cache median)
    names = [] if args.configs == "none" else (
        [n for n in workloads.ALL if n != args.workload] if args.configs == "all" else args.configs.split(","))
    if names:
        result["configs"] = {}
        for name in names:
            res, ex2 = _eviction_leg(workloads.ALL[name](), args, probe)
            result["configs"][name] = res
            del ex2
            torch.cuda.empty_cache()
    if not args.no_decode:
        print("# decode leg", file=sys.stderr, flush=True)
        result["decode"] = _decode_leg(args.decode_steps, not args.no_cpu_baseline)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
