"""Thin ctypes binding of libkvevict.so.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory (tensors, workspaces) and the stream.  The
binding fails loudly if the shared library is missing; there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libkvevict.so")

KVE_OK, KVE_EINVAL, KVE_ENOTSUP, KVE_EWORKSPACE, KVE_EHIP, KVE_ENOCONV = range(6)
KVE_BF16, KVE_F32 = 0, 1
KVE_TOPK, KVE_SAMPLE = 0, 1
SCORE_KINDS = {"perturb": 0, "h2o": 1, "h2o_h": 2, "tova": 3, "min": 4, "min_h": 5, "knorm": 6}
POOL_MODES = {"max": 0, "avg": 1}

EXPORTS = [
    "kvevict_score_workspace", "kvevict_score", "kvevict_score_ex", "kvevict_select_workspace", "kvevict_select",
    "kvevict_select_ex", "kvevict_select_soft", "kvevict_select_literal_workspace", "kvevict_select_literal",
    "kvevict_merge_workspace", "kvevict_merge",
    "kvevict_compact", "kvevict_evict_workspace", "kvevict_evict", "kvevict_decode_workspace", "kvevict_decode_snis", "kvevict_decode_scratch_max",
    "kvevict_decode_snis_noalloc", "kvevict_decode_snis_append", "kvevict_last_error",
    "kvevict_version", "kvevict_timing_enable", "kvevict_timing_summary",
]

STAGES = ["score_pass1", "score_merge", "score_pass2", "score_pool", "select", "compact",
          "decode_split", "decode_merge"]


class KveLayout(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("w", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("seq_off", ctypes.c_void_p), ("seq_off_host", ctypes.c_void_p),
    ]


class KvevictError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libkvevict.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or _LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"libkvevict.so not found at {path}; build it with "
                          "`python -m long_context_attention_kvevict_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, U64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
    LP = ctypes.POINTER(KveLayout)
    lib.kvevict_score_workspace.argtypes = [LP]
    lib.kvevict_score_workspace.restype = SZ
    lib.kvevict_score.argtypes = [LP, P, P, P, F32, I32, I32, P, P, SZ, P]
    lib.kvevict_score.restype = I32
    lib.kvevict_score_ex.argtypes = [LP, P, P, P, F32, I32, I32, I32, I32, P, P, SZ, P]
    lib.kvevict_score_ex.restype = I32
    lib.kvevict_select_workspace.argtypes = [LP, P, I32]
    lib.kvevict_select_workspace.restype = SZ
    lib.kvevict_select.argtypes = [LP, P, P, P, I32, F32, F32, U64, P, P, P, P, P, SZ, P]
    lib.kvevict_select.restype = I32
    lib.kvevict_select_ex.argtypes = [LP, P, P, P, I32, F32, F32, F32, U64, P, P, P, P, P, SZ, P]
    lib.kvevict_select_ex.restype = I32
    lib.kvevict_select_soft.argtypes = [LP, P, P, P, P, P, F32, F32, F32, U64, P, P, P, P, P, P, SZ, P]
    lib.kvevict_select_soft.restype = I32
    lib.kvevict_select_literal_workspace.argtypes = [LP]
    lib.kvevict_select_literal_workspace.restype = SZ
    lib.kvevict_select_literal.argtypes = [LP, P, P, P, P, F32, F32, F32, U64, P, P, P, P, P, SZ, P]
    lib.kvevict_select_literal.restype = I32
    lib.kvevict_merge_workspace.argtypes = [LP, P]
    lib.kvevict_merge_workspace.restype = SZ
    lib.kvevict_merge.argtypes = [LP, P, P, P, P, F32, P, P, P, P, SZ, P]
    lib.kvevict_merge.restype = I32
    lib.kvevict_compact.argtypes = [LP, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.kvevict_compact.restype = I32
    lib.kvevict_evict_workspace.argtypes = [LP, P, I32]
    lib.kvevict_evict_workspace.restype = SZ
    lib.kvevict_evict.argtypes = [LP, P, P, P, F32, I32, I32, P, P, I32, F32, F32, U64, P, P, P, P, P, P, P, P, P,
                                  P, P, SZ, P]
    lib.kvevict_evict.restype = I32
    lib.kvevict_decode_workspace.argtypes = [LP, I32]
    lib.kvevict_decode_workspace.restype = SZ
    lib.kvevict_decode_snis.argtypes = [LP, P, P, P, P, P, P, P, I32, F32, P, P, SZ, P]
    lib.kvevict_decode_snis.restype = I32
    lib.kvevict_decode_scratch_max.argtypes = []
    lib.kvevict_decode_scratch_max.restype = SZ
    lib.kvevict_decode_snis_noalloc.argtypes = [LP, P, P, P, P, P, P, P, I32, F32, P, P]
    lib.kvevict_decode_snis_noalloc.restype = I32
    lib.kvevict_decode_snis_append.argtypes = [LP, P, P, P, P, P, P, P, P, P, I32, F32, P, P, SZ, P]
    lib.kvevict_decode_snis_append.restype = I32
    lib.kvevict_last_error.argtypes = []
    lib.kvevict_last_error.restype = ctypes.c_char_p
    lib.kvevict_version.argtypes = []
    lib.kvevict_version.restype = I32
    lib.kvevict_timing_enable.argtypes = [I32]
    lib.kvevict_timing_enable.restype = I32
    lib.kvevict_timing_summary.argtypes = [P, P, I32]
    lib.kvevict_timing_summary.restype = I32
    _lib = lib
    return lib


def timing_enable(on=True):
    """on: True (every stage), False (off), or a list of stage names."""
    if on is True:
        mask = (1 << len(STAGES)) - 1
    elif not on:
        mask = 0
    else:
        mask = sum(1 << STAGES.index(name) for name in on)
    _check(load_library().kvevict_timing_enable(mask))


def timing_summary() -> dict:
    """Mean per-launch duration (ms) and launch count of each stage since
    timing_enable(True)."""
    n = len(STAGES)
    avg = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(load_library().kvevict_timing_summary(ctypes.cast(avg, ctypes.c_void_p),
                                                 ctypes.cast(cnt, ctypes.c_void_p), n))
    return {STAGES[i]: (avg[i], cnt[i]) for i in range(n) if cnt[i]}


def _check(st: int):
    if st != KVE_OK:
        raise KvevictError(st, load_library().kvevict_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ws(nbytes: int, device) -> torch.Tensor:
    # 256-byte aligned allocation (torch's caching allocator aligns to >= 512)
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class Batch:
    """Shape of a ragged batch plus its offsets on host and device.

    seq_lens: per-sequence token counts.  Keeps the host offsets alive for
    the C calls and mirrors them on the device.
    """

    def __init__(self, seq_lens, Hq: int, Hkv: int, d: int, w: int, dtype: str,
                 device="cuda"):
        self.lens = [int(x) for x in seq_lens]
        self.S = len(self.lens)
        self.Hq, self.Hkv, self.d, self.w = Hq, Hkv, d, w
        self.dtype = KVE_BF16 if dtype == "bf16" else KVE_F32
        self.device = torch.device(device)
        off = [0]
        for n in self.lens:
            off.append(off[-1] + n)
        self.T = off[-1]
        self.seq_off_host = torch.tensor(off, dtype=torch.int32)
        self.seq_off = self.seq_off_host.to(self.device)
        self.layout = KveLayout(self.S, Hq, Hkv, d, w, self.dtype, self.seq_off.data_ptr(),
                                self.seq_off_host.data_ptr())
        self._lib = load_library()
        self._ws_cache = {}

    @staticmethod
    def offsets(counts, device):
        off = [0]
        for n in counts:
            off.append(off[-1] + int(n))
        host = torch.tensor(off, dtype=torch.int32)
        return host, host.to(device)

    def _workspace(self, key, nbytes):
        t = self._ws_cache.get(key)
        if t is None or t.numel() < nbytes:
            t = _ws(nbytes, self.device)
            self._ws_cache[key] = t
        return t

    # ------------------------------------------------------------ calls
    def score(self, q_win, k, v, sm_scale: float, causal: bool = True, pool_kernel: int = 7,
              out=None, stream=None, score_kind="perturb", pool_mode="max"):
        """score_kind: a name of SCORE_KINDS or its code; pool_mode: "max" or "avg"."""
        kind = SCORE_KINDS[score_kind] if isinstance(score_kind, str) else int(score_kind)
        pmode = POOL_MODES[pool_mode] if isinstance(pool_mode, str) else int(pool_mode)
        lay = ctypes.byref(self.layout)
        nbytes = self._lib.kvevict_score_workspace(lay)
        if nbytes == 0:
            # invalid layout: let the call report why
            nbytes = 256
        ws = self._workspace("score", nbytes)
        if out is None:
            out = torch.empty((self.Hkv, self.T), dtype=torch.float32, device=self.device)
        if kind == 0 and pmode == 0:
            st = self._lib.kvevict_score(lay, _ptr(q_win), _ptr(k), _ptr(v), float(sm_scale),
                                         int(bool(causal)), int(pool_kernel), _ptr(out), _ptr(ws),
                                         ws.numel(), _stream(stream))
        else:
            st = self._lib.kvevict_score_ex(lay, _ptr(q_win), _ptr(k), _ptr(v), float(sm_scale),
                                            int(bool(causal)), int(pool_kernel), kind, pmode, _ptr(out),
                                            _ptr(ws), ws.numel(), _stream(stream))
        _check(st)
        return out

    def select(self, scores, budgets, mode: int = KVE_TOPK, tau: float = 1.0, tau_w: float = 1.0,
               seed: int = 0, out=None, stream=None, bud_offsets=None, mix: float = 1.0):
        """budgets: per-sequence kept counts; mix < 1 mixes the sampling
        proposal with the uniform.  Returns (idx, bias, m, status)."""
        bud_host, bud_dev = bud_offsets if bud_offsets is not None else self.offsets(budgets, self.device)
        lay = ctypes.byref(self.layout)
        nbytes = self._lib.kvevict_select_workspace(lay, bud_host.data_ptr(), int(mode)) or 256
        ws = self._workspace("select", nbytes)
        total = int(bud_host[-1])
        if out is None:
            idx = torch.empty((self.Hkv, max(total, 1)), dtype=torch.int32, device=self.device)
            bias = torch.empty((self.Hkv, max(total, 1)), dtype=torch.float32, device=self.device)
            m = torch.empty((self.S, self.Hkv), dtype=torch.float64, device=self.device)
            status = torch.empty((self.S, self.Hkv), dtype=torch.int32, device=self.device)
        else:
            idx, bias, m, status = out
        seed64 = ctypes.c_uint64(seed & (2 ** 64 - 1))
        if mix == 1.0:
            st = self._lib.kvevict_select(lay, _ptr(scores), _ptr(bud_dev), bud_host.data_ptr(), int(mode),
                                          float(tau), float(tau_w), seed64, _ptr(idx), _ptr(bias), _ptr(m),
                                          _ptr(status), _ptr(ws), ws.numel(), _stream(stream))
        else:
            st = self._lib.kvevict_select_ex(lay, _ptr(scores), _ptr(bud_dev), bud_host.data_ptr(), int(mode),
                                             float(tau), float(tau_w), float(mix), seed64, _ptr(idx), _ptr(bias),
                                             _ptr(m), _ptr(status), _ptr(ws), ws.numel(), _stream(stream))
        _check(st)
        self._bud = (bud_host, bud_dev)   # keep alive until the stream has consumed them
        return idx[:, :total], bias[:, :total], m, status

    def select_soft(self, scores, budgets, caps, tau: float = 1.0, tau_w: float = 1.0, seed: int = 0,
                    mix: float = 1.0, stream=None):
        """Sampling selection with one m per sequence for all KV heads: the
        heads keep budgets[s] entries on average.  caps: output slots per
        head of each sequence (<= n_s).  Returns (idx, bias, kept, m, status);
        idx/bias are [Hkv][sum caps] with -1 / -inf in unused slots."""
        bud_host, bud_dev = self.offsets(budgets, self.device)
        cap_host, cap_dev = self.offsets(caps, self.device)
        lay = ctypes.byref(self.layout)
        nbytes = self._lib.kvevict_select_workspace(lay, bud_host.data_ptr(), KVE_SAMPLE) or 256
        ws = self._workspace("select", nbytes)
        C = int(cap_host[-1])
        idx = torch.empty((self.Hkv, max(C, 1)), dtype=torch.int32, device=self.device)
        bias = torch.empty((self.Hkv, max(C, 1)), dtype=torch.float32, device=self.device)
        kept = torch.empty((self.S, self.Hkv), dtype=torch.int32, device=self.device)
        m = torch.empty((self.S, self.Hkv), dtype=torch.float64, device=self.device)
        status = torch.empty((self.S, self.Hkv), dtype=torch.int32, device=self.device)
        _check(self._lib.kvevict_select_soft(lay, _ptr(scores), _ptr(bud_dev), bud_host.data_ptr(), _ptr(cap_dev),
                                             cap_host.data_ptr(), float(tau), float(tau_w), float(mix),
                                             ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(idx), _ptr(bias),
                                             _ptr(kept), _ptr(m), _ptr(status), _ptr(ws), ws.numel(),
                                             _stream(stream)))
        self._soft = (bud_host, bud_dev, cap_host, cap_dev)   # alive until the stream has used them
        return idx[:, :C], bias[:, :C], kept, m, status

    def select_literal(self, scores, m, caps, tau: float = 1.0, tau_w: float = 1.0, seed: int = 0,
                       mix: float = 1.0, stream=None):
        """m draws with replacement per (sequence, head) (float64 [S][Hkv] on
        the device, e.g. select()'s m); keeps the drawn entries.  Returns
        (idx, bias, kept, status) with idx/bias [Hkv][sum caps]."""
        cap_host, cap_dev = self.offsets(caps, self.device)
        lay = ctypes.byref(self.layout)
        nbytes = self._lib.kvevict_select_literal_workspace(lay) or 256
        ws = self._workspace("literal", nbytes)
        C = int(cap_host[-1])
        m = m.to(device=self.device, dtype=torch.float64).contiguous()
        idx = torch.empty((self.Hkv, max(C, 1)), dtype=torch.int32, device=self.device)
        bias = torch.empty((self.Hkv, max(C, 1)), dtype=torch.float32, device=self.device)
        kept = torch.empty((self.S, self.Hkv), dtype=torch.int32, device=self.device)
        status = torch.empty((self.S, self.Hkv), dtype=torch.int32, device=self.device)
        _check(self._lib.kvevict_select_literal(lay, _ptr(scores), _ptr(m), _ptr(cap_dev), cap_host.data_ptr(),
                                                float(tau), float(tau_w), float(mix),
                                                ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(idx), _ptr(bias),
                                                _ptr(kept), _ptr(status), _ptr(ws), ws.numel(), _stream(stream)))
        self._lit = (cap_host, cap_dev, m)
        return idx[:, :C], bias[:, :C], kept, status

    def merge(self, k, budgets, idx, bias, tau_merge: float, want_target: bool = False, stream=None):
        """Partition-conserving merge: bias (updated in place) of the kept
        entries grows by log(1 + merged).  Returns (bias, merged, target)."""
        bud_host, bud_dev = self.offsets(budgets, self.device)
        lay = ctypes.byref(self.layout)
        nbytes = self._lib.kvevict_merge_workspace(lay, bud_host.data_ptr()) or 256
        ws = self._workspace("merge", nbytes)
        idx = idx.contiguous()
        merged = torch.empty_like(idx)
        target = torch.empty((self.Hkv, self.T), dtype=torch.int32, device=self.device) if want_target else None
        _check(self._lib.kvevict_merge(lay, _ptr(k), _ptr(bud_dev), bud_host.data_ptr(), _ptr(idx), float(tau_merge),
                                       _ptr(bias), _ptr(merged), _ptr(target) if target is not None else None,
                                       _ptr(ws), ws.numel(), _stream(stream)))
        self._mrg = (bud_host, bud_dev)
        return bias, merged, target

    def compact(self, k, v, budgets, idx, bias, caps, out=None, stream=None, bud_offsets=None,
                cap_offsets=None):
        """Returns (k_c, v_c, bias_c) with per-sequence capacities caps."""
        bud_host, bud_dev = bud_offsets if bud_offsets is not None else self.offsets(budgets, self.device)
        cap_host, cap_dev = cap_offsets if cap_offsets is not None else self.offsets(caps, self.device)
        C = int(cap_host[-1])
        if out is None:
            k_c = torch.zeros((self.Hkv, C, self.d), dtype=k.dtype, device=self.device)
            v_c = torch.zeros((self.Hkv, C, self.d), dtype=v.dtype, device=self.device)
            b_c = torch.zeros((self.Hkv, C), dtype=torch.float32, device=self.device)
        else:
            k_c, v_c, b_c = out
        idx = idx.contiguous()
        bias = bias.contiguous()
        _check(self._lib.kvevict_compact(ctypes.byref(self.layout), _ptr(k), _ptr(v), _ptr(bud_dev),
                                         bud_host.data_ptr(), _ptr(idx), _ptr(bias), _ptr(cap_dev),
                                         cap_host.data_ptr(), _ptr(k_c), _ptr(v_c), _ptr(b_c),
                                         _stream(stream)))
        self._cmp = (bud_host, bud_dev, cap_host, cap_dev)
        return k_c, v_c, b_c

    def evict(self, q_win, k, v, sm_scale: float, budgets, caps, mode: int = KVE_TOPK, causal: bool = True,
              pool_kernel: int = 7, tau: float = 1.0, tau_w: float = 1.0, seed: int = 0, out=None, stream=None,
              bud_offsets=None, cap_offsets=None):
        """score + select + compact in one call (max pooling, per-head
        budgets, unmixed proposal).  out: (scores, idx, bias, m, status,
        k_c, v_c, bias_c) to reuse, or None.  Returns that tuple (idx and
        bias cut to the total budget)."""
        bud_host, bud_dev = bud_offsets if bud_offsets is not None else self.offsets(budgets, self.device)
        cap_host, cap_dev = cap_offsets if cap_offsets is not None else self.offsets(caps, self.device)
        lay = ctypes.byref(self.layout)
        nbytes = self._lib.kvevict_evict_workspace(lay, bud_host.data_ptr(), int(mode)) or 256
        ws = self._workspace("evict", nbytes)
        total, C = int(bud_host[-1]), int(cap_host[-1])
        if out is None:
            dev = self.device
            out = (torch.empty((self.Hkv, self.T), dtype=torch.float32, device=dev),
                   torch.empty((self.Hkv, max(total, 1)), dtype=torch.int32, device=dev),
                   torch.empty((self.Hkv, max(total, 1)), dtype=torch.float32, device=dev),
                   torch.empty((self.S, self.Hkv), dtype=torch.float64, device=dev),
                   torch.empty((self.S, self.Hkv), dtype=torch.int32, device=dev),
                   torch.zeros((self.Hkv, C, self.d), dtype=k.dtype, device=dev),
                   torch.zeros((self.Hkv, C, self.d), dtype=v.dtype, device=dev),
                   torch.zeros((self.Hkv, C), dtype=torch.float32, device=dev))
        sc, idx, bias, m, status, k_c, v_c, b_c = out
        _check(self._lib.kvevict_evict(lay, _ptr(q_win), _ptr(k), _ptr(v), float(sm_scale), int(bool(causal)),
                                       int(pool_kernel), _ptr(bud_dev), bud_host.data_ptr(), int(mode), float(tau),
                                       float(tau_w), ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(sc), _ptr(idx),
                                       _ptr(bias), _ptr(m), _ptr(status), _ptr(cap_dev), cap_host.data_ptr(),
                                       _ptr(k_c), _ptr(v_c), _ptr(b_c), _ptr(ws), ws.numel(), _stream(stream)))
        self._evk = (bud_host, bud_dev, cap_host, cap_dev)   # alive until the stream has used them
        return sc, idx[:, :total], bias[:, :total], m, status, k_c, v_c, b_c

    def decode(self, q, k_c, v_c, bias_c, caps, cache_len, max_cache_len: int, sm_scale: float,
               out=None, stream=None, cap_offsets=None):
        """q [S][Hq][d]; cache_len int32 device [S].  Returns out [S][Hq][d] fp32."""
        if cap_offsets is None:
            cap_offsets = self.offsets(caps, self.device)
        cap_host, cap_dev = cap_offsets
        lay = ctypes.byref(self.layout)
        nbytes = self._lib.kvevict_decode_workspace(lay, int(max_cache_len)) or 256
        ws = self._workspace("decode", nbytes)
        if out is None:
            out = torch.empty((self.S, self.Hq, self.d), dtype=torch.float32, device=self.device)
        _check(self._lib.kvevict_decode_snis(lay, _ptr(q), _ptr(k_c), _ptr(v_c), _ptr(bias_c), _ptr(cap_dev),
                                             cap_host.data_ptr(), _ptr(cache_len), int(max_cache_len),
                                             float(sm_scale), _ptr(out), _ptr(ws), ws.numel(),
                                             _stream(stream)))
        self._dec = (cap_host, cap_dev)
        return out

    def decode_append(self, q, k_new, v_new, k_c, v_c, bias_c, caps, cache_len, max_cache_len: int,
                      sm_scale: float, out=None, stream=None, cap_offsets=None):
        """kvevict_decode_snis_append: one decode step that attends to and
        stores the step's token (k_new, v_new [Hkv][S][d]) at slot
        cache_len[s] and advances cache_len (int32 device [S]) on the device.
        Returns out [S][Hq][d] fp32."""
        if cap_offsets is None:
            cap_offsets = self.offsets(caps, self.device)
        cap_host, cap_dev = cap_offsets
        lay = ctypes.byref(self.layout)
        nbytes = self._lib.kvevict_decode_workspace(lay, int(max_cache_len)) or 256
        ws = self._workspace("decode", nbytes)
        if out is None:
            out = torch.empty((self.S, self.Hq, self.d), dtype=torch.float32, device=self.device)
        _check(self._lib.kvevict_decode_snis_append(lay, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_c), _ptr(v_c),
                                                    _ptr(bias_c), _ptr(cap_dev), cap_host.data_ptr(),
                                                    _ptr(cache_len), int(max_cache_len), float(sm_scale), _ptr(out),
                                                    _ptr(ws), ws.numel(), _stream(stream)))
        self._dec = (cap_host, cap_dev)
        return out

    def decode_noalloc(self, q, k_c, v_c, bias_c, cap_offsets, cache_len, max_cache_len: int, sm_scale: float,
                       out, stream=None):
        """kvevict_decode_snis_noalloc: the same decode with the library's
        per-device scratch instead of a workspace; nothing is allocated
        (the caller passes `out` and the capacity offsets (host, device))."""
        cap_host, cap_dev = cap_offsets
        _check(self._lib.kvevict_decode_snis_noalloc(ctypes.byref(self.layout), _ptr(q), _ptr(k_c), _ptr(v_c),
                                                     _ptr(bias_c), _ptr(cap_dev), cap_host.data_ptr(),
                                                     _ptr(cache_len), int(max_cache_len), float(sm_scale),
                                                     _ptr(out), _stream(stream)))
        return out


def to_device(arr, dtype: str, device="cuda") -> torch.Tensor:
    """Stored input bits (numpy uint16 bf16 bits or float32) -> device tensor."""
    import numpy as np
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)
