"""CPU tier: the C-ABI library loads, exports every declared entry point, and
rejects invalid arguments on the host before any launch."""
import ctypes
import os
import re

import pytest
import torch

from long_context_attention_kvevict_amd import kvevict as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvevict.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kvevict_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("kvevict_score", "kvevict_select", "kvevict_compact", "kvevict_decode_snis"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = K.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(K.EXPORTS) == set(_declared_functions())
    assert lib.kvevict_version() == 100


def _layout(S=1, Hq=4, Hkv=2, d=128, w=8, dtype=K.KVE_BF16, lens=(100,)):
    off = [0]
    for n in lens:
        off.append(off[-1] + n)
    host = torch.tensor(off, dtype=torch.int32)
    lay = K.KveLayout(S, Hq, Hkv, d, w, dtype, host.data_ptr(), host.data_ptr())
    return lay, host


DUMMY = 0x1000   # never dereferenced: validation fails first


def _score(lay, **kw):
    lib = K.load_library()
    args = dict(q=DUMMY, k=DUMMY, v=DUMMY, scale=0.1, causal=1, pool=7, out=DUMMY, ws=DUMMY,
                ws_bytes=1 << 40)
    args.update(kw)
    return lib.kvevict_score(ctypes.byref(lay), args["q"], args["k"], args["v"], args["scale"], args["causal"],
                             args["pool"], args["out"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("field,value,status", [
    ("Hq", 5, K.KVE_EINVAL), ("w", 0, K.KVE_EINVAL), ("w", 65, K.KVE_EINVAL), ("d", 64, K.KVE_ENOTSUP),
    ("d", 96, K.KVE_ENOTSUP), ("dtype", 7, K.KVE_EINVAL), ("S", 0, K.KVE_EINVAL),
])
def test_score_rejects_bad_layout(field, value, status):
    lay, keep = _layout()
    setattr(lay, field, value)
    assert _score(lay) == status
    assert K.load_library().kvevict_last_error().startswith(b"kvevict_score")


def test_score_rejects_bad_arguments():
    lay, keep = _layout()
    assert _score(lay, q=None) == K.KVE_EINVAL
    assert _score(lay, pool=6) == K.KVE_EINVAL
    assert _score(lay, pool=33) == K.KVE_EINVAL
    assert _score(lay, scale=0.0) == K.KVE_EINVAL
    assert _score(lay, ws_bytes=16) == K.KVE_EWORKSPACE
    assert _score(lay, k=DUMMY + 8) == K.KVE_EINVAL          # misaligned
    lay2, keep2 = _layout(lens=(5,))                          # w > n
    assert _score(lay2) == K.KVE_EINVAL
    lay3, keep3 = _layout(S=2, lens=(50, 0))                  # empty sequence
    assert _score(lay3) == K.KVE_EINVAL


def _score_ex(lay, kind, pool_mode, ws_bytes=1 << 40):
    lib = K.load_library()
    return lib.kvevict_score_ex(ctypes.byref(lay), DUMMY, DUMMY, DUMMY, 0.1, 1, 7, kind, pool_mode, DUMMY, DUMMY,
                                ws_bytes, None)


def test_score_ex_rejects_bad_kind_and_pool_mode():
    lay, keep = _layout()
    assert _score_ex(lay, 7, 0) == K.KVE_EINVAL
    assert _score_ex(lay, -1, 0) == K.KVE_EINVAL
    assert _score_ex(lay, 1, 2) == K.KVE_EINVAL
    assert K.load_library().kvevict_last_error().startswith(b"kvevict_score")
    # attention-weight kinds are bf16-only; fp32 reports "not supported"
    lay32, keep32 = _layout(dtype=K.KVE_F32)
    for kind in range(1, 6):
        assert _score_ex(lay32, kind, 0) == K.KVE_ENOTSUP
    assert _score_ex(lay32, 6, 1, ws_bytes=16) == K.KVE_EWORKSPACE   # K-norm takes fp32
    # every valid kind/mode pair reaches the workspace check
    for kind in range(7):
        for mode in range(2):
            assert _score_ex(lay, kind, mode, ws_bytes=16) == K.KVE_EWORKSPACE


def test_select_rejects_bad_budgets():
    lib = K.load_library()
    lay, keep = _layout(S=2, lens=(50, 60))
    for bud, st in (([0, 51, 60], K.KVE_EINVAL), ([0, 10, 5], K.KVE_EINVAL), ([1, 10, 20], K.KVE_EINVAL)):
        b = torch.tensor(bud, dtype=torch.int32)
        r = lib.kvevict_select(ctypes.byref(lay), DUMMY, DUMMY, b.data_ptr(), 0, 1.0, 1.0, 0, DUMMY, DUMMY,
                               None, None, DUMMY, 1 << 40, None)
        assert r == st
    b = torch.tensor([0, 5, 10], dtype=torch.int32)
    r = lib.kvevict_select(ctypes.byref(lay), DUMMY, DUMMY, b.data_ptr(), 1, 0.0, 1.0, 0, DUMMY, DUMMY,
                           None, None, DUMMY, 1 << 40, None)
    assert r == K.KVE_EINVAL                                   # tau must be > 0
    r = lib.kvevict_select(ctypes.byref(lay), DUMMY, DUMMY, b.data_ptr(), 1, 0.5, 1.0, 0, DUMMY, DUMMY,
                           None, None, DUMMY, 8, None)
    assert r == K.KVE_EWORKSPACE
    r = lib.kvevict_select(ctypes.byref(lay), DUMMY, DUMMY, b.data_ptr(), 9, 0.5, 1.0, 0, DUMMY, DUMMY,
                           None, None, DUMMY, 1 << 40, None)
    assert r == K.KVE_EINVAL


def test_compact_and_decode_reject_bad_arguments():
    lib = K.load_library()
    lay, keep = _layout(S=1, lens=(50,))
    bud = torch.tensor([0, 10], dtype=torch.int32)
    cap = torch.tensor([0, 8], dtype=torch.int32)      # capacity below budget
    r = lib.kvevict_compact(ctypes.byref(lay), DUMMY, DUMMY, DUMMY, bud.data_ptr(), DUMMY, DUMMY, DUMMY,
                            cap.data_ptr(), DUMMY + 4096, DUMMY + 8192, DUMMY, None)
    assert r == K.KVE_EINVAL
    cap = torch.tensor([0, 12], dtype=torch.int32)
    r = lib.kvevict_compact(ctypes.byref(lay), DUMMY, DUMMY, DUMMY, bud.data_ptr(), DUMMY, DUMMY, DUMMY,
                            cap.data_ptr(), DUMMY, DUMMY + 8192, DUMMY, None)
    assert r == K.KVE_EINVAL                            # k_c aliases k
    r = lib.kvevict_decode_snis(ctypes.byref(lay), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, cap.data_ptr(), DUMMY,
                                13, 0.1, DUMMY, DUMMY, 1 << 40, None)
    assert r == K.KVE_EINVAL                            # max_cache_len > capacity
    assert lib.kvevict_decode_workspace(ctypes.byref(lay), 12) > 0
    r = lib.kvevict_decode_snis(ctypes.byref(lay), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, cap.data_ptr(), DUMMY,
                                12, 0.1, DUMMY, DUMMY, 16, None)
    assert r == K.KVE_EWORKSPACE
    # the appending decode validates the same way, and needs its new-token rows
    r = lib.kvevict_decode_snis_append(ctypes.byref(lay), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                       cap.data_ptr(), DUMMY, 13, 0.1, DUMMY, DUMMY, 1 << 40, None)
    assert r == K.KVE_EINVAL                            # max_cache_len > capacity
    r = lib.kvevict_decode_snis_append(ctypes.byref(lay), DUMMY, None, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                       cap.data_ptr(), DUMMY, 12, 0.1, DUMMY, DUMMY, 1 << 40, None)
    assert r == K.KVE_EINVAL                            # no k_new
    r = lib.kvevict_decode_snis_append(ctypes.byref(lay), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                       cap.data_ptr(), DUMMY, 12, 0.1, DUMMY, DUMMY, 16, None)
    assert r == K.KVE_EWORKSPACE


def test_workspace_scales_with_shape():
    lib = K.load_library()
    lay, keep = _layout(Hq=32, Hkv=8, w=32, lens=(131072,))
    big = lib.kvevict_score_workspace(ctypes.byref(lay))
    lay2, keep2 = _layout(Hq=32, Hkv=8, w=32, lens=(4096,))
    small = lib.kvevict_score_workspace(ctypes.byref(lay2))
    assert big > small > 0
    # O(w d + n) per head: far below the w x n x d intermediates of a naive scorer
    assert big < 8 * 131072 * 32 * 4 * 128 * 2 / 50


def test_select_ex_rejects_bad_mix():
    lib = K.load_library()
    lay, keep = _layout(S=2, lens=(50, 60))
    b = torch.tensor([0, 5, 10], dtype=torch.int32)
    for mix, st in ((-0.1, K.KVE_EINVAL), (1.5, K.KVE_EINVAL), (float("nan"), K.KVE_EINVAL),
                    (0.0, K.KVE_EWORKSPACE), (0.5, K.KVE_EWORKSPACE), (1.0, K.KVE_EWORKSPACE)):
        r = lib.kvevict_select_ex(ctypes.byref(lay), DUMMY, DUMMY, b.data_ptr(), 1, 0.5, 1.0, mix, 0, DUMMY,
                                  DUMMY, None, None, DUMMY, 16, None)
        assert r == st, mix


def test_select_soft_rejects_bad_capacities():
    lib = K.load_library()
    lay, keep = _layout(S=2, lens=(50, 60))
    b = torch.tensor([0, 5, 65], dtype=torch.int32)          # B_1 = n_1 = 60

    def call(caps, ws_bytes=16, tau=0.5):
        c = torch.tensor(caps, dtype=torch.int32)
        return lib.kvevict_select_soft(ctypes.byref(lay), DUMMY, DUMMY, b.data_ptr(), DUMMY, c.data_ptr(), tau,
                                       1.0, 1.0, 0, DUMMY, DUMMY, None, None, None, DUMMY, ws_bytes, None)
    assert call([0, 51, 111]) == K.KVE_EINVAL                 # cap_0 > n_0
    assert call([0, 20, 70]) == K.KVE_EINVAL                  # B_1 = n_1 but cap_1 < n_1
    assert call([1, 20, 80]) == K.KVE_EINVAL                  # cap_off[0] != 0
    assert call([0, 20, 80], tau=0.0) == K.KVE_EINVAL
    assert call([0, 20, 80]) == K.KVE_EWORKSPACE              # valid up to the workspace


def test_select_literal_rejects_bad_arguments():
    lib = K.load_library()
    lay, keep = _layout(S=2, lens=(50, 60))
    assert lib.kvevict_select_literal_workspace(ctypes.byref(lay)) > 0

    def call(caps, ws_bytes=16, tau=0.5, mix=1.0, m=DUMMY):
        c = torch.tensor(caps, dtype=torch.int32)
        return lib.kvevict_select_literal(ctypes.byref(lay), DUMMY, m, DUMMY, c.data_ptr(), tau, 1.0, mix, 0,
                                          DUMMY, DUMMY, None, None, DUMMY, ws_bytes, None)
    assert call([0, 51, 60]) == K.KVE_EINVAL                  # cap_0 > n_0
    assert call([2, 20, 60]) == K.KVE_EINVAL                  # cap_off[0] != 0
    assert call([0, 20, 60], tau=0.0) == K.KVE_EINVAL
    assert call([0, 20, 60], mix=2.0) == K.KVE_EINVAL
    assert call([0, 20, 60], m=None) == K.KVE_EINVAL
    assert call([0, 20, 60]) == K.KVE_EWORKSPACE


def test_merge_rejects_bad_arguments():
    lib = K.load_library()
    lay, keep = _layout(S=2, lens=(50, 60))
    b = torch.tensor([0, 5, 10], dtype=torch.int32)
    assert lib.kvevict_merge_workspace(ctypes.byref(lay), b.data_ptr()) > 0

    def call(lay_, bud, tau=0.5, ws_bytes=16, k=DUMMY):
        return lib.kvevict_merge(ctypes.byref(lay_), k, DUMMY, bud.data_ptr(), DUMMY, tau, DUMMY, None, None, DUMMY,
                                 ws_bytes, None)
    assert call(lay, torch.tensor([0, 51, 60], dtype=torch.int32)) == K.KVE_EINVAL   # B_0 > n_0
    assert call(lay, b, tau=1.5) == K.KVE_EINVAL
    assert call(lay, b, k=DUMMY + 8) == K.KVE_EINVAL                                  # misaligned
    assert call(lay, b) == K.KVE_EWORKSPACE
    lay32, keep32 = _layout(S=2, lens=(50, 60), dtype=K.KVE_F32)
    assert call(lay32, b) == K.KVE_ENOTSUP


def test_noalloc_decode_rejects_batches_beyond_its_scratch():
    # 8 sequences x 32 q-heads with caches of 20000 entries need about 10 MiB
    # of split partials, more than the 8 MiB the allocation-free decode
    # holds: the host check refuses before any launch (pointers unused)
    lib = K.load_library()
    assert lib.kvevict_decode_scratch_max() == 8 << 20
    lay, host = _layout(S=8, Hq=32, Hkv=8, lens=(200000,) * 8)
    cap = torch.tensor([20016 * i for i in range(9)], dtype=torch.int32)
    st = lib.kvevict_decode_snis_noalloc(ctypes.byref(lay), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, cap.data_ptr(),
                                         DUMMY, 20000, 0.1, DUMMY, None)
    assert st == K.KVE_EWORKSPACE
    assert "scratch" in lib.kvevict_last_error().decode()
    # the workspace entry point takes the same batch
    assert lib.kvevict_decode_workspace(ctypes.byref(lay), 20000) > (8 << 20)


def test_evict_rejects_bad_arguments_and_sizes_its_workspace():
    lib = K.load_library()
    lay, keep = _layout(Hq=8, Hkv=2, w=8, lens=(3000,))
    bud = torch.tensor([0, 300], dtype=torch.int32)
    cap = torch.tensor([0, 310], dtype=torch.int32)
    seed = ctypes.c_uint64(1)

    def call(pool=7, mode=K.KVE_TOPK, cap_t=cap, ws_bytes=1 << 40, tau=0.5, k_c=DUMMY + 4096):
        return lib.kvevict_evict(ctypes.byref(lay), DUMMY, DUMMY, DUMMY, 0.1, 1, pool, DUMMY, bud.data_ptr(), mode,
                                 tau, 1.0, seed, DUMMY, DUMMY, DUMMY, None, None, DUMMY, cap_t.data_ptr(), k_c,
                                 DUMMY + 8192, DUMMY, DUMMY, ws_bytes, None)
    for m in (K.KVE_TOPK, K.KVE_SAMPLE):
        need = lib.kvevict_evict_workspace(ctypes.byref(lay), bud.data_ptr(), m)
        parts = (lib.kvevict_score_workspace(ctypes.byref(lay))
                 + lib.kvevict_select_workspace(ctypes.byref(lay), bud.data_ptr(), m))
        assert parts <= need <= parts + 256
        assert call(mode=m, ws_bytes=need - 1) == K.KVE_EWORKSPACE
    assert call(pool=4) == K.KVE_EINVAL                     # even pooling width
    assert call(mode=K.KVE_SAMPLE, tau=0.0) == K.KVE_EINVAL   # tau must be > 0
    assert call(cap_t=torch.tensor([0, 299], dtype=torch.int32)) == K.KVE_EINVAL   # capacity below budget
    assert call(k_c=DUMMY) == K.KVE_EINVAL                   # k_c aliases k
    assert b"kvevict_evict" in lib.kvevict_last_error()
