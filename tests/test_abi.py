"""CPU checks of the C ABI: the library loads without a GPU, exports every entry point
declared in include/ea.h, reports its tile shapes and workspace sizes, and rejects bad
arguments on the host with the documented status before any HIP call (so fake, never
dereferenced pointers are safe here)."""
import ctypes
import os
import re

import pytest
import torch

from full_attention_long_amd import ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails validation


def header_functions():
    text = open(os.path.join(ROOT, "include", "ea.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ea_[a-z_0-9]+)\s*\(", text)))


def test_exports_match_header():
    L = ea.lib()
    names = header_functions()
    assert set(names) == set(ea.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_tile_config_and_workspace():
    assert ea.tile_config(ea.EA_BF16, 128) == (256, 64)
    assert ea.tile_config(ea.EA_BF16, 64) == (256, 64)
    assert ea.tile_config(ea.EA_F32, 64) == (64, 32)
    assert ea.tile_config(ea.EA_F32, 96) == (0, 0)
    assert ea.tile_config(7, 128) == (0, 0)
    a = ea.workspace_size(1, 32768, 32)
    b = ea.workspace_size(1, 32768, 32, 1024, 256)
    c = ea.workspace_size(4, 32768, 32)
    assert 0 < a <= b and a < c
    assert ea.workspace_size(0, 10, 1) == 0 and ea.workspace_size(1, -1, 1) == 0
    for s in range(5):
        assert ea.status_string(s)
    assert ea.status_string(99) == "unknown status"


def prefill(**kw):
    args = dict(q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000, o=FAKE + 0x3000, dt=ea.EA_BF16,
                cu=FAKE, cu_host=None, batch=1, max_seqlen=128, hq=4, hkv=2, d=128,
                route=FAKE, sink=4, window=16, scale=0.0, lse=None, wl=None, wlcap=0, ws=FAKE,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return ea.lib().ea_hybrid_attn_prefill(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ea.EA_ERR_INVALID_ARG),
    (dict(ws=None), ea.EA_ERR_INVALID_ARG),
    (dict(route=None), ea.EA_ERR_INVALID_ARG),
    (dict(dt=5), ea.EA_ERR_INVALID_ARG),
    (dict(batch=0), ea.EA_ERR_INVALID_ARG),
    (dict(max_seqlen=-1), ea.EA_ERR_INVALID_ARG),
    (dict(hq=6, hkv=4), ea.EA_ERR_INVALID_ARG),
    (dict(hkv=0), ea.EA_ERR_INVALID_ARG),
    (dict(window=0), ea.EA_ERR_INVALID_ARG),
    (dict(sink=-1), ea.EA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), ea.EA_ERR_INVALID_ARG),
    (dict(d=96), ea.EA_ERR_UNSUPPORTED),
    (dict(q=FAKE + 8), ea.EA_ERR_INVALID_ARG),
    (dict(o=FAKE), ea.EA_ERR_INVALID_ARG),
    (dict(max_seqlen=1 << 24), ea.EA_ERR_UNSUPPORTED),
    (dict(ws_bytes=16), ea.EA_ERR_WORKSPACE),
    (dict(batch=1025, max_seqlen=8), ea.EA_ERR_UNSUPPORTED),
    (dict(hq=130, hkv=2), ea.EA_ERR_UNSUPPORTED),
    (dict(max_seqlen=1100000), ea.EA_ERR_UNSUPPORTED),
    (dict(wl=FAKE, wlcap=4 * 1 - 1), ea.EA_ERR_INVALID_ARG),
])
def test_prefill_rejects(kw, status):
    assert prefill(**kw) == status
    assert ea.last_error()


def test_prefill_host_cu_checks():
    bad = [(0, 200), (5, 10), (0, 10, 5)]
    for cu in bad:
        n = len(cu) - 1
        arr = (ctypes.c_int32 * len(cu))(*cu)
        assert prefill(cu_host=arr, batch=n) == ea.EA_ERR_INVALID_ARG
    # o overlapping k inside its extent
    arr = (ctypes.c_int32 * 2)(0, 100)
    assert prefill(cu_host=arr, o=FAKE + 0x1000 + 0x10) == ea.EA_ERR_INVALID_ARG


def test_route_and_worklist_reject():
    L = ea.lib()
    ok = dict(ks=FAKE, kdt=ea.EA_BF16, kv=1024, cu=FAKE, batch=1, w1=FAKE, b1=FAKE, hid=256,
              w2=FAKE, b2=FAKE, hq=32, logits=None, r=FAKE, ws=FAKE, wsb=1 << 30, st=None)
    for kw, st in [(dict(ks=None), 1), (dict(r=None), 1), (dict(kv=0), 1), (dict(kdt=3), 1),
                   (dict(ks=FAKE + 4), 1), (dict(wsb=0), 3)]:
        a = dict(ok)
        a.update(kw)
        assert L.ea_route(*a.values()) == st, kw
    okw = dict(r=FAKE, cu=FAKE, batch=1, maxlen=100, hq=4, sink=0, win=1, dt=0, d=128, wl=FAKE,
               wlcap=1 << 20, nout=None, nhost=None, ws=FAKE, wsb=1 << 30, st=None)
    for kw, st in [(dict(wl=None), 1), (dict(win=0), 1), (dict(d=80), 2), (dict(dt=9), 1),
                   (dict(wsb=8), 3), (dict(maxlen=1 << 26), 2), (dict(wlcap=3), 1)]:
        a = dict(okw)
        a.update(kw)
        assert L.ea_build_worklist(*a.values()) == st, kw


def test_run_rejects():
    L = ea.lib()
    base = [FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, 0, FAKE, 1, 128, 4, 2, 128,
            FAKE, 0, 16, 0.0, None, FAKE, 1 << 20, FAKE, 0, FAKE, 1 << 30, None]
    a = list(base)
    a[16] = None  # work list
    assert L.ea_hybrid_attn_run(*a) == ea.EA_ERR_INVALID_ARG
    a = list(base)
    a[19] = -1    # grid_blocks
    assert L.ea_hybrid_attn_run(*a) == ea.EA_ERR_INVALID_ARG
    a = list(base)
    a[17] = -1    # worklist_capacity
    assert L.ea_hybrid_attn_run(*a) == ea.EA_ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_valid_call_without_gpu_reports_hip_error():
    # every check passes, so the first HIP call runs and fails: the status is EA_ERR_HIP
    assert prefill() == ea.EA_ERR_HIP
    assert "device" in ea.last_error() or "launch" in ea.last_error()


def decode_call(**kw):
    args = dict(q=FAKE, kc=FAKE + 0x100000, vc=FAKE + 0x200000, o=FAKE + 0x10000,
                dt=ea.EA_BF16, seqlens=FAKE, seqlens_host=None, batch=2, cap=4096,
                max_seqlen=4096, hq=32, hkv=8, d=128, route=FAKE, sink=128, window=1024,
                scale=0.0, lse=None, ws=0x40000000, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return ea.lib().ea_hybrid_attn_decode(*args.values())


def test_decode_workspace_size():
    a = ea.decode_workspace_size(1, 32768, 32, 128)
    assert a >= 32 * 128 * (128 + 2) * 4  # 128 splits of 256 keys
    assert ea.decode_workspace_size(2, 32768, 32, 128) > a
    assert ea.decode_workspace_size(0, 10, 1, 128) == 0
    assert ea.decode_workspace_size(1, 0, 1, 128) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ea.EA_ERR_INVALID_ARG),
    (dict(seqlens=None), ea.EA_ERR_INVALID_ARG),
    (dict(ws=None), ea.EA_ERR_INVALID_ARG),
    (dict(dt=5), ea.EA_ERR_INVALID_ARG),
    (dict(batch=0), ea.EA_ERR_INVALID_ARG),
    (dict(max_seqlen=5000), ea.EA_ERR_INVALID_ARG),       # beyond the cache capacity
    (dict(hq=30), ea.EA_ERR_INVALID_ARG),                 # not a multiple of hkv
    (dict(hq=72), ea.EA_ERR_UNSUPPORTED),                 # 9 query heads per KV head
    (dict(d=96), ea.EA_ERR_UNSUPPORTED),
    (dict(window=0), ea.EA_ERR_INVALID_ARG),
    (dict(sink=-1), ea.EA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), ea.EA_ERR_INVALID_ARG),
    (dict(o=FAKE + 8), ea.EA_ERR_INVALID_ARG),            # misaligned
    (dict(ws=0x40000010), ea.EA_ERR_INVALID_ARG),         # workspace not 256-byte aligned
    (dict(o=FAKE + 0x100000), ea.EA_ERR_INVALID_ARG),     # o overlaps the K cache
    (dict(ws_bytes=1024), ea.EA_ERR_WORKSPACE),
    (dict(cap=1 << 20, max_seqlen=1 << 20), ea.EA_ERR_UNSUPPORTED),  # 32-bit offsets
])
def test_decode_rejects(kw, status):
    assert decode_call(**kw) == status
    assert ea.last_error()


def test_decode_host_seqlens_checks():
    bad = (ctypes.c_int32 * 2)(0, 17)
    assert decode_call(seqlens_host=bad) == ea.EA_ERR_INVALID_ARG
    bad = (ctypes.c_int32 * 2)(4097, 17)
    assert decode_call(seqlens_host=bad) == ea.EA_ERR_INVALID_ARG


# ---- pooled decode cache

def test_pool_layout():
    """Linear regions of `capacity` rows for KV heads with a full query head, sink + window
    rows for all-sparse ones, packed in (sequence, KV head) order."""
    import numpy as np
    route = np.array([[1, 1, 0, 1, 1, 1],
                      [1, 1, 1, 1, 1, 1],
                      [0, 0, 0, 0, 0, 0]], dtype=np.uint8)   # 3 sequences, 6 q heads, 3 KV heads
    base, rows, total = ea.decode_pool_layout(route, 3, capacity=1000, sink=4, window=60)
    want_rows = [64, 1000, 64, 64, 64, 64, 1000, 1000, 1000]
    assert rows.tolist() == want_rows
    assert base.tolist() == [sum(want_rows[:i]) for i in range(9)]
    assert total == sum(want_rows)
    # a ring longer than the capacity is still sink + window rows (its slot rule needs them)
    _, rows, _ = ea.decode_pool_layout(np.ones((1, 2), np.uint8), 1, capacity=10, sink=4, window=60)
    assert rows.tolist() == [64]


def test_pool_layout_rejects():
    import numpy as np
    r = np.ones((2, 4), np.uint8)
    for kw in (dict(capacity=0), dict(window=0), dict(sink=-1)):
        args = dict(capacity=100, sink=4, window=16)
        args.update(kw)
        with pytest.raises(ea.EAError):
            ea.decode_pool_layout(r, 2, **args)
    with pytest.raises(ea.EAError):
        ea.decode_pool_layout(r, 3, capacity=100, sink=4, window=16)  # 4 q heads, 3 KV heads


def pool_decode_call(**kw):
    args = dict(q=FAKE, kp=FAKE + 0x100000, vp=FAKE + 0x200000, o=FAKE + 0x10000,
                dt=ea.EA_BF16, seqlens=FAKE, seqlens_host=None, batch=2, max_seqlen=4096,
                hq=32, hkv=8, d=128, rbase=FAKE, rrows=FAKE, pool_rows=2048, route=FAKE,
                sink=128, window=1024, scale=0.0, lse=None, ws=0x40000000, ws_bytes=1 << 30,
                stream=None)
    args.update(kw)
    return ea.lib().ea_hybrid_attn_decode_pool(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ea.EA_ERR_INVALID_ARG),
    (dict(rbase=None), ea.EA_ERR_INVALID_ARG),
    (dict(rrows=None), ea.EA_ERR_INVALID_ARG),
    (dict(dt=5), ea.EA_ERR_INVALID_ARG),
    (dict(batch=0), ea.EA_ERR_INVALID_ARG),
    (dict(max_seqlen=0), ea.EA_ERR_INVALID_ARG),
    (dict(pool_rows=0), ea.EA_ERR_INVALID_ARG),
    (dict(hq=30), ea.EA_ERR_INVALID_ARG),
    (dict(hq=72), ea.EA_ERR_UNSUPPORTED),
    (dict(d=96), ea.EA_ERR_UNSUPPORTED),
    (dict(window=0), ea.EA_ERR_INVALID_ARG),
    (dict(sink=-1), ea.EA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), ea.EA_ERR_INVALID_ARG),
    (dict(kp=FAKE + 0x100008), ea.EA_ERR_INVALID_ARG),    # misaligned pool
    (dict(vp=FAKE + 0x100000), ea.EA_ERR_INVALID_ARG),    # pools overlap
    (dict(o=FAKE + 0x100000), ea.EA_ERR_INVALID_ARG),     # o overlaps the K pool
    (dict(ws=0x40000010), ea.EA_ERR_INVALID_ARG),
    (dict(ws_bytes=1024), ea.EA_ERR_WORKSPACE),
])
def test_pool_decode_rejects(kw, status):
    assert pool_decode_call(**kw) == status
    assert ea.last_error()


def test_pool_decode_host_seqlens_checks():
    bad = (ctypes.c_int32 * 2)(0, 17)
    assert pool_decode_call(seqlens_host=bad) == ea.EA_ERR_INVALID_ARG
    bad = (ctypes.c_int32 * 2)(4097, 17)
    assert pool_decode_call(seqlens_host=bad) == ea.EA_ERR_INVALID_ARG


def test_pool_writers_reject():
    L = ea.lib()
    fill = dict(k=FAKE, v=FAKE + 0x1000, dt=ea.EA_BF16, cu=FAKE, batch=2, max_seqlen=64, hq=8,
                hkv=2, d=128, route=FAKE, sink=4, window=16, rbase=FAKE, rrows=FAKE,
                pool_rows=100, kp=FAKE + 0x100000, vp=FAKE + 0x200000, stream=None)
    for kw in (dict(k=None), dict(cu=None), dict(max_seqlen=0), dict(d=32), dict(hq=7),
               dict(pool_rows=0), dict(k=FAKE + 4), dict(vp=FAKE + 0x100010)):
        a = dict(fill)
        a.update(kw)
        assert L.ea_decode_pool_fill(*a.values()) != ea.EA_OK, kw
    app = dict(k=FAKE, v=FAKE + 0x1000, dt=ea.EA_BF16, pos=FAKE, batch=2, hq=8, hkv=2, d=128,
               route=FAKE, sink=4, window=16, rbase=FAKE, rrows=FAKE, pool_rows=100,
               kp=FAKE + 0x100000, vp=FAKE + 0x200000, stream=None)
    for kw in (dict(pos=None), dict(batch=0), dict(window=0), dict(dt=3), dict(v=FAKE + 8)):
        a = dict(app)
        a.update(kw)
        assert L.ea_decode_pool_append(*a.values()) != ea.EA_OK, kw


def chunked_call(**kw):
    args = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, o=FAKE + 0x3000000,
                dt=ea.EA_BF16, cu_q=FAKE, cu_k=FAKE + 0x100, cu_q_host=None, cu_k_host=None,
                batch=2, max_q=1024, max_k=4096, hq=32, hkv=8, d=128, route=FAKE, sink=128,
                window=1024, scale=0.0, lse=None, wl=None, wl_cap=0, ws=0x40000000,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return ea.lib().ea_hybrid_attn_prefill_chunked(*args.values())


def test_chunked_prefill_rejects():
    assert chunked_call(cu_k=None) == ea.EA_ERR_INVALID_ARG
    assert chunked_call(max_q=5000) == ea.EA_ERR_INVALID_ARG           # beyond max_seqlen_k
    assert chunked_call(max_q=-1) == ea.EA_ERR_INVALID_ARG
    assert chunked_call(d=96) == ea.EA_ERR_UNSUPPORTED
    assert chunked_call(o=FAKE + 0x1000000) == ea.EA_ERR_INVALID_ARG   # o is k
    assert chunked_call(wl=FAKE, wl_cap=10) == ea.EA_ERR_INVALID_ARG   # work list too short
    assert chunked_call(ws_bytes=16) == ea.EA_ERR_WORKSPACE
    q_host = (ctypes.c_int32 * 3)(0, 100, 150)
    assert chunked_call(cu_q_host=q_host) == ea.EA_ERR_INVALID_ARG     # only one host copy
    k_host = (ctypes.c_int32 * 3)(0, 90, 300)                          # 100 queries, 90 keys
    assert chunked_call(cu_q_host=q_host, cu_k_host=k_host) == ea.EA_ERR_INVALID_ARG
    k_host = (ctypes.c_int32 * 3)(0, 5000, 5100)                       # a key sequence > max_k
    assert chunked_call(cu_q_host=q_host, cu_k_host=k_host) == ea.EA_ERR_INVALID_ARG
    assert ea.last_error()


def test_chunked_workspace_size():
    a = ea.prefill_chunked_workspace_size(1, 4096, 32, 128)
    assert a >= 512 * 256 * 128 * 4 + ea.workspace_size(1, 4096, 32)
    assert ea.prefill_chunked_workspace_size(1, 4096, 32, 64) < a
    assert ea.prefill_chunked_workspace_size(0, 4096, 32, 128) == 0


def backward_call(**kw):
    args = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, o=FAKE + 0x3000000,
                do=FAKE + 0x4000000, dt=ea.EA_BF16, lse=FAKE + 0x5000000, cu_q=FAKE,
                cu_k=None, cu_q_host=None, cu_k_host=None, batch=1, max_q=1024, max_k=1024,
                hq=32, hkv=8, d=128, route=FAKE, sink=128, window=1024, scale=0.0,
                dq=FAKE + 0x6000000, dk=FAKE + 0x7000000, dv=FAKE + 0x8000000, ws=0x40000000,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return ea.lib().ea_hybrid_attn_backward(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ea.EA_ERR_INVALID_ARG),
    (dict(lse=None), ea.EA_ERR_INVALID_ARG),
    (dict(dq=None), ea.EA_ERR_INVALID_ARG),
    (dict(ws=None), ea.EA_ERR_INVALID_ARG),
    (dict(dt=7), ea.EA_ERR_INVALID_ARG),
    (dict(batch=0), ea.EA_ERR_INVALID_ARG),
    (dict(max_q=2048), ea.EA_ERR_INVALID_ARG),        # beyond max_seqlen_k
    (dict(hq=12, hkv=8), ea.EA_ERR_INVALID_ARG),
    (dict(window=0), ea.EA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), ea.EA_ERR_INVALID_ARG),
    (dict(d=96), ea.EA_ERR_UNSUPPORTED),
    (dict(dk=FAKE + 0x7000004), ea.EA_ERR_INVALID_ARG),  # misaligned
    (dict(ws=0x40000010), ea.EA_ERR_INVALID_ARG),         # workspace not 256-aligned
    (dict(dv=FAKE + 0x7000000), ea.EA_ERR_INVALID_ARG),   # dv is dk
    (dict(ws_bytes=1024), ea.EA_ERR_WORKSPACE),
])
def test_backward_rejects(kw, status):
    assert backward_call(**kw) == status
    assert ea.last_error()


def test_backward_host_checks():
    q_host = (ctypes.c_int32 * 2)(0, 100)
    # a gradient overlapping an input inside its extent
    assert backward_call(cu_q_host=q_host, dq=FAKE + 0x1000000 + 0x100) == ea.EA_ERR_INVALID_ARG
    # only one host copy with an explicit key packing
    assert backward_call(cu_k=FAKE + 0x100, cu_q_host=q_host) == ea.EA_ERR_INVALID_ARG
    k_host = (ctypes.c_int32 * 2)(0, 90)                     # chunk of 100 rows over 90 keys
    assert backward_call(cu_k=FAKE + 0x100, cu_q_host=q_host,
                         cu_k_host=k_host) == ea.EA_ERR_INVALID_ARG
    long_host = (ctypes.c_int32 * 2)(0, 2000)                 # longer than max_seqlen_q
    assert backward_call(cu_q_host=long_host) == ea.EA_ERR_INVALID_ARG


def test_backward_sequence_length_limit():
    # bf16: one sequence's q rows (all heads) must fit 2^31 bytes; 256K at 32 x 128 is the edge
    big = dict(max_q=262145, max_k=262145, ws_bytes=1 << 40)
    assert backward_call(**big) == ea.EA_ERR_UNSUPPORTED
    # fp32 (64-bit indexing) has no such limit: the same sizes pass the host checks
    if torch.cuda.device_count() == 0:
        assert backward_call(dt=ea.EA_F32, **big) == ea.EA_ERR_HIP
        assert backward_call(max_q=262144, max_k=262144, ws_bytes=1 << 40) == ea.EA_ERR_HIP


def test_backward_workspace_size():
    f = ea.attn_backward_workspace_size
    a = f(ea.EA_F32, 2, 4096, 4096, 32, 8, 128)
    assert a >= 2 * 4096 * 32 * 4
    # bf16 with 4 query heads per KV head: plus per-head dk and dv partials
    b = f(ea.EA_BF16, 2, 4096, 8192, 32, 8, 128)
    assert b >= a + 2 * 2 * 8192 * 32 * 128 * 4
    assert f(ea.EA_BF16, 2, 4096, 8192, 8, 8, 128) < b      # one query head per KV head
    assert f(ea.EA_F32, 0, 4096, 4096, 32, 8, 128) == 0
    assert f(ea.EA_F32, 1, -1, 4096, 32, 8, 128) == 0
    assert f(ea.EA_F32, 1, 4096, 1024, 32, 8, 128) == 0     # max_seqlen_q > max_seqlen_k
    assert f(7, 1, 16, 16, 4, 2, 64) == 0


def route_backward_call(**kw):
    args = dict(ks=FAKE, kdt=ea.EA_BF16, kv=1024, cu=FAKE, batch=2, w1=FAKE, b1=FAKE, hid=256,
                w2=FAKE, b2=FAKE, hq=32, of=FAKE, osp=FAKE, do=FAKE, odt=ea.EA_BF16, d=128,
                noise=None, tau=1.0, dr=None, dz=FAKE, dw1=FAKE, db1=FAKE, dw2=FAKE, db2=FAKE,
                dks=None, ws=0x40000000, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return ea.lib().ea_route_backward(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), ea.EA_ERR_INVALID_ARG),
    (dict(dz=None), ea.EA_ERR_INVALID_ARG),
    (dict(dw1=None), ea.EA_ERR_INVALID_ARG),
    (dict(of=None), ea.EA_ERR_INVALID_ARG),
    (dict(odt=4), ea.EA_ERR_INVALID_ARG),
    (dict(kv=0), ea.EA_ERR_INVALID_ARG),
    (dict(d=80), ea.EA_ERR_UNSUPPORTED),
    (dict(tau=0.0), ea.EA_ERR_INVALID_ARG),
    (dict(tau=float("nan")), ea.EA_ERR_INVALID_ARG),
    (dict(dks=FAKE, kv=1022), ea.EA_ERR_UNSUPPORTED),
    (dict(do=FAKE + 2), ea.EA_ERR_INVALID_ARG),
    (dict(ws=0x40000004), ea.EA_ERR_INVALID_ARG),
    (dict(ws_bytes=64), ea.EA_ERR_WORKSPACE),
])
def test_route_backward_rejects(kw, status):
    assert route_backward_call(**kw) == status
    assert ea.last_error()


def test_route_backward_workspace_size():
    a = ea.route_backward_workspace_size(2, 1024, 256, 32, 128)
    assert a >= 2 * (2 * 1024 + 3 * 256) * 4
    assert ea.route_backward_workspace_size(0, 1024, 256, 32, 128) == 0
    assert ea.route_backward_workspace_size(2, 1024, 256, 32, 128) < \
        ea.route_backward_workspace_size(4, 1024, 256, 32, 128)


def test_binding_rejects_host_and_strided_tensors():
    import torch
    assert ea._ptr(None) is None and ea._ptr(1234) == 1234
    with pytest.raises(ValueError, match="GPU tensor"):
        ea._ptr(torch.zeros(4, 4))
    with pytest.raises(ValueError, match="GPU tensor"):
        ea._ptr(torch.zeros(4, 4).t())


def test_binding_rejects_mismatched_tensors():
    import torch
    q = torch.zeros(8, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(8, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    args = (cu, 8, torch.zeros(1, 4, dtype=torch.uint8), 0, 16, torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="dtypes differ"):
        ea.hybrid_attn_prefill(q, k, k.float(), q, *args)
    with pytest.raises(ValueError, match="shapes differ"):
        ea.hybrid_attn_prefill(q, k, k, q[:4], *args)
    with pytest.raises(ValueError, match="head_dim differs"):
        ea.hybrid_attn_prefill(q, k[..., :32], k[..., :32], q, *args)


def test_binding_rejects_wrong_small_arrays():
    import torch
    q = torch.zeros(8, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(8, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="route_bits: expected 4 elements"):
        ea.hybrid_attn_prefill(q, k, k, q, cu, 8, torch.zeros(1, 3, dtype=torch.uint8), 0, 16, ws)
    with pytest.raises(ValueError, match="cu_seqlens: expected int32"):
        ea.hybrid_attn_prefill(q, k, k, q, cu.long(), 8, torch.zeros(1, 4, dtype=torch.uint8), 0,
                               16, ws)
    with pytest.raises(ValueError, match="lse_out: expected 32 elements"):
        ea.hybrid_attn_prefill(q, k, k, q, cu, 8, torch.zeros(1, 4, dtype=torch.uint8), 0, 16, ws,
                               lse_out=torch.zeros(4, 7))


def test_binding_rejects_router_shape_mismatch():
    import torch
    ks = torch.zeros(8, 16, dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    w1, b1 = torch.zeros(4, 16), torch.zeros(4)
    w2, b2 = torch.zeros(3, 4), torch.zeros(3)
    out, ws = torch.zeros(1, 3, dtype=torch.uint8), torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="w1: expected shape"):
        ea.route(ks, cu, torch.zeros(4, 15), b1, w2, b2, out, ws)
    with pytest.raises(ValueError, match="b2: expected shape"):
        ea.route(ks, cu, w1, b1, w2, torch.zeros(4), out, ws)
    with pytest.raises(ValueError, match="route_out: expected 3 elements"):
        ea.route(ks, cu, w1, b1, w2, b2, torch.zeros(1, 2, dtype=torch.uint8), ws)


def test_chunked_plan_limit_counts_chunk_rows():
    """The planner tiles the chunk's rows, so its cell bound uses max_seqlen_q: 8 sequences
    of 256K cached keys with 4K-row chunks pass every host check up to the workspace size
    (2 * 8 * ceil(262144 / 256) cells would exceed the planner, 2 * 8 * 16 do not)."""
    st = chunked_call(batch=8, max_q=4096, max_k=262144, ws_bytes=16)
    assert st == ea.EA_ERR_WORKSPACE, ea.last_error()
    need = ea.prefill_chunked_workspace_size(8, 4096, 32, 128)
    assert need > 0
    # beyond the planner's cells by the chunk rows themselves: still rejected
    assert chunked_call(batch=8, max_q=262144, max_k=262144) == ea.EA_ERR_UNSUPPORTED


def test_binding_rejects_pool_mismatch():
    """The pool writers take the row size from k and the row count from k_pool: a pool of
    another dtype or width, or region arrays of the wrong type or length, are refused before
    the C call (these tensors never reach the GPU)."""
    import torch
    B, hkv, d = 2, 2, 64
    k = torch.zeros(5, hkv, d, dtype=torch.bfloat16)
    kp = torch.zeros(40, d, dtype=torch.bfloat16)
    cu = torch.tensor([0, 3, 5], dtype=torch.int32)
    route = torch.zeros(B, 4, dtype=torch.uint8)
    base = torch.zeros(B * hkv, dtype=torch.int64)
    rows = torch.zeros(B * hkv, dtype=torch.int32)
    with pytest.raises(ValueError, match="k, k_pool: dtypes differ"):
        ea.decode_pool_fill(k.float(), k.float(), cu, 3, 4, route, 4, 16, base, rows, kp, kp)
    with pytest.raises(ValueError, match="k_pool, v_pool: shapes differ"):
        ea.decode_pool_fill(k, k, cu, 3, 4, route, 4, 16, base, rows, kp, kp[:20])
    with pytest.raises(ValueError, match="k_pool: expected"):
        ea.decode_pool_fill(k, k, cu, 3, 4, route, 4, 16, base, rows, kp[:, :32], kp[:, :32])
    with pytest.raises(ValueError, match="region_base: expected int64"):
        ea.decode_pool_fill(k, k, cu, 3, 4, route, 4, 16, base.int(), rows, kp, kp)
    with pytest.raises(ValueError, match="region_rows: expected 4 elements"):
        ea.decode_pool_fill(k, k, cu, 3, 4, route, 4, 16, base, rows[:3], kp, kp)
    kn = torch.zeros(B, hkv, d, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="positions: expected int32"):
        ea.decode_pool_append(kn, kn, torch.zeros(B, dtype=torch.int64), 4, route, 4, 16, base,
                              rows, kp, kp)
    with pytest.raises(ValueError, match="k, v: shapes differ"):
        ea.decode_pool_append(kn, kn[:1], torch.zeros(B, dtype=torch.int32), 4, route, 4, 16,
                              base, rows, kp, kp)
