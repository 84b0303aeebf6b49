"""Thin ctypes binding of libea.so (include/ea.h).  Argument marshalling only: every step
of the path runs in the library's HIP kernels.  Tensors are torch tensors on the GPU
(torch supplies device memory and the current stream); the functions keep the C names
without the ``ea_`` prefix.  A non-OK status raises :class:`EAError`.

The library must have been built (``python -m full_attention_long_amd.build``); if it is
missing, loading raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libea.so")

EA_OK, EA_ERR_INVALID_ARG, EA_ERR_UNSUPPORTED, EA_ERR_WORKSPACE, EA_ERR_HIP = range(5)
EA_BF16, EA_F32 = 0, 1

EXPORTS = ("ea_workspace_size", "ea_tile_config", "ea_status_string", "ea_last_error",
           "ea_route", "ea_build_worklist", "ea_hybrid_attn_prefill", "ea_hybrid_attn_run",
           "ea_decode_workspace_size", "ea_hybrid_attn_decode", "ea_decode_pool_layout",
           "ea_decode_pool_fill", "ea_decode_pool_append", "ea_hybrid_attn_decode_pool",
           "ea_hybrid_attn_prefill_chunked", "ea_prefill_chunked_workspace_size",
           "ea_attn_backward_workspace_size", "ea_hybrid_attn_backward",
           "ea_route_backward_workspace_size", "ea_route_backward",
           "ea_hybrid_attn_prefill_noalloc")

_lib = None


class EAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)} ({status}): {detail}")
        self.status = status
        self.detail = detail


def lib():
    """Load libea.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} not found: build it with python -m full_attention_long_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    L.ea_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.ea_workspace_size.restype = sz
    L.ea_tile_config.argtypes = [i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.ea_tile_config.restype = None
    L.ea_status_string.argtypes = [i32]
    L.ea_status_string.restype = ctypes.c_char_p
    L.ea_last_error.argtypes = []
    L.ea_last_error.restype = ctypes.c_char_p
    L.ea_route.argtypes = [P, i32, i32, P, i32, P, P, i32, P, P, i32, P, P, P, sz, P]
    L.ea_route.restype = i32
    i64 = ctypes.c_int64
    L.ea_build_worklist.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, P, i64, P, P, P,
                                    sz, P]
    L.ea_build_worklist.restype = i32
    L.ea_hybrid_attn_prefill.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, P,
                                         i32, i32, f32, P, P, i64, P, sz, P]
    L.ea_hybrid_attn_prefill.restype = i32
    L.ea_hybrid_attn_prefill_noalloc.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, i32,
                                                 P, i32, i32, f32, P, P, i64, P]
    L.ea_hybrid_attn_prefill_noalloc.restype = i32
    L.ea_hybrid_attn_run.argtypes = [P, P, P, P, i32, P, i32, i32, i32, i32, i32, P, i32, i32,
                                     f32, P, P, i64, P, i32, P, sz, P]
    L.ea_hybrid_attn_run.restype = i32
    L.ea_decode_workspace_size.argtypes = [i32, i32, i32, i32]
    L.ea_decode_workspace_size.restype = sz
    L.ea_hybrid_attn_decode.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, P,
                                        i32, i32, f32, P, P, sz, P]
    L.ea_hybrid_attn_decode.restype = i32
    L.ea_hybrid_attn_prefill_chunked.argtypes = [P, P, P, P, i32, P, P, P, P, i32, i32, i32, i32,
                                                 i32, i32, P, i32, i32, f32, P, P, i64, P, sz,
                                                 P]
    L.ea_hybrid_attn_prefill_chunked.restype = i32
    L.ea_prefill_chunked_workspace_size.argtypes = [i32, i32, i32, i32]
    L.ea_prefill_chunked_workspace_size.restype = sz
    L.ea_decode_pool_layout.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P]
    L.ea_decode_pool_layout.restype = i32
    L.ea_decode_pool_fill.argtypes = [P, P, i32, P, i32, i32, i32, i32, i32, P, i32, i32, P, P,
                                      i64, P, P, P]
    L.ea_decode_pool_fill.restype = i32
    L.ea_decode_pool_append.argtypes = [P, P, i32, P, i32, i32, i32, i32, P, i32, i32, P, P, i64,
                                        P, P, P]
    L.ea_decode_pool_append.restype = i32
    L.ea_hybrid_attn_decode_pool.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, P, P,
                                             i64, P, i32, i32, f32, P, P, sz, P]
    L.ea_hybrid_attn_decode_pool.restype = i32
    L.ea_attn_backward_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.ea_attn_backward_workspace_size.restype = sz
    L.ea_hybrid_attn_backward.argtypes = [P, P, P, P, P, i32, P, P, P, P, P, i32, i32, i32, i32,
                                          i32, i32, P, i32, i32, f32, P, P, P, P, sz, P]
    L.ea_hybrid_attn_backward.restype = i32
    L.ea_route_backward_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.ea_route_backward_workspace_size.restype = sz
    L.ea_route_backward.argtypes = [P, i32, i32, P, i32, P, P, i32, P, P, i32, P, P, P, i32, i32,
                                    P, f32, P, P, P, P, P, P, P, P, sz, P]
    L.ea_route_backward.restype = i32
    _lib = L
    return L


def status_string(s: int) -> str:
    return lib().ea_status_string(int(s)).decode()


def last_error() -> str:
    return lib().ea_last_error().decode()


def _check(status: int):
    if status != EA_OK:
        raise EAError(status, last_error())


def _ptr(t):
    """Device address of a tensor argument (a plain int passes through as an address).  The
    library reads dense row-major buffers in GPU memory, so a host tensor or a strided view
    raises here instead of being misread."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"expected a GPU tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"expected a contiguous tensor, got strides {tuple(t.stride())}")
    return t.data_ptr()


def _same(what, *ts, shape=True):
    """The C calls take one dtype code and the sizes of the first tensor: the others must
    match it (dtype, and shape unless shape=False), or the kernels would misread them or
    write past their end."""
    ts = [t for t in ts if t is not None and not isinstance(t, int)]
    for t in ts[1:]:
        if t.dtype != ts[0].dtype:
            raise ValueError(f"{what}: dtypes differ ({ts[0].dtype} vs {t.dtype})")
        if shape and tuple(t.shape) != tuple(ts[0].shape):
            raise ValueError(f"{what}: shapes differ ({tuple(ts[0].shape)} vs {tuple(t.shape)})")


def _qkvo(q, k, v, o):
    _same("q, o", q, o)
    _same("k, v", k, v)
    _same("q, k", q, k, shape=False)
    if k.shape[-1] != q.shape[-1]:
        raise ValueError(f"head_dim differs: q {q.shape[-1]}, k {k.shape[-1]}")


def _arr(t, dtype, numel, what):
    """A small device array argument: its dtype, and its element count where the call fixes it
    (the library cannot see either)."""
    if t is None or isinstance(t, int):
        return
    if t.dtype != getattr(__import__("torch"), dtype):
        raise ValueError(f"{what}: expected {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what}: expected {numel} elements, got {t.numel()}")


def _router_shapes(key_states, w1, b1, w2, b2):
    """w1 [H, C], b1 [H], w2 [Hq, H], b2 [Hq] fp32 with C the key-state width: the C call
    takes C from key_states, H from w1 and Hq from w2, so the others must agree."""
    C, Hh, Hq = key_states.shape[-1], w1.shape[0], w2.shape[0]
    for t, want, what in ((w1, (Hh, C), "w1"), (b1, (Hh,), "b1"), (w2, (Hq, Hh), "w2"),
                          (b2, (Hq,), "b2")):
        _arr(t, "float32", None, what)
        if tuple(t.shape) != want:
            raise ValueError(f"{what}: expected shape {want}, got {tuple(t.shape)}")
    return Hq


def _capacity(worklist):
    """Work-list capacity in items: rows of an int32 [n, 4] tensor."""
    if worklist is None or isinstance(worklist, int):
        return 0
    return worklist.numel() // 4


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return EA_BF16
    if dtype == torch.float32:
        return EA_F32
    raise TypeError(f"unsupported dtype {dtype}")


def workspace_size(batch, max_seqlen, n_heads_q, kv_dim=0, hidden=0) -> int:
    return int(lib().ea_workspace_size(batch, max_seqlen, n_heads_q, kv_dim, hidden))


def tile_config(dt: int, head_dim: int):
    bm, bn = ctypes.c_int32(0), ctypes.c_int32(0)
    lib().ea_tile_config(int(dt), int(head_dim), ctypes.byref(bm), ctypes.byref(bn))
    return bm.value, bn.value


def route(key_states, cu_seqlens, w1, b1, w2, b2, route_out, workspace, logits_out=None,
          stream=None):
    """ea_route: key_states [T, C] (bf16/fp32), w1 [H, C], b1 [H], w2 [Hq, H], b2 [Hq] fp32;
    writes route_out [B, Hq] uint8 and optionally logits_out [B, Hq] fp32."""
    batch = cu_seqlens.numel() - 1
    hq = _router_shapes(key_states, w1, b1, w2, b2)
    _arr(cu_seqlens, "int32", None, "cu_seqlens")
    _arr(route_out, "uint8", batch * hq, "route_out")
    _arr(logits_out, "float32", batch * hq, "logits_out")
    _check(lib().ea_route(_ptr(key_states), dtype_code(key_states.dtype), key_states.shape[-1],
                          _ptr(cu_seqlens), batch, _ptr(w1), _ptr(b1), w1.shape[0],
                          _ptr(w2), _ptr(b2), w2.shape[0], _ptr(logits_out), _ptr(route_out),
                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                          _stream(stream)))


def build_worklist(route_bits, cu_seqlens, max_seqlen, n_heads_q, sink, window, dt, head_dim,
                   worklist_out, workspace, n_items_out=None, want_count=True, stream=None):
    """ea_build_worklist; returns the item count when want_count (synchronises)."""
    batch = cu_seqlens.numel() - 1
    n_host = ctypes.c_int32(-1)
    _check(lib().ea_build_worklist(_ptr(route_bits), _ptr(cu_seqlens), batch, max_seqlen,
                                   n_heads_q, sink, window, int(dt), head_dim,
                                   _ptr(worklist_out), _capacity(worklist_out), _ptr(n_items_out),
                                   ctypes.byref(n_host) if want_count else None,
                                   _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(stream)))
    return n_host.value if want_count else None


def hybrid_attn_prefill(q, k, v, o, cu_seqlens, max_seqlen, route_bits, sink, window,
                        workspace, scale=0.0, cu_seqlens_host=None, lse_out=None,
                        worklist_out=None, stream=None):
    """ea_hybrid_attn_prefill: q/o [T, Hq, D], k/v [T, Hkv, D] (bf16 or fp32)."""
    _qkvo(q, k, v, o)
    _arr(cu_seqlens, "int32", None, "cu_seqlens")
    _arr(route_bits, "uint8", (cu_seqlens.numel() - 1) * q.shape[1], "route_bits")
    _arr(lse_out, "float32", q.shape[1] * q.shape[0], "lse_out")
    batch = cu_seqlens.numel() - 1
    host = None
    if cu_seqlens_host is not None:
        host = (ctypes.c_int32 * (batch + 1))(*[int(x) for x in cu_seqlens_host])
    _check(lib().ea_hybrid_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), dtype_code(q.dtype),
                                        _ptr(cu_seqlens), host, batch, max_seqlen,
                                        q.shape[1], k.shape[1], q.shape[2], _ptr(route_bits),
                                        sink, window, float(scale), _ptr(lse_out),
                                        _ptr(worklist_out), _capacity(worklist_out),
                                        _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)))


def hybrid_attn_prefill_noalloc(q, k, v, o, cu_seqlens, max_seqlen, route_bits, sink, window,
                                scale=0.0, cu_seqlens_host=None, lse_out=None, worklist_out=None,
                                stream=None):
    """ea_hybrid_attn_prefill_noalloc: ea_hybrid_attn_prefill without a workspace argument
    (the library's device-resident scratch; the call allocates nothing)."""
    _qkvo(q, k, v, o)
    _arr(cu_seqlens, "int32", None, "cu_seqlens")
    _arr(route_bits, "uint8", (cu_seqlens.numel() - 1) * q.shape[1], "route_bits")
    _arr(lse_out, "float32", q.shape[1] * q.shape[0], "lse_out")
    batch = cu_seqlens.numel() - 1
    host = None
    if cu_seqlens_host is not None:
        host = (ctypes.c_int32 * (batch + 1))(*[int(x) for x in cu_seqlens_host])
    _check(lib().ea_hybrid_attn_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), dtype_code(q.dtype), _ptr(cu_seqlens), host, batch,
        max_seqlen, q.shape[1], k.shape[1], q.shape[2], _ptr(route_bits), sink, window,
        float(scale), _ptr(lse_out), _ptr(worklist_out), _capacity(worklist_out),
        _stream(stream)))


def hybrid_attn_run(q, k, v, o, cu_seqlens, max_seqlen, route_bits, sink, window, worklist,
                    n_items, workspace, scale=0.0, lse_out=None, grid_blocks=0, stream=None):
    """ea_hybrid_attn_run on a work list from build_worklist (n_items: device int32)."""
    _qkvo(q, k, v, o)
    _arr(cu_seqlens, "int32", None, "cu_seqlens")
    _arr(route_bits, "uint8", (cu_seqlens.numel() - 1) * q.shape[1], "route_bits")
    _arr(lse_out, "float32", q.shape[1] * q.shape[0], "lse_out")
    batch = cu_seqlens.numel() - 1
    _check(lib().ea_hybrid_attn_run(_ptr(q), _ptr(k), _ptr(v), _ptr(o), dtype_code(q.dtype),
                                    _ptr(cu_seqlens), batch, max_seqlen, q.shape[1], k.shape[1],
                                    q.shape[2], _ptr(route_bits), sink, window, float(scale),
                                    _ptr(lse_out), _ptr(worklist), _capacity(worklist),
                                    _ptr(n_items),
                                    int(grid_blocks), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(stream)))


def decode_workspace_size(batch, max_seqlen, n_heads_q, head_dim) -> int:
    return int(lib().ea_decode_workspace_size(batch, max_seqlen, n_heads_q, head_dim))


def hybrid_attn_decode(q, k_cache, v_cache, o, seqlens, max_seqlen, route_bits, sink, window,
                       workspace, scale=0.0, seqlens_host=None, lse_out=None, stream=None):
    """ea_hybrid_attn_decode: q/o [B, Hq, D], k_cache/v_cache [B, cap, Hkv, D] (bf16 or fp32),
    seqlens [B] int32 device."""
    _qkvo(q, k_cache, v_cache, o)
    _arr(seqlens, "int32", q.shape[0], "seqlens")
    _arr(route_bits, "uint8", q.shape[0] * q.shape[1], "route_bits")
    _arr(lse_out, "float32", q.shape[0] * q.shape[1], "lse_out")
    batch = q.shape[0]
    host = None
    if seqlens_host is not None:
        host = (ctypes.c_int32 * batch)(*[int(x) for x in seqlens_host])
    _check(lib().ea_hybrid_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o),
                                       dtype_code(q.dtype), _ptr(seqlens), host, batch,
                                       k_cache.shape[1], max_seqlen, q.shape[1], k_cache.shape[2],
                                       q.shape[2], _ptr(route_bits), sink, window, float(scale),
                                       _ptr(lse_out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream)))


def decode_pool_layout(route_host, n_heads_kv, capacity, sink, window):
    """ea_decode_pool_layout on a host routing [B, Hq] (uint8 tensor or array): returns
    (region_base int64 [B*Hkv], region_rows int32 [B*Hkv], total_rows) as CPU tensors / int."""
    import numpy as np
    import torch
    r = np.ascontiguousarray(np.asarray(route_host, dtype=np.uint8))
    batch, hq = r.shape
    base = torch.empty(batch * n_heads_kv, dtype=torch.int64)
    rows = torch.empty(batch * n_heads_kv, dtype=torch.int32)
    total = ctypes.c_int64(0)
    _check(lib().ea_decode_pool_layout(r.ctypes.data, batch, hq, n_heads_kv, capacity, sink, window,
                                       base.data_ptr(), rows.data_ptr(), ctypes.byref(total)))
    return base, rows, int(total.value)


def _pool_args(k, v, k_pool, v_pool, region_base, region_rows, route_bits, batch):
    """The pool writers take the row size from k and the pool's row count from k_pool: the
    pools must hold rows of k's dtype and head_dim, the region arrays one entry per
    (sequence, KV head), or the kernels would write past the pool's end."""
    _same("k, v", k, v)
    _same("k_pool, v_pool", k_pool, v_pool)
    _same("k, k_pool", k, k_pool, shape=False)
    if k_pool.dim() != 2 or k_pool.shape[1] != k.shape[-1]:
        raise ValueError(f"k_pool: expected [rows, {k.shape[-1]}], got {tuple(k_pool.shape)}")
    n_regions = batch * k.shape[1]
    _arr(region_base, "int64", n_regions, "region_base")
    _arr(region_rows, "int32", n_regions, "region_rows")
    _arr(route_bits, "uint8", None, "route_bits")
    if route_bits is not None and not isinstance(route_bits, int) and route_bits.dim() == 2 \
            and route_bits.shape[0] != batch:
        raise ValueError(f"route_bits: expected {batch} rows, got {route_bits.shape[0]}")


def decode_pool_fill(k, v, cu_seqlens, max_seqlen, n_heads_q, route_bits, sink, window,
                     region_base, region_rows, k_pool, v_pool, stream=None):
    """ea_decode_pool_fill: k/v [T, Hkv, D] packed by cu_seqlens into k_pool/v_pool [rows, D]."""
    _arr(cu_seqlens, "int32", None, "cu_seqlens")
    _pool_args(k, v, k_pool, v_pool, region_base, region_rows, route_bits, cu_seqlens.numel() - 1)
    _check(lib().ea_decode_pool_fill(_ptr(k), _ptr(v), dtype_code(k.dtype), _ptr(cu_seqlens),
                                     cu_seqlens.numel() - 1, max_seqlen, n_heads_q, k.shape[1],
                                     k.shape[2], _ptr(route_bits), sink, window,
                                     _ptr(region_base), _ptr(region_rows), k_pool.shape[0],
                                     _ptr(k_pool), _ptr(v_pool), _stream(stream)))


def decode_pool_append(k_new, v_new, positions, n_heads_q, route_bits, sink, window,
                       region_base, region_rows, k_pool, v_pool, stream=None):
    """ea_decode_pool_append: k_new/v_new [B, Hkv, D] at positions [B] (int32 device)."""
    _arr(positions, "int32", k_new.shape[0], "positions")
    _pool_args(k_new, v_new, k_pool, v_pool, region_base, region_rows, route_bits,
               k_new.shape[0])
    _check(lib().ea_decode_pool_append(_ptr(k_new), _ptr(v_new), dtype_code(k_new.dtype),
                                       _ptr(positions), k_new.shape[0], n_heads_q, k_new.shape[1],
                                       k_new.shape[2], _ptr(route_bits), sink, window,
                                       _ptr(region_base), _ptr(region_rows), k_pool.shape[0],
                                       _ptr(k_pool), _ptr(v_pool), _stream(stream)))


def hybrid_attn_decode_pool(q, k_pool, v_pool, o, seqlens, max_seqlen, n_heads_kv, region_base,
                            region_rows, route_bits, sink, window, workspace, scale=0.0,
                            seqlens_host=None, lse_out=None, stream=None):
    """ea_hybrid_attn_decode_pool: q/o [B, Hq, D]; k_pool/v_pool [rows, D]; regions from
    decode_pool_layout (device copies)."""
    _qkvo(q, k_pool, v_pool, o)
    _arr(seqlens, "int32", q.shape[0], "seqlens")
    _arr(route_bits, "uint8", q.shape[0] * q.shape[1], "route_bits")
    _arr(lse_out, "float32", q.shape[0] * q.shape[1], "lse_out")
    batch = q.shape[0]
    host = None
    if seqlens_host is not None:
        host = (ctypes.c_int32 * batch)(*[int(x) for x in seqlens_host])
    _check(lib().ea_hybrid_attn_decode_pool(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(o),
                                            dtype_code(q.dtype), _ptr(seqlens), host, batch,
                                            max_seqlen, q.shape[1], n_heads_kv, q.shape[2],
                                            _ptr(region_base), _ptr(region_rows), k_pool.shape[0],
                                            _ptr(route_bits), sink, window, float(scale),
                                            _ptr(lse_out), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(),
                                            _stream(stream)))


def hybrid_attn_prefill_chunked(q, k, v, o, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                max_seqlen_k, route_bits, sink, window, workspace, scale=0.0,
                                cu_seqlens_q_host=None, cu_seqlens_k_host=None, lse_out=None,
                                worklist_out=None, stream=None):
    """ea_hybrid_attn_prefill_chunked: q/o [Tq, Hq, D] (each sequence's last Lq positions),
    k/v [Tk, Hkv, D] packed by cu_seqlens_k."""
    _qkvo(q, k, v, o)
    _arr(cu_seqlens_q, "int32", None, "cu_seqlens_q")
    _arr(cu_seqlens_k, "int32", cu_seqlens_q.numel(), "cu_seqlens_k")
    _arr(route_bits, "uint8", (cu_seqlens_q.numel() - 1) * q.shape[1], "route_bits")
    _arr(lse_out, "float32", q.shape[1] * q.shape[0], "lse_out")
    batch = cu_seqlens_q.numel() - 1
    hq = hk = None
    if cu_seqlens_q_host is not None:
        hq = (ctypes.c_int32 * (batch + 1))(*[int(x) for x in cu_seqlens_q_host])
        hk = (ctypes.c_int32 * (batch + 1))(*[int(x) for x in cu_seqlens_k_host])
    _check(lib().ea_hybrid_attn_prefill_chunked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), dtype_code(q.dtype), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), hq, hk, batch, max_seqlen_q, max_seqlen_k, q.shape[1], k.shape[1],
        q.shape[2], _ptr(route_bits), sink, window, float(scale), _ptr(lse_out),
        _ptr(worklist_out), _capacity(worklist_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def prefill_chunked_workspace_size(batch, max_seqlen_q, n_heads_q, head_dim) -> int:
    return int(lib().ea_prefill_chunked_workspace_size(batch, max_seqlen_q, n_heads_q, head_dim))


def attn_backward_workspace_size(dt, batch, max_seqlen_q, max_seqlen_k, n_heads_q, n_heads_kv,
                                 head_dim) -> int:
    return int(lib().ea_attn_backward_workspace_size(dt, batch, max_seqlen_q, max_seqlen_k,
                                                     n_heads_q, n_heads_kv, head_dim))


def _host_cu(cu, batch):
    if cu is None:
        return None
    return (ctypes.c_int32 * (batch + 1))(*[int(x) for x in cu])


def hybrid_attn_backward(q, k, v, o, dout, lse, cu_seqlens_q, max_seqlen_q, route_bits, sink,
                         window, dq, dk, dv, workspace, scale=0.0, cu_seqlens_k=None,
                         max_seqlen_k=None, cu_seqlens_q_host=None, cu_seqlens_k_host=None,
                         stream=None):
    """ea_hybrid_attn_backward: q/o/dout [Tq, Hq, D], k/v [Tk, Hkv, D] (one dtype), lse
    [Hq, Tq] from the forward; dq/dk/dv fp32 outputs of the shapes of q/k/v."""
    _qkvo(q, k, v, o)
    _same("q, dout", q, dout)
    _same("dq, dk, dv (fp32)", dq, dk, dv, shape=False)
    _same("dk, dv", dk, dv)
    _arr(cu_seqlens_q, "int32", None, "cu_seqlens_q")
    _arr(cu_seqlens_k, "int32", cu_seqlens_q.numel(), "cu_seqlens_k")
    _arr(route_bits, "uint8", (cu_seqlens_q.numel() - 1) * q.shape[1], "route_bits")
    _arr(lse, "float32", q.shape[1] * q.shape[0], "lse")
    if dq.dtype.itemsize != 4 or tuple(dq.shape) != tuple(q.shape) or tuple(dk.shape) != tuple(k.shape):
        raise ValueError("dq, dk, dv must be fp32 with the shapes of q, k, v")
    batch = cu_seqlens_q.numel() - 1
    if max_seqlen_k is None:
        max_seqlen_k = max_seqlen_q
    _check(lib().ea_hybrid_attn_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), dtype_code(q.dtype), _ptr(lse),
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _host_cu(cu_seqlens_q_host, batch),
        _host_cu(cu_seqlens_k_host, batch), batch, max_seqlen_q, max_seqlen_k, q.shape[1],
        k.shape[1], q.shape[2], _ptr(route_bits), sink, window, float(scale), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def route_backward_workspace_size(batch, kv_dim, hidden, n_heads_q, head_dim) -> int:
    return int(lib().ea_route_backward_workspace_size(batch, kv_dim, hidden, n_heads_q,
                                                      head_dim))


def route_backward(key_states, cu_seqlens, w1, b1, w2, b2, o_full, o_sparse, dout, dz, dw1,
                   db1, dw2, db2, workspace, tau=1.0, noise=None, dr_out=None,
                   dkey_states=None, stream=None):
    """ea_route_backward: key_states [T, C]; o_full/o_sparse/dout [T, Hq, D] (one dtype);
    fp32 outputs dz [B, Hq], dw1 [H, C], db1 [H], dw2 [Hq, H], db2 [Hq], optional dr_out
    [B, Hq] and dkey_states [T, C]."""
    batch = cu_seqlens.numel() - 1
    hq = _router_shapes(key_states, w1, b1, w2, b2)
    _arr(cu_seqlens, "int32", None, "cu_seqlens")
    _same("o_full, o_sparse, dout", o_full, o_sparse, dout)
    if dout.dim() != 3 or dout.shape[1] != hq or dout.shape[0] != key_states.shape[0]:
        raise ValueError(f"dout: expected [{key_states.shape[0]}, {hq}, D], got {tuple(dout.shape)}")
    for t, want, what in ((dz, (batch, hq), "dz"), (dw1, tuple(w1.shape), "dw1"),
                          (db1, tuple(b1.shape), "db1"), (dw2, tuple(w2.shape), "dw2"),
                          (db2, tuple(b2.shape), "db2"), (dr_out, (batch, hq), "dr_out"),
                          (noise, (batch, hq), "noise"),
                          (dkey_states, tuple(key_states.shape), "dkey_states")):
        if t is None or isinstance(t, int):
            continue
        _arr(t, "float32", None, what)
        if tuple(t.shape) != want:
            raise ValueError(f"{what}: expected shape {want}, got {tuple(t.shape)}")
    _check(lib().ea_route_backward(
        _ptr(key_states), dtype_code(key_states.dtype), key_states.shape[1], _ptr(cu_seqlens),
        batch, _ptr(w1), _ptr(b1), w1.shape[0], _ptr(w2), _ptr(b2), w2.shape[0], _ptr(o_full),
        _ptr(o_sparse), _ptr(dout), dtype_code(dout.dtype), dout.shape[2], _ptr(noise),
        float(tau), _ptr(dr_out), _ptr(dz), _ptr(dw1), _ptr(db1), _ptr(dw2), _ptr(db2),
        _ptr(dkey_states), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
