"""Oracle for the routed hybrid-attention prefill -- TEST INFRASTRUCTURE ONLY.

Plain, slow fp64 CPU reference.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product library never does, and
this package imports nothing from the product package.

The arithmetic lives in ``ea_oracle.c`` (fp64, OpenMP); this module compiles it with gcc
and marshals arguments through ctypes.  The C header comment lists the pages each
function follows (Elastic Attention blog post, section 2.1 "Attention Router",
section 1 and section 3 "Fused Kernel"; gist.science explanation, section "问题所在")
and the readings taken where the pages are silent.

Functions:
  attn(...)      masked-softmax attention over explicit per-head visible sets
  decode(...)    one decode step of the same attention over a per-sequence KV cache
  route(...)     mean-pool -> MLP (SiLU) -> logits -> hard threshold
  worklist(...)  (seq, head, q_tile, cost) items, longest first
  build()        compile the C oracle (gcc -O2 -fopenmp)

Parity pins for every function are in tests/test_oracle.py (brute force, closed forms,
identities, library special cases, hand-derived router fixture).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ea_oracle.c")
_LIB = os.path.join(_HERE, "libea_oracle.so")
_lib = None

_DT_BF16, _DT_F32, _DT_F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile ea_oracle.c into oracle/libea_oracle.so with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_attn.argtypes = [P, P, P, i32, P, P, i32, i32, i32, i32, P, i32, i32, dbl,
                                    P, i64, P, P, i32]
        lib.oracle_attn.restype = i32
        lib.oracle_decode.argtypes = [P, P, P, i32, P, i32, i32, i32, i32, i32, P, i32, i32,
                                      dbl, P, P, i32]
        lib.oracle_decode.restype = i32
        lib.oracle_route.argtypes = [P, i32, i32, P, i32, P, P, i32, P, P, i32, P, P, P]
        lib.oracle_route.restype = i32
        lib.oracle_worklist.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, i64,
                                        ctypes.POINTER(i64)]
        lib.oracle_worklist.restype = i32
        lib.oracle_attn_backward.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, P, i32,
                                             i32, dbl, P, P, P, i32]
        lib.oracle_attn_backward.restype = i32
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i32
        _lib = lib
    return _lib


def _as_elements(x):
    """Return (contiguous numpy array holding the exact stored bits, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy(), _DT_BF16
            if x.dtype == torch.float32:
                return x.numpy(), _DT_F32
            if x.dtype == torch.float64:
                return x.numpy(), _DT_F64
            raise TypeError(f"unsupported tensor dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, _DT_F32
    if x.dtype == np.float64:
        return x, _DT_F64
    raise TypeError(f"unsupported array dtype {x.dtype}")


def _np(x, dtype):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=dtype))


def _f64(x):
    """Any tensor or array (bf16 included) as a float64 numpy array, values exact."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().cpu().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def attn(q, k, v, cu_seqlens, n_heads_q, n_heads_kv, route, sink, window, scale=None,
         rows=None, nthreads=0, cu_seqlens_k=None):
    """fp64 routed attention.  q [T, Hq, D], k/v [T, Hkv, D] (bf16, fp32 or fp64; all
    three the same dtype), cu_seqlens [B+1], route [B, Hq] (0 full, 1 sparse).
    rows: packed token indices to evaluate (None = all).
    cu_seqlens_k: packing of k/v [Tk, Hkv, D] for a chunked prefill over a KV prefix (each
    sequence's Lq queries are its last Lq of Lk positions); None = cu_seqlens.
    Returns (o [n_rows, Hq, D] float64, lse [n_rows, Hq] float64)."""
    lib = _load()
    qa, dt = _as_elements(q)
    ka, dtk = _as_elements(k)
    va, dtv = _as_elements(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share one dtype")
    d = int(qa.shape[-1])
    cu = _np(cu_seqlens, np.int32)
    batch = int(cu.shape[0] - 1)
    r = _np(route, np.uint8).reshape(batch, n_heads_q)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if rows is None:
        rows_arr, n_rows = None, int(cu[-1])
    else:
        rows_arr = _np(rows, np.int64).reshape(-1)
        n_rows = int(rows_arr.shape[0])
    o = np.empty((n_rows, n_heads_q, d), dtype=np.float64)
    lse = np.empty((n_rows, n_heads_q), dtype=np.float64)
    cuk = None if cu_seqlens_k is None else _np(cu_seqlens_k, np.int32)
    if cuk is not None and cuk.shape != cu.shape:
        raise ValueError("cu_seqlens_k must have batch + 1 entries")
    rc = lib.oracle_attn(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt,
                         cu.ctypes.data, None if cuk is None else cuk.ctypes.data,
                         batch, n_heads_q, n_heads_kv, d,
                         r.ctypes.data, int(sink), int(window), float(scale),
                         None if rows_arr is None else rows_arr.ctypes.data, n_rows,
                         o.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attn failed with code {rc}")
    return o, lse


def attn_backward(q, k, v, dout, cu_seqlens, n_heads_q, n_heads_kv, route, sink, window,
                  scale=None, nthreads=0, cu_seqlens_k=None):
    """fp64 gradients of the routed attention: q/dout [Tq, Hq, D], k/v [Tk, Hkv, D] (one dtype),
    packing as for attn.  Returns (dq [Tq, Hq, D], dk [Tk, Hkv, D], dv [Tk, Hkv, D]) float64."""
    lib = _load()
    qa, dt = _as_elements(q)
    ka, dtk = _as_elements(k)
    va, dtv = _as_elements(v)
    oa, dto = _as_elements(dout)
    if not (dt == dtk == dtv == dto):
        raise TypeError("q, k, v, dout must share one dtype")
    d = int(qa.shape[-1])
    cu = _np(cu_seqlens, np.int32)
    batch = int(cu.shape[0] - 1)
    cuk = cu if cu_seqlens_k is None else _np(cu_seqlens_k, np.int32)
    r = _np(route, np.uint8).reshape(batch, n_heads_q)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.empty((int(cu[-1]), n_heads_q, d), dtype=np.float64)
    dk = np.empty((int(cuk[-1]), n_heads_kv, d), dtype=np.float64)
    dv = np.empty_like(dk)
    rc = lib.oracle_attn_backward(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, oa.ctypes.data,
                                  dt, cu.ctypes.data, cuk.ctypes.data, batch, n_heads_q,
                                  n_heads_kv, d, r.ctypes.data, int(sink), int(window),
                                  float(scale), dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                                  int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attn_backward failed with code {rc}")
    return dq, dk, dv


def decode(q, k_cache, v_cache, seqlens, n_heads_kv, route, sink, window, scale=None,
           nthreads=0):
    """fp64 decode step.  q [B, Hq, D], k_cache/v_cache [B, cap, Hkv, D] (one dtype),
    seqlens [B] (tokens in each cache, the newest being the query's own), route [B, Hq].
    Returns (o [B, Hq, D] float64, lse [B, Hq] float64)."""
    lib = _load()
    qa, dt = _as_elements(q)
    ka, dtk = _as_elements(k_cache)
    va, dtv = _as_elements(v_cache)
    if not (dt == dtk == dtv):
        raise TypeError("q, k_cache, v_cache must share one dtype")
    batch, hq, d = (int(x) for x in qa.shape)
    cap = int(ka.shape[1])
    sl = _np(seqlens, np.int32).reshape(batch)
    r = _np(route, np.uint8).reshape(batch, hq)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((batch, hq, d), dtype=np.float64)
    lse = np.empty((batch, hq), dtype=np.float64)
    rc = lib.oracle_decode(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt, sl.ctypes.data,
                           batch, cap, hq, int(n_heads_kv), d, r.ctypes.data, int(sink),
                           int(window), float(scale), o.ctypes.data, lse.ctypes.data,
                           int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_decode failed with code {rc}")
    return o, lse


def route(key_states, cu_seqlens, w1, b1, w2, b2):
    """fp64 Attention Router.  key_states [T, C] (bf16/fp32/fp64), w1 [H, C], b1 [H],
    w2 [Hq, H], b2 [Hq] (fp32).  Returns (pooled [B, C], logits [B, Hq], r [B, Hq] uint8)."""
    lib = _load()
    ks, dt = _as_elements(key_states)
    kv_dim = int(ks.shape[-1])
    cu = _np(cu_seqlens, np.int32)
    batch = int(cu.shape[0] - 1)
    w1a, b1a = _np(w1, np.float32), _np(b1, np.float32)
    w2a, b2a = _np(w2, np.float32), _np(b2, np.float32)
    hidden, n_heads = int(w1a.shape[0]), int(w2a.shape[0])
    pooled = np.empty((batch, kv_dim), dtype=np.float64)
    logits = np.empty((batch, n_heads), dtype=np.float64)
    r = np.empty((batch, n_heads), dtype=np.uint8)
    rc = lib.oracle_route(ks.ctypes.data, dt, kv_dim, cu.ctypes.data, batch,
                          w1a.ctypes.data, b1a.ctypes.data, hidden,
                          w2a.ctypes.data, b2a.ctypes.data, n_heads,
                          pooled.ctypes.data, logits.ctypes.data, r.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_route failed with code {rc}")
    return pooled, logits, r


def worklist(route, cu_seqlens, n_heads_q, sink, window, bm, bn, cu_seqlens_k=None):
    """Sorted work items int32 [N, 4] = (seq, head, q_tile, cost).  cu_seqlens_k as for
    attn (chunk rows at positions Lk - Lq ...)."""
    lib = _load()
    cu = _np(cu_seqlens, np.int32)
    batch = int(cu.shape[0] - 1)
    cuk = None if cu_seqlens_k is None else _np(cu_seqlens_k, np.int32)
    cukp = None if cuk is None else cuk.ctypes.data
    r = _np(route, np.uint8).reshape(batch, n_heads_q)
    n = ctypes.c_int64(0)
    rc = lib.oracle_worklist(r.ctypes.data, cu.ctypes.data, cukp, batch, n_heads_q, int(sink),
                             int(window), int(bm), int(bn), None, 0, ctypes.byref(n))
    if rc != 0:
        raise ValueError(f"oracle_worklist failed with code {rc}")
    items = np.empty((max(n.value, 1), 4), dtype=np.int32)
    rc = lib.oracle_worklist(r.ctypes.data, cu.ctypes.data, cukp, batch, n_heads_q, int(sink),
                             int(window), int(bm), int(bn), items.ctypes.data, n.value,
                             ctypes.byref(n))
    if rc != 0:
        raise ValueError(f"oracle_worklist failed with code {rc}")
    return items[: n.value]


def route_backward(key_states, cu_seqlens, w1, b1, w2, b2, o_full, o_sparse, dout, tau=1.0,
                   noise=None):
    """fp64 gradients of the router through its straight-through decision (Elastic Attention
    blog post, section 2.1, "training trick": Gumbel-Softmax with a straight-through estimator
    keeps the 0/1 routing decision differentiable).  Reading: the relaxed decision is
    r_soft = sigmoid((z + g) / tau) with g the logistic (Gumbel-difference) noise of the draw
    (noise [B, Hq], None = 0); the forward uses the hard decision r = (z + g > 0) and the
    output of head h is r O_sparse + (1 - r) O_full, so dL/dr = sum_t <dO_t, O_sparse_t -
    O_full_t> over the sequence's rows; the backward takes dr/dz = r_soft (1 - r_soft) / tau.
    Then through the router MLP z = W2 SiLU(W1 xbar + b1) + b2 and the mean pool
    xbar_b = mean_t key_states[t] (an empty sequence pools to 0 and gets no gradient).
    key_states [T, C]; o_full, o_sparse, dout [T, Hq, D].
    Returns dict with dr, dz [B, Hq], dw1 [H, C], db1 [H], dw2 [Hq, H], db2 [Hq],
    dkey_states [T, C]."""
    ks = _f64(key_states)
    cu = _np(cu_seqlens, np.int32)
    W1, B1, W2, B2 = (_f64(t) for t in (w1, b1, w2, b2))
    of, osp, do = (_f64(t) for t in (o_full, o_sparse, dout))
    B = int(cu.shape[0] - 1)
    hq = W2.shape[0]
    xbar = np.zeros((B, ks.shape[1]))
    for b in range(B):
        if cu[b + 1] > cu[b]:
            xbar[b] = ks[cu[b]:cu[b + 1]].sum(axis=0) / (cu[b + 1] - cu[b])
    u = xbar @ W1.T + B1
    sg = 1.0 / (1.0 + np.exp(-u))
    hs = u * sg
    z = hs @ W2.T + B2
    g = np.zeros_like(z) if noise is None else _f64(noise)
    r_soft = 1.0 / (1.0 + np.exp(-(z + g) / tau))
    dr = np.zeros((B, hq))
    for b in range(B):
        dr[b] = np.einsum("thd,thd->h", do[cu[b]:cu[b + 1]],
                          osp[cu[b]:cu[b + 1]] - of[cu[b]:cu[b + 1]])
    dz = dr * r_soft * (1.0 - r_soft) / tau
    dw2 = dz.T @ hs
    db2 = dz.sum(axis=0)
    dhs = dz @ W2
    du = dhs * (sg + u * sg * (1.0 - sg))
    dw1 = du.T @ xbar
    db1 = du.sum(axis=0)
    dxbar = du @ W1
    dks = np.zeros_like(ks)
    for b in range(B):
        n = cu[b + 1] - cu[b]
        if n > 0:
            dks[cu[b]:cu[b + 1]] = dxbar[b] / n
    return {"dr": dr, "dz": dz, "dw1": dw1, "db1": db1, "dw2": dw2, "db2": db2,
            "dkey_states": dks, "z": z, "r_soft": r_soft}
