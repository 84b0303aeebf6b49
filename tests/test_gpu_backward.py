"""GPU parity of the training backward (through the C ABI) against the fp64 oracle:
ea_hybrid_attn_backward against oracle.attn_backward (dq, dk, dv of the routed attention; the
forward's O and LSE come from the HIP prefill, as in training) and ea_route_backward against
oracle.route_backward (the router's straight-through gradient).

Bounds.  A gradient is a sum over a sequence, so its size grows with the length; the bounds
scale with S = max(1, max |reference|) of the tensor checked:
  bf16 inputs (fp32 arithmetic): max-abs <= 1e-2 S and mean-abs <= 1e-3 S.  The inputs are
    exact in both; the kernel's D_i = <dO_i, O_i> uses the bf16-rounded forward output
    (relative error 2^-9 per element), the one source of error beyond fp32 rounding.
  fp32 inputs: max-abs <= 2e-5 S (fp32 rounding of sums over up to a few thousand terms, and
    the forward's fp32 LSE).
  router gradients (fp32 arithmetic over exact inputs): max-abs <= 1e-5 S.
Integer routing and packings are inputs here, shared by both sides."""
import numpy as np
import pytest
import torch

import oracle
from full_attention_long_amd import ea, inputs
from tests import harness as H

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


def check_grad(got, ref, dtype, what):
    got = got.double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    S = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    say(f"  {what}: max_abs {mx:.3e} mean_abs {mean:.3e} scale {S:.3e}")
    if dtype == torch.bfloat16:
        assert mx <= 1e-2 * S and mean <= 1e-3 * S, f"{what}: max {mx:.3e} mean {mean:.3e} S {S:.3e}"
    else:
        assert mx <= 2e-5 * S, f"{what}: max {mx:.3e} S {S:.3e}"


def gen_inputs(lens, hq, hkv, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    T = sum(lens)
    q = torch.randn(T, hq, d, generator=g).to(dtype)
    k = torch.randn(T, hkv, d, generator=g).to(dtype)
    v = torch.randn(T, hkv, d, generator=g).to(dtype)
    do = torch.randn(T, hq, d, generator=g).to(dtype)
    return q, k, v, do


def run_backward(q, k, v, o, do, lse, cu_q, route, sink, window, cu_k=None, max_q=None,
                 max_k=None, host=True, sentinel=None, scale=0.0):
    dev = H.device()
    lens_q = (cu_q[1:] - cu_q[:-1]).tolist()
    mq = max(lens_q) if max_q is None else max_q
    if cu_k is not None:
        lens_k = (cu_k[1:] - cu_k[:-1]).tolist()
        mk = max(lens_k) if max_k is None else max_k
    else:
        mk = mq if max_k is None else max_k
    fill = float("nan") if sentinel is None else sentinel
    dq = torch.full(q.shape, fill, dtype=torch.float32, device=dev)
    dk = torch.full(k.shape, fill, dtype=torch.float32, device=dev)
    dv = torch.full(v.shape, fill, dtype=torch.float32, device=dev)
    ws = torch.empty(ea.attn_backward_workspace_size(ea.dtype_code(q.dtype), len(lens_q), mq, mk,
                                                     q.shape[1], k.shape[1], q.shape[2]),
                     dtype=torch.uint8, device=dev)
    ea.hybrid_attn_backward(
        H.to_gpu(q), H.to_gpu(k), H.to_gpu(v), H.to_gpu(o), H.to_gpu(do), H.to_gpu(lse),
        H.to_gpu(cu_q), mq, H.to_gpu(route.to(torch.uint8).contiguous()), sink, window, dq, dk,
        dv, ws, scale=scale, cu_seqlens_k=None if cu_k is None else H.to_gpu(cu_k), max_seqlen_k=mk,
        cu_seqlens_q_host=cu_q.tolist() if host else None,
        cu_seqlens_k_host=(cu_k.tolist() if cu_k is not None else None) if host else None)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def prefill_then_backward(lens, hq, hkv, d, dtype, route, sink, window, seed, what, scale=0.0):
    q, k, v, do = gen_inputs(lens, hq, hkv, d, dtype, seed)
    cu = inputs.cu_seqlens(lens)
    say(f"case {what}: lens={lens} hq={hq} hkv={hkv} d={d} {dtype} sink={sink} window={window}")
    o, lse, _, _ = H.run_prefill(q, k, v, lens, route, sink, window, scale=scale, worklist=False)
    dq, dk, dv = run_backward(q, k, v, o, do, lse, cu, route, sink, window, scale=scale)
    rq, rk, rv = oracle.attn_backward(q, k, v, do, cu, hq, hkv, route.numpy(), sink, window,
                                      scale=scale if scale > 0 else None)
    check_grad(dq, rq, dtype, f"{what} dq")
    check_grad(dk, rk, dtype, f"{what} dk")
    check_grad(dv, rv, dtype, f"{what} dv")
    return dq, dk, dv


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 128), (torch.float32, 64)])
def test_backward_ragged(dtype, d):
    lens = [300, 1000, 0, 777, 1, 64, 513]
    hq, hkv = 8, 2
    g = torch.Generator().manual_seed(11)
    route = (torch.rand(len(lens), hq, generator=g) < 0.6).to(torch.uint8)
    prefill_then_backward(lens, hq, hkv, d, dtype, route, 16, 200, 40 + d, f"ragged d{d}")


@pytest.mark.parametrize("kind", ["full", "sparse", "w1_nosink", "w1_sink", "window_covers"])
def test_backward_routing_edges(kind):
    lens = [640, 129]
    hq, hkv, d = 8, 2, 128
    sink, window = 4, 96
    route = torch.ones(len(lens), hq, dtype=torch.uint8)
    if kind == "full":
        route.zero_()
    elif kind == "w1_nosink":
        sink, window = 0, 1           # each row sees only itself
    elif kind == "w1_sink":
        sink, window = 16, 1          # each row sees the sink keys and itself
    elif kind == "window_covers":
        window = 4096                 # the sparse mask equals the causal one
    prefill_then_backward(lens, hq, hkv, d, torch.bfloat16, route, sink, window, 7, kind)


def test_backward_chunked_prefix():
    lens_k, lens_q = [300, 1000, 777, 64], [300, 257, 1, 64]
    hq, hkv, d, sink, window = 8, 2, 128, 16, 200
    dtype = torch.bfloat16
    g = torch.Generator().manual_seed(3)
    Tk = sum(lens_k)
    qfull = torch.randn(Tk, hq, d, generator=g).to(dtype)
    k = torch.randn(Tk, hkv, d, generator=g).to(dtype)
    v = torch.randn(Tk, hkv, d, generator=g).to(dtype)
    cu_k = inputs.cu_seqlens(lens_k)
    q = torch.cat([qfull[int(cu_k[b + 1]) - lq:int(cu_k[b + 1])] for b, lq in enumerate(lens_q)])
    cu_q = inputs.cu_seqlens(lens_q)
    do = torch.randn(q.shape, generator=g).to(dtype)
    route = (torch.rand(len(lens_q), hq, generator=g) < 0.5).to(torch.uint8)
    say(f"case chunked backward: lens_k={lens_k} lens_q={lens_q}")
    dev = H.device()
    o = torch.empty(q.shape, dtype=dtype, device=dev)
    lse = torch.empty((hq, q.shape[0]), dtype=torch.float32, device=dev)
    ws = torch.empty(ea.prefill_chunked_workspace_size(len(lens_q), max(lens_q), hq, d),
                     dtype=torch.uint8, device=dev)
    ea.hybrid_attn_prefill_chunked(H.to_gpu(q), H.to_gpu(k), H.to_gpu(v), o, H.to_gpu(cu_q),
                                   H.to_gpu(cu_k), max(lens_q), max(lens_k),
                                   H.to_gpu(route), sink, window, ws, lse_out=lse)
    torch.cuda.synchronize()
    dq, dk, dv = run_backward(q, k, v, o.cpu(), do, lse.cpu(), cu_q, route, sink, window,
                              cu_k=cu_k)
    rq, rk, rv = oracle.attn_backward(q, k, v, do, cu_q, hq, hkv, route.numpy(), sink, window,
                                      cu_seqlens_k=cu_k)
    check_grad(dq, rq, dtype, "chunked dq")
    check_grad(dk, rk, dtype, "chunked dk")
    check_grad(dv, rv, dtype, "chunked dv")


def test_backward_deterministic():
    lens = [700, 300]
    hq, hkv, d = 8, 4, 128
    q, k, v, do = gen_inputs(lens, hq, hkv, d, torch.bfloat16, 9)
    route = torch.tensor([[0, 1, 1, 0, 1, 0, 0, 1], [1, 1, 0, 0, 1, 1, 1, 0]], dtype=torch.uint8)
    cu = inputs.cu_seqlens(lens)
    say("case backward determinism")
    o, lse, _, _ = H.run_prefill(q, k, v, lens, route, 8, 64, worklist=False)
    a = run_backward(q, k, v, o, do, lse, cu, route, 8, 64)
    b = run_backward(q, k, v, o, do, lse, cu, route, 8, 64)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_device_packing_beyond_bounds(dtype):
    # without host copies, a sequence longer than max_seqlen_q is left unwritten; the others
    # are computed as usual (bf16 with 2 query heads per KV head: the partial reduce too)
    lens = [100, 300]
    hq, hkv, d = 4, 2, 64
    q, k, v, do = gen_inputs(lens, hq, hkv, d, dtype, 21)
    route = torch.tensor([[0, 1, 0, 1], [1, 0, 1, 0]], dtype=torch.uint8)
    cu = inputs.cu_seqlens(lens)
    say("case backward packing beyond max_seqlen")
    o, lse, _, _ = H.run_prefill(q, k, v, lens, route, 4, 32, worklist=False)
    sentinel = -777.0
    dq, dk, dv = run_backward(q, k, v, o, do, lse, cu, route, 4, 32, max_q=200, host=False,
                              sentinel=sentinel)
    assert torch.all(dq[100:] == sentinel) and torch.all(dk[100:] == sentinel)
    assert torch.all(dv[100:] == sentinel)
    rq, rk, rv = oracle.attn_backward(q[:100], k[:100], v[:100], do[:100],
                                      inputs.cu_seqlens([100]), hq, hkv, route[:1].numpy(), 4, 32)
    check_grad(dq[:100], rq, dtype, "in-bounds dq")
    check_grad(dk[:100], rk, dtype, "in-bounds dk")
    check_grad(dv[:100], rv, dtype, "in-bounds dv")


# ----------------------------------------------------------------------------- router


def run_route_backward(ks, cu, w1, b1, w2, b2, of, osp, do, noise, tau, want_dks=True):
    dev = H.device()
    B = cu.numel() - 1
    hid, C = w1.shape
    hq = w2.shape[0]
    d = do.shape[2]
    outs = dict(dr=torch.full((B, hq), float("nan"), device=dev),
                dz=torch.full((B, hq), float("nan"), device=dev),
                dw1=torch.full((hid, C), float("nan"), device=dev),
                db1=torch.full((hid,), float("nan"), device=dev),
                dw2=torch.full((hq, hid), float("nan"), device=dev),
                db2=torch.full((hq,), float("nan"), device=dev))
    dks = torch.full(ks.shape, float("nan"), device=dev) if want_dks else None
    ws = torch.empty(ea.route_backward_workspace_size(B, C, hid, hq, d), dtype=torch.uint8,
                     device=dev)
    g = lambda t: None if t is None else H.to_gpu(t)
    ea.route_backward(g(ks), g(cu), g(w1), g(b1), g(w2), g(b2), g(of), g(osp), g(do),
                      outs["dz"], outs["dw1"], outs["db1"], outs["dw2"], outs["db2"], ws,
                      tau=tau, noise=g(noise), dr_out=outs["dr"], dkey_states=dks)
    torch.cuda.synchronize()
    res = {k: t.cpu() for k, t in outs.items()}
    if want_dks:
        res["dkey_states"] = dks.cpu()
    return res


def route_case(lens, kv_dim, hid, hq, d, kdt, odt, seed, tau, with_noise):
    g = torch.Generator().manual_seed(seed)
    T = sum(lens)
    ks = torch.randn(T, kv_dim, generator=g).to(kdt)
    w1 = (torch.randn(hid, kv_dim, generator=g) / kv_dim ** 0.5).float()
    b1 = (0.1 * torch.randn(hid, generator=g)).float()
    w2 = (torch.randn(hq, hid, generator=g) / hid ** 0.5).float()
    b2 = (0.1 * torch.randn(hq, generator=g)).float()
    of = torch.randn(T, hq, d, generator=g).to(odt)
    osp = (of.float() + 0.3 * torch.randn(T, hq, d, generator=g)).to(odt)
    do = torch.randn(T, hq, d, generator=g).to(odt)
    noise = None
    if with_noise:
        u = torch.rand(len(lens), hq, generator=g).clamp(1e-6, 1 - 1e-6)
        noise = (torch.log(u) - torch.log1p(-u)).float()   # logistic draw
    return ks, inputs.cu_seqlens(lens), w1, b1, w2, b2, of, osp, do, noise


@pytest.mark.parametrize("kdt,odt,with_noise,tau", [
    (torch.bfloat16, torch.bfloat16, True, 0.5),
    (torch.float32, torch.float32, False, 1.0),
    (torch.bfloat16, torch.float32, True, 2.0),
])
def test_route_backward(kdt, odt, with_noise, tau):
    lens = [500, 0, 1234, 1, 77]
    args = route_case(lens, 256, 64, 8, 128, kdt, odt, 17, tau, with_noise)
    say(f"case route backward: lens={lens} kdt={kdt} odt={odt} tau={tau} noise={with_noise}")
    got = run_route_backward(*args, tau)
    ks, cu, w1, b1, w2, b2, of, osp, do, noise = args
    ref = oracle.route_backward(ks, cu, w1, b1, w2, b2, of, osp, do, tau=tau, noise=noise)
    for name in ("dr", "dz", "dw1", "db1", "dw2", "db2", "dkey_states"):
        r = ref[name]
        got_n = got[name].double().numpy()
        err = np.abs(got_n - r)
        S = max(1.0, float(np.abs(r).max()))
        say(f"  {name}: max_abs {err.max():.3e} scale {S:.3e}")
        assert np.all(np.isfinite(got_n)) and err.max() <= 1e-5 * S, name
    # the empty sequence: no rows, zero routing gradient
    assert torch.all(got["dr"][1] == 0)


def test_route_backward_workload_shape():
    # the Qwen3-8B-shaped layer: key states [T, 8 * 128], hidden 256, 32 query heads of 128,
    # one 32K sequence next to a short one
    lens = [32768, 3000]
    args = route_case(lens, 1024, 256, 32, 128, torch.bfloat16, torch.bfloat16, 23, 1.0, True)
    say(f"case route backward workload: lens={lens}")
    got = run_route_backward(*args, 1.0, want_dks=True)
    ks, cu, w1, b1, w2, b2, of, osp, do, noise = args
    ref = oracle.route_backward(ks, cu, w1, b1, w2, b2, of, osp, do, tau=1.0, noise=noise)
    for name in ("dr", "dz", "dw1", "db1", "dw2", "db2", "dkey_states"):
        r = ref[name]
        err = np.abs(got[name].double().numpy() - r)
        S = max(1.0, float(np.abs(r).max()))
        say(f"  {name}: max_abs {err.max():.3e} scale {S:.3e}")
        assert err.max() <= 1e-5 * S, name


def test_backward_workload_32k_sampled():
    """The Qwen3-8B-shaped 32K layer as bench.py runs it (router routing, bf16): sampled dq
    rows against one-row oracle chunks (exact for the row), dk and dv of the last 64 keys
    against the oracle backward of the last 64 rows as a chunk (every row that sees those keys
    is in it), and for every key the identities sum_j dk_j = 0 and sum_j dv_j = sum over rows
    and group heads of dO (softmax rows sum to one)."""
    import json
    import os
    w = inputs.WORKLOADS["qwen3_8b_32k"]
    L = w.lengths[0]
    hq, hkv, d = w.n_heads_q, w.n_heads_kv, w.head_dim
    G = hq // hkv
    dev = H.device()
    q, k, v = inputs.qkv(w, L)
    do = inputs.dout(w, L)
    cu = inputs.cu_seqlens([L])
    w1, b1, w2, b2 = inputs.router_weights(w)
    with open(os.path.join(os.path.dirname(__file__), "golden", "router_bias_qwen3_8b_32k.json")) as f:
        b2 = torch.full_like(b2, json.load(f)["b2"])
    ks = k.view(L, hkv * d)
    route = torch.empty(1, hq, dtype=torch.uint8, device=dev)
    ws = H.workspace(1, L, hq, ks.shape[1], w1.shape[0])
    ea.route(H.to_gpu(ks), H.to_gpu(cu), H.to_gpu(w1), H.to_gpu(b1), H.to_gpu(w2), H.to_gpu(b2),
             route, ws)
    torch.cuda.synchronize()
    route = route.cpu()
    say(f"case backward 32K workload: sparse heads {int(route.sum())}")
    o, lse, _, _ = H.run_prefill(q, k, v, [L], route, w.sink, w.window, worklist=False)
    dq, dk, dv = run_backward(q, k, v, o, do, lse, cu, route, w.sink, w.window)
    r = route.numpy()
    # sampled dq rows: boundaries of the sink and window and spread rows
    rows = sorted({0, 1, w.sink - 1, w.sink, w.window - 1, w.window, w.sink + w.window - 1,
                   w.sink + w.window, 5000, 12345, 20000, 27777, L - 2, L - 1})
    for i in rows:
        rq, _, _ = oracle.attn_backward(q[i:i + 1], k[:i + 1], v[:i + 1], do[i:i + 1],
                                        inputs.cu_seqlens([1]), hq, hkv, r, w.sink, w.window,
                                        cu_seqlens_k=inputs.cu_seqlens([i + 1]))
        check_grad(dq[i:i + 1], rq, torch.bfloat16, f"dq row {i}")
    # dk, dv of the last 64 keys
    m = 64
    _, rk, rv = oracle.attn_backward(q[L - m:], k, v, do[L - m:], inputs.cu_seqlens([m]), hq,
                                     hkv, r, w.sink, w.window,
                                     cu_seqlens_k=inputs.cu_seqlens([L]))
    check_grad(dk[L - m:], rk[L - m:], torch.bfloat16, "dk last 64 keys")
    check_grad(dv[L - m:], rv[L - m:], torch.bfloat16, "dv last 64 keys")
    # column identities over every key, per KV head
    sk = dk.double().sum(dim=0)                            # [hkv, d]
    sv = dv.double().sum(dim=0)
    want_v = do.double().sum(dim=0).view(hkv, G, d).sum(dim=1)
    abs_k = dk.double().abs().sum(dim=0)
    err_k = float((sk.abs() / abs_k.clamp_min(1e-30)).max())
    err_v = float(((sv - want_v).abs() / do.double().abs().sum(dim=0).view(hkv, G, d).sum(dim=1)).max())
    say(f"  sum dk relative {err_k:.3e}, sum dv relative {err_v:.3e}")
    # bf16 P and dS operands: each term is within 2^-8 relative of the exact one
    assert err_k <= 2e-3 and err_v <= 2e-3


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (4, 4, 64), (8, 1, 128), (16, 2, 64),
                                      (96, 8, 64)])
def test_backward_group_sizes(hq, hkv, d):
    # one query head per KV head (dk, dv written directly, no partials), large groups
    # (partials of up to 8 heads summed in head order) and 96 query heads
    lens = [333, 700, 65]
    g = torch.Generator().manual_seed(hq * 100 + hkv * 10 + d)
    route = (torch.rand(len(lens), hq, generator=g) < 0.5).to(torch.uint8)
    prefill_then_backward(lens, hq, hkv, d, torch.bfloat16, route, 8, 150, 60 + hq + hkv,
                          f"groups hq{hq} hkv{hkv} d{d}")


def test_backward_long_256k_sampled():
    """The 256K long-context layer (Bernoulli routing, bf16): the largest sequence the bf16
    kernels address (one sequence's q rows are 2^31 bytes).  Sampled dq rows against one-row
    oracle chunks, dk and dv of the last 16 keys against the oracle chunk backward, and the
    column identities for every key."""
    w = inputs.WORKLOADS["long_256k"]
    L = w.lengths[0]
    hq, hkv, d = w.n_heads_q, w.n_heads_kv, w.head_dim
    G = hq // hkv
    q, k, v = inputs.qkv(w, L)
    do = inputs.dout(w, L)
    cu = inputs.cu_seqlens([L])
    route = inputs.bernoulli_route(w, 1)
    say(f"case backward 256K: sparse heads {int(route.sum())}")
    o, lse, _, _ = H.run_prefill(q, k, v, [L], route, w.sink, w.window, worklist=False)
    dq, dk, dv = run_backward(q, k, v, o, do, lse, cu, route, w.sink, w.window)
    r = route.numpy()
    for i in (0, w.sink, w.window + w.sink, 100000, 200001, L - 1):
        rq, _, _ = oracle.attn_backward(q[i:i + 1], k[:i + 1], v[:i + 1], do[i:i + 1],
                                        inputs.cu_seqlens([1]), hq, hkv, r, w.sink, w.window,
                                        cu_seqlens_k=inputs.cu_seqlens([i + 1]))
        check_grad(dq[i:i + 1], rq, torch.bfloat16, f"dq row {i}")
    m = 16
    _, rk, rv = oracle.attn_backward(q[L - m:], k, v, do[L - m:], inputs.cu_seqlens([m]), hq,
                                     hkv, r, w.sink, w.window,
                                     cu_seqlens_k=inputs.cu_seqlens([L]))
    check_grad(dk[L - m:], rk[L - m:], torch.bfloat16, "dk last 16 keys")
    check_grad(dv[L - m:], rv[L - m:], torch.bfloat16, "dv last 16 keys")
    sk = dk.double().sum(dim=0)
    sv = dv.double().sum(dim=0)
    want_v = do.double().sum(dim=0).view(hkv, G, d).sum(dim=1)
    err_k = float((sk.abs() / dk.double().abs().sum(dim=0).clamp_min(1e-30)).max())
    err_v = float(((sv - want_v).abs() /
                   do.double().abs().sum(dim=0).view(hkv, G, d).sum(dim=1)).max())
    say(f"  sum dk relative {err_k:.3e}, sum dv relative {err_v:.3e}")
    assert err_k <= 2e-3 and err_v <= 2e-3


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_custom_scale(dtype):
    # a softmax scale other than 1/sqrt(D): it enters P (through the forward's LSE) and both
    # dq and dk (scale * dS)
    lens = [400, 77]
    hq, hkv, d = 8, 2, 64
    g = torch.Generator().manual_seed(5)
    route = (torch.rand(len(lens), hq, generator=g) < 0.5).to(torch.uint8)
    prefill_then_backward(lens, hq, hkv, d, dtype, route, 8, 100, 33, f"scale 0.07 {dtype}",
                          scale=0.07)


def test_backward_chunked_prefix_fp32():
    # the fp32 kernels over a KV prefix (chunk rows at positions Lk - Lq + r)
    lens_k, lens_q = [200, 513, 64], [200, 100, 1]
    hq, hkv, d, sink, window = 4, 2, 64, 8, 90
    g = torch.Generator().manual_seed(8)
    Tk = sum(lens_k)
    qfull = torch.randn(Tk, hq, d, generator=g)
    k = torch.randn(Tk, hkv, d, generator=g)
    v = torch.randn(Tk, hkv, d, generator=g)
    cu_k = inputs.cu_seqlens(lens_k)
    q = torch.cat([qfull[int(cu_k[b + 1]) - lq:int(cu_k[b + 1])] for b, lq in enumerate(lens_q)])
    cu_q = inputs.cu_seqlens(lens_q)
    do = torch.randn(q.shape, generator=g)
    route = (torch.rand(len(lens_q), hq, generator=g) < 0.5).to(torch.uint8)
    say(f"case chunked backward fp32: lens_k={lens_k} lens_q={lens_q}")
    dev = H.device()
    o = torch.empty(q.shape, dtype=q.dtype, device=dev)
    lse = torch.empty((hq, q.shape[0]), dtype=torch.float32, device=dev)
    ws = torch.empty(ea.prefill_chunked_workspace_size(len(lens_q), max(lens_q), hq, d),
                     dtype=torch.uint8, device=dev)
    ea.hybrid_attn_prefill_chunked(H.to_gpu(q), H.to_gpu(k), H.to_gpu(v), o, H.to_gpu(cu_q),
                                   H.to_gpu(cu_k), max(lens_q), max(lens_k), H.to_gpu(route),
                                   sink, window, ws, lse_out=lse)
    torch.cuda.synchronize()
    dq, dk, dv = run_backward(q, k, v, o.cpu(), do, lse.cpu(), cu_q, route, sink, window,
                              cu_k=cu_k)
    rq, rk, rv = oracle.attn_backward(q, k, v, do, cu_q, hq, hkv, route.numpy(), sink, window,
                                      cu_seqlens_k=cu_k)
    check_grad(dq, rq, torch.float32, "chunked fp32 dq")
    check_grad(dk, rk, torch.float32, "chunked fp32 dk")
    check_grad(dv, rv, torch.float32, "chunked fp32 dv")


@pytest.mark.parametrize("seed", range(12))
def test_backward_random_configs(seed):
    # seeded random shapes: lengths (empty and tile-ragged ones included), group size, head_dim,
    # dtype, sink, window and routing all drawn
    rng = np.random.default_rng(1000 + seed)
    nseq = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.choice([0, 1, 31, 64, 97, 128, 200, 333, 513], size=nseq)]
    if sum(lens) == 0:
        lens[0] = 77
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.75 else torch.float32
    sink = int(rng.choice([0, 1, 4, 16, 64]))
    window = int(rng.choice([1, 8, 50, 128, 1000]))
    g = torch.Generator().manual_seed(seed)
    route = (torch.rand(len(lens), hq, generator=g) < float(rng.random())).to(torch.uint8)
    prefill_then_backward(lens, hq, hkv, d, dtype, route, sink, window, 200 + seed,
                          f"random {seed}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_window_of_int32_max_equals_full(dtype):
    """window = 2^31 - 1 on every head: the gradients equal the full-attention ones (the
    host clamps the window, so j + window stays inside 32 bits in the dk/dv row plan)."""
    lens = [700, 129, 1]
    hq, hkv, d = 8, 2, 128
    q, k, v, do = gen_inputs(lens, hq, hkv, d, dtype, 23)
    cu = inputs.cu_seqlens(lens)
    route = torch.ones(len(lens), hq, dtype=torch.uint8)
    big = 2**31 - 1
    o, lse, _, _ = H.run_prefill(q, k, v, lens, route, 2, big, worklist=False)
    dq, dk, dv = run_backward(q, k, v, o, do, lse, cu, route, 2, big)
    full = np.zeros((len(lens), hq), np.uint8)
    rq, rk, rv = oracle.attn_backward(q, k, v, do, cu, hq, hkv, full, 0, 1)
    check_grad(dq, rq, dtype, "window 2^31-1 dq")
    check_grad(dk, rk, dtype, "window 2^31-1 dk")
    check_grad(dv, rv, dtype, "window 2^31-1 dv")
