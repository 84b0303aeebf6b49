"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle on identical
seeded input bytes.  bf16: max-abs <= 1e-2 and mean-abs <= 1e-3; fp32: max-abs <= 1e-5;
routing bits and work lists bit-exact.  The pages (Elastic Attention blog post, sections
2.1 and 3) fix what is computed; the oracle is the plain definition of it."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from full_attention_long_amd import ea, inputs
from tests import harness as H

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()
    torch.cuda.init()


def oracle_worklist(route, lens, hq, sink, window, dt, d):
    bm, bn = {(ea.EA_BF16, 64): (256, 64), (ea.EA_BF16, 128): (256, 64),
              (ea.EA_F32, 64): (64, 32), (ea.EA_F32, 128): (64, 32)}[(dt, d)]
    assert ea.tile_config(dt, d) == (bm, bn)
    return oracle.worklist(route.numpy(), inputs.cu_seqlens(lens).numpy(), hq, sink, window, bm, bn)


def check_case(q, k, v, lens, route, sink, window, rows=None, what="", guard=0, strict=True):
    hq, hkv = q.shape[1], k.shape[1]
    say(f"case {what}: lens={lens} hq={hq} hkv={hkv} d={q.shape[2]} {q.dtype} s={sink} W={window}")
    o, lse, items, guard_ok = H.run_prefill(q, k, v, lens, route, sink, window, guard=guard)
    assert guard_ok, "writes outside O"
    # every row, compared or not, is finite; lse starts as NaN, so every entry was written
    assert bool(torch.isfinite(o).all()), f"{what}: non-finite output"
    assert bool(torch.isfinite(lse).all()), f"{what}: lse not finite or not written"
    cu = inputs.cu_seqlens(lens)
    ro, rlse = oracle.attn(q, k, v, cu, hq, hkv, route.numpy(), sink, window, rows=rows)
    sel = slice(None) if rows is None else torch.as_tensor(rows)
    H.compare(o[sel], ro, q.dtype, what, strict=strict)
    # bf16: the row sum adds the bf16-rounded weights P (each within the unit roundoff
    # 2^-8 relative of the exact value), so ln(l) is within ln(1 + 2^-8) < 3.9e-3 of the
    # exact log-sum-exp, plus fp32 accumulation of the scores.  fp32: 1e-5.
    tol = 4e-3 if q.dtype == torch.bfloat16 else 1e-5
    lse_sel = lse[:, sel].T.double().numpy()
    assert np.abs(lse_sel - rlse).max() <= tol, what
    ref_items = oracle_worklist(route, lens, hq, sink, window, ea.dtype_code(q.dtype), q.shape[2])
    assert np.array_equal(items, ref_items), f"{what}: work list differs"
    return o


def rand_qkv(T, hq, hkv, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    mk = lambda h: torch.randn(T, h, d, generator=g).to(dtype)
    return mk(hq), mk(hkv), mk(hkv)


def test_tiny_fp32_workload():
    w = inputs.WORKLOADS["tiny_fp32"]
    lens = inputs.lengths(w)
    q, k, v = inputs.qkv(w, sum(lens))
    check_case(q, k, v, lens, inputs.bernoulli_route(w, 1), w.sink, w.window, what=w.name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_small_ragged_all_rows(d, dtype):
    lens = [1, 200, 0, 129, 384, 70]
    hq, hkv = 8, 2
    q, k, v = rand_qkv(sum(lens), hq, hkv, d, dtype, 11 + d)
    route = (torch.rand(len(lens), hq, generator=torch.Generator().manual_seed(3)) < 0.5).to(torch.uint8)
    check_case(q, k, v, lens, route, 16, 64, what=f"ragged d{d} {dtype}", guard=3)


@pytest.mark.parametrize("sink,window", [(0, 1), (1, 1), (200, 1), (0, 5000), (64, 64),
                                         (3, 130), (130, 3)])
def test_sink_window_edges_bf16(sink, window):
    lens = [700, 333]
    hq, hkv = 4, 1
    q, k, v = rand_qkv(sum(lens), hq, hkv, 128, torch.bfloat16, 5)
    route = torch.tensor([[1, 1, 0, 1], [1, 0, 1, 1]], dtype=torch.uint8)
    check_case(q, k, v, lens, route, sink, window, what=f"s{sink} W{window}", strict=False)


@pytest.mark.parametrize("mode", ["all_full", "all_sparse"])
def test_degenerate_routing(mode):
    lens = [1000, 513]
    hq, hkv = 8, 8
    q, k, v = rand_qkv(sum(lens), hq, hkv, 128, torch.bfloat16, 9)
    route = torch.full((2, hq), 0 if mode == "all_full" else 1, dtype=torch.uint8)
    check_case(q, k, v, lens, route, 32, 256, what=mode)


def test_determinism_across_grid_sizes():
    lens = [1500, 900]
    hq, hkv, d = 8, 2, 128
    q, k, v = rand_qkv(sum(lens), hq, hkv, d, torch.bfloat16, 21)
    route = torch.tensor([[0, 1, 1, 0, 1, 1, 1, 0], [1, 1, 1, 1, 0, 0, 1, 1]], dtype=torch.uint8)
    cu = H.to_gpu(inputs.cu_seqlens(lens))
    dq, dk, dv = H.to_gpu(q), H.to_gpu(k), H.to_gpu(v)
    droute = H.to_gpu(route)
    ws = H.workspace(2, max(lens), hq)
    wl = torch.empty(2 * hq * 12, 4, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    n = ea.build_worklist(droute, cu, max(lens), hq, 32, 256, ea.EA_BF16, d, wl, ws,
                          n_items_out=cnt)
    bm, _ = ea.tile_config(ea.EA_BF16, d)
    assert n == hq * sum(-(-L // bm) for L in lens)
    outs = []
    for grid in (1, 7, 0, 1000):
        o = torch.empty_like(dq)
        ea.hybrid_attn_run(dq, dk, dv, o, cu, max(lens), droute, 32, 256, wl, cnt, ws,
                           grid_blocks=grid)
        torch.cuda.synchronize()
        outs.append(o.cpu())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_llama8b_8k_all_rows():
    w = inputs.WORKLOADS["llama8b_8k"]
    lens = inputs.lengths(w)
    q, k, v = inputs.qkv(w, sum(lens))
    route = inputs.bernoulli_route(w, 1)
    check_case(q, k, v, lens, route, w.sink, w.window, what=w.name)


def test_qwen3_32k_router_and_sampled_rows():
    w = inputs.WORKLOADS["qwen3_8b_32k"]
    lens = inputs.lengths(w)
    T = sum(lens)
    q, k, v = inputs.qkv(w, T)
    ks = k.view(T, w.n_heads_kv * w.head_dim)
    w1, b1, w2, b2 = inputs.router_weights(w)
    with open(os.path.join(GOLDEN, "router_bias_qwen3_8b_32k.json")) as f:
        b2 = torch.full_like(b2, json.load(f)["b2"])
    cu = inputs.cu_seqlens(lens)
    _, ref_logits, ref_r = oracle.route(ks, cu, w1, b1, w2, b2)
    say("router: oracle done")
    dcu = H.to_gpu(cu)
    r_gpu = torch.empty(1, w.n_heads_q, dtype=torch.uint8, device="cuda")
    z_gpu = torch.empty(1, w.n_heads_q, dtype=torch.float32, device="cuda")
    ws = H.workspace(1, T, w.n_heads_q, ks.shape[1], w1.shape[0])
    ea.route(H.to_gpu(ks), dcu, H.to_gpu(w1), H.to_gpu(b1), H.to_gpu(w2), H.to_gpu(b2), r_gpu, ws,
             logits_out=z_gpu)
    torch.cuda.synchronize()
    assert np.array_equal(r_gpu.cpu().numpy(), ref_r)
    assert int(ref_r.sum()) == 27
    assert np.abs(z_gpu.cpu().double().numpy() - ref_logits).max() < 1e-6
    rows = inputs.sampled_rows(w, lens, w.sampled_rows)
    check_case(q, k, v, lens, torch.from_numpy(ref_r), w.sink, w.window, rows=rows.numpy(),
               what=w.name)


@pytest.mark.timeout(900)  # the fp64 oracle over 4 x 2048 rows takes a minute or more of CPU
def test_ragged4_sampled_rows():
    w = inputs.WORKLOADS["ragged4"]
    lens = inputs.lengths(w)
    q, k, v = inputs.qkv(w, sum(lens))
    route = inputs.bernoulli_route(w, len(lens))
    rows = inputs.sampled_rows(w, lens, 2048)  # 2048 rows per sequence, at the strict bound
    check_case(q, k, v, lens, route, w.sink, w.window, rows=rows.numpy(), what=w.name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["all_full", "all_sparse"])
def test_ragged4_degenerate_masks(mode):
    w = inputs.WORKLOADS["ragged4"]
    lens = inputs.lengths(w)
    q, k, v = inputs.qkv(w, sum(lens))
    route = torch.full((len(lens), w.n_heads_q), 0 if mode == "all_full" else 1, dtype=torch.uint8)
    rows = inputs.sampled_rows(w, lens, 2048)
    check_case(q, k, v, lens, route, w.sink, w.window, rows=rows.numpy(), what=f"ragged4 {mode}")


def test_long_256k_sampled_rows():
    w = inputs.WORKLOADS["long_256k"]
    lens = inputs.lengths(w)
    q, k, v = inputs.qkv(w, sum(lens))
    route = inputs.bernoulli_route(w, 1)
    rows = inputs.sampled_rows(w, lens, w.sampled_rows)
    check_case(q, k, v, lens, route, w.sink, w.window, rows=rows.numpy(), what=w.name)


@pytest.mark.parametrize("kdt", [torch.bfloat16, torch.float32])
def test_router_ragged_with_empty_sequence(kdt):
    lens = [300, 0, 1, 77]
    cu = inputs.cu_seqlens(lens)
    C, Hh, Hq = 200, 48, 6   # kv_dim not a multiple of 8: the scalar pooling path
    g = torch.Generator().manual_seed(42)
    ks = torch.randn(sum(lens), C, generator=g).to(kdt)
    w1 = torch.randn(Hh, C, generator=g) * 0.3
    b1 = torch.randn(Hh, generator=g) * 0.1
    w2 = torch.randn(Hq, Hh, generator=g) * 0.3
    b2 = torch.randn(Hq, generator=g) * 0.1
    _, ref_z, ref_r = oracle.route(ks, cu, w1, b1, w2, b2)
    r = torch.empty(len(lens), Hq, dtype=torch.uint8, device="cuda")
    z = torch.empty(len(lens), Hq, dtype=torch.float32, device="cuda")
    ws = H.workspace(len(lens), max(lens), Hq, C, Hh)
    ea.route(H.to_gpu(ks), H.to_gpu(cu), H.to_gpu(w1), H.to_gpu(b1), H.to_gpu(w2), H.to_gpu(b2),
             r, ws, logits_out=z)
    torch.cuda.synchronize()
    zz = z.cpu().double().numpy()
    assert np.abs(zz - ref_z).max() < 1e-5
    # bits must agree wherever the logit is not within float rounding of the threshold
    decided = np.abs(ref_z) > 1e-5
    assert np.array_equal(r.cpu().numpy()[decided], ref_r[decided])


@pytest.mark.parametrize("seed", range(10))
def test_prefill_random_configs(seed):
    """Seeded random shapes: 1-5 sequences of mixed lengths (empty, one token, on and around
    tile edges), group sizes 1-8, head_dim 64 or 128, bf16 or fp32, sink and window from the
    degenerate to the covering, random routing; every row against the oracle."""
    rng = np.random.default_rng(2000 + seed)
    nseq = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.choice([0, 1, 2, 63, 64, 65, 255, 256, 257, 700, 1100], size=nseq)]
    if sum(lens) == 0:
        lens[0] = 129
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.75 else torch.float32
    sink = int(rng.choice([0, 1, 5, 64, 300]))
    window = int(rng.choice([1, 7, 64, 333, 5000]))
    q, k, v = rand_qkv(sum(lens), hq, hkv, d, dtype, 300 + seed)
    g = torch.Generator().manual_seed(seed)
    route = (torch.rand(len(lens), hq, generator=g) < float(rng.random())).to(torch.uint8)
    check_case(q, k, v, lens, route, sink, window, what=f"random {seed}", strict=False)


@pytest.mark.parametrize("hq,hkv,dtype", [(96, 8, torch.bfloat16), (128, 16, torch.bfloat16),
                                           (128, 32, torch.float32)])
def test_many_query_heads(hq, hkv, dtype):
    """Query heads past 64 (the second word of the planner's per-sequence head masks, up to
    its limit of 128): the work list bit for bit and every row, with both modes mixed."""
    lens = [300, 1, 520]
    q, k, v = rand_qkv(sum(lens), hq, hkv, 64, dtype, 77)
    g = torch.Generator().manual_seed(5)
    route = (torch.rand(len(lens), hq, generator=g) < 0.6).to(torch.uint8)
    route[0, 70] = 0   # a full head and a sparse head past 64 in every configuration
    route[0, 90] = 1
    # rows with one to a few visible keys (the one-token sequence, a sequence's first rows)
    # reach |o| > 2, where bf16 itself is coarser than 1e-2: the relative form of the bound
    check_case(q, k, v, lens, route, 16, 128, what=f"hq {hq} {dtype}", strict=False)


def test_worklist_route_run_share_a_workspace():
    """ea_build_worklist, then ea_route, then ea_hybrid_attn_run on one workspace: the
    router's scratch lies past the queue counters the run takes items through, so the run
    still starts from a zero queue head and writes every row."""
    lens = [700, 300]
    hq, hkv, d = 8, 2, 128
    q, k, v = rand_qkv(sum(lens), hq, hkv, d, torch.bfloat16, 31)
    cu = inputs.cu_seqlens(lens)
    g = torch.Generator().manual_seed(8)
    C, Hh = hkv * d, 64
    w1 = torch.randn(Hh, C, generator=g) * 0.05
    b1 = torch.zeros(Hh)
    w2 = torch.randn(hq, Hh, generator=g) * 0.05
    b2 = torch.zeros(hq)
    ks = k.reshape(sum(lens), C)
    dcu, droute = H.to_gpu(cu), torch.empty(len(lens), hq, dtype=torch.uint8, device="cuda")
    router = [H.to_gpu(t) for t in (ks, w1, b1, w2, b2)]
    ws = H.workspace(len(lens), max(lens), hq, C, Hh)
    ea.route(router[0], dcu, *router[1:], droute, ws)
    wl = torch.empty(len(lens) * hq * 4, 4, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    ea.build_worklist(droute, dcu, max(lens), hq, 16, 128, ea.EA_BF16, d, wl, ws, n_items_out=cnt)
    ea.route(router[0], dcu, *router[1:], droute, ws)   # the same bits, the scratch rewritten
    o = torch.full((sum(lens), hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ea.hybrid_attn_run(H.to_gpu(q), H.to_gpu(k), H.to_gpu(v), o, dcu, max(lens), droute, 16, 128,
                       wl, cnt, ws)
    torch.cuda.synchronize()
    route = droute.cpu()
    ro, _ = oracle.attn(q, k, v, cu, hq, hkv, route.numpy(), 16, 128)
    H.compare(o.cpu(), ro, torch.bfloat16, "build -> route -> run")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_window_of_int32_max_equals_full(dtype):
    """window = 2^31 - 1 hides nothing: every sparse head equals a full head (the mask
    arithmetic stays in 32 bits because the host clamps the window to the longest sequence)."""
    lens = [513, 70, 300]
    hq, hkv, d = 4, 2, 128
    q, k, v = rand_qkv(sum(lens), hq, hkv, d, dtype, 17)
    route = torch.ones(len(lens), hq, dtype=torch.uint8)
    o, lse, _, _ = H.run_prefill(q, k, v, lens, route, 3, 2**31 - 1, worklist=False)
    cu = inputs.cu_seqlens(lens)
    ro, rlse = oracle.attn(q, k, v, cu, hq, hkv, np.zeros((len(lens), hq), np.uint8), 0, 1)
    H.compare(o, ro, dtype, "window 2^31-1")
    tol = 4e-3 if dtype == torch.bfloat16 else 1e-5
    assert np.abs(lse.T.double().numpy() - rlse).max() <= tol
