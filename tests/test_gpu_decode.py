"""GPU parity of the decode step (ea_hybrid_attn_decode, through the C ABI) against the fp64
oracle's decode on identical seeded bytes: bf16 max-abs <= 1e-2 and mean-abs <= 1e-3 (the
spec bound for bf16 outputs), fp32 max-abs <= 1e-5, LSE within 1e-3 (bf16: fp32
arithmetic, no bf16 rounding of P on this path) or 1e-5 (fp32).  The step is the same routed
attention as the prefill (Elastic Attention blog post, section 2.1), evaluated at the newest
position of each sequence's cache."""
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
    torch.cuda.init()


def run_decode(q, kc, vc, lens, route, sink, window, max_seqlen=None, scale=0.0,
               poison=True, dev_lens=None):
    """Caches go to the GPU with every slot past a sequence's length set to NaN (they must
    never be read); returns (o, lse) on the CPU."""
    dev = H.device()
    B, hq, d = q.shape
    cap = kc.shape[1]
    max_seqlen = max_seqlen or max(lens)
    kg, vg = H.to_gpu(kc), H.to_gpu(vc)
    if poison:
        for b, L in enumerate(lens):
            if L < cap:
                kg[b, L:] = float("nan")
                vg[b, L:] = float("nan")
    qg = H.to_gpu(q)
    o = torch.full_like(qg, float("nan"))
    lse = torch.full((B, hq), float("nan"), dtype=torch.float32, device=dev)
    sl = torch.tensor(dev_lens if dev_lens is not None else lens, dtype=torch.int32, device=dev)
    ws = torch.empty(ea.decode_workspace_size(B, max_seqlen, hq, d), dtype=torch.uint8,
                     device=dev)
    ea.hybrid_attn_decode(qg, kg, vg, o, sl, max_seqlen, H.to_gpu(route), sink, window, ws,
                          scale=scale, seqlens_host=None if dev_lens is not None else lens,
                          lse_out=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check_decode(q, kc, vc, lens, route, sink, window, what, strict=False, **kw):
    """strict: the workload bound (bf16 max-abs 1e-2); otherwise rows with a handful of
    visible keys may output |o| > 2, where one bf16 ulp exceeds 1e-2 (the harness then
    bounds 1e-2 * max(1, |o| / 2))."""
    say(f"case {what}: B={q.shape[0]} lens={lens if len(lens) <= 8 else str(lens[:8]) + '...'} "
        f"hq={q.shape[1]} hkv={kc.shape[2]} d={q.shape[2]} {q.dtype} s={sink} W={window}")
    o, lse = run_decode(q, kc, vc, lens, route, sink, window, **kw)
    ro, rl = oracle.decode(q, kc, vc, lens, kc.shape[2], route.numpy(), sink, window)
    H.compare(o, ro, q.dtype, what, strict=strict)
    tol = 1e-3 if q.dtype == torch.bfloat16 else 1e-5
    err = np.abs(lse.double().numpy() - rl).max()
    assert err <= tol, f"{what}: lse max-abs {err:.3e}"
    return o, lse


def test_decode_tiny_fp32_workload():
    w = inputs.DECODE_WORKLOADS["decode_tiny_fp32"]
    q, kc, vc, lens, route = inputs.decode_inputs(w)
    check_decode(q, kc, vc, lens, route, w.sink, w.window, "decode tiny fp32")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_split_boundaries(dtype, d, G):
    """Lengths on and around the 256-key split size, every routing of a group."""
    hkv = 2
    hq = G * hkv
    lens = [1, 2, 255, 256, 257, 511, 512, 700, 1500]
    cap = 1536
    g = torch.Generator().manual_seed(1000 + G * 10 + d)
    q = torch.randn(len(lens), hq, d, generator=g).to(dtype)
    kc = torch.randn(len(lens), cap, hkv, d, generator=g).to(dtype)
    vc = torch.randn(len(lens), cap, hkv, d, generator=g).to(dtype)
    route = (torch.rand(len(lens), hq, generator=g) < 0.6).to(torch.uint8)
    route[0, :G] = 1   # an all-sparse group
    route[1, :G] = 0   # an all-full group
    check_decode(q, kc, vc, lens, route, 16, 200, f"splits d{d} G{G} {dtype}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_many_query_heads(dtype):
    """128 query heads on 16 KV heads (group 8, the kernel's largest), with full and sparse
    heads past head 64 and an all-sparse group."""
    hq, hkv, d, cap = 128, 16, 64, 1200
    lens = [1, 300, 1100]
    g = torch.Generator().manual_seed(4242)
    q = torch.randn(len(lens), hq, d, generator=g).to(dtype)
    kc = torch.randn(len(lens), cap, hkv, d, generator=g).to(dtype)
    vc = torch.randn(len(lens), cap, hkv, d, generator=g).to(dtype)
    route = (torch.rand(len(lens), hq, generator=g) < 0.6).to(torch.uint8)
    route[2, 64:72] = 1   # an all-sparse group past head 64
    route[2, 72] = 0      # and a full head in the next one
    check_decode(q, kc, vc, lens, route, 16, 200, f"decode hq {hq} {dtype}")


@pytest.mark.parametrize("sink,window", [(0, 1), (1, 1), (300, 5), (0, 2000), (64, 256)])
def test_decode_sink_window_edges(sink, window):
    lens = [1, 5, 300, 301, 1024, 1800]
    hq, hkv, d, cap = 8, 2, 128, 1800
    g = torch.Generator().manual_seed(77 + sink + window)
    q = torch.randn(len(lens), hq, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(len(lens), cap, hkv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(len(lens), cap, hkv, d, generator=g).to(torch.bfloat16)
    route = torch.ones(len(lens), hq, dtype=torch.uint8)
    route[:, 1] = 0  # group 0 mixed, group 1 all sparse
    check_decode(q, kc, vc, lens, route, sink, window, f"edges s{sink} W{window}")


@pytest.mark.parametrize("name,batch", [("decode_llama8b_8k", 4), ("decode_qwen3_8b_32k", 4),
                                        ("decode_ragged", 8)])
def test_decode_workloads(name, batch):
    w = inputs.DECODE_WORKLOADS[name]
    q, kc, vc, lens, route = inputs.decode_inputs(w, batch)
    check_decode(q, kc, vc, lens, route, w.sink, w.window, name, strict=True)


def test_decode_long_256k():
    w = inputs.DECODE_WORKLOADS["decode_long_256k"]
    q, kc, vc, lens, route = inputs.decode_inputs(w)
    check_decode(q, kc, vc, lens, route, w.sink, w.window, "decode 256k", strict=True,
                 poison=False)


def test_decode_degenerate_routes_and_determinism():
    w = inputs.DECODE_WORKLOADS["decode_ragged"]
    q, kc, vc, lens, _ = inputs.decode_inputs(w, 4)
    for mode in (0, 1):
        route = torch.full((4, w.n_heads_q), mode, dtype=torch.uint8)
        o1, l1 = check_decode(q, kc, vc, lens, route, w.sink, w.window, f"all {'sparse' if mode else 'full'}")
        o2, l2 = run_decode(q, kc, vc, lens, route, w.sink, w.window)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_lengths_outside_contract_give_nan():
    """Device lengths 0 and > max_seqlen: that sequence's outputs are NaN, the others are
    unaffected (and no cache slot past a length is read: the slots hold NaN)."""
    hq, hkv, d, cap = 8, 2, 128, 600
    lens = [100, 200, 300]
    g = torch.Generator().manual_seed(5)
    q = torch.randn(3, hq, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(3, cap, hkv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(3, cap, hkv, d, generator=g).to(torch.bfloat16)
    route = (torch.rand(3, hq, generator=g) < 0.5).to(torch.uint8)
    o, lse = run_decode(q, kc, vc, lens, route, 4, 50, max_seqlen=300, dev_lens=[0, 200, 301])
    assert torch.isnan(o[0].float()).all() and torch.isnan(o[2].float()).all()
    assert torch.isnan(lse[0]).all() and torch.isnan(lse[2]).all()
    ro, _ = oracle.decode(q[1:2], kc[1:2], vc[1:2], [200], hkv, route[1:2].numpy(), 4, 50)
    H.compare(o[1:2], ro, torch.bfloat16, "contract: valid sequence", strict=False)


# ---- pooled cache: linear regions for KV heads with a full query head, sink + ring regions
# for all-sparse ones (ea_decode_pool_layout / _fill / _append, ea_hybrid_attn_decode_pool)

def ring_row(j, sink, window):
    """Row of position j in a sink + ring region (the layout documented in include/ea.h)."""
    return j if j < sink else sink + (j - sink) % window


def pack(kc, lens):
    """Dense per-sequence caches [B, cap, Hkv, D] -> packed [T, Hkv, D] and cu_seqlens."""
    return torch.cat([kc[b, :L] for b, L in enumerate(lens)]), inputs.cu_seqlens(lens)


def build_pool(kc, vc, lens, route, sink, window, capacity):
    """Lay out the pool for `route`, poison it with NaN, fill it from the first lens[b]
    positions of the dense caches; returns GPU (k_pool, v_pool, base, rows) and the layout."""
    hkv = kc.shape[2]
    base, rows, total = ea.decode_pool_layout(route.numpy(), hkv, capacity, sink, window)
    kp = torch.full((total, kc.shape[3]), float("nan"), dtype=kc.dtype, device=H.device())
    vp = torch.full_like(kp, float("nan"))
    k, cu = pack(kc, lens)
    v, _ = pack(vc, lens)
    gb, gr = H.to_gpu(base), H.to_gpu(rows)
    ea.decode_pool_fill(H.to_gpu(k), H.to_gpu(v), H.to_gpu(cu), max(lens), route.shape[1],
                        H.to_gpu(route), sink, window, gb, gr, kp, vp)
    torch.cuda.synchronize()
    return kp, vp, gb, gr, base, rows


def run_pool_decode(q, kp, vp, gb, gr, lens, route, hkv, sink, window, max_seqlen=None):
    dev = H.device()
    B, hq, d = q.shape
    qg = H.to_gpu(q)
    o = torch.full_like(qg, float("nan"))
    lse = torch.full((B, hq), float("nan"), dtype=torch.float32, device=dev)
    max_seqlen = max_seqlen or max(lens)
    ws = torch.empty(ea.decode_workspace_size(B, max_seqlen, hq, d), dtype=torch.uint8, device=dev)
    ea.hybrid_attn_decode_pool(qg, kp, vp, o, torch.tensor(lens, dtype=torch.int32, device=dev),
                               max_seqlen, hkv, gb, gr, H.to_gpu(route), sink, window, ws,
                               lse_out=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def test_pool_fill_placement():
    """Every kept position lands in its row bit for bit; rows no position maps to keep the
    poison."""
    lens, hq, hkv, d, sink, window = [5, 40, 300], 4, 2, 128, 4, 16
    g = torch.Generator().manual_seed(11)
    kc = torch.randn(3, 300, hkv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(3, 300, hkv, d, generator=g).to(torch.bfloat16)
    route = torch.tensor([[1, 1, 0, 1], [1, 1, 1, 1], [0, 1, 1, 1]], dtype=torch.uint8)
    kp, vp, _, _, base, rows = build_pool(kc, vc, lens, route, sink, window, capacity=300)
    kp, vp = kp.cpu(), vp.cpu()
    G = hq // hkv
    for b, L in enumerate(lens):
        for h in range(hkv):
            r0, n = int(base[b * hkv + h]), int(rows[b * hkv + h])
            all_sparse = bool(route[b, h * G:(h + 1) * G].all())
            written = set()
            for j in range(L):
                if all_sparse:
                    if not (j < sink or j >= L - window):
                        continue
                    r = ring_row(j, sink, window)
                else:
                    r = j
                written.add(r)
                assert torch.equal(kp[r0 + r].view(torch.int16), kc[b, j, h].view(torch.int16)), (b, h, j)
                assert torch.equal(vp[r0 + r].view(torch.int16), vc[b, j, h].view(torch.int16)), (b, h, j)
            for r in set(range(n)) - written:
                assert torch.isnan(kp[r0 + r].float()).all() and torch.isnan(vp[r0 + r].float()).all()


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 128)])
def test_pool_decode_matches_dense_and_oracle(dtype, d):
    """Lengths below the sink, inside sink + window, one past it (first wrap), on split
    boundaries and far beyond; every group routing.  The pooled step equals the dense-cache
    step bit for bit (same keys in the same order) and the oracle within the bounds."""
    lens = [2, 20, 24, 25, 257, 700, 1500]
    hkv, G, sink, window, cap = 2, 4, 4, 20, 1536
    hq = hkv * G
    g = torch.Generator().manual_seed(400 + d)
    B = len(lens)
    q = torch.randn(B, hq, d, generator=g).to(dtype)
    kc = torch.randn(B, cap, hkv, d, generator=g).to(dtype)
    vc = torch.randn(B, cap, hkv, d, generator=g).to(dtype)
    route = (torch.rand(B, hq, generator=g) < 0.7).to(torch.uint8)
    route[0, :G] = 1
    route[1, :] = 1
    route[2, G:] = 0
    route[4, :G] = 1
    kp, vp, gb, gr, base, rows = build_pool(kc, vc, lens, route, sink, window, cap)
    say(f"case pool d{d} {dtype}: pool rows {int(rows.sum())} vs dense {B * cap * hkv}")
    o, lse = run_pool_decode(q, kp, vp, gb, gr, lens, route, hkv, sink, window)
    od, ld = run_decode(q, kc, vc, lens, route, sink, window)
    assert torch.equal(o.view(torch.int16) if dtype == torch.bfloat16 else o, od.view(torch.int16) if dtype == torch.bfloat16 else od)
    assert torch.equal(lse, ld)
    ro, rl = oracle.decode(q, kc, vc, lens, hkv, route.numpy(), sink, window)
    H.compare(o, ro, dtype, f"pool d{d}", strict=False)
    tol = 1e-3 if dtype == torch.bfloat16 else 1e-5
    assert np.abs(lse.double().numpy() - rl).max() <= tol


def test_pool_append_then_decode_steps():
    """Prefill, then 40 steps of append + decode with a window of 8: rings wrap five times;
    every step matches the oracle over the dense history."""
    hkv, G, d, sink, window, steps = 2, 4, 128, 3, 8, 40
    hq = hkv * G
    lens0 = [1, 3, 6, 11, 30]
    B = len(lens0)
    cap = max(lens0) + steps
    g = torch.Generator().manual_seed(77)
    kc = torch.randn(B, cap, hkv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, cap, hkv, d, generator=g).to(torch.bfloat16)
    route = torch.ones(B, hq, dtype=torch.uint8)
    route[2, 1] = 0      # sequence 2, KV head 0 keeps a linear region
    route[4, G:] = 0     # sequence 4, KV head 1 too
    kp, vp, gb, gr, base, rows = build_pool(kc, vc, lens0, route, sink, window, cap)
    groute = H.to_gpu(route)
    dev = H.device()
    for s in range(steps):
        lens = [L + s + 1 for L in lens0]
        pos = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device=dev)
        k_new = torch.stack([kc[b, lens[b] - 1] for b in range(B)])
        v_new = torch.stack([vc[b, lens[b] - 1] for b in range(B)])
        ea.decode_pool_append(H.to_gpu(k_new), H.to_gpu(v_new), pos, hq, groute, sink, window,
                              gb, gr, kp, vp)
        q = torch.randn(B, hq, d, generator=g).to(torch.bfloat16)
        o, lse = run_pool_decode(q, kp, vp, gb, gr, lens, route, hkv, sink, window,
                                 max_seqlen=cap)
        ro, rl = oracle.decode(q, kc, vc, lens, hkv, route.numpy(), sink, window)
        H.compare(o, ro, torch.bfloat16, f"append step {s}", strict=False)
        assert np.abs(lse.double().numpy() - rl).max() <= 1e-3, s


def test_pool_regions_that_cannot_serve_give_nan():
    """A ring one row short of sink + window, and a region past the pool's end: that KV head's
    query heads get NaN; every other head is exact."""
    hkv, G, d, sink, window = 2, 2, 128, 4, 16
    hq = hkv * G
    lens = [50, 50]
    g = torch.Generator().manual_seed(3)
    q = torch.randn(2, hq, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(2, 64, hkv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(2, 64, hkv, d, generator=g).to(torch.bfloat16)
    route = torch.tensor([[1, 1, 0, 1], [1, 1, 1, 1]], dtype=torch.uint8)
    kp, vp, gb, gr, base, rows = build_pool(kc, vc, lens, route, sink, window, 64)
    rows_bad = rows.clone()
    rows_bad[0] = sink + window - 1                 # (b 0, kvh 0): ring too short
    base_bad = base.clone()
    base_bad[3] = kp.shape[0] - 5                   # (b 1, kvh 1): runs past the pool
    o, lse = run_pool_decode(q, kp, vp, H.to_gpu(base_bad), H.to_gpu(rows_bad), lens, route, hkv,
                             sink, window)
    ro, _ = oracle.decode(q, kc, vc, lens, hkv, route.numpy(), sink, window)
    for b, h in ((0, 0), (0, 1), (1, 2), (1, 3)):
        assert torch.isnan(o[b, h].float()).all() and torch.isnan(lse[b, h])
    for b, h in ((0, 2), (0, 3), (1, 0), (1, 1)):
        H.compare(o[b, h][None, None], ro[b, h][None, None], torch.bfloat16, f"valid {b},{h}",
                  strict=False)


@pytest.mark.parametrize("seed", range(8))
def test_decode_random_configs(seed):
    """Seeded random decode batches: 1-8 sequences with lengths from 1 to the cache capacity,
    group sizes 1-8, head_dim 64 or 128, bf16 or fp32, random sink, window and routing."""
    rng = np.random.default_rng(4000 + seed)
    B = int(rng.integers(1, 9))
    cap = int(rng.choice([64, 300, 1024, 2100]))
    lens = [int(rng.integers(1, cap + 1)) for _ in range(B)]
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.75 else torch.float32
    sink = int(rng.choice([0, 1, 16, 128]))
    window = int(rng.choice([1, 50, 256, 3000]))
    g = torch.Generator().manual_seed(500 + seed)
    q = torch.randn(B, hq, d, generator=g).to(dtype)
    kc = torch.randn(B, cap, hkv, d, generator=g).to(dtype)
    vc = torch.randn(B, cap, hkv, d, generator=g).to(dtype)
    route = (torch.rand(B, hq, generator=g) < float(rng.random())).to(torch.uint8)
    check_decode(q, kc, vc, lens, route, sink, window, f"random {seed}")


@pytest.mark.parametrize("seed", range(6))
def test_pool_random_configs(seed):
    """Seeded random pooled-cache steps: 1-8 sequences of lengths 1 up to the capacity, group
    sizes 1-8, head_dim 64 or 128, bf16 or fp32, random sink, window and routing.  The pooled
    step equals the dense-cache step bit for bit and the oracle within the bounds."""
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 9))
    cap = int(rng.choice([64, 300, 1024, 2100]))
    lens = [int(rng.integers(1, cap + 1)) for _ in range(B)]
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * G
    d = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.75 else torch.float32
    sink = int(rng.choice([0, 1, 16, 128]))
    window = int(rng.choice([1, 50, 256, 3000]))
    g = torch.Generator().manual_seed(700 + seed)
    q = torch.randn(B, hq, d, generator=g).to(dtype)
    kc = torch.randn(B, cap, hkv, d, generator=g).to(dtype)
    vc = torch.randn(B, cap, hkv, d, generator=g).to(dtype)
    route = (torch.rand(B, hq, generator=g) < float(rng.random())).to(torch.uint8)
    kp, vp, gb, gr, base, rows = build_pool(kc, vc, lens, route, sink, window, cap)
    say(f"case pool random {seed}: B={B} cap={cap} lens={lens} hq={hq} hkv={hkv} d={d} {dtype} "
        f"s={sink} W={window}")
    o, lse = run_pool_decode(q, kp, vp, gb, gr, lens, route, hkv, sink, window)
    od, ld = run_decode(q, kc, vc, lens, route, sink, window)
    if dtype == torch.bfloat16:
        assert torch.equal(o.view(torch.int16), od.view(torch.int16))
    else:
        assert torch.equal(o, od)
    assert torch.equal(lse, ld)
    ro, rl = oracle.decode(q, kc, vc, lens, hkv, route.numpy(), sink, window)
    H.compare(o, ro, dtype, f"pool random {seed}", strict=False)
    tol = 1e-3 if dtype == torch.bfloat16 else 1e-5
    assert np.abs(lse.double().numpy() - rl).max() <= tol
