"""GPU parity of the chunked prefill over a KV prefix (ea_hybrid_attn_prefill_chunked, through
the C ABI) against the fp64 oracle with a separate key packing: each sequence's queries are
its last Lq of Lk positions.  Bounds as for the prefill: bf16 max-abs 1e-2 and mean-abs 1e-3
(edge cases with a handful of visible keys: 1e-2 * max(1, |o|/2)), fp32 1e-5, LSE 4e-3 / 1e-5;
the work list is compared bit for bit."""
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


def chunk_inputs(lens_k, lens_q, hq, hkv, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    Tk = sum(lens_k)
    qfull = torch.randn(Tk, hq, d, generator=g).to(dtype)
    k = torch.randn(Tk, hkv, d, generator=g).to(dtype)
    v = torch.randn(Tk, hkv, d, generator=g).to(dtype)
    cu_k = inputs.cu_seqlens(lens_k)
    q = torch.cat([qfull[int(cu_k[b + 1]) - lq:int(cu_k[b + 1])] for b, lq in enumerate(lens_q)])
    return q, k, v, inputs.cu_seqlens(lens_q), cu_k


def run_chunked(q, k, v, cu_q, cu_k, route, sink, window, worklist=True, host=True):
    dev = H.device()
    lens_q = (cu_q[1:] - cu_q[:-1]).tolist()
    lens_k = (cu_k[1:] - cu_k[:-1]).tolist()
    Tq, hq, d = q.shape
    sentinel = -12288.0
    o = torch.full((Tq, hq, d), sentinel, dtype=q.dtype, device=dev)
    lse = torch.full((hq, Tq), float("nan"), dtype=torch.float32, device=dev)
    dt = ea.dtype_code(q.dtype)
    bm, _ = ea.tile_config(dt, d)
    mq, mk = max(lens_q), max(lens_k)
    cap = max(1, len(lens_q) * hq * -(-mq // bm))
    wl = torch.full((cap, 4), -1, dtype=torch.int32, device=dev) if worklist else None
    ws = torch.empty(ea.prefill_chunked_workspace_size(len(lens_q), mq, hq, d), dtype=torch.uint8,
                     device=dev)
    ea.hybrid_attn_prefill_chunked(H.to_gpu(q), H.to_gpu(k), H.to_gpu(v), o, H.to_gpu(cu_q),
                                   H.to_gpu(cu_k), mq, mk, H.to_gpu(route.to(torch.uint8)), sink,
                                   window, ws, cu_seqlens_q_host=cu_q.tolist() if host else None,
                                   cu_seqlens_k_host=cu_k.tolist() if host else None,
                                   lse_out=lse, worklist_out=wl)
    torch.cuda.synchronize()
    items = None
    if worklist:
        items = wl.cpu().numpy()
    return o.cpu(), lse.cpu(), items, bm


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 128)])
def test_chunked_ragged(dtype, d):
    lens_k, lens_q = [300, 1000, 777, 64, 513], [300, 257, 1, 64, 100]
    hq, hkv, sink, window = 8, 2, 16, 200
    q, k, v, cu_q, cu_k = chunk_inputs(lens_k, lens_q, hq, hkv, d, dtype, 31 + d)
    g = torch.Generator().manual_seed(5)
    route = (torch.rand(len(lens_q), hq, generator=g) < 0.6).to(torch.uint8)
    say(f"case chunked d{d} {dtype}: lens_k={lens_k} lens_q={lens_q}")
    o, lse, items, bm = run_chunked(q, k, v, cu_q, cu_k, route, sink, window)
    ro, rl = oracle.attn(q, k, v, cu_q, hq, hkv, route.numpy(), sink, window,
                         cu_seqlens_k=cu_k)
    H.compare(o, ro, dtype, f"chunked d{d}", strict=False)
    tol = 4e-3 if dtype == torch.bfloat16 else 1e-5
    assert np.abs(lse.double().numpy().T - rl).max() <= tol
    _, bn = ea.tile_config(ea.dtype_code(dtype), d)
    want = oracle.worklist(route.numpy(), cu_q, hq, sink, window, bm, bn, cu_seqlens_k=cu_k)
    assert np.array_equal(items[:len(want)], want)
    assert np.all(items[len(want):] == -1)


def test_chunk_of_32k_sequence_sampled_rows():
    """A 4096-token chunk at the end of a 32768-token sequence, Qwen3-8B-shaped heads, the
    32K layer's sink and window, mixed routing: 512 sampled chunk rows against the oracle."""
    lk, lq, hq, hkv, d, sink, window = 32768, 4096, 32, 8, 128, 128, 2048
    q, k, v, cu_q, cu_k = chunk_inputs([lk], [lq], hq, hkv, d, torch.bfloat16, 99)
    g = torch.Generator().manual_seed(8)
    route = (torch.rand(1, hq, generator=g) < 0.85).to(torch.uint8)
    route[0, 0] = 0
    o, lse, _, _ = run_chunked(q, k, v, cu_q, cu_k, route, sink, window, worklist=False)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rows = np.sort(np.random.default_rng(3).choice(lq, 512, replace=False))
    rows[0], rows[-1] = 0, lq - 1
    ro, rl = oracle.attn(q, k, v, cu_q, hq, hkv, route.numpy(), sink, window, rows=rows,
                         cu_seqlens_k=cu_k)
    H.compare(o[rows], ro, torch.bfloat16, "chunk of 32K", strict=True)
    assert np.abs(lse.double().numpy().T[rows] - rl).max() <= 4e-3


def test_whole_sequence_chunk_equals_prefill():
    """cu_seqlens_k == cu_seqlens_q: bit-identical to ea_hybrid_attn_prefill."""
    lens = [700, 129, 1000]
    hq, hkv, d, sink, window = 8, 2, 128, 32, 256
    q, k, v, cu_q, cu_k = chunk_inputs(lens, lens, hq, hkv, d, torch.bfloat16, 17)
    route = torch.tensor([[0, 1, 1, 1, 0, 1, 1, 0]] * 3, dtype=torch.uint8)
    o, lse, items, _ = run_chunked(q, k, v, cu_q, cu_k, route, sink, window)
    po, plse, pitems, _ = H.run_prefill(q, k, v, lens, route, sink, window)
    assert torch.equal(o.view(torch.int16), po.view(torch.int16))
    assert torch.equal(lse, plse)
    assert np.array_equal(items[:len(pitems)], pitems)


def test_device_chunk_longer_than_keys_is_skipped():
    """Without host copies, a sequence whose chunk is longer than its keys gets no work (its
    rows keep the sentinel); the other sequences are exact."""
    lens_k, lens_q = [200, 50, 300], [100, 80, 300]   # sequence 1: 80 queries, 50 keys
    hq, hkv, d, sink, window = 4, 1, 128, 8, 64
    q, k, v, cu_q, cu_k = chunk_inputs([200, 80, 300], lens_q, hq, hkv, d, torch.bfloat16, 2)
    # keys packed with sequence 1 cut to its first 50 positions
    k = torch.cat([k[:200], k[200:250], k[280:580]])
    v = torch.cat([v[:200], v[200:250], v[280:580]])
    cu_k = inputs.cu_seqlens(lens_k)
    route = torch.tensor([[0, 1, 1, 0]] * 3, dtype=torch.uint8)
    o, _, _, _ = run_chunked(q, k, v, cu_q, cu_k, route, sink, window, worklist=False, host=False)
    assert torch.all(o[100:180].float() == -12288.0)
    for b, (s0, s1) in enumerate(((0, 100), (180, 480))):
        bb = 0 if b == 0 else 2
        ro, _ = oracle.attn(q[s0:s1], k[cu_k[bb]:cu_k[bb + 1]], v[cu_k[bb]:cu_k[bb + 1]],
                            [0, s1 - s0], hq, hkv, route[bb:bb + 1].numpy(), sink, window,
                            cu_seqlens_k=[0, int(cu_k[bb + 1] - cu_k[bb])])
        H.compare(o[s0:s1], ro, torch.bfloat16, f"valid sequence {bb}", strict=False)


def test_device_lengths_beyond_max_seqlen_give_an_empty_work_list():
    """Without host copies the planner cannot trust the device lengths: a sequence longer than
    max_seqlen makes more items than the work list holds, so the list comes out empty and
    nothing is written (no item past the list's capacity, no cell past the planner's LDS)."""
    L, hq, hkv, d = 4096, 4, 1, 128
    g = torch.Generator().manual_seed(1)
    q = torch.randn(L, hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(L, hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(L, hkv, d, generator=g).to(torch.bfloat16)
    dev = H.device()
    o = torch.full((L, hq, d), -12288.0, dtype=torch.bfloat16, device=dev)
    route = torch.tensor([[0, 1, 1, 0]], dtype=torch.uint8, device=dev)
    cu = torch.tensor([0, L], dtype=torch.int32, device=dev)
    ws = H.workspace(1, 256, hq)
    ea.hybrid_attn_prefill(H.to_gpu(q), H.to_gpu(k), H.to_gpu(v), o, cu, 256, route, 4, 64, ws)
    torch.cuda.synchronize()
    assert torch.all(o.float() == -12288.0)
    wsc = torch.empty(ea.prefill_chunked_workspace_size(1, 256, hq, d), dtype=torch.uint8,
                      device=dev)
    ea.hybrid_attn_prefill_chunked(H.to_gpu(q), H.to_gpu(k), H.to_gpu(v), o, cu, cu, 256, 256,
                                   route, 4, 64, wsc)
    torch.cuda.synchronize()
    assert torch.all(o.float() == -12288.0)


def test_chunked_many_query_heads():
    """128 query heads on 16 KV heads, long enough that full-head items split: the planner's
    split phase over many items (costs read from its sorted cells), every row and the work
    list against the oracle."""
    lens_k, lens_q = [2600, 900], [700, 900]
    hq, hkv, d = 128, 16, 64
    q, k, v, cu_q, cu_k = chunk_inputs(lens_k, lens_q, hq, hkv, d, torch.bfloat16, 4711)
    g = torch.Generator().manual_seed(4712)
    route = (torch.rand(len(lens_k), hq, generator=g) < 0.5).to(torch.uint8)
    sink, window = 16, 256
    say(f"case chunked hq {hq}: lens_k={lens_k} lens_q={lens_q} hkv={hkv} d={d}")
    o, lse, items, bm = run_chunked(q, k, v, cu_q, cu_k, route, sink, window)
    ro, rl = oracle.attn(q, k, v, cu_q, hq, hkv, route.numpy(), sink, window, cu_seqlens_k=cu_k)
    H.compare(o, ro, torch.bfloat16, f"chunked hq {hq}", strict=False)
    assert np.abs(lse.double().numpy().T - rl).max() <= 4e-3
    _, bn = ea.tile_config(ea.dtype_code(torch.bfloat16), d)
    want = oracle.worklist(route.numpy(), cu_q, hq, sink, window, bm, bn, cu_seqlens_k=cu_k)
    assert np.array_equal(items[:len(want)], want)
    assert np.all(items[len(want):] == -1)


@pytest.mark.parametrize("seed", range(8))
def test_chunked_random_configs(seed):
    """Seeded random chunks: 1-4 sequences, key lengths from 1 to 2600, chunk lengths from
    empty to the whole sequence, group sizes 1-8, head_dim 64 or 128, bf16 or fp32, random
    sink, window and routing; every chunk row and the work list against the oracle."""
    rng = np.random.default_rng(3000 + seed)
    nseq = int(rng.integers(1, 5))
    lens_k = [int(x) for x in rng.choice([1, 64, 65, 300, 777, 1500, 2600], size=nseq)]
    lens_q = [lk if rng.random() < 0.3 else int(rng.integers(0, lk + 1)) for lk in lens_k]
    if sum(lens_q) == 0:
        lens_q[0] = lens_k[0]
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.75 else torch.float32
    sink = int(rng.choice([0, 1, 16, 128]))
    window = int(rng.choice([1, 50, 256, 3000]))
    q, k, v, cu_q, cu_k = chunk_inputs(lens_k, lens_q, hq, hkv, d, dtype, 400 + seed)
    g = torch.Generator().manual_seed(600 + seed)
    route = (torch.rand(nseq, hq, generator=g) < float(rng.random())).to(torch.uint8)
    say(f"case chunked random {seed}: lens_k={lens_k} lens_q={lens_q} hq={hq} hkv={hkv} d={d} "
        f"{dtype} s={sink} W={window}")
    o, lse, items, bm = run_chunked(q, k, v, cu_q, cu_k, route, sink, window)
    ro, rl = oracle.attn(q, k, v, cu_q, hq, hkv, route.numpy(), sink, window, cu_seqlens_k=cu_k)
    H.compare(o, ro, dtype, f"chunked random {seed}", strict=False)
    tol = 4e-3 if dtype == torch.bfloat16 else 1e-5
    assert np.abs(lse.double().numpy().T - rl).max() <= tol
    _, bn = ea.tile_config(ea.dtype_code(dtype), d)
    want = oracle.worklist(route.numpy(), cu_q, hq, sink, window, bm, bn, cu_seqlens_k=cu_k)
    assert np.array_equal(items[:len(want)], want)
    assert np.all(items[len(want):] == -1)
