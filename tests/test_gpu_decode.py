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
