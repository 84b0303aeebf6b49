"""The entry point that allocates nothing (ea_hybrid_attn_prefill_noalloc, for callers that
cannot call hipMalloc) against ea_hybrid_attn_prefill on the same inputs: two calls in a
row, the second smaller, each bit-identical to the workspace entry point (same kernels,
same work list) and within the oracle's bounds."""
import numpy as np
import pytest
import torch

import oracle
from full_attention_long_amd import ea, inputs
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


def one_case(lens, hq, hkv, d, dtype, sink, window, seed):
    print(f"no-alloc case lens={lens} hq={hq} hkv={hkv} d={d} {dtype} s={sink} W={window}",
          flush=True)
    g = torch.Generator().manual_seed(seed)
    T = sum(lens)
    q = torch.randn(T, hq, d, generator=g).to(dtype)
    k = torch.randn(T, hkv, d, generator=g).to(dtype)
    v = torch.randn(T, hkv, d, generator=g).to(dtype)
    route = (torch.rand(len(lens), hq, generator=g) < 0.6).to(torch.uint8)
    cu = inputs.cu_seqlens(lens)
    dq, dk, dv, dcu, dr = (H.to_gpu(t) for t in (q, k, v, cu, route))
    o_ref = torch.empty_like(dq)
    lse_ref = torch.empty(hq, T, dtype=torch.float32, device="cuda")
    ws = H.workspace(len(lens), max(lens), hq)
    ea.hybrid_attn_prefill(dq, dk, dv, o_ref, dcu, max(lens), dr, sink, window, ws,
                           cu_seqlens_host=cu.tolist(), lse_out=lse_ref)
    o = torch.full_like(dq, float("nan"))
    lse = torch.full((hq, T), float("nan"), dtype=torch.float32, device="cuda")
    ea.hybrid_attn_prefill_noalloc(dq, dk, dv, o, dcu, max(lens), dr, sink, window,
                                   cu_seqlens_host=cu.tolist(), lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       o_ref.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    assert torch.equal(lse, lse_ref)
    ro, _ = oracle.attn(q, k, v, cu, hq, hkv, route.numpy(), sink, window)
    H.compare(o.cpu(), ro, dtype, "no-alloc prefill", strict=False)


def test_noalloc_matches_workspace_entry_point_twice():
    # a larger call, then a smaller one on the same device array
    one_case([3000, 700, 1], 8, 2, 128, torch.bfloat16, 64, 512, 1)
    one_case([300, 45], 4, 1, 64, torch.bfloat16, 16, 64, 2)
    one_case([129, 64], 4, 2, 64, torch.float32, 3, 40, 3)


def test_noalloc_rejects_beyond_its_array():
    q = torch.empty(8, 32, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(8, 8, 128, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 4, 8] + [8] * 30, dtype=torch.int32, device="cuda")
    route = torch.zeros(32, 32, dtype=torch.uint8, device="cuda")
    # 32 sequences x 32 heads x ceil(20000 / 64) = 320512 work items > 262128
    with pytest.raises(ea.EAError, match="no-allocation"):
        ea.hybrid_attn_prefill_noalloc(q, k, k, q.clone(), cu, 20000, route, 0, 16)
