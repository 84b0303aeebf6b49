"""Shared helpers for the GPU parity tests: put seeded inputs on the GPU, run the HIP path
through the C ABI binding, run the oracle on the same bytes, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from full_attention_long_amd import ea, inputs

BF16_MAX_ABS = 1e-2    # bf16 outputs, fp32 accumulation
BF16_MEAN_ABS = 1e-3
F32_MAX_ABS = 1e-5     # fp32 path


def device():
    return torch.device("cuda:0")


def to_gpu(t):
    return t.to(device(), non_blocking=False)


def workspace(batch, max_seqlen, n_heads_q, kv_dim=0, hidden=0):
    n = ea.workspace_size(batch, max_seqlen, n_heads_q, kv_dim, hidden)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=device())


def run_prefill(q, k, v, lens, route, sink, window, scale=0.0, want_lse=True, guard=0,
                worklist=True):
    """Run ea_hybrid_attn_prefill on CPU tensors (copied to the GPU).  Returns
    (o_cpu, lse_cpu or None, worklist int32 [n,4] or None, guard_ok)."""
    T, hq, d = q.shape
    batch = len(lens)
    cu = inputs.cu_seqlens(lens)
    max_len = max(lens) if lens else 0
    dq, dk, dv = to_gpu(q), to_gpu(k), to_gpu(v)
    sentinel = -12288.0  # exact in bf16 and fp32
    o_full = torch.full((T + 2 * guard, hq, d), sentinel, dtype=q.dtype, device=device())
    o = o_full[guard:guard + T]
    lse = torch.full((hq, T), float("nan"), dtype=torch.float32, device=device()) if want_lse else None
    dt = ea.dtype_code(q.dtype)
    bm, _ = ea.tile_config(dt, d)
    cap = max(1, batch * hq * -(-max_len // bm))
    wl = torch.full((cap, 4), -1, dtype=torch.int32, device=device()) if worklist else None
    ws = workspace(batch, max_len, hq)
    dcu = to_gpu(cu)
    droute = to_gpu(route.to(torch.uint8).contiguous())
    ea.hybrid_attn_prefill(dq, dk, dv, o, dcu, max_len, droute, sink, window, ws, scale=scale,
                           cu_seqlens_host=cu.tolist(), lse_out=lse, worklist_out=wl)
    torch.cuda.synchronize()
    guard_ok = True
    if guard:
        head = o_full[:guard].float().cpu()
        tail = o_full[guard + T:].float().cpu()
        guard_ok = bool(torch.all(head == sentinel)) and bool(torch.all(tail == sentinel))
    items = None
    if worklist:
        items = wl.cpu().numpy()
        n_items = sum(hq * -(-L // bm) for L in lens)
        assert np.all(items[n_items:] == -1)
        items = items[:n_items]
    return o.cpu(), (lse.cpu() if want_lse else None), items, guard_ok


def compare(o_gpu, o_ref, dtype, what="", strict=True):
    """Element-wise check of GPU output (any float dtype) against the fp64 oracle.

    bf16, strict (the workload layers): max-abs <= 1e-2 and mean-abs <= 1e-3.
    bf16, not strict (synthetic rows with only a handful of visible keys, where |o| can
    exceed 2): a bf16 number near 4 is itself up to 2^-6 = 0.0156 away from the exact
    value, so the bound is 1e-2 * max(1, |o|/2) per element -- 1e-2 absolute where the
    format allows it, 0.5% relative (about one bf16 ulp) above 2; mean-abs <= 1e-3.
    fp32: max-abs <= 1e-5."""
    got = o_gpu.double().numpy()
    err = np.abs(got - o_ref)
    max_abs = float(err.max()) if err.size else 0.0
    mean_abs = float(err.mean()) if err.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if dtype == torch.bfloat16:
        floor = float(np.abs(torch.from_numpy(o_ref).to(torch.bfloat16).double().numpy()
                             - o_ref).max()) if err.size else 0.0
        tol = BF16_MAX_ABS if strict else BF16_MAX_ABS * np.maximum(1.0, np.abs(o_ref) / 2)
        worst = np.unravel_index(int((err - tol).argmax()), err.shape) if err.size else None
        assert np.all(err <= tol) and mean_abs <= BF16_MEAN_ABS, (
            f"{what}: max_abs {max_abs:.3e} mean_abs {mean_abs:.3e} (bf16 rounding floor "
            f"{floor:.3e}) worst at {worst}")
    else:
        assert max_abs <= F32_MAX_ABS, f"{what}: max_abs {max_abs:.3e}"
    return max_abs, mean_abs
