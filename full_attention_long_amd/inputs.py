"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random numbers and fixes
workload shapes.  Both the HIP path and the oracle receive the exact bytes made here.

Seed scheme: workload k draws stream s from ``torch.Generator().manual_seed(1000*k + s)``.
Streams: 0 Q, 1 K, 2 V, 3 key states, 4 W1, 5 W2, 6 routing bits, 7 sequence lengths,
8 sampled query rows, 9-12 decode inputs, 13 the output gradient dO, 14 the router's
noise draw (training).  Values are ``randn`` in fp32, rounded to bf16 with
round-to-nearest-even by ``Tensor.to(torch.bfloat16)`` where the workload is bf16.

The workloads stand in for the pages' long-context evaluations (LongBench-E/V2 and RULER
up to 256K tokens, Elastic Attention blog post section 4); their sparse-head ratios follow
the per-task ratios the post reports for its Figure 6 (about 85% for code, 68% for QA).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

STREAM_Q, STREAM_K, STREAM_V, STREAM_KS, STREAM_W1, STREAM_W2 = 0, 1, 2, 3, 4, 5
STREAM_ROUTE, STREAM_LENS, STREAM_ROWS = 6, 7, 8
STREAM_DEC_Q, STREAM_DEC_K, STREAM_DEC_V, STREAM_DEC_LENS = 9, 10, 11, 12
STREAM_DOUT, STREAM_NOISE = 13, 14


def seed(workload: int, stream: int) -> int:
    return 1000 * workload + stream


def gen(workload: int, stream: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed(workload, stream))


@dataclass(frozen=True)
class Workload:
    """One synthetic prefill layer."""
    index: int                      # k in the seed scheme
    name: str
    dtype: torch.dtype
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    sink: int
    window: int
    lengths: tuple = ()             # fixed lengths; empty -> drawn (ragged)
    ragged_count: int = 0
    ragged_range: tuple = (0, 0)
    p_sparse: float = 0.0           # Bernoulli routing (ignored when fixed_route/router)
    fixed_route: tuple = ()         # explicit route for batch 1
    router: bool = False            # routing bits come from the Attention Router
    router_hidden: int = 256
    router_w_std: float = 0.02
    sampled_rows: int = 0           # 0 -> oracle evaluates every row
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # tiny fp32 correctness case: 1 x 512, 4 q heads on 2 KV heads, D=64, r=[0,1,0,1]
    "tiny_fp32": Workload(1, "tiny_fp32", torch.float32, 4, 2, 64, 16, 64,
                          lengths=(512,), fixed_route=(0, 1, 0, 1)),
    # Llama-3.1-8B-shaped layer at 8K, Bernoulli(0.7) sparse heads, sink 128, window 1024
    "llama8b_8k": Workload(2, "llama8b_8k", torch.bfloat16, 32, 8, 128, 128, 1024,
                           lengths=(8192,), p_sparse=0.7),
    # Qwen3-8B-shaped layer at 32K, routing from the Attention Router (27/32 sparse),
    # sink 128, window 2048
    "qwen3_8b_32k": Workload(3, "qwen3_8b_32k", torch.bfloat16, 32, 8, 128, 128, 2048,
                             lengths=(32768,), router=True, sampled_rows=2048),
    # ragged batch of 4, lengths U[4096, 32768], Bernoulli(0.68), sink 64, window 1024
    "ragged4": Workload(4, "ragged4", torch.bfloat16, 32, 8, 128, 64, 1024,
                        ragged_count=4, ragged_range=(4096, 32768), p_sparse=0.68,
                        sampled_rows=2048),
    # long context 256K, Bernoulli(0.8), sink 128, window 4096
    "long_256k": Workload(5, "long_256k", torch.bfloat16, 32, 8, 128, 128, 4096,
                          lengths=(262144,), p_sparse=0.8, sampled_rows=2048),
}


def lengths(w: Workload) -> list:
    if w.lengths:
        return list(w.lengths)
    lo, hi = w.ragged_range
    g = gen(w.index, STREAM_LENS)
    return [int(x) for x in torch.randint(lo, hi + 1, (w.ragged_count,), generator=g)]


def cu_seqlens(lens) -> torch.Tensor:
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def normal(shape, workload: int, stream: int, dtype: torch.dtype, std: float = 1.0,
           chunk_rows: int = 16384) -> torch.Tensor:
    """randn(shape) * std from the (workload, stream) generator, drawn in chunks of
    ``chunk_rows`` along dim 0 (bounded fp32 temporaries), then cast to ``dtype``."""
    g = gen(workload, stream)
    out = torch.empty(shape, dtype=dtype)
    n0 = shape[0]
    for a in range(0, n0, chunk_rows):
        b = min(n0, a + chunk_rows)
        x = torch.randn((b - a,) + tuple(shape[1:]), generator=g, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[a:b] = x.to(dtype)
    return out


def qkv(w: Workload, total_tokens: int):
    """Q [T, Hq, D], K [T, Hkv, D], V [T, Hkv, D] on the CPU."""
    q = normal((total_tokens, w.n_heads_q, w.head_dim), w.index, STREAM_Q, w.dtype)
    k = normal((total_tokens, w.n_heads_kv, w.head_dim), w.index, STREAM_K, w.dtype)
    v = normal((total_tokens, w.n_heads_kv, w.head_dim), w.index, STREAM_V, w.dtype)
    return q, k, v


def dout(w: Workload, total_tokens: int) -> torch.Tensor:
    """Output gradient dO [T, Hq, D] on the CPU (training)."""
    return normal((total_tokens, w.n_heads_q, w.head_dim), w.index, STREAM_DOUT, w.dtype)


def logistic_noise(w: Workload, batch: int) -> torch.Tensor:
    """fp32 [batch, Hq] draw of the logistic distribution, log(u) - log(1 - u) with
    u ~ U(0, 1) clamped to [1e-6, 1 - 1e-6] (the difference of two Gumbel draws)."""
    u = torch.rand((batch, w.n_heads_q), generator=gen(w.index, STREAM_NOISE))
    u = u.clamp(1e-6, 1.0 - 1e-6)
    return (torch.log(u) - torch.log1p(-u)).float()


def bernoulli_route(w: Workload, batch: int) -> torch.Tensor:
    """uint8 [batch, Hq]; 1 (sparse) with probability p_sparse, i.i.d."""
    if w.fixed_route:
        return torch.tensor([list(w.fixed_route)] * batch, dtype=torch.uint8)
    g = gen(w.index, STREAM_ROUTE)
    return (torch.rand((batch, w.n_heads_q), generator=g) < w.p_sparse).to(torch.uint8)


def router_weights(w: Workload):
    """Router parameters with the bias-free second layer: W1 [hidden, Hkv*D] and
    W2 [Hq, hidden] ~ N(0, std^2) fp32, b1 = 0, b2 = 0.  The output bias that sets the
    sparse ratio is a stored fixture (tests/golden), written from the oracle."""
    c = w.n_heads_kv * w.head_dim
    w1 = normal((w.router_hidden, c), w.index, STREAM_W1, torch.float32, std=w.router_w_std)
    w2 = normal((w.n_heads_q, w.router_hidden), w.index, STREAM_W2, torch.float32,
                std=w.router_w_std)
    b1 = torch.zeros(w.router_hidden, dtype=torch.float32)
    b2 = torch.zeros(w.n_heads_q, dtype=torch.float32)
    return w1, b1, w2, b2


def sampled_rows(w: Workload, lens, per_seq: int, bm: int = 128) -> torch.Tensor:
    """Packed token indices to check: for every sequence the boundary positions
    (0, 1, sink-1, sink, window-1, window, sink+window-2, sink+window-1, L-1 and the
    rows on both sides of a few q-tile edges) plus uniform draws without replacement,
    ``per_seq`` rows in all per sequence (fewer when the sequence is shorter)."""
    g = gen(w.index, STREAM_ROWS)
    out = []
    start = 0
    for n in lens:
        n = int(n)
        fixed = {0, 1, w.sink - 1, w.sink, w.window - 1, w.window,
                 w.sink + w.window - 2, w.sink + w.window - 1, n - 1}
        for t in (1, 2, 7, n // (2 * bm), n // bm - 1):
            fixed.update({t * bm - 1, t * bm})
        fixed = sorted(x for x in fixed if 0 <= x < n)
        want = min(per_seq, n)
        fixed_set = set(fixed)
        rest = [x for x in torch.randperm(n, generator=g).tolist() if x not in fixed_set]
        pick = sorted(fixed_set | set(rest[: max(0, want - len(fixed))]))
        out.extend(start + x for x in pick)
        start += n
    return torch.tensor(out, dtype=torch.int64)


# ---- decode steps: one new query per sequence over a per-sequence KV cache
@dataclass(frozen=True)
class DecodeWorkload:
    index: int                      # k in the seed scheme (distinct from the prefill ones)
    name: str
    dtype: torch.dtype
    batch: int
    capacity: int                   # cache slots per sequence
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    sink: int
    window: int
    p_sparse: float
    lengths: tuple = ()             # fixed lengths; empty -> U[len_range] per sequence
    len_range: tuple = (1, 1)


DECODE_WORKLOADS = {
    w.name: w for w in [
        DecodeWorkload(11, "decode_tiny_fp32", torch.float32, 3, 320, 4, 2, 64, 16, 64, 0.5,
                       lengths=(1, 70, 300)),
        DecodeWorkload(12, "decode_llama8b_8k", torch.bfloat16, 4, 8192, 32, 8, 128, 128, 1024,
                       0.7, lengths=(8192,) * 4),
        DecodeWorkload(13, "decode_qwen3_8b_32k", torch.bfloat16, 16, 32768, 32, 8, 128, 128,
                       2048, 0.85, lengths=(32768,) * 16),
        DecodeWorkload(14, "decode_ragged", torch.bfloat16, 8, 32768, 32, 8, 128, 64, 1024, 0.68,
                       len_range=(1, 32768)),
        DecodeWorkload(15, "decode_long_256k", torch.bfloat16, 1, 262144, 32, 8, 128, 128, 4096,
                       0.8, lengths=(262144,)),
    ]
}


def decode_lengths(w: DecodeWorkload) -> list:
    if w.lengths:
        return list(w.lengths)
    g = gen(w.index, STREAM_DEC_LENS)
    lo, hi = w.len_range
    return [int(x) for x in torch.randint(lo, hi + 1, (w.batch,), generator=g)]


def decode_inputs(w: DecodeWorkload, batch: int = 0):
    """q [B, Hq, D] and caches [B, cap, Hkv, D] (N(0,1) in w.dtype) for the first `batch`
    sequences (0 = all), plus their lengths and Bernoulli(p_sparse) routing [B, Hq]."""
    B = batch or w.batch
    lens = decode_lengths(w)[:B]
    q = normal((B, w.n_heads_q, w.head_dim), w.index, STREAM_DEC_Q, w.dtype)
    kc = normal((B * w.capacity, w.n_heads_kv, w.head_dim), w.index, STREAM_DEC_K, w.dtype)
    vc = normal((B * w.capacity, w.n_heads_kv, w.head_dim), w.index, STREAM_DEC_V, w.dtype)
    shape = (B, w.capacity, w.n_heads_kv, w.head_dim)
    g = gen(w.index, STREAM_ROUTE)
    route = (torch.rand(w.batch, w.n_heads_q, generator=g) < w.p_sparse).to(torch.uint8)[:B]
    return q, kc.view(shape), vc.view(shape), lens, route
