"""Work counts used to report effective throughput.

Effective FLOPs count only the (query, key) score positions the mask keeps: each kept
position costs 2*D FLOPs in Q K^T and 2*D in P V, i.e. 4*D in all.  Masked positions that
a tiled kernel still computes are not counted.

Visible keys of row i (0-based) of one sequence:
  full head (r = 0):     i + 1
  sparse head (r = 1):   min(i+1, W) window keys plus min(s, i-W+1) sink keys that the
                         window does not already cover (when i-W+1 > 0).
Summed over the L rows of a sequence:
  full:   L(L+1)/2
  sparse: window part L(L+1)/2 if L <= W else W(W+1)/2 + (L-W)W;
          sink part with n = L-W: 0 if n <= 0, n(n+1)/2 if n <= s, else s(s+1)/2 + (n-s)s.
"""
from __future__ import annotations


def visible_pairs(length: int, sparse: bool, sink: int, window: int) -> int:
    L, s, W = int(length), int(sink), int(window)
    if L <= 0:
        return 0
    if not sparse:
        return L * (L + 1) // 2
    win = L * (L + 1) // 2 if L <= W else W * (W + 1) // 2 + (L - W) * W
    n = L - W
    if n <= 0:
        snk = 0
    elif n <= s:
        snk = n * (n + 1) // 2
    else:
        snk = s * (s + 1) // 2 + (n - s) * s
    return win + snk


def effective_flops(lengths, route, head_dim: int, sink: int, window: int) -> int:
    """Sum over sequences b and query heads h of 4*D*visible_pairs(L_b, route[b][h])."""
    total = 0
    for b, L in enumerate(lengths):
        for r in route[b]:
            total += 4 * int(head_dim) * visible_pairs(L, bool(int(r)), sink, window)
    return total


def chunk_flops(lengths_k, lengths_q, route, head_dim: int, sink: int, window: int) -> int:
    """Effective FLOPs of a chunked prefill: the chunk rows are the last Lq of Lk positions and
    a row's visible keys depend only on its position, so their pairs are
    visible_pairs(Lk) - visible_pairs(Lk - Lq)."""
    total = 0
    for b, (Lk, Lq) in enumerate(zip(lengths_k, lengths_q)):
        for r in route[b]:
            sp = bool(int(r))
            total += 4 * int(head_dim) * (visible_pairs(Lk, sp, sink, window) -
                                          visible_pairs(Lk - Lq, sp, sink, window))
    return total


def io_bytes(total_tokens: int, n_heads_q: int, n_heads_kv: int, head_dim: int,
             elem_bytes: int) -> int:
    """Algorithmic HBM bytes of one attention launch: Q, K, V read once, O written once."""
    return int(total_tokens) * int(head_dim) * int(elem_bytes) * (2 * n_heads_q + 2 * n_heads_kv)


def decode_group_keys(length: int, all_sparse: bool, sink: int, window: int) -> int:
    """Cache rows a KV-head group must read for the query at i = L - 1: all L when any
    query head of the group is full; otherwise the window min(W, L) plus the sink keys
    below it, min(s, L - W) when L > W."""
    L, s, W = int(length), int(sink), int(window)
    if L <= 0:
        return 0
    if not all_sparse:
        return L
    return min(W, L) + min(s, max(0, L - W))


def decode_bytes(lengths, route, n_heads_kv: int, head_dim: int, sink: int, window: int,
                 elem_bytes: int) -> int:
    """Algorithmic HBM bytes of one decode step: for every sequence and KV head, the K and
    V rows its group of query heads sees, read once; plus q read and o written."""
    total = 0
    for b, L in enumerate(lengths):
        r = [int(x) for x in route[b]]
        G = len(r) // int(n_heads_kv)
        for kvh in range(int(n_heads_kv)):
            grp = r[kvh * G:(kvh + 1) * G]
            n = decode_group_keys(L, all(grp), sink, window)
            total += 2 * n * int(head_dim) * int(elem_bytes)
        total += 2 * len(r) * int(head_dim) * int(elem_bytes)
    return total


MI355X_BF16_DENSE_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU, dense (no sparsity)
MI355X_HBM_GBPS = 8000.0
MI355X_FP32_VECTOR_TFLOPS = 157.3   # 256 CU x 2.4 GHz x 256 FLOP/clk/CU (fp32 FMA, vector ALU)


def backward_flops(lengths, route, head_dim: int, sink: int, window: int) -> int:
    """Effective FLOPs of the attention backward: per kept position the five products
    S = Q K^T (recomputed), dP = dO V^T, dV = P^T dO, dQ = dS K and dK = dS^T Q at 2*D each,
    i.e. 10*D = 2.5 x the forward's 4*D (the usual accounting for attention backward)."""
    return effective_flops(lengths, route, head_dim, sink, window) * 5 // 2


def backward_kernel_flops(lengths, route, head_dim: int, sink: int, window: int):
    """Algorithmic FLOPs of the two backward kernels as built: the dq kernel computes S, dP and
    dQ per kept position (6*D), the dk/dv kernel S, dP, dV and dK (8*D).
    Returns (dq_flops, dkv_flops)."""
    pairs = 0
    for b, L in enumerate(lengths):
        for r in route[b]:
            pairs += visible_pairs(L, bool(int(r)), sink, window)
    return 6 * int(head_dim) * pairs, 8 * int(head_dim) * pairs


def route_backward_bytes(total_tokens: int, n_heads_q: int, head_dim: int, kv_dim: int,
                         out_elem: int, key_elem: int) -> int:
    """Algorithmic HBM bytes of the router backward: O_full, O_sparse and dO read once
    ([T, Hq, D] each), the key states read once for the mean pool, the fp32 key-state gradient
    written once (the router's own weights are small)."""
    T = int(total_tokens)
    return 3 * T * n_heads_q * head_dim * out_elem + T * kv_dim * (key_elem + 4)
