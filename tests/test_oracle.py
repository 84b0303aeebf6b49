"""Pins for the fp64 oracle, each against something other than the oracle itself:
brute force over an explicitly built dense mask, torch's scaled_dot_product_attention
(a library routine) on masks built from torch.tril/triu, closed forms, identities,
GQA invariants, a hand-derived router fixture and brute-force tile enumeration.

Pages: Elastic Attention blog post, section 1 (hybrid heads: full heads and heads that
only see a local / sliding window), section 2.1 "Attention Router" (r=0 full, r=1 sparse,
outputs concatenated per head, router = MLP over the key hidden states, 0.27M parameters
per layer for an 8B model in section 2.2), section 3 (routing handed to one kernel as
metadata); gist.science explanation, section "问题所在" (sparse = first and last pages).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle
from full_attention_long_amd import inputs, metrics

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
rng = np.random.default_rng(1234)


def lib_mask(L, sparse, sink, window):
    """Boolean [L, L] visibility built from torch primitives, not from a per-pair rule:
    causal = tril(ones); window = causal minus tril(ones, -window); sink = causal & the
    first `sink` columns."""
    ones = torch.ones(L, L, dtype=torch.bool)
    causal = torch.tril(ones)
    if not sparse:
        return causal
    band = causal & ~torch.tril(ones, diagonal=-window)
    cols = torch.zeros(L, L, dtype=torch.bool)
    cols[:, : min(sink, L)] = True
    return band | (causal & cols)


def sdpa_reference(q, k, v, cu, route, sink, window, scale):
    """Per sequence and head: torch SDPA in fp64 with the library-built mask."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    out = np.zeros((T, hq, d))
    lse = np.zeros((T, hq))
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        L = s1 - s0
        if L == 0:
            continue
        for h in range(hq):
            m = lib_mask(L, bool(route[b][h]), sink, window)
            qq = torch.as_tensor(q[s0:s1, h], dtype=torch.float64)
            kk = torch.as_tensor(k[s0:s1, h // G], dtype=torch.float64)
            vv = torch.as_tensor(v[s0:s1, h // G], dtype=torch.float64)
            o = F.scaled_dot_product_attention(qq[None], kk[None], vv[None], attn_mask=m[None],
                                               scale=scale)
            out[s0:s1, h] = o[0].numpy()
            sc = (qq @ kk.T * scale).masked_fill(~m, -math.inf).numpy()
            lse[s0:s1, h] = logsumexp(sc, axis=1)
    return out, lse


def dense_bruteforce(q, k, v, L, sparse, sink, window, scale):
    """Tiny-case brute force: explicit pair loop for the mask, dense softmax."""
    vis = np.zeros((L, L), dtype=bool)
    for i in range(L):
        for j in range(L):
            in_window = (i - window) < j <= i
            in_sink = j < sink and j <= i
            vis[i, j] = (j <= i) if not sparse else (in_window or in_sink)
    s = scale * (q @ k.T)
    s = np.where(vis, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


@pytest.mark.parametrize("L,sink,window", [(1, 0, 1), (5, 1, 2), (8, 2, 3), (8, 0, 4),
                                           (11, 3, 1), (12, 4, 20), (9, 12, 2)])
def test_tiny_bruteforce(L, sink, window):
    d, hq, hkv = 6, 4, 2
    q = rng.standard_normal((L, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    route = [[0, 1, 1, 0]]
    scale = 0.37
    o, _ = oracle.attn(q, k, v, [0, L], hq, hkv, route, sink, window, scale)
    for h in range(hq):
        ref = dense_bruteforce(q[:, h], k[:, h // 2], v[:, h // 2], L, route[0][h], sink,
                               window, scale)
        np.testing.assert_allclose(o[:, h], ref, atol=1e-12, rtol=0)


def test_sdpa_library_case_ragged_gqa():
    """Mixed routing, GQA 4:1, ragged packed batch against fp64 SDPA per sequence."""
    lens = [37, 1, 64, 50]
    cu = np.cumsum([0] + lens)
    T, hq, hkv, d = cu[-1], 8, 2, 16
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    route = rng.integers(0, 2, size=(len(lens), hq))
    sink, window, scale = 3, 9, 1 / 4
    o, lse = oracle.attn(q, k, v, cu, hq, hkv, route, sink, window, scale)
    ro, rlse = sdpa_reference(q, k, v, cu, route, sink, window, scale)
    np.testing.assert_allclose(o, ro, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, rlse, atol=1e-12, rtol=0)


def test_all_full_is_causal_sdpa():
    L, hq, hkv, d = 96, 4, 1, 32
    q = rng.standard_normal((L, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    o, _ = oracle.attn(q, k, v, [0, L], hq, hkv, [[0] * hq], 5, 7)
    kk = torch.as_tensor(k).permute(1, 0, 2).expand(hq, L, d)
    vv = torch.as_tensor(v).permute(1, 0, 2).expand(hq, L, d)
    ref = F.scaled_dot_product_attention(torch.as_tensor(q).permute(1, 0, 2), kk, vv,
                                         is_causal=True)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)


def test_window_or_sink_covering_sequence_equals_full():
    L, hq, hkv, d = 40, 2, 1, 8
    q = rng.standard_normal((L, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    full, lf = oracle.attn(q, k, v, [0, L], hq, hkv, [[0, 0]], 4, 8)
    for sink, window in [(0, L), (3, L + 5), (L, 1), (L + 3, 2)]:
        sp, ls = oracle.attn(q, k, v, [0, L], hq, hkv, [[1, 1]], sink, window)
        assert np.array_equal(sp, full) and np.array_equal(ls, lf)


def test_window_one_no_sink_returns_own_value():
    L, hq, hkv, d = 33, 4, 2, 8
    q = rng.standard_normal((L, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    o, lse = oracle.attn(q, k, v, [0, L], hq, hkv, [[1, 1, 1, 1]], 0, 1, 0.5)
    for h in range(hq):
        assert np.array_equal(o[:, h], v[:, h // 2])
        np.testing.assert_allclose(lse[:, h], 0.5 * np.einsum("td,td->t", q[:, h], k[:, h // 2]),
                                   atol=1e-13)


def test_constant_values_and_zero_queries():
    lens = [30, 17]
    cu = np.cumsum([0] + lens)
    T, hq, hkv, d = cu[-1], 4, 2, 8
    sink, window = 2, 5
    route = [[0, 1, 1, 0], [1, 1, 0, 0]]
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (T, hkv, d)).copy()
    o, _ = oracle.attn(q, k, v, cu, hq, hkv, route, sink, window)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-14, rtol=0)
    # Q = 0: every visible key gets the same weight, so o_i is the mean of the visible
    # values; the visible set is enumerated from ranges: [0, min(s, i+1)) and
    # [max(0, i-W+1), i] for sparse heads, [0, i] for full heads.
    v = rng.standard_normal((T, hkv, d))
    o, lse = oracle.attn(np.zeros_like(q), k, v, cu, hq, hkv, route, sink, window)
    for b in range(2):
        for h in range(hq):
            for i in range(lens[b]):
                if route[b][h]:
                    js = set(range(0, min(sink, i + 1))) | set(range(max(0, i - window + 1), i + 1))
                else:
                    js = set(range(0, i + 1))
                js = sorted(js)
                ref = v[cu[b] + np.array(js), h // 2].mean(axis=0)
                np.testing.assert_allclose(o[cu[b] + i, h], ref, atol=1e-14, rtol=0)
                assert abs(lse[cu[b] + i, h] - math.log(len(js))) < 1e-14


def test_gqa_invariants_and_packing():
    lens = [23, 41]
    cu = np.cumsum([0] + lens)
    T, hq, hkv, d = cu[-1], 8, 2, 8
    q = rng.standard_normal((T, hq, d))
    q[:, 1] = q[:, 0]  # heads 0, 1 share KV head 0
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    route = np.array([[1, 1, 0, 1, 0, 0, 1, 0], [0, 0, 1, 1, 1, 0, 0, 1]], dtype=np.uint8)
    sink, window = 3, 6
    o, lse = oracle.attn(q, k, v, cu, hq, hkv, route, sink, window)
    assert np.array_equal(o[:, 0], o[:, 1])
    # expanding K/V to one KV head per query head (MHA) gives the same result
    ke, ve = np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1)
    oe, lsee = oracle.attn(q, ke, ve, cu, hq, hq, route, sink, window)
    assert np.array_equal(o, oe) and np.array_equal(lse, lsee)
    # the packed batch equals separate single-sequence calls
    for b in range(2):
        s0, s1 = cu[b], cu[b + 1]
        ob, lb = oracle.attn(q[s0:s1], k[s0:s1], v[s0:s1], [0, lens[b]], hq, hkv,
                             route[b:b + 1], sink, window)
        assert np.array_equal(o[s0:s1], ob) and np.array_equal(lse[s0:s1], lb)
    # a subset of rows equals the same rows of the full evaluation
    rows = np.array([0, 5, 22, 23, 40, 63])
    os_, ls_ = oracle.attn(q, k, v, cu, hq, hkv, route, sink, window, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls_, lse[rows])


def test_bf16_and_fp32_inputs_decode_exactly():
    L, hq, hkv, d = 20, 2, 1, 16
    qb = torch.randn(L, hq, d).to(torch.bfloat16)
    kb = torch.randn(L, hkv, d).to(torch.bfloat16)
    vb = torch.randn(L, hkv, d).to(torch.bfloat16)
    a = oracle.attn(qb, kb, vb, [0, L], hq, hkv, [[0, 1]], 2, 4)
    b = oracle.attn(qb.double(), kb.double(), vb.double(), [0, L], hq, hkv, [[0, 1]], 2, 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = oracle.attn(qb.float(), kb.float(), vb.float(), [0, L], hq, hkv, [[0, 1]], 2, 4)
    assert np.array_equal(a[0], c[0])


def test_oracle_rejects_bad_arguments():
    q = np.zeros((4, 3, 8))
    k = np.zeros((4, 2, 8))
    with pytest.raises(ValueError):
        oracle.attn(q, k, k, [0, 4], 3, 2, [[0, 0, 0]], 0, 1)  # 3 % 2 != 0
    with pytest.raises(ValueError):
        oracle.attn(q, np.zeros((4, 1, 8)), np.zeros((4, 1, 8)), [0, 4], 3, 1, [[0, 0, 0]], 0, 0)


# ---------------------------------------------------------------- router


def test_router_hand_derived_fixture():
    with open(os.path.join(GOLDEN, "router_tiny.json")) as f:
        g = json.load(f)
    ks = np.array(g["key_states"], dtype=np.float32)
    pooled, logits, r = oracle.route(ks, g["cu_seqlens"], g["w1"], g["b1"], g["w2"], g["b2"])
    np.testing.assert_allclose(pooled, np.array(g["pooled"], dtype=np.float64), atol=0)
    t = g["tanh1"]
    want = np.array([[a * t + c for a, c in row] for row in g["logits_in_tanh1"]])
    np.testing.assert_allclose(logits, want, atol=1e-15, rtol=0)
    assert r.tolist() == g["route"]


def test_router_against_torch_layers_and_mean():
    lens = [5, 0, 19, 8]
    cu = np.cumsum([0] + lens)
    C, H, Hq = 12, 7, 5
    ks = torch.randn(int(cu[-1]), C).to(torch.bfloat16)
    w1 = torch.randn(H, C) * 0.3
    b1 = torch.randn(H) * 0.1
    w2 = torch.randn(Hq, H) * 0.3
    b2 = torch.randn(Hq) * 0.1
    pooled, logits, r = oracle.route(ks, cu, w1, b1, w2, b2)
    for b in range(len(lens)):
        seg = ks[cu[b]:cu[b + 1]].double()
        mean = seg.mean(dim=0) if lens[b] else torch.zeros(C, dtype=torch.float64)
        np.testing.assert_allclose(pooled[b], mean.numpy(), atol=1e-15)
        z = F.linear(F.silu(F.linear(mean, w1.double(), b1.double())), w2.double(), b2.double())
        np.testing.assert_allclose(logits[b], z.numpy(), atol=1e-14, rtol=0)
        assert r[b].tolist() == [int(x > 0) for x in z.tolist()]


def test_router_tie_routes_full_and_linearity():
    ks = np.random.default_rng(5).standard_normal((9, 4))
    w1, b1 = np.ones((3, 4), np.float32), np.zeros(3, np.float32)
    w2, b2 = np.zeros((2, 3), np.float32), np.zeros(2, np.float32)
    _, logits, r = oracle.route(ks, [0, 9], w1, b1, w2, b2)
    assert np.all(logits == 0) and np.all(r == 0)  # z == 0 -> full attention
    a, b = 0.75, -2.0
    ks2 = np.random.default_rng(6).standard_normal((9, 4))
    p1, _, _ = oracle.route(ks, [0, 4, 9], w1, b1, w2, b2)
    p2, _, _ = oracle.route(ks2, [0, 4, 9], w1, b1, w2, b2)
    p3, _, _ = oracle.route(a * ks + b * ks2, [0, 4, 9], w1, b1, w2, b2)
    np.testing.assert_allclose(p3, a * p1 + b * p2, atol=1e-14)


def test_router_parameter_count_matches_pages():
    # 8B-scale layer: 8 KV heads x 128 = 1024 key features, hidden 256, 32 query heads.
    w = inputs.WORKLOADS["qwen3_8b_32k"]
    w1, b1, w2, b2 = inputs.router_weights(w)
    n = sum(x.numel() for x in (w1, b1, w2, b2))
    assert n == 270624
    assert round(n / 1e6, 2) == 0.27


def test_router_bias_fixture_reproduces_ratio():
    with open(os.path.join(GOLDEN, "router_bias_qwen3_8b_32k.json")) as f:
        g = json.load(f)
    assert g["n_sparse"] == 27 and g["decision_margin"] >= 1e-7
    assert abs(g["n_sparse"] / 32 - 0.85) < 0.01


# ---------------------------------------------------------------- work list


def brute_costs(L, sparse, sink, window, bm, bn):
    m = lib_mask(L, sparse, sink, window).numpy()
    nq, nk = -(-L // bm), -(-L // bn)
    return [sum(bool(m[qt * bm:(qt + 1) * bm, kt * bn:(kt + 1) * bn].any()) for kt in range(nk))
            for qt in range(nq)]


@pytest.mark.parametrize("L,sink,window,bm,bn", [(1, 0, 1, 4, 4), (37, 3, 5, 8, 4),
                                                 (64, 0, 16, 16, 16), (100, 20, 7, 16, 8),
                                                 (130, 5, 200, 32, 16), (77, 9, 30, 8, 16)])
def test_worklist_costs_bruteforce(L, sink, window, bm, bn):
    route = [[0, 1, 1]]
    items = oracle.worklist(route, [0, L], 3, sink, window, bm, bn)
    got = {(int(s), int(h), int(q)): int(c) for s, h, q, c in items}
    for h in range(3):
        for qt, c in enumerate(brute_costs(L, route[0][h], sink, window, bm, bn)):
            assert got[(0, h, qt)] == c


def test_worklist_order_and_coverage():
    lens = [300, 0, 129, 1000]
    cu = np.cumsum([0] + lens)
    hq = 6
    route = np.random.default_rng(7).integers(0, 2, size=(4, hq))
    items = oracle.worklist(route, cu, hq, 16, 100, 64, 32)
    keys = [(int(s), int(h), int(q)) for s, h, q, _ in items]
    want = {(b, h, q) for b in range(4) for h in range(hq) for q in range(-(-lens[b] // 64))}
    assert len(keys) == len(set(keys)) and set(keys) == want
    order = [(-int(c), int(s), int(q), int(h)) for s, h, q, c in items]
    assert order == sorted(order)


def test_worklist_closed_forms():
    bm = bn = 128
    L = 32768
    items = oracle.worklist([[0, 1]], [0, L], 2, 128, 2048, bm, bn)
    for s, h, q, c in items:
        if h == 0:
            assert c == (q + 1) * bm // bn
        elif q * bm >= 2048 + 128:  # sink and window no longer touch
            assert c == -(-128 // bn) + 2048 // bn + bm // bn == 18
    items = oracle.worklist([[0, 1]], [0, L], 2, 128, 2048, 128, 64)
    for s, h, q, c in items:
        if h == 0:
            assert c == (q + 1) * 2
        elif q * 128 >= 2048 + 128:
            assert c == 2 + 32 + 2


# ---------------------------------------------------------------- counts


@pytest.mark.parametrize("L,sink,window", [(1, 0, 1), (10, 3, 4), (50, 0, 7), (64, 64, 1),
                                           (33, 5, 40), (200, 17, 31)])
def test_visible_pair_closed_form(L, sink, window):
    for sparse in (False, True):
        assert metrics.visible_pairs(L, sparse, sink, window) == int(
            lib_mask(L, sparse, sink, window).sum())


@pytest.mark.parametrize("L,sink,window", [(1, 0, 1), (10, 3, 4), (50, 0, 7), (64, 64, 1),
                                           (33, 5, 40), (200, 17, 31), (300, 300, 5)])
def test_decode_group_keys_is_union_of_last_rows(L, sink, window):
    """Rows a group reads = keys visible to the last query row under any head of the group."""
    full_last = lib_mask(L, False, sink, window)[L - 1]
    sparse_last = lib_mask(L, True, sink, window)[L - 1]
    assert metrics.decode_group_keys(L, True, sink, window) == int(sparse_last.sum())
    assert metrics.decode_group_keys(L, False, sink, window) == int((full_last | sparse_last).sum())
    lens, route = [L, 3], [[1, 1, 0, 1], [1, 1, 1, 1]]
    want = 2 * 8 * 2 * (int(sparse_last.sum()) + L
                        + metrics.decode_group_keys(3, True, sink, window) * 2) + 2 * 2 * 4 * 8 * 2
    assert metrics.decode_bytes(lens, route, 2, 8, sink, window, 2) == want


# ---- decode step (one new query per sequence over its KV cache) ----

def make_cache(lens, cap, hq, hkv, d, seed, poison=True):
    """Per-sequence caches [B, cap, Hkv, D] with the slots past each length filled with NaN
    (they must never be read), plus the query of each sequence's newest token."""
    g = np.random.default_rng(seed)
    B = len(lens)
    kc = g.standard_normal((B, cap, hkv, d))
    vc = g.standard_normal((B, cap, hkv, d))
    if poison:
        for b, L in enumerate(lens):
            kc[b, L:] = np.nan
            vc[b, L:] = np.nan
    q = g.standard_normal((B, hq, d))
    return q, kc, vc


@pytest.mark.parametrize("L,sink,window", [(1, 0, 1), (2, 1, 1), (7, 2, 3), (9, 0, 4),
                                           (12, 4, 20), (10, 12, 2), (13, 3, 13)])
def test_decode_tiny_bruteforce(L, sink, window):
    """The decode output of a cache holding L tokens is the last row of the brute-force
    prefill of those L tokens (pair-loop mask, dense softmax)."""
    d, hq, hkv, cap = 5, 4, 2, L + 3
    q, kc, vc = make_cache([L], cap, hq, hkv, d, seed=L * 31 + sink)
    route = [[1, 0, 0, 1]]
    scale = 0.41
    o, lse = oracle.decode(q, kc, vc, [L], hkv, route, sink, window, scale)
    for h in range(hq):
        kk, vv = kc[0, :L, h // 2], vc[0, :L, h // 2]
        qq = np.zeros((L, d))
        qq[L - 1] = q[0, h]
        ref = dense_bruteforce(qq, kk, vv, L, route[0][h], sink, window, scale)[L - 1]
        np.testing.assert_allclose(o[0, h], ref, atol=1e-12, rtol=0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_decode_matches_sdpa_last_row_ragged_gqa():
    """Library routine: torch SDPA (fp64) of the whole sequence under the library-built
    mask, last row, for a ragged batch with GQA 4:1 and mixed routing."""
    lens, cap, hq, hkv, d = [1, 37, 130, 64, 200], 211, 8, 2, 16
    q, kc, vc = make_cache(lens, cap, hq, hkv, d, seed=77)
    route = np.array([[(b + h) % 3 == 0 for h in range(hq)] for b in range(len(lens))],
                     dtype=np.uint8)
    sink, window, scale = 5, 40, 0.23
    o, lse = oracle.decode(q, kc, vc, lens, hkv, route, sink, window, scale)
    G = hq // hkv
    for b, L in enumerate(lens):
        for h in range(hq):
            m = lib_mask(L, bool(route[b, h]), sink, window)[L - 1:L]
            qq = torch.as_tensor(q[b, h][None], dtype=torch.float64)
            kk = torch.as_tensor(kc[b, :L, h // G], dtype=torch.float64)
            vv = torch.as_tensor(vc[b, :L, h // G], dtype=torch.float64)
            ref = F.scaled_dot_product_attention(qq[None], kk[None], vv[None],
                                                 attn_mask=m[None], scale=scale)[0, 0]
            np.testing.assert_allclose(o[b, h], ref.numpy(), atol=1e-12, rtol=0)
            sc = (qq @ kk.T * scale).masked_fill(~m, -math.inf).numpy()
            assert abs(lse[b, h] - logsumexp(sc[0])) < 1e-12


def test_decode_special_cases():
    d, hq, hkv, cap = 6, 2, 1, 20
    # one cached token: the output is that token's value, lse = scale * q.k0
    q, kc, vc = make_cache([1], cap, hq, hkv, d, seed=5)
    o, lse = oracle.decode(q, kc, vc, [1], hkv, [[0, 1]], 0, 1, 0.5)
    for h in range(hq):
        np.testing.assert_array_equal(o[0, h], vc[0, 0, 0])
        assert abs(lse[0, h] - 0.5 * float(q[0, h] @ kc[0, 0, 0])) < 1e-12
    # a window (or sink) covering the cache makes a sparse head equal to a full head
    q, kc, vc = make_cache([17], cap, hq, hkv, d, seed=6)
    full, _ = oracle.decode(q, kc, vc, [17], hkv, [[0, 0]], 0, 1, 0.3)
    for sink, window in [(0, 17), (17, 1), (3, 40)]:
        sp, _ = oracle.decode(q, kc, vc, [17], hkv, [[1, 1]], sink, window, 0.3)
        np.testing.assert_array_equal(sp, full)
    # constant values give that constant whatever the scores
    vc2 = np.where(np.isnan(vc), np.nan, 2.5)
    o, _ = oracle.decode(q, kc, vc2, [17], hkv, [[0, 1]], 2, 5, 0.3)
    np.testing.assert_allclose(o, 2.5, atol=1e-14, rtol=0)
    # sink 1, window 1: exactly key 0 and the newest key
    o, _ = oracle.decode(q, kc, vc, [17], hkv, [[1, 1]], 1, 1, 0.3)
    for h in range(hq):
        x0, x1 = 0.3 * q[0, h] @ kc[0, 0, 0], 0.3 * q[0, h] @ kc[0, 16, 0]
        w0 = 1.0 / (1.0 + math.exp(x1 - x0))
        np.testing.assert_allclose(o[0, h], w0 * vc[0, 0, 0] + (1 - w0) * vc[0, 16, 0],
                                   atol=1e-12, rtol=0)


def test_decode_rejects_bad_arguments():
    q, kc, vc = make_cache([3], 4, 2, 1, 4, seed=9, poison=False)
    for lens in ([0], [5]):
        with pytest.raises(ValueError):
            oracle.decode(q, kc, vc, lens, 1, [[0, 0]], 0, 2)
    with pytest.raises(ValueError):
        oracle.decode(q, kc, vc, [3], 1, [[0, 0]], 0, 0)


# ---- chunked prefill over a KV prefix (each sequence's Lq queries are its last Lq of Lk
# positions; keys and values packed separately)

def chunk_case(lens_k, lens_q, hq, hkv, d, seed):
    """Full-sequence q/k/v per sequence; the chunk's queries are the last Lq positions."""
    g = np.random.default_rng(seed)
    cu_k = np.cumsum([0] + list(lens_k)).astype(np.int32)
    cu_q = np.cumsum([0] + list(lens_q)).astype(np.int32)
    qfull = g.standard_normal((int(cu_k[-1]), hq, d))
    k = g.standard_normal((int(cu_k[-1]), hkv, d))
    v = g.standard_normal((int(cu_k[-1]), hkv, d))
    q = np.concatenate([qfull[cu_k[b + 1] - lq:cu_k[b + 1]] for b, lq in enumerate(lens_q)])
    return qfull, q, k, v, cu_q, cu_k


def test_chunked_matches_sdpa_last_rows():
    """Chunk rows = the last Lq rows of torch SDPA over the whole sequence (library masks),
    ragged GQA batch, mixed routing, chunks from 1 row to the whole sequence."""
    lens_k, lens_q = [40, 97, 130, 64], [40, 13, 1, 33]
    hq, hkv, d, sink, window = 4, 2, 16, 3, 20
    qfull, q, k, v, cu_q, cu_k = chunk_case(lens_k, lens_q, hq, hkv, d, 5)
    route = np.array([[0, 1, 1, 0], [1, 1, 1, 1], [1, 0, 1, 1], [0, 0, 1, 1]], np.uint8)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attn(q, k, v, cu_q, hq, hkv, route, sink, window, cu_seqlens_k=cu_k)
    ro, rl = sdpa_reference(qfull, k, v, cu_k, route, sink, window, scale)
    for b in range(4):
        want = slice(int(cu_k[b + 1]) - lens_q[b], int(cu_k[b + 1]))
        got = slice(int(cu_q[b]), int(cu_q[b + 1]))
        assert np.abs(o[got] - ro[want]).max() < 1e-12
        assert np.abs(lse[got] - rl[want]).max() < 1e-12


def test_chunked_single_row_is_decode():
    """A one-row chunk is a decode step over the same history."""
    lens_k = [1, 50, 300]
    hq, hkv, d, sink, window = 4, 2, 32, 4, 64
    _, q, k, v, cu_q, cu_k = chunk_case(lens_k, [1, 1, 1], hq, hkv, d, 9)
    route = np.array([[1, 1, 0, 1], [1, 1, 1, 1], [0, 1, 1, 1]], np.uint8)
    o, lse = oracle.attn(q, k, v, cu_q, hq, hkv, route, sink, window, cu_seqlens_k=cu_k)
    cap = max(lens_k)
    kc = np.zeros((3, cap, hkv, d))
    vc = np.zeros((3, cap, hkv, d))
    for b, L in enumerate(lens_k):
        kc[b, :L] = k[cu_k[b]:cu_k[b + 1]]
        vc[b, :L] = v[cu_k[b]:cu_k[b + 1]]
    od, ld = oracle.decode(q, kc, vc, lens_k, hkv, route, sink, window)
    assert np.abs(o - od).max() < 1e-12 and np.abs(lse - ld).max() < 1e-12


def test_chunks_compose_to_the_prefill():
    """Cutting a sequence into chunks (each over its full prefix) gives the prefill's rows."""
    L, hq, hkv, d, sink, window = 150, 2, 1, 16, 5, 30
    qfull, _, k, v, _, _ = chunk_case([L], [L], hq, hkv, d, 21)
    route = np.array([[0, 1]], np.uint8)
    full, _ = oracle.attn(qfull, k, v, [0, L], hq, hkv, route, sink, window)
    at = 0
    for c in (1, 63, 64, 22):
        o, _ = oracle.attn(qfull[at:at + c], k[:at + c], v[:at + c], [0, c], hq, hkv, route,
                           sink, window, cu_seqlens_k=[0, at + c])
        assert np.abs(o - full[at:at + c]).max() < 1e-12
        at += c
    assert at == L


@pytest.mark.parametrize("lk,lq,sink,window,bm,bn", [(300, 300, 5, 40, 64, 32),
                                                    (300, 77, 5, 40, 64, 32),
                                                    (1000, 1, 16, 100, 256, 64),
                                                    (2500, 600, 128, 2048, 256, 64)])
def test_chunked_worklist_costs_bruteforce(lk, lq, sink, window, bm, bn):
    """Costs of chunk q-tiles = key tiles with a visible pair for the tile's rows, counted
    by brute force on the library mask's rows Lk - Lq + [m0, m1)."""
    route = [[0, 1]]
    items = oracle.worklist(route, [0, lq], 2, sink, window, bm, bn, cu_seqlens_k=[0, lk])
    got = {(int(h), int(q)): int(c) for s, h, q, c in items}
    assert len(got) == 2 * -(-lq // bm)
    off = lk - lq
    for h in range(2):
        m = lib_mask(lk, bool(route[0][h]), sink, window)
        for qt in range(-(-lq // bm)):
            rows = m[off + qt * bm:off + min((qt + 1) * bm, lq)]
            want = sum(bool(rows[:, t * bn:(t + 1) * bn].any()) for t in range(-(-lk // bn)))
            assert got[(h, qt)] == want


def test_chunked_rejects_short_key_sequences():
    _, q, k, v, cu_q, _ = chunk_case([10], [10], 2, 1, 8, 1)
    with pytest.raises(ValueError):
        oracle.attn(q, k, v, cu_q, 2, 1, [[0, 1]], 2, 4, cu_seqlens_k=[0, 9])
    with pytest.raises(ValueError):
        oracle.worklist([[0, 1]], [0, 10], 2, 2, 4, 64, 32, cu_seqlens_k=[0, 9])


@pytest.mark.parametrize("lk,lq,sink,window", [(100, 100, 3, 20), (100, 1, 3, 20), (257, 60, 0, 7),
                                               (64, 30, 64, 1)])
def test_chunk_flops_closed_form(lk, lq, sink, window):
    """Pairs of the chunk rows = the library mask's rows Lk - Lq .. Lk - 1."""
    for sparse in (0, 1):
        want = int(lib_mask(lk, bool(sparse), sink, window)[lk - lq:].sum())
        assert metrics.chunk_flops([lk], [lq], [[sparse]], 1, sink, window) == 4 * want


# ---- training side: attention backward and the router's straight-through gradient
# (blog post section 2.1, "training trick": Gumbel-Softmax + straight-through estimator)

def autograd_attention(q, k, v, dout, cu, route, sink, window, scale):
    """torch autograd in fp64 over SDPA-free explicit attention with library-built masks."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    loss = 0.0
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        L = s1 - s0
        for h in range(hq):
            m = lib_mask(L, bool(route[b][h]), sink, window)
            sc = (qt[s0:s1, h] @ kt[s0:s1, h // G].T) * scale
            p = torch.softmax(sc.masked_fill(~m, -math.inf), dim=-1)
            o = p @ vt[s0:s1, h // G]
            loss = loss + (o * torch.tensor(dout[s0:s1, h])).sum()
    loss.backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_attn_backward_matches_autograd():
    lens, hq, hkv, d, sink, window = [37, 1, 60], 4, 2, 8, 3, 10
    cu = np.cumsum([0] + lens)
    g = np.random.default_rng(41)
    q = g.standard_normal((cu[-1], hq, d))
    k = g.standard_normal((cu[-1], hkv, d))
    v = g.standard_normal((cu[-1], hkv, d))
    do = g.standard_normal((cu[-1], hq, d))
    route = np.array([[0, 1, 1, 0], [1, 0, 1, 1], [1, 1, 0, 1]], np.uint8)
    dq, dk, dv = oracle.attn_backward(q, k, v, do, cu, hq, hkv, route, sink, window)
    rq, rk, rv = autograd_attention(q, k, v, do, cu, route, sink, window, 1 / math.sqrt(d))
    assert np.abs(dq - rq).max() < 1e-10
    assert np.abs(dk - rk).max() < 1e-10
    assert np.abs(dv - rv).max() < 1e-10


def test_attn_backward_chunked_matches_full_prefill_rows():
    """With a KV prefix, the chunk rows' dq equal the full prefill's dq of those rows when the
    earlier rows carry no output gradient; dk, dv then equal the full prefill's too."""
    L, lq, hq, hkv, d = 50, 17, 2, 1, 8
    g = np.random.default_rng(5)
    q = g.standard_normal((L, hq, d))
    k = g.standard_normal((L, hkv, d))
    v = g.standard_normal((L, hkv, d))
    do = g.standard_normal((L, hq, d))
    do[:L - lq] = 0.0
    route = np.array([[0, 1]], np.uint8)
    fq, fk, fv = oracle.attn_backward(q, k, v, do, [0, L], hq, hkv, route, 4, 9)
    cq, ck, cv = oracle.attn_backward(q[L - lq:], k, v, do[L - lq:], [0, lq], hq, hkv, route, 4, 9,
                                      cu_seqlens_k=[0, L])
    assert np.abs(cq - fq[L - lq:]).max() < 1e-12
    assert np.abs(ck - fk).max() < 1e-12 and np.abs(cv - fv).max() < 1e-12


def test_attn_backward_window_one_is_identity_path():
    """s = 0, W = 1: o_i = v_i, so dv = dO (per KV head, summed over its heads), dq = dk = 0."""
    T, hq, hkv, d = 12, 2, 1, 4
    g = np.random.default_rng(2)
    q, k, v = (g.standard_normal((T, h, d)) for h in (hq, hkv, hkv))
    do = g.standard_normal((T, hq, d))
    dq, dk, dv = oracle.attn_backward(q, k, v, do, [0, T], hq, hkv, [[1, 1]], 0, 1)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
    assert np.abs(dv[:, 0] - do.sum(axis=1)).max() < 1e-12


def test_route_backward_matches_autograd_straight_through():
    """The straight-through construction r = r_hard + r_soft - stop_gradient(r_soft) with
    r_soft = sigmoid((z + g) / tau), output r O_sparse + (1 - r) O_full, router MLP and mean
    pool, differentiated by torch autograd in fp64."""
    lens, C, Hd, hq, d, tau = [5, 0, 9], 12, 6, 4, 3, 0.7
    cu = np.cumsum([0] + lens)
    gen = np.random.default_rng(8)
    ks = gen.standard_normal((cu[-1], C))
    w1, b1 = gen.standard_normal((Hd, C)) * 0.5, gen.standard_normal(Hd) * 0.1
    w2, b2 = gen.standard_normal((hq, Hd)) * 0.5, gen.standard_normal(hq) * 0.1
    of, osp, do = (gen.standard_normal((cu[-1], hq, d)) for _ in range(3))
    noise = gen.logistic(size=(3, hq))
    got = oracle.route_backward(ks, cu, w1, b1, w2, b2, of, osp, do, tau=tau, noise=noise)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    kst, w1t, b1t, w2t, b2t = T(ks), T(w1), T(b1), T(w2), T(b2)
    xs = []
    for b in range(3):
        seg = kst[cu[b]:cu[b + 1]]
        xs.append(seg.mean(dim=0) if lens[b] else torch.zeros(C, dtype=torch.float64))
    xbar = torch.stack(xs)
    z = F.linear(F.silu(F.linear(xbar, w1t, b1t)), w2t, b2t)
    z.retain_grad()
    r_soft = torch.sigmoid((z + torch.tensor(noise)) / tau)
    r = (r_soft > 0.5).double() + r_soft - r_soft.detach()
    loss = 0.0
    for b in range(3):
        s = slice(cu[b], cu[b + 1])
        o = r[b][None, :, None] * torch.tensor(osp[s]) + (1 - r[b])[None, :, None] * torch.tensor(of[s])
        loss = loss + (o * torch.tensor(do[s])).sum()
    loss.backward()
    for name, ref in (("dz", z.grad), ("dw1", w1t.grad), ("db1", b1t.grad), ("dw2", w2t.grad),
                      ("db2", b2t.grad), ("dkey_states", kst.grad)):
        assert np.abs(got[name] - ref.numpy()).max() < 1e-12, name
    assert np.abs(got["dz"][1]).max() == 0  # the empty sequence: no rows, no routing gradient
