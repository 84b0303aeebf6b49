"""Benchmark of the routed hybrid-attention prefill layer on one MI355X.

One step = the whole hot path of one layer on resident inputs:
  ea_route (mean-pool + router MLP + threshold) -> ea_hybrid_attn_prefill (work-list
  planner + persistent fused attention), for the Qwen3-8B-shaped layer at 32K tokens
  (32 query / 8 KV heads, head_dim 128, bf16, sink 128, window 2048, 27 of 32 heads sparse
  by the router).

Prints ONE JSON line: effective TFLOP/s (only unmasked score positions count, 4*D FLOPs
each), ms per layer, % of the bf16 dense MFMA peak, the roofline of the attention kernel
(timed with HIP events on the launch stream) and the fp64 oracle's throughput on a bounded
sample of the same workload on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cpu-seconds S]

With --mode decode it instead times one decode step of the same routed attention
(ea_hybrid_attn_decode: every sequence's newest token against its KV cache) on 16 sequences
of 32K cached tokens, priced against HBM bandwidth: the bytes are the K and V cache rows each
KV-head group must see (all rows if any of its query heads is full, else sink and window),
plus q and o.  --mode decode_pool times the same step over the pooled cache (KV heads whose
query heads are all sparse keep only a sink + ring buffer of sink + window rows) and reports
its size next to the dense cache's.  --mode prefill_chunk times the router plus a chunked
prefill of the layer's last 4096 tokens over the other 28672 as a KV prefix.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from full_attention_long_amd import ea, inputs, metrics  # noqa: E402

METRIC = "hybrid-attn prefill ms/layer + effective TFLOP/s (% bf16 MFMA peak), {}"
WORKLOAD_LABEL = {"qwen3_8b_32k": "32K", "llama8b_8k": "8K (Llama-3.1-8B-shaped)",
                  "ragged4": "ragged 4-sequence batch", "long_256k": "256K",
                  "tiny_fp32": "tiny fp32"}
CHUNK_METRIC = "hybrid-attn chunked prefill (4K chunk over a 28K prefix) effective TFLOP/s"
BACKWARD_METRIC = "hybrid-attn training backward (router STE + dq/dk/dv) effective TFLOP/s"
DECODE_METRIC = "hybrid-attn decode step: cache GB/s (% HBM peak), 16 x 32K"
DECODE_POOL_METRIC = "hybrid-attn decode step, pooled sink+ring cache: cache GB/s (% HBM peak), 16 x 32K"
GOLDEN_BIAS = os.path.join(ROOT, "tests", "golden", "router_bias_qwen3_8b_32k.json")
ATTN_SOURCE = os.path.join(ROOT, "full_attention_long_amd", "csrc", "ea_attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_qwen3_8b_32k_traffic.json")
DECODE_SOURCE = os.path.join(ROOT, "full_attention_long_amd", "csrc", "ea_decode.hip")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_bf16_qwen3_8b_32k_traffic.json")
DECODE_POOL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_pool_bf16_qwen3_8b_32k_traffic.json")
CHUNK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_chunked_qwen3_8b_32k_chunk4096_traffic.json")
BWD_SOURCE = os.path.join(ROOT, "full_attention_long_amd", "csrc", "ea_backward_bf16.hip")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_backward_qwen3_8b_32k_traffic.json")


def source_sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload, traffic_file=TRAFFIC_FILE, source=ATTN_SOURCE):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by what they read for a plain 1 GiB copy), or None
    if there is none for this workload or the kernel source changed since the counters
    were taken."""
    if not os.path.exists(traffic_file):
        return None
    with open(traffic_file) as f:
        t = json.load(f)
    if t.get("workload") != workload or t.get("kernel_source_sha256") != source_sha256(source):
        return None
    kib = t["fetch_kib_per_dispatch"] * t["fetch_scale"] + t["write_kib_per_dispatch"] * t["write_scale"]
    return int(round(kib * 1024))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Layer:
    """Resident device buffers of one synthetic layer."""

    def __init__(self, name: str):
        w = inputs.WORKLOADS[name]
        self.w = w
        self.lens = inputs.lengths(w)
        T = sum(self.lens)
        self.T = T
        dev = torch.device("cuda:0")
        q, k, v = inputs.qkv(w, T)
        self.cpu = (q, k, v)
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        self.o = torch.empty_like(self.q)
        self.cu_host = inputs.cu_seqlens(self.lens)
        self.cu = self.cu_host.to(dev)
        self.max_len = max(self.lens)
        B, hq = len(self.lens), w.n_heads_q
        self.route = torch.empty(B, hq, dtype=torch.uint8, device=dev)
        if w.router:
            w1, b1, w2, b2 = inputs.router_weights(w)
            with open(GOLDEN_BIAS) as f:
                b2 = torch.full_like(b2, json.load(f)["b2"])
            self.router = [t.to(dev) for t in (w1, b1, w2, b2)]
            self.ks = self.k.view(T, w.n_heads_kv * w.head_dim)
            kv_dim, hidden = self.ks.shape[1], w1.shape[0]
        else:
            self.router = None
            self.route.copy_(inputs.bernoulli_route(w, B))
            kv_dim = hidden = 0
        self.ws = torch.empty(ea.workspace_size(B, self.max_len, hq, kv_dim, hidden),
                              dtype=torch.uint8, device=dev)
        bm, _ = ea.tile_config(ea.EA_BF16, w.head_dim)
        self.wl = torch.empty(B * hq * -(-self.max_len // bm), 4, dtype=torch.int32, device=dev)
        self.n_items = torch.empty(1, dtype=torch.int32, device=dev)

    def do_route(self):
        if self.router is not None:
            w1, b1, w2, b2 = self.router
            ea.route(self.ks, self.cu, w1, b1, w2, b2, self.route, self.ws)

    def do_plan(self):
        w = self.w
        ea.build_worklist(self.route, self.cu, self.max_len, w.n_heads_q, w.sink, w.window,
                          ea.EA_BF16, w.head_dim, self.wl, self.ws, n_items_out=self.n_items,
                          want_count=False)

    def do_attn(self):
        w = self.w
        ea.hybrid_attn_run(self.q, self.k, self.v, self.o, self.cu, self.max_len, self.route,
                           w.sink, w.window, self.wl, self.n_items, self.ws)

    def step(self):
        """One layer: router, then the fused prefill (planner + attention)."""
        w = self.w
        self.do_route()
        ea.hybrid_attn_prefill(self.q, self.k, self.v, self.o, self.cu, self.max_len,
                               self.route, w.sink, w.window, self.ws)

    def flops(self):
        r = self.route.cpu().tolist()
        return metrics.effective_flops(self.lens, r, self.w.head_dim, self.w.sink, self.w.window)


def copy_calibration():
    """One elementwise kernel that reads 1 GiB and writes 1 GiB: a known-size launch for
    scaling rocprofv3's FETCH_SIZE / WRITE_SIZE."""
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def settle(fn, seconds):
    """Run fn until `seconds` of wall time have passed (at least once): untimed work before
    the warm-up steps that brings the shader clock to its loaded steady state (the first
    launches of a fresh process run up to 25% slower while it ramps).  Returns the count."""
    n, t0 = 0, time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()
        n += 1
    return n


def time_events_evict(fn, n, scratch):
    """Average ms of fn() over n calls, each timed alone with HIP events after a write of
    the whole `scratch` buffer (512 MiB: the 256 MiB MALL and the 8 x 4 MiB L2 hold none of
    the step's inputs when it starts); the write itself is not timed."""
    total = 0.0
    for _ in range(n):
        if scratch is not None:
            scratch.fill_(1.0)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        total += s.elapsed_time(e)
    return total / n


def time_events(fn, n):
    """Average ms of fn() over n calls, HIP events on the current (launch) stream."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / n


def cpu_baseline(layer: Layer, seconds: float):
    """fp64 oracle on sampled query rows of the same workload, all host cores."""
    import numpy as np
    import oracle
    w = layer.w
    q, k, v = layer.cpu
    route = layer.route.cpu().numpy()
    g = torch.Generator().manual_seed(inputs.seed(w.index, inputs.STREAM_ROWS) + 7)
    perm = torch.randperm(layer.T, generator=g).numpy()
    cu = layer.cu_host.numpy()
    done_rows, flops, t_used, at, batch = 0, 0, 0.0, 0, 8
    threads = oracle.max_threads()
    while t_used < seconds and at < layer.T:
        rows = np.sort(perm[at:at + batch])
        at += batch
        t0 = time.perf_counter()
        oracle.attn(q, k, v, cu, w.n_heads_q, w.n_heads_kv, route, w.sink, w.window, rows=rows)
        t_used += time.perf_counter() - t0
        for t in rows:
            b = int(np.searchsorted(cu, t, side="right") - 1)
            i = int(t - cu[b])
            for h in range(w.n_heads_q):
                if route[b, h]:
                    n_vis = min(i + 1, w.window) + max(0, min(w.sink, i - w.window + 1))
                else:
                    n_vis = i + 1
                flops += 4 * w.head_dim * n_vis
        done_rows += len(rows)
        batch = min(256, batch * 2)
    tflops = flops / t_used / 1e12
    full_layer_s = layer.flops() / (flops / t_used)
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done_rows} uniformly drawn query rows x {w.n_heads_q} heads of the "
                      f"same layer ({t_used:.1f} s of fp64 oracle work); full layer "
                      f"extrapolated to {full_layer_s:.0f} s"}


class DecodeStep:
    """Resident device buffers of one synthetic decode step."""

    def __init__(self, name: str):
        w = inputs.DECODE_WORKLOADS[name]
        self.w = w
        q, kc, vc, lens, route = inputs.decode_inputs(w)
        self.cpu = (q, kc, vc, route)
        self.lens = lens
        dev = torch.device("cuda:0")
        self.q, self.kc, self.vc = q.to(dev), kc.to(dev), vc.to(dev)
        self.o = torch.empty_like(self.q)
        self.sl = torch.tensor(lens, dtype=torch.int32, device=dev)
        self.route = route.to(dev)
        self.max_len = max(lens)
        self.ws = torch.empty(ea.decode_workspace_size(len(lens), self.max_len, w.n_heads_q,
                                                       w.head_dim), dtype=torch.uint8, device=dev)
        self.elt = q.element_size()
        self.bytes = metrics.decode_bytes(lens, route.tolist(), w.n_heads_kv, w.head_dim,
                                          w.sink, w.window, self.elt)

    def step(self):
        """One decode step: lengths only on the device, as in a serving loop."""
        w = self.w
        ea.hybrid_attn_decode(self.q, self.kc, self.vc, self.o, self.sl, self.max_len,
                              self.route, w.sink, w.window, self.ws)


class DecodePoolStep(DecodeStep):
    """The same step over a pooled cache: linear regions for KV heads with a full query
    head, sink + ring regions of sink + window rows for all-sparse ones, filled from the
    dense cache's contents."""

    def __init__(self, name: str):
        super().__init__(name)
        w = self.w
        dev = torch.device("cuda:0")
        route_cpu = self.cpu[3]
        base, rows, total = ea.decode_pool_layout(route_cpu.numpy(), w.n_heads_kv, w.capacity,
                                                  w.sink, w.window)
        self.pool_rows = total
        self.kp = torch.empty(total, w.head_dim, dtype=self.q.dtype, device=dev)
        self.vp = torch.empty_like(self.kp)
        self.rbase, self.rrows = base.to(dev), rows.to(dev)
        k = torch.cat([self.kc[b, :L] for b, L in enumerate(self.lens)])
        v = torch.cat([self.vc[b, :L] for b, L in enumerate(self.lens)])
        cu = inputs.cu_seqlens(self.lens).to(dev)
        ea.decode_pool_fill(k, v, cu, self.max_len, w.n_heads_q, self.route, w.sink, w.window,
                            self.rbase, self.rrows, self.kp, self.vp)
        torch.cuda.synchronize()
        del k, v
        self.dense_cache_bytes = 2 * self.kc.numel() * self.elt
        self.pool_bytes = 2 * self.kp.numel() * self.elt
        self.kc = self.vc = None  # the step reads only the pool
        torch.cuda.empty_cache()

    def step(self):
        w = self.w
        ea.hybrid_attn_decode_pool(self.q, self.kp, self.vp, self.o, self.sl, self.max_len,
                                   w.n_heads_kv, self.rbase, self.rrows, self.route, w.sink,
                                   w.window, self.ws)


def decode_cpu_baseline(st: DecodeStep, seconds: float):
    """fp64 oracle decode of whole sequences of the same batch, one at a time and cycling
    through the batch until `seconds` of work, all cores."""
    import oracle
    w = st.w
    q, kc, vc, route = st.cpu
    threads = oracle.max_threads()
    done, nbytes, t_used = 0, 0, 0.0
    while t_used < seconds:
        b = done % len(st.lens)
        t0 = time.perf_counter()
        oracle.decode(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], st.lens[b:b + 1], w.n_heads_kv,
                      route[b:b + 1].numpy(), w.sink, w.window)
        t_used += time.perf_counter() - t0
        nbytes += metrics.decode_bytes(st.lens[b:b + 1], route[b:b + 1].tolist(), w.n_heads_kv,
                                       w.head_dim, w.sink, w.window, st.elt)
        done += 1
    return {"value": round(nbytes / t_used / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} single-sequence decodes cycling through the {len(st.lens)} "
                      f"sequences of the same step ({t_used:.1f} s of fp64 oracle work)"}


def decode_main(args, pooled=False):
    st = DecodePoolStep(args.workload) if pooled else DecodeStep(args.workload)
    w = st.w
    log(f"decode workload {w.name}: B={len(st.lens)} lens={st.lens[:4]}... "
        f"sparse heads {int(st.route.sum().item())} of {st.route.numel()}")
    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_events(st.step, args.steps)
    torch.cuda.synchronize()
    log(f"timed {args.steps} steps: {ms:.4f} ms/step (wall {time.perf_counter() - t0:.3f} s)")
    gbps = st.bytes / (ms * 1e-3) / 1e9
    peak = metrics.MI355X_HBM_GBPS
    r = st.route.cpu()
    G = w.n_heads_q // w.n_heads_kv
    groups_sparse = int(r.view(len(st.lens), w.n_heads_kv, G).all(dim=2).sum().item())
    rec = {
        "metric": DECODE_POOL_METRIC if pooled else DECODE_METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if st.elt == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": len(st.lens), "cached_tokens": st.max_len,
                   "n_heads_q": w.n_heads_q, "n_heads_kv": w.n_heads_kv,
                   "head_dim": w.head_dim, "sink": w.sink, "window": w.window,
                   "sparse_heads": int(r.sum().item()), "all_sparse_kv_groups": groups_sparse,
                   "routing": f"bernoulli({w.p_sparse})",
                   "cache": "pooled sink+ring" if pooled else "dense [B, cap, Hkv, D]"},
        "pct_hbm_peak": round(100.0 * gbps / peak, 2),
        "roofline": {"bound": "hbm",
                     "kernel": "decode_split_bf16_kernel<128,4> + decode_combine_kernel",
                     "achieved": round(gbps, 1), "peak": peak, "unit": "GB/s",
                     "frac": round(gbps / peak, 4),
                     "traffic": measured_traffic(
                         w.name, DECODE_POOL_TRAFFIC_FILE if pooled else DECODE_TRAFFIC_FILE,
                         DECODE_SOURCE),
                     "algorithmic_bytes": st.bytes, "launch_ms": round(ms, 5)},
    }
    if pooled:
        rec["cache_bytes"] = {"pooled": st.pool_bytes, "dense": st.dense_cache_bytes,
                              "ratio": round(st.pool_bytes / st.dense_cache_bytes, 4)}
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        rec["cpu_baseline"] = decode_cpu_baseline(st, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def chunk_main(args):
    """Router over the layer's key states, then the chunked prefill of the last `chunk`
    tokens over the rest as a KV prefix (ea_hybrid_attn_prefill_chunked)."""
    layer = Layer(args.workload)
    w = layer.w
    assert len(layer.lens) == 1, "one sequence"
    Lk = layer.T
    Lq = min(args.chunk, Lk)
    dev = torch.device("cuda:0")
    q = layer.q[Lk - Lq:].contiguous()
    o = torch.empty_like(q)
    cu_q = inputs.cu_seqlens([Lq]).to(dev)
    cu_k = layer.cu
    ws = torch.empty(ea.prefill_chunked_workspace_size(1, Lq, w.n_heads_q, w.head_dim),
                     dtype=torch.uint8, device=dev)
    layer.do_route()
    torch.cuda.synchronize()

    def step():
        layer.do_route()
        ea.hybrid_attn_prefill_chunked(q, layer.k, layer.v, o, cu_q, cu_k, Lq, Lk, layer.route,
                                       w.sink, w.window, ws)

    def attn_only():
        ea.hybrid_attn_prefill_chunked(q, layer.k, layer.v, o, cu_q, cu_k, Lq, Lk, layer.route,
                                       w.sink, w.window, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms = time_events(step, args.steps)
    ms_attn = time_events(attn_only, args.steps)
    r = layer.route.cpu().tolist()
    F = metrics.chunk_flops([Lk], [Lq], r, w.head_dim, w.sink, w.window)
    peak = metrics.MI355X_BF16_DENSE_TFLOPS
    value = F / (ms * 1e-3) / 1e12
    attn_tf = F / (ms_attn * 1e-3) / 1e12
    rec = {
        "metric": CHUNK_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + f"_chunk{Lq}", "cached_prefix": Lk - Lq, "chunk": Lq,
                   "n_heads_q": w.n_heads_q, "n_heads_kv": w.n_heads_kv, "head_dim": w.head_dim,
                   "sink": w.sink, "window": w.window,
                   "sparse_heads": int(layer.route.sum().item()), "routing": "router"},
        "pct_bf16_peak": round(100.0 * value / peak, 2),
        "effective_tflop": round(F / 1e12, 4),
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_kernel<128>", "achieved": round(attn_tf, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(attn_tf / peak, 4),
                     "traffic": measured_traffic(w.name + f"_chunk{Lq}", CHUNK_TRAFFIC_FILE),
                     "launch_ms": round(ms_attn, 4),
                     "note": "launch_ms includes the planner launch"},
    }
    if args.copy_calibration:
        copy_calibration()
    print(json.dumps(rec), flush=True)


def backward_cpu_baseline(layer: Layer, do_cpu, seconds: float):
    """fp64 oracle backward on a bounded sample of the same layer: the last m rows of the
    first sequence as a chunk over its whole prefix (their dq and their share of dk, dv),
    m doubling until the time budget is spent."""
    import numpy as np
    import oracle
    w = layer.w
    q, k, v = layer.cpu
    L = layer.lens[0]
    route = layer.route.cpu().numpy()[:1]
    threads = oracle.max_threads()
    cu_k = np.array([0, L], dtype=np.int32)
    m, t_used, flops, rows = 4, 0.0, 0, 0
    while t_used < seconds and m <= L:
        cu_q = np.array([0, m], dtype=np.int32)
        t0 = time.perf_counter()
        oracle.attn_backward(q[L - m:L], k[:L], v[:L], do_cpu[L - m:L], cu_q, w.n_heads_q,
                             w.n_heads_kv, route, w.sink, w.window, cu_seqlens_k=cu_k,
                             nthreads=threads)
        t_used += time.perf_counter() - t0
        flops += metrics.chunk_flops([L], [m], route.tolist(), w.head_dim, w.sink,
                                     w.window) * 5 // 2
        rows += m
        m *= 2
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"backward of the last 4..{m // 2} rows of the {L}-token sequence as chunks "
                      f"over its prefix ({rows} rows x {w.n_heads_q} heads, {t_used:.1f} s of "
                      f"fp64 oracle work); effective FLOPs as for the GPU"}


def backward_main(args):
    """Training backward of the layer: the router's straight-through gradient
    (ea_route_backward) and the routed attention's dq, dk, dv (ea_hybrid_attn_backward), with
    the forward's O, LSE and both branch outputs resident."""
    layer = Layer(args.workload)
    w = layer.w
    dev = torch.device("cuda:0")
    T, hq, d = layer.q.shape
    B = len(layer.lens)
    layer.do_route()
    lse = torch.empty(hq, T, dtype=torch.float32, device=dev)
    ea.hybrid_attn_prefill(layer.q, layer.k, layer.v, layer.o, layer.cu, layer.max_len,
                           layer.route, w.sink, w.window, layer.ws, lse_out=lse)
    # the two branch outputs the straight-through router gradient compares
    o_full, o_sp = torch.empty_like(layer.q), torch.empty_like(layer.q)
    for val, out in ((0, o_full), (1, o_sp)):
        r = torch.full_like(layer.route, val)
        ea.hybrid_attn_prefill(layer.q, layer.k, layer.v, out, layer.cu, layer.max_len, r,
                               w.sink, w.window, layer.ws)
    do = inputs.dout(w, T).to(dev)
    noise = inputs.logistic_noise(w, B).to(dev)
    dq = torch.empty(T, hq, d, dtype=torch.float32, device=dev)
    dk = torch.empty(T, w.n_heads_kv, d, dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws_b = torch.empty(ea.attn_backward_workspace_size(ea.EA_BF16, B, layer.max_len, layer.max_len,
                                                       hq, w.n_heads_kv, d),
                       dtype=torch.uint8, device=dev)
    have_router = layer.router is not None
    if have_router:
        w1, b1, w2, b2 = layer.router
        kv_dim, hid = layer.ks.shape[1], w1.shape[0]
        rg = dict(dz=torch.empty(B, hq, device=dev), dw1=torch.empty_like(w1),
                  db1=torch.empty_like(b1), dw2=torch.empty_like(w2), db2=torch.empty_like(b2))
        dks = torch.empty(T, kv_dim, dtype=torch.float32, device=dev)
        ws_r = torch.empty(ea.route_backward_workspace_size(B, kv_dim, hid, hq, d),
                           dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def attn_bwd():
        ea.hybrid_attn_backward(layer.q, layer.k, layer.v, layer.o, do, lse, layer.cu,
                                layer.max_len, layer.route, w.sink, w.window, dq, dk, dv, ws_b)

    def route_bwd():
        if have_router:
            ea.route_backward(layer.ks, layer.cu, w1, b1, w2, b2, o_full, o_sp, do, rg["dz"],
                              rg["dw1"], rg["db1"], rg["dw2"], rg["db2"], ws_r, tau=1.0,
                              noise=noise, dkey_states=dks)

    def step():
        route_bwd()
        attn_bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms = time_events(step, args.steps)
    ms_attn = time_events(attn_bwd, args.steps)
    ms_route = time_events(route_bwd, args.steps) if have_router else 0.0
    r = layer.route.cpu().tolist()
    F = metrics.backward_flops(layer.lens, r, d, w.sink, w.window)
    f_dq, f_dkv = metrics.backward_kernel_flops(layer.lens, r, d, w.sink, w.window)
    value = F / (ms * 1e-3) / 1e12
    peak = metrics.MI355X_BF16_DENSE_TFLOPS
    kern_tf = (f_dq + f_dkv) / (ms_attn * 1e-3) / 1e12
    rec = {
        "metric": BACKWARD_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + "_backward", "batch": B, "seq_len": layer.max_len,
                   "n_heads_q": hq, "n_heads_kv": w.n_heads_kv, "head_dim": d, "sink": w.sink,
                   "window": w.window, "sparse_heads": int(layer.route.sum().item()),
                   "routing": "router" if have_router else "bernoulli",
                   "inputs": "bf16", "gradients": "fp32"},
        "effective_tflop": round(F / 1e12, 4),
        "attn_backward_ms": round(ms_attn, 4), "route_backward_ms": round(ms_route, 4),
        "roofline": {"bound": "mfma",
                     "kernel": "ea_hybrid_attn_backward (bwd_dq_mfma<128> + bwd_dkv_mfma<128>)",
                     "achieved": round(kern_tf, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(kern_tf / peak, 4),
                     "traffic": measured_traffic(w.name + "_backward", BWD_TRAFFIC_FILE,
                                                 BWD_SOURCE),
                     "launch_ms": round(ms_attn, 4),
                     "note": "launch_ms is the whole ea_hybrid_attn_backward call (D, dq, dk/dv, "
                             "partial reduce); achieved counts the products the two matrix-core "
                             "kernels run per kept position and head: 6*D (dq: S, dP, dQ) + "
                             "8*D (dk/dv: S, dP, dV, dK); traffic is the dk/dv kernel's"},
    }
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        rec["cpu_baseline"] = backward_cpu_baseline(layer, inputs.dout(w, T), args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--mode", choices=("prefill", "prefill_chunk", "decode", "decode_pool",
                                       "backward"),
                    default="prefill")
    ap.add_argument("--chunk", type=int, default=4096, help="chunk length for --mode prefill_chunk")
    ap.add_argument("--workload", default=None,
                    help="default qwen3_8b_32k (prefill) or decode_qwen3_8b_32k (decode)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="untimed steps before the warm-up steps, until this much wall time "
                         "has passed (the shader clock ramps over the first launches)")
    ap.add_argument("--alone", action="store_true",
                    help="prefill: time every step alone (synchronised before it), no eviction "
                         "write: the reference for --evict")
    ap.add_argument("--evict", action="store_true",
                    help="prefill: write a 512 MiB scratch buffer before each timed step and "
                         "time every step alone (cold L2 / MALL); default: back-to-back steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one elementwise copy kernel of 1 GiB in and 1 GiB "
                         "out (a known-size kernel for scaling rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the routed "
                                   "prefill is not sharded across GPUs (--gpus 1)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    ea.lib()  # fail loudly if the HIP library is missing
    if args.mode in ("decode", "decode_pool"):
        args.workload = args.workload or "decode_qwen3_8b_32k"
        decode_main(args, pooled=args.mode == "decode_pool")
        return
    args.workload = args.workload or "qwen3_8b_32k"
    if args.mode == "prefill_chunk":
        chunk_main(args)
        return
    if args.mode == "backward":
        backward_main(args)
        return

    layer = Layer(args.workload)
    w = layer.w
    log(f"workload {w.name}: lens={layer.lens} T={layer.T}")
    layer.do_route()
    torch.cuda.synchronize()
    n_sparse = int(layer.route.sum().item())
    F = layer.flops()
    n_settle = settle(layer.step, args.settle_seconds)
    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.evict or args.alone:
        scratch = torch.empty(1 << 27, dtype=torch.float32, device="cuda") if args.evict else None
        ms = time_events_evict(layer.step, args.steps, scratch)
    else:
        ms = time_events(layer.step, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (wall {wall:.3f} s, after {n_settle} "
        f"settle steps)")

    # phase breakdown and the attention kernel alone (same stream)
    ms_route = time_events(layer.do_route, args.steps) if layer.router is not None else 0.0
    ms_plan = time_events(layer.do_plan, args.steps)
    layer.do_plan()
    ms_attn = time_events(layer.do_attn, args.steps)
    io = metrics.io_bytes(layer.T, w.n_heads_q, w.n_heads_kv, w.head_dim, 2)
    attn_tflops = F / (ms_attn * 1e-3) / 1e12
    peak = metrics.MI355X_BF16_DENSE_TFLOPS
    value = F / (ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC.format(WORKLOAD_LABEL.get(w.name, w.name)),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": len(layer.lens), "seq_len": layer.max_len,
                   "total_tokens": layer.T, "n_heads_q": w.n_heads_q,
                   "n_heads_kv": w.n_heads_kv, "head_dim": w.head_dim, "sink": w.sink,
                   "window": w.window, "sparse_heads": n_sparse,
                   "routing": "router" if w.router else f"bernoulli({w.p_sparse})"},
        "pct_bf16_peak": round(100.0 * value / peak, 2),
        "effective_tflop": round(F / 1e12, 4),
        "settle_steps": n_settle,
        "timing": ("each step alone after a 512 MiB eviction write" if args.evict
                   else "each step alone" if args.alone else "back-to-back steps"),
        "ms_breakdown": {"route": round(ms_route, 4), "plan": round(ms_plan, 4),
                         "attention": round(ms_attn, 4)},
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_kernel<128>",
                     "achieved": round(attn_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / peak, 4), "traffic": measured_traffic(w.name),
                     "algorithmic_bytes": io, "launch_ms": round(ms_attn, 4)},
    }
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        rec["cpu_baseline"] = cpu_baseline(layer, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
