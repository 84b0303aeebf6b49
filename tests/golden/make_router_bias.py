"""Writes router_bias_qwen3_8b_32k.json: the output bias of the Attention Router for the
Qwen3-8B-shaped 32K workload.

The blog post on Elastic Attention (section 4.2, Figure 6) reports that the router sends
about 85% of heads to sparse attention on code tasks.  The synthetic router has random
weights, so its output bias is chosen to reproduce that ratio: with b1 = 0 and the
bias-free logits z (computed by the fp64 oracle from the workload's key states),
b2 = beta for every head with beta = -(z_(5) + z_(6)) / 2, the midpoint between the 5th
and 6th smallest logits.  Then exactly 5 heads have z + beta < 0 (full attention) and 27
heads (84.4%) have z + beta > 0 (sparse).  beta is stored rounded to fp32, the precision
of the router's parameters, and the smallest |z + beta| (the decision margin) is
recorded.  Only the oracle computes anything here.

Run from the repository root:  python tests/golden/make_router_bias.py
"""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from full_attention_long_amd import inputs  # noqa: E402

N_FULL = 5


def main():
    w = inputs.WORKLOADS["qwen3_8b_32k"]
    lens = inputs.lengths(w)
    total = sum(lens)
    k = inputs.normal((total, w.n_heads_kv, w.head_dim), w.index, inputs.STREAM_K, w.dtype)
    ks = k.view(total, w.n_heads_kv * w.head_dim)
    w1, b1, w2, b2 = inputs.router_weights(w)
    _, logits, _ = oracle.route(ks, inputs.cu_seqlens(lens), w1, b1, w2, b2)
    z = np.sort(logits[0])
    beta = float(np.float32(-(z[N_FULL - 1] + z[N_FULL]) / 2.0))
    shifted = logits[0] + beta
    margin = float(np.min(np.abs(shifted)))
    n_sparse = int(np.sum(shifted > 0))
    assert n_sparse == w.n_heads_q - N_FULL, n_sparse
    assert margin >= 1e-7, margin
    out = {
        "workload": w.name,
        "b1": 0.0,
        "b2": beta,
        "n_full": N_FULL,
        "n_sparse": n_sparse,
        "decision_margin": margin,
        "logit_scale": float(np.std(logits[0])),
        "note": "b2 = -(z_(5)+z_(6))/2 over the bias-free fp64 oracle logits, as fp32",
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "router_bias_qwen3_8b_32k.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
