"""Routed hybrid-attention prefill (Elastic Attention) for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libea.so`` (hand-written HIP kernels) declared
in ``include/ea.h``; ``full_attention_long_amd.ea`` is its thin ctypes binding.
``full_attention_long_amd.inputs`` holds the seeded synthetic workloads.
Importing the package does not load the library; the binding loads it on first use and
raises if it has not been built.
"""
__all__ = ["ea", "inputs", "metrics"]
