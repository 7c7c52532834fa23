"""Exact attention for AMD MI355X (gfx950): FlashAttention-style tiled forward,
backward with recomputation, block-sparse forward and backward, and grouped
(multi-query / grouped-query) K/V heads, and an fp8 forward, as hand-written HIP
kernels behind a C ABI (include/fa.h, libfa.so).

    from exact_io_aware_45_amd import forward, backward, forward_blocksparse
    o, lse = forward(q, k, v, causal=True)            # bf16 or fp32 [B,H,N,d]
    dq, dk, dv = backward(q, k, v, o, do, lse, causal=True)

The library is loaded lazily on the first call; a missing libfa.so raises.
"""
from ._lib import (FAError, backward, backward_blocksparse, backward_gqa,  # noqa: F401
                   backward_workspace_size, error_string, forward, forward_blocksparse,
                   forward_fp8, forward_gqa, load, runtime_version, version)

__all__ = ["forward", "backward", "forward_blocksparse", "backward_blocksparse", "forward_gqa",
           "forward_fp8",
           "backward_gqa", "backward_workspace_size", "error_string", "version",
           "runtime_version", "load", "FAError"]
