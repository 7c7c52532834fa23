"""Shared helpers of the GPU parity tests: element-by-element comparison of
library outputs with the fp64 oracle at the stated tolerances.

Tolerances (absolute, per output tensor, over all compared elements):
  bf16 storage, fp32 accumulation: max |err| <= 2e-2 and mean |err| <= 2e-3
  fp32 path:                       max |err| <= 1e-5
LSE is held to the same bounds.  Rows whose oracle LSE is -inf (no visible
key) must be -inf on the GPU too and have O == 0 exactly.
"""
import sys

import numpy as np
import torch

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def errors(gpu, ref):
    g = to64(gpu) if torch.is_tensor(gpu) else np.asarray(gpu, dtype=np.float64)
    e = np.abs(g - ref)
    return float(e.max()) if e.size else 0.0, float(e.mean()) if e.size else 0.0


def check(name, gpu, ref, bf16=True, scale=1.0):
    """Max and mean absolute error against the bounds (times `scale`, for
    sums of several independently rounded gradients)."""
    mx, mean = errors(gpu, ref)
    log(f"  {name}: max_abs={mx:.3e} mean_abs={mean:.3e}")
    if bf16:
        assert mx <= BF16_MAX * scale and mean <= BF16_MEAN * scale, (name, mx, mean)
    else:
        assert mx <= F32_MAX, (name, mx)
    return mx, mean


def check_lse(gpu_lse, ref_lse, bf16=True):
    g = to64(gpu_lse)
    ref_inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(g), ref_inf), "LSE -inf pattern differs"
    if ref_inf.all():
        return 0.0, 0.0
    return check("lse", g[~ref_inf], ref_lse[~ref_inf], bf16)
