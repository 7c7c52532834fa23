"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The library's product path never does: it shares
no code with the HIP kernels and neither side imports the other.

The arithmetic lives in ``oracle.c`` (plain C, double precision, libm); this
module only builds it with gcc, loads it with ctypes and marshals numpy
arrays.  What it computes is the plain definition of attention,
O = softmax(scale * Q K^T) V with the row log-sum-exp, and the derived
backward (see the header of ``oracle.c`` for the readings it takes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (portable -O3, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    u8p = ctypes.POINTER(ctypes.c_ubyte)
    lib.oracle_forward.argtypes = [dp, dp, dp, dp, dp, ctypes.c_long, ctypes.c_long,
                                   ctypes.c_int, ctypes.c_double, ctypes.c_int, u8p,
                                   ctypes.c_int, ctypes.c_int]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_backward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_long,
                                    ctypes.c_long, ctypes.c_int, ctypes.c_double,
                                    ctypes.c_int, u8p, ctypes.c_int, ctypes.c_int]
    lib.oracle_backward.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    """OpenMP threads the oracle uses when none are requested."""
    return int(_load().oracle_max_threads())


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: widen exactly to fp64 on the host
        import torch
        x = x.detach().to(device="cpu", dtype=torch.float64)
        return np.ascontiguousarray(x.numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _mask(block_mask, N: int, mask_block: int):
    if block_mask is None:
        return None, None
    if hasattr(block_mask, "detach"):
        block_mask = block_mask.detach().cpu().numpy()
    m = np.ascontiguousarray(np.asarray(block_mask, dtype=np.uint8))
    nb = -(-N // mask_block)
    if m.shape != (nb, nb):
        raise ValueError(f"block mask must be [{nb}][{nb}] for N={N}, block={mask_block}")
    return m, m.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte))


def _heads(q):
    *lead, N, d = q.shape
    return int(np.prod(lead)) if lead else 1, N, d, lead


def forward(q, k, v, scale: float, causal: bool = False, block_mask=None,
            mask_block: int = 128, threads: int = 0):
    """O and LSE of exact attention for arrays shaped [..., N, d] (fp64 copies)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one shape [..., N, d]")
    nh, N, d, lead = _heads(q)
    o = np.zeros_like(q)
    lse = np.zeros(tuple(lead) + (N,), dtype=np.float64)
    m, mp = _mask(block_mask, N, mask_block)
    rc = _load().oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), nh, N, d,
                                float(scale), int(bool(causal)), mp, int(mask_block),
                                int(threads))
    if rc != 0:
        raise RuntimeError("oracle_forward failed")
    return o, lse


def backward(q, k, v, dout, scale: float, causal: bool = False, block_mask=None,
             mask_block: int = 128, threads: int = 0):
    """dQ, dK, dV (and LSE, D) of exact attention for arrays shaped [..., N, d]."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout must share one shape [..., N, d]")
    nh, N, d, lead = _heads(q)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    lse = np.zeros(tuple(lead) + (N,), dtype=np.float64)
    delta = np.zeros_like(lse)
    m, mp = _mask(block_mask, N, mask_block)
    rc = _load().oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(lse), _ptr(delta), nh, N, d, float(scale),
                                 int(bool(causal)), mp, int(mask_block), int(threads))
    if rc != 0:
        raise RuntimeError("oracle_backward failed")
    return dq, dk, dv, lse, delta


def _groups(q, k):
    """Query heads per K/V head for q [..., H, N, d] and k [..., Hkv, N, d]."""
    if q.ndim < 3 or k.ndim != q.ndim or q.shape[:-3] != k.shape[:-3] or \
            q.shape[-2:] != k.shape[-2:]:
        raise ValueError("q must be [..., H, N, d] and k, v [..., Hkv, N, d]")
    H, Hkv = q.shape[-3], k.shape[-3]
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"Hkv={Hkv} must divide H={H}")
    return H // Hkv


def forward_gqa(q, k, v, scale: float, causal: bool = False, threads: int = 0):
    """Grouped K/V heads: query head h reads K/V head h // (H / Hkv).

    Multi-query and grouped-query attention ("Flash Attention: IO-Aware
    Attention Computation", closing paragraph on future directions) are plain
    attention per query head with some K/V heads shared; each query head's
    result is the plain definition above with its group's K and V.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    g = _groups(q, k)
    return forward(q, np.repeat(k, g, axis=-3), np.repeat(v, g, axis=-3), scale, causal,
                   threads=threads)


def backward_gqa(q, k, v, dout, scale: float, causal: bool = False, threads: int = 0):
    """dQ [..., H, N, d] and dK, dV [..., Hkv, N, d] of forward_gqa.

    A K/V head read by several query heads is one parameter used several
    times, so its gradient is the sum of the per-query-head gradients.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    g = _groups(q, k)
    dq, dk, dv, lse, delta = backward(q, np.repeat(k, g, axis=-3), np.repeat(v, g, axis=-3),
                                      dout, scale, causal, threads=threads)
    shape = k.shape[:-3] + (k.shape[-3], g) + k.shape[-2:]
    return dq, dk.reshape(shape).sum(axis=-3), dv.reshape(shape).sum(axis=-3), lse, delta
