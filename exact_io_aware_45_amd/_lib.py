"""ctypes binding of libfa.so (include/fa.h).  Argument marshalling only.

Every step of attention runs in the HIP kernels behind the C ABI; this module
checks tensors, allocates outputs with torch (torch is used for device memory
and streams only) and passes raw device pointers plus torch's current HIP
stream.  If libfa.so is missing, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FA_LIB_PATH") or os.path.join(_HERE, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
SYMBOLS = ("fa_forward", "fa_forward_f32", "fa_backward_workspace_size", "fa_backward",
           "fa_forward_blocksparse", "fa_error_string", "fa_version", "fa_runtime_version")

_lib = None


class FAError(RuntimeError):
    """A non-zero fa_status returned by the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {error_string(status)} (status {status})")


def load():
    """Load libfa.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m exact_io_aware_45_amd.build` "
                           "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_forward_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_forward_blocksparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
    lib.fa_backward_workspace_size.argtypes = [i, i, i, i]
    lib.fa_backward_workspace_size.restype = sz
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    for name in ("fa_forward", "fa_forward_f32", "fa_forward_blocksparse", "fa_backward",
                 "fa_version", "fa_runtime_version"):
        getattr(lib, name).restype = i
    lib.fa_error_string.argtypes = [i]
    lib.fa_error_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_runtime_version.argtypes = []
    _lib = lib
    return lib


def error_string(status: int) -> str:
    return load().fa_error_string(int(status)).decode()


def version() -> int:
    return int(load().fa_version())


def runtime_version() -> int:
    return int(load().fa_runtime_version())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, what: str):
    if status != FA_OK:
        raise FAError(status, what)


def _shape(q, k, v, dtype):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same shape [B, H, N, d]")
    return tuple(int(x) for x in q.shape)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward(q, k, v, causal: bool = False, scale: float | None = None):
    """fa_forward (bf16) or fa_forward_f32 (fp32). Returns (o, lse)."""
    lib = load()
    if q.dtype == torch.float32:
        B, H, N, d = _shape(q, k, v, torch.float32)
        fn, what = lib.fa_forward_f32, "fa_forward_f32"
    else:
        B, H, N, d = _shape(q, k, v, torch.bfloat16)
        fn, what = lib.fa_forward, "fa_forward"
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _scale(scale, d),
              int(bool(causal)), _stream(q.device)), what)
    return o, lse


def forward_blocksparse(q, k, v, block_mask, mask_block: int = 128, causal: bool = False,
                        scale: float | None = None):
    """fa_forward_blocksparse: block_mask is a uint8 device tensor [nb][nb]."""
    lib = load()
    B, H, N, d = _shape(q, k, v, torch.bfloat16)
    nb = -(-N // mask_block) if mask_block > 0 else 0
    if (block_mask.dtype != torch.uint8 or not block_mask.is_cuda
            or tuple(block_mask.shape) != (nb, nb) or not block_mask.is_contiguous()):
        raise ValueError(f"block_mask must be a contiguous uint8 device tensor [{nb}][{nb}]")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(lib.fa_forward_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                      _scale(scale, d), int(bool(causal)), _ptr(block_mask),
                                      int(mask_block), _stream(q.device)),
           "fa_forward_blocksparse")
    return o, lse


def backward_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load().fa_backward_workspace_size(B, H, N, d))


def backward(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
             workspace=None):
    """fa_backward: returns (dq, dk, dv), fp32."""
    lib = load()
    B, H, N, d = _shape(q, k, v, torch.bfloat16)
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bf16 device tensor shaped like q")
    if (lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or not lse.is_cuda):
        raise ValueError("lse must be a contiguous fp32 device tensor [B, H, N]")
    ws_bytes = backward_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    _check(lib.fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), B, H, N, d,
                           _scale(scale, d), int(bool(causal)), _stream(q.device)),
           "fa_backward")
    return dq, dk, dv
