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

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 8 << 20  # FA_NOALLOC_SCRATCH_BYTES
SYMBOLS = ("fa_forward", "fa_forward_f32", "fa_backward_workspace_size", "fa_backward",
           "fa_backward_noalloc",
           "fa_forward_blocksparse", "fa_backward_blocksparse", "fa_forward_gqa",
           "fa_backward_gqa", "fa_backward_gqa_workspace_size", "fa_forward_fp8",
           "fa_error_string", "fa_version", "fa_runtime_version")

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
    lib.fa_backward_gqa_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_backward_gqa_workspace_size.restype = sz
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    lib.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_backward_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i,
                                            i, f, i, vp, i, vp]
    lib.fa_forward_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, f, f, f, i, vp]
    lib.fa_backward_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f,
                                    i, vp]
    for name in ("fa_forward", "fa_forward_f32", "fa_forward_blocksparse", "fa_backward",
                 "fa_backward_noalloc",
                 "fa_backward_blocksparse", "fa_forward_gqa", "fa_backward_gqa",
                 "fa_forward_fp8", "fa_version", "fa_runtime_version"):
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


def _tensor(name, t, dtype, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _shape(q, k, v, dtype, grouped: bool = False):
    """(B, H, Hkv, N, d) of q [B,H,N,d] and k, v [B,Hkv,N,d] (Hkv == H unless grouped)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _tensor(name, t, dtype)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
    B, H, N, d = (int(x) for x in q.shape)
    Hkv = int(k.shape[1])
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if grouped:
        if (int(k.shape[0]), int(k.shape[2]), int(k.shape[3])) != (B, N, d):
            raise ValueError("k, v must be [B, Hkv, N, d] with q's B, N and d")
    elif k.shape != q.shape:
        raise ValueError("q, k, v must have the same shape [B, H, N, d]")
    return B, H, Hkv, N, d


def _mask(block_mask, N, mask_block):
    nb = -(-N // mask_block) if mask_block > 0 else 0
    if (not isinstance(block_mask, torch.Tensor) or block_mask.dtype != torch.uint8
            or not block_mask.is_cuda or tuple(block_mask.shape) != (nb, nb)
            or not block_mask.is_contiguous()):
        raise ValueError(f"block_mask must be a contiguous uint8 device tensor [{nb}][{nb}]")


def _fwd_out(q, B, H, N, odtype, out):
    """(o, lse): new tensors, or the caller's `out` pair after checking it."""
    if out is None:
        return (torch.empty(q.shape, dtype=odtype, device=q.device),
                torch.empty((B, H, N), dtype=torch.float32, device=q.device))
    o, lse = out
    _tensor("o", o, odtype, q.shape)
    _tensor("lse", lse, torch.float32, (B, H, N))
    return o, lse


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None):
    """fa_forward (bf16) or fa_forward_f32 (fp32). Returns (o, lse), written into
    `out` = (o, lse) when given (o like q, lse fp32 [B,H,N])."""
    lib = load()
    if q.dtype == torch.float32:
        B, H, _, N, d = _shape(q, k, v, torch.float32)
        fn, what = lib.fa_forward_f32, "fa_forward_f32"
    else:
        B, H, _, N, d = _shape(q, k, v, torch.bfloat16)
        fn, what = lib.fa_forward, "fa_forward"
    o, lse = _fwd_out(q, B, H, N, q.dtype, out)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _scale(scale, d),
              int(bool(causal)), _stream(q.device)), what)
    return o, lse


def forward_blocksparse(q, k, v, block_mask, mask_block: int = 128, causal: bool = False,
                        scale: float | None = None, out=None):
    """fa_forward_blocksparse: block_mask is a uint8 device tensor [nb][nb]."""
    lib = load()
    B, H, _, N, d = _shape(q, k, v, torch.bfloat16)
    _mask(block_mask, N, mask_block)
    o, lse = _fwd_out(q, B, H, N, q.dtype, out)
    _check(lib.fa_forward_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                      _scale(scale, d), int(bool(causal)), _ptr(block_mask),
                                      int(mask_block), _stream(q.device)),
           "fa_forward_blocksparse")
    return o, lse


def forward_gqa(q, k, v, causal: bool = False, scale: float | None = None, out=None):
    """fa_forward_gqa: q [B,H,N,d], k, v [B,Hkv,N,d] bf16 (Hkv divides H)."""
    lib = load()
    B, H, Hkv, N, d = _shape(q, k, v, torch.bfloat16, grouped=True)
    o, lse = _fwd_out(q, B, H, N, q.dtype, out)
    _check(lib.fa_forward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                              _scale(scale, d), int(bool(causal)), _stream(q.device)),
           "fa_forward_gqa")
    return o, lse


def forward_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float,
                causal: bool = False, scale: float | None = None, out=None):
    """fa_forward_fp8: q, k, v torch.float8_e4m3fn [B,H,N,d] codes; returns (o bf16, lse)."""
    lib = load()
    B, H, _, N, d = _shape(q, k, v, torch.float8_e4m3fn)
    o, lse = _fwd_out(q, B, H, N, torch.bfloat16, out)
    _check(lib.fa_forward_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                              _scale(scale, d), float(q_descale), float(k_descale),
                              float(v_descale), int(bool(causal)), _stream(q.device)),
           "fa_forward_fp8")
    return o, lse


def backward_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load().fa_backward_workspace_size(B, H, N, d))


def backward_gqa_workspace_size(B: int, H: int, Hkv: int, N: int, d: int) -> int:
    return int(load().fa_backward_gqa_workspace_size(B, H, Hkv, N, d))


def _backward_args(q, k, v, o, dout, lse, grouped, workspace, out=None):
    B, H, Hkv, N, d = _shape(q, k, v, torch.bfloat16, grouped)
    _tensor("o", o, torch.bfloat16, q.shape)
    _tensor("dout", dout, torch.bfloat16, q.shape)
    _tensor("lse", lse, torch.float32, (B, H, N))
    ws_bytes = (backward_gqa_workspace_size(B, H, Hkv, N, d) if grouped
                else backward_workspace_size(B, H, N, d))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    else:
        _tensor("workspace", workspace, torch.uint8)
    if out is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        dk, dv = (torch.empty(k.shape, dtype=torch.float32, device=q.device) for _ in range(2))
    else:
        dq, dk, dv = out
        _tensor("dq", dq, torch.float32, q.shape)
        _tensor("dk", dk, torch.float32, k.shape)
        _tensor("dv", dv, torch.float32, k.shape)
    return (B, H, Hkv, N, d), workspace, (dq, dk, dv)


def backward(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
             workspace=None, out=None):
    """fa_backward: returns (dq, dk, dv), fp32."""
    lib = load()
    (B, H, _, N, d), ws, (dq, dk, dv) = _backward_args(q, k, v, o, dout, lse, False, workspace, out)
    _check(lib.fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), B, H, N, d,
                           _scale(scale, d), int(bool(causal)), _stream(q.device)),
           "fa_backward")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
                     out=None):
    """fa_backward_noalloc: fa_backward with the library's fixed per-device
    scratch as workspace (B*H*N <= 1048576 rows).  Returns (dq, dk, dv)."""
    lib = load()
    B, H, _, N, d = _shape(q, k, v, torch.bfloat16)
    _tensor("o", o, torch.bfloat16, q.shape)
    _tensor("dout", dout, torch.bfloat16, q.shape)
    _tensor("lse", lse, torch.float32, (B, H, N))
    if out is None:
        dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=q.device)
                      for _ in range(3))
    else:
        dq, dk, dv = out
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            _tensor(name, t, torch.float32, q.shape)
    _check(lib.fa_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, _scale(scale, d),
                                   int(bool(causal)), _stream(q.device)),
           "fa_backward_noalloc")
    return dq, dk, dv


def backward_blocksparse(q, k, v, o, dout, lse, block_mask, mask_block: int = 128,
                         causal: bool = False, scale: float | None = None, workspace=None,
                         out=None):
    """fa_backward_blocksparse: the gradients of fa_forward_blocksparse, fp32."""
    lib = load()
    (B, H, _, N, d), ws, (dq, dk, dv) = _backward_args(q, k, v, o, dout, lse, False, workspace, out)
    _mask(block_mask, N, mask_block)
    _check(lib.fa_backward_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), B, H,
                                       N, d, _scale(scale, d), int(bool(causal)),
                                       _ptr(block_mask), int(mask_block), _stream(q.device)),
           "fa_backward_blocksparse")
    return dq, dk, dv


def backward_gqa(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
                 workspace=None, out=None):
    """fa_backward_gqa: dq [B,H,N,d]; dk, dv [B,Hkv,N,d] summed over each group, fp32."""
    lib = load()
    (B, H, Hkv, N, d), ws, (dq, dk, dv) = _backward_args(q, k, v, o, dout, lse, True, workspace, out)
    _check(lib.fa_backward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), B, H, Hkv, N,
                               d, _scale(scale, d), int(bool(causal)), _stream(q.device)),
           "fa_backward_gqa")
    return dq, dk, dv
