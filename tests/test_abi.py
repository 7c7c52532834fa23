"""The C ABI without a GPU: libfa.so loads, exports every function that
include/fa.h declares, and rejects invalid arguments before anything is
enqueued (these calls never reach a kernel launch)."""
import ctypes
import os
import re

import pytest

from exact_io_aware_45_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libfa.so not built")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first
MIS = 0x10002   # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fa_forward", "fa_backward", "fa_forward_blocksparse", "fa_backward_blocksparse",
              "fa_forward_gqa", "fa_backward_gqa", "fa_forward_fp8"):
        assert n in names
    assert set(names) == set(_lib.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_version_and_error_strings():
    lib = _lib.load()
    assert _lib.version() == 400
    for st in range(5):
        s = _lib.error_string(st)
        assert isinstance(s, str) and s
    assert _lib.error_string(99) == "unknown status"
    assert _lib.error_string(0) == "success"
    del lib


def fwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, scale=0.125, causal=0):
    return _lib.load().fa_forward(q, k, v, o, lse, B, H, N, d, scale, causal, None)


def test_forward_argument_errors():
    INV, UNS = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED
    assert fwd(q=None) == INV
    assert fwd(k=None) == INV
    assert fwd(v=None) == INV
    assert fwd(o=None) == INV
    assert fwd(lse=None) == INV
    assert fwd(q=MIS) == INV
    assert fwd(o=MIS) == INV
    assert fwd(lse=FAKE + 2) == INV
    assert fwd(B=-1) == INV
    assert fwd(H=-2) == INV
    assert fwd(N=-3) == INV
    assert fwd(d=0) == INV
    assert fwd(d=96) == UNS
    assert fwd(d=256) == UNS
    assert fwd(scale=0.0) == INV
    assert fwd(scale=-1.0) == INV
    assert fwd(scale=float("nan")) == INV
    assert fwd(scale=float("inf")) == INV


def test_empty_problems_are_no_ops():
    OK = _lib.FA_OK
    assert fwd(q=None, k=None, v=None, o=None, lse=None, N=0) == OK
    assert fwd(q=None, k=None, v=None, o=None, lse=None, B=0) == OK
    assert fwd(q=None, k=None, v=None, o=None, lse=None, H=0) == OK
    lib = _lib.load()
    assert lib.fa_forward_f32(None, None, None, None, None, 0, 4, 8, 64, 0.1, 0, None) == OK
    assert lib.fa_backward(None, None, None, None, None, None, None, None, None, None, 0,
                           2, 2, 0, 128, 0.1, 1, None) == OK
    assert lib.fa_forward_blocksparse(None, None, None, None, None, 1, 1, 0, 64, 0.1, 0, None,
                                      128, None) == OK
    # even empty, an unsupported head size is reported
    assert fwd(N=0, d=80) == _lib.FA_ERR_UNSUPPORTED


def test_blocksparse_argument_errors():
    lib = _lib.load()
    f = lib.fa_forward_blocksparse
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 256, 64, 0.1, 0, None, 128, None) == \
        _lib.FA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 256, 64, 0.1, 0, FAKE, 64, None) == \
        _lib.FA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 256, 64, 0.1, 0, FAKE, 256, None) == \
        _lib.FA_ERR_UNSUPPORTED
    assert f(MIS, FAKE, FAKE, FAKE, FAKE, 1, 1, 256, 64, 0.1, 0, FAKE, 128, None) == \
        _lib.FA_ERR_INVALID_ARG


def test_backward_workspace_and_argument_errors():
    lib = _lib.load()
    assert _lib.backward_workspace_size(4, 16, 4096, 128) == 2 * 4 * 16 * 4096 * 4
    assert _lib.backward_workspace_size(1, 1, 3, 64) == 256
    assert _lib.backward_workspace_size(1, 1, 0, 64) == 0
    assert _lib.backward_workspace_size(1, 1, 16, 80) == 0
    ws = _lib.backward_workspace_size(1, 1, 16, 64)

    def bwd(ws_ptr=FAKE, ws_bytes=ws, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE)
        a.update(kw)
        return lib.fa_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                               a["dk"], a["dv"], ws_ptr, ws_bytes, 1, 1, 16, 64, 0.125, 1, None)

    INV = _lib.FA_ERR_INVALID_ARG
    assert bwd(ws_ptr=None) == INV
    assert bwd(ws_bytes=ws - 1) == INV
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert bwd(**{name: None}) == INV, name
    assert bwd(dq=MIS) == INV
    assert bwd(do=MIS) == INV


def test_blocksparse_backward_argument_errors():
    lib = _lib.load()
    ws = _lib.backward_workspace_size(1, 1, 256, 64)

    def bwd(mask=FAKE, mb=128, N=256, q=FAKE, ws_bytes=ws):
        return lib.fa_backward_blocksparse(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, ws_bytes, 1, 1, N, 64, 0.125, 0, mask, mb, None)

    assert bwd(mask=None) == _lib.FA_ERR_INVALID_ARG
    assert bwd(mb=64) == _lib.FA_ERR_UNSUPPORTED
    assert bwd(mb=64, N=0) == _lib.FA_ERR_UNSUPPORTED
    assert bwd(q=MIS) == _lib.FA_ERR_INVALID_ARG
    assert bwd(ws_bytes=ws - 4) == _lib.FA_ERR_INVALID_ARG
    assert bwd(mask=None, q=None, N=0) == _lib.FA_OK


def test_gqa_argument_errors():
    lib = _lib.load()
    INV, OK = _lib.FA_ERR_INVALID_ARG, _lib.FA_OK

    def fwd_g(H=8, Hkv=2, N=64, d=64, q=FAKE):
        return lib.fa_forward_gqa(q, FAKE, FAKE, FAKE, FAKE, 1, H, Hkv, N, d, 0.125, 1, None)

    assert fwd_g(Hkv=0) == INV
    assert fwd_g(Hkv=-1) == INV
    assert fwd_g(Hkv=3) == INV      # does not divide H
    assert fwd_g(Hkv=16) == INV     # more K/V heads than query heads
    assert fwd_g(q=None) == INV
    assert fwd_g(d=96) == _lib.FA_ERR_UNSUPPORTED
    assert fwd_g(N=0, q=None) == OK
    ws = _lib.backward_workspace_size(1, 8, 64, 64)

    def bwd_g(Hkv=2, ws_bytes=ws, dk=FAKE):
        return lib.fa_backward_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dk, FAKE, FAKE,
                                   ws_bytes, 1, 8, Hkv, 64, 64, 0.125, 0, None)

    assert bwd_g(Hkv=3) == INV
    assert bwd_g(Hkv=0) == INV
    assert bwd_g(dk=None) == INV
    assert bwd_g(ws_bytes=ws - 4) == INV


def test_fp8_argument_errors():
    lib = _lib.load()
    INV = _lib.FA_ERR_INVALID_ARG

    def f8(qs=0.01, ks=0.01, vs=0.01, q=FAKE, d=128, N=64):
        return lib.fa_forward_fp8(q, FAKE, FAKE, FAKE, FAKE, 1, 2, N, d, 0.088, qs, ks, vs, 1, None)

    assert f8(qs=0.0) == INV
    assert f8(ks=-1.0) == INV
    assert f8(vs=float("nan")) == INV
    assert f8(vs=float("inf")) == INV
    assert f8(q=None) == INV
    assert f8(q=MIS) == INV
    assert f8(d=96) == _lib.FA_ERR_UNSUPPORTED
    assert f8(q=None, N=0) == _lib.FA_OK


def test_gqa_workspace_size():
    """Extra room for the sliced dK/dV partials exactly when a group must be
    split: slices S = the smallest divisor of H/Hkv giving 512 dK/dV
    workgroups (128 keys each), else H/Hkv."""
    base = _lib.backward_workspace_size
    gqa = _lib.backward_gqa_workspace_size
    # MQA at B1 H32 N8192: 64 key tiles, S = 8 (64 * 8 = 512)
    assert gqa(1, 32, 1, 8192, 128) == base(1, 32, 8192, 128) + 256 + 2 * 8 * 8192 * 128 * 4
    # B1 H32 Hkv8: 64 * 8 = 512 workgroups already, no split
    assert gqa(1, 32, 8, 8192, 128) == base(1, 32, 8192, 128)
    # Hkv == H: never split
    assert gqa(4, 16, 16, 4096, 128) == base(4, 16, 4096, 128)
    # tiny: every divisor is too small, so S = H/Hkv = 4
    assert gqa(2, 4, 1, 200, 64) == base(2, 4, 200, 64) + 256 + 2 * 4 * 2 * 200 * 64 * 4
    # invalid grouping or shape
    assert gqa(1, 6, 4, 128, 64) == 0
    assert gqa(1, 4, 0, 128, 64) == 0
    assert gqa(1, 4, 2, 128, 80) == 0
    assert gqa(1, 4, 2, 0, 64) == 0


def test_noalloc_backward_argument_errors_and_limit():
    """fa_backward_noalloc validates like fa_backward and refuses problems whose
    workspace exceeds the fixed scratch before any HIP call."""
    lib = _lib.load()
    INV, BIG, OK = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_TOO_LARGE, _lib.FA_OK

    def nb(B=1, H=1, N=16, d=64, q=FAKE, dq=FAKE, lse=FAKE, scale=0.125):
        return lib.fa_backward_noalloc(q, FAKE, FAKE, FAKE, FAKE, lse, dq, FAKE, FAKE, B, H, N, d,
                                       scale, 1, None)

    assert nb(q=None) == INV
    assert nb(dq=MIS) == INV
    assert nb(lse=FAKE + 2) == INV
    assert nb(scale=0.0) == INV
    assert nb(d=96) == _lib.FA_ERR_UNSUPPORTED
    assert nb(q=None, dq=None, lse=None, N=0) == OK
    rows = _lib.NOALLOC_SCRATCH_BYTES // 8  # two fp32 per row
    assert rows == 1 << 20
    assert _lib.backward_workspace_size(1, 1, rows, 64) == _lib.NOALLOC_SCRATCH_BYTES
    assert nb(N=rows + 1) == BIG
    assert nb(B=4, H=16, N=16385) == BIG
    assert nb(B=4, H=16, N=16385, q=None) == INV  # pointers are checked first
    assert "no-allocation" in _lib.error_string(BIG)
