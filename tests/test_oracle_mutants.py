"""Mutation test of the oracle's pins (CPU only).

Each case copies oracle/oracle.c to a temporary directory, plants one plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, an
off-by-one mask), compiles it with gcc and runs a compact set of the pins from
test_oracle.py against the mutant: brute force in decimal arithmetic, closed
forms, invariants and finite differences.  The test passes only if every
mutant is caught by at least one pin, which shows the pins can tell the
oracle's definition apart from its likely corruptions.  The real oracle must
pass all of the same checks.
"""
import ctypes
import math
import os
import shutil
import subprocess
import tempfile
from decimal import Decimal, getcontext

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("causal_off_by_one", "if (causal && j > i)", "if (causal && j >= i)"),
    ("causal_reversed", "if (causal && j > i)", "if (causal && j < i)"),
    ("mask_transposed", "mask[(i / mb) * nkb + (j / mb)]", "mask[(j / mb) * nkb + (i / mb)]"),
    ("no_scale", "p[j] = scale * dot(qi, K + j * d, d);", "p[j] = dot(qi, K + j * d, d);"),
    ("no_max_shift_in_lse", "return m + log(l);", "return log(l);"),
    ("lse_log2", "return m + log(l);", "return m + log2(l);"),
    ("no_normalisation", "p[j] /= l;", "p[j] /= 1.0;"),
    ("dot_skips_last", "for (int c = 0; c < d; ++c)\n        acc += a[c] * b[c];",
     "for (int c = 0; c + 1 < d; ++c)\n        acc += a[c] * b[c];"),
    ("v_row_index", "oi[c] += p[j] * V[j * d + c];", "oi[c] += p[j] * V[i * d + c];"),
    ("dv_uses_q", "dvj[c] += pij * dO[i * d + c];", "dvj[c] += pij * Q[i * d + c];"),
    ("ds_sign", "const double dsij = p[j] * (dp[j] - Di);", "const double dsij = p[j] * (Di - dp[j]);"),
    ("ds_drops_delta", "const double dsij = p[j] * (dp[j] - Di);", "const double dsij = p[j] * dp[j];"),
    ("dk_no_scale", "dkj[c] += scale * dsij * Q[i * d + c];", "dkj[c] += dsij * Q[i * d + c];"),
    ("dk_uses_k", "dkj[c] += scale * dsij * Q[i * d + c];", "dkj[c] += scale * dsij * kj[c];"),
    ("dq_uses_q", "dqi[c] += scale * dsij * K[j * d + c];", "dqi[c] += scale * dsij * q[r * d + c];"),
    ("column_sweep_causal_flip", "if (!visible(i, j, causal, mask, mb, nkb) || L[i] == -INFINITY)",
     "if (!visible(j, i, causal, mask, mb, nkb) || L[i] == -INFINITY)"),
    ("masked_row_nan", "        return -INFINITY;\n    }\n    double l = 0.0;",
     "        return NAN;\n    }\n    double l = 0.0;"),
]


def build(src_text, tmp):
    path = os.path.join(tmp, "oracle.c")
    with open(path, "w") as f:
        f.write(src_text)
    lib = os.path.join(tmp, "liboracle.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", lib, path,
                    "-lm"], check=True, capture_output=True)
    return lib


class Oracle:
    """Minimal ctypes front end over a given oracle build (test-local)."""

    def __init__(self, path):
        self.lib = ctypes.CDLL(path)
        dp, u8p = ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_ubyte)
        self.lib.oracle_forward.argtypes = [dp] * 5 + [ctypes.c_long, ctypes.c_long, ctypes.c_int,
                                                       ctypes.c_double, ctypes.c_int, u8p,
                                                       ctypes.c_int, ctypes.c_int]
        self.lib.oracle_backward.argtypes = [dp] * 9 + [ctypes.c_long, ctypes.c_long,
                                                        ctypes.c_int, ctypes.c_double,
                                                        ctypes.c_int, u8p, ctypes.c_int,
                                                        ctypes.c_int]

    @staticmethod
    def _p(a):
        return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))

    def forward(self, q, k, v, scale, causal, mask=None, mb=1):
        q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
        N, d = q.shape
        o, lse = np.zeros_like(q), np.zeros(N)
        mp = None
        if mask is not None:
            mask = np.ascontiguousarray(mask, dtype=np.uint8)
            mp = mask.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte))
        rc = self.lib.oracle_forward(self._p(q), self._p(k), self._p(v), self._p(o), self._p(lse),
                                     1, N, d, scale, int(causal), mp, mb, 1)
        assert rc == 0
        return o, lse

    def backward(self, q, k, v, do, scale, causal):
        q, k, v, do = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, do))
        N, d = q.shape
        dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
        lse, delta = np.zeros(N), np.zeros(N)
        rc = self.lib.oracle_backward(self._p(q), self._p(k), self._p(v), self._p(do),
                                      self._p(dq), self._p(dk), self._p(dv), self._p(lse),
                                      self._p(delta), 1, N, d, scale, int(causal), None, 1, 1)
        assert rc == 0
        return dq, dk, dv


def brute(q, k, v, scale, vis):
    getcontext().prec = 40
    N, d = q.shape
    O, L = np.zeros((N, d)), np.zeros(N)
    for i in range(N):
        w, z = [], Decimal(0)
        for j in range(N):
            if vis(i, j):
                e = (Decimal(float(scale)) * sum(Decimal(float(q[i, c])) * Decimal(float(k[j, c]))
                                                 for c in range(d))).exp()
                w.append((j, e))
                z += e
        if not w:
            L[i] = -math.inf
            continue
        for c in range(d):
            O[i, c] = float(sum(e * Decimal(float(v[j, c])) for j, e in w) / z)
        L[i] = float(z.ln())
    return O, L


def pins_fail(orc) -> list:
    """Names of the pins the given oracle build fails (empty list: all pass)."""
    rng = np.random.default_rng(77)
    failed = []

    def close(a, b, tol):
        a, b = np.asarray(a), np.asarray(b)
        if a.shape != b.shape:
            return False
        fa, fb = np.isfinite(a), np.isfinite(b)
        if not np.array_equal(fa, fb) or not np.array_equal(a[~fa], b[~fb]):
            return False
        return bool(np.all(np.abs(a[fa] - b[fb]) <= tol))

    N, d = 6, 3
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    for causal in (False, True):
        o, lse = orc.forward(q, k, v, 0.7, causal)
        ob, lb = brute(q, k, v, 0.7, (lambda i, j: j <= i) if causal else (lambda i, j: True))
        if not (close(o, ob, 1e-12) and close(lse, lb, 1e-12)):
            failed.append(f"brute_force_causal={causal}")
    mask = (rng.random((N, N)) < 0.6).astype(np.uint8)
    mask[2] = 0
    mask[0, 3] = 1
    o, lse = orc.forward(q, k, v, 0.5, False, mask, 1)
    ob, lb = brute(q, k, v, 0.5, lambda i, j: bool(mask[i, j]))
    if not (close(o, ob, 1e-12) and close(lse, lb, 1e-12)):
        failed.append("brute_force_mask")
    # closed form: equal scores
    o, lse = orc.forward(np.zeros((N, d)), k, v, 0.3, True)
    if not (close(o, np.cumsum(v, 0) / np.arange(1, N + 1)[:, None], 1e-13)
            and close(lse, np.log(np.arange(1, N + 1)), 1e-13)):
        failed.append("equal_scores")
    # backward: finite differences of sum(dO * O)
    for causal in (False, True):
        dq, dk, dv = orc.backward(q, k, v, do, 0.6, causal)
        h, worst = 1e-6, 0.0
        for which, g in ((0, dq), (1, dk), (2, dv)):
            for idx in np.ndindex(N, d):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                lp = float(np.sum(do * orc.forward(*args, 0.6, causal)[0]))
                args[which][idx] -= 2 * h
                lm = float(np.sum(do * orc.forward(*args, 0.6, causal)[0]))
                worst = max(worst, abs((lp - lm) / (2 * h) - g[idx]))
        if not worst < 1e-6:
            failed.append(f"finite_differences_causal={causal}")
    return failed


def test_real_oracle_passes_every_pin():
    tmp = tempfile.mkdtemp()
    try:
        assert pins_fail(Oracle(build(open(SRC).read(), tmp))) == []
    finally:
        shutil.rmtree(tmp)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    text = open(SRC).read()
    assert old in text, f"mutation site for {name} not found in oracle.c"
    tmp = tempfile.mkdtemp()
    try:
        lib = build(text.replace(old, new, 1), tmp)
        failed = pins_fail(Oracle(lib))
    finally:
        shutil.rmtree(tmp)
    assert failed, f"no pin catches the planted mistake {name}"


# ------------------------------------------ grouped K/V heads (oracle/__init__.py)
PY_MUTANTS = [
    ("gqa_heads_tiled", "np.repeat(k, g, axis=-3), np.repeat(v, g, axis=-3), scale, causal,\n"
     "                   threads=threads)",
     "np.concatenate([k] * g, axis=-3), np.concatenate([v] * g, axis=-3), scale, causal,\n"
     "                   threads=threads)"),
    ("gqa_group_sum_transposed", "shape = k.shape[:-3] + (k.shape[-3], g) + k.shape[-2:]\n"
     "    return dq, dk.reshape(shape).sum(axis=-3), dv.reshape(shape).sum(axis=-3), lse, delta",
     "shape = k.shape[:-3] + (g, k.shape[-3]) + k.shape[-2:]\n"
     "    return dq, dk.reshape(shape).sum(axis=-4), dv.reshape(shape).sum(axis=-4), lse, delta"),
    ("gqa_dk_not_summed", "dk.reshape(shape).sum(axis=-3), dv.reshape",
     "dk.reshape(shape)[..., 0, :, :], dv.reshape"),
]


def load_oracle_package(init_text, tmp):
    import importlib.util
    import sys
    pkg = os.path.join(tmp, "oracle_mut")
    os.makedirs(pkg)
    shutil.copy(SRC, os.path.join(pkg, "oracle.c"))
    with open(os.path.join(pkg, "__init__.py"), "w") as f:
        f.write(init_text)
    spec = importlib.util.spec_from_file_location("oracle_mut", os.path.join(pkg, "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    sys.modules.pop("oracle_mut", None)
    spec.loader.exec_module(mod)
    return mod


def gqa_pins_fail(orc) -> list:
    rng = np.random.default_rng(5)
    failed = []
    B, H, Hkv, N, d = 1, 4, 2, 4, 2
    q, do = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))
    k, v = rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hkv, N, d))
    o, _ = orc.forward_gqa(q, k, v, 0.9, True)
    for h in range(H):
        ob, _ = brute(q[0, h], k[0, h // 2], v[0, h // 2], 0.9, lambda i, j: j <= i)
        if not np.allclose(o[0, h], ob, rtol=0, atol=1e-12):
            failed.append("brute_force")
            break
    _, dk, dv, _, _ = orc.backward_gqa(q, k, v, do, 0.9, True)
    eps, worst = 1e-6, 0.0
    for which, g in ((1, dk), (2, dv)):
        for idx in np.ndindex(*g.shape):
            args = [q, k.copy(), v.copy()]
            args[which][idx] += eps
            lp = float(np.sum(do * orc.forward_gqa(*args, 0.9, True)[0]))
            args[which][idx] -= 2 * eps
            lm = float(np.sum(do * orc.forward_gqa(*args, 0.9, True)[0]))
            worst = max(worst, abs((lp - lm) / (2 * eps) - g[idx]))
    if not worst < 1e-6:
        failed.append("finite_differences")
    return failed


INIT = os.path.join(ROOT, "oracle", "__init__.py")


def test_real_gqa_oracle_passes_its_pins():
    tmp = tempfile.mkdtemp()
    try:
        assert gqa_pins_fail(load_oracle_package(open(INIT).read(), tmp)) == []
    finally:
        shutil.rmtree(tmp)


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_gqa_mutant_is_caught(name, old, new):
    text = open(INIT).read()
    assert old in text, f"mutation site for {name} not found in oracle/__init__.py"
    tmp = tempfile.mkdtemp()
    try:
        failed = gqa_pins_fail(load_oracle_package(text.replace(old, new, 1), tmp))
    finally:
        shutil.rmtree(tmp)
    assert failed, f"no pin catches the planted mistake {name}"
