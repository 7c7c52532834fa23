"""CPU emulation of the generated key loop of the d = 128 dQ kernel.

The instruction text that gen_bwd_dq128.py emits (fa_bwd_dq128_loop.inc) is
executed for the four waves of one workgroup by the emulator in _emu.py.
The setup (registers, and K, V tiles 0 and 1 staged before the loop)
restates the C++ of fa_bwd_dq128.hip; L = LSE log2(e) and D come from the
oracle's forward statistics, rounded to fp32 and (D) negated as the delta
pass stores them.
dQ is scaled as the kernel's epilogue does and compared with the fp64
oracle at the bf16 tolerances; the sequence of loop bodies each tile step
takes is checked against the rule that selects them.
"""
import importlib.util
import os

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_45_amd import inputs
from _emu import Machine, Memory, Program, bf16_bits, tile_swz

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", "gen_bwd_dq128.py")
spec = importlib.util.spec_from_file_location("gen_bwd_dq128_emu", GEN)
G = importlib.util.module_from_spec(spec)
spec.loader.exec_module(G)
LINES = G.generate()
PROGRAM = Program(LINES, ("FQ_BODY", "FQ_GB", "FQ_ITM", "FQ_FIN"))
D, BC, BR = 128, 64, 256
LOG2E = 1.4426950408889634


def item_shape(N, q0, causal):
    nt = -(-N // BC)
    qmax = min(q0 + BR, N) - 1
    tend = min(nt, qmax // BC + 1) if causal else nt
    ragged = N % BC != 0
    fm = tend
    if causal:
        fm = min(fm, q0 // BC)
    if ragged:
        fm = min(fm, nt - 1)
    return nt, tend, ragged, fm


def expected_bodies(N, q0, causal):
    """Straight body while tile j + 1 needs no mask and tile j + 2 loads whole;
    the masked body when tile j + 1 needs a mask; the general one otherwise;
    the final one last."""
    nt, tend, ragged, fm = item_shape(N, q0, causal)
    out = []
    for j in range(tend - 1):
        whole = j + 2 < tend and not (ragged and j + 2 == nt - 1)
        out.append("ITM" if j + 1 >= fm else "BODY" if whole else "GB")
    return out + ["FIN"]


def emulate_dq(q, k, v, do, lse2, delta, N, q0, causal, scale):
    """dQ [256, 128] (float64, rows past N left 0) of the workgroup whose rows
    start at q0 (one head)."""
    KBASE, VBASE = 0x10000000, 0x20000000
    kb = bf16_bits(k).astype(np.uint16).reshape(-1).view(np.uint8).copy()
    vb = bf16_bits(v).astype(np.uint16).reshape(-1).view(np.uint8).copy()
    mem = Memory([(KBASE, kb), (VBASE, vb)])
    lds = np.zeros(98304, np.uint8)
    TILE = BC * D
    nt, tend, ragged, fm = item_shape(N, q0, causal)
    tail = ragged and tend == nt
    tlast = tend - 1
    c = np.float32(scale * LOG2E)
    qbits, dobits = bf16_bits(q), bf16_bits(do)

    def stage_tile(buf, t, stage_byte):   # the kernel's dma_tile, all waves
        rows = min(BC, N - t * BC)
        for w in range(4):
            for i in range(4):
                for lane in range(64):
                    row = 16 * w + 4 * i + (lane >> 4)
                    col = 8 * ((lane & 15) ^ tile_swz(row))
                    src = (t * TILE + min(row, rows - 1) * D + col) * 2
                    dst = stage_byte + 4096 * w + 1024 * i + 16 * lane
                    lds[dst:dst + 16] = buf[src:src + 16]

    stage_tile(kb, 0, G.kst(0))
    stage_tile(vb, 0, G.vst(0))
    if tend > 1:
        stage_tile(kb, 1, G.kst(1))
        stage_tile(vb, 1, G.vst(1))
    f = max(fm - 1, 0)
    waves = []
    for w in range(4):
        m = Machine()
        wrow0 = q0 + 64 * w
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            for rb in range(2):
                r = min(wrow0 + 32 * rb + l32, N - 1)
                for cc in range(8):
                    for base, bits in ((G.QT_BASE, qbits), (G.DOT_BASE, dobits)):
                        e = bits[r, 16 * cc + 8 * h:16 * cc + 8 * h + 8]
                        for t in range(4):
                            m.a[base + 32 * rb + 4 * cc + t, lane] = e[2 * t] | (e[2 * t + 1] << 16)
                m.v[G.LSEL + rb, lane] = np.float32(lse2[r]).view(np.uint32)
                m.v[G.DDEL + rb, lane] = np.float32(-delta[r]).view(np.uint32)   # stored negated
                row = wrow0 + 32 * rb + l32
                lim = min(row, N - 1) if causal else N - 1
                m.v[G.THR1 + rb, lane] = np.uint32((lim - 4 * h - BC * f) & 0xFFFFFFFF)
                m.v[G.THR + rb, lane] = np.uint32((lim - 4 * h - BC * (f + 1)) & 0xFFFFFFFF)
            sw_row = tile_swz(l32)
            for cc in range(8):
                ra = l32 * 256 + 16 * ((2 * cc + h) ^ sw_row)
                m.v[G.RADDR + cc, lane] = ra
                m.v[G.VRADDR + cc, lane] = ra + G.V_STAGE0
            tr_row = 4 * h + ((lane & 15) >> 2)
            tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
            sw_lo, sw_hi = tile_swz(tr_row), tile_swz(tr_row + 8)
            tq, te = tr_col >> 3, tr_col & 7

            def tr_off(row, sw, b):
                return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te
            for db in range(4):
                m.v[G.TADDR + 2 * db, lane] = 2 * tr_off(tr_row, sw_lo, db)
                m.v[G.TADDR + 2 * db + 1, lane] = 2 * tr_off(tr_row + 8, sw_hi, db)
            for i in range(4):
                row = 16 * w + 4 * i + (lane >> 4)
                col = 8 * ((lane & 15) ^ tile_swz(row))
                m.v[G.GOFF + i, lane] = (row * D + col) * 2 - 1024 * i
                m.v[G.GOFF_TAIL + i, lane] = ((min(tlast * BC + row, N - 1) - tlast * BC) * D
                                              + col) * 2
        m.v[G.NINF] = np.full(64, -np.inf, np.float32).view(np.uint32)
        kp, vp = KBASE + 2 * TILE * 2, VBASE + 2 * TILE * 2
        m.s[G.S_KPTR], m.s[G.S_KPTR + 1] = kp & 0xFFFFFFFF, kp >> 32
        m.s[G.S_VPTR], m.s[G.S_VPTR + 1] = vp & 0xFFFFFFFF, vp >> 32
        m.s[G.S_M0K] = 4096 * w
        m.s[G.S_M0V] = G.V_STAGE0 + 4096 * w
        m.s[G.S_C] = int(c.view(np.uint32))
        m.s[G.S_LAST] = tend - 1
        m.s[G.S_KEND] = max(0, tend - 2)
        m.s[G.S_TAILJ] = nt - 3 if tail and nt >= 3 else 0xFFFFFFFF
        m.s[G.S_FM] = fm
        m.s[G.S_FAST] = max(0, min(fm - 1, (nt - 1 if tail else tend) - 2))
        m.s[G.S_J] = 0
        waves.append(m)
    PROGRAM.run_workgroup(waves, lds, mem)
    dq = np.zeros((BR, D))
    for w, m in enumerate(waves):
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            for rb in range(2):
                acc = m.a[G.DQ_BASE + 64 * rb:G.DQ_BASE + 64 * rb + 64, lane].view(np.float32)
                for db in range(4):
                    for r in range(16):
                        d = 32 * db + 8 * (r // 4) + 4 * h + r % 4
                        dq[64 * w + 32 * rb + l32, d] = float(acc[16 * db + r]) * scale
    return dq


CASES = [
    # (N, q0, causal): entry mask, tails, diagonals, straight / general /
    # masked / final bodies, every tile index modulo 4
    (40, 0, False),
    (100, 0, True),
    (130, 0, False),
    (300, 256, True),
    (512, 0, False),
    (700, 0, False),
    (700, 512, True),
    (1024, 512, True),
]


@pytest.mark.parametrize("N,q0,causal", CASES)
def test_generated_dq_loop_matches_the_oracle(N, q0, causal):
    q, k, v = (t[0, 0].float().numpy() for t in inputs.qkv(1, 1, N, D, torch.bfloat16,
                                                             seed=N + q0 + int(causal)))
    do = inputs.qkv(1, 1, N, D, torch.bfloat16, seed=N + q0 + 7)[0][0, 0].float().numpy()
    scale = D ** -0.5
    rdq, _, _, rlse, rdelta = oracle.backward(q[None], k[None], v[None], do[None], scale, causal)
    lse2 = (rlse[0].astype(np.float32) * np.float32(LOG2E)).astype(np.float32)
    delta = rdelta[0].astype(np.float32)
    PROGRAM.bodies_run.clear()
    dq = emulate_dq(q, k, v, do, lse2, delta, N, q0, causal, scale)
    assert [b[3:] for b in PROGRAM.bodies_run] == expected_bodies(N, q0, causal), PROGRAM.bodies_run
    rows = np.arange(q0, min(q0 + BR, N))
    err = np.abs(dq[rows - q0] - rdq[0][rows])
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
