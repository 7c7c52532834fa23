"""CPU emulation of the generated query loop of the d = 128 dK/dV kernel.

The instruction text that gen_bwd_dkdv128.py emits (fa_bwd_dkdv128_loop.inc)
is executed for the four waves of one workgroup by the emulator in _emu.py.
The setup (registers, and the Q, dO tiles and L, D values staged before the
loop) restates the C++ of fa_bwd_dkdv128.hip; L = LSE log2(e) and D come from
the oracle's forward statistics, rounded to fp32 and (D) negated as the delta
pass stores them.  dK is scaled as the kernel's epilogue does; dK and dV are compared
with the fp64 oracle at the bf16 tolerances, and the sequence of loop bodies
each query tile step takes is checked against the rule that selects them.
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
GEN = os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", "gen_bwd_dkdv128.py")
spec = importlib.util.spec_from_file_location("gen_bwd_dkdv128_emu", GEN)
G = importlib.util.module_from_spec(spec)
spec.loader.exec_module(G)
LINES = G.generate()
PROGRAM = Program(LINES, ("FK_BODY", "FK_GB", "FK_ITM", "FK_FIN"))
D, BQ, BK = 128, 64, 128
LOG2E = 1.4426950408889634


def item_shape(N, k0, causal):
    nt = -(-N // BQ)
    ts = k0 // BQ if causal else 0
    cnt = nt - ts
    ragged = N % BQ != 0
    mlo = 2 if causal else 0
    mhi = cnt - 1 if ragged else cnt
    return nt, ts, cnt, ragged, mlo, mhi


def expected_bodies(N, k0, causal):
    """Straight body while tiles j and j + 1 need no mask and tile j + 3
    loads whole; the masked body when either needs a mask; the general one
    otherwise; the final one last."""
    nt, ts, cnt, ragged, mlo, mhi = item_shape(N, k0, causal)
    out = []
    for j in range(cnt - 1):
        if mlo <= j < mhi - 3:
            out.append("BODY")
        elif j < mlo or j + 1 >= mhi:
            out.append("ITM")
        else:
            out.append("GB")
    return out + ["FIN"]


def emulate_dkdv(q, k, v, do, lse2, delta, N, k0, causal, scale, acc=None):
    """dK, dV [128, 128] (float64, keys past N left 0) of the workgroup whose
    keys start at k0 (one head), and the four waves' accumulation registers
    after the statement.  acc: those registers from a previous run of the
    statement (another query head of the group), which the kernel passes in
    unchanged; zero when None."""
    QBASE, OBASE, LBASE, DBASE = 0x10000000, 0x20000000, 0x30000000, 0x40000000
    qb = bf16_bits(q).astype(np.uint16).reshape(-1).view(np.uint8).copy()
    ob = bf16_bits(do).astype(np.uint16).reshape(-1).view(np.uint8).copy()
    lb = np.asarray(lse2, np.float32).view(np.uint8).copy()
    db_ = np.asarray(-delta, np.float32).view(np.uint8).copy()   # the delta pass stores -D
    mem = Memory([(QBASE, qb), (OBASE, ob), (LBASE, lb), (DBASE, db_)])
    lds = np.zeros(139264, np.uint8)
    TILE = BQ * D
    nt, ts, cnt, ragged, mlo, mhi = item_shape(N, k0, causal)
    tlast = nt - 1
    c = np.float32(scale * LOG2E)
    kbits, vbits = bf16_bits(k), bf16_bits(v)

    def stage_tile(buf, t, stage_byte):   # the kernel's dma_tile128, all waves
        rows = min(BQ, N - t * BQ)
        for w in range(4):
            for i in range(4):
                for lane in range(64):
                    row = 16 * w + 4 * i + (lane >> 4)
                    col = 8 * ((lane & 15) ^ tile_swz(row))
                    src = (t * TILE + min(row, rows - 1) * D + col) * 2
                    dst = stage_byte + 4096 * w + 1024 * i + 16 * lane
                    lds[dst:dst + 16] = buf[src:src + 16]

    def stage_vec(vec, t, byte):           # the kernel's dma_vec64, one wave
        rows = np.minimum(t * BQ + np.arange(64), N - 1)
        lds[byte:byte + 256] = np.asarray(vec, np.float32)[rows].view(np.uint8)

    for s in range(min(3, cnt)):
        stage_tile(qb, ts + s, G.Q_STAGE * s)
        stage_tile(ob, ts + s, G.O_STAGE0 + G.Q_STAGE * s)
        for w in range(4):
            stage_vec(lse2, ts + s, G.L_STAGE0 + G.LD_STAGE * s + 512 * w)
            stage_vec(-delta, ts + s, G.L_STAGE0 + G.LD_STAGE * s + 512 * w + 256)
    waves = []
    for w in range(4):
        m = Machine()
        if acc is not None:
            m.a[G.DK_BASE:G.DV_BASE + 64] = acc[w]
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            key = k0 + 32 * w + l32
            kr = min(key, N - 1)
            for cc in range(8):
                for base, bits in ((G.KB_BASE, kbits), (G.VB_BASE, vbits)):
                    e = bits[kr, 16 * cc + 8 * h:16 * cc + 8 * h + 8]
                    for t in range(4):
                        m.a[base + 4 * cc + t, lane] = e[2 * t] | (e[2 * t + 1] << 16)
            sw_row = tile_swz(l32)
            for cc in range(8):
                ra = l32 * 256 + 16 * ((2 * cc + h) ^ sw_row)
                m.v[G.RADDR + cc, lane] = ra
                m.v[G.DRADDR + cc, lane] = ra + G.O_STAGE0
            tr_row = 4 * h + ((lane & 15) >> 2)
            tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
            sw_lo, sw_hi = tile_swz(tr_row), tile_swz(tr_row + 8)
            tq, te = tr_col >> 3, tr_col & 7

            def tr_off(row, sw, b):
                return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te
            for dbk in range(4):
                for hi, (row, sw) in enumerate(((tr_row, sw_lo), (tr_row + 8, sw_hi))):
                    m.v[G.TADDR + 2 * dbk + hi, lane] = 2 * tr_off(row, sw, dbk)
                    m.v[G.TDADDR + 2 * dbk + hi, lane] = 2 * tr_off(row, sw, dbk) + G.O_STAGE0
            m.v[G.LADDR, lane] = G.L_STAGE0 + 512 * w + 16 * h
            for i in range(4):
                row = 16 * w + 4 * i + (lane >> 4)
                col = 8 * ((lane & 15) ^ tile_swz(row))
                m.v[G.GOFF + i, lane] = (row * D + col) * 2 - 1024 * i
                m.v[G.GOFF_TAIL + i, lane] = ((min(tlast * BQ + row, N - 1) - tlast * BQ) * D
                                              + col) * 2
            m.v[G.LOFF, lane] = 4 * lane
            m.v[G.LOFF_TAIL, lane] = 4 * (min(tlast * BQ + lane, N - 1) - tlast * BQ)
            base = key if causal else 0
            m.v[G.TA, lane] = np.uint32((base - 4 * h - BQ * ts) & 0xFFFFFFFF)
            m.v[G.RANGE, lane] = max(N - base, 0)
        m.v[G.NINF] = np.full(64, -np.inf, np.float32).view(np.uint32)
        for reg, addr in ((G.S_QPTR, QBASE + 2 * TILE * (ts + 3)),
                          (G.S_OPTR, OBASE + 2 * TILE * (ts + 3)),
                          (G.S_LPTR, LBASE + 4 * BQ * (ts + 3)),
                          (G.S_DPTR, DBASE + 4 * BQ * (ts + 3) - 256)):
            m.s[reg], m.s[reg + 1] = addr & 0xFFFFFFFF, addr >> 32
        m.s[G.S_M0Q] = 4096 * w
        m.s[G.S_M0O] = G.O_STAGE0 + 4096 * w
        m.s[G.S_M0L] = G.L_STAGE0 + 512 * w
        m.s[G.S_C] = int(c.view(np.uint32))
        m.s[G.S_LAST] = cnt - 1
        m.s[G.S_KEND] = max(0, cnt - 3)
        m.s[G.S_TAILJ] = cnt - 4 if ragged and cnt >= 4 else 0xFFFFFFFF
        m.s[G.S_MLO] = mlo
        m.s[G.S_MHI] = mhi
        m.s[G.S_FAST] = max(0, mhi - 3)
        m.s[G.S_MASK0] = 1 if (mlo > 0 or mhi == 0) else 0
        m.s[G.S_J] = 0
        waves.append(m)
    PROGRAM.run_workgroup(waves, lds, mem)
    dk = np.zeros((BK, D))
    dv = np.zeros((BK, D))
    for w, m in enumerate(waves):
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            ak = m.a[G.DK_BASE:G.DK_BASE + 64, lane].view(np.float32)
            av = m.a[G.DV_BASE:G.DV_BASE + 64, lane].view(np.float32)
            for dbk in range(4):
                for r in range(16):
                    d = 32 * dbk + 8 * (r // 4) + 4 * h + r % 4
                    dk[32 * w + l32, d] = float(ak[16 * dbk + r]) * scale
                    dv[32 * w + l32, d] = float(av[16 * dbk + r])
    return dk, dv, [m.a[G.DK_BASE:G.DV_BASE + 64].copy() for m in waves]


CASES = [
    # (N, k0, causal): entry mask, partial tiles and key blocks, diagonals,
    # straight / general / masked / final bodies, every tile index modulo 4
    (40, 0, False),
    (100, 0, True),
    (130, 0, False),
    (300, 128, True),
    (512, 0, False),
    (700, 0, False),
    (700, 640, True),
    (704, 256, True),
    (1024, 384, True),
]


@pytest.mark.parametrize("N,k0,causal", CASES)
def test_generated_dkdv_loop_matches_the_oracle(N, k0, causal):
    q, k, v = (t[0, 0].float().numpy() for t in inputs.qkv(1, 1, N, D, torch.bfloat16,
                                                             seed=N + k0 + int(causal)))
    do = inputs.qkv(1, 1, N, D, torch.bfloat16, seed=N + k0 + 7)[0][0, 0].float().numpy()
    scale = D ** -0.5
    _, rdk, rdv, rlse, rdelta = oracle.backward(q[None], k[None], v[None], do[None], scale, causal)
    lse2 = (rlse[0].astype(np.float32) * np.float32(LOG2E)).astype(np.float32)
    delta = rdelta[0].astype(np.float32)
    PROGRAM.bodies_run.clear()
    dk, dv, _ = emulate_dkdv(q, k, v, do, lse2, delta, N, k0, causal, scale)
    assert [b[3:] for b in PROGRAM.bodies_run] == expected_bodies(N, k0, causal), PROGRAM.bodies_run
    keys = np.arange(k0, min(k0 + BK, N))
    for got, ref in ((dk, rdk[0]), (dv, rdv[0])):
        err = np.abs(got[keys - k0] - ref[keys])
        tol = 2e-2 * max(1.0, float(np.abs(ref[keys]).max()))
        assert err.max() <= tol and err.mean() <= tol / 10, (err.max(), err.mean(), tol)


@pytest.mark.parametrize("N,k0,causal", [(300, 128, True), (330, 0, False)])
def test_grouped_heads_accumulate_over_statements(N, k0, causal):
    """Grouped K/V heads: the kernel runs the statement once per query head
    of the group, passing the accumulators on; the sum over two query heads
    matches the oracle's grouped-head dK, dV (one K/V parameter used twice)."""
    q2, _, _ = (t[0].float().numpy() for t in inputs.qkv(1, 2, N, D, torch.bfloat16, seed=N + 11))
    _, k, v = (t[0, 0].float().numpy() for t in inputs.qkv(1, 1, N, D, torch.bfloat16, seed=N + 12))
    do2 = inputs.qkv(1, 2, N, D, torch.bfloat16, seed=N + 13)[0][0].float().numpy()
    scale = D ** -0.5
    _, rdk, rdv, rlse, rdelta = oracle.backward_gqa(q2, k[None], v[None], do2, scale, causal)
    acc = None
    for g in range(2):
        lse2 = (rlse[g].astype(np.float32) * np.float32(LOG2E)).astype(np.float32)
        dk, dv, acc = emulate_dkdv(q2[g], k, v, do2[g], lse2, rdelta[g].astype(np.float32), N, k0,
                                   causal, scale, acc)
    keys = np.arange(k0, min(k0 + BK, N))
    for got, ref in ((dk, rdk[0]), (dv, rdv[0])):
        err = np.abs(got[keys - k0] - ref[keys])
        tol = 2e-2 * max(1.0, float(np.abs(ref[keys]).max()))
        assert err.max() <= tol and err.mean() <= tol / 10, (err.max(), err.mean(), tol)
