"""CPU emulation of the generated key loops of the d = 128 and d = 64
forward kernels.

The instruction text that gen_fwd128.py emits (fa_fwd128_loop.inc,
fa_fwd64_loop.inc, and fa_fwd64w2_loop.inc for 2-wave workgroups) is
executed for the waves of one workgroup by the emulator in _emu.py (registers, LDS, bounds-checked K/V buffers, barriers).
The setup (registers and the three tiles staged before the loop) restates
the C++ of fa_fwd128.hip / fa_fwd64.hip.  The output is normalised as the kernel's epilogue does and
compared with the fp64 oracle at the bf16 tolerances.  Hazards and timing
are not modelled (test_fwd128_schedule.py checks those on the text).
"""
import importlib.util
import os

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_45_amd import inputs
from _emu import Machine, Memory, Program, bf16_bits, bf16_to_f32

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", "gen_fwd128.py")
BC = 64
# generated loops: head dim and waves per workgroup ("64w2": d = 64, 2 waves)
VARIANTS = {128: (128, 4), 64: (64, 4), "64w2": (64, 2)}


def load_gen(d, nw):
    spec = importlib.util.spec_from_file_location(f"gen_fwd_emu{d}w{nw}", GEN)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.configure(d, nw)
    return mod


GENS = {key: load_gen(*dn) for key, dn in VARIANTS.items()}
PROGRAMS = {key: Program(G.generate(), ("FA_BODY", "FA_GB", "FA_ITM", "FA_FIN", "FA_IDLEA",
                                        "FA_IDLEB"), "FA_SLOW")
            for key, G in GENS.items()}


def swz_of(D):
    """The kernels' chunk swizzle of an LDS tile row (tile_swz in fa_common.hpp)."""
    if D == 128:
        return lambda r: 4 * (r & 3) + ((r >> 2) & 3)
    return lambda r: 4 * ((r >> 1) & 1) + ((r >> 2) & 3)


def emulate_workgroup(q, k, v, N, q0, causal, scale, key=128):
    """Run the generated loop `key` for the workgroup whose rows start at q0
    (one head); returns O [64 NW, D] (float64, rows past N left 0) and LSE."""
    D, NW = VARIANTS[key]
    G, PROGRAM, tile_swz = GENS[key], PROGRAMS[key], swz_of(D)
    BR = 64 * NW
    NC, NDB, NLOAD = D // 16, D // 32, 64 * D * 2 // 1024 // NW
    LPR = D // 8             # lanes (16-byte chunks) per tile row in a direct load
    RW = 64 // NW            # tile rows each wave loads
    KBASE, VBASE = 0x10000000, 0x20000000
    kb = bf16_bits(k).astype(np.uint16).reshape(-1).view(np.uint8).copy()
    vb = bf16_bits(v).astype(np.uint16).reshape(-1).view(np.uint8).copy()
    mem = Memory([(KBASE, kb), (VBASE, vb)])
    lds = np.zeros(65536, np.uint8)
    TILE = BC * D
    nt = -(-N // BC)
    qmax = min(q0 + BR, N) - 1
    tend = min(nt, qmax // BC + 1) if causal else nt
    ragged = N % BC != 0
    fm = tend
    if causal:
        fm = min(fm, q0 // BC)
    if ragged:
        fm = min(fm, nt - 1)
    tlast = tend - 1
    sl2 = np.float32(scale * 1.4426950408889634)
    qbits = bf16_bits(q)

    def load_tile(buf, t, stage_byte):        # the C++ prologue's tile loads, all waves
        for row in range(BC):
            for slot in range(LPR):
                qq = slot ^ tile_swz(row)
                src = (min(t * BC + row, N - 1) * D + 8 * qq) * 2
                dst = stage_byte + row * 2 * D + 16 * slot
                lds[dst:dst + 16] = buf[src:src + 16]

    load_tile(kb, 0, 2 * TILE * 2)
    load_tile(vb, 0, 0)
    if tend > 1:
        load_tile(kb, 1, 3 * TILE * 2)
    waves = []
    for w in range(NW):
        m = Machine()
        wrow0 = q0 + 64 * w
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            for rb in range(2):
                r = min(wrow0 + 32 * rb + l32, N - 1)
                for c in range(NC):
                    e = qbits[r, 16 * c + 8 * h:16 * c + 8 * h + 8]
                    for t in range(4):
                        m.a[G.Q_BASE + 4 * NC * rb + 4 * c + t, lane] = e[2 * t] | (e[2 * t + 1] << 16)
            sw_row = tile_swz(l32)
            for c in range(NC):
                m.v[G.KADDR + c, lane] = 2 * (2 * TILE + l32 * D + 8 * ((2 * c + h) ^ sw_row))
            tr_row = 4 * h + ((lane & 15) >> 2)
            tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
            sw_lo, sw_hi = tile_swz(tr_row), tile_swz(tr_row + 8)
            tq, te = tr_col >> 3, tr_col & 7

            def tr_off(row, sw, b):
                return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te
            for db in range(NDB):
                m.v[G.VADDR + 2 * db, lane] = 2 * tr_off(tr_row, sw_lo, db)
                m.v[G.VADDR + 2 * db + 1, lane] = 2 * tr_off(tr_row + 8, sw_hi, db)
            for i in range(NLOAD):
                row = RW * w + (RW // NLOAD) * i + lane // LPR
                col = 8 * ((lane % LPR) ^ tile_swz(row))
                m.v[G.GOFF + i, lane] = (row * D + col) * 2 - 1024 * i
                m.v[G.GOFF_TAIL + i, lane] = ((min(tlast * BC + row, N - 1) - tlast * BC) * D
                                              + col) * 2
            for rb in range(2):
                row = wrow0 + 32 * rb + l32
                lim = min(row, N - 1) if causal else N - 1
                m.v[G.THR + rb, lane] = np.uint32((lim - 4 * h - BC * fm) & 0xFFFFFFFF)
            m.v[G.BPERM, lane] = (lane ^ 32) << 2
        m.v[G.NINF] = np.full(64, -np.inf, np.float32).view(np.uint32)
        kp, vp = KBASE + 2 * TILE * 2, VBASE + TILE * 2
        m.s[G.S_KPTR], m.s[G.S_KPTR + 1] = kp & 0xFFFFFFFF, kp >> 32
        m.s[G.S_VPTR], m.s[G.S_VPTR + 1] = vp & 0xFFFFFFFF, vp >> 32
        m.s[G.S_M0K] = 2 * TILE * 2 + w * RW * D * 2
        m.s[G.S_M0V] = w * RW * D * 2
        m.s[G.S_C] = int(np.float32(sl2).view(np.uint32))
        tail = ragged and tend == nt
        m.s[G.S_LAST] = tend - 1
        m.s[G.S_KEND] = max(0, tend - 2)
        m.s[G.S_KTAILJ] = nt - 3 if tail and nt >= 3 else 0xFFFFFFFF
        m.s[G.S_VTAILJ] = nt - 2 if tail and nt >= 2 else 0xFFFFFFFF
        m.s[G.S_FM] = fm
        m.s[G.S_FAST] = max(0, min(fm - 1, (nt - 1 if tail else tend) - 2))
        m.s[G.S_WDIAG] = wave_last_tile(N, q0, w, tend, causal)
        m.s[G.S_J] = 0
        waves.append(m)
    PROGRAM.run_workgroup(waves, lds, mem)
    O = np.zeros((BR, D))
    L = np.full(BR, np.nan)
    for w, m in enumerate(waves):
        lsum = m.v[G.LSUM:G.LSUM + 2].view(np.float32)
        mref = -m.v[G.MNEG:G.MNEG + 2].view(np.float32)
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            for rb in range(2):
                row = 64 * w + 32 * rb + l32
                ltot = float(lsum[rb, lane]) + float(lsum[rb, lane ^ 32])
                L[row] = (float(mref[rb, lane]) + np.log2(ltot)) * np.log(2.0)
                acc = m.a[G.O_BASE + 16 * NDB * rb:G.O_BASE + 16 * NDB * (rb + 1), lane].view(np.float32)
                for db in range(NDB):
                    for r in range(16):
                        d = 32 * db + 8 * (r // 4) + 4 * h + r % 4
                        O[row, d] = acc[16 * db + r] / ltot
    return O, L


CASES = [
    # (N, q0, causal, key scale from key 192 on): entry mask, tail, diagonal,
    # final-only and slow-path cases
    (40, 0, False, 1.0),
    (100, 0, True, 1.0),
    (300, 256, True, 1.0),
    (700, 0, False, 1.0),
    (700, 512, True, 1.0),
    (600, 256, False, 3.0),
    (520, 256, True, 3.0),
    (512, 0, False, 1.0),
    (130, 0, False, 1.0),
    (1024, 512, True, 1.0),
]


def wave_last_tile(N, q0, w, tend, causal):
    """The last tile holding a key wave w sees (the kernel's formula)."""
    return min(tend - 1, min(q0 + 64 * w + 63, N - 1) // BC) if causal else tend - 1


def expected_bodies(N, q0, causal, w=0, BR=256):
    """Which body each tile step of wave w should take: straight while the
    next tile is unmasked and both loads are whole tiles, the masked body
    when the next tile needs a mask, the general one otherwise, the final
    one last; idle past the wave's last visible tile."""
    nt = -(-N // BC)
    qmax = min(q0 + BR, N) - 1
    tend = min(nt, qmax // BC + 1) if causal else nt
    ragged = N % BC != 0
    fm = tend
    if causal:
        fm = min(fm, q0 // BC)
    if ragged:
        fm = min(fm, nt - 1)
    last = wave_last_tile(N, q0, w, tend, causal)
    out = []
    for j in range(tend - 1):
        k_whole = j + 2 < tend and not (ragged and j + 2 == nt - 1)
        v_whole = not (ragged and j + 1 == nt - 1)
        if j > last:
            out.append("IDLE")
        elif j + 1 >= fm:
            out.append("ITM")
        elif k_whole and v_whole:
            out.append("BODY")
        else:
            out.append("GB")
    return out + ["IDLE" if tend - 1 > last else "FIN"]


@pytest.mark.parametrize("key", list(VARIANTS))
@pytest.mark.parametrize("N,q0,causal,kscale", CASES)
def test_generated_loop_matches_the_oracle(N, q0, causal, kscale, key):
    D, NW = VARIANTS[key]
    BR = 64 * NW
    q, k, v = (t[0, 0].float().numpy() for t in inputs.qkv(1, 1, N, D, torch.bfloat16,
                                                             seed=N + q0 + int(causal)))
    PROGRAM = PROGRAMS[key]
    if kscale != 1.0:
        k[192:] *= kscale
        k = bf16_to_f32(bf16_bits(k))
    scale = D ** -0.5
    PROGRAM.slow_taken = 0
    PROGRAM.bodies_run.clear()
    PROGRAM.bodies_by_wave.clear()
    O, L = emulate_workgroup(q, k, v, N, q0, causal, scale, key)
    for w in range(NW):
        got = [b[3:7] if b.startswith("FA_IDLE") else b[3:] for b in PROGRAM.bodies_by_wave[w]]
        assert got == expected_bodies(N, q0, causal, w, BR), (w, got)
    # keys scaled by 3 from key 192 on lift those tiles' weights far past 2^8
    # above the reference set by tile 0: the exact slow path must run there
    assert (PROGRAM.slow_taken > 0) == (kscale != 1.0), PROGRAM.slow_taken
    rows = np.arange(q0, min(q0 + BR, N))
    ro, rl = oracle.forward(q[None], k[None], v[None], scale, causal)
    err = np.abs(O[rows - q0] - ro[0][rows])
    lerr = np.abs(L[rows - q0] - rl[0][rows])
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
    assert lerr.max() <= 2e-2, lerr.max()
