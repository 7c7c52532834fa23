"""CPU emulation of the generated key loop of the d = 128 forward kernel.

The instruction text that gen_fwd128.py emits (fa_fwd128_loop.inc) is
executed for the four waves of one workgroup on a model of their registers,
the workgroup's LDS and the global K/V buffers:
  * scalar and vector instructions with their ISA semantics (fp32 vector
    arithmetic in float32, bf16 packing by round-to-nearest-even);
  * v_mfma_f32_32x32x16_bf16 with the operand and accumulator layouts
    measured on the device (fa_common.hpp);
  * ds_read_b128 / ds_read_b64_tr_b16 / ds_bpermute_b32 and the direct
    HBM -> LDS loads (global_load_lds_dwordx4 with M0);
  * s_barrier: every wave runs up to its next barrier before any goes on.
Every global load is checked to lie inside the K or V buffer.  The setup
(registers and the three tiles staged before the loop) restates the C++ of
fa_fwd128.hip.  The output is normalised as the kernel's epilogue does and
compared with the fp64 oracle at the bf16 tolerances.  Hazards and timing
are not modelled (test_fwd128_schedule.py checks those on the text).
"""
import importlib.util
import os
import re

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_45_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", "gen_fwd128.py")
spec = importlib.util.spec_from_file_location("gen_fwd128_emu", GEN)
G = importlib.util.module_from_spec(spec)
spec.loader.exec_module(G)
LINES = G.generate()
D, BC, BR = 128, 64, 256


def tile_swz(r):
    return 4 * (r & 3) + ((r >> 2) & 3)


def bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    nan = np.isnan(np.asarray(x, np.float32))
    r[nan] = 0x7FC0
    return r.astype(np.uint32)


def bf16_to_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


REG = re.compile(r"^(-?)([vas])(?:\[(\d+):(\d+)\]|(\d+))$")


class Machine:
    """Registers of one wave."""

    def __init__(self):
        self.v = np.zeros((256, 64), np.uint32)
        self.a = np.zeros((256, 64), np.uint32)
        self.s = [0] * 106
        self.vcc = np.zeros(64, bool)
        self.scc = 0
        self.m0 = 0

    # operand access -------------------------------------------------------
    def rng(self, tok):
        m = REG.match(tok)
        neg, kind = m.group(1) == "-", m.group(2)
        lo = int(m.group(3) if m.group(3) is not None else m.group(5))
        hi = int(m.group(4)) if m.group(4) is not None else lo
        return neg, kind, lo, hi

    def vread(self, tok):
        """A 32-bit vector operand as float32 per lane (SGPRs broadcast,
        literals and inline constants accepted)."""
        if REG.match(tok):
            neg, kind, lo, _ = self.rng(tok)
            if kind == "v":
                x = self.v[lo].view(np.float32).copy()
            elif kind == "a":
                x = self.a[lo].view(np.float32).copy()
            else:
                x = np.full(64, np.uint32(self.s[lo]), np.uint32).view(np.float32).copy()
            return -x if neg else x
        if tok.startswith("0x"):
            return np.full(64, np.uint32(int(tok, 16)), np.uint32).view(np.float32).copy()
        return np.full(64, float(tok), np.float32)

    def vread_u(self, tok):
        if REG.match(tok):
            _, kind, lo, _ = self.rng(tok)
            src = {"v": self.v, "a": self.a}[kind] if kind != "s" else None
            if src is None:
                return np.full(64, np.uint32(self.s[lo]), np.uint32)
            return src[lo].copy()
        return np.full(64, np.uint32(int(tok, 0) & 0xFFFFFFFF), np.uint32)

    def vwrite(self, tok, x):
        _, kind, lo, _ = self.rng(tok)
        arr = self.v if kind == "v" else self.a
        arr[lo] = np.asarray(x).astype(np.float32).view(np.uint32) \
            if np.asarray(x).dtype != np.uint32 else x

    def block(self, tok):
        _, kind, lo, hi = self.rng(tok)
        arr = self.v if kind == "v" else self.a
        return arr, lo, hi

    def sval(self, tok):
        if tok == "m0":
            return self.m0
        m = REG.match(tok)
        if m and m.group(2) == "s":
            return self.s[int(m.group(5))]
        return int(tok, 0) & 0xFFFFFFFF

    def swrite(self, tok, x):
        x &= 0xFFFFFFFF
        if tok == "m0":
            self.m0 = x
        else:
            self.s[int(REG.match(tok).group(5))] = x


class Memory:
    """Global buffers (K, V) at fake addresses; every access is bounds-checked."""

    def __init__(self, bufs):
        self.bufs = bufs   # list of (base address, uint8 array)

    def read16(self, addr):
        for base, arr in self.bufs:
            if base <= addr and addr + 16 <= base + arr.size:
                return arr[addr - base: addr - base + 16]
        raise AssertionError(f"global load outside the K/V buffers at {addr:#x}")


def parse(lines):
    prog, labels = [], {}
    for l in lines:
        if l.endswith(":"):
            labels[l[:-1]] = len(prog)
            continue
        op, _, rest = l.partition(" ")
        args = [x.strip() for x in rest.split(",")] if rest else []
        off = 0
        if args and " offset:" in args[-1]:
            reg, _, o = args[-1].partition(" offset:")
            args[-1] = reg.strip()
            off = int(o)
        prog.append((op, args, off))
    return prog, labels


PROG, LABELS = parse(LINES)
# body entry points: straight (BODY), general unmasked (GB), masked (ITM), final (FIN)
BODY_AT = {}
for _name, _pc in LABELS.items():
    for _kind in ("FA_BODY", "FA_GB", "FA_ITM", "FA_FIN"):
        if _name.startswith(_kind):
            BODY_AT[_pc] = _kind[3:]


def mfma(m, args):
    A = lane_bf16(m, args[1])
    B = lane_bf16(m, args[2])
    Amat = np.zeros((32, 16))
    Bmat = np.zeros((16, 32))
    for l in range(64):
        h, i = l >> 5, l & 31
        Amat[i, 8 * h:8 * h + 8] = A[l]
        Bmat[8 * h:8 * h + 8, i] = B[l]
    arr, lo, hi = m.block(args[0])
    if args[3] == "0":
        C = np.zeros((16, 64), np.float32)
    else:
        carr, clo, _ = m.block(args[3])
        C = carr[clo:clo + 16].view(np.float32).copy()
    Cmat = np.zeros((32, 32))
    for l in range(64):
        h, j = l >> 5, l & 31
        for r in range(16):
            Cmat[8 * (r // 4) + 4 * h + r % 4, j] = C[r, l]
    Dm = Amat @ Bmat + Cmat
    out = np.zeros((16, 64), np.float32)
    for l in range(64):
        h, j = l >> 5, l & 31
        for r in range(16):
            out[r, l] = Dm[8 * (r // 4) + 4 * h + r % 4, j]
    arr[lo:lo + 16] = out.view(np.uint32)


def lane_bf16(m, tok):
    """8 bf16 per lane from a 4-register operand."""
    arr, lo, _ = m.block(tok)
    w = arr[lo:lo + 4]                       # 4 x 64 dwords
    out = np.zeros((64, 8))
    for t in range(4):
        out[:, 2 * t] = bf16_to_f32(w[t] & 0xFFFF)
        out[:, 2 * t + 1] = bf16_to_f32(w[t] >> 16)
    return out


SLOW_TAKEN = [0]
BODIES_RUN = []   # body kinds entered by wave 0, in order


def run_wave(m, lds, mem, pc, wave=0):
    """Execute from pc until a barrier (returns its pc + 1) or the end (None)."""
    while pc < len(PROG):
        if wave == 0 and pc in BODY_AT:
            BODIES_RUN.append(BODY_AT[pc])
        op, args, off = PROG[pc]
        pc += 1
        if op in ("s_nop", "s_waitcnt"):
            continue
        if op == "s_barrier":
            return pc
        if op == "s_branch":
            pc = LABELS[args[0]]
        elif op in ("s_cbranch_scc1", "s_cbranch_scc0", "s_cbranch_vccnz"):
            take = {"s_cbranch_scc1": m.scc == 1, "s_cbranch_scc0": m.scc == 0,
                    "s_cbranch_vccnz": bool(m.vcc.any())}[op]
            if take:
                pc = LABELS[args[0]]
                if args[0].startswith("FA_SLOW"):
                    SLOW_TAKEN[0] += 1
        elif op.startswith("s_cmp_"):
            a, b = m.sval(args[0]), m.sval(args[1])
            m.scc = int({"s_cmp_eq_u32": a == b, "s_cmp_lg_u32": a != b,
                         "s_cmp_ge_u32": a >= b, "s_cmp_lt_u32": a < b}[op])
        elif op == "s_add_u32":
            t = m.sval(args[1]) + m.sval(args[2])
            m.scc = int(t > 0xFFFFFFFF)
            m.swrite(args[0], t)
        elif op == "s_addc_u32":
            t = m.sval(args[1]) + m.sval(args[2]) + m.scc
            m.scc = int(t > 0xFFFFFFFF)
            m.swrite(args[0], t)
        elif op == "s_sub_u32":
            a, b = m.sval(args[1]), m.sval(args[2])
            m.scc = int(b > a)
            m.swrite(args[0], a - b)
        elif op == "s_cselect_b32":
            m.swrite(args[0], m.sval(args[1]) if m.scc else m.sval(args[2]))
        elif op == "global_load_lds_dwordx4":
            lo = int(REG.match(args[1]).group(3))
            base = m.s[lo] | (m.s[lo + 1] << 32)
            voff = m.vread_u(args[0])
            for l in range(64):
                # the instruction offset applies to both addresses
                data = mem.read16(base + int(voff[l]) + off)
                dst = m.m0 + off + 16 * l
                assert 0 <= dst and dst + 16 <= lds.size, "LDS write out of range"
                lds[dst:dst + 16] = data
        elif op == "ds_read_b128":
            arr, lo, _ = m.block(args[0])
            addr = m.vread_u(args[1]) + off
            for l in range(64):
                a0 = int(addr[l])
                assert 0 <= a0 and a0 + 16 <= lds.size, "LDS read out of range"
                arr[lo:lo + 4, l] = lds[a0:a0 + 16].view(np.uint32)
        elif op == "ds_read_b64_tr_b16":
            arr, lo, _ = m.block(args[0])
            addr = m.vread_u(args[1]) + off
            res = np.zeros((64, 4), np.uint16)
            for l in range(64):
                g, i = l // 16, l % 16
                for t in range(4):
                    src = int(addr[16 * g + 4 * t + i // 4])
                    res[l, t] = lds[src + 2 * (i % 4): src + 2 * (i % 4) + 2].view(np.uint16)[0]
            arr[lo:lo + 2] = res.view(np.uint32).T
        elif op == "ds_bpermute_b32":
            addr = m.vread_u(args[1])
            src = m.vread_u(args[2])
            m.vwrite(args[0], src[(addr // 4) % 64])
        elif op == "v_mfma_f32_32x32x16_bf16":
            mfma(m, args)
        elif op == "v_fma_f32":
            x = np.float32(1) * (m.vread(args[1]).astype(np.float64) * m.vread(args[2])
                                 + m.vread(args[3]))
            m.vwrite(args[0], x.astype(np.float32))
        elif op in ("v_exp_f32", "v_exp_f32_e64"):
            with np.errstate(over="ignore"):
                m.vwrite(args[0], np.exp2(m.vread(args[1])).astype(np.float32))
        elif op == "v_add_f32":
            m.vwrite(args[0], m.vread(args[1]) + m.vread(args[2]))
        elif op == "v_sub_f32":
            m.vwrite(args[0], m.vread(args[1]) - m.vread(args[2]))
        elif op == "v_mul_f32":
            with np.errstate(invalid="ignore"):
                m.vwrite(args[0], m.vread(args[1]) * m.vread(args[2]))
        elif op in ("v_max_f32", "v_max_f32_e64"):
            m.vwrite(args[0], np.fmax(m.vread(args[1]), m.vread(args[2])))
        elif op == "v_max3_f32":
            m.vwrite(args[0], np.fmax(np.fmax(m.vread(args[1]), m.vread(args[2])),
                                      m.vread(args[3])))
        elif op == "v_mov_b32":
            m.vwrite(args[0], m.vread_u(args[1]))
        elif op == "v_dot2_f32_bf16":
            x, y = m.vread_u(args[1]), m.vread_u(args[2])
            prod = (bf16_to_f32(x & 0xFFFF).astype(np.float64) * bf16_to_f32(y & 0xFFFF)
                    + bf16_to_f32(x >> 16).astype(np.float64) * bf16_to_f32(y >> 16))
            m.vwrite(args[0], (prod + m.vread(args[3])).astype(np.float32))
        elif op == "v_cvt_pk_bf16_f32":
            lo_, hi_ = bf16_bits(m.vread(args[1])), bf16_bits(m.vread(args[2]))
            m.vwrite(args[0], (lo_ | (hi_ << 16)).astype(np.uint32))
        elif op == "v_cmp_lt_f32":
            m.vcc = m.vread(args[1]) < m.vread(args[2])
        elif op == "v_cmp_gt_i32_e64":
            mask = np.int64(int(args[1])) > m.vread_u(args[2]).view(np.int32).astype(np.int64)
            lo = int(REG.match(args[0]).group(3))
            bits = int(sum(1 << l for l in range(64) if mask[l]))
            m.s[lo], m.s[lo + 1] = bits & 0xFFFFFFFF, bits >> 32
        elif op == "v_cndmask_b32_e64":
            lo = int(REG.match(args[3]).group(3))
            bits = m.s[lo] | (m.s[lo + 1] << 32)
            mask = np.array([(bits >> l) & 1 for l in range(64)], bool)
            m.vwrite(args[0], np.where(mask, m.vread_u(args[2]), m.vread_u(args[1])).astype(np.uint32))
        elif op == "v_sub_u32_e64":
            m.vwrite(args[0], (m.vread_u(args[1]) - np.uint32(int(args[2]))).astype(np.uint32))
        elif op == "v_accvgpr_read_b32":
            m.vwrite(args[0], m.vread_u(args[1]))
        elif op == "v_accvgpr_write_b32":
            _, _, lo, _ = m.rng(args[0])
            m.a[lo] = m.vread_u(args[1])
        else:
            raise NotImplementedError(op)
    return None


def emulate_workgroup(q, k, v, N, q0, causal, scale):
    """Run the generated loop for the workgroup whose rows start at q0 (one
    head); returns O [256, 128] (float64, rows past N left 0) and LSE."""
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

    def load_tile(buf, t, stage_byte):        # the C++ prologue's load_tile, all waves
        for w in range(4):
            for i in range(4):
                for lane in range(64):
                    p = (4 * i + w) * 64 + lane
                    row = p >> 4
                    qq = (p & 15) ^ tile_swz(row)
                    src = (min(t * BC + row, N - 1) * D + 8 * qq) * 2
                    dst = stage_byte + ((4 * i + w) * 64 + lane) * 16
                    lds[dst:dst + 16] = buf[src:src + 16]

    load_tile(kb, 0, 2 * TILE * 2)
    load_tile(vb, 0, 0)
    if tend > 1:
        load_tile(kb, 1, 3 * TILE * 2)
    waves = []
    for w in range(4):
        m = Machine()
        wrow0 = q0 + 64 * w
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            for rb in range(2):
                r = min(wrow0 + 32 * rb + l32, N - 1)
                for c in range(8):
                    e = qbits[r, 16 * c + 8 * h:16 * c + 8 * h + 8]
                    for t in range(4):
                        m.a[G.Q_BASE + 32 * rb + 4 * c + t, lane] = e[2 * t] | (e[2 * t + 1] << 16)
            sw_row = tile_swz(l32)
            for c in range(8):
                m.v[G.KADDR + c, lane] = 2 * (2 * TILE + l32 * D + 8 * ((2 * c + h) ^ sw_row))
            tr_row = 4 * h + ((lane & 15) >> 2)
            tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
            sw_lo, sw_hi = tile_swz(tr_row), tile_swz(tr_row + 8)
            tq, te = tr_col >> 3, tr_col & 7

            def tr_off(row, sw, b):
                return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te
            for db in range(4):
                m.v[G.VADDR + 2 * db, lane] = 2 * tr_off(tr_row, sw_lo, db)
                m.v[G.VADDR + 2 * db + 1, lane] = 2 * tr_off(tr_row + 8, sw_hi, db)
            for i in range(4):
                p = (4 * w + i) * 64 + lane
                row = p >> 4
                col = 8 * ((p & 15) ^ tile_swz(row))
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
        m.s[G.S_M0K] = 2 * TILE * 2 + w * 4096
        m.s[G.S_M0V] = w * 4096
        m.s[G.S_C] = int(np.float32(sl2).view(np.uint32))
        tail = ragged and tend == nt
        m.s[G.S_LAST] = tend - 1
        m.s[G.S_KEND] = max(0, tend - 2)
        m.s[G.S_KTAILJ] = nt - 3 if tail and nt >= 3 else 0xFFFFFFFF
        m.s[G.S_VTAILJ] = nt - 2 if tail and nt >= 2 else 0xFFFFFFFF
        m.s[G.S_FM] = fm
        m.s[G.S_FAST] = max(0, min(fm - 1, (nt - 1 if tail else tend) - 2))
        m.s[G.S_J] = 0
        waves.append([m, 0])
    while True:
        for w, wv in enumerate(waves):
            wv[1] = run_wave(wv[0], lds, mem, wv[1], w)
        done = [wv[1] is None for wv in waves]
        assert all(done) or not any(done), "waves disagree on the barrier count"
        if all(done):
            break
    O = np.zeros((BR, D))
    L = np.full(BR, np.nan)
    for w, (m, _) in enumerate(waves):
        lsum = m.v[G.LSUM:G.LSUM + 2].view(np.float32)
        mref = -m.v[G.MNEG:G.MNEG + 2].view(np.float32)
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            for rb in range(2):
                row = 64 * w + 32 * rb + l32
                ltot = float(lsum[rb, lane]) + float(lsum[rb, lane ^ 32])
                L[row] = (float(mref[rb, lane]) + np.log2(ltot)) * np.log(2.0)
                acc = m.a[G.O_BASE + 64 * rb:G.O_BASE + 64 * rb + 64, lane].view(np.float32)
                for db in range(4):
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


def expected_bodies(N, q0, causal):
    """Which body each tile step should take: straight while the next tile is
    unmasked and both loads are whole tiles, the masked body when the next
    tile needs a mask, the general one otherwise, the final one last."""
    nt = -(-N // BC)
    qmax = min(q0 + BR, N) - 1
    tend = min(nt, qmax // BC + 1) if causal else nt
    ragged = N % BC != 0
    fm = tend
    if causal:
        fm = min(fm, q0 // BC)
    if ragged:
        fm = min(fm, nt - 1)
    out = []
    for j in range(tend - 1):
        k_whole = j + 2 < tend and not (ragged and j + 2 == nt - 1)
        v_whole = not (ragged and j + 1 == nt - 1)
        if j + 1 >= fm:
            out.append("ITM")
        elif k_whole and v_whole:
            out.append("BODY")
        else:
            out.append("GB")
    return out + ["FIN"]


@pytest.mark.parametrize("N,q0,causal,kscale", CASES)
def test_generated_loop_matches_the_oracle(N, q0, causal, kscale):
    q, k, v = (t[0, 0].float().numpy() for t in inputs.qkv(1, 1, N, D, torch.bfloat16,
                                                             seed=N + q0 + int(causal)))
    if kscale != 1.0:
        k[192:] *= kscale
        k = bf16_to_f32(bf16_bits(k))
    scale = D ** -0.5
    SLOW_TAKEN[0] = 0
    BODIES_RUN.clear()
    O, L = emulate_workgroup(q, k, v, N, q0, causal, scale)
    assert BODIES_RUN == expected_bodies(N, q0, causal), BODIES_RUN
    # keys scaled by 3 from key 192 on lift those tiles' weights far past 2^8
    # above the reference set by tile 0: the exact slow path must run there
    assert (SLOW_TAKEN[0] > 0) == (kscale != 1.0), SLOW_TAKEN[0]
    rows = np.arange(q0, min(q0 + BR, N))
    ro, rl = oracle.forward(q[None], k[None], v[None], scale, causal)
    err = np.abs(O[rows - q0] - ro[0][rows])
    lerr = np.abs(L[rows - q0] - rl[0][rows])
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
    assert lerr.max() <= 2e-2, lerr.max()
