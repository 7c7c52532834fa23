"""Instruction-level CPU emulation of the generated inline-assembly loops
(fa_fwd128_loop.inc, fa_bwd_dq128_loop.inc, fa_bwd_dkdv128_loop.inc),
shared by their tests.

The instruction text is executed for the four waves of one workgroup on a
model of their registers, the workgroup's LDS and global buffers:
  * scalar and vector instructions with their ISA semantics (fp32 vector
    arithmetic in float32, bf16 packing by round-to-nearest-even);
  * v_mfma_f32_32x32x16_bf16 with the operand and accumulator layouts
    measured on the device (fa_common.hpp);
  * ds_read_b128 / ds_read_b64_tr_b16 / ds_bpermute_b32 and the direct
    HBM -> LDS loads (global_load_lds_dwordx4 / _dword with M0 and an
    instruction offset that applies to both addresses);
  * s_barrier: every wave runs up to its next barrier before any goes on.
Every global load is checked to lie inside a registered buffer and every LDS
access inside LDS.  Hazards and timing are not modelled.
"""
import re

import numpy as np


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

    def read(self, addr, n):
        for base, arr in self.bufs:
            if base <= addr and addr + n <= base + arr.size:
                return arr[addr - base: addr - base + n]
        raise AssertionError(f"global load outside the buffers at {addr:#x}")

    def read16(self, addr):
        return self.read(addr, 16)


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


class Program:
    """A parsed statement.  body_kinds: label prefixes whose entries wave 0
    records (in order) in bodies_run, and every wave w in bodies_by_wave[w];
    slow_prefix: branch targets counted in slow_taken when taken."""

    def __init__(self, lines, body_kinds=(), slow_prefix=None):
        self.prog, self.labels = parse(lines)
        self.body_at = {}
        for name, pc in self.labels.items():
            for kind in body_kinds:
                if name.startswith(kind):
                    self.body_at[pc] = kind
        self.slow_prefix = slow_prefix
        self.slow_taken = 0
        self.bodies_run = []
        self.bodies_by_wave = {}

    def run_wave(self, m, lds, mem, pc, wave=0):
        """Execute from pc until a barrier (returns its pc + 1) or the end (None)."""
        while pc < len(self.prog):
            if pc in self.body_at:
                self.bodies_by_wave.setdefault(wave, []).append(self.body_at[pc])
                if wave == 0:
                    self.bodies_run.append(self.body_at[pc])
            op, args, off = self.prog[pc]
            pc += 1
            if op in ("s_nop", "s_waitcnt"):
                continue
            if op == "s_barrier":
                return pc
            if op == "s_branch":
                pc = self.labels[args[0]]
            elif op in ("s_cbranch_scc1", "s_cbranch_scc0", "s_cbranch_vccnz"):
                take = {"s_cbranch_scc1": m.scc == 1, "s_cbranch_scc0": m.scc == 0,
                        "s_cbranch_vccnz": bool(m.vcc.any())}[op]
                if take:
                    pc = self.labels[args[0]]
                    if self.slow_prefix and args[0].startswith(self.slow_prefix):
                        self.slow_taken += 1
            elif op.startswith("s_cmp_"):
                a, b = m.sval(args[0]), m.sval(args[1])
                m.scc = int({"s_cmp_eq_u32": a == b, "s_cmp_lg_u32": a != b,
                             "s_cmp_ge_u32": a >= b, "s_cmp_lt_u32": a < b,
                             "s_cmp_gt_u32": a > b}[op])
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
            elif op == "global_load_lds_dword":
                lo = int(REG.match(args[1]).group(3))
                base = m.s[lo] | (m.s[lo + 1] << 32)
                voff = m.vread_u(args[0])
                for l in range(64):
                    data = mem.read(base + int(voff[l]) + off, 4)
                    dst = m.m0 + off + 4 * l
                    assert 0 <= dst and dst + 4 <= lds.size, "LDS write out of range"
                    lds[dst:dst + 4] = data
            elif op == "s_mov_b32":
                m.swrite(args[0], m.sval(args[1]))
            elif op == "s_lshl_b32":
                t = m.sval(args[1]) << m.sval(args[2])
                m.scc = int((t & 0xFFFFFFFF) != 0)
                m.swrite(args[0], t)
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
            elif op == "v_cmp_ge_u32_e64":
                mask = m.vread_u(args[1]) >= m.vread_u(args[2])
                lo = int(REG.match(args[0]).group(3))
                bits = int(sum(1 << l for l in range(64) if mask[l]))
                m.s[lo], m.s[lo + 1] = bits & 0xFFFFFFFF, bits >> 32
            elif op == "v_sub_u32":
                m.vwrite(args[0], (m.vread_u(args[1]) - m.vread_u(args[2])).astype(np.uint32))
            elif op == "v_subrev_u32":
                m.vwrite(args[0], (m.vread_u(args[2]) - m.vread_u(args[1])).astype(np.uint32))
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



    def run_workgroup(self, waves, lds, mem):
        """Run the machines of `waves` (one workgroup) to the end, barrier
        by barrier."""
        pcs = [0] * len(waves)
        while True:
            for w, m in enumerate(waves):
                pcs[w] = self.run_wave(m, lds, mem, pcs[w], w)
            done = [p is None for p in pcs]
            assert all(done) or not any(done), "waves disagree on the barrier count"
            if all(done):
                return
