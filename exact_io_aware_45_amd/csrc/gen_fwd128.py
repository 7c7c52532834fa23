"""Generate the hand-scheduled main loops of the d = 128 and d = 64 bf16
forward kernels.

    python exact_io_aware_45_amd/csrc/gen_fwd128.py      # rewrites fa_fwd128_loop.inc,
                                                         # fa_fwd64_loop.inc (4 waves)
                                                         # and fa_fwd64w2_loop.inc (2 waves)

The loop runs inside fa_fwd128.hip (fa_fwd64.hip) as one inline-assembly statement; its
registers are pinned (the register map below), so the instruction order and
the register allocation are both fixed here rather than left to the compiler,
which serialised the three phases of a key tile (scores, softmax, P V) when it
scheduled them itself.

What one iteration computes is the tiled online softmax of exact attention
("FlashAttention." plate, opening section and "Never write the scores"; "Flash
Attention: IO-Aware Attention Computation", paragraph on fused kernels and the
online softmax): scores of a 64-key tile on the matrix cores, exponentials
against a running reference, the tile's weighted values added into the output.
How it is laid out is specific to gfx950:

  * one wave owns 64 query rows (two 32-row blocks) for the whole key loop,
    one wave per SIMD, so every K and V^T operand read from LDS feeds two
    matrix instructions;
  * iteration j issues the products of S_{j+1} = K_{j+1} Q^T (32 at d = 128,
    16 at d = 64) while the vector unit finishes tile j's exponentials
    (second 32-key half), then those of O += V_j^T P_j^T while it starts
    tile j+1's exponentials (first half): matrix and vector work of
    neighbouring tiles overlap.  The vector work is the same at both head
    dims, so at d = 64 it is the longer of the two and is spread evenly
    over the products;
  * the exponentials use a running per-row reference m instead of each
    tile's maximum (softmax is unchanged by the reference; the final
    normalisation divides by a sum taken against the same reference).  A
    tile whose per-lane sum of weights exceeds 2^8 (which any weight above
    2^8 implies, including an overflow) takes a slow path: the tile's exact
    row maximum from the raw scores, the reference moved to it, output and
    sums rescaled, weights recomputed.  So no weight ever exceeds 2^8 in the
    output, and the per-tile maximum costs nothing on the fast path;
  * K tiles arrive two tiles ahead and V tiles one tile ahead, by direct
    HBM -> LDS loads (double-buffered stages), one workgroup barrier per tile;
  * the statement runs the whole key loop of a workgroup: the first tile's
    scores and their exact row maxima (the first reference), every tile
    after it, and the masked ones at the end (causal diagonal tiles, the
    ragged tail), whose scores are set to -inf where key > row or key >= N
    by one threshold compare per element before their exponentials.  Causal
    tiles wholly past a wave's last row hold no visible key for it: from
    there on the wave only issues its share of the loads and the barriers.

The generator also checks its own output: data hazards between matrix and
vector instructions (wait states counted in instructions, conservatively),
LDS read counts against each product's s_waitcnt, and the operand rings.
"""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

# ------------------------------------------------------------------ head dim
# configure() sets these for one head dim (d = 128 when imported).
D = 128           # head dim
NC = D // 16      # 16-wide d chunks: K row operands per 32 keys, Q^T operands per row block
NDB = D // 32     # 32-wide d blocks of O^T
NLOAD = D // 32   # direct loads (1 KiB each) per wave per K or V tile
OUT = os.path.join(HERE, "fa_fwd128_loop.inc")
MACRO = "FA_FWD128_LOOP"
KERNEL = "fwd128_kernel (fa_fwd128.hip)"

# ---------------------------------------------------------------- register map
# AGPRs
O_BASE = 0        # a[0:16 NDB * 2]  O^T accumulators: O[rb][db] = a[16 NDB rb + 16 db : +16]
Q_BASE = 128      # a[128:128 + 8 NC] Q^T operands:  Q[rb][c]  = a[128 + 4 NC rb + 4 c : +4]
KRING = 8         # K operand ring slots (4 registers each)
VRING = 8         # V^T operand ring slots
KAHEAD = 3        # K operands read ahead of their first product
VAHEAD = 3        # V^T operands read ahead of their first product
KR_BASE = 192     # a[192:223] K operand ring
VR_BASE = 224     # a[224:255] V^T operand ring
# VGPRs
S_BASE = (0, 64)  # v[0:63], v[64:127]   scores S[rb][kb] = v[base + 32 rb + 16 kb : +16]
P_BASE = (128, 160)  # v[128:159], v[160:191] packed weights P[rb][kb][cc] = v[base + 16 rb + 8 kb + 4 cc : +4]
KADDR = 192       # v[192:192 + NC] K operand LDS addresses (stage 0, kb 0), one per c
VADDR = 200       # v[200:200 + 2 NDB] V^T LDS addresses (stage 0), index 2 db + hi
GOFF = 208        # v[208:208 + NLOAD] per-lane byte offsets of the direct loads within a tile
MNEG = 212        # v212, v213: -m (reference, log2 units) per row block
LSUM = 214        # v214, v215: running row sums (this lane's keys) per row block
TS = 216          # v[216:219] tile partial sums ts[rb][i] = v[216 + 2 rb + i], i = 0, 1
BPERM = 224       # v224: byte address lane ^ 32 for ds_bpermute (slow path)
TMP = 225         # v[225:248] temporaries
NTMP = 24
THR = 249         # v249, v250: mask threshold per row block for the next masked tile
NINF = 251        # v251: -inf
GOFF_TAIL = 252   # v[252:252 + NLOAD] direct-load offsets of the ragged last tile (rows clamped)
# SGPRs
S_KPTR = 60       # s[60:61] global address of the next K tile to load
S_VPTR = 62       # s[62:63] global address of the next V tile to load
S_M0K = 64        # LDS address of this wave's first K load (stage 0)
S_M0V = 65        # LDS address of this wave's first V load (stage 0)
S_C = 66          # scale * log2(e) (fp32 bits)
S_LAST = 67       # index of the last tile: its iteration is the final one
S_KEND = 68       # iterations j >= this load no K tile (tile j + 2 does not exist)
S_KTAILJ = 69     # iteration whose K load is the partial last tile (~0 when none)
S_FM = 70         # first tile that needs a mask (tend when none)
S_J = 71          # index of the current tile
S_VTAILJ = 72     # iteration whose V load is the partial last tile (~0 when none)
S_T = 73          # scratch
S_MASK = (74, 76, 78, 80)   # SGPR pairs for element masks
S_FAST = 82       # iterations j < this take the straight body: tile j + 1 needs no
                  # mask and both of its loads are whole tiles
S_WDIAG = 83      # this wave's last tile holding a visible key (causal: the tile of
                  # its last row); iterations past it only load and synchronise

# LDS map (bytes): V stage 0 at 0, V stage 1 at STAGE_BYTES, K stage 0 at
# 2 STAGE_BYTES, K stage 1 at 3 STAGE_BYTES (one 64-key tile each: 16 KiB at
# d = 128, 8 KiB at d = 64).  KADDR/VADDR hold stage-0 addresses.
STAGE_BYTES = 64 * D * 2
TILE_BYTES = 64 * D * 2   # one 64-key tile of K or V in global memory

THRESH = "0x43800000"   # 256.0: the per-lane tile sum that sends a tile to the slow path

# Conservative issue-cycle costs used to fill the shadow of each product.
COST = {"valu": 4.5, "trans": 8.0, "accw": 4.5, "lds": 4.0, "salu": 4.0, "vmem": 4.0, "nop": 1.0}
SLOT = 27.0   # vector/LDS issue cycles placed beside one product


def configure(d, nw=4):
    """Set the module's head-dim dependent values (d = 128 or 64) for a
    workgroup of `nw` waves (4, or 2 at d = 64).  The waves share each K and
    V tile's direct loads, so a wave issues 64 d 2 / 1024 / nw of them.  At
    d = 64 the vector work of a half-tile (the same as at d = 128) exceeds
    the shadow of its 16 products, so the slot budget grows to spread it
    evenly instead of leaving a tail after the last product."""
    global D, NC, NDB, NLOAD, OUT, MACRO, KERNEL, STAGE_BYTES, TILE_BYTES, SLOT
    assert (d, nw) in ((128, 4), (64, 4), (64, 2))
    D, NC, NDB, NLOAD = d, d // 16, d // 32, 64 * d * 2 // 1024 // nw
    tag = f"{d}" if nw == 4 else f"{d}w{nw}"
    OUT = os.path.join(HERE, f"fa_fwd{tag}_loop.inc")
    MACRO = f"FA_FWD{tag.upper()}_LOOP"
    KERNEL = f"fwd{d}_kernel (fa_fwd{d}.hip" + (")" if nw == 4 else f", {nw} waves)")
    STAGE_BYTES = TILE_BYTES = 64 * d * 2
    SLOT = 27.0 if d == 128 else SLOT64


# the (head dim, waves per workgroup) pairs whose loops the kernels include
VARIANTS = ((128, 4), (64, 4), (64, 2))
SLOT64 = 40.0

# Hazard distances (in issued instructions; s_nop N counts N+1).
H_MFMA_TO_READ = 18   # product result -> vector/LDS/accvgpr read
H_VALU_TO_MFMA = 4    # vector write -> product source read
H_TRANS_TO_USE = 2    # exponential -> vector read
H_SMASK = 3           # vector compare writing an SGPR mask -> vector read of the mask


def v(i):
    return f"v{i}"


def a(i):
    return f"a{i}"


def vr(lo, n):
    return f"v[{lo}:{lo + n - 1}]"


def ar(lo, n):
    return f"a[{lo}:{lo + n - 1}]"


class Ins:
    """One instruction: text, kind, registers it defines and uses."""

    def __init__(self, text, kind, defs=(), uses=(), srcc=()):
        self.text, self.kind = text, kind
        self.defs, self.uses, self.srcc = set(defs), set(uses), set(srcc)

    @property
    def cost(self):
        if self.kind == "mfma":
            return 1.0
        if self.kind == "nop":
            return float(int(self.text.split()[1]) + 1)
        return COST.get(self.kind, 1.0)

    @property
    def states(self):
        return int(self.text.split()[1]) + 1 if self.kind == "nop" else 1


def regs_v(lo, n):
    return [v(lo + i) for i in range(n)]


def regs_a(lo, n):
    return [a(lo + i) for i in range(n)]


class Stream:
    """An instruction list with hazard bookkeeping: before appending an
    instruction it inserts s_nop until every hazard distance is met."""

    def __init__(self, out):
        self.out = out          # list of text lines (shared by all streams)
        self.last_def = {}      # reg -> (kind, index in self.count units)
        self.count = 0          # wait states issued so far

    def need(self, ins):
        wait = 0
        for r in ins.uses | ins.srcc:
            if r not in self.last_def:
                continue
            kind, at = self.last_def[r]
            dist = self.count - at
            if kind == "mfma" and ins.kind != "mfma":
                wait = max(wait, H_MFMA_TO_READ - dist)
            elif kind == "mfma" and ins.kind == "mfma" and r in ins.uses:
                wait = max(wait, H_MFMA_TO_READ - dist)
            elif kind in ("valu", "trans", "accw") and ins.kind == "mfma":
                wait = max(wait, H_VALU_TO_MFMA - dist)
            elif kind == "trans" and ins.kind in ("valu", "trans"):
                wait = max(wait, H_TRANS_TO_USE - dist)
            if r.startswith("s") and kind == "valu":
                wait = max(wait, H_SMASK - dist)
        return max(0, wait)

    def emit(self, ins):
        w = self.need(ins)
        while w > 0:
            n = min(w, 8)
            self.out.append(f"s_nop {n - 1}")
            self.count += n
            w -= n
        self.out.append(ins.text)
        self.count += ins.states
        kind = ins.kind
        for r in ins.defs:
            self.last_def[r] = (kind, self.count - 1)

    def label(self, name):
        self.out.append(f"{name}:")

    def raw(self, text, states=1):
        self.out.append(text)
        self.count += states

    def settle(self):
        """Forget pending hazards after a point that all paths reach only
        after enough wait states (used at labels)."""
        self.last_def = {r: (k, at) for r, (k, at) in self.last_def.items()}


# ------------------------------------------------------------ building blocks
def s_reg(buf, rb, kb, r):
    return S_BASE[buf] + 32 * rb + 16 * kb + r


def p_reg(pbuf, rb, kb, cc):
    return P_BASE[pbuf] + 16 * rb + 8 * kb + 4 * cc


SKEW = True   # software-pipeline the per-element chain across groups of four
LOOKAHEAD = 8  # pending vector instructions the slot filler may pick from


def softmax_half(buf, pbuf, kb, fresh, tmp_ring, rbs=(0, 1), skew=None):
    """Vector work of one 32-key half (kb) of a tile for the given row blocks:
    t = s * c - m; p = 2^t; P = bf16 pairs of p; ts[rb][g % 2] += both fp32
    weights of the pair (two adds: a bf16 dot product against (1, 1) sums
    the rounded weights in one instruction, but it issues far slower and
    needs extra wait states before its result is read).
    `fresh`: the first weight into each partial sum overwrites it.

    Elements go in groups of four (two pairs of neighbouring keys per row
    block).  With SKEW the stream is software-pipelined: round k issues the
    scaled differences of group k, the exponentials of group k - 1 and the
    packs and sums of group k - 2, so every dependent instruction comes
    several instructions after the one it waits for."""
    first = {(rb, i): fresh for rb in rbs for i in range(2)}
    groups = []
    for g in range(8):            # pairs of elements r = 2g, 2g + 1
        elems = [(rb, 2 * g + e) for rb in rbs for e in range(2)]
        tmps = {e: next(tmp_ring) for e in elems}
        fma = [Ins(f"v_fma_f32 {v(tmps[(rb, r)])}, {v(s_reg(buf, rb, kb, r))}, s{S_C}, {v(MNEG + rb)}",
                   "valu", [v(tmps[(rb, r)])], [v(s_reg(buf, rb, kb, r)), v(MNEG + rb)])
               for (rb, r) in elems]
        exp = [Ins(f"v_exp_f32 {v(tmps[e])}, {v(tmps[e])}", "trans", [v(tmps[e])], [v(tmps[e])])
               for e in elems]
        pk, dots = [], []
        for rb in rbs:
            r = 2 * g
            cc, i = r // 8, (r % 8) // 2
            dst = p_reg(pbuf, rb, kb, cc) + i
            pk.append(Ins(f"v_cvt_pk_bf16_f32 {v(dst)}, {v(tmps[(rb, r)])}, {v(tmps[(rb, r + 1)])}",
                          "valu", [v(dst)], [v(tmps[(rb, r)]), v(tmps[(rb, r + 1)])]))
            ts = TS + 2 * rb + (g % 2)
            for e in range(2):
                t = tmps[(rb, r + e)]
                if first[(rb, g % 2)] and e == 0:
                    dots.append(Ins(f"v_mov_b32 {v(ts)}, {v(t)}", "valu", [v(ts)], [v(t)]))
                else:
                    dots.append(Ins(f"v_add_f32 {v(ts)}, {v(ts)}, {v(t)}", "valu", [v(ts)],
                                    [v(ts), v(t)]))
            first[(rb, g % 2)] = False
        groups.append((fma, exp, pk + dots))
    ops = []
    if not (SKEW if skew is None else skew):
        for fma, exp, fin in groups:
            ops += fma + exp + fin
        return ops
    n = len(groups)
    for k in range(n + 2):
        if k < n:
            ops += groups[k][0]
        if 0 <= k - 1 < n:
            ops += groups[k - 1][1]
        if 0 <= k - 2 < n:
            ops += groups[k - 2][2]
    return ops


def tmp_cycle():
    i = 0
    while True:
        yield TMP + (i % NTMP)
        i += 1


def check_ops():
    """Per-lane tile sums, the slow-path test and the running-sum update."""
    t0, t1, t2 = TMP + NTMP - 4, TMP + NTMP - 3, TMP + NTMP - 2
    ops = []
    for rb, x in enumerate((t0, t2)):
        ops.append(Ins(f"v_add_f32 {v(x)}, {v(TS + 2 * rb)}, {v(TS + 2 * rb + 1)}", "valu",
                       [v(x)], [v(TS + 2 * rb), v(TS + 2 * rb + 1)]))
    ops.append(Ins(f"v_max_f32 {v(t1)}, {v(t0)}, {v(t2)}", "valu", [v(t1)], [v(t0), v(t2)]))
    ops.append(Ins(f"v_cmp_lt_f32 vcc, {THRESH}, {v(t1)}", "valu", ["vcc"], [v(t1)]))
    return ops, (t0, t2)


def lsum_ops(tsums):
    return [Ins(f"v_add_f32 {v(LSUM + rb)}, {v(LSUM + rb)}, {v(tsums[rb])}", "valu",
                [v(LSUM + rb)], [v(LSUM + rb), v(tsums[rb])]) for rb in range(2)]


def full_loads(which, stage):
    """Direct HBM -> LDS loads of one whole K or V tile into `stage`: M0 is
    the wave's base in the stage and load i fills LDS [M0 + 1024 i, +1024)
    from offsets GOFF + i, which have 1024 i taken off (the instruction
    offset is added to both addresses).  Returns (M0 set-up, the NLOAD loads,
    the pointer step to the next tile); M0 must be written at least one
    instruction before the first load."""
    sptr, sm0 = (S_KPTR, S_M0K) if which == "K" else (S_VPTR, S_M0V)
    pre = [f"s_add_u32 m0, s{sm0}, {STAGE_BYTES * stage}"]
    loads = [f"global_load_lds_dwordx4 {v(GOFF + i)}, s[{sptr}:{sptr + 1}] offset:{1024 * i}"
             for i in range(NLOAD)]
    post = [f"s_add_u32 s{sptr}, s{sptr}, {TILE_BYTES}", f"s_addc_u32 s{sptr + 1}, s{sptr + 1}, 0"]
    return pre, loads, post


def tail_loads(which, stage):
    """Loads of the partial last tile: offsets with the rows clamped to the
    sequence (absolute, so M0 carries the 1024 i)."""
    sptr, sm0 = (S_KPTR, S_M0K) if which == "K" else (S_VPTR, S_M0V)
    out = []
    for i in range(NLOAD):
        out += [f"s_add_u32 m0, s{sm0}, {STAGE_BYTES * stage + 1024 * i}", "s_nop 0",
                f"global_load_lds_dwordx4 {v(GOFF_TAIL + i)}, s[{sptr}:{sptr + 1}]"]
    return out


def load_block(st, which, stage, uid, can_skip, can_tail):
    """The loads of a body other than the straight one, before its products:
    none when the tile does not exist (K only: tile j + 2 past the end), the
    clamped ones for the partial last tile, else the whole tile."""
    skip = f"FA_SKIP{which}{uid}_%="
    tail = f"FA_TAIL{which}{uid}_%="
    done = f"FA_LDONE{which}{uid}_%="
    if can_skip:
        st.raw(f"s_cmp_ge_u32 s{S_J}, s{S_KEND}")
        st.raw(f"s_cbranch_scc1 {skip}")
    if can_tail:
        st.raw(f"s_cmp_eq_u32 s{S_J}, s{S_KTAILJ if which == 'K' else S_VTAILJ}")
        st.raw(f"s_cbranch_scc1 {tail}")
    pre, loads, post = full_loads(which, stage)
    for l in pre + ["s_nop 0"] + loads:
        st.raw(l)
    if can_tail:
        st.raw(f"s_branch {done}")
        st.label(tail)
        for l in tail_loads(which, stage):
            st.raw(l)
        st.label(done)
    for l in post:
        st.raw(l)
    if can_skip:
        st.label(skip)


def mask_ops(buf, kbs, rbs=(0, 1)):
    """Scores whose key lies past the row's last visible key become -inf:
    element r of block (rb, kb) holds key k0 + 32 kb + 8 (r / 4) + 4 h + r % 4,
    and THR[rb] = last visible key - k0 - 4 h, so the test is one compare of
    a constant against THR.  Compares go to a ring of four SGPR pairs, each
    read three instructions later.  THR moves on by one tile afterwards."""
    ops = []
    elems = [(rb, kb, r) for kb in kbs for r in range(16) for rb in rbs]
    for g in range(0, len(elems), 4):
        grp = elems[g:g + 4]
        for i, (rb, kb, r) in enumerate(grp):
            off = 32 * kb + 8 * (r // 4) + r % 4
            pr = S_MASK[i]
            ops.append(Ins(f"v_cmp_gt_i32_e64 s[{pr}:{pr + 1}], {off}, {v(THR + rb)}", "valu",
                           [f"s{pr}"], [v(THR + rb)]))
        for i, (rb, kb, r) in enumerate(grp):
            sr = s_reg(buf, rb, kb, r)
            pr = S_MASK[i]
            ops.append(Ins(f"v_cndmask_b32_e64 {v(sr)}, {v(sr)}, {v(NINF)}, s[{pr}:{pr + 1}]",
                           "valu", [v(sr)], [v(sr), v(NINF), f"s{pr}"]))
    return ops


def thr_step():
    return [Ins(f"v_sub_u32_e64 {v(THR + rb)}, {v(THR + rb)}, 64", "valu", [v(THR + rb)],
                [v(THR + rb)]) for rb in range(2)]


def k_read(o, stage):
    """K operand o = (c, kb) into ring slot o % KRING."""
    c, kb = o // 2, o % 2
    slot = KR_BASE + 4 * (o % KRING)
    off = STAGE_BYTES * stage + 32 * 2 * D * kb
    return Ins(f"ds_read_b128 {ar(slot, 4)}, {v(KADDR + c)} offset:{off}", "lds",
               regs_a(slot, 4), [v(KADDR + c)])


def v_reads(o, stage):
    """V^T operand o = (block b = 2 kb + cc, db): two transpose reads into
    ring slot o % VRING (rows of the block's first and second 8-key groups)."""
    b, db = o // NDB, o % NDB
    kb, cc = b // 2, b % 2
    slot = VR_BASE + 4 * (o % VRING)
    off = STAGE_BYTES * stage + (32 * kb + 16 * cc) * 2 * D
    return [Ins(f"ds_read_b64_tr_b16 {ar(slot + 2 * hi, 2)}, {v(VADDR + 2 * db + hi)} offset:{off}",
                "lds", regs_a(slot + 2 * hi, 2), [v(VADDR + 2 * db + hi)]) for hi in range(2)]


def s_mfma(m, nxt):
    """Product m of the score phase: c = m // 4, kb = (m // 2) % 2, rb = m % 2."""
    c, kb, rb = m // 4, (m // 2) % 2, m % 2
    o = m // 2
    dst = s_reg(nxt, rb, kb, 0)
    src_c = "0" if c == 0 else vr(dst, 16)
    slot = KR_BASE + 4 * (o % KRING)
    q = Q_BASE + 4 * NC * rb + 4 * c
    srcc = regs_v(dst, 16) if c else []
    return Ins(f"v_mfma_f32_32x32x16_bf16 {vr(dst, 16)}, {ar(slot, 4)}, {ar(q, 4)}, {src_c}",
               "mfma", regs_v(dst, 16), regs_a(slot, 4) + regs_a(q, 4), srcc)


def pv_mfma(m, pbuf):
    """Product m of the P V phase: block b = m // (2 NDB) (kb = b // 2,
    cc = b % 2), db = (m // 2) % NDB, rb = m % 2."""
    b, db, rb = m // (2 * NDB), (m // 2) % NDB, m % 2
    kb, cc = b // 2, b % 2
    o = m // 2
    slot = VR_BASE + 4 * (o % VRING)
    dst = O_BASE + 16 * NDB * rb + 16 * db
    p = p_reg(pbuf, rb, kb, cc)
    return Ins(f"v_mfma_f32_32x32x16_bf16 {ar(dst, 16)}, {ar(slot, 4)}, {vr(p, 4)}, {ar(dst, 16)}",
               "mfma", regs_a(dst, 16), regs_a(slot, 4) + regs_v(p, 4), regs_a(dst, 16))


class LdsCounter:
    """Outstanding LDS reads of this wave, in issue order (they return in
    order): a product waits with lgkmcnt(k) until its operand has landed."""

    def __init__(self):
        self.pending = []   # ids of issued, not yet waited-for reads

    def issue(self, rid):
        self.pending.append(rid)

    def wait_for(self, rids):
        """lgkmcnt value that guarantees every read in rids has completed, or
        None if no wait is needed."""
        idx = [i for i, r in enumerate(self.pending) if r in rids]
        if not idx:
            return None
        last = max(idx)
        k = len(self.pending) - 1 - last
        self.pending = self.pending[last + 1:]
        return k


def interleave(st, mfmas, reads_before, valu, lds, read_sched, operand_reads, tail_valu=True,
               raw_sched=None):
    """Emit the products in order; after product i, the LDS reads scheduled
    for it, the scalar/load lines raw_sched[i], then vector work up to the
    slot budget.  `reads_before` are issued first (with some vector work
    after them to cover their latency).
    read_sched[i]: list of (rid, Ins) issued after product i.
    operand_reads[i]: rids product i needs."""
    raw_sched = raw_sched or {}
    valu = list(valu)

    def ready(i):
        """Instruction i of the pending list can go now: no hazard wait, and no
        data dependence on an earlier pending instruction (it neither reads
        what they write nor writes what they read or write)."""
        ins = valu[i]
        if st.need(ins) > 0:
            return False
        for prev in valu[:i]:
            if (ins.uses | ins.srcc) & prev.defs or ins.defs & (prev.uses | prev.srcc | prev.defs):
                return False
        return True

    def fill(budget):
        used = 0.0
        while valu:
            pick = next((i for i in range(min(LOOKAHEAD, len(valu))) if ready(i)), None)
            if pick is None or used + valu[pick].cost > budget + 1e-9:
                break
            ins = valu.pop(pick)
            st.emit(ins)
            used += ins.cost

    for rid, ins in reads_before:
        st.emit(ins)
        lds.issue(rid)
    if mfmas:
        fill(2 * SLOT)
    for i, mf in enumerate(mfmas):
        k = lds.wait_for(operand_reads[i])
        if k is not None:
            st.raw(f"s_waitcnt lgkmcnt({min(k, 15)})")
        st.emit(mf)
        spent = 0.0
        for rid, ins in read_sched.get(i, []):
            st.emit(ins)
            lds.issue(rid)
            spent += ins.cost
        for line in raw_sched.get(i, []):
            st.raw(line)
            spent += COST["vmem"] if line.startswith("global_") else COST["salu"]
        fill(SLOT - spent)
    if tail_valu:
        for ins in valu:
            st.emit(ins)
        valu.clear()
    return valu


def interleave_even(st, mfmas, reads_before, valu, lds, read_sched, operand_reads,
                    raw_sched=None, gap=28.0, init=0.0):
    """Emit the products in order; after product i the LDS reads scheduled
    for it, the scalar/load lines raw_sched[i], then vector work.  Unlike
    the forward's filler, which packs each product's shadow full, the
    vector work is spread evenly: after product i it takes the remaining
    work's share of the remaining products (at most `gap` cycles with the
    reads and scalar lines), so the matrix pipe never waits on a burst and
    no work is left for the end.  A product waits (s_waitcnt) until its
    operand reads have landed."""
    raw_sched = raw_sched or {}
    valu = list(valu)

    def ready(i):
        ins = valu[i]
        if st.need(ins) > 0:
            return False
        for prev in valu[:i]:
            if (ins.uses | ins.srcc) & prev.defs or ins.defs & (prev.uses | prev.srcc | prev.defs):
                return False
        return True

    def fill(budget):
        used = 0.0
        while valu:
            pick = next((i for i in range(min(LOOKAHEAD, len(valu))) if ready(i)), None)
            if pick is None or used + valu[pick].cost > budget + 1e-9:
                break
            ins = valu.pop(pick)
            st.emit(ins)
            used += ins.cost

    for rid, ins in reads_before:
        st.emit(ins)
        lds.issue(rid)
    if mfmas and init:
        fill(init)
    n = len(mfmas)
    for i, mf in enumerate(mfmas):
        k = lds.wait_for(operand_reads[i])
        if k is not None:
            st.raw(f"s_waitcnt lgkmcnt({min(k, 15)})")
        st.emit(mf)
        spent = 0.0
        for rid, ins in read_sched.get(i, []):
            st.emit(ins)
            lds.issue(rid)
            spent += ins.cost
        for line in raw_sched.get(i, []):
            st.raw(line)
            spent += COST["vmem"] if line.startswith("global_") else COST["salu"]
        left = sum(x.cost for x in valu)
        share = left / max(1, n - i)
        fill(min(gap - spent, share + 4.5))
    for ins in valu:
        st.emit(ins)


def phase_a(st, lds, cur, pcur, nxt, kstage, final, tmp_ring, raw_sched=None):
    """Scores of the next tile (4 NC products) beside the second half of the
    current tile's weights, then the sum test.  Returns the tile-sum regs."""
    soft = softmax_half(cur, pcur, 1, False, tmp_ring)
    chk, tsums = check_ops()
    if final:
        for ins in soft + chk:
            st.emit(ins)
        return tsums
    mf = [s_mfma(m, nxt) for m in range(4 * NC)]
    before = [(("K", o), k_read(o, kstage)) for o in range(KAHEAD)]
    sched, need = {}, {}
    for m in range(4 * NC):   # one wait per two operands
        o = m // 2
        need[m] = {("K", o), ("K", o + 1)} if o % 2 == 0 else {("K", o)}
    for o in range(KAHEAD, 2 * NC):   # operand o's read after product 2(o - KAHEAD)
        sched.setdefault(2 * (o - KAHEAD), []).append((("K", o), k_read(o, kstage)))
    interleave(st, mf, before, soft + chk, lds, sched, need, raw_sched=raw_sched)
    return tsums


def phase_b(st, lds, cur_p, vstage, nxt, pnxt, final, tmp_ring, prefetched, nextmask=False):
    """O += V^T P^T for the current tile (8 NDB products) beside the first
    half of the next tile's weights (its mask first, when it needs one)."""
    mf = [pv_mfma(m, cur_p) for m in range(8 * NDB)]
    soft = [] if final else softmax_half(nxt, pnxt, 0, True, tmp_ring)
    if nextmask and not final:
        soft = mask_ops(nxt, (0,)) + soft + mask_ops(nxt, (1,)) + thr_step()
    sched, need = {}, {}
    for m in range(8 * NDB):   # one wait per two operands
        o = m // 2
        need[m] = ({("V", o, 0), ("V", o, 1), ("V", o + 1, 0), ("V", o + 1, 1)}
                   if o % 2 == 0 else {("V", o, 0), ("V", o, 1)})
    for o in range(VAHEAD, 4 * NDB):
        reads = v_reads(o, vstage)
        sched.setdefault(2 * (o - VAHEAD) + 1, []).extend([(("V", o, h), reads[h])
                                                           for h in range(2)])
    before = []
    for o in range(VAHEAD):
        if o not in prefetched:
            reads = v_reads(o, vstage)
            before += [(("V", o, h), reads[h]) for h in range(2)]
    interleave(st, mf, before, soft, lds, sched, need)


def slow_path(st, cur, pcur, tmp_ring, back_label):
    """Exact path for a tile whose weights grew past 2^8: the row maximum of
    the raw scores (both halves of the wave), the reference moved to it, the
    output and running sums rescaled, all 64 weights recomputed."""
    st.raw("s_nop 7")
    st.raw("s_nop 7")
    st.raw("s_waitcnt lgkmcnt(0)")
    mx = [TMP + 0, TMP + 1]
    oth = [TMP + 2, TMP + 3]
    alpha = [TMP + 4, TMP + 5]
    for rb in range(2):
        els = [s_reg(cur, rb, kb, r) for kb in range(2) for r in range(16)]
        st.emit(Ins(f"v_max3_f32 {v(mx[rb])}, {v(els[0])}, {v(els[1])}, {v(els[2])}", "valu",
                    [v(mx[rb])], [v(e) for e in els[:3]]))
        for i in range(3, 32, 2):
            b = els[i + 1] if i + 1 < 32 else els[i]
            st.emit(Ins(f"v_max3_f32 {v(mx[rb])}, {v(mx[rb])}, {v(els[i])}, {v(b)}", "valu",
                        [v(mx[rb])], [v(mx[rb]), v(els[i]), v(b)]))
        st.raw(f"ds_bpermute_b32 {v(oth[rb])}, {v(BPERM)}, {v(mx[rb])}")
    st.raw("s_waitcnt lgkmcnt(0)")
    for rb in range(2):
        # m_new = max(m_old, rowmax * c); alpha = 2^(m_old - m_new); mneg = -m_new
        st.emit(Ins(f"v_max_f32 {v(mx[rb])}, {v(mx[rb])}, {v(oth[rb])}", "valu", [v(mx[rb])],
                    [v(mx[rb]), v(oth[rb])]))
        st.emit(Ins(f"v_mul_f32 {v(mx[rb])}, s{S_C}, {v(mx[rb])}", "valu", [v(mx[rb])],
                    [v(mx[rb])]))
        st.emit(Ins(f"v_max_f32_e64 {v(mx[rb])}, -{v(MNEG + rb)}, {v(mx[rb])}", "valu",
                    [v(mx[rb])], [v(mx[rb]), v(MNEG + rb)]))
        st.emit(Ins(f"v_add_f32 {v(alpha[rb])}, {v(MNEG + rb)}, {v(mx[rb])}", "valu",
                    [v(alpha[rb])], [v(MNEG + rb), v(mx[rb])]))
        st.emit(Ins(f"v_exp_f32_e64 {v(alpha[rb])}, -{v(alpha[rb])}", "trans", [v(alpha[rb])],
                    [v(alpha[rb])]))
        st.emit(Ins(f"v_sub_f32 {v(MNEG + rb)}, 0, {v(mx[rb])}", "valu", [v(MNEG + rb)],
                    [v(mx[rb])]))
        st.emit(Ins(f"v_mul_f32 {v(LSUM + rb)}, {v(LSUM + rb)}, {v(alpha[rb])}", "valu",
                    [v(LSUM + rb)], [v(LSUM + rb), v(alpha[rb])]))
    # rescale O (AGPRs) 8 registers at a time
    work = [TMP + 8 + i for i in range(8)]
    for rb in range(2):
        orb = O_BASE + 16 * NDB * rb
        for base in range(0, 16 * NDB, 8):
            for i in range(8):
                st.emit(Ins(f"v_accvgpr_read_b32 {v(work[i])}, {a(orb + base + i)}",
                            "valu", [v(work[i])], [a(orb + base + i)]))
            for i in range(8):
                st.emit(Ins(f"v_mul_f32 {v(work[i])}, {v(alpha[rb])}, {v(work[i])}", "valu",
                            [v(work[i])], [v(alpha[rb]), v(work[i])]))
            for i in range(8):
                st.emit(Ins(f"v_accvgpr_write_b32 {a(orb + base + i)}, {v(work[i])}",
                            "accw", [a(orb + base + i)], [v(work[i])]))
    ring = tmp_cycle_from(TMP + 16, NTMP - 16 - 4)   # four: one group at a time, unskewed
    for ins in (softmax_half(cur, pcur, 0, True, ring, skew=False)
                + softmax_half(cur, pcur, 1, False, ring, skew=False)):
        st.emit(ins)
    chk, tsums = check_ops()
    for ins in chk[:-2]:       # the sums only (no second test: every weight is now <= 1)
        st.emit(ins)
    for ins in lsum_ops(tsums):
        st.emit(ins)
    st.raw("s_nop 4")
    st.raw(f"s_branch {back_label}")


def tmp_cycle_from(lo, n):
    i = 0
    while True:
        yield lo + (i % n)
        i += 1


def iteration(out, name, cur, nxt, kstage_read, vstage, kstage_load, vstage_load, kind):
    """One tile step: loads, phase A, test, phase B, barrier.  `name` makes
    the labels unique within the statement.  kind: "fast" (the straight
    body: whole loads spread over the first products, the tile counter
    stepped and compared there too, leaving SCC = the next step is straight
    as well), "gen" (next tile unmasked, loads decided by the tile index),
    "masked" (next tile masked) or "final" (no next tile, no loads)."""
    st = Stream(out)
    lds = LdsCounter()
    tmp_ring = tmp_cycle_from(TMP, NTMP - 4)
    pcur, pnxt = cur, nxt
    final = kind == "final"
    raw_sched = None
    if kind == "fast":
        kpre, kloads, kpost = full_loads("K", kstage_load)
        vpre, vloads, vpost = full_loads("V", vstage_load)
        step = [f"s_add_u32 s{S_J}, s{S_J}, 1", f"s_cmp_lt_u32 s{S_J}, s{S_FAST}"]
        # one load after each of the first products: M0 before product 0,
        # the K loads after products 1 .. NLOAD, then the V loads
        raw_sched = {0: kpre}
        for i, l in enumerate(kloads + vloads):
            raw_sched.setdefault(i + 1, []).append(l)
        raw_sched[NLOAD] += kpost + vpre
        raw_sched[2 * NLOAD] += vpost + step
    elif kind in ("gen", "masked"):
        load_block(st, "K", kstage_load, name, can_skip=True, can_tail=True)
        load_block(st, "V", vstage_load, name, can_skip=False, can_tail=kind == "masked")
    tsums = phase_a(st, lds, cur, pcur, nxt, kstage_read, final, tmp_ring, raw_sched)
    # V^T reads for the first products of phase B go out before the test
    pre = []
    for o in range(VAHEAD):
        for h, ins in enumerate(v_reads(o, vstage)):
            st.emit(ins)
            lds.issue(("V", o, h))
        pre.append(o)
    slow_lbl = f"FA_SLOW{name}_%="
    back_lbl = f"FA_PB{name}_%="
    st.raw(f"s_cbranch_vccnz {slow_lbl}")
    for ins in lsum_ops(tsums):
        st.emit(ins)
    st.label(back_lbl)
    phase_b(st, lds, pcur, vstage, nxt, pnxt, final, tmp_ring, pre, kind == "masked")
    st.raw("s_waitcnt vmcnt(0)")
    st.raw("s_barrier")
    return slow_lbl, back_lbl, cur, pcur


def entry(out):
    """Scores of tile 0 into buffer 0 (K stage 0) with the output
    accumulators cleared beside them, their mask when tile 0 needs one, the
    exact row maxima as the first reference, and tile 0's first-half
    weights."""
    st = Stream(out)
    st.raw("s_nop 4")
    lds = LdsCounter()
    mf = [s_mfma(m, 0) for m in range(4 * NC)]
    before = [(("K", o), k_read(o, 0)) for o in range(KAHEAD)]
    sched, need = {}, {}
    for m in range(4 * NC):
        o = m // 2
        need[m] = {("K", o), ("K", o + 1)} if o % 2 == 0 else {("K", o)}
    for o in range(KAHEAD, 2 * NC):
        sched.setdefault(2 * (o - KAHEAD), []).append((("K", o), k_read(o, 0)))
    zero = [Ins(f"v_accvgpr_write_b32 {a(O_BASE + i)}, 0", "accw", [a(O_BASE + i)])
            for i in range(32 * NDB)]
    interleave(st, mf, before, zero, lds, sched, need)
    # every wave has read K_0 before iteration 0 loads K_2 into its stage
    st.raw("s_waitcnt lgkmcnt(0)")
    st.raw("s_barrier")
    # settle the products' results before the branch: both paths read them
    st.raw("s_nop 7", 8)
    st.raw("s_nop 7", 8)
    st.raw("s_nop 3", 4)
    skip = "FA_EMASK_%="
    st.raw(f"s_cmp_lg_u32 s{S_FM}, 0")
    st.raw(f"s_cbranch_scc1 {skip}")
    for ins in mask_ops(0, (0, 1)) + thr_step():
        st.emit(ins)
    st.label(skip)
    mx, oth = [TMP + 0, TMP + 1], [TMP + 2, TMP + 3]
    for rb in range(2):
        els = [s_reg(0, rb, kb, r) for kb in range(2) for r in range(16)]
        st.emit(Ins(f"v_max3_f32 {v(mx[rb])}, {v(els[0])}, {v(els[1])}, {v(els[2])}", "valu",
                    [v(mx[rb])], [v(e) for e in els[:3]]))
        for i in range(3, 32, 2):
            b = els[i + 1] if i + 1 < 32 else els[i]
            st.emit(Ins(f"v_max3_f32 {v(mx[rb])}, {v(mx[rb])}, {v(els[i])}, {v(b)}", "valu",
                        [v(mx[rb])], [v(mx[rb]), v(els[i]), v(b)]))
        st.raw(f"ds_bpermute_b32 {v(oth[rb])}, {v(BPERM)}, {v(mx[rb])}")
    st.raw("s_waitcnt lgkmcnt(0)")
    for rb in range(2):
        st.emit(Ins(f"v_max_f32 {v(mx[rb])}, {v(mx[rb])}, {v(oth[rb])}", "valu", [v(mx[rb])],
                    [v(mx[rb]), v(oth[rb])]))
        st.emit(Ins(f"v_mul_f32 {v(mx[rb])}, s{S_C}, {v(mx[rb])}", "valu", [v(mx[rb])],
                    [v(mx[rb])]))
        st.emit(Ins(f"v_sub_f32 {v(MNEG + rb)}, 0, {v(mx[rb])}", "valu", [v(MNEG + rb)],
                    [v(mx[rb])]))
    ring = tmp_cycle_from(TMP + 4, NTMP - 8)
    for ins in softmax_half(0, 0, 0, True, ring):
        st.emit(ins)


def generate():
    """The entry, then per parity of the tile index (which stages hold the
    operands): the dispatch, the straight body, the general unmasked body,
    the masked body; the final bodies; the slow paths."""
    out = []
    entry(out)
    slows = []

    def stages(parity):
        cur, nxt = (0, 1) if parity == 0 else (1, 0)
        kread, vst = (1, 0) if parity == 0 else (0, 1)
        kload, vload = (0, 1) if parity == 0 else (1, 0)
        return cur, nxt, kread, vst, kload, vload

    for parity, P in ((0, "A"), (1, "B")):
        Q = "B" if P == "A" else "A"
        out.append(f"FA_L{P}_%=:")
        out.append(f"s_cmp_lt_u32 s{S_J}, s{S_FAST}")
        out.append(f"s_cbranch_scc0 FA_GEN{P}_%=")
        out.append(f"FA_BODY{P}_%=:")
        slows.append(iteration(out, P, *stages(parity), "fast"))
        out.append(f"s_cbranch_scc1 FA_BODY{Q}_%=")
        out.append(f"s_branch FA_GEN{Q}_%=")
        out.append(f"FA_GEN{P}_%=:")
        out.append(f"s_cmp_gt_u32 s{S_J}, s{S_WDIAG}")
        out.append(f"s_cbranch_scc1 FA_IDLE{P}_%=")
        out.append(f"s_cmp_eq_u32 s{S_J}, s{S_LAST}")
        out.append(f"s_cbranch_scc1 FA_FIN{P}_%=")
        out.append(f"s_add_u32 s{S_T}, s{S_J}, 1")
        out.append(f"s_cmp_ge_u32 s{S_T}, s{S_FM}")
        out.append(f"s_cbranch_scc1 FA_ITM{P}_%=")
        out.append(f"FA_GB{P}_%=:")
        slows.append(iteration(out, "G" + P, *stages(parity), "gen"))
        out.append(f"s_add_u32 s{S_J}, s{S_J}, 1")
        out.append(f"s_branch FA_L{Q}_%=")
        out.append(f"FA_ITM{P}_%=:")
        slows.append(iteration(out, "M" + P, *stages(parity), "masked"))
        out.append(f"s_add_u32 s{S_J}, s{S_J}, 1")
        out.append(f"s_branch FA_L{Q}_%=")
        # idle steps: tile j holds no key this wave sees, nor does any later
        # one; the wave still loads its rows of K_{j+2} and V_{j+1} and meets
        # the barrier, and ends with the others at the last tile
        out.append(f"FA_IDLE{P}_%=:")
        out.append(f"s_cmp_eq_u32 s{S_J}, s{S_LAST}")
        out.append("s_cbranch_scc1 FA_IDLEF_%=")
        st = Stream(out)
        _, _, _, _, kload, vload = stages(parity)
        load_block(st, "K", kload, "I" + P, can_skip=True, can_tail=True)
        load_block(st, "V", vload, "I" + P, can_skip=False, can_tail=True)
        out.append("s_waitcnt vmcnt(0)")
        out.append("s_barrier")
        out.append(f"s_add_u32 s{S_J}, s{S_J}, 1")
        out.append(f"s_branch FA_IDLE{Q}_%=")
    out.append("FA_IDLEF_%=:")
    out.append("s_waitcnt vmcnt(0)")
    out.append("s_barrier")
    out.append("s_branch FA_DONE_%=")
    for parity, P in ((0, "A"), (1, "B")):
        out.append(f"FA_FIN{P}_%=:")
        slows.append(iteration(out, "F" + P, *stages(parity), "final"))
        out.append("s_branch FA_DONE_%=")
    for slow_lbl, back_lbl, cur, pcur in slows:
        st = Stream(out)
        st.label(slow_lbl)
        slow_path(st, cur, pcur, None, back_lbl)
    out.append("FA_DONE_%=:")
    out.append("s_nop 7")
    out.append("s_nop 7")
    out.append("s_nop 7")
    return out


def clobbers():
    """Registers the statement overwrites that are not operands."""
    regs = [f"v{i}" for i in range(0, 192)]              # both S and both P buffers
    regs += [f"v{i}" for i in range(TS, TS + 4)]
    regs += [f"v{i}" for i in range(TMP, TMP + NTMP)]
    regs += [f"a{i}" for i in range(KR_BASE, VR_BASE + 4 * VRING)]
    regs += [f"s{i}" for i in range(S_T, S_T + 9)]
    regs += ["vcc", "scc", "m0", "memory"]
    return regs


def render(lines):
    body = "\n".join(f'  "{l}\\n"' for l in lines)
    clob = ", ".join(f'"{r}"' for r in clobbers())
    return (
        "// Generated by gen_fwd128.py -- do not edit.  The main loop of\n"
        f"// {KERNEL}: see the generator for the schedule.\n"
        f"#define {MACRO}_ASM \\\n" + body.replace("\n", " \\\n") + "\n\n"
        f"#define {MACRO}_CLOBBERS " + clob + "\n"
        f"// {len(lines)} lines\n")


def main():
    stale = False
    for d, nw in VARIANTS:
        configure(d, nw)
        lines = generate()
        text = render(lines)
        if len(sys.argv) > 1 and sys.argv[1] == "--check":
            cur = open(OUT).read() if os.path.exists(OUT) else ""
            stale |= cur != text
            continue
        with open(OUT, "w") as f:
            f.write(text)
        print(f"wrote {OUT}: {len(lines)} lines")
    configure(128)
    if stale:
        sys.exit(1)


if __name__ == "__main__":
    main()
