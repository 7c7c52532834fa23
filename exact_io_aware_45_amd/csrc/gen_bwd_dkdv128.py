"""Generate the hand-scheduled query loop of the d = 128 bf16 dK/dV kernel.

    python exact_io_aware_45_amd/csrc/gen_bwd_dkdv128.py   # rewrites fa_bwd_dkdv128_loop.inc

The dK/dV pass of the backward recomputes, for each key and query tile, the
probabilities from the saved log-sum-exp and the gradient of the scores
("FlashAttention." plate, "Never write the scores"):

    S  = Q K^T,  dP = dO V^T                (two products per query tile)
    P  = exp2(S c - L),  dS = P (dP - D)    (L = LSE log2(e), c = scale log2(e))
    dV += P^T dO,  dK += dS^T Q             (two more; dK's scale at the store)

The statement runs one wave's whole query loop for its 32 keys, at one wave
per SIMD, with every register assigned here (the machinery is the forward's,
gen_fwd128.py, and the half-tile pipeline the dQ loop's, gen_bwd_dq128.py):

  * a[0:63] dK^T and a[64:127] dV^T accumulators (lane = key), a[128:159]
    the wave's K rows and a[160:191] its V rows as the B operands of the
    score products, a[192:255] four operand rings (Q rows, dO rows, Q^T and
    dO^T by transpose reads);
  * v[0:63] two slots of S and dP (lane = key, register = query) for one
    32-query half each, v[64:95] two slots of packed P and dS, v[96:127] two
    slots of the L values of the slot's 16 queries per lane half, v[128:143]
    the -D values that start the next dP product chain (so that it leaves
    dP - D and the vector unit never subtracts D).

Step 1 of query tile j: the exponentials and dS of (j, second half) beside
the products dV/dK of (j, first half) and S/dP of (j + 1, first half); step 2:
the vector work of (j + 1, first half) beside dV/dK of (j, second half) and
S/dP of (j + 1, second half).  One barrier per tile.  Tile step j reads
tiles j and j + 1 only, so with four LDS stages Q, dO and the L, D rows of
tile j + 3 load during step j and have until the end of step j + 1 to land
(the body is generated for each tile index modulo 4, counted from the
item's first query tile).  Scores whose key follows the query (causal) or whose query
lies past the sequence become -inf before the exponential, in the first two
tiles of a causal item and in a partial last tile.
"""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)
import gen_fwd128 as F  # noqa: E402
from gen_bwd_dq128 import Stream  # noqa: E402
from gen_fwd128 import Ins, LdsCounter, a, ar, regs_a, regs_v, v, vr  # noqa: E402

OUT = os.path.join(HERE, "fa_bwd_dkdv128_loop.inc")

# ------------------------------------------------------------- register map
DK_BASE = 0       # a[0:63]    dK^T accumulators: DK[db] = a[16 db : +16]
DV_BASE = 64      # a[64:127]  dV^T accumulators: DV[db] = a[64 + 16 db : +16]
KB_BASE = 128     # a[128:159] K rows (B operands of S): KB[c] = a[128 + 4 c : +4]
VB_BASE = 160     # a[160:191] V rows (B operands of dP)
QR_BASE = 192     # a[192:207] Q row operand ring
OR_BASE = 208     # a[208:223] dO row operand ring
QT_BASE = 224     # a[224:239] Q^T operand ring (two transpose reads per slot)
OT_BASE = 240     # a[240:255] dO^T operand ring
SP_BASE = 0       # v[0:63]    slot x: S[x] = v[32 x : +16], dP[x] = v[32 x + 16 : +16]
PS_BASE = 64      # v[64:95]   slot x: P[x][cc] = v[64 + 16 x + 4 cc : +4], dS[x][cc] = +8
LV_BASE = 96      # v[96:127]  slot x: L[x] = v[96 + 16 x : +16]
DB_BASE = 128     # v[128:143] -D of the half whose dP products come next (their C input)
RADDR = 160       # v[160:167] Q row-read addresses per d chunk c (stage 0, half 0)
DRADDR = 168      # v[168:175] dO row-read addresses
TADDR = 176       # v[176:183] Q^T transpose-read addresses, index 2 db + hi
TDADDR = 184      # v[184:191] dO^T transpose-read addresses
LADDR = 192       # v192: this wave's L/D area + 16 h (stage 0)
GOFF = 196        # v[196:199] direct-load offsets within a tile (whole tiles)
GOFF_TAIL = 200   # v[200:203] direct-load offsets of the partial last tile
LOFF = 204        # v204: L/D direct-load offset (4 lane), whole tiles
LOFF_TAIL = 205   # v205: the same with the row clamped, partial last tile
TA = 206          # v206: key - 4 h - 64 ts: a score is visible iff TA - 64 j - 32 qb <= off
RANGE = 207       # v207: ... and off < RANGE + that (N - key: queries past N hidden)
NINF = 208        # v208: -inf
TMP = 209         # v[209:216] temporaries of the mask test

RING = 4          # slots per operand ring
LEAD = 5          # products between an operand's read and its product

S_QPTR = 60       # s[60:61] global address of the next Q tile to load
S_OPTR = 62       # s[62:63] the same for dO
S_M0Q = 64        # LDS byte address of this wave's slice of Q stage 0
S_M0O = 65        # ... of dO stage 0
S_C = 66          # scale * log2(e) (fp32 bits)
S_LAST = 67       # relative index of the last query tile
S_KEND = 68       # steps j >= this load no tile (tile j + 3 does not exist)
S_TAILJ = 69      # step whose loads are the partial last tile (~0 when none)
S_MLO = 70        # tiles before this need a mask (causal diagonal)
S_J = 71          # relative index of the current query tile
S_MHI = 72        # tiles from this on need a mask (partial last tile)
S_T = 73          # scratch
S_MASK = (74, 76, 78, 80)
S_FAST = 82       # straight steps: S_MLO <= j < S_FAST
NLOAD = 10        # direct loads of one tile step (Q 4, dO 4, L 1, D 1)
S_LPTR = 84       # s[84:85] global address of the next L row
S_DPTR = 86       # s[86:87] ... of the next D row
S_M0L = 88        # LDS byte address of this wave's L/D area of stage 0
S_MASK0 = 89      # nonzero: the first tile needs a mask

NPAR = 4
Q_STAGE = 16384        # Q stage s at 16 KiB s
O_STAGE0 = 65536       # dO stage s at 64 KiB + 16 KiB s
L_STAGE0 = 131072      # L/D stage s at 128 KiB + 2 KiB s; wave w at + 512 w, D at + 256
LD_STAGE = 2048
TILE_BYTES = 64 * 256
ROW_BYTES = 64 * 4


def s_reg(x, r):
    return SP_BASE + 32 * x + r


def dp_reg(x, r):
    return SP_BASE + 32 * x + 16 + r


def p_reg(x, cc):
    return PS_BASE + 16 * x + 4 * cc


def ds_reg(x, cc):
    return PS_BASE + 16 * x + 8 + 4 * cc


def l_reg(x, r):
    return LV_BASE + 16 * x + r


# --------------------------------------------------------------- operands
def row_read(which, c, stage, half):
    """Q (which = "Q") or dO row operand of d chunk c for query half `half`
    into its ring slot c % RING."""
    base, addr = (QR_BASE, RADDR) if which == "Q" else (OR_BASE, DRADDR)
    slot = base + 4 * (c % RING)
    off = Q_STAGE * stage + 8192 * half
    return Ins(f"ds_read_b128 {ar(slot, 4)}, {v(addr + c)} offset:{off}", "lds",
               regs_a(slot, 4), [v(addr + c)])


def tr_reads(which, o, stage, half):
    """Q^T or dO^T operand o = (cc = o // 4, db = o % 4) of query half
    `half`: two transpose reads into ring slot o % RING."""
    cc, db = o // 4, o % 4
    base, addr = (QT_BASE, TADDR) if which == "Q" else (OT_BASE, TDADDR)
    slot = base + 4 * (o % RING)
    off = Q_STAGE * stage + (32 * half + 16 * cc) * 256
    return [Ins(f"ds_read_b64_tr_b16 {ar(slot + 2 * hi, 2)}, {v(addr + 2 * db + hi)} offset:{off}",
                "lds", regs_a(slot + 2 * hi, 2), [v(addr + 2 * db + hi)]) for hi in range(2)]


def lv_reads(stage, half, x):
    """L of query half `half` into slot x: register 4g + e holds query
    32 half + 8 g + 4 h + e (the row of the score products' results)."""
    out = []
    for g in range(4):
        off = LD_STAGE * stage + 4 * (32 * half + 8 * g)
        out.append((("L", g), Ins(f"ds_read_b128 {vr(l_reg(x, 4 * g), 4)}, {v(LADDR)} offset:{off}",
                                  "lds", regs_v(l_reg(x, 4 * g), 4), [v(LADDR)])))
    return out


def d_reads(stage, half):
    """-D of query half `half` (the delta pass stores it negated) into the
    C input of the half's first dP product, laid out as its results, so that
    the products leave dP - D."""
    out = []
    for g in range(4):
        off = LD_STAGE * stage + 4 * (32 * half + 8 * g) + 256
        out.append((("D", g), Ins(f"ds_read_b128 {vr(DB_BASE + 4 * g, 4)}, {v(LADDR)} offset:{off}",
                                  "lds", regs_v(DB_BASE + 4 * g, 4), [v(LADDR)])))
    return out


def sdp_mfma(which, c, dst):
    """S (which = "Q") or dP (which = "O") product of d chunk c into slot
    dst; the dP chain starts from -D (DB_BASE), the S chain from 0."""
    d0 = s_reg(dst, 0) if which == "Q" else dp_reg(dst, 0)
    ring = QR_BASE if which == "Q" else OR_BASE
    slot = ring + 4 * (c % RING)
    b = (KB_BASE if which == "Q" else VB_BASE) + 4 * c
    cin = d0 if c else (DB_BASE if which == "O" else None)
    src_c = "0" if cin is None else vr(cin, 16)
    return Ins(f"v_mfma_f32_32x32x16_bf16 {vr(d0, 16)}, {ar(slot, 4)}, {ar(b, 4)}, {src_c}",
               "mfma", regs_v(d0, 16), regs_a(slot, 4) + regs_a(b, 4),
               regs_v(cin, 16) if cin is not None else [])


def grad_mfma(which, o, src):
    """dV^T[db] += dO^T (cc, db) P[src][cc] (which = "O"), or dK^T[db] +=
    Q^T (cc, db) dS[src][cc] (which = "Q"); o = 4 cc + db."""
    cc, db = o // 4, o % 4
    ring = OT_BASE if which == "O" else QT_BASE
    slot = ring + 4 * (o % RING)
    dst = (DV_BASE if which == "O" else DK_BASE) + 16 * db
    b = p_reg(src, cc) if which == "O" else ds_reg(src, cc)
    return Ins(f"v_mfma_f32_32x32x16_bf16 {ar(dst, 16)}, {ar(slot, 4)}, {vr(b, 4)}, {ar(dst, 16)}",
               "mfma", regs_a(dst, 16), regs_a(slot, 4) + regs_v(b, 4), regs_a(dst, 16))


# ----------------------------------------------------------- vector work
def mask_ops(x, half):
    """Scores of slot x (query half `half` of the current tile j, or of tile
    j + 1 when x = 0 in step 2: the caller sets s73 = 64 j' + 32 half) whose
    key follows the query or whose query lies past N become -inf.  Element r
    holds query q0 + 8 (r / 4) + 4 h + r % 4 =: q0 + 4 h + off; it is visible
    iff (off - thr) < RANGE unsigned, thr = TA - s73."""
    ops = [Ins(f"v_subrev_u32 {v(TMP + 7)}, s{S_T}, {v(TA)}", "valu", [v(TMP + 7)], [v(TA), f"s{S_T}"])]
    for g in range(0, 16, 4):
        rs = list(range(g, g + 4))
        for i, r in enumerate(rs):
            off = 8 * (r // 4) + r % 4
            ops.append(Ins(f"v_sub_u32 {v(TMP + i)}, {off}, {v(TMP + 7)}", "valu", [v(TMP + i)],
                           [v(TMP + 7)]))
        for i, r in enumerate(rs):
            pr = S_MASK[i]
            ops.append(Ins(f"v_cmp_ge_u32_e64 s[{pr}:{pr + 1}], {v(TMP + i)}, {v(RANGE)}", "valu",
                           [f"s{pr}"], [v(TMP + i), v(RANGE)]))
        for i, r in enumerate(rs):
            pr = S_MASK[i]
            sr = s_reg(x, r)
            ops.append(Ins(f"v_cndmask_b32_e64 {v(sr)}, {v(sr)}, {v(NINF)}, s[{pr}:{pr + 1}]",
                           "valu", [v(sr)], [v(sr), v(NINF), f"s{pr}"]))
    return ops


def elem_half(x):
    """P = exp2(S c - L), dS = P (dP - D) for slot x (the products leave
    dP - D), in place, P and dS packed to bf16 pairs; software-pipelined over
    groups of four elements."""
    groups = []
    for g in range(4):
        rs = list(range(4 * g, 4 * g + 4))
        fma = [Ins(f"v_fma_f32 {v(s_reg(x, r))}, {v(s_reg(x, r))}, s{S_C}, -{v(l_reg(x, r))}",
                   "valu", [v(s_reg(x, r))], [v(s_reg(x, r)), v(l_reg(x, r))]) for r in rs]
        ex = [Ins(f"v_exp_f32 {v(s_reg(x, r))}, {v(s_reg(x, r))}", "trans", [v(s_reg(x, r))],
                  [v(s_reg(x, r))]) for r in rs]
        fin = [Ins(f"v_mul_f32 {v(dp_reg(x, r))}, {v(s_reg(x, r))}, {v(dp_reg(x, r))}", "valu",
                   [v(dp_reg(x, r))], [v(s_reg(x, r)), v(dp_reg(x, r))]) for r in rs]
        for r in (4 * g, 4 * g + 2):
            cc, i = r // 8, (r % 8) // 2
            fin.append(Ins(f"v_cvt_pk_bf16_f32 {v(p_reg(x, cc) + i)}, {v(s_reg(x, r))}, {v(s_reg(x, r + 1))}",
                           "valu", [v(p_reg(x, cc) + i)], [v(s_reg(x, r)), v(s_reg(x, r + 1))]))
            fin.append(Ins(f"v_cvt_pk_bf16_f32 {v(ds_reg(x, cc) + i)}, {v(dp_reg(x, r))}, {v(dp_reg(x, r + 1))}",
                           "valu", [v(ds_reg(x, cc) + i)], [v(dp_reg(x, r)), v(dp_reg(x, r + 1))]))
        groups.append((fma, ex, fin))
    ops = []
    n = len(groups)
    for k in range(n + 2):
        if k < n:
            ops += groups[k][0]
        if 0 <= k - 1 < n:
            ops += groups[k - 1][1]
        if 0 <= k - 2 < n:
            ops += groups[k - 2][2]
    return ops


# ------------------------------------------------------------------ steps
def units_of(sdp, grad):
    """The products of one step with their operand reads: the S/dP products
    of sdp = (stage, half, dst slot) (16, reading Q and dO rows) and the
    dV/dK products of grad = (stage, half, P/dS slot) (16, reading dO^T and
    Q^T).  The two sets touch disjoint registers; pairs of them alternate
    (spreading the row and transpose reads evenly), the gradient pairs one
    pair ahead: their operands are in LDS before the barrier that publishes
    the next tile, so the first products of a tile step need no read issued
    after it."""
    g, sd = [], []
    if grad:
        g_stg, g_half, src = grad
        for i in range(8):
            g.append([(grad_mfma("O", i, src),
                       [(("TO", i, hi), r) for hi, r in enumerate(tr_reads("O", i, g_stg, g_half))]),
                      (grad_mfma("Q", i, src),
                       [(("TQ", i, hi), r) for hi, r in enumerate(tr_reads("Q", i, g_stg, g_half))])])
    if sdp:
        s_stg, s_half, dst = sdp
        for i in range(8):
            dreads = d_reads(s_stg, s_half) if i == 0 else []
            sd.append([(sdp_mfma("Q", i, dst), [(("Q", i), row_read("Q", i, s_stg, s_half))]),
                       (sdp_mfma("O", i, dst), dreads + [(("O", i), row_read("O", i, s_stg, s_half))])])
    if not g or not sd:
        return [u for pair in g + sd for u in pair]
    order = g[:1]
    for i in range(8):
        order += g[i + 1:i + 2] + sd[i:i + 1]
    return [u for pair in order for u in pair]


PRE = 4   # leading gradient products of a tile step whose reads the previous step issues


def pre_rids():
    """Ids of the reads a tile step finds in flight when it starts (issued
    at the end of the step before it, in this order)."""
    return [rid for _, reads in units_of(None, (0, 0, 0))[:PRE] for rid, _ in reads]


def products(st, lds, units, lv, valu, raw_sched=None, pre=0, nxt=None):
    """Issue `units` (a list from units_of) with `valu` in the issue slots
    beside them.  Each product's operand reads go out LEAD products ahead of
    it: the reads of the first `pre` units were issued before this call, and
    the reads of the first nxt[0] units of the list nxt[1] (the next call's)
    go out in this call's last products.  The L/D reads lv = (stage, half,
    slot) for the next step's vector work go out one every other product."""
    mf = [m for m, _ in units]
    need = {p: {rid for rid, _ in reads} for p, (_, reads) in enumerate(units)}
    before, sched = [], {}
    for p, (_, reads) in enumerate(units):
        if p < pre:
            continue
        if p < LEAD:
            before += reads
        else:
            sched.setdefault(p - LEAD, []).extend(reads)
    if nxt:
        n, later = nxt
        for p in range(n):
            sched.setdefault(len(mf) - LEAD + p, []).extend(later[p][1])
    if lv:
        stg, half, x = lv
        for i, rd in enumerate(lv_reads(stg, half, x)):
            sched.setdefault(min(2 * i + 1, len(mf) - LEAD - 1), []).append(rd)
    F.interleave_even(st, mf, before, valu, lds, sched, need, raw_sched=raw_sched, gap=GAP,
                      init=INIT)


GAP = 28.0        # most issue cycles of other work between two products
INIT = 0.0        # vector work before the first product of a call


def end_step(st, lds, last):
    """Wait for every LDS read but the next step's first operands (none
    after the last step), which must be the last reads in flight."""
    keep = [] if last else pre_rids()
    assert lds.pending[len(lds.pending) - len(keep):] == keep, lds.pending
    st.raw(f"s_waitcnt lgkmcnt({len(keep)})")
    lds.pending = list(keep)


def wait_lv(st, lds, lv):
    """Wait until the L/D reads lv = (stage, half, slot) have landed."""
    stg, half, x = lv
    k = lds.wait_for({rid for rid, _ in lv_reads(stg, half, x)})
    if k is not None:
        st.raw(f"s_waitcnt lgkmcnt({min(k, 15)})")


def full_loads(stage):
    """Whole-tile direct loads of Q, dO (four each) and the L, D rows (one
    each) into `stage`, and the pointer steps to the next tile."""
    pre_q = [f"s_add_u32 m0, s{S_M0Q}, {Q_STAGE * stage}"]
    q = [f"global_load_lds_dwordx4 {v(GOFF + i)}, s[{S_QPTR}:{S_QPTR + 1}] offset:{1024 * i}"
         for i in range(4)]
    pre_o = [f"s_add_u32 m0, s{S_M0O}, {Q_STAGE * stage}"]
    o = [f"global_load_lds_dwordx4 {v(GOFF + i)}, s[{S_OPTR}:{S_OPTR + 1}] offset:{1024 * i}"
         for i in range(4)]
    pre_l = [f"s_add_u32 m0, s{S_M0L}, {LD_STAGE * stage}"]
    ld = [f"global_load_lds_dword {v(LOFF)}, s[{S_LPTR}:{S_LPTR + 1}]",
          f"global_load_lds_dword {v(LOFF)}, s[{S_DPTR}:{S_DPTR + 1}] offset:256"]
    post = [f"s_add_u32 s{S_QPTR}, s{S_QPTR}, {TILE_BYTES}", f"s_addc_u32 s{S_QPTR + 1}, s{S_QPTR + 1}, 0",
            f"s_add_u32 s{S_OPTR}, s{S_OPTR}, {TILE_BYTES}", f"s_addc_u32 s{S_OPTR + 1}, s{S_OPTR + 1}, 0",
            f"s_add_u32 s{S_LPTR}, s{S_LPTR}, {ROW_BYTES}", f"s_addc_u32 s{S_LPTR + 1}, s{S_LPTR + 1}, 0",
            f"s_add_u32 s{S_DPTR}, s{S_DPTR}, {ROW_BYTES}", f"s_addc_u32 s{S_DPTR + 1}, s{S_DPTR + 1}, 0"]
    return pre_q, q, pre_o, o, pre_l, ld, post


def tail_loads(stage):
    out = []
    for sm0, ptr in ((S_M0Q, S_QPTR), (S_M0O, S_OPTR)):
        for i in range(4):
            out += [f"s_add_u32 m0, s{sm0}, {Q_STAGE * stage + 1024 * i}", "s_nop 0",
                    f"global_load_lds_dwordx4 {v(GOFF_TAIL + i)}, s[{ptr}:{ptr + 1}]"]
    out += [f"s_add_u32 m0, s{S_M0L}, {LD_STAGE * stage}", "s_nop 0",
            f"global_load_lds_dword {v(LOFF_TAIL)}, s[{S_LPTR}:{S_LPTR + 1}]",
            f"global_load_lds_dword {v(LOFF_TAIL)}, s[{S_DPTR}:{S_DPTR + 1}] offset:256"]
    return out


def load_block(st, stage, uid):
    """Loads of tile j + 3 in a body other than the straight one: none past
    the end, the clamped ones for the partial last tile, else whole."""
    skip, tail, done = f"FK_SKIP{uid}_%=", f"FK_TAIL{uid}_%=", f"FK_LDONE{uid}_%="
    st.raw(f"s_cmp_ge_u32 s{S_J}, s{S_KEND}")
    st.raw(f"s_cbranch_scc1 {skip}")
    st.raw(f"s_cmp_eq_u32 s{S_J}, s{S_TAILJ}")
    st.raw(f"s_cbranch_scc1 {tail}")
    pre_q, q, pre_o, o, pre_l, ld, post = full_loads(stage)
    for l in pre_q + ["s_nop 0"] + q + pre_o + ["s_nop 0"] + o + pre_l + ["s_nop 0"] + ld + post:
        st.raw(l)
    st.raw(f"s_branch {done}")
    st.label(tail)
    for l in tail_loads(stage):
        st.raw(l)
    st.label(done)
    st.label(skip)


def mask_setup(st, extra):
    """s73 = 64 (j + extra_tiles) + 32 half for the mask of the next
    vector work (extra = 64 * tiles + 32 * half)."""
    st.raw(f"s_lshl_b32 s{S_T}, s{S_J}, 6")
    if extra:
        st.raw(f"s_add_u32 s{S_T}, s{S_T}, {extra}")


def iteration(out, p, kind, name):
    """Query tile step j (j % 4 = p): kind "fast", "gen", "masked" or "final"."""
    st = Stream(out)
    lds = LdsCounter()
    lds.pending = pre_rids()
    sj, sn, sl = p % 4, (p + 1) % 4, (p + 3) % 4
    final = kind == "final"
    masked = kind in ("masked", "final")
    raw = None
    if kind == "fast":
        pre_q, q, pre_o, o, pre_l, ld, post = full_loads(sl)
        step = [f"s_add_u32 s{S_J}, s{S_J}, 1", f"s_cmp_lt_u32 s{S_J}, s{S_FAST}"]
        raw = {0: pre_q, 1: q[:1], 2: q[1:2], 3: q[2:3], 4: q[3:] + pre_o, 5: o[:1], 6: o[1:2],
               7: o[2:3], 8: o[3:] + pre_l, 9: ld[:1], 10: ld[1:] + post + step}
    elif kind in ("gen", "masked"):
        load_block(st, sl, name)
    # step 1: vector work of (j, second half); dV/dK of (j, first half);
    # S/dP of (j + 1, first half); L/D of (j + 1, first half)
    u1 = units_of(None if final else (sn, 0, 0), (sj, 0, 0))
    u2 = units_of(None if final else (sn, 1, 1), (sj, 1, 1))
    lv1 = None if final else (sn, 0, 0)
    if masked:
        mask_setup(st, 32)
    valu = (mask_ops(1, 1) if masked else []) + elem_half(1)
    products(st, lds, u1, lv1, valu, raw, pre=PRE, nxt=(LEAD, u2))
    # step 2: vector work of (j + 1, first half); dV/dK of (j, second half);
    # S/dP of (j + 1, second half); L/D of (j + 1, second half); the reads
    # of the next step's first gradient products
    if not final:
        wait_lv(st, lds, lv1)
    if masked and not final:
        mask_setup(st, 64)
    valu = [] if final else ((mask_ops(0, 0) if masked else []) + elem_half(0))
    nxt = None if final else (PRE, units_of(None, (sn, 0, 0)))
    products(st, lds, u2, None if final else (sn, 1, 1), valu, pre=LEAD, nxt=nxt)
    end_step(st, lds, final)
    # tile j + 2 (loaded by the step before) must have landed before the
    # barrier publishes it; this step's loads (tile j + 3) may stay in flight
    if kind == "fast":
        st.raw(f"s_waitcnt vmcnt({NLOAD})")
    elif kind == "final":
        st.raw("s_waitcnt vmcnt(0)")
    else:
        none, done = f"FK_VM0{name}_%=", f"FK_VMD{name}_%="
        st.raw(f"s_cmp_ge_u32 s{S_J}, s{S_KEND}")
        st.raw(f"s_cbranch_scc1 {none}")
        st.raw(f"s_waitcnt vmcnt({NLOAD})")
        st.raw(f"s_branch {done}")
        st.label(none)
        st.raw("s_waitcnt vmcnt(0)")
        st.label(done)
    st.raw("s_barrier")


def entry(out):
    """Query tile 0: its first half's L/D and S/dP products, that half's mask
    when the tile needs one, its vector work beside the second half's S/dP
    products and L/D reads and the reads of the first step's first gradient
    products.  The dK/dV accumulators come in holding the sums so far (zero
    for an item's first query head; with grouped heads the statement runs
    once per query head of the group)."""
    st = Stream(out)
    st.raw("s_nop 4")
    lds = LdsCounter()
    u1, u2 = units_of((0, 0, 0), None), units_of((0, 1, 1), None)
    products(st, lds, u1, (0, 0, 0), [], nxt=(LEAD, u2))
    wait_lv(st, lds, (0, 0, 0))
    st.raw("s_nop 7", 8)
    st.raw("s_nop 7", 8)
    st.raw("s_nop 3", 4)
    skip = "FK_EMASK_%="
    st.raw(f"s_cmp_eq_u32 s{S_MASK0}, 0")
    st.raw(f"s_cbranch_scc1 {skip}")
    st.raw(f"s_mov_b32 s{S_T}, 0")
    for ins in mask_ops(0, 0):
        st.emit(ins)
    st.label(skip)
    products(st, lds, u2, (0, 1, 1), elem_half(0), pre=LEAD, nxt=(PRE, units_of(None, (0, 0, 0))))
    end_step(st, lds, False)


def generate():
    out = []
    entry(out)
    for p in range(NPAR):
        q = (p + 1) % NPAR
        out.append(f"FK_L{p}_%=:")
        out.append(f"s_cmp_lt_u32 s{S_J}, s{S_FAST}")
        out.append(f"s_cbranch_scc0 FK_GEN{p}_%=")
        out.append(f"s_cmp_lt_u32 s{S_J}, s{S_MLO}")
        out.append(f"s_cbranch_scc1 FK_GEN{p}_%=")
        out.append(f"FK_BODY{p}_%=:")
        iteration(out, p, "fast", f"F{p}")
        out.append(f"s_cbranch_scc1 FK_BODY{q}_%=")
        out.append(f"s_branch FK_GEN{q}_%=")
        out.append(f"FK_GEN{p}_%=:")
        out.append(f"s_cmp_eq_u32 s{S_J}, s{S_LAST}")
        out.append(f"s_cbranch_scc1 FK_FIN{p}_%=")
        out.append(f"s_cmp_lt_u32 s{S_J}, s{S_MLO}")
        out.append(f"s_cbranch_scc1 FK_ITM{p}_%=")
        out.append(f"s_add_u32 s{S_T}, s{S_J}, 1")
        out.append(f"s_cmp_ge_u32 s{S_T}, s{S_MHI}")
        out.append(f"s_cbranch_scc1 FK_ITM{p}_%=")
        out.append(f"FK_GB{p}_%=:")
        iteration(out, p, "gen", f"G{p}")
        out.append(f"s_add_u32 s{S_J}, s{S_J}, 1")
        out.append(f"s_branch FK_L{q}_%=")
        out.append(f"FK_ITM{p}_%=:")
        iteration(out, p, "masked", f"M{p}")
        out.append(f"s_add_u32 s{S_J}, s{S_J}, 1")
        out.append(f"s_branch FK_L{q}_%=")
    for p in range(NPAR):
        out.append(f"FK_FIN{p}_%=:")
        iteration(out, p, "final", f"N{p}")
        out.append("s_branch FK_DONE_%=")
    out.append("FK_DONE_%=:")
    out.append("s_nop 7")
    out.append("s_nop 7")
    out.append("s_nop 7")
    return out


def clobbers():
    regs = [f"v{i}" for i in range(0, LV_BASE + 64)]   # S/dP, P/dS, L slots, -D, v[144:159]
    regs += [f"v{i}" for i in range(TMP, TMP + 8)]
    regs += [f"a{i}" for i in range(QR_BASE, 256)]     # operand rings
    regs += [f"s{i}" for i in range(S_T, S_T + 9)]
    regs += ["vcc", "scc", "m0", "memory"]
    return regs


def render(lines):
    body = "\n".join(f'  "{l}\\n"' for l in lines)
    clob = ", ".join(f'"{r}"' for r in clobbers())
    return (
        "// Generated by gen_bwd_dkdv128.py -- do not edit.  The query loop of\n"
        "// bwd_dkdv128_kernel (fa_bwd_dkdv128.hip): see the generator for the schedule.\n"
        "#define FA_BWD_DKDV128_LOOP_ASM \\\n" + body.replace("\n", " \\\n") + "\n\n"
        "#define FA_BWD_DKDV128_LOOP_CLOBBERS " + clob + "\n"
        f"// {len(lines)} lines\n")


def main():
    lines = generate()
    text = render(lines)
    if len(sys.argv) > 1 and sys.argv[1] == "--check":
        cur = open(OUT).read() if os.path.exists(OUT) else ""
        sys.exit(0 if cur == text else 1)
    with open(OUT, "w") as f:
        f.write(text)
    print(f"wrote {OUT}: {len(lines)} lines")


if __name__ == "__main__":
    main()
