"""Host-side model of the generated main loops of the d = 128 and d = 64
forward kernels (exact_io_aware_45_amd/csrc/gen_fwd128.py -> fa_fwd128_loop.inc,
fa_fwd64_loop.inc, fa_fwd64w2_loop.inc), CPU only.

The emitted instruction text is parsed and executed on a model of one
workgroup's LDS and registers:
  * the direct loads (global offsets from the kernel's formula, LDS
    destinations from the emitted M0 values) stage a K and a V tile;
  * every K operand read (ds_read_b128) and V^T operand read
    (ds_read_b64_tr_b16, with the transpose-read lane semantics measured on
    the device) is followed into the product that consumes it, and each
    lane's operand must be exactly the tile elements that the product's
    register layout needs (the layouts recorded in fa_common.hpp);
  * every product's LDS operand must have landed by the emitted s_waitcnt,
    no ring slot is overwritten while a product may still read it, every
    barrier is preceded by vmcnt(0), and the emitted wait states cover the
    matrix/vector hazards;
  * the scalar control flow of the whole statement, executed for many
    sequence lengths, loads every tile once and in order (whole tiles through
    the plain offsets, only a partial last tile through the clamped ones),
    masks exactly the tiles holding an invisible key, and takes the straight
    body exactly where it applies.
"""
import importlib.util
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", "gen_fwd128.py")
# generated loops: head dim and waves per workgroup ("64w2": d = 64, 2 waves)
VARIANTS = {128: (128, 4), 64: (64, 4), "64w2": (64, 2)}
DIMS = list(VARIANTS)


def load_gen(d, nw):
    spec = importlib.util.spec_from_file_location(f"gen_fwd_sched{d}w{nw}", GEN)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.configure(d, nw)
    return mod


def swz_of(D):
    """Chunk swizzle of an LDS tile row (tile_swz in fa_common.hpp)."""
    if D == 128:
        return lambda r: 4 * (r & 3) + ((r >> 2) & 3)
    return lambda r: 4 * ((r >> 1) & 1) + ((r >> 2) & 3)


class Loop:
    """One generated statement (head dim, waves per workgroup) and the
    kernel's per-lane values."""

    def __init__(self, key):
        d, nw = VARIANTS[key]
        self.D, self.NW, self.BR = d, nw, 64 * nw
        self.G = load_gen(d, nw)
        self.LINES = self.G.generate()
        self.NC, self.NDB = d // 16, d // 32
        self.NLOAD = 64 * d * 2 // 1024 // nw   # 1 KiB direct loads per wave and tile
        self.LPR = d // 8                 # 16-byte chunks per tile row
        self.RPL = 64 // self.LPR         # tile rows per direct load
        self.RW = 64 // nw                # tile rows each wave loads
        self.STAGE = 64 * d * 2           # bytes of one K or V stage
        self.WAVE = self.RW * d * 2       # bytes of one wave's rows of a tile
        self.M0K = 2 * self.STAGE         # LDS byte address of K stage 0 (+ wave * WAVE in s64)
        self.M0V = 0
        self.swz = swz_of(d)
        self.KADDR, self.VADDR, self.GOFF = self.kernel_offsets()

    def kernel_offsets(self):
        """Per-lane values the kernel computes before the loop (restated from
        fa_fwd128.hip / fa_fwd64.hip): K read addresses (stage 0), V^T read
        addresses (stage 0), direct-load offsets, in bytes relative to the
        start of LDS / of a tile."""
        D, tile_swz = self.D, self.swz
        kaddr = np.zeros((self.NC, 64), np.int64)
        vaddr = np.zeros((2 * self.NDB, 64), np.int64)
        TILE = 64 * D
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            sw_row = tile_swz(l32)
            for c in range(self.NC):
                kaddr[c, lane] = 2 * (2 * TILE + l32 * D + 8 * ((2 * c + h) ^ sw_row))
            tr_row = 4 * h + ((lane & 15) >> 2)
            tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
            sw_lo, sw_hi = tile_swz(tr_row), tile_swz(tr_row + 8)
            tq, te = tr_col >> 3, tr_col & 7

            def tr_off(row, sw, b):
                return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te
            for db in range(self.NDB):
                vaddr[2 * db, lane] = 2 * tr_off(tr_row, sw_lo, db)
                vaddr[2 * db + 1, lane] = 2 * tr_off(tr_row + 8, sw_hi, db)
        goff = np.zeros((self.NW, self.NLOAD, 64), np.int64)   # [wave][load][lane]
        for w in range(self.NW):
            for i in range(self.NLOAD):
                for lane in range(64):
                    row = self.RW * w + self.RPL * i + lane // self.LPR
                    col = 8 * ((lane % self.LPR) ^ tile_swz(row))
                    goff[w, i, lane] = 2 * (row * D + col) - 1024 * i
        return kaddr, vaddr, goff

    def section(self, start_label, end_marker):
        """Lines from a label up to (excluding) the first line starting with end_marker."""
        i = self.LINES.index(start_label)
        out = []
        for l in self.LINES[i + 1:]:
            if l.startswith(end_marker):
                break
            out.append(l)
        return out


LOOPS = {key: Loop(key) for key in DIMS}


@pytest.mark.parametrize("d", DIMS)
def test_committed_loop_matches_the_generator(d):
    L = LOOPS[d]
    text = L.G.render(L.LINES)
    assert open(L.G.OUT).read() == text, f"{L.G.OUT} is stale: rerun gen_fwd128.py"


# ------------------------------------------------------------- parsing
REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+))")


def regs(operand):
    m = REG.fullmatch(operand.strip().lstrip("-"))
    if not m:
        return []
    kind = m.group(1)
    if m.group(4) is not None:
        return [f"{kind}{m.group(4)}"]
    lo, hi = int(m.group(2)), int(m.group(3))
    return [f"{kind}{i}" for i in range(lo, hi + 1)]


def split(line):
    """(opcode, operands); a trailing ` offset:N` becomes its own operand."""
    op, _, rest = line.partition(" ")
    args = [x.strip() for x in rest.split(",")] if rest else []
    if args and " offset:" in args[-1]:
        reg, _, off = args[-1].partition(" offset:")
        args[-1:] = [reg.strip(), "offset:" + off.strip()]
    return op, args


# --------------------------------------------------------- lane-level model
NONE = 0xFFFFFFFF


def follow(lines, env):
    """The lines a body executes for the given scalar registers: compares and
    branches are evaluated (a branch to a label outside `lines` ends the
    path); every other line is kept in order."""
    labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":")}
    out, pc, scc = [], 0, None
    while pc < len(lines):
        l = lines[pc]
        pc += 1
        op, args = split(l)
        if op.startswith("s_cmp_"):
            x, y = (env[int(t[1:])] if t.startswith("s") else int(t, 0) for t in args[:2])
            scc = {"s_cmp_eq_u32": x == y, "s_cmp_lg_u32": x != y, "s_cmp_ge_u32": x >= y,
                   "s_cmp_lt_u32": x < y, "s_cmp_gt_u32": x > y}[op]
        elif op in ("s_cbranch_scc0", "s_cbranch_scc1"):
            assert scc is not None, l
            if scc == (op == "s_cbranch_scc1"):
                if args[0] + ":" not in lines:
                    break
                pc = labels[args[0]]
            continue
        elif op == "s_branch":
            if args[0] + ":" not in lines:
                break
            pc = labels[args[0]]
            continue
        elif op in ("s_add_u32", "s_addc_u32"):
            scc = None     # carry, not a comparison
        out.append(l)
    return out


# the load cases of one step, tile j = 5: whole loads, the clamped K tile,
# no K tile, or no K tile and the clamped V tile (SGPR numbers are the same
# at both head dims)
def load_cases(G):
    return {
        "whole": {G.S_KEND: 10, G.S_KTAILJ: NONE, G.S_VTAILJ: NONE},
        "ktail": {G.S_KEND: 10, G.S_KTAILJ: 5, G.S_VTAILJ: NONE},
        "kskip": {G.S_KEND: 5, G.S_KTAILJ: NONE, G.S_VTAILJ: NONE},
        "vtail": {G.S_KEND: 5, G.S_KTAILJ: NONE, G.S_VTAILJ: 5},
    }


def env_of(L, case):
    G = L.G
    return {**load_cases(G)[case], G.S_J: 5, G.S_FAST: 0, G.S_LAST: 11}


def stage_tiles(L, lines, ktile, vtile, tail_offs=None):
    """Execute the direct loads in `lines` for all waves into a 64 KiB LDS
    image (uint16 elements): whole-tile loads use the kernel's offsets, the
    clamped ones `tail_offs`; the instruction offset applies to both
    addresses.  Returns the image and {(K|V, stage, clamped)} loaded."""
    G = L.G
    lds = np.full(32768, -1, np.int64)
    loaded = set()
    for w in range(L.NW):
        m0 = None
        for l in lines:
            op, args = split(l)
            if op == "s_add_u32" and args[0] == "m0":
                m0 = {"s64": L.M0K, "s65": L.M0V}[args[1]] + L.WAVE * w + int(args[2])
            elif op == "global_load_lds_dwordx4":
                reg = int(args[0][1:])
                clamped = reg >= G.GOFF_TAIL
                i = reg - (G.GOFF_TAIL if clamped else G.GOFF)
                assert 0 <= i < L.NLOAD, l
                off = int(args[2].split(":")[1]) if len(args) > 2 else 0
                offs = tail_offs if clamped else L.GOFF
                is_k = args[1] == f"s[{G.S_KPTR}:{G.S_KPTR + 1}]"
                flat = (ktile if is_k else vtile).reshape(-1)
                for lane in range(64):
                    src = (offs[w, i, lane] + off) // 2
                    dst = (m0 + off + 16 * lane) // 2
                    assert 0 <= src and src + 8 <= flat.size
                    lds[dst:dst + 8] = flat[src:src + 8]
                base = L.M0K if is_k else L.M0V
                loaded.add(("K" if is_k else "V", (m0 - base - L.WAVE * w) // L.STAGE, clamped))
    return lds, loaded


def tr_read(lds, addrs):
    """ds_read_b64_tr_b16: in each 16-lane group, lane i receives element
    (i % 4) of the 8-byte chunk addressed by lane 4t + i / 4, t = 0..3."""
    out = np.zeros((64, 4), np.int64)
    for lane in range(64):
        g, i = lane // 16, lane % 16
        for t in range(4):
            src = addrs[16 * g + 4 * t + i // 4] // 2
            out[lane, t] = lds[src + i % 4]
    return out


def run_operand_model(L, body, kstage, vstage):
    """Follow every LDS operand read of `body` into its product and check the
    operand each lane receives."""
    G, D = L.G, L.D
    # element values encode (row, col) so every mismatch is visible
    ktile = np.arange(64 * D).reshape(64, D) + 10 ** 6
    vtile = np.arange(64 * D).reshape(64, D) + 2 * 10 ** 6
    lds = np.full(32768, -1, np.int64)
    # place the tiles the way the direct loads do (checked separately)
    for r in range(64):
        for q in range(L.LPR):
            slot = q ^ L.swz(r)
            kdst = (L.M0K + kstage * L.STAGE) // 2 + r * D + 8 * slot
            vdst = (L.M0V + vstage * L.STAGE) // 2 + r * D + 8 * slot
            lds[kdst:kdst + 8] = ktile[r, 8 * q:8 * q + 8]
            lds[vdst:vdst + 8] = vtile[r, 8 * q:8 * q + 8]
    ring = {}   # agpr -> per-lane values (one column per register half)
    checked = {"k": 0, "v": 0}
    for l in body:
        op, args = split(l)
        if op == "ds_read_b128":
            dst = regs(args[0])
            c = int(args[1][1:]) - G.KADDR
            assert 0 <= c < L.NC, l
            off = int(args[2].split(":")[1]) if len(args) > 2 else 0
            assert (off // L.STAGE) == kstage
            vals = np.zeros((64, 8), np.int64)
            for lane in range(64):
                a0 = (L.KADDR[c, lane] + off) // 2
                vals[lane] = lds[a0:a0 + 8]
            ring[dst[0]] = ("K", vals)
        elif op == "ds_read_b64_tr_b16":
            dst = regs(args[0])
            idx = int(args[1][1:]) - G.VADDR
            assert 0 <= idx < 2 * L.NDB, l
            off = int(args[2].split(":")[1]) if len(args) > 2 else 0
            assert (off // L.STAGE) == vstage
            vals = tr_read(lds, L.VADDR[idx] + off)
            ring[dst[0]] = ("V", vals)
        elif op == "v_mfma_f32_32x32x16_bf16":
            dst, sa, sb = regs(args[0]), regs(args[1]), regs(args[2])
            if sa[0].startswith("a") and int(sa[0][1:]) >= G.VR_BASE:
                # P V product: O[rb][db] += V^T P^T
                lo = ring[sa[0]]
                hi = ring[sa[2]]
                assert lo[0] == "V" and hi[0] == "V"
                A = np.concatenate([lo[1], hi[1]], axis=1)   # lane x 8 (k = 8h + t)
                o = int(dst[0][1:]) - G.O_BASE
                rb, db = o // (16 * L.NDB), (o % (16 * L.NDB)) // 16
                assert rb < 2
                p = int(sb[0][1:])
                pb = 0 if p < G.P_BASE[1] else 1
                rel = p - G.P_BASE[pb]
                assert rel // 16 == rb
                kb, cc = (rel % 16) // 8, (rel % 8) // 4
                for lane in range(64):
                    h = lane >> 5
                    for t in range(8):
                        key = 32 * kb + 16 * cc + (8 if t >= 4 else 0) + 4 * h + t % 4
                        assert A[lane, t] == vtile[key, 32 * db + (lane & 31)], (l, lane, t)
                checked["v"] += 1
            else:
                # score product: S[rb][kb] (+)= K Q^T
                kv = ring[sa[0]]
                assert kv[0] == "K"
                q = int(sb[0][1:]) - G.Q_BASE
                rb, c = q // (4 * L.NC), (q % (4 * L.NC)) // 4
                assert rb < 2
                s = int(dst[0][1:])
                buf = 0 if s < G.S_BASE[1] else 1
                rel = s - G.S_BASE[buf]
                assert rel // 32 == rb
                kb = (rel % 32) // 16
                if args[3].strip() == "0":
                    assert c == 0
                for lane in range(64):
                    h, l32 = lane >> 5, lane & 31
                    assert np.array_equal(kv[1][lane], ktile[32 * kb + l32, 16 * c + 8 * h:
                                                             16 * c + 8 * h + 8]), (l, lane)
                checked["k"] += 1
    return checked


BODIES = {  # name: (label, K read stage, V read stage, K load stage, V load stage, final)
    "A": ("FA_BODYA_%=:", 1, 0, 0, 1, False), "B": ("FA_BODYB_%=:", 0, 1, 1, 0, False),
    "GA": ("FA_GBA_%=:", 1, 0, 0, 1, False), "GB": ("FA_GBB_%=:", 0, 1, 1, 0, False),
    "MA": ("FA_ITMA_%=:", 1, 0, 0, 1, False), "MB": ("FA_ITMB_%=:", 0, 1, 1, 0, False),
    "FA": ("FA_FINA_%=:", 1, 0, 0, 1, True), "FB": ("FA_FINB_%=:", 0, 1, 1, 0, True),
}
# the load cases each body can meet: the straight body only whole tiles, the
# general unmasked one never the clamped V tile (tile j + 1 would be masked)
ALL_CASES = ["whole", "ktail", "kskip", "vtail"]
BODY_CASES = {"A": ["whole"], "B": ["whole"], "GA": ["whole", "ktail", "kskip"],
              "GB": ["whole", "ktail", "kskip"], "MA": ALL_CASES, "MB": ALL_CASES,
              "FA": ["whole"], "FB": ["whole"]}


# idle steps (a wave past its last visible tile): loads and the barrier only
IDLE = {"IA": ("FA_IDLEA_%=:", None, None, 0, 1, False),
        "IB": ("FA_IDLEB_%=:", None, None, 1, 0, False)}
BODY_CASES.update({"IA": ALL_CASES, "IB": ALL_CASES})


def body_of(L, name):
    label = (BODIES.get(name) or IDLE[name])[0]
    return L.section(label, "s_barrier")


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("name", list(BODIES))
def test_operands_of_every_product(name, d):
    L = LOOPS[d]
    _, kst, vst, _, _, final = BODIES[name]
    checked = run_operand_model(L, body_of(L, name), kst, vst)
    nk, nv = 4 * L.NC, 8 * L.NDB
    assert checked == ({"k": 0, "v": nv} if final else {"k": nk, "v": nv})


@pytest.mark.parametrize("d", DIMS)
def test_operands_of_the_first_tile_scores(d):
    """The entry computes tile 0's scores from K stage 0."""
    L = LOOPS[d]
    body = L.LINES[:L.LINES.index("s_cbranch_scc1 FA_EMASK_%=")]
    checked = run_operand_model(L, body, 0, 0)
    assert checked == {"k": 4 * L.NC, "v": 0}


def tail_offsets(L, N, tlast):
    """Clamped direct-load offsets of the partial last tile (the kernel's
    formula): rows past N - 1 repeat row N - 1."""
    out = np.zeros((L.NW, L.NLOAD, 64), np.int64)
    for w in range(L.NW):
        for i in range(L.NLOAD):
            for lane in range(64):
                row = L.RW * w + L.RPL * i + lane // L.LPR
                col = 8 * ((lane % L.LPR) ^ L.swz(row))
                out[w, i, lane] = 2 * ((min(tlast * 64 + row, N - 1) - tlast * 64) * L.D + col)
    return out


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("name,case", [(n, c) for n in list(BODIES) + list(IDLE)
                                       for c in BODY_CASES[n]])
def test_direct_loads_place_tiles_as_the_reads_expect(name, case, d):
    """The emitted loads (M0 values, offset registers, instruction offsets)
    write chunk q of tile row r to slot q ^ swz(r) of the right stage, for
    all waves, and cover each loaded stage exactly once; a partial last
    tile (here 37 rows) goes through the clamped offsets, its missing rows
    repeating the last one; a tile past the end is not loaded."""
    L = LOOPS[d]
    D = L.D
    _, _, _, kst, vst, final = (BODIES.get(name) or IDLE[name])
    N, tlast = 3 * 64 + 37, 3
    ktile = np.arange(64 * D).reshape(64, D) + 10 ** 6
    vtile = np.arange(64 * D).reshape(64, D) + 2 * 10 ** 6
    lines = follow(body_of(L, name), env_of(L, case))
    lds, loaded = stage_tiles(L, lines, ktile, vtile, tail_offsets(L, N, tlast))
    want = set() if final else {
        "whole": {("K", kst, False), ("V", vst, False)},
        "ktail": {("K", kst, True), ("V", vst, False)},
        "kskip": {("V", vst, False)},
        "vtail": {("V", vst, True)}}[case]
    assert loaded == want
    for which, stage, clamped in loaded:
        tile, base = (ktile, L.M0K) if which == "K" else (vtile, L.M0V)
        for r in range(64):
            src = min(r, 36) if clamped else r
            for q in range(L.LPR):
                at = (base + stage * L.STAGE) // 2 + r * D + 8 * (q ^ L.swz(r))
                assert np.array_equal(lds[at:at + 8], tile[src, 8 * q:8 * q + 8])
    assert (lds >= 0).sum() == len(loaded) * 64 * D


def mask_semantics(L, lines):
    """(score register, constant) pairs of the emitted mask: the compare
    `v_cmp_gt_i32 s[p], OFF, THR[rb]` feeds the next cndmask on s[p]."""
    G = L.G
    pend, out = {}, []
    for l in lines:
        op, args = split(l)
        if op == "v_cmp_gt_i32_e64":
            pend[args[0]] = (int(args[1]), int(args[2][1:]) - G.THR)
        elif op == "v_cndmask_b32_e64":
            assert args[1] == args[0] and args[2] == f"v{G.NINF}"
            off, rb = pend.pop(args[3])
            out.append((int(args[0][1:]), off, rb))
    return out


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("where", ["entry", "MA", "MB"])
def test_masks_hide_exactly_the_invisible_keys(where, d):
    """For every lane, row and tile position, the emitted compares mask a
    score iff its key is past the row's last visible key (key > row when
    causal, key >= N always), with the kernel's threshold formula."""
    L = LOOPS[d]
    if where == "entry":
        lines = L.section("s_cbranch_scc1 FA_EMASK_%=", "FA_EMASK_%=:")
        buf = 0
    else:
        lines = body_of(L, where)
        buf = 1 if where == "MA" else 0
    sem = mask_semantics(L, lines)
    assert len(sem) == 64
    regs_seen = sorted(r for r, _, _ in sem)
    base = L.G.S_BASE[buf]
    assert regs_seen == list(range(base, base + 64))
    for (N, causal, t, wrow0) in ((1000, True, 12, 768), (1000, False, 15, 512), (700, True, 10, 640),
                                  (130, False, 2, 0), (300, True, 4, 256)):
        for lane in range(64):
            h, l32 = lane >> 5, lane & 31
            for reg, off, rb in sem:
                rel = reg - base
                assert rel // 32 == rb
                kb, r = (rel % 32) // 16, rel % 16
                row = wrow0 + 32 * rb + l32
                lim = min(row, N - 1) if causal else N - 1
                thr = lim - 4 * h - 64 * t
                key = 64 * t + 32 * kb + 8 * (r // 4) + 4 * h + r % 4
                assert (off > thr) == (key > lim)


# ------------------------------------------------------ ordering and hazards
def wait_states(line):
    op, args = split(line)
    if op == "s_nop":
        return int(args[0]) + 1
    if line.endswith(":"):
        return 0
    return 1


def classify(op):
    if op.startswith("v_mfma"):
        return "mfma"
    if op.startswith("v_exp"):
        return "trans"
    if op.startswith("v_dot"):
        return "dot"
    if op.startswith("ds_"):
        return "lds"
    if op.startswith("v_"):
        return "valu"
    return "other"


def straight_paths(L):
    """Instruction sequences as executed: the entry (with and without the
    first tile's mask), each loop body for each load case it can meet, on
    its fast path and with its slow path spliced in at its branch."""
    LINES = L.LINES
    paths = []
    entry = LINES[:LINES.index("FA_LA_%=:")]
    i, j = entry.index("s_cbranch_scc1 FA_EMASK_%="), entry.index("FA_EMASK_%=:")
    paths += [entry, entry[:i] + entry[j:]]
    for name in BODIES:
        for case in BODY_CASES[name]:
            body = follow(body_of(L, name), env_of(L, case))
            paths.append(body)
            slow = L.section(f"FA_SLOW{name}_%=:", "s_branch")
            i = body.index(f"s_cbranch_vccnz FA_SLOW{name}_%=")
            j = body.index(f"FA_PB{name}_%=:")
            paths.append(body[:i] + slow + body[j:])
    return paths


PATHS = {d: straight_paths(L) for d, L in LOOPS.items()}
NPATHS = len(PATHS[128])
assert all(len(p) == NPATHS for p in PATHS.values())


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("path", range(NPATHS))
def test_lds_operands_landed_and_rings_not_overwritten_in_flight(path, d):
    body = PATHS[d][path]
    pending = []          # outstanding LDS reads: list of register sets
    last_use = {}         # agpr -> index of the last product reading it
    n_mfma = 0
    for l in body:
        op, args = split(l)
        if op == "s_waitcnt" and "lgkmcnt" in l:
            k = int(re.search(r"lgkmcnt\((\d+)\)", l).group(1))
            while len(pending) > k:
                pending.pop(0)
        elif op.startswith("ds_read"):
            dst = set(regs(args[0]))
            for r in dst:
                # the product that last read this slot must not be the most
                # recent one: another product (32 cycles of matrix pipe) must
                # have issued since, so its operand read is long over
                if r in last_use:
                    assert n_mfma - last_use[r] >= 1, (l, r)
            pending.append(dst)
            assert len(pending) <= 15, "more LDS reads in flight than lgkmcnt counts"
        elif op == "ds_bpermute_b32":
            pending.append(set(regs(args[0])))
        elif op.startswith("v_mfma"):
            srcs = set(regs(args[1])) | set(regs(args[2]))
            for p in pending:
                assert not (p & srcs), ("operand not landed", l)
            n_mfma += 1
            for r in srcs:
                last_use[r] = n_mfma
        elif op.startswith("v_") and not op.startswith("v_mfma"):
            used = set()
            for x in args[1:]:
                used |= set(regs(x))
            for p in pending:
                assert not (p & used), ("LDS result read before it landed", l)


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("path", range(NPATHS))
def test_matrix_vector_hazards(path, d):
    """Wait states (instructions issued; s_nop n counts n + 1) between a
    product writing a register and a vector/LDS instruction reading it >= 12
    (gfx950, 8-pass 32x32x16 product), between a vector write and a product
    reading it >= 2, between an exponential and its reader >= 1, between a
    dot product and any reader of its result (its own accumulation included)
    >= 3, between a vector write and a dot product reading it >= 2."""
    body = PATHS[d][path]
    t = 0
    last = {}   # reg -> (kind, time)
    for l in body:
        op, args = split(l)
        kind = classify(op)
        if kind in ("mfma", "valu", "trans", "lds", "dot"):
            if kind == "mfma":
                reads = set(regs(args[1])) | set(regs(args[2])) | set(regs(args[3]))
                writes = set(regs(args[0]))
            elif op.startswith("ds_read"):
                reads, writes = set(regs(args[1])), set(regs(args[0]))
            elif op == "v_cmp_lt_f32":
                reads, writes = set(regs(args[2])), set()
            elif op == "v_cmp_gt_i32_e64":
                reads, writes = set(regs(args[2])), {args[0]}
            elif op == "v_cndmask_b32_e64":
                reads, writes = set(regs(args[1])) | set(regs(args[2])) | {args[3]}, set(regs(args[0]))
            else:
                reads = set()
                for x in args[1:]:
                    reads |= set(regs(x))
                writes = set(regs(args[0]))
            for r in reads:
                if r not in last:
                    continue
                pk, pt = last[r]
                dist = t - pt
                if pk == "mfma" and kind != "mfma":
                    assert dist >= 12, (l, r, dist)
                if pk == "mfma" and kind == "mfma" and r in set(regs(args[1])) | set(regs(args[2])):
                    assert dist >= 12, (l, r, dist)
                if pk in ("valu", "trans") and kind == "mfma":
                    assert dist >= 2, (l, r, dist)
                if pk == "trans" and kind in ("valu", "trans", "dot"):
                    assert dist >= 1, (l, r, dist)
                if pk == "dot" and kind != "mfma":
                    assert dist >= 3, (l, r, dist)
                if r.startswith("s[") and pk == "valu":
                    assert dist >= 2, (l, r, dist)   # compare -> mask read
                if pk in ("valu", "trans") and kind == "dot":
                    assert dist >= 2, (l, r, dist)
            for r in writes:
                last[r] = (kind, t)
        t += wait_states(l)


@pytest.mark.parametrize("d", DIMS)
def test_every_barrier_waits_for_the_direct_loads(d):
    """A barrier that follows direct loads is preceded by vmcnt(0); the one
    after the first tile's scores (no loads since the prologue's) waits for
    the wave's LDS reads instead, so no wave reloads K stage 0 while another
    still reads it."""
    LINES = LOOPS[d].LINES
    loads_since = False
    for i, l in enumerate(LINES):
        if l.startswith("global_load_lds"):
            loads_since = True
        if l == "s_barrier":
            if loads_since or LINES[i - 1] != "s_waitcnt lgkmcnt(0)":
                assert LINES[i - 1] == "s_waitcnt vmcnt(0)", i
            loads_since = False
    first = LINES.index("s_barrier")
    assert LINES[first - 1] == "s_waitcnt lgkmcnt(0)"
    assert not any(x.startswith("global_load_lds") for x in LINES[:first])


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("path", range(NPATHS + 8))
def test_m0_set_at_least_one_state_before_each_direct_load(path, d):
    idle = [follow(body_of(LOOPS[d], n), env_of(LOOPS[d], c)) for n in IDLE for c in ALL_CASES]
    body = (PATHS[d] + idle)[path]
    last_m0 = None
    for i, l in enumerate(body):
        if l.startswith("s_add_u32 m0,"):
            last_m0 = i
        elif l.startswith("global_load_lds"):
            assert last_m0 is not None and i - last_m0 >= 2, (path, i, l)


@pytest.mark.parametrize("d", DIMS)
def test_straight_body_keeps_its_branch_condition(d):
    """The straight body compares the next tile index with the straight
    limit early and branches on SCC after its barrier: nothing in between
    (its slow path included) may write SCC."""
    L = LOOPS[d]
    for P in "AB":
        body = L.section(f"FA_BODY{P}_%=:", "s_cbranch_scc1 FA_BODY")
        k = body.index(f"s_cmp_lt_u32 s{L.G.S_J}, s{L.G.S_FAST}")
        slow = L.section(f"FA_SLOW{P}_%=:", "s_branch")
        for l in body[k + 1:] + slow:
            op = l.split()[0]
            assert not op.startswith("s_") or op in (
                "s_nop", "s_waitcnt", "s_barrier", "s_cbranch_vccnz"), l


# ------------------------------------------------------------ tile counts
def wave_last_tile(N, q0, w, tend, causal):
    """The last tile holding a key wave w sees (the kernel's formula)."""
    return min(tend - 1, min(q0 + 64 * w + 63, N - 1) // 64) if causal else tend - 1


def run_control(L, N, q0, causal, w=0):
    """Execute the scalar part of the whole statement with the kernel's
    start values for wave w (no slow path): which K and V tiles get loaded
    (and whether through the clamped offsets), which tiles get masked, which
    body each step takes, how many barriers the wave meets."""
    G, LINES = L.G, L.LINES
    BC, BR = 64, L.BR
    nt = -(-N // BC)
    qmax = min(q0 + BR, N) - 1
    tend = min(nt, qmax // BC + 1) if causal else nt
    ragged = N % BC != 0
    fm = tend
    if causal:
        fm = min(fm, q0 // BC)
    if ragged:
        fm = min(fm, nt - 1)
    tail = ragged and tend == nt
    kfull = nt - 1 if tail else tend
    TB = 64 * 2 * L.D
    KB, VB = 1 << 40, 2 << 40
    s = {G.S_LAST: tend - 1, G.S_KEND: max(0, tend - 2),
         G.S_KTAILJ: nt - 3 if tail and nt >= 3 else NONE,
         G.S_VTAILJ: nt - 2 if tail and nt >= 2 else NONE,
         G.S_FM: fm, G.S_FAST: max(0, min(fm - 1, kfull - 2)), G.S_J: 0,
         G.S_WDIAG: wave_last_tile(N, q0, w, tend, causal)}
    ptr = {G.S_KPTR: KB + 2 * TB, G.S_VPTR: VB + TB}
    kload = [(0, False)] + ([(1, False)] if tend > 1 else [])   # the C++ prologue's
    vload = [(0, False)]
    masked, bodies, barriers = [], [], 0
    labels = {l[:-1]: i for i, l in enumerate(LINES) if l.endswith(":")}
    pc, scc, steps = 0, None, 0
    while True:
        steps += 1
        assert steps < 10 ** 6
        l = LINES[pc]
        pc += 1
        if l == "FA_DONE_%=:":
            break
        for kind in ("FA_BODY", "FA_GB", "FA_ITM", "FA_FIN", "FA_IDLEA", "FA_IDLEB"):
            if l.startswith(kind) and l.endswith(":"):
                bodies.append(kind[3:7] if kind.startswith("FA_IDLE") else kind[3:])
                if kind == "FA_ITM":
                    masked.append(s[G.S_J] + 1)
        if l == "s_barrier":
            barriers += 1
        if l == "s_cbranch_scc1 FA_EMASK_%=" and s[G.S_FM] == 0:
            masked.append(0)
        op, args = split(l)
        if op.startswith("s_cmp_"):
            x, y = (s[int(t[1:])] if t.startswith("s") else int(t, 0) for t in args[:2])
            scc = {"s_cmp_eq_u32": x == y, "s_cmp_lg_u32": x != y, "s_cmp_ge_u32": x >= y,
                   "s_cmp_lt_u32": x < y, "s_cmp_gt_u32": x > y}[op]
        elif op in ("s_cbranch_scc0", "s_cbranch_scc1"):
            if scc == (op == "s_cbranch_scc1"):
                pc = labels[args[0]]
        elif op == "s_branch":
            pc = labels[args[0]]
        elif op == "s_add_u32" and args[0] in (f"s{G.S_KPTR}", f"s{G.S_VPTR}"):
            ptr[int(args[0][1:])] += int(args[2])
        elif op == "s_add_u32" and args[0] != "m0":
            s[int(args[0][1:])] = s[int(args[1][1:])] + int(args[2])
        elif op == "global_load_lds_dwordx4":
            reg = int(args[0][1:])
            if reg in (G.GOFF, G.GOFF_TAIL):
                p = ptr[int(args[1][2:].split(":")[0])]
                is_k = p < VB
                t = (p - (KB if is_k else VB)) // TB
                assert 0 <= t < nt, (N, q0, t)
                (kload if is_k else vload).append((t, reg == G.GOFF_TAIL))
    return tend, fm, kload, vload, masked, bodies, barriers


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 200, 256, 300, 511, 512,
                               700, 1000, 1024, 8192])
def test_loop_loads_and_masks(N, causal, d):
    """For every wave: every tile in [0, tend) is loaded once, in order, whole
    tiles through the plain offsets and only a partial last tile through the
    clamped ones; exactly the tiles that hold an invisible key are masked, up
    to the one after the wave's last visible tile; every step before the
    last takes the straight body when its next tile is unmasked and both its
    loads are whole tiles, and steps past the wave's last visible tile are
    idle (never a straight one); all waves meet the same barriers."""
    for q0 in range(0, N, LOOPS[d].BR):
        nbar = set()
        for w in range(LOOPS[d].NW):
            tend, fm, kload, vload, masked, bodies, barriers = run_control(LOOPS[d], N, q0,
                                                                           causal, w)
            nbar.add(barriers)
            last = wave_last_tile(N, q0, w, tend, causal)
            assert [t for t, _ in kload] == list(range(tend))
            assert [t for t, _ in vload] == list(range(tend))
            for t, clamped in kload[2:] + vload[1:]:
                assert clamped == (t * 64 + 63 >= N)
            need = [t for t in range(tend)
                    if t * 64 + 63 >= N or (causal and t * 64 + 63 > q0)]
            need = [t for t in need if t == 0 or t - 1 <= last]
            assert masked == need, (N, q0, w, masked, need)
            want = []
            for j in range(tend - 1):
                whole = j + 2 < tend and (j + 2) * 64 + 63 < N and (j + 1) * 64 + 63 < N
                if j > last:
                    want.append("IDLE")
                else:
                    want.append("ITM" if j + 1 in need else "BODY" if whole else "GB")
            want.append("IDLE" if tend - 1 > last else "FIN")
            assert bodies == want, (N, q0, w, bodies, want)
        assert len(nbar) == 1, (N, q0, nbar)
