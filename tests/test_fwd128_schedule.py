"""Host-side model of the generated main loop of the d = 128 forward kernel
(exact_io_aware_45_amd/csrc/gen_fwd128.py -> fa_fwd128_loop.inc), CPU only.

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
  * the loop's load counters never load a tile outside the sequence.
"""
import importlib.util
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", "gen_fwd128.py")


def load_gen():
    spec = importlib.util.spec_from_file_location("gen_fwd128", GEN)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


G = load_gen()
LINES = G.generate()
D = 128


def tile_swz(r):
    return 4 * (r & 3) + ((r >> 2) & 3)


def test_committed_loop_matches_the_generator():
    text = G.render(LINES)
    assert open(G.OUT).read() == text, "fa_fwd128_loop.inc is stale: rerun gen_fwd128.py"


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


def section(start_label, end_marker):
    """Lines from a label up to (excluding) the first line starting with end_marker."""
    i = LINES.index(start_label)
    out = []
    for l in LINES[i + 1:]:
        if l.startswith(end_marker):
            break
        out.append(l)
    return out


# --------------------------------------------------------- lane-level model
def kernel_offsets():
    """Per-lane values the kernel computes before the loop (restated from
    fa_fwd128.hip): K read addresses (stage 0), V^T read addresses (stage 0),
    direct-load offsets, all in bytes relative to the start of LDS / of a tile."""
    kaddr = np.zeros((8, 64), np.int64)
    vaddr = np.zeros((8, 64), np.int64)
    TILE = 64 * D
    for lane in range(64):
        h, l32 = lane >> 5, lane & 31
        sw_row = tile_swz(l32)
        for c in range(8):
            kaddr[c, lane] = 2 * (2 * TILE + l32 * D + 8 * ((2 * c + h) ^ sw_row))
        tr_row = 4 * h + ((lane & 15) >> 2)
        tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
        sw_lo, sw_hi = tile_swz(tr_row), tile_swz(tr_row + 8)
        tq, te = tr_col >> 3, tr_col & 7

        def tr_off(row, sw, b):
            return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te
        for db in range(4):
            vaddr[2 * db, lane] = 2 * tr_off(tr_row, sw_lo, db)
            vaddr[2 * db + 1, lane] = 2 * tr_off(tr_row + 8, sw_hi, db)
    goff = np.zeros((4, 4, 64), np.int64)   # [wave][load][lane]
    for w in range(4):
        for i in range(4):
            for lane in range(64):
                p = (4 * i + w) * 64 + lane
                row = p >> 4
                goff[w, i, lane] = 2 * (row * D + 8 * ((p & 15) ^ tile_swz(row)))
    return kaddr, vaddr, goff


KADDR, VADDR, GOFF = kernel_offsets()
M0K = 32768   # LDS byte address of K stage 0 (+ wave * 1024 in s64)
M0V = 0


def load_path(lines, tail):
    """The instructions executed by the load blocks when the load is (not) the
    partial last tile: the tail branch jumps over the plain loads, the plain
    path jumps over the tail loads."""
    out, skip_to = [], None
    for l in lines:
        if skip_to is not None:
            if l == skip_to:
                skip_to = None
                out.append(l)
            continue
        out.append(l)
        if tail and l.startswith("s_cbranch_scc1 FA_TAIL"):
            skip_to = l.split()[1] + ":"
        elif not tail and l.startswith("s_branch FA_LDONE"):
            skip_to = l.split()[1] + ":"
    return out


def stage_tiles(lines, ktile, vtile, tail=False, offs=None):
    """Execute the direct loads in `lines` for all four waves into a 64 KiB LDS
    image (uint16 elements).  Returns the image and which stages were loaded."""
    lds = np.full(32768, -1, np.int64)
    loaded = set()
    offs = GOFF if offs is None else offs
    lines = load_path(lines, tail)
    for w in range(4):
        m0 = None
        for l in lines:
            op, args = split(l)
            if op == "s_add_u32" and args[0] == "m0":
                base = {"s64": M0K, "s65": M0V}[args[1]] + 1024 * w
                m0 = base + int(args[2])
            elif op == "global_load_lds_dwordx4":
                reg = int(args[0][1:])
                i = reg - (G.GOFF_TAIL if tail else G.GOFF)
                assert 0 <= i < 4, l
                tile = ktile if args[1] == f"s[{G.S_KPTR}:{G.S_KPTR + 1}]" else vtile
                flat = tile.reshape(-1)
                for lane in range(64):
                    src = offs[w, i, lane] // 2
                    dst = (m0 + 16 * lane) // 2
                    lds[dst:dst + 8] = flat[src:src + 8]
                loaded.add(("K" if tile is ktile else "V", (m0 - (M0K if tile is ktile else M0V)
                                                           - 1024 * w) // 16384))
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


def run_operand_model(body, kstage, vstage):
    """Follow every LDS operand read of `body` into its product and check the
    operand each lane receives."""
    # element values encode (row, col) so every mismatch is visible
    ktile = np.arange(64 * D).reshape(64, D) + 10 ** 6
    vtile = np.arange(64 * D).reshape(64, D) + 2 * 10 ** 6
    lds = np.full(32768, -1, np.int64)
    kb0 = 2 * 64 * D
    for stage in range(2):
        lds[kb0 + stage * 8192: kb0 + stage * 8192 + 8192] = -1
    # place the tiles the way the direct loads do (checked separately)
    for r in range(64):
        for q in range(16):
            slot = q ^ tile_swz(r)
            kdst = (M0K + kstage * 16384) // 2 + r * D + 8 * slot
            vdst = (M0V + vstage * 16384) // 2 + r * D + 8 * slot
            lds[kdst:kdst + 8] = ktile[r, 8 * q:8 * q + 8]
            lds[vdst:vdst + 8] = vtile[r, 8 * q:8 * q + 8]
    ring = {}   # agpr -> per-lane values (one column per register half)
    checked = {"k": 0, "v": 0}
    for l in body:
        op, args = split(l)
        if op == "ds_read_b128":
            dst = regs(args[0])
            c = int(args[1][1:]) - G.KADDR
            off = int(args[2].split(":")[1]) if len(args) > 2 else 0
            assert (off // 16384) == kstage
            vals = np.zeros((64, 8), np.int64)
            for lane in range(64):
                a0 = (KADDR[c, lane] + off) // 2
                vals[lane] = lds[a0:a0 + 8]
            ring[dst[0]] = ("K", vals)
        elif op == "ds_read_b64_tr_b16":
            dst = regs(args[0])
            idx = int(args[1][1:]) - G.VADDR
            off = int(args[2].split(":")[1]) if len(args) > 2 else 0
            assert (off // 16384) == vstage
            vals = tr_read(lds, VADDR[idx] + off)
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
                rb, db = o // 64, (o % 64) // 16
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
                rb, c = q // 32, (q % 32) // 4
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
    "A": ("FA_LA_%=:", 1, 0, 0, 1, False), "MA": ("FA_ITMA_%=:", 1, 0, 0, 1, False),
    "B": ("FA_LB_%=:", 0, 1, 1, 0, False), "MB": ("FA_ITMB_%=:", 0, 1, 1, 0, False),
    "FA": ("FA_FINA_%=:", 1, 0, 0, 1, True), "FB": ("FA_FINB_%=:", 0, 1, 1, 0, True),
}


def body_of(name):
    return section(BODIES[name][0], "s_barrier")


@pytest.mark.parametrize("name", list(BODIES))
def test_operands_of_every_product(name):
    _, kst, vst, _, _, final = BODIES[name]
    checked = run_operand_model(body_of(name), kst, vst)
    assert checked == ({"k": 0, "v": 32} if final else {"k": 32, "v": 32})


def test_operands_of_the_first_tile_scores():
    """The entry computes tile 0's scores from K stage 0."""
    body = LINES[:LINES.index("s_cbranch_scc1 FA_EMASK_%=")]
    checked = run_operand_model(body, 0, 0)
    assert checked == {"k": 32, "v": 0}


def tail_offsets(N, tlast):
    """Clamped direct-load offsets of the partial last tile (the kernel's
    formula): rows past N - 1 repeat row N - 1."""
    out = np.zeros((4, 4, 64), np.int64)
    for w in range(4):
        for i in range(4):
            for lane in range(64):
                p = (4 * i + w) * 64 + lane
                row = p >> 4
                col = 8 * ((p & 15) ^ tile_swz(row))
                out[w, i, lane] = 2 * ((min(tlast * 64 + row, N - 1) - tlast * 64) * D + col)
    return out


@pytest.mark.parametrize("name", list(BODIES))
@pytest.mark.parametrize("tail", [False, True])
def test_direct_loads_place_tiles_as_the_reads_expect(name, tail):
    """The emitted loads (M0 values, offset registers) write chunk q of tile
    row r to slot q ^ swz(r) of the right stage, for all four waves, and
    cover each stage exactly once; a partial last tile (here 37 rows) goes
    through the clamped offsets, its missing rows repeating the last one."""
    _, _, _, kst, vst, _ = BODIES[name]
    N, tlast = 3 * 64 + 37, 3
    ktile = np.arange(64 * D).reshape(64, D) + 10 ** 6
    vtile = np.arange(64 * D).reshape(64, D) + 2 * 10 ** 6
    offs = tail_offsets(N, tlast) if tail else None
    lds, loaded = stage_tiles(body_of(name), ktile, vtile, tail, offs)
    assert loaded == {("K", kst), ("V", vst)}
    for r in range(64):
        src = min(r, 36) if tail else r
        for q in range(16):
            slot = q ^ tile_swz(r)
            k = (M0K + kst * 16384) // 2 + r * D + 8 * slot
            v = (M0V + vst * 16384) // 2 + r * D + 8 * slot
            assert np.array_equal(lds[k:k + 8], ktile[src, 8 * q:8 * q + 8])
            assert np.array_equal(lds[v:v + 8], vtile[src, 8 * q:8 * q + 8])
    assert (lds >= 0).sum() == 2 * 64 * D


def mask_semantics(lines):
    """(score register, constant) pairs of the emitted mask: the compare
    `v_cmp_gt_i32 s[p], OFF, THR[rb]` feeds the next cndmask on s[p]."""
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


@pytest.mark.parametrize("where", ["entry", "MA", "MB"])
def test_masks_hide_exactly_the_invisible_keys(where):
    """For every lane, row and tile position, the emitted compares mask a
    score iff its key is past the row's last visible key (key > row when
    causal, key >= N always), with the kernel's threshold formula."""
    if where == "entry":
        lines = section("s_cbranch_scc1 FA_EMASK_%=", "FA_EMASK_%=:")
        buf = 0
    else:
        lines = body_of(where)
        buf = 1 if where == "MA" else 0
    sem = mask_semantics(lines)
    assert len(sem) == 64
    regs_seen = sorted(r for r, _, _ in sem)
    base = G.S_BASE[buf]
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


def straight_paths():
    """Instruction sequences as executed: the entry (with and without the
    first tile's mask), each loop body on its fast path and with its slow
    path spliced in at its branch, each with the normal and the tail loads."""
    paths = []
    entry = LINES[:LINES.index("FA_LA_%=:")]
    i, j = entry.index("s_cbranch_scc1 FA_EMASK_%="), entry.index("FA_EMASK_%=:")
    paths += [entry, entry[:i] + entry[j:]]
    for name in BODIES:
        for tail in (False, True):
            body = load_path(body_of(name), tail)
            paths.append(body)
            slow = section(f"FA_SLOW{name}_%=:", "s_branch")
            i = body.index(f"s_cbranch_vccnz FA_SLOW{name}_%=")
            j = body.index(f"FA_PB{name}_%=:")
            paths.append(body[:i] + slow + body[j:])
    return paths


NPATHS = len(straight_paths())


@pytest.mark.parametrize("path", range(NPATHS))
def test_lds_operands_landed_and_rings_not_overwritten_in_flight(path):
    body = straight_paths()[path]
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


@pytest.mark.parametrize("path", range(NPATHS))
def test_matrix_vector_hazards(path):
    """Wait states (instructions issued; s_nop n counts n + 1) between a
    product writing a register and a vector/LDS instruction reading it >= 12
    (gfx950, 8-pass 32x32x16 product), between a vector write and a product
    reading it >= 2, between an exponential and its reader >= 1, between a
    dot product and any reader of its result (its own accumulation included)
    >= 3, between a vector write and a dot product reading it >= 2."""
    body = straight_paths()[path]
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


def test_every_barrier_waits_for_the_direct_loads():
    """A barrier that follows direct loads is preceded by vmcnt(0); the one
    after the first tile's scores (no loads since the prologue's) waits for
    the wave's LDS reads instead, so no wave reloads K stage 0 while another
    still reads it."""
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


def test_m0_set_one_state_before_each_direct_load():
    for i, l in enumerate(LINES):
        if l.startswith("global_load_lds"):
            assert LINES[i - 1] == "s_nop 0" and LINES[i - 2].startswith("s_add_u32 m0,")


# ------------------------------------------------------------ tile counts
def loop_loads(N, q0, causal):
    """Replay the loop's control flow and load counters with the kernel's
    start values: which K and V tiles get loaded (and whether through the
    clamped offsets), which iterations mask their next tile."""
    BC, BR = 64, 256
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
    kload = [(0, False)] + ([(1, False)] if tend > 1 else [])   # prologue (C++, clamped itself)
    vload = [(0, False)]
    iters, nk, nv, j = tend - 1, max(0, tend - 2), max(0, tend - 1), 0
    kt, vt = 2, 1
    masked = [0] if fm == 0 else []
    while True:
        last = iters == 0
        if nk:
            kload.append((kt, nk == 1 and tail))
            kt += 1
            nk -= 1
        if nv:
            vload.append((vt, nv == 1 and tail))
            vt += 1
            nv -= 1
        if last:
            break
        if j + 1 >= fm:
            masked.append(j + 1)
        j += 1
        iters -= 1
    return tend, fm, kload, vload, masked


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 127, 128, 129, 200, 256, 300, 511, 512, 700, 1000,
                               1024, 8192])
def test_loop_loads_and_masks(N, causal):
    """Every tile in [0, tend) is loaded once, in order, whole tiles through
    the plain offsets and only a partial last tile through the clamped ones;
    exactly the tiles that hold an invisible key are masked."""
    for q0 in range(0, N, 256):
        tend, fm, kload, vload, masked = loop_loads(N, q0, causal)
        assert [t for t, _ in kload] == list(range(tend))
        assert [t for t, _ in vload] == list(range(tend))
        for t, clamped in kload[2:] + vload[1:]:
            assert clamped == (t * 64 + 63 >= N)
        need = [t for t in range(tend)
                if t * 64 + 63 >= N or (causal and t * 64 + 63 > q0)]
        assert masked == need, (N, q0, masked, need)
