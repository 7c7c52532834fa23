"""Host-side checks of the generated query loop of the d = 128 dK/dV kernel
(exact_io_aware_45_amd/csrc/gen_bwd_dkdv128.py -> fa_bwd_dkdv128_loop.inc),
CPU only.  On the emitted text:
  * every product's LDS operand has landed by the emitted s_waitcnt, no
    operand ring slot is reread before another product has issued, and no
    more LDS reads are in flight than the 4-bit wait counter can name;
  * the wait states cover the matrix/vector hazards, including a vector
    write of a register a product read as an operand;
  * M0 is set before each direct load, and every barrier follows lgkmcnt(0)
    and vmcnt(0);
  * the direct loads of each body put each 64-query tile's Q and dO rows
    and its L, D values where the operand reads expect them (stage t % 4,
    whole or with rows clamped to the sequence);
  * the scalar control flow of the whole statement, executed for many
    lengths and key blocks, loads every query tile once and in order, masks
    every half-tile that holds an invisible score, and takes the straight
    body where it applies.
The lane-level arithmetic is checked by test_bwd_dkdv128_emulate.py.
"""
import importlib.util
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", "gen_bwd_dkdv128.py")
spec = importlib.util.spec_from_file_location("gen_bwd_dkdv128_sched", GEN)
G = importlib.util.module_from_spec(spec)
spec.loader.exec_module(G)
LINES = G.generate()
D = 128
NONE = 0xFFFFFFFF
REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+))")


def tile_swz(r):
    return 4 * (r & 3) + ((r >> 2) & 3)


def regs(operand):
    m = REG.search(operand)
    if not m or operand.startswith("s"):
        return []
    kind = m.group(1)
    if m.group(4) is not None:
        return [f"{kind}{m.group(4)}"]
    return [f"{kind}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)]


def split(line):
    op, _, rest = line.partition(" ")
    args = [x.strip() for x in rest.split(",")] if rest else []
    if args and " offset:" in args[-1]:
        reg, _, off = args[-1].partition(" offset:")
        args[-1:] = [reg.strip(), "offset:" + off.strip()]
    return op, args


def section(start_label, end_marker):
    i = LINES.index(start_label)
    out = []
    for l in LINES[i + 1:]:
        if l.startswith(end_marker):
            break
        out.append(l)
    return out


def test_committed_loop_matches_the_generator():
    with open(G.OUT) as f:
        assert f.read() == G.render(LINES), "regenerate fa_bwd_dkdv128_loop.inc"


def follow(lines, env):
    """Lines a body executes for the given scalar registers (branches to a
    label outside `lines` end the path)."""
    labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":")}
    out, pc, scc = [], 0, None
    while pc < len(lines):
        l = lines[pc]
        pc += 1
        op, args = split(l)
        if op.startswith("s_cmp_"):
            x, y = (env[int(t[1:])] if t.startswith("s") else int(t, 0) for t in args[:2])
            scc = {"s_cmp_eq_u32": x == y, "s_cmp_lg_u32": x != y, "s_cmp_ge_u32": x >= y,
                   "s_cmp_lt_u32": x < y}[op]
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
        elif op in ("s_add_u32", "s_addc_u32", "s_lshl_b32"):
            scc = None
        out.append(l)
    return out


LOAD_CASES = {   # step j = 5
    "whole": {G.S_KEND: 10, G.S_TAILJ: NONE},
    "tail": {G.S_KEND: 10, G.S_TAILJ: 5},
    "skip": {G.S_KEND: 5, G.S_TAILJ: NONE},
}


def env_of(case):
    return {**LOAD_CASES[case], G.S_J: 5, G.S_FAST: 0}


BODIES = {}
for _p in range(G.NPAR):
    BODIES[f"F{_p}"] = (f"FK_BODY{_p}_%=:", _p, ["whole"])
    BODIES[f"G{_p}"] = (f"FK_GB{_p}_%=:", _p, ["whole", "tail", "skip"])
    BODIES[f"M{_p}"] = (f"FK_ITM{_p}_%=:", _p, ["whole", "tail", "skip"])
    BODIES[f"N{_p}"] = (f"FK_FIN{_p}_%=:", _p, ["whole"])


def body_of(name):
    return section(BODIES[name][0], "s_barrier")


def pre_reads(stage):
    """The reads a tile step finds in flight when it starts: those of the
    first gradient products of its tile (in `stage`), issued by the step
    before it (or the entry)."""
    return [ins.text for _, reads in G.units_of(None, (stage, 0, 0))[:G.PRE] for _, ins in reads]


def straight_paths():
    """(lines, reads in flight at the start, p of the body or None)."""
    paths = []
    entry = LINES[:LINES.index("FK_L0_%=:")]
    i, j = entry.index("s_cbranch_scc1 FK_EMASK_%="), entry.index("FK_EMASK_%=:")
    paths += [(entry, [], None), (entry[:i] + entry[j:], [], None)]
    for name, (_, p, cases) in BODIES.items():
        for case in cases:
            paths.append((follow(body_of(name), env_of(case)), pre_reads(p % 4), name))
    return paths


PATHS = straight_paths()


@pytest.mark.parametrize("path", range(len(PATHS)))
def test_lds_operands_landed_and_rings_not_overwritten_in_flight(path):
    lines, pre, _ = PATHS[path]
    pending, last_use, n_mfma = [set(regs(split(l)[1][0])) for l in pre], {}, 0
    for l in lines:
        op, args = split(l)
        if op == "s_waitcnt" and "lgkmcnt" in l:
            k = int(re.search(r"lgkmcnt\((\d+)\)", l).group(1))
            while len(pending) > k:
                pending.pop(0)
        elif op.startswith("ds_read"):
            dst = set(regs(args[0]))
            for r in dst:
                if r in last_use:
                    assert n_mfma - last_use[r] >= 1, (l, r)
            pending.append(dst)
            assert len(pending) <= 15, ("more LDS reads in flight than lgkmcnt can count", l)
        elif op.startswith("v_mfma"):
            srcs = set(regs(args[1])) | set(regs(args[2])) | set(regs(args[3]))
            for p in pending:
                assert not (p & srcs), ("operand not landed", l)
            n_mfma += 1
            for r in srcs:
                last_use[r] = n_mfma
        elif op.startswith("v_"):
            used = set()
            for x in args[1:]:
                used |= set(regs(x))
            for p in pending:
                assert not (p & used), ("LDS result read before it landed", l)


def wait_states(line):
    op, args = split(line)
    if op == "s_nop":
        return int(args[0]) + 1
    return 0 if line.endswith(":") else 1


@pytest.mark.parametrize("path", range(len(PATHS)))
def test_matrix_vector_hazards(path):
    """Product result -> vector/LDS read >= 12 wait states, vector write ->
    product read >= 2, exponential -> use >= 1, compare -> mask read >= 2,
    product reading a register as A/B -> vector write of it >= 8."""
    t, last, src_read = 0, {}, {}
    for l in PATHS[path][0]:
        op, args = split(l)
        kind = ("mfma" if op.startswith("v_mfma") else "trans" if op.startswith("v_exp") else
                "lds" if op.startswith("ds_") else "valu" if op.startswith("v_") else "other")
        if kind != "other":
            if kind == "mfma":
                reads = set(regs(args[1])) | set(regs(args[2])) | set(regs(args[3]))
                writes = set(regs(args[0]))
            elif op.startswith("ds_read"):
                reads, writes = set(regs(args[1])), set(regs(args[0]))
            elif op == "v_cmp_ge_u32_e64":
                reads, writes = set(regs(args[1])) | set(regs(args[2])), {args[0]}
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
                if pk == "trans" and kind in ("valu", "trans"):
                    assert dist >= 1, (l, r, dist)
                if r.startswith("s[") and pk == "valu":
                    assert dist >= 2, (l, r, dist)
            if kind in ("valu", "trans"):
                for r in writes:
                    if r in src_read:
                        assert t - src_read[r] >= 8, ("operand overwritten", l, r)
            if kind == "mfma":
                for r in set(regs(args[1])) | set(regs(args[2])):
                    src_read[r] = t
            for r in writes:
                last[r] = (kind, t)
        t += wait_states(l)


def test_every_barrier_follows_the_lds_reads_and_the_direct_loads():
    """Before each barrier every direct load has landed, and every LDS read
    but the last 2 PRE (the next step's first operands, of a tile already
    published) has returned: the L/D values the next step's vector work
    reads among them."""
    entry = LINES[:LINES.index("FK_L0_%=:")]
    assert not any(x.startswith("global_load_lds") or x == "s_barrier" for x in entry)
    npre = len(pre_reads(0))
    assert entry[-1] == f"s_waitcnt lgkmcnt({npre})"
    for i, l in enumerate(LINES):
        if l == "s_barrier":
            k = i - 1
            while (LINES[k].endswith(":") or LINES[k].startswith("s_waitcnt vmcnt")
                   or LINES[k].split()[0] in ("s_branch", "s_cbranch_scc1", "s_cmp_ge_u32")):
                k -= 1
            assert LINES[k] in (f"s_waitcnt lgkmcnt({npre})", "s_waitcnt lgkmcnt(0)"), i
            assert LINES[i - 1].startswith("s_waitcnt vmcnt") or LINES[i - 1].startswith("FK_VMD"), i


@pytest.mark.parametrize("path", range(len(PATHS)))
def test_each_step_issues_the_reads_the_next_one_expects(path):
    """A tile step that is not the last (and the entry) ends with the reads
    of the next step's first gradient products, from the next tile's stage,
    as its last LDS reads, and waits for all reads before them; the final
    step leaves none in flight."""
    lines, _, name = PATHS[path]
    reads = [l for l in lines if l.startswith("ds_read")]
    npre = len(pre_reads(0))
    if name is not None and name.startswith("N"):
        assert lines[-2:] == ["s_waitcnt lgkmcnt(0)", "s_waitcnt vmcnt(0)"]
        return
    stage = 0 if name is None else (BODIES[name][1] + 1) % 4
    assert reads[-npre:] == pre_reads(stage)
    tail = lines[len(lines) - lines[::-1].index(reads[-npre]) - 1:]
    assert f"s_waitcnt lgkmcnt({npre})" in tail


@pytest.mark.parametrize("path", range(len(PATHS)))
def test_m0_set_at_least_one_state_before_each_direct_load(path):
    last_m0 = None
    for i, l in enumerate(PATHS[path][0]):
        if l.startswith("s_add_u32 m0,"):
            last_m0 = i
        elif l.startswith("global_load_lds"):
            assert last_m0 is not None and i - last_m0 >= 2, (path, i, l)


def kernel_goff():
    goff = np.zeros((4, 4, 64), np.int64)
    for w in range(4):
        for i in range(4):
            for lane in range(64):
                row = 16 * w + 4 * i + (lane >> 4)
                goff[w, i, lane] = 2 * (row * D + 8 * ((lane & 15) ^ tile_swz(row))) - 1024 * i
    return goff


def tail_goff(N, tlast):
    out = np.zeros((4, 4, 64), np.int64)
    for w in range(4):
        for i in range(4):
            for lane in range(64):
                row = 16 * w + 4 * i + (lane >> 4)
                col = 8 * ((lane & 15) ^ tile_swz(row))
                out[w, i, lane] = 2 * ((min(tlast * 64 + row, N - 1) - tlast * 64) * D + col)
    return out


@pytest.mark.parametrize("name,case", [(n, c) for n, (_, _, cs) in BODIES.items() for c in cs])
def test_direct_loads_place_tiles_as_the_reads_expect(name, case):
    """Tile j + 3 lands in Q, dO and L/D stage (j + 3) % 4: chunk q of row r
    at slot q ^ swz(r) for all four waves, and the tile's 64 L and D values
    in each wave's own area; a partial last tile (37 rows here) through the
    clamped offsets; nothing past the end, nothing in the final step."""
    _, p, _ = BODIES[name]
    lines = follow(body_of(name), env_of(case))
    N, tlast = 3 * 64 + 37, 3
    qtile = np.arange(64 * D).reshape(64, D) + 10 ** 6
    otile = np.arange(64 * D).reshape(64, D) + 2 * 10 ** 6
    lvec = np.arange(64) + 3 * 10 ** 6
    dvec = np.arange(64) + 4 * 10 ** 6
    goff, gtail = kernel_goff(), tail_goff(N, tlast)
    ltail = [min(tlast * 64 + lane, N - 1) - tlast * 64 for lane in range(64)]
    lds2 = np.full(G.L_STAGE0 // 2, -1, np.int64)        # tiles, per bf16 element
    lds4 = np.full(8192 // 4, -1, np.int64)             # L/D area, per fp32 element
    loaded = set()
    m0base = {f"s{G.S_M0Q}": lambda w: 4096 * w, f"s{G.S_M0O}": lambda w: G.O_STAGE0 + 4096 * w,
              f"s{G.S_M0L}": lambda w: G.L_STAGE0 + 512 * w}
    for w in range(4):
        m0 = None
        for l in lines:
            op, args = split(l)
            if op == "s_add_u32" and args[0] == "m0":
                m0 = m0base[args[1]](w) + int(args[2])
            elif op == "global_load_lds_dwordx4":
                reg = int(args[0][1:])
                clamped = reg >= G.GOFF_TAIL
                i = reg - (G.GOFF_TAIL if clamped else G.GOFF)
                off = int(args[2].split(":")[1]) if len(args) > 2 else 0
                is_q = args[1] == f"s[{G.S_QPTR}:{G.S_QPTR + 1}]"
                flat = (qtile if is_q else otile).reshape(-1)
                offs = gtail if clamped else goff
                for lane in range(64):
                    src = (offs[w, i, lane] + off) // 2
                    dst = (m0 + off + 16 * lane) // 2
                    lds2[dst:dst + 8] = flat[src:src + 8]
                base = 0 if is_q else G.O_STAGE0
                loaded.add(("Q" if is_q else "O", (m0 - base - 4096 * w) // 16384, clamped))
            elif op == "global_load_lds_dword":
                reg = int(args[0][1:])
                clamped = reg == G.LOFF_TAIL
                off = int(args[2].split(":")[1]) if len(args) > 2 else 0
                is_l = args[1] == f"s[{G.S_LPTR}:{G.S_LPTR + 1}]"
                # the D pointer is set 256 bytes before its tile (the offset adds them back)
                vec = lvec if is_l else dvec
                for lane in range(64):
                    src = (ltail[lane] if clamped else lane) * 4 + off - (0 if is_l else 256)
                    dst = m0 + off + 4 * lane - G.L_STAGE0
                    assert src % 4 == 0 and dst % 4 == 0
                    lds4[dst // 4] = vec[src // 4]
                loaded.add(("L" if is_l else "D", (m0 - G.L_STAGE0 - 512 * w) // G.LD_STAGE, clamped))
    final = name.startswith("N")
    st = (p + 3) % 4
    want = set() if final or case == "skip" else {(x, st, case == "tail") for x in "QOLD"}
    assert loaded == want
    for which, stage, clamped in loaded:
        if which in "QO":
            tile, base = (qtile, 0) if which == "Q" else (otile, G.O_STAGE0)
            for r in range(64):
                src = min(r, 36) if clamped else r
                for q in range(16):
                    at = (base + stage * 16384) // 2 + r * D + 8 * (q ^ tile_swz(r))
                    assert np.array_equal(lds2[at:at + 8], tile[src, 8 * q:8 * q + 8])
        else:
            vec, extra = (lvec, 0) if which == "L" else (dvec, 256)
            for w in range(4):
                for lane in range(64):
                    src = min(lane, 36) if clamped else lane
                    at = (G.LD_STAGE * stage + 512 * w + extra) // 4 + lane
                    assert lds4[at] == vec[src]
    assert (lds2 >= 0).sum() == sum(x in "QO" for x, _, _ in loaded) * 64 * D
    assert (lds4 >= 0).sum() == sum(x in "LD" for x, _, _ in loaded) * 4 * 64


def pend_loads(pend):
    return [(t, None, None) for t in pend]


def run_control(N, k0, causal):
    """Execute the scalar part of the statement with the kernel's start
    values: query tiles loaded (relative index, stages, clamped), halves
    masked, bodies taken."""
    BQ = 64
    nt = -(-N // BQ)
    ts = k0 // BQ if causal else 0
    cnt = nt - ts
    ragged = N % BQ != 0
    mlo = 2 if causal else 0
    mhi = cnt - 1 if ragged else cnt
    TB, VB = 64 * 256, 64 * 4
    QB, OB, LB, DB = 1 << 40, 2 << 40, 3 << 40, 4 << 40
    s = {G.S_LAST: cnt - 1, G.S_KEND: max(0, cnt - 3),
         G.S_TAILJ: cnt - 4 if ragged and cnt >= 4 else NONE, G.S_MLO: mlo, G.S_MHI: mhi,
         G.S_FAST: max(0, mhi - 3), G.S_J: 0, G.S_MASK0: 1 if (mlo > 0 or mhi == 0) else 0}
    ptr = {G.S_QPTR: QB + (ts + 3) * TB, G.S_OPTR: OB + (ts + 3) * TB,
           G.S_LPTR: LB + (ts + 3) * VB, G.S_DPTR: DB + (ts + 3) * VB - 256}
    bases = {G.S_QPTR: (QB, TB, 0), G.S_OPTR: (OB, TB, 0), G.S_LPTR: (LB, VB, 0),
             G.S_DPTR: (DB, VB, 256)}
    stage_of = {f"s{G.S_M0Q}": lambda o: o // 16384, f"s{G.S_M0O}": lambda o: o // 16384,
                f"s{G.S_M0L}": lambda o: o // G.LD_STAGE}
    loads = [(t, (t, t, t, t), t * 64 + 63 >= N - ts * 64) for t in range(min(3, cnt))]
    pend = {}
    vm_out = []          # tile of each direct load in flight, in issue order
    published = set(range(min(3, cnt)))   # the C++ prologue's, behind its barrier
    masked, bodies = [], []
    step = None
    labels = {l[:-1]: i for i, l in enumerate(LINES) if l.endswith(":")}
    pc, scc, m0, steps = 0, None, None, 0
    while True:
        steps += 1
        assert steps < 10 ** 6
        l = LINES[pc]
        pc += 1
        if l == "FK_DONE_%=:":
            break
        for kind in ("FK_BODY", "FK_GB", "FK_ITM", "FK_FIN"):
            if l.startswith(kind) and l.endswith(":"):
                bodies.append(kind[3:])
                j = s[G.S_J]
                # the step reads tiles j and j + 1: both published
                assert {j, j + 1} & set(range(cnt)) <= published, (N, k0, j, published)
                step = j
                if kind == "FK_ITM":
                    masked += [(j, 1), (j + 1, 0)]
                if kind == "FK_FIN":
                    masked.append((j, 1))
        if l == "s_cbranch_scc1 FK_EMASK_%=" and s[G.S_MASK0] != 0:
            masked.append((0, 0))
        op, args = split(l)
        if op.startswith("s_cmp_"):
            x, y = (s[int(t[1:])] if t.startswith("s") else int(t, 0) for t in args[:2])
            scc = {"s_cmp_eq_u32": x == y, "s_cmp_lg_u32": x != y, "s_cmp_ge_u32": x >= y,
                   "s_cmp_lt_u32": x < y}[op]
        elif op in ("s_cbranch_scc0", "s_cbranch_scc1"):
            if scc == (op == "s_cbranch_scc1"):
                pc = labels[args[0]]
        elif op == "s_branch":
            pc = labels[args[0]]
        elif op == "s_add_u32" and args[0] == "m0":
            m0 = (args[1], int(args[2]))
        elif op == "s_add_u32" and int(args[0][1:]) in ptr:
            ptr[int(args[0][1:])] += int(args[2])
        elif op == "s_add_u32":
            s[int(args[0][1:])] = s[int(args[1][1:])] + int(args[2])
        elif op == "s_lshl_b32":
            s[int(args[0][1:])] = s[int(args[1][1:])] << int(args[2])
        elif op == "s_mov_b32":
            s[int(args[0][1:])] = int(args[1], 0)
        elif op == "s_addc_u32":
            pass
        elif op == "s_waitcnt" and args[0].startswith("vmcnt"):
            n = int(args[0][6:-1])
            vm_out = vm_out[len(vm_out) - n:] if n else []
        elif op == "s_barrier":
            loaded = {t for t, _, _ in pend_loads(pend)} | set(range(min(3, cnt)))
            published |= loaded - set(vm_out)
            # the next step reads tile step + 2: it must be published now
            assert step + 2 >= cnt or step + 2 in published, (N, k0, step, vm_out)
        elif op.startswith("global_load_lds"):
            reg = int(args[0][1:])
            key = int(args[1][2:].split(":")[0])
            off = int(args[2].split(":")[1]) if len(args) > 2 else 0
            base, size, extra = bases[key]
            if op == "global_load_lds_dwordx4" and reg not in (G.GOFF, G.GOFF_TAIL):
                continue   # loads 1-3 of a tile follow load 0
            assert (ptr[key] + extra - base) % size == 0
            t = (ptr[key] + extra - base) // size - ts
            assert 0 <= t < cnt, (N, k0, t)
            clamped = reg in (G.GOFF_TAIL, G.LOFF_TAIL)
            vm_out += [t] * (4 if op == "global_load_lds_dwordx4" else 1)
            pend.setdefault(t, []).append((key, stage_of[m0[0]](m0[1] + (off if key == G.S_DPTR else 0)
                                                                    - (256 if key == G.S_DPTR else 0)),
                                           clamped))
    got = []
    for t in sorted(pend):
        parts = sorted(pend[t])
        assert [k for k, _, _ in parts] == sorted([G.S_QPTR, G.S_OPTR, G.S_LPTR, G.S_DPTR]), parts
        assert len({c for _, _, c in parts}) == 1
        got.append((t, tuple(st for _, st, _ in parts), parts[0][2]))
    return cnt, ts, loads + got, sorted(set(masked)), bodies


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 200, 256, 300, 511, 512,
                               700, 1000, 1024, 8192])
def test_loop_loads_and_masks(N, causal):
    for k0 in range(0, N, 128):
        cnt, ts, loads, masked, bodies = run_control(N, k0, causal)
        assert [t for t, _, _ in loads] == list(range(cnt))
        for t, stages, clamped in loads:
            assert stages == (t % 4,) * 4
            assert clamped == ((ts + t) * 64 + 63 >= N)
        need = {(t, h) for t in range(cnt) for h in range(2)
                if (ts + t) * 64 + 32 * h + 31 >= N or (causal and (ts + t) * 64 + 32 * h < k0 + 127)}
        assert need <= set(masked), (N, k0, need - set(masked))
        mlo = 2 if causal else 0
        mhi = cnt - 1 if N % 64 else cnt
        want = []
        for j in range(cnt - 1):
            if mlo <= j < mhi - 3:
                want.append("BODY")
            elif j < mlo or j + 1 >= mhi:
                want.append("ITM")
            else:
                want.append("GB")
        assert bodies == want + ["FIN"], (N, k0, bodies, want)
        # the straight body is taken for every step it can take
        assert bodies.count("BODY") == max(0, mhi - 3 - mlo)


def test_statement_writes_none_of_its_read_only_operands():
    """With grouped heads the kernel runs the statement once per query head
    and keeps its plain inputs (addresses, constants) and the K/V rows
    (in-out operands it must leave unchanged) in place between the runs: no
    instruction of the statement may write them."""
    hip = open(os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", "fa_bwd_dkdv128.hip")).read()
    stmt = hip[hip.index("asm volatile(FA_BWD_DKDV128_LOOP_ASM"):hip.index("FA_BWD_DKDV128_LOOP_CLOBBERS);")]
    kept = set()
    for prefix, spec in re.findall(r'"([+=]?)\{([^}]+)\}"\(', stmt):
        m = re.fullmatch(r"([vas])\[(\d+):(\d+)\]", spec)
        names = ([f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)]
                 if m else [spec])
        kv_rows = prefix == "+" and m is not None and m.group(1) == "a" and int(m.group(2)) >= 128
        if prefix == "" or kv_rows:
            kept.update(names)
    assert {"v160", "a128", "a191", "s64", "s89"} <= kept
    for l in LINES:
        if l.endswith(":"):
            continue
        op, _, rest = l.partition(" ")
        if not rest or op.startswith(("s_cmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop",
                                      "s_barrier", "global_load_lds")):
            continue
        if op.startswith("v_cmp") and not op.endswith("_e64"):
            continue
        dst = rest.split(",")[0].split(" offset:")[0].strip()
        m = re.fullmatch(r"([vas])\[(\d+):(\d+)\]", dst)
        names = [f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)] if m \
            else [dst]
        assert not (set(names) & kept), l
