"""Host-side checks of the generated key loop of the d = 128 dQ kernel
(exact_io_aware_45_amd/csrc/gen_bwd_dq128.py -> fa_bwd_dq128_loop.inc), CPU
only.  On the emitted text:
  * every product's LDS operand has landed by the emitted s_waitcnt, and no
    operand ring slot is reread before another product has issued;
  * the wait states cover the matrix/vector hazards, including a vector
    write of a register a product read as an operand;
  * M0 is set before each direct load, every barrier after direct loads is
    preceded by vmcnt(0);
  * the direct loads of each body put each 64-key tile's rows where the
    operand reads expect them (K stage t % 4, V stage t % 2, whole or with
    rows clamped to the sequence);
  * the scalar control flow of the whole statement, executed for many
    lengths, loads every tile once and in order, masks every half-tile that
    holds an invisible key, and takes the straight body where it applies.
The lane-level arithmetic is checked by test_bwd_dq128_emulate.py.
"""
import importlib.util
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", "gen_bwd_dq128.py")
spec = importlib.util.spec_from_file_location("gen_bwd_dq128_sched", GEN)
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
        assert f.read() == G.render(LINES), "regenerate fa_bwd_dq128_loop.inc"


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
        elif op in ("s_add_u32", "s_addc_u32"):
            scc = None
        out.append(l)
    return out


LOAD_CASES = {   # tile j = 5
    "whole": {G.S_KEND: 10, G.S_TAILJ: NONE},
    "tail": {G.S_KEND: 10, G.S_TAILJ: 5},
    "skip": {G.S_KEND: 5, G.S_TAILJ: NONE},
}


def env_of(case):
    return {**LOAD_CASES[case], G.S_J: 5, G.S_FAST: 0}


BODIES = {}
for _p in range(G.NPAR):
    BODIES[f"F{_p}"] = (f"FQ_BODY{_p}_%=:", _p, ["whole"])
    BODIES[f"G{_p}"] = (f"FQ_GB{_p}_%=:", _p, ["whole", "tail", "skip"])
    BODIES[f"M{_p}"] = (f"FQ_ITM{_p}_%=:", _p, ["whole", "tail", "skip"])
    BODIES[f"N{_p}"] = (f"FQ_FIN{_p}_%=:", _p, ["whole"])


def body_of(name):
    return section(BODIES[name][0], "s_barrier")


def straight_paths():
    paths = []
    entry = LINES[:LINES.index("FQ_L0_%=:")]
    i, j = entry.index("s_cbranch_scc1 FQ_EMASK_%="), entry.index("FQ_EMASK_%=:")
    paths += [entry, entry[:i] + entry[j:]]
    for name, (_, _, cases) in BODIES.items():
        for case in cases:
            paths.append(follow(body_of(name), env_of(case)))
    return paths


PATHS = straight_paths()


@pytest.mark.parametrize("path", range(len(PATHS)))
def test_lds_operands_landed_and_rings_not_overwritten_in_flight(path):
    pending, last_use, n_mfma = [], {}, 0
    for l in PATHS[path]:
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
        elif op.startswith("v_mfma"):
            srcs = set(regs(args[1])) | set(regs(args[2]))
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
    for l in PATHS[path]:
        op, args = split(l)
        kind = ("mfma" if op.startswith("v_mfma") else "trans" if op.startswith("v_exp") else
                "lds" if op.startswith("ds_") else "valu" if op.startswith("v_") else "other")
        if kind != "other":
            if kind == "mfma":
                reads = set(regs(args[1])) | set(regs(args[2])) | set(regs(args[3]))
                writes = set(regs(args[0]))
            elif op.startswith("ds_read"):
                reads, writes = set(regs(args[1])), set(regs(args[0]))
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


def test_every_barrier_waits_for_the_direct_loads():
    loads_since = False
    for i, l in enumerate(LINES):
        if l.startswith("global_load_lds"):
            loads_since = True
        if l == "s_barrier":
            if loads_since:
                assert LINES[i - 1] == "s_waitcnt vmcnt(0)", i
            loads_since = False
    first = LINES.index("s_barrier")
    assert LINES[first - 1] == "s_waitcnt lgkmcnt(0)"
    assert not any(x.startswith("global_load_lds") for x in LINES[:first])


@pytest.mark.parametrize("path", range(len(PATHS)))
def test_m0_set_at_least_one_state_before_each_direct_load(path):
    last_m0 = None
    for i, l in enumerate(PATHS[path]):
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
    """Tile j + 2 lands in K stage (j + 2) % 4 and V stage j % 2, chunk q of
    row r at slot q ^ swz(r), for all four waves; a partial last tile (37
    rows here) through the clamped offsets; nothing past the end, nothing in
    the final step."""
    _, p, _ = BODIES[name]
    lines = follow(body_of(name), env_of(case))
    N, tlast = 3 * 64 + 37, 3
    ktile = np.arange(64 * D).reshape(64, D) + 10 ** 6
    vtile = np.arange(64 * D).reshape(64, D) + 2 * 10 ** 6
    goff, gtail = kernel_goff(), tail_goff(N, tlast)
    lds = np.full(98304 // 2, -1, np.int64)
    loaded = set()
    for w in range(4):
        m0 = None
        for l in lines:
            op, args = split(l)
            if op == "s_add_u32" and args[0] == "m0":
                m0 = {f"s{G.S_M0K}": 4096 * w, f"s{G.S_M0V}": G.V_STAGE0 + 4096 * w}[args[1]] + int(args[2])
            elif op == "global_load_lds_dwordx4":
                reg = int(args[0][1:])
                clamped = reg >= G.GOFF_TAIL
                i = reg - (G.GOFF_TAIL if clamped else G.GOFF)
                off = int(args[2].split(":")[1]) if len(args) > 2 else 0
                is_k = args[1] == f"s[{G.S_KPTR}:{G.S_KPTR + 1}]"
                flat = (ktile if is_k else vtile).reshape(-1)
                offs = gtail if clamped else goff
                for lane in range(64):
                    src = (offs[w, i, lane] + off) // 2
                    dst = (m0 + off + 16 * lane) // 2
                    lds[dst:dst + 8] = flat[src:src + 8]
                base = 0 if is_k else G.V_STAGE0
                loaded.add(("K" if is_k else "V", (m0 - base - 4096 * w) // 16384, clamped))
    final = name.startswith("N")
    want = set() if final or case == "skip" else {("K", (p + 2) % 4, case == "tail"),
                                                  ("V", p % 2, case == "tail")}
    assert loaded == want
    for which, stage, clamped in loaded:
        tile, base = (ktile, 0) if which == "K" else (vtile, G.V_STAGE0)
        for r in range(64):
            src = min(r, 36) if clamped else r
            for q in range(16):
                at = (base + stage * 16384) // 2 + r * D + 8 * (q ^ tile_swz(r))
                assert np.array_equal(lds[at:at + 8], tile[src, 8 * q:8 * q + 8])
    assert (lds >= 0).sum() == len(loaded) * 64 * D


def run_control(N, q0, causal):
    """Execute the scalar part of the statement with the kernel's start
    values: tiles loaded (index, K stage, V stage, clamped), halves masked,
    bodies taken."""
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
    kfull = nt - 1 if tail else tend
    TB = 64 * 256
    KB, VB = 1 << 40, 2 << 40
    s = {G.S_LAST: tend - 1, G.S_KEND: max(0, tend - 2),
         G.S_TAILJ: nt - 3 if tail and nt >= 3 else NONE,
         G.S_FM: fm, G.S_FAST: max(0, min(fm - 1, kfull - 2)), G.S_J: 0}
    ptr = {G.S_KPTR: KB + 2 * TB, G.S_VPTR: VB + 2 * TB}
    loads = [(0, 0, 0, False)] + ([(1, 1, 1, False)] if tend > 1 else [])   # the C++ prologue's
    kload = {}
    masked, bodies = [], []
    labels = {l[:-1]: i for i, l in enumerate(LINES) if l.endswith(":")}
    pc, scc, m0, steps = 0, None, None, 0
    while True:
        steps += 1
        assert steps < 10 ** 6
        l = LINES[pc]
        pc += 1
        if l == "FQ_DONE_%=:":
            break
        for kind in ("FQ_BODY", "FQ_GB", "FQ_ITM", "FQ_FIN"):
            if l.startswith(kind) and l.endswith(":"):
                bodies.append(kind[3:])
                j = s[G.S_J]
                if kind == "FQ_ITM":
                    masked += [(j, 1), (j + 1, 0)]
                if kind == "FQ_FIN":
                    masked.append((j, 1))
        if l == "s_cbranch_scc1 FQ_EMASK_%=" and s[G.S_FM] == 0:
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
        elif op == "s_add_u32" and args[0] in (f"s{G.S_KPTR}", f"s{G.S_VPTR}"):
            ptr[int(args[0][1:])] += int(args[2])
        elif op == "s_add_u32":
            s[int(args[0][1:])] = s[int(args[1][1:])] + int(args[2])
        elif op == "global_load_lds_dwordx4":
            reg = int(args[0][1:])
            if reg in (G.GOFF, G.GOFF_TAIL):
                key = int(args[1][2:].split(":")[0])
                p = ptr[key]
                is_k = key == G.S_KPTR
                t = (p - (KB if is_k else VB)) // TB
                assert 0 <= t < nt, (N, q0, t)
                stage = (m0[1] // 16384) if is_k else (m0[1] // 16384)
                if is_k:
                    kload[t] = (stage, reg == G.GOFF_TAIL)
                else:
                    ks, kc = kload.pop(t)
                    assert kc == (reg == G.GOFF_TAIL)
                    loads.append((t, ks, stage, kc))
    assert not kload
    return tend, fm, loads, sorted(set(masked)), bodies


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 200, 256, 300, 511, 512,
                               700, 1000, 1024, 8192])
def test_loop_loads_and_masks(N, causal):
    for q0 in range(0, N, 256):
        tend, fm, loads, masked, bodies = run_control(N, q0, causal)
        assert [t for t, _, _, _ in loads] == list(range(tend))
        for t, ks, vs, clamped in loads[2:]:
            assert (ks, vs) == (t % 4, t % 2)
            assert clamped == (t * 64 + 63 >= N)
        need = {(t, h) for t in range(tend) for h in range(2)
                if t * 64 + 63 >= N or (causal and t * 64 + 63 > q0)}
        assert need <= set(masked), (N, q0, need - set(masked))
        # a half is masked only by a step whose tile index is at fm - 1 or later
        assert all(t >= fm - 1 for t, _ in masked), (N, q0, masked, fm)
        want = []
        for j in range(tend - 1):
            whole = j + 2 < tend and (j + 2) * 64 + 63 < N
            want.append("ITM" if j + 1 >= fm else "BODY" if whole else "GB")
        assert bodies == want + ["FIN"], (N, q0, bodies, want)
