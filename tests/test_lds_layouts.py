"""Properties of the kernels' LDS tile layouts (CPU only).

The formulas below restate the kernels' index arithmetic (the XOR swizzles
of 16-byte chunks, the fp8 V-row permutation and the lanes' read addresses)
and check on a model of the LDS (64 banks of 4 bytes) that
  * every read of a staged tile returns the operand bytes the matrix
    instruction's slot mapping needs (for the fp8 transpose reads, with the
    ds_read_b64_tr_b8 lane semantics measured on the device), and
  * each access pattern is free of bank conflicts.
"""
import numpy as np
import pytest


# ---------------------------------------------------------------- bf16 tiles
def tile_swz(D, r):
    return 4 * (r & 3) + ((r >> 2) & 3) if D == 128 else 4 * ((r >> 1) & 1) + ((r >> 2) & 3)


def bank_groups(byte_addrs, width):
    """4-byte bank indices touched by the accesses (each `width` bytes)."""
    return [((a + o) // 4) % 64 for a in byte_addrs for o in range(0, width, 4)]


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_row_reads_conflict_free(D):
    # 16 consecutive rows read the same 16-byte chunk (ds_read_b128 operand rows)
    for r0 in range(0, 64, 16):
        for q in range(D // 8):
            addrs = [2 * ((r0 + i) * D + 8 * (q ^ tile_swz(D, r0 + i))) for i in range(16)]
            assert len(set(bank_groups(addrs, 16))) == 64


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_transpose_reads_conflict_free(D):
    # 4 consecutive rows (first a multiple of 4) x 4 consecutive chunks (first a
    # multiple of 4): half a wave of ds_read_b64_tr_b16, 8 bytes per lane
    for r0 in range(0, 64, 4):
        for q0 in range(0, D // 8, 4):
            addrs = []
            for t in range(4):
                for qq in range(4):
                    base = 2 * ((r0 + t) * D + 8 * ((q0 + qq) ^ tile_swz(D, r0 + t)))
                    addrs += [base, base + 8]
            assert len(set(bank_groups(addrs, 8))) == 64


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_swizzle_is_a_permutation_per_row(D):
    for r in range(64):
        assert sorted(q ^ tile_swz(D, r) for q in range(D // 8)) == list(range(D // 8))


# ------------------------------------------------------------------ fp8 tiles
def k_swz(D, r):
    return ((r >> 1) & 7) if D == 128 else ((r >> 2) & 3)


def v_swz(D, r):
    return 2 * ((r >> 1) & 3) if D == 128 else 2 * ((r >> 2) & 1)


def v_key_of_row(R):
    """Key (within a 64-key tile) stored at LDS row R of the fp8 V tile."""
    return 32 * ((R & 31) >> 4) + 8 * ((R & 15) >> 2) + 4 * (R >> 5) + (R & 3)


def stage_fp8(D, Kt, Vt):
    CH = D // 16
    KL = np.zeros(64 * D, np.uint8)
    VL = np.zeros(64 * D, np.uint8)
    for p in range(64 * CH):
        row, slot = p // CH, p % CH
        KL[16 * p:16 * p + 16] = Kt[row, 16 * (slot ^ k_swz(D, row)):][:16]
        VL[16 * p:16 * p + 16] = Vt[v_key_of_row(row), 16 * (slot ^ v_swz(D, row)):][:16]
    return KL, VL


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_v_row_permutation_is_a_bijection(D):
    assert sorted(v_key_of_row(R) for R in range(64)) == list(range(64))


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_k_operand_reads(D):
    rng = np.random.default_rng(1)
    Kt = rng.integers(0, 256, (64, D), dtype=np.uint8)
    KL, _ = stage_fp8(D, Kt, Kt)
    for kb in range(2):
        for c in range(D // 64):
            per_quarter = {}
            for lane in range(64):
                h, l32 = lane >> 5, lane & 31
                row = 32 * kb + l32
                a0 = row * D + 16 * ((4 * c + 2 * h) ^ k_swz(D, l32))
                a1 = row * D + 16 * ((4 * c + 2 * h + 1) ^ k_swz(D, l32))
                got = np.concatenate([KL[a0:a0 + 16], KL[a1:a1 + 16]])
                # byte t of half h is d = 64c + 32h + t
                assert np.array_equal(got, Kt[row, 64 * c + 32 * h:64 * c + 32 * h + 32])
                per_quarter.setdefault(lane // 16, ([], []))
                per_quarter[lane // 16][0].append(a0)
                per_quarter[lane // 16][1].append(a1)
            for first, second in per_quarter.values():
                assert len(set(bank_groups(first, 16))) == 64
                assert len(set(bank_groups(second, 16))) == 64


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_v_transpose_reads(D):
    """ds_read_b64_tr_b8: in each 16-lane group, lane 2e + s addresses row
    r0 + e, bytes c0 + 8s .. + 7; lane i receives byte (i % 8) of the chunk
    addressed by lane 2e + i / 8, for e = 0..7."""
    rng = np.random.default_rng(2)
    Vt = rng.integers(0, 256, (64, D), dtype=np.uint8)
    _, VL = stage_fp8(D, Vt, Vt)

    def addr(lane, b, q):
        h, tr_row, tr_half, tr_s = lane >> 5, (lane & 15) >> 1, (lane >> 4) & 1, lane & 1
        return (32 * h + 8 * q + tr_row) * D + 16 * ((2 * b + tr_half) ^ v_swz(D, tr_row)) + 8 * tr_s

    for b in range(D // 32):
        for q in range(4):
            A = [addr(lane, b, q) for lane in range(64)]
            for half in range(2):
                assert len(set(bank_groups(A[32 * half:32 * half + 32], 8))) == 64
            for lane in range(64):
                g16, j16, h = lane // 16, lane % 16, lane >> 5
                got = [VL[A[16 * g16 + 2 * e + j16 // 8] + j16 % 8] for e in range(8)]
                for e in range(8):
                    t = 8 * q + e  # operand byte of half h
                    key = 32 * (t // 16) + 8 * ((t % 16) // 4) + 4 * h + t % 4
                    assert got[e] == Vt[key, 32 * b + (lane & 31)]
