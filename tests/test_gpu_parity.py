"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle,
element by element, on seeded synthetic inputs.

Small cases span several tiles and a ragged tail and are compared in full.
The five full-size workloads run in the same launch configuration the
benchmark times, and every element of every (batch, head) is compared with
the oracle, which streams the heads in chunks (heads are independent).  Their
outputs are written into buffers pre-filled with NaN, so an element the
kernels never write fails the comparison.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_45_amd import _lib, inputs
from _parity import Stats, check, check_lse, log, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def run_forward(q, k, v, causal, mask=None):
    if mask is None:
        o, lse = _lib.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    else:
        o, lse = _lib.forward_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), mask.to(DEV),
                                          causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def heads_of(t, pairs):
    """fp64 numpy [len(pairs), N, d] of the selected (b, h) pairs."""
    return np.stack([to64(t[b, h]) for b, h in pairs])


def all_pairs(t):
    return [(b, h) for b in range(t.shape[0]) for h in range(t.shape[1])]


def chunks(pairs, n):
    for i in range(0, len(pairs), n):
        yield pairs[i:i + n]


NAN = float("nan")


def nan_fwd_out(q, odtype=None):
    """(o, lse) device buffers pre-filled with NaN."""
    B, H, N, _ = q.shape
    return (torch.full(q.shape, NAN, dtype=odtype or q.dtype, device=DEV),
            torch.full((B, H, N), NAN, dtype=torch.float32, device=DEV))


def nan_bwd_out(q, k):
    """(dq, dk, dv) fp32 device buffers pre-filled with NaN."""
    return (torch.full(q.shape, NAN, dtype=torch.float32, device=DEV),
            torch.full(k.shape, NAN, dtype=torch.float32, device=DEV),
            torch.full(k.shape, NAN, dtype=torch.float32, device=DEV))


def forward_parity_all_heads(q, k, v, causal, mask=None, chunk=8, magnitude_scaled=False):
    """The whole forward output (every head, row and column) against the
    oracle, written over NaN-filled buffers.  magnitude_scaled: the max bound
    of O scales with max |O_ref| / 2 (inputs outside the i.i.d. recipe)."""
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out = nan_fwd_out(qd)
    if mask is None:
        o, lse = _lib.forward(qd, kd, vd, causal=causal, out=out)
    else:
        o, lse = _lib.forward_blocksparse(qd, kd, vd, mask.to(DEV), causal=causal, out=out)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any(), "unwritten output"
    scale = q.shape[-1] ** -0.5
    so, sl = Stats("O"), Stats("lse")
    for pc in chunks(all_pairs(q), chunk):
        ro, rl = oracle.forward(heads_of(q, pc), heads_of(k, pc), heads_of(v, pc), scale, causal,
                                block_mask=None if mask is None else mask.numpy(),
                                mask_block=128)
        so.add(heads_of(o, pc), ro)
        check_lse(torch.stack([lse[b, h] for b, h in pc]), rl, stats=sl)
    so.check(max_scale=max(1.0, so.refmax / 2) if magnitude_scaled else 1.0)
    sl.check()
    return o, lse


def backward_parity_all_heads(q, k, v, do, causal, mask=None, chunk=8):
    """Forward (LSE) and the whole backward output against the oracle, the
    gradients written over NaN-filled buffers."""
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out = nan_bwd_out(qd, kd)
    if mask is None:
        o, lse = _lib.forward(qd, kd, vd, causal=causal)
        dq, dk, dv = _lib.backward(qd, kd, vd, o, dod, lse, causal=causal, out=out)
    else:
        md = mask.to(DEV)
        o, lse = _lib.forward_blocksparse(qd, kd, vd, md, causal=causal)
        dq, dk, dv = _lib.backward_blocksparse(qd, kd, vd, o, dod, lse, md, causal=causal,
                                               out=out)
    torch.cuda.synchronize()
    dq, dk, dv, lse = dq.cpu(), dk.cpu(), dv.cpu(), lse.cpu()
    for name, g in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert not torch.isnan(g).any(), f"unwritten {name}"
    scale = q.shape[-1] ** -0.5
    st = {n: Stats(n) for n in ("dQ", "dK", "dV", "lse")}
    for pc in chunks(all_pairs(q), chunk):
        rdq, rdk, rdv, rl, _ = oracle.backward(heads_of(q, pc), heads_of(k, pc),
                                               heads_of(v, pc), heads_of(do, pc), scale, causal,
                                               block_mask=None if mask is None else mask.numpy(),
                                               mask_block=128)
        for name, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
            st[name].add(heads_of(g, pc), r)
        check_lse(torch.stack([lse[b, h] for b, h in pc]), rl, stats=st["lse"])
    for x in st.values():
        x.check()
    return dq, dk, dv


def forward_parity(q, k, v, causal, pairs, mask=None, bf16=True):
    o, lse = run_forward(q, k, v, causal, mask)
    scale = q.shape[-1] ** -0.5
    ro, rl = oracle.forward(heads_of(q, pairs), heads_of(k, pairs), heads_of(v, pairs), scale,
                            causal, block_mask=None if mask is None else mask.numpy(),
                            mask_block=128)
    go = np.stack([to64(o[b, h]) for b, h in pairs])
    gl = torch.stack([lse[b, h] for b, h in pairs])
    check("O", go, ro, bf16)
    check_lse(gl, rl, bf16)
    return o, lse


# ------------------------------------------------------------------ forward
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 63, 65, 129, 200, 333])
def test_forward_bf16_small(N, d, causal):
    need_gpu()
    log(f"forward bf16 B2 H3 N{N} d{d} causal={causal}")
    q, k, v = inputs.qkv(2, 3, N, d, torch.bfloat16, seed=N + d)
    forward_parity(q, k, v, causal, all_pairs(q))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 128, 150])
def test_forward_f32_small(N, d, causal):
    need_gpu()
    log(f"forward f32 B2 H2 N{N} d{d} causal={causal}")
    q, k, v = inputs.qkv(2, 2, N, d, torch.float32, seed=7 * N + d)
    forward_parity(q, k, v, causal, all_pairs(q), bf16=False)


def test_forward_f32_single_head_workload():
    need_gpu()
    w = inputs.WORKLOADS["single_head_f32"]
    for seed in (0, 1, 2):
        log(f"{w.name} seed {seed}")
        x = inputs.workload_inputs(w, seed)
        forward_parity(x["q"], x["k"], x["v"], w.causal, all_pairs(x["q"]), bf16=False)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", ["batched_d64", "batched_d64_causal", "long_d128_causal"])
def test_forward_full_workloads(name, seed):
    """Every head of the batched (B8 H16 N1024 d64, causal and not) and long
    (B1 H32 N8192 d128 causal) forward workloads."""
    need_gpu()
    w = inputs.WORKLOADS[name]
    log(f"{name} seed {seed} (B{w.B} H{w.H} N{w.N} d{w.d} causal={w.causal}), all heads")
    x = inputs.workload_inputs(w, seed)
    forward_parity_all_heads(x["q"], x["k"], x["v"], w.causal)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 50, 64, 65, 128, 129, 192, 200, 333, 600])
def test_forward_resident_grid(N, causal, d):
    """Enough heads (B4 H130: at least one 256-row query tile per CU) that
    the launch takes the resident hand-scheduled kernel of its head dim, at
    short, ragged N: 1, 2, 3, ... key tiles per item, so the K/V stages
    start and end at every phase."""
    need_gpu()
    log(f"forward bf16 B4 H130 N{N} d{d} causal={causal} (resident grid)")
    q, k, v = inputs.qkv(4, 130, N, d, torch.bfloat16, seed=1000 + N + d)
    forward_parity_all_heads(q, k, v, causal, chunk=130)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_resident_grid_odd_item_count(causal, d):
    """B1 H261 N300: 522 query tiles of 256 rows (783 of 128 rows), a count
    that is no multiple of the 8 XCDs, so the resident kernels hand out their
    items by the plain serpentine over all workgroups instead of per-XCD
    shares; every head against the oracle."""
    need_gpu()
    log(f"forward bf16 B1 H261 N300 d{d} causal={causal} (item count not a multiple of 8)")
    q, k, v = inputs.qkv(1, 261, 300, d, torch.bfloat16, seed=4000 + d + int(causal))
    forward_parity_all_heads(q, k, v, causal, chunk=87)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("H", [255, 256])
def test_forward_resident_threshold(H, d):
    """B1 N256: H 255 gives 255 query tiles of 256 rows (the compiler-scheduled
    kernel), H 256 gives 256 (the first grid the resident kernel takes); both
    sides of the switch against the oracle, causal."""
    need_gpu()
    log(f"forward bf16 B1 H{H} N256 d{d} causal (resident threshold)")
    q, k, v = inputs.qkv(1, H, 256, d, torch.bfloat16, seed=4200 + H + d)
    forward_parity_all_heads(q, k, v, True, chunk=64)


@pytest.mark.parametrize("H", [127, 128, 256])
def test_backward_resident_threshold(H):
    """B1 N256 d128 causal: H 127 gives 254 dK/dV items of 128 keys (both
    passes compiler-scheduled), H 128 gives 256 (the resident dK/dV kernel,
    with 128 dQ items still compiler-scheduled), H 256 makes both resident;
    every gradient against the oracle."""
    need_gpu()
    log(f"backward bf16 B1 H{H} N256 d128 causal (resident thresholds)")
    q, k, v, do = inputs.qkv(1, H, 256, 128, torch.bfloat16, seed=4300 + H, with_dout=True)
    backward_parity_all_heads(q, k, v, do, True, chunk=64)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_resident_odd_item_count(causal):
    """B1 H261 N300 d128: 783 dK/dV items of 128 keys and 522 dQ items of 256
    rows, neither a multiple of the 8 XCDs, so both resident backward kernels
    use the plain serpentine over all workgroups; every gradient of every
    head against the oracle."""
    need_gpu()
    log(f"backward bf16 B1 H261 N300 d128 causal={causal} (item counts not multiples of 8)")
    q, k, v, do = inputs.qkv(1, 261, 300, 128, torch.bfloat16, seed=4100 + int(causal),
                             with_dout=True)
    backward_parity_all_heads(q, k, v, do, causal, chunk=87)


@pytest.mark.parametrize("N", [4096, 4097])
def test_forward_d64_causal_workgroup_shapes(N):
    """Causal d = 64 at the longest sequence that takes the 2-wave, 128-row
    workgroups (N = 4096) and one past it (4-wave, 256-row workgroups, with a
    ragged last tile): B1 H16 gives at least 256 query tiles of 256 rows, so
    both take the resident kernel; every head against the oracle."""
    need_gpu()
    log(f"forward bf16 B1 H16 N{N} d64 causal (2-wave / 4-wave boundary)")
    q, k, v = inputs.qkv(1, 16, N, 64, torch.bfloat16, seed=3000 + N)
    forward_parity_all_heads(q, k, v, True, chunk=4)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [700, 1500])
def test_forward_reference_moves_mid_sequence(N, causal, d):
    """Keys from the fourth 64-key tile on scaled by 3, so that those tiles'
    scores exceed the running reference set by the first tiles by far more
    than 2^3 per weight: the hand-scheduled loop must take its exact path
    (row maximum, rescale, recomputed weights) there, in the launch
    configuration of the long workloads (B2 H130: more than one 256-row
    workgroup per CU).  Such keys make the attention nearly one-hot, so O
    reaches V's magnitude (|O| up to about 4.3, where one bf16 ulp is
    2^-6 and rounding O alone costs 7.8e-3): the max bound of O scales with
    max |O_ref| / 2."""
    need_gpu()
    log(f"forward bf16 B2 H130 N{N} d{d} causal={causal}, keys x3 from key 192 on")
    q, k, v = inputs.qkv(2, 130, N, d, torch.bfloat16, seed=2000 + N + d)
    kscale = torch.ones(N, dtype=torch.float32)
    kscale[192:] = 3.0
    k = (k.float() * kscale[None, None, :, None]).to(torch.bfloat16)
    forward_parity_all_heads(q, k, v, causal, chunk=65, magnitude_scaled=True)


def test_caller_outputs_match_fresh_outputs():
    """forward/backward with caller-owned output buffers (out=) write exactly
    what they return with fresh ones, also over stale contents."""
    need_gpu()
    q, k, v, do = (t.to(DEV) for t in inputs.qkv(2, 3, 200, 128, torch.bfloat16, seed=5,
                                                  with_dout=True))
    o, lse = _lib.forward(q, k, v, causal=True)
    fo = (torch.full_like(o, 7.0), torch.full_like(lse, -3.0))
    ro = _lib.forward(q, k, v, causal=True, out=fo)
    g = _lib.backward(q, k, v, o, do, lse, causal=True)
    bo = tuple(torch.full_like(x, 11.0) for x in g)
    rb = _lib.backward(q, k, v, o, do, lse, causal=True, out=bo)
    torch.cuda.synchronize()
    assert ro[0] is fo[0] and ro[1] is fo[1] and all(x is y for x, y in zip(rb, bo))
    assert torch.equal(fo[0], o) and torch.equal(fo[1], lse)
    for x, y in zip(bo, g):
        assert torch.equal(x, y)
    with pytest.raises(ValueError):
        _lib.forward(q, k, v, out=(fo[0].float(), fo[1]))


def test_caller_outputs_other_entry_points():
    """out= on the tile-mask, grouped-head and fp8 entry points."""
    need_gpu()
    q, k, v, do = (t.to(DEV) for t in inputs.qkv(1, 4, 300, 64, torch.bfloat16, seed=6,
                                                  with_dout=True))
    mask = inputs.block_mask(300, 128, 1, 0.5, 6).to(DEV)
    calls = [
        (lambda out=None: _lib.forward_blocksparse(q, k, v, mask, causal=True, out=out)),
        (lambda out=None: _lib.forward_gqa(q, k[:, :2].contiguous(), v[:, :2].contiguous(),
                                           causal=False, out=out)),
    ]
    f8 = inputs.qkv_fp8(1, 4, 300, 64, 6)
    q8, k8, v8 = (x[0].to(DEV) for x in f8)
    calls.append(lambda out=None: _lib.forward_fp8(q8, k8, v8, *(x[1] for x in f8),
                                                   causal=True, out=out))
    for fn in calls:
        o, lse = fn()
        buf = (torch.full_like(o, 5.0), torch.full_like(lse, 2.0))
        fn(out=buf)
        torch.cuda.synchronize()
        assert torch.equal(buf[0], o) and torch.equal(buf[1], lse)
    o, lse = _lib.forward_blocksparse(q, k, v, mask, causal=True)
    g = _lib.backward_blocksparse(q, k, v, o, do, lse, mask, causal=True)
    bo = tuple(torch.full_like(x, 3.0) for x in g)
    _lib.backward_blocksparse(q, k, v, o, do, lse, mask, causal=True, out=bo)
    torch.cuda.synchronize()
    for x, y in zip(bo, g):
        assert torch.equal(x, y)


def test_causal_row_zero_is_v0_exactly():
    need_gpu()
    q, k, v = inputs.qkv(2, 2, 300, 128, torch.bfloat16, seed=3)
    o, lse = run_forward(q, k, v, True)
    assert torch.equal(o[:, :, 0], v[:, :, 0])


def test_forward_on_a_side_stream_matches_default_stream():
    need_gpu()
    q, k, v = (t.to(DEV) for t in inputs.qkv(2, 4, 777, 128, torch.bfloat16, seed=5))
    o1, l1 = _lib.forward(q, k, v, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = _lib.forward(q, k, v, causal=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_forward_allocates_nothing_quadratic():
    need_gpu()
    B, H, N, d = 1, 8, 8192, 128
    q, k, v = (t.to(DEV) for t in inputs.qkv(B, H, N, d, torch.bfloat16, seed=0))
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    o, lse = _lib.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated() - base
    outputs = o.numel() * 2 + lse.numel() * 4
    log(f"  peak extra {extra} B, outputs {outputs} B, one score matrix {N * N * 2} B")
    assert extra <= outputs + (1 << 20)


# ----------------------------------------------------------------- backward
def backward_parity(q, k, v, do, causal, pairs):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = _lib.forward(qd, kd, vd, causal=causal)
    dq, dk, dv = _lib.backward(qd, kd, vd, o, dod, lse, causal=causal)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    scale = q.shape[-1] ** -0.5
    rdq, rdk, rdv, _, _ = oracle.backward(heads_of(q, pairs), heads_of(k, pairs),
                                          heads_of(v, pairs), heads_of(do, pairs), scale, causal)
    for name, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        check(name, np.stack([to64(g[b, h]) for b, h in pairs]), r)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 40, 64, 129, 200, 333])
def test_backward_small(N, d, causal):
    need_gpu()
    log(f"backward B2 H2 N{N} d{d} causal={causal}")
    q, k, v, do = inputs.qkv(2, 2, N, d, torch.bfloat16, seed=11 * N + d, with_dout=True)
    backward_parity(q, k, v, do, causal, all_pairs(q))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_full_workload(seed):
    """Every head of the backward workload (B4 H16 N4096 d128 causal)."""
    need_gpu()
    w = inputs.WORKLOADS["bwd_d128_causal"]
    log(f"{w.name} seed {seed} (B{w.B} H{w.H} N{w.N} d{w.d} causal={w.causal}), all heads")
    x = inputs.workload_inputs(w, seed)
    backward_parity_all_heads(x["q"], x["k"], x["v"], x["dout"], w.causal)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_batched_d64(causal):
    """d=64 backward at the batched shape (B8 H16 N1024), every head."""
    need_gpu()
    log(f"backward B8 H16 N1024 d64 causal={causal}, all heads")
    q, k, v, do = inputs.qkv(8, 16, 1024, 64, torch.bfloat16, seed=5, with_dout=True)
    backward_parity_all_heads(q, k, v, do, causal, chunk=32)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 129, 200, 333, 700])
def test_backward_resident_grid(N, causal):
    """Enough heads (B2 H130: at least one 256-row query tile and one 128-key
    block per CU) that the dQ and dK/dV passes take the resident
    hand-scheduled d = 128 kernels, at short and ragged N: 1 to 11 tiles per
    item, so their stages start and end at every tile index modulo 4, with
    masked, general and final steps, and partial key blocks."""
    need_gpu()
    log(f"backward bf16 B2 H130 N{N} d128 causal={causal} (resident dQ, dK/dV)")
    q, k, v, do = inputs.qkv(2, 130, N, 128, torch.bfloat16, seed=3000 + N, with_dout=True)
    backward_parity_all_heads(q, k, v, do, causal, chunk=65)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_resident_dq_grouped_heads(causal, d):
    """Grouped K/V heads (130 query heads over 26) through the resident
    forward kernels and the resident dQ kernel (d = 128): each query head
    reads its group's K and V."""
    need_gpu()
    log(f"gqa forward+backward B2 H130 Hkv26 N333 d{d} causal={causal} (resident)")
    gqa_parity(2, 130, 26, 333, d, causal, seed=44 + d)


@pytest.mark.parametrize("B,H,Hkv,N,causal", [(2, 130, 65, 700, False), (2, 130, 65, 700, True),
                                              (1, 32, 1, 4096, True), (1, 32, 1, 4096, False)])
def test_backward_resident_grouped_heads(B, H, Hkv, N, causal):
    """Grouped K/V heads through the resident dK/dV kernel, which runs its
    query loop once per query head of an item's group and carries the
    accumulators: two heads per group, one slice (B2 H130 Hkv65, 780 items);
    MQA with the group in 16 slices of two heads, partial sums reduced
    (B1 H32 Hkv1 N4096, 512 items)."""
    need_gpu()
    log(f"gqa backward B{B} H{H} Hkv{Hkv} N{N} d128 causal={causal} (resident dK/dV)")
    gqa_parity(B, H, Hkv, N, 128, causal, seed=N + H + Hkv)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_resident_long(causal):
    """The resident d = 128 backward kernels over long sequences (B2 H16
    N2048: 32 query tiles per dK/dV item, 32 key tiles per dQ item), every
    head."""
    need_gpu()
    log(f"backward bf16 B2 H16 N2048 d128 causal={causal} (resident), all heads")
    q, k, v, do = inputs.qkv(2, 16, 2048, 128, torch.bfloat16, seed=77, with_dout=True)
    backward_parity_all_heads(q, k, v, do, causal, chunk=8)


def test_backward_resident_is_deterministic():
    need_gpu()
    q, k, v, do = (t.to(DEV) for t in inputs.qkv(2, 130, 333, 128, torch.bfloat16, seed=8,
                                                 with_dout=True))
    o, lse = _lib.forward(q, k, v, causal=True)
    a = _lib.backward(q, k, v, o, do, lse, causal=True)
    b = _lib.backward(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_is_deterministic():
    need_gpu()
    q, k, v, do = (t.to(DEV) for t in inputs.qkv(2, 4, 1000, 128, torch.bfloat16, seed=9,
                                                 with_dout=True))
    outs = []
    for _ in range(3):
        o, lse = _lib.forward(q, k, v, causal=True)
        outs.append((o, lse) + _lib.backward(q, k, v, o, do, lse, causal=True))
    torch.cuda.synchronize()
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)


# ------------------------------------------------------------- block-sparse
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [100, 300, 700])
def test_blocksparse_small(N, d, causal):
    need_gpu()
    log(f"block-sparse B2 H2 N{N} d{d} causal={causal}")
    q, k, v = inputs.qkv(2, 2, N, d, torch.bfloat16, seed=13 * N + d)
    nb = -(-N // 128)
    g = torch.Generator().manual_seed(N)
    mask = (torch.rand(nb, nb, generator=g) < 0.5).to(torch.uint8)
    if nb > 1:
        mask[1, :] = 0  # an empty mask row: O = 0, LSE = -inf
    forward_parity(q, k, v, causal, all_pairs(q), mask=mask)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_full_workload(causal, seed):
    """Every head of the block-sparse workload (B1 H16 N16384 d64, 2048 of
    16384 tiles)."""
    need_gpu()
    w = inputs.WORKLOADS["blocksparse_d64"]
    x = inputs.workload_inputs(w, seed)
    log(f"{w.name} seed {seed} causal={causal}: {int(x['mask'].sum())} of "
        f"{x['mask'].numel()} tiles, all heads")
    forward_parity_all_heads(x["q"], x["k"], x["v"], causal, mask=x["mask"])


def test_blocksparse_mask_identities():
    need_gpu()
    N = 1000
    nb = -(-N // 128)
    q, k, v = inputs.qkv(1, 4, N, 64, torch.bfloat16, seed=21)
    od, ld = run_forward(q, k, v, False)
    o1, l1 = run_forward(q, k, v, False, mask=torch.ones(nb, nb, dtype=torch.uint8))
    assert torch.equal(od, o1) and torch.equal(ld, l1)
    oc, lc = run_forward(q, k, v, True)
    tri = torch.ones(nb, nb, dtype=torch.uint8).tril()
    o2, l2 = run_forward(q, k, v, True, mask=tri)
    assert torch.equal(oc, o2) and torch.equal(lc, l2)
    o3, l3 = run_forward(q, k, v, False, mask=torch.zeros(nb, nb, dtype=torch.uint8))
    assert torch.all(o3 == 0) and torch.all(torch.isneginf(l3))


def test_blocksparse_two_key_halves_merge_to_the_full_result():
    """The sequence-sharding combine rule: attention over two disjoint key sets,
    merged with their LSEs, equals attention over all keys."""
    need_gpu()
    N, nb = 1000, 8
    q, k, v = inputs.qkv(1, 4, N, 128, torch.bfloat16, seed=31)
    full_o, full_l = run_forward(q, k, v, False)
    left = torch.zeros(nb, nb, dtype=torch.uint8)
    left[:, : nb // 2] = 1
    oa, la = run_forward(q, k, v, False, mask=left)
    ob, lb = run_forward(q, k, v, False, mask=1 - left)
    lse = torch.logaddexp(la, lb)
    o = torch.exp(la - lse)[..., None] * oa.float() + torch.exp(lb - lse)[..., None] * ob.float()
    assert (o - full_o.float()).abs().max() <= 1e-2
    assert (lse - full_l).abs().max() <= 1e-5


# ------------------------------------------------------ block-sparse backward
def backward_parity_sparse(q, k, v, do, causal, pairs, mask):
    qd, kd, vd, dod, md = (t.to(DEV) for t in (q, k, v, do, mask))
    o, lse = _lib.forward_blocksparse(qd, kd, vd, md, causal=causal)
    dq, dk, dv = _lib.backward_blocksparse(qd, kd, vd, o, dod, lse, md, causal=causal)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    scale = q.shape[-1] ** -0.5
    rdq, rdk, rdv, _, _ = oracle.backward(heads_of(q, pairs), heads_of(k, pairs),
                                          heads_of(v, pairs), heads_of(do, pairs), scale, causal,
                                          block_mask=mask.numpy(), mask_block=128)
    for name, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        check(name, np.stack([to64(g[b, h]) for b, h in pairs]), r)
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_mask_rows_longer_than_one_chunk(d, causal):
    """Mask rows and columns of 71 blocks (N = 9000); the kernels read the mask
    64 entries at a time.  Rows 0-9 see only block 70 (in the second chunk;
    causal: nothing), rows 10-19 see nothing (O = 0, LSE = -inf, dQ = 0), the
    rest see the diagonal and blocks 3 and 66; no row sees block 5 (dK = dV =
    0 there)."""
    need_gpu()
    N, nb = 9000, 71
    log(f"block-sparse 71-block mask rows B1 H2 N{N} d{d} causal={causal}")
    mask = torch.zeros(nb, nb, dtype=torch.uint8)
    mask[0:10, 70] = 1
    for i in range(20, nb):
        mask[i, i] = 1
        mask[i, 3] = 1
        mask[i, 66] = 1
    q, k, v, do = inputs.qkv(1, 2, N, d, torch.bfloat16, seed=900 + d, with_dout=True)
    o, lse = forward_parity(q, k, v, causal, all_pairs(q), mask=mask)
    dead = slice(0, 1280) if causal else slice(1280, 2560)
    assert torch.all(o[:, :, dead] == 0) and torch.all(torch.isneginf(lse[:, :, dead]))
    dq, dk, dv = backward_parity_sparse(q, k, v, do, causal, all_pairs(q), mask)
    assert torch.all(dq[:, :, dead] == 0)
    assert torch.all(dk[:, :, 640:768] == 0) and torch.all(dv[:, :, 640:768] == 0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [100, 300, 700])
def test_blocksparse_backward_small(N, d, causal):
    need_gpu()
    log(f"block-sparse backward B2 H2 N{N} d{d} causal={causal}")
    q, k, v, do = inputs.qkv(2, 2, N, d, torch.bfloat16, seed=17 * N + d, with_dout=True)
    nb = -(-N // 128)
    g = torch.Generator().manual_seed(N + 1)
    mask = (torch.rand(nb, nb, generator=g) < 0.5).to(torch.uint8)
    if nb > 2:
        mask[1, :] = 0  # an empty mask row: dQ = 0
        mask[:, 2] = 0  # an empty mask column: dK = dV = 0
    dq, dk, dv = backward_parity_sparse(q, k, v, do, causal, all_pairs(q), mask)
    if nb > 2:
        assert torch.all(dq[:, :, 128:256] == 0)
        assert torch.all(dk[:, :, 256:384] == 0) and torch.all(dv[:, :, 256:384] == 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_backward_full_workload(causal, seed):
    """Every head of the block-sparse workload's backward (dO drawn fourth
    from the same seed, as for the dense backward workload)."""
    need_gpu()
    w = inputs.WORKLOADS["blocksparse_d64"]
    q, k, v, do = inputs.qkv(w.B, w.H, w.N, w.d, torch.bfloat16, seed=seed, with_dout=True)
    mask = inputs.block_mask(w.N, w.mask_block, w.band, w.density, seed)
    log(f"{w.name} backward seed {seed} causal={causal}, all heads")
    backward_parity_all_heads(q, k, v, do, causal, mask=mask)


@pytest.mark.parametrize("d", [64, 128])
def test_blocksparse_backward_mask_identities(d):
    """All-ones mask = dense and lower-triangular mask + causal = causal, bitwise."""
    need_gpu()
    N = 1000
    nb = -(-N // 128)
    q, k, v, do = (t.to(DEV) for t in inputs.qkv(1, 3, N, d, torch.bfloat16, seed=23,
                                                 with_dout=True))
    for causal, mask in ((False, torch.ones(nb, nb, dtype=torch.uint8)),
                         (True, torch.ones(nb, nb, dtype=torch.uint8).tril())):
        o, lse = _lib.forward(q, k, v, causal=causal)
        dense = _lib.backward(q, k, v, o, do, lse, causal=causal)
        sparse = _lib.backward_blocksparse(q, k, v, o, do, lse, mask.to(DEV), causal=causal)
        torch.cuda.synchronize()
        for a, b in zip(dense, sparse):
            assert torch.equal(a, b)


# ------------------------------------------------------- grouped K/V heads
def gqa_parity(B, H, Hkv, N, d, causal, seed, backward=True):
    q, _, _, do = inputs.qkv(B, H, N, d, torch.bfloat16, seed=seed, with_dout=True)
    _, k, v = inputs.qkv(B, Hkv, N, d, torch.bfloat16, seed=seed + 1)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = _lib.forward_gqa(qd, kd, vd, causal=causal)
    scale = d ** -0.5
    ro, rl = oracle.forward_gqa(q, k, v, scale, causal)
    check("O", to64(o.cpu()), ro)
    check_lse(lse.cpu(), rl, True)
    if backward:
        dq, dk, dv = _lib.backward_gqa(qd, kd, vd, o, dod, lse, causal=causal)
        rdq, rdk, rdv, _, _ = oracle.backward_gqa(q, k, v, do, scale, causal)
        check("dQ", to64(dq.cpu()), rdq)
        # A shared head's dK, dV sum H/Hkv per-head gradients with independent
        # rounding errors: the max bound grows as sqrt(H/Hkv).  The mean bound
        # is not widened.
        for name, g, r in (("dK", dk, rdk), ("dV", dv, rdv)):
            check(name, to64(g.cpu()), r, max_scale=(H // Hkv) ** 0.5)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward_sliced_and_whole_groups(d, causal):
    """fa_backward_gqa with the larger workspace splits each group's query
    heads over several dK/dV workgroups and adds their partials in order;
    with the plain workspace one workgroup sums the group.  Both match the
    oracle, and each other up to fp32 summation order."""
    need_gpu()
    B, H, Hkv, N = 1, 8, 1, 333
    log(f"gqa sliced vs whole B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    q, _, _, do = inputs.qkv(B, H, N, d, torch.bfloat16, seed=77, with_dout=True)
    _, k, v = inputs.qkv(B, Hkv, N, d, torch.bfloat16, seed=78)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = _lib.forward_gqa(qd, kd, vd, causal=causal)
    small = _lib.backward_workspace_size(B, H, N, d)
    big = _lib.backward_gqa_workspace_size(B, H, Hkv, N, d)
    assert big > small
    whole = _lib.backward_gqa(qd, kd, vd, o, dod, lse, causal=causal,
                              workspace=torch.empty(small, dtype=torch.uint8, device=DEV))
    sliced = _lib.backward_gqa(qd, kd, vd, o, dod, lse, causal=causal,
                               workspace=torch.full((big,), 255, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    rdq, rdk, rdv, _, _ = oracle.backward_gqa(q, k, v, do, d ** -0.5, causal)
    for name, gw, gs, r in zip(("dQ", "dK", "dV"), whole, sliced, (rdq, rdk, rdv)):
        grow = 1.0 if name == "dQ" else (H // Hkv) ** 0.5  # sum over the group
        check(name + " whole", to64(gw.cpu()), r, max_scale=grow)
        check(name + " sliced", to64(gs.cpu()), r, max_scale=grow)
        assert torch.allclose(gw, gs, rtol=1e-5, atol=1e-5), name
    assert torch.equal(whole[0], sliced[0])  # dQ does not depend on the split


def test_gqa_sliced_backward_is_deterministic():
    """The sliced grouped-head backward adds the slices' partials in a fixed
    order: two runs give bitwise the same gradients."""
    need_gpu()
    B, H, Hkv, N, d = 1, 8, 1, 700, 128
    q, _, _, do = (t.to(DEV) for t in inputs.qkv(B, H, N, d, torch.bfloat16, seed=3,
                                                  with_dout=True))
    _, k, v = (t.to(DEV) for t in inputs.qkv(B, Hkv, N, d, torch.bfloat16, seed=4))
    o, lse = _lib.forward_gqa(q, k, v, causal=True)
    assert _lib.backward_gqa_workspace_size(B, H, Hkv, N, d) > _lib.backward_workspace_size(B, H, N, d)
    a = _lib.backward_gqa(q, k, v, o, do, lse, causal=True)
    b = _lib.backward_gqa(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_mqa_backward_sliced_long():
    """One K/V head shared by 16 query heads at N = 4096: the dK/dV pass runs
    16 query-head slices (32 key tiles x 16 = 512 workgroups) and adds their
    partials; the whole result against the oracle."""
    need_gpu()
    log("mqa B1 H16 Hkv1 N4096 d128 causal (sliced dK/dV)")
    assert (_lib.backward_gqa_workspace_size(1, 16, 1, 4096, 128)
            - _lib.backward_workspace_size(1, 16, 4096, 128)) == 256 + 2 * 16 * 4096 * 128 * 4
    gqa_parity(1, 16, 1, 4096, 128, True, seed=91)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv,N", [(4, 2, 65), (4, 1, 200), (6, 3, 333)])
def test_gqa_small(H, Hkv, N, d, causal):
    need_gpu()
    log(f"gqa B2 H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    gqa_parity(2, H, Hkv, N, d, causal, seed=N + H + d)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_larger(causal):
    need_gpu()
    log(f"gqa B1 H8 Hkv2 N1024 d128 causal={causal}")
    gqa_parity(1, 8, 2, 1024, 128, causal, seed=41)


def test_gqa_with_hkv_equal_h_is_plain_attention():
    need_gpu()
    q, k, v, do = (t.to(DEV) for t in inputs.qkv(2, 4, 300, 128, torch.bfloat16, seed=43,
                                                 with_dout=True))
    o1, l1 = _lib.forward(q, k, v, causal=True)
    o2, l2 = _lib.forward_gqa(q, k, v, causal=True)
    g1 = _lib.backward(q, k, v, o1, do, l1, causal=True)
    g2 = _lib.backward_gqa(q, k, v, o1, do, l1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ fp8
# The fp8 forward is compared with the oracle on the dequantized inputs
# (code * descale, exact in fp64).  Its one rounding beyond fp32 level is the
# attention weights' conversion to e4m3 for the second product: weights are
# stored as w' = 2^8 exp(s - m), rounded with relative error <= 2^-4 in the
# normal range and absolute error <= 2^-10 below it, and the row sum uses the
# unrounded weights.  So, per output element,
#   |dO_c| <= sum_j (2^-4 w_j + 2^-10 / L') |v_jc| + fp32 accumulation
#             + 2^-8 |O_c| (bf16 output rounding),
# with w_j = exp(s_j - LSE) the oracle's weights and L' = 2^8 sum_j exp(s_j - m) >= 2^8.
# (The bf16 tolerance of the other tests does not apply: e4m3 keeps 3 mantissa
# bits, so a row with few visible keys can legitimately miss by more.)
def fp8_dequant(codes, descale, pairs):
    return np.stack([codes[b, h].to(torch.float64).numpy() * descale for b, h in pairs])


def fp8_bound(qd, kd, vd, lse, scale, causal):
    """Per-element error bound [n, N, d] for the fp8 forward (fp64, row chunks)."""
    n, N, d = qd.shape
    out = np.zeros_like(qd)
    for i in range(n):
        for r0 in range(0, N, 512):
            s = scale * qd[i, r0:r0 + 512] @ kd[i].T
            rows = np.arange(r0, min(r0 + 512, N))
            if causal:
                s = np.where(np.arange(N)[None, :] > rows[:, None], -np.inf, s)
            w = np.exp(s - lse[i, r0:r0 + 512, None])
            visible = np.isfinite(s)
            absv = np.abs(vd[i])
            rel = 2.0 ** -4 + N * 2.0 ** -24 + 1e-5
            out[i, r0:r0 + 512] = rel * (w @ absv) + 2.0 ** -18 * (visible @ absv)
    return out


def fp8_parity(B, H, N, d, causal, seed, chunk=8):
    """Every head of an fp8 forward against the oracle on the dequantized
    inputs, each element within its derived bound (output over NaN)."""
    (q8, qs), (k8, ks), (v8, vs) = inputs.qkv_fp8(B, H, N, d, seed=seed)
    out = nan_fwd_out(q8, odtype=torch.bfloat16)
    o, lse = _lib.forward_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), qs, ks, vs, causal=causal,
                              out=out)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any(), "unwritten output"
    scale = d ** -0.5
    worst, esum, bsum, n, lmax, emax = 0.0, 0.0, 0.0, 0, 0.0, 0.0
    for pairs in chunks(all_pairs(q8), chunk):
        qd, kd, vd = (fp8_dequant(c, s, pairs) for c, s in ((q8, qs), (k8, ks), (v8, vs)))
        ro, rl = oracle.forward(qd, kd, vd, scale, causal)
        go = np.stack([to64(o[b, h]) for b, h in pairs])
        gl = np.stack([to64(lse[b, h]) for b, h in pairs])
        err = np.abs(go - ro)
        # bf16 output rounding: relative error at most 2^-8 (half an ulp of an
        # 8-significant-bit format).
        bound = fp8_bound(qd, kd, vd, rl, scale, causal) + 2.0 ** -8 * np.abs(ro) + 1e-6
        assert bool((err <= bound).all()), "fp8 O outside its derived error bound"
        worst = max(worst, float((err / bound).max()))
        emax = max(emax, float(err.max()))
        esum += float(err.sum())
        bsum += float(bound.sum())
        n += err.size
        lmax = max(lmax, float(np.abs(gl - rl).max()))
    log(f"  fp8 O: max_abs={emax:.3e} mean_abs={esum / n:.3e} max err/bound={worst:.3f}")
    # The bound lines every rounding up against the output; independent
    # roundings leave the typical element far inside it.  A systematic error
    # (a wrong scale, a biased rounding) would not.
    assert esum <= 0.25 * bsum, (esum / n, bsum / n)
    log(f"  fp8 LSE: max_abs={lmax:.3e}")
    assert lmax <= 1e-3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 200, 333])
def test_fp8_forward_small(N, d, causal):
    need_gpu()
    log(f"fp8 forward B2 H2 N{N} d{d} causal={causal}")
    fp8_parity(2, 2, N, d, causal, seed=N + 3 * d)


def test_fp8_forward_long_workload():
    """The long causal shape (B1 H32 N8192 d128) in fp8, every head."""
    need_gpu()
    log("fp8 forward B1 H32 N8192 d128 causal, all heads")
    fp8_parity(1, 32, 8192, 128, True, seed=0, chunk=4)


def test_fp8_forward_batched_workload():
    need_gpu()
    log("fp8 forward B8 H16 N1024 d64 non-causal, all heads")
    fp8_parity(8, 16, 1024, 64, False, seed=1, chunk=32)
