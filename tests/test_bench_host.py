"""Host-side logic of bench.py (CPU only): FLOP conventions and pair counts."""
import dataclasses

import torch

import bench
from exact_io_aware_45_amd import inputs


def brute_pairs(N, mb, mask, causal):
    n = 0
    for i in range(N):
        for j in range(N):
            if mask[i // mb, j // mb] and (not causal or j <= i):
                n += 1
    return n


def test_visible_pairs_match_brute_force():
    g = torch.Generator().manual_seed(3)
    for N, causal in ((300, False), (300, True), (256, True), (77, False)):
        w = dataclasses.replace(inputs.WORKLOADS["blocksparse_d64"], N=N, causal=causal,
                                mask_block=64)
        nb = -(-N // 64)
        mask = (torch.rand(nb, nb, generator=g) < 0.6).to(torch.uint8)
        assert bench.visible_pairs(w, mask) == brute_pairs(N, 64, mask, causal)


def test_flop_conventions():
    w = inputs.WORKLOADS["long_d128_causal"]
    assert bench.flops(w, "fwd") == 4 * 32 * 8192 ** 2 * 128 / 2
    assert bench.flops(w, "bwd") == 10 * 32 * 8192 ** 2 * 128 / 2
    s = inputs.WORKLOADS["blocksparse_d64"]
    m = inputs.block_mask(s.N, 128, 1, 0.125, 0)
    assert bench.flops(s, "fwd", m) == 4 * 16 * 64 * 2048 * 128 * 128
    full = torch.ones(128, 128, dtype=torch.uint8)
    dense = dataclasses.replace(s, sparse=False)
    assert bench.flops(s, "fwd", full) == bench.flops(dense, "fwd")


def test_roofline_picks_the_bound_by_intensity():
    causal = inputs.WORKLOADS["batched_d64_causal"]
    r = bench.roofline(causal, "fwd", 0.01, bench.flops(causal, "fwd"), None, "k")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    long = inputs.WORKLOADS["long_d128_causal"]
    r = bench.roofline(long, "fwd", 0.5, bench.flops(long, "fwd"), None, "k")
    assert r["bound"] == "mfma" and abs(r["frac"] - bench.flops(long, "fwd") / 0.5e-3 / 1e12
                                        / bench.PEAK_BF16_TFLOPS) < 1e-4


def test_fp8_traffic_and_peak():
    import dataclasses as dc
    w = dc.replace(inputs.WORKLOADS["long_d128_causal"], dtype="fp8")
    t = 32 * 8192 * 128
    assert bench.traffic_bytes(w, "fwd") == 3 * t + 2 * t + 32 * 8192 * 4
    assert bench.mfma_peak(w) == 2 * bench.PEAK_BF16_TFLOPS


def test_grouped_head_traffic():
    """K and V (and dK, dV) carry Hkv heads; Q, O, dO, dQ and the row vectors H."""
    w = inputs.WORKLOADS["long_d128_causal"]
    g = dataclasses.replace(w, Hkv=8)
    t = 32 * 8192 * 128 * 2.0   # one bf16 tensor with 32 heads
    kv = t / 4                  # with 8 heads
    rows = 32 * 8192 * 4.0
    assert g.kv_heads == 8 and w.kv_heads == 32
    assert bench.traffic_bytes(g, "fwd") == 2 * t + 2 * kv + rows
    # Q, O, dO (bf16) + K, V (bf16) + LSE in; dQ (fp32, H heads), dK, dV (fp32, Hkv) out;
    # D written and read.
    assert bench.traffic_bytes(g, "bwd") == 3 * t + 2 * kv + rows + 2 * t + 4 * kv + 2 * rows
    assert bench.traffic_bytes(w, "bwd") == 5 * t + rows + 6 * t + 2 * rows
    assert bench.flops(g, "fwd") == bench.flops(w, "fwd")


def test_clock_sampler_reads_the_marked_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1893Mhz *\n2: 2400Mhz\n")
    c = bench.ClockSampler(period=0.001)
    c.path = str(f)
    assert c._read() == 1893
    with c:
        import time
        time.sleep(0.01)
    s = c.summary()
    assert s["mean"] == 1893 and s["min"] == 1893 and s["samples"] >= 1
    assert c.summary(after=time.perf_counter() + 10) is None
    assert c.max_mhz() == 2400
    # 256 CUs at the listed 2400 MHz give the peak the roofline uses
    assert abs(256 * c.max_mhz() * 1e6 * 4096 / 1e12 - bench.PEAK_BF16_TFLOPS) < 0.1
    none = bench.ClockSampler()
    none.path = None
    with none:
        pass
    assert none.summary() is None
