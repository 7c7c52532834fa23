"""Benchmark of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default: one step = fa_forward + fa_backward (the whole forward/backward path)
on the long causal workload: B=1, H=32, N=8192, d=128, bf16, causal, inputs
already resident in HBM.  Timing uses HIP events on the stream the kernels run
on.  Prints ONE JSON line:
  value        whole-step TFLOP/s with the algorithmic FLOP counts
               forward 4*B*H*N^2*d, backward 10*B*H*N^2*d, both halved for causal
               (block-sparse: 4*d resp. 10*d per visible (query, key) pair)
  fwd / bwd    each pass's own time (mean, median and minimum over the timed
               steps), TFLOP/s and fraction of the bf16 MFMA peak
  roofline     the forward kernel (one launch per fa_forward) against the bf16
               dense MFMA peak, or against HBM bandwidth when its arithmetic
               intensity is below the ridge point; the backward call gets the
               same treatment in roofline_bwd
  cpu_baseline the fp64 CPU oracle, timed on this host on a bounded sample of
               the same workload (whole heads, the same passes)
  sclk_mhz     the sustained shader clock the driver reports, sampled over
               the second half of --clock-window seconds of untimed steps run
               after the timed ones (its reading trails the load)

--workload runs one of the other named workloads (exact_io_aware_45_amd.inputs)
with the same line format; forward-only workloads time fa_forward alone.
--fp8 runs a dense workload's forward through fa_forward_fp8 (e4m3 inputs),
priced against the fp8 peak.  --cold writes a 512 MiB buffer before every step
(untimed), so that the inputs come from HBM rather than the last-level cache.
--kv-heads HKV runs a dense workload through the grouped-head entry points.
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 bf16 FLOP/clk/CU (dense; published 2.5 PF)
PEAK_FP8_TFLOPS = 5033.2    # 256 CU x 2.4 GHz x 8192 fp8 FLOP/clk/CU (dense; published 5.0 PF)
PEAK_F32_TFLOPS = 157.3     # fp32 vector
PEAK_HBM_GBS = 8000.0


def mfma_peak(w) -> float:
    """Dense peak of the arithmetic the workload's forward runs in (TFLOP/s)."""
    return {"f32": PEAK_F32_TFLOPS, "fp8": PEAK_FP8_TFLOPS}.get(w.dtype, PEAK_BF16_TFLOPS)


def visible_pairs(w, mask) -> float:
    """(query, key) pairs a block-sparse head computes: sum over set tiles of rows x keys."""
    import torch
    nb = mask.shape[0]
    sizes = torch.tensor([min(w.mask_block, w.N - i * w.mask_block) for i in range(nb)],
                         dtype=torch.float64)
    tiles = mask.to(torch.float64) * sizes[:, None] * sizes[None, :]
    if w.causal:  # diagonal tiles keep their lower triangle, tiles above it nothing
        on_diag = torch.diagonal(mask).to(torch.float64) * sizes * (sizes + 1) / 2
        return float(torch.tril(tiles, -1).sum() + on_diag.sum())
    return float(tiles.sum())


def flops(w, which: str, mask=None) -> float:
    per = {"fwd": 4.0, "bwd": 10.0}[which]
    if mask is not None:
        return per * w.B * w.H * w.d * visible_pairs(w, mask)
    f = per * w.B * w.H * float(w.N) ** 2 * w.d
    return f / 2 if w.causal else f


def traffic_bytes(w, which: str) -> float:
    """Algorithmic HBM bytes of one call: read the inputs once, write the outputs once."""
    es = {"f32": 4.0, "fp8": 1.0}.get(w.dtype, 2.0)
    t = w.B * w.H * w.N * w.d * es   # one input-dtype tensor with the query heads
    tkv = t * w.kv_heads / w.H       # K or V (fewer heads when grouped)
    to = w.B * w.H * w.N * w.d * (4.0 if w.dtype == "f32" else 2.0)  # O (bf16 unless fp32)
    rows = w.B * w.H * w.N * 4.0     # one fp32 [B,H,N] vector
    if which == "fwd":
        return t + 2 * tkv + to + rows  # Q K V in, O + LSE out
    # Q K V O dO + LSE in; fp32 dQ dK dV out; D out/in
    return 3 * t + 2 * tkv + rows + 2 * t + 2 * 2 * tkv + 2 * rows


KERNEL_SOURCES = {
    "fwd_bf16_kernel": ("fa_fwd.hip", "fa_common.hpp"),
    "fwd128_kernel": ("fa_fwd128.hip", "fa_fwd128_loop.inc", "fa_resident.hpp", "fa_common.hpp"),
    "fwd64_kernel": ("fa_fwd64.hip", "fa_fwd64_loop.inc", "fa_fwd64w2_loop.inc", "fa_resident.hpp",
                     "fa_common.hpp"),
    "fa_backward": ("fa_bwd.hip", "fa_bwd_dkdv128.hip", "fa_bwd_dkdv128_loop.inc", "fa_bwd_dq128.hip",
                    "fa_bwd_dq128_loop.inc", "fa_resident.hpp", "fa_common.hpp"),
}


def uses_resident_fwd(w) -> bool:
    """Whether fa_forward takes the hand-scheduled kernel of its head dim
    (fwd128_kernel, fwd64_kernel): bf16, no tile mask, at least 256 query
    tiles of 256 rows."""
    return (w.dtype == "bf16" and w.d in (64, 128) and not w.sparse
            and -(-w.N // 256) * w.B * w.H >= 256)


def source_sha(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "exact_io_aware_45_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(path: str) -> dict:
    """Counter-measured HBM bytes per launch, kept only for unchanged kernel sources."""
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        t = json.load(f)
    shas = t.get("source_sha", {})
    return {k: t[k] for k, files in KERNEL_SOURCES.items()
            if k in t and shas.get(k) == source_sha(files)}


class ClockSampler:
    """Samples the shader clock the driver reports (the line marked '*' of
    pp_dpm_sclk) every `period` seconds on a background thread; summary() is
    None where the file is not readable.  The driver's value trails the load
    by a few hundred milliseconds (it reads ~850 MHz over a 50 ms burst that
    sustains ~1.95 GHz), so summary(after=t) keeps the samples from time t on."""

    def __init__(self, period: float = 0.002):
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if len(paths) == 1 else None  # one GPU: one card
        self.period, self.mhz, self.at = period, [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return int(line.split(":")[1].strip().rstrip("*").strip().lower()
                               .replace("mhz", ""))
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except (OSError, ValueError, IndexError):
                return
            if v is not None:
                self.mhz.append(v)
                self.at.append(time.perf_counter())
            time.sleep(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.path:
            self._stop.set()
            self._thread.join()

    def max_mhz(self):
        """The highest clock level the driver lists (the device's peak clock)."""
        if not self.path:
            return None
        try:
            with open(self.path) as f:
                levels = [int(line.split(":")[1].strip().rstrip("*").strip().lower()
                              .replace("mhz", "")) for line in f if ":" in line]
        except (OSError, ValueError, IndexError):
            return None
        return max(levels) if levels else None

    def summary(self, after: float = 0.0, source: str = ""):
        mhz = [m for m, t in zip(self.mhz, self.at) if t >= after]
        if not mhz:
            return None
        return {"mean": round(sum(mhz) / len(mhz), 1), "min": min(mhz), "max": max(mhz),
                "samples": len(mhz), "source": source or "pp_dpm_sclk"}


def sustained_clock(step, seconds: float):
    """Runs `step` back to back (untimed) for `seconds` and returns the shader
    clock the driver reports over the second half of that window."""
    import torch
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
    return clock.summary(after=t0 + seconds / 2,
                         source=f"pp_dpm_sclk every 2 ms over the second half of {seconds:g} s "
                                "of untimed steps run after the timed ones")


def cpu_baseline(w, inp, passes, mask=None, budget_s: float = 25.0, max_heads: int = 32):
    """Time the fp64 oracle (the same passes, whole heads) on the host cores:
    heads in turn until `max_heads` or `budget_s` seconds (all 32 heads of the
    long workload take about 17 s on 16 threads)."""
    import oracle
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["dout"]
    oracle.build(force=False)
    threads = oracle.max_threads()
    m = None if mask is None else mask.cpu().numpy()
    kw = {} if m is None else {"block_mask": m, "mask_block": w.mask_block}
    G = w.H // w.kv_heads  # query heads per K/V head
    done, t_total = 0, 0.0
    while done < min(max_heads, w.B * w.H) and t_total < budget_s:
        b, h = divmod(done, w.H)
        t0 = time.perf_counter()
        oracle.forward(q[b, h], k[b, h // G], v[b, h // G], w.scale, w.causal, **kw)
        if "bwd" in passes:
            oracle.backward(q[b, h], k[b, h // G], v[b, h // G], do[b, h], w.scale, w.causal,
                            **kw)
        t_total += time.perf_counter() - t0
        done += 1
    per_head = sum(flops(w, p, mask) for p in passes) / (w.B * w.H)
    what = " + ".join({"fwd": "forward", "bwd": "backward"}[p] for p in passes)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         None)
    except OSError:
        pass
    return {"value": round(per_head * done / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "nproc": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)), "cpu_model": model, "kind": "oracle",
            "sample": f"{done} whole head(s) of the workload ({what}, all {w.N} rows), "
                      f"{t_total:.1f} s, fp64, same FLOP convention"}


def roofline(w, which, ms, fl, traffic, kernel):
    """The pass against MFMA peak, or HBM peak when its intensity is below the ridge."""
    by = traffic_bytes(w, which)
    tf = fl / (ms * 1e-3) / 1e12
    gbs = by / (ms * 1e-3) / 1e9
    peak_mfma = mfma_peak(w)
    hbm = fl / by < peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)
    r = {"bound": "hbm" if hbm else "mfma",
         "achieved": round(gbs if hbm else tf, 2),
         "peak": PEAK_HBM_GBS if hbm else peak_mfma,
         "unit": "GB/s" if hbm else "TFLOP/s",
         "frac": round(gbs / PEAK_HBM_GBS if hbm else tf / peak_mfma, 4),
         "traffic": traffic, "kernel": kernel,
         ("flops_per_launch" if which == "fwd" else "flops_per_call"): fl,
         ("avg_launch_ms" if which == "fwd" else "avg_call_ms"): round(ms, 4),
         ("algorithmic_bytes_per_launch" if which == "fwd" else
          "algorithmic_bytes_per_call"): by,
         "intensity_flop_per_byte": round(fl / by, 1),
         "tflops": round(tf, 2), "gbs": round(gbs, 1)}
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters, if present")
    ap.add_argument("--workload", default="long_d128_causal",
                    help="named workload (exact_io_aware_45_amd.inputs.WORKLOADS)")
    ap.add_argument("--causal", choices=("default", "on", "off"), default="default",
                    help="override the workload's causal flag")
    ap.add_argument("--passes", choices=("default", "fwd", "fwd+bwd"), default="default",
                    help="forward only or forward + backward (default: per workload)")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB buffer before every step (outside the timed passes) so "
                         "the inputs are not served from the 256 MB last-level cache")
    ap.add_argument("--fp8", action="store_true",
                    help="fp8 (OCP e4m3) inputs through fa_forward_fp8, forward only")
    ap.add_argument("--clock-window", type=float, default=0.6,
                    help="seconds of untimed steps after the timed ones, over which the "
                         "sustained shader clock is sampled (0: skip)")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="grouped K/V heads: run a dense bf16 workload through fa_forward_gqa "
                         "(and fa_backward_gqa) with this many K/V heads")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import dataclasses

    import torch
    from exact_io_aware_45_amd import _lib, inputs

    if args.workload not in inputs.WORKLOADS:
        print(json.dumps({"error": f"unknown workload {args.workload}",
                          "workloads": sorted(inputs.WORKLOADS)}))
        sys.exit(2)
    w = inputs.WORKLOADS[args.workload]
    if args.causal != "default":
        w = dataclasses.replace(w, causal=args.causal == "on")
    if args.passes == "default":
        passes = ("fwd", "bwd") if (w.backward or w.name == "long_d128_causal") else ("fwd",)
    else:
        passes = tuple(args.passes.split("+"))
    if args.fp8:
        if w.dtype != "bf16" or w.sparse or args.passes == "fwd+bwd":
            print(json.dumps({"error": "fp8 runs the dense bf16 workloads, forward only"}))
            sys.exit(2)
        w = dataclasses.replace(w, dtype="fp8")
        passes = ("fwd",)
    if args.kv_heads:
        if (w.dtype != "bf16" or w.sparse or args.fp8 or args.kv_heads < 1
                or w.H % args.kv_heads):
            print(json.dumps({"error": "--kv-heads takes a dense bf16 workload and a divisor "
                                       "of its head count"}))
            sys.exit(2)
        w = dataclasses.replace(w, Hkv=args.kv_heads)
    if w.dtype == "f32" and "bwd" in passes:
        print(json.dumps({"error": "the fp32 path is forward only"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _lib.load()

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if w.dtype == "fp8":
        f8 = inputs.qkv_fp8(w.B, w.H, w.N, w.d, args.seed)
        descales = [x[1] for x in f8]
        q, k, v = (x[0].to(dev) for x in f8)
        do = None
        # the oracle baseline runs on the dequantized values
        inp = {n: x[0].to(torch.float32) * x[1] for n, x in zip(("q", "k", "v"), f8)}
        inp["dout"] = None
    else:
        host = inputs.qkv(w.B, w.H, w.N, w.d, w.torch_dtype, args.seed, with_dout=True)
        inp = dict(zip(("q", "k", "v", "dout"), host))
        if w.Hkv:  # K, V with their own head count, from the next seed
            _, inp["k"], inp["v"] = inputs.qkv(w.B, w.Hkv, w.N, w.d, w.torch_dtype,
                                               args.seed + 1)
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    mask = None
    if w.sparse:
        mask = inputs.block_mask(w.N, w.mask_block, w.band, w.density, args.seed)
    maskd = None if mask is None else mask.to(dev)
    ws_bytes = (_lib.backward_gqa_workspace_size(w.B, w.H, w.Hkv, w.N, w.d) if w.Hkv
                else _lib.backward_workspace_size(w.B, w.H, w.N, w.d))
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)

    # Outputs are allocated once, outside the timed region, as a serving loop
    # would reuse them: the timed calls are argument checks plus launches.
    fout = (torch.empty(q.shape, dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16,
                        device=dev),
            torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev))
    bout = tuple(torch.empty(x.shape, dtype=torch.float32, device=dev) for x in (q, k, v))

    def fwd():
        if w.dtype == "fp8":
            return _lib.forward_fp8(q, k, v, *descales, causal=w.causal, out=fout)
        if maskd is not None:
            return _lib.forward_blocksparse(q, k, v, maskd, causal=w.causal, out=fout)
        if w.Hkv:
            return _lib.forward_gqa(q, k, v, causal=w.causal, out=fout)
        return _lib.forward(q, k, v, causal=w.causal, out=fout)

    def bwd(o, lse):
        if maskd is not None:
            _lib.backward_blocksparse(q, k, v, o, do, lse, maskd, causal=w.causal, workspace=ws,
                                      out=bout)
        elif w.Hkv:
            _lib.backward_gqa(q, k, v, o, do, lse, causal=w.causal, workspace=ws, out=bout)
        else:
            _lib.backward(q, k, v, o, do, lse, causal=w.causal, workspace=ws, out=bout)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        o, lse = fwd()
        if ev is not None:
            ev[1].record()
        if "bwd" in passes:
            bwd(o, lse)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    flush = (torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None)
    start.record()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 255)
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = sustained_clock(step, args.clock_window) if args.clock_window > 0 else None
    total_ms = start.elapsed_time(end)
    fwd_each = sorted(e[0].elapsed_time(e[1]) for e in evs)
    bwd_each = sorted(e[1].elapsed_time(e[2]) for e in evs)
    fwd_ms = sum(fwd_each) / args.steps
    bwd_ms = sum(bwd_each) / args.steps

    def spread(each):  # median and minimum of the per-step event times
        n = len(each)
        med = each[n // 2] if n % 2 else 0.5 * (each[n // 2 - 1] + each[n // 2])
        return {"ms_median": round(med, 4), "ms_min": round(each[0], 4)}
    # cold runs: the step is the passes alone (the flush between them is not timed)
    ms_per_step = (fwd_ms + bwd_ms) if args.cold else total_ms / args.steps

    ff = flops(w, "fwd", mask)
    fb = flops(w, "bwd", mask) if "bwd" in passes else 0.0
    value = (ff + fb) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = ff / (fwd_ms * 1e-3) / 1e12

    # Counter-measured bytes exist only for the default workload's kernels.
    traffic = (load_traffic(args.traffic_json)
               if w.name == "long_d128_causal" and w.dtype == "bf16" and not w.Hkv else {})

    mode = ("block-sparse " if w.sparse else "") + ("causal" if w.causal else "non-causal")
    nw = 4 if w.sparse else 8
    if w.dtype == "f32":
        fwd_kernel = f"fwd_f32_kernel<d={w.d}> (1 launch per fa_forward_f32)"
    elif w.dtype == "fp8":
        fwd_kernel = (f"fwd_fp8_kernel<d={w.d}, BC=64, {8 if w.d == 128 else 4} waves, {mode}> "
                      "(1 launch per fa_forward_fp8)")
    elif uses_resident_fwd(w):
        entry = "_gqa" if w.Hkv else ""
        shape = ("two resident 2-wave workgroups per CU, 128-row query tiles"
                 if w.d == 64 and w.causal and w.N <= 4096 else
                 "one resident 4-wave workgroup per CU, 256-row query tiles")
        fwd_kernel = f"fwd{w.d}_kernel<{mode}> (1 launch per fa_forward{entry}; {shape})"
    else:
        entry = "_blocksparse" if w.sparse else ("_gqa" if w.Hkv else "")
        fwd_kernel = (f"fwd_bf16_kernel<d={w.d}, BC=64, {nw} waves, {mode}> "
                      f"(1 launch per fa_forward{entry})")
    props = torch.cuda.get_device_properties(dev)
    peak = mfma_peak(w)
    line = {
        "metric": "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak, N=8192 d=128 causal",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "fp8": "fp8-e4m3"}.get(w.dtype, "bf16"),
        "data": "synthetic (i.i.d. N(0,1) Q, K, V, dO from a seeded generator)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal,
                   "pass": "forward+backward" if "bwd" in passes else "forward",
                   "cache": "cold" if args.cold else "warm",
                   "seed": args.seed},
        "frac_of_peak": round(value / peak, 4),
        "fwd": {"ms": round(fwd_ms, 4), **spread(fwd_each), "tflops": round(fwd_tf, 2),
                "frac_of_peak": round(fwd_tf / peak, 4), "flops": ff},
        "roofline": roofline(w, "fwd", fwd_ms, ff,
                             traffic.get(f"fwd{w.d}_kernel" if uses_resident_fwd(w)
                                         else "fwd_bf16_kernel"),
                             fwd_kernel),
    }
    if w.Hkv:
        line["config"]["Hkv"] = w.Hkv
    if w.sparse:
        line["config"]["mask"] = {"tiles": int(mask.sum()), "of": int(mask.numel()),
                                  "block": w.mask_block, "band": w.band,
                                  "density": w.density}
        line["dense_equivalent_fwd_tflops"] = round(
            flops(dataclasses.replace(w, sparse=False), "fwd") / (fwd_ms * 1e-3) / 1e12, 2)
    if "bwd" in passes:
        bwd_tf = fb / (bwd_ms * 1e-3) / 1e12
        line["bwd"] = {"ms": round(bwd_ms, 4), **spread(bwd_each), "tflops": round(bwd_tf, 2),
                       "frac_of_peak": round(bwd_tf / peak, 4), "flops": fb}
        line["roofline_bwd"] = roofline(
            w, "bwd", bwd_ms, fb, traffic.get("fa_backward"),
            f"fa_backward{entry if w.dtype == 'bf16' else ''} call = bwd_delta + bwd_dkdv + "
            "bwd_dq launches")
    line["device"] = {"name": props.name, "cus": props.multi_processor_count,
                      "hip_runtime": _lib.runtime_version(), "libfa": _lib.version()}
    max_mhz = ClockSampler().max_mhz()
    if max_mhz:  # bf16 dense peak from the device: CUs x peak clock x 4096 FLOP/clk/CU
        line["device"]["max_sclk_mhz"] = max_mhz
        line["device"]["bf16_peak_tflops"] = round(
            props.multi_processor_count * max_mhz * 1e6 * 4096 / 1e12, 1)
    line["wall_s_timed_region"] = round(wall, 3)
    line["sclk_mhz"] = sclk
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, passes, mask)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
