#!/usr/bin/env python3
"""Throughput bench for the exact-attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
fa_forward + fa_backward with no mask, then fa_forward + fa_backward with the causal
mask, on the large-head workload (B=2, H=16, N=8192, d=128, bf16 ~ N(0,1), scale
1/sqrt(128); the N >= 4096, d = 128 regime the throughput target is quoted on).

FLOP convention: forward 4*B*H*N^2*d, halved when causal; backward 2.5x the forward.
`value` = total FLOPs of the K timed steps / their wall time (inputs resident in HBM).
The backward runs as its two passes (fa_backward_dq_pass, fa_backward_dkdv_pass: the
same kernels fa_backward launches) so each kernel is timed with its own HIP events.
Algorithmic FLOPs per kernel (for the roofline): forward 4*B*H*N^2*d; dK/dV pass
8*B*H*N^2*d (S, dP, dV, dK); dQ pass 2*B*H*N^2*d (dQ; its recomputation of S and dP is
not algorithmic work); all halved when causal.

Printed JSON line (rank 0 only):
  metric, value (TFLOP/s), unit, n_gpus, steps, warmup, ms_per_step, higher_is_better,
  scaling, vs_baseline, dtype, data, config, detail (per call: TFLOP/s, % of the bf16
  dense peak; "ms" is the mean over the timed steps, with median, min and p90 beside
  it; "machine": the bf16 MFMA, v_exp_f32, LDS-read and fp32-atomic rates the chip
  sustains, from the microbenchmark library), roofline (dominant launch: the largest
  median share of the step; achieved and frac from its mean launch time by HIP events on
  the launch stream, "kernel_ms_median" and "frac_median" from the median launch, which a
  single stalled launch does not move; "frac_of_sustained_mfma" is the mean rate against
  the measured MFMA rate), cpu_baseline (the fp64 oracle on a bounded sample, host cores of this
  machine) and env (device name, architecture, compute units, HBM size, torch and HIP
  runtime versions).

Options: --sweep prints one extra line per workload of the sweep to stderr (for the
short-sequence workloads also a cold-cache time per call: median of single calls, each
after overwriting 512 MiB so that neither the MALL nor an L2 holds the inputs).
Profiling helpers (rocprofv3 runs whose summaries are committed under profiles/):
  --copy-calibration      also time a plain 256 MiB device copy (10 times), the
                          known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters
  --summarize-pmc FETCH_CSV WRITE_CSV OUT.md
                          turn two rocprofv3 --pmc counter CSVs into the traffic summary
                          that `roofline.traffic` reads (valid while the kernel sources
                          keep the hash recorded in it)
"""

import argparse
import csv
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s (bf16, causal & non) + % of MI355X bf16 MFMA peak"


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


# algorithmic FLOPs of one kernel launch, as a multiple of the forward's
KERNEL_FLOP_SHARE = {"fwd": 1.0, "dq": 0.5, "dkdv": 2.0}
KERNEL_NAME = {"fwd": "fa_fwd_kernel", "dq": "fa_bwd_dq_kernel", "dkdv": "fa_bwd_dkdv_kernel"}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attention_b2h16n8192d128_hbm_traffic.md")
COPY_CAL_MIB = 256  # plain device copy that calibrates FETCH_SIZE / WRITE_SIZE


def kernel_source_hash():
    """Hash of the device-code sources of the attention library (the kernels and the
    launch rules that pick them; not the host-side argument checks): a traffic figure
    taken on other kernels is stale."""
    from exact_io_aware_19_amd.build import CSRC, KERNEL_SOURCES

    h = hashlib.sha256()
    for name in sorted(n for n in KERNEL_SOURCES if n != "fa_api.cpp"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 summary, or None
    when there is none or it was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    with open(TRAFFIC_SUMMARY) as f:
        text = f.read()
    m = re.search(r"kernel_source_sha: (\w+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(r"^\| %s \| ([0-9.]+) \|" % re.escape(kernel), text, re.M)
    return float(m.group(1)) if m else None


def _alg_bytes(B, H, N, d, direction, hkv=None):
    """Algorithmic HBM bytes of one call: fwd reads Q,K,V and writes O (bf16) + LSE (fp32);
    bwd reads Q,K,V,O,dO (bf16) + LSE, writes dQ,dK,dV (bf16), writes and reads D (fp32).
    With grouped K/V heads (hkv < H) the K, V, dK, dV terms count hkv heads."""
    rows = B * H * N
    kv_rows = B * (hkv or H) * N
    if direction == "fwd":
        return 4.0 * rows * d + 4.0 * kv_rows * d + 4.0 * rows
    return 8.0 * rows * d + 8.0 * kv_rows * d + 12.0 * rows


def _quantile(xs, q):
    """Linear-interpolated quantile of a list of timings."""
    ys = sorted(xs)
    pos = q * (len(ys) - 1)
    lo = int(math.floor(pos))
    hi = min(lo + 1, len(ys) - 1)
    return ys[lo] + (ys[hi] - ys[lo]) * (pos - lo)


def parse_current_sclk_mhz(text):
    """Current gfx clock (MHz) from the text of the amdgpu sysfs file pp_dpm_sclk: the
    line marked with '*' (a live reading such as 'S: 1843Mhz *', or a DPM level)."""
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            m = re.search(r"(\d+)\s*mhz", line, re.IGNORECASE)
            if m:
                return int(m.group(1))
    return None


def gpu_sysfs_dir(torch):
    """sysfs device directory of GPU 0 (the card with pp_dpm_sclk; with several cards, the
    one on GPU 0's PCI bus), or None."""
    import glob

    cards = sorted(os.path.dirname(f) for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if len(cards) <= 1:
        return cards[0] if cards else None
    bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
    for c in cards:
        addr = os.path.basename(os.path.realpath(c))  # domain:bus:device.function
        try:
            if bus is not None and int(addr.split(":")[1], 16) == int(bus):
                return c
        except (IndexError, ValueError):
            pass
    return None


class ClockSampler:
    """Samples the gfx clock (pp_dpm_sclk) and the board power (hwmon power1_input) from
    sysfs on a host thread: file reads only, no GPU calls (but each clock read queries the
    power-management firmware, which perturbs the GPU, so never during timed work)."""

    def __init__(self, devdir, period_s=0.005):
        import glob
        import threading

        self.devdir, self.period = devdir, period_s
        hw = sorted(glob.glob(os.path.join(devdir, "hwmon", "hwmon*"))) if devdir else []
        self.power_in = os.path.join(hw[0], "power1_input") if hw else None
        self.power_cap = os.path.join(hw[0], "power1_cap") if hw else None
        self.temp_in = None  # the sensor labelled "junction"
        for lab in sorted(glob.glob(os.path.join(hw[0], "temp*_label"))) if hw else []:
            try:
                if self._read(lab).strip() == "junction":
                    self.temp_in = lab[: -len("_label")] + "_input"
            except OSError:
                pass
        self.sclk, self.power, self.temp = [], [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(path):
        with open(path) as f:
            return f.read()

    def _run(self):
        while not self._stop.is_set():
            try:
                mhz = parse_current_sclk_mhz(self._read(os.path.join(self.devdir, "pp_dpm_sclk")))
                if mhz is not None:
                    self.sclk.append(mhz)
                if self.power_in and os.path.exists(self.power_in):
                    self.power.append(int(self._read(self.power_in)) / 1e6)
                if self.temp_in and os.path.exists(self.temp_in):
                    self.temp.append(int(self._read(self.temp_in)) / 1e3)
            except (OSError, ValueError):
                return
            self._stop.wait(self.period)

    def start(self):
        if self.devdir:
            self._thread.start()
        return self

    def stop(self):
        """Summary of the samples (None without a readable clock)."""
        if not self.devdir:
            return None
        self._stop.set()
        self._thread.join(timeout=2.0)
        if not self.sclk:
            return None
        cap = None
        try:
            if self.power_cap and os.path.exists(self.power_cap):
                cap = round(int(self._read(self.power_cap)) / 1e6, 1)
        except (OSError, ValueError):
            pass
        out = {
            "source": "sysfs pp_dpm_sclk (current gfx clock), hwmon power1_input and junction temperature, read every "
                      f"{self.period * 1e3:.0f} ms on a host thread",
            "samples": len(self.sclk),
            "sclk_mhz_median": round(_quantile(self.sclk, 0.5), 1),
            "sclk_mhz_min": min(self.sclk),
            "sclk_mhz_max": max(self.sclk),
            "power_cap_w": cap,
        }
        if self.power:
            out["power_w_median"] = round(_quantile(self.power, 0.5), 1)
            out["power_w_max"] = round(max(self.power), 1)
        if self.temp:
            out["junction_c_median"] = round(_quantile(self.temp, 0.5), 1)
            out["junction_c_max"] = round(max(self.temp), 1)
        return out


def bench_workload(n):
    """The large-head workload of the step: B=2, H=16, d=128, N=n, scale 1/sqrt(d), seeded
    like the sweep's (the same inputs for both mask modes)."""
    from exact_io_aware_19_amd import workloads as wl

    return wl.Workload(f"sweep_n{n}", 2, 16, n, 128, False, 1.0 / math.sqrt(128), 1040 + int(math.log2(n)))


def run_gpu(args):
    import torch
    import exact_io_aware_19_amd as fa
    from exact_io_aware_19_amd import workloads as wl

    dev = torch.device("cuda:0")
    w = bench_workload(args.n)
    B, H, N, d = w.shape
    scale = w.scale
    inp = wl.generate(w, with_do=True)
    t = inp.to_torch(dev)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = {m: torch.empty_like(q) for m in (False, True)}
    lse = {m: torch.empty((B, H, N), dtype=torch.float32, device=dev) for m in (False, True)}
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_backward_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # one step = forward and backward, no mask then causal; the backward as its two
    # passes so that every kernel has its own events
    kern_calls = [("fwd", False), ("dq", False), ("dkdv", False), ("fwd", True), ("dq", True), ("dkdv", True)]
    ev = {c: [] for c in kern_calls}

    def launch(kind, causal):
        if kind == "fwd":
            fa.fa_forward(q, k, v, o[causal], lse[causal], scale, causal, stream=stream)
        else:
            fa.fa_backward_pass(kind, q, k, v, o[causal], do, lse[causal], dq, dk, dv, scale, causal, ws,
                                stream=stream)

    # every timing event exists before the timed region: creating events inside it put
    # host work between an event and its kernel
    pool = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in kern_calls]
            for _ in range(args.steps)]

    def step(record, i=0):
        for j, c in enumerate(kern_calls):
            if record:
                e0, e1 = pool[i][j]
                e0.record(stream)
            launch(*c)
            if record:
                e1.record(stream)
                ev[c].append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The gfx clock and board power, sampled while 20 more (untimed) steps of the same work
    # run right after the timed ones, once they are all enqueued: reading the clock from
    # sysfs queries the power-management firmware and, done during the timed steps,
    # left the GPU idle between kernels (whole-step rate -17%, kernel times unchanged).
    # Only runs that time at least 10 steps do this: the short runs the profiler commands
    # make keep their launch counts and read no sysfs while counters are collected.
    clock = None
    if args.steps >= 10 and args.clock_steps > 0:
        sampler = ClockSampler(gpu_sysfs_dir(torch))
        for _ in range(args.clock_steps):
            step(False)
        sampler.start()
        torch.cuda.synchronize()
        clock = sampler.stop()
        if clock:
            clock["during"] = f"{args.clock_steps} untimed steps of the same work right after the timed steps"

    kms = {c: sum(a.elapsed_time(b) for a, b in ev[c]) / len(ev[c]) for c in kern_calls}
    per_step = {c: [a.elapsed_time(b) for a, b in ev[c]] for c in kern_calls}
    step_flops = 0.0
    detail = {}
    for direction in ("fwd", "bwd"):
        for causal in (False, True):
            f = fwd_flops(B, H, N, d, causal) * (1.0 if direction == "fwd" else 2.5)
            step_flops += f
            ms = kms[("fwd", causal)] if direction == "fwd" else kms[("dq", causal)] + kms[("dkdv", causal)]
            if direction == "fwd":
                samples = per_step[("fwd", causal)]
            else:
                samples = [x + y for x, y in zip(per_step[("dq", causal)], per_step[("dkdv", causal)])]
            tf = f / (ms * 1e-3) / 1e12
            entry = {
                "ms": round(ms, 4),
                "ms_median": round(_quantile(samples, 0.5), 4),
                "ms_min": round(min(samples), 4),
                "ms_p90": round(_quantile(samples, 0.9), 4),
                "tflops": round(tf, 1),
                "pct_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
                "alg_gbs": round(_alg_bytes(B, H, N, d, direction) / (ms * 1e-3) / 1e9, 1),
            }
            if direction == "bwd":
                entry["dq_pass_ms"] = round(kms[("dq", causal)], 4)
                entry["dkdv_pass_ms"] = round(kms[("dkdv", causal)], 4)
            detail[f"{direction}_{'causal' if causal else 'full'}"] = entry
    value = step_flops * args.steps / wall / 1e12
    # per-step kernel time (the six launches' events), whose median a stalled launch
    # does not move
    step_ms = [sum(per_step[c][i] for c in kern_calls) for i in range(args.steps)]
    detail["step_kernels_ms_median"] = round(_quantile(step_ms, 0.5), 4)
    detail["step_kernels_ms_max"] = round(max(step_ms), 4)
    # the gfx clock this work runs at (the peak assumes 2.4 GHz)
    detail["clock"] = clock
    # dominant kernel = the one with the largest share of the step time, by the median
    # launch (a single stalled launch must not make another kernel the dominant one)
    kmed = {c: _quantile(per_step[c], 0.5) for c in kern_calls}
    dom = max(kern_calls, key=lambda c: kmed[c])
    kind, causal = dom
    dom_flops = KERNEL_FLOP_SHARE[kind] * fwd_flops(B, H, N, d, causal)
    achieved = dom_flops / (kms[dom] * 1e-3) / 1e12
    # template arguments: head dim, tile, causal, key padding, then the form the step's
    # launches take: forward unsplit, dQ pass one wave group, dK/dV pass ungrouped heads
    kname = f"{KERNEL_NAME[kind]}<{d}, {64 if d == 128 else 128}, {'true' if causal else 'false'}, false" + (
        {"fwd": ", false>", "dq": ", 1>", "dkdv": ", false>"}[kind])
    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": read_traffic(kname),
        "kernel": kname,
        "kernel_ms": round(kms[dom], 4),
        "kernel_ms_median": round(kmed[dom], 4),
        "frac_median": round(dom_flops / (kmed[dom] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "algorithmic_flops_per_launch": dom_flops,
    }
    if args.fp8:
        detail.update(run_fp8(fa, wl, torch, dev, stream, t, w, args.fp8_iters))
    sweep = []
    if args.sweep:
        sweep = run_sweep(fa, wl, torch, dev, stream)
    return value, wall, detail, roofline, (B, H, N, d), inp, sweep


def copy_calibration(torch):
    """Ten plain device copies of COPY_CAL_MIB MiB (plus one untimed) whose FETCH_SIZE and
    WRITE_SIZE readings calibrate the counters.  main() runs them as the last GPU work of
    the run: the counter summary takes the last ten copy dispatches."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    nbytes = COPY_CAL_MIB << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(e0.elapsed_time(e1) / 10, 4)}


def run_fp8(fa, wl, torch, dev, stream, t, w, iters):
    """FP8 forward (block quantisation + incoherent processing) on the bench inputs: the
    three quantiser calls once per iteration, then fa_forward_fp8 without and with the
    causal mask, each between its own HIP events; TFLOP/s against the fp8 dense peak."""
    B, H, N, d = w.shape
    nb = -(-N // 64)
    signs = torch.from_numpy(wl.fp8_signs(d, w.seed)).to(dev)
    q8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=dev)
    k8 = torch.empty_like(q8)
    v8t = torch.empty((B, H, nb, d, 64), dtype=torch.uint8, device=dev)
    sq = torch.empty((B, H, nb), dtype=torch.float32, device=dev)
    sk = torch.empty_like(sq)
    sv = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    def quant():
        fa.fa_fp8_quantize_qk(t["q"], q8, sq, signs, 1.0 / d, stream=stream)
        fa.fa_fp8_quantize_qk(t["k"], k8, sk, signs, 1.0, stream=stream)
        fa.fa_fp8_quantize_v(t["v"], v8t, sv, stream=stream)

    calls = {"quant": quant}
    for causal in (False, True):
        calls[causal] = (lambda c: lambda: fa.fa_forward_fp8(q8, sq, k8, sk, v8t, sv, o, lse, w.scale, c,
                                                              stream=stream))(causal)
    for fn in calls.values():
        for _ in range(3):
            fn()
    # the events exist before the timed calls (see run_gpu)
    ev = {key: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
          for key in calls}
    torch.cuda.synchronize()
    for i in range(iters):
        for key, fn in calls.items():
            e0, e1 = ev[key][i]
            e0.record(stream)
            fn()
            e1.record(stream)
    torch.cuda.synchronize()
    ms = {key: sum(a.elapsed_time(b) for a, b in v) / len(v) for key, v in ev.items()}
    out = {}
    for causal in (False, True):
        f = fwd_flops(B, H, N, d, causal)
        tf = f / (ms[causal] * 1e-3) / 1e12
        out[f"fwd_fp8_{'causal' if causal else 'full'}"] = {
            "ms": round(ms[causal], 4), "tflops": round(tf, 1), "pct_peak_fp8": round(100.0 * tf / PEAK_FP8_TFLOPS, 2),
            "pct_peak_bf16": round(100.0 * tf / PEAK_BF16_TFLOPS, 2), "quantize_ms": round(ms["quant"], 4)}
    return out


def run_machine(torch, dev, stream, reps=3):
    """Machine microbenchmarks (libfa355_micro.so, include/fa_micro.h), each launched
    `reps` times between HIP events on the bench stream; the median is reported.  They
    give what the chip sustains at its running clock: the bf16 MFMA rate, the v_exp_f32
    rate, LDS read bandwidth, fp32 atomic-add throughput, and how far an MFMA stream and
    a VALU stream of two waves on one SIMD overlap."""
    import ctypes

    from exact_io_aware_19_amd.build import MICRO_LIB_PATH

    if not os.path.exists(MICRO_LIB_PATH):
        raise RuntimeError(f"{MICRO_LIB_PATH} is missing: build it with `python -m exact_io_aware_19_amd.build`")
    lib = ctypes.CDLL(MICRO_LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    for name in ("fa_micro_mfma_bf16", "fa_micro_exp", "fa_micro_lds_read"):
        getattr(lib, name).argtypes = [vp, i, i, vp]
        getattr(lib, name).restype = i
    lib.fa_micro_atomic_tiles.argtypes = [vp, i, i, i, vp]
    lib.fa_micro_atomic_tiles.restype = i
    lib.fa_micro_grid_blocks.restype = i
    blocks = lib.fa_micro_grid_blocks()
    if blocks < 1:
        raise RuntimeError("fa_micro_grid_blocks failed")
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    ntiles, tiles = 4096, 64
    buf = torch.zeros(ntiles * 64 * 128, dtype=torch.float32, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    iters = {"mfma": 20000, "exp": 50000, "lds": 20000}
    # (call, units of work per call, scale to the reported unit)
    cases = {
        "mfma_bf16_tflops": (lambda: lib.fa_micro_mfma_bf16(out.data_ptr(), blocks, iters["mfma"], sp),
                             blocks * 4 * 8 * iters["mfma"] * 32768, 1e-12),
        "exp2_gops": (lambda: lib.fa_micro_exp(out.data_ptr(), blocks, iters["exp"], sp),
                      blocks * 256 * 16 * iters["exp"], 1e-9),
        "lds_read_tbs": (lambda: lib.fa_micro_lds_read(out.data_ptr(), blocks, iters["lds"], sp),
                         blocks * 4 * 8 * iters["lds"] * 1024, 1e-12),
        "atomic_f32_gbs": (lambda: lib.fa_micro_atomic_tiles(buf.data_ptr(), ntiles, blocks, tiles, sp),
                           blocks * tiles * 64 * 128 * 4, 1e-9),
    }
    res = {}
    for key, (call, work, unit) in cases.items():
        if call() != 0:  # warm-up launch, also checks the arguments
            raise RuntimeError(f"{key}: launch failed")
        evs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)[len(evs) // 2]
        res[key] = round(work / (ms * 1e-3) * unit, 1)
    res["mfma_bf16_pct_of_peak"] = round(100.0 * res["mfma_bf16_tflops"] / PEAK_BF16_TFLOPS, 1)
    # MFMA and VALU streams of two waves on one SIMD (one 8-wave workgroup per CU): alone,
    # then together; overlap = (mfma + valu - both) / min(mfma, valu), 1 = the shorter
    # stream hidden entirely, 0 = the two serialised
    lib.fa_micro_coexec.argtypes = [vp, i, i, i, i, i, vp]
    lib.fa_micro_coexec.restype = i
    cblocks = blocks // 2
    cout = torch.empty(cblocks * 512, dtype=torch.float32, device=dev)
    for kind, vk, v_iters in (("exp", 0, 30000), ("fma", 1, 80000)):
        ms = {}
        for mode, key in ((1, "mfma_ms"), (2, "valu_ms"), (3, "both_ms")):
            def call():
                return lib.fa_micro_coexec(cout.data_ptr(), cblocks, mode, vk, iters["mfma"], v_iters, sp)
            if call() != 0:
                raise RuntimeError(f"coexec {kind} mode {mode}: launch failed")
            evs = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                call()
                e1.record(stream)
                evs.append((e0, e1))
            torch.cuda.synchronize()
            ms[key] = round(sorted(a.elapsed_time(b) for a, b in evs)[len(evs) // 2], 4)
        ms["overlap"] = round((ms["mfma_ms"] + ms["valu_ms"] - ms["both_ms"]) / min(ms["mfma_ms"], ms["valu_ms"]), 3)
        res[f"coexec_mfma_{kind}"] = ms
    # v_exp_f32 chains beside v_fma_f32 chains: on two waves of one SIMD (kind 2) and
    # interleaved in one wave (kind 3); exp_ms / fma_ms alone, both_ms together
    for name, vk in (("coexec_exp_fma_two_waves", 2), ("coexec_exp_fma_one_wave", 3)):
        ms = {}
        for mode, key in ((1, "exp_ms"), (2, "fma_ms"), (3, "both_ms")):
            def call():
                return lib.fa_micro_coexec(cout.data_ptr(), cblocks, mode, vk, 30000, 60000, sp)
            if call() != 0:
                raise RuntimeError(f"coexec {name} mode {mode}: launch failed")
            evs = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                call()
                e1.record(stream)
                evs.append((e0, e1))
            torch.cuda.synchronize()
            ms[key] = round(sorted(a.elapsed_time(b) for a, b in evs)[len(evs) // 2], 4)
        ms["overlap"] = round((ms["exp_ms"] + ms["fma_ms"] - ms["both_ms"]) / min(ms["exp_ms"], ms["fma_ms"]), 3)
        res[name] = ms
    # shader-clock cycles per 32 products in the attention forward's order against 8
    # independent chains (32 x 32 = 1024 at best), one wave per SIMD on every CU
    lib.fa_micro_mfma_order.argtypes = [vp, vp, i, i, i, vp]
    lib.fa_micro_mfma_order.restype = i
    oblocks, oiters = blocks // 2, 2000
    ticks = torch.zeros(oblocks * 4, dtype=torch.int64, device=dev)
    order = {}
    for variant, key in ((0, "independent_chains"), (1, "forward_order"), (2, "forward_order_scores_4_chains"),
                         (3, "forward_order_lds_operands")):
        if lib.fa_micro_mfma_order(ticks.data_ptr(), out.data_ptr(), oblocks, variant, oiters, sp) != 0:
            raise RuntimeError(f"mfma order variant {variant}: launch failed")
        torch.cuda.synchronize()
        order[key] = round(float(ticks.double().median().item()) / oiters, 1)
    res["mfma_order_cycles_per_32_products"] = order
    return res


def run_env():
    """Device and software the numbers were taken on."""
    import torch

    prop = torch.cuda.get_device_properties(0)
    return {"device": prop.name, "arch": getattr(prop, "gcnArchName", None), "compute_units": prop.multi_processor_count,
            "hbm_gib": round(prop.total_memory / 2**30, 1), "torch": torch.__version__, "hip_runtime": torch.version.hip}


def _lib_handle():
    from exact_io_aware_19_amd import _lib

    return _lib.load()


COLD_WORKLOADS = ("tiny", "bert_large", "gpt2", "sweep_n2048_full", "sweep_n2048_causal")


def run_sweep(fa, wl, torch, dev, stream, iters=10):
    out = []
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev).view(torch.float32)
    for name in ["tiny", "bert_large", "gpt2"] + [f"sweep_n{n}_{m}" for n in (2048, 4096, 8192, 16384)
                                                   for m in ("full", "causal")] + ["long_64k", "gqa_n8192",
                                                                                   "mqa_n4096"]:
        w = wl.get_workload(name)
        inp = wl.generate(w)
        t = inp.to_torch(dev)
        B, H, N, d = w.shape
        o = torch.empty_like(t["q"])
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        res = {"workload": name}
        grouped = w.kv_heads != w.H
        if grouped:
            res["h_kv"] = w.kv_heads
        for direction in (("fwd", "bwd") if w.backward else ("fwd",)):
            # each call is validated once through the binding, then timed as a direct C-ABI
            # call with prepared arguments: for the small workloads the binding's checks
            # take longer on the host than the kernels take on the GPU
            lib = _lib_handle()
            kvp = None if t["kv_len"] is None else t["kv_len"].data_ptr()
            sp = stream.cuda_stream
            if direction == "fwd":
                fwd = fa.fa_forward_gqa if grouped else fa.fa_forward
                fwd(t["q"], t["k"], t["v"], o, lse, w.scale, w.causal, kv_len=t["kv_len"], stream=stream)
                args = (t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                        w.kv_heads, N, d, w.scale, int(w.causal), kvp, sp)

                def call():
                    lib.fa_forward_gqa(*args)
            else:
                dq = torch.empty_like(t["q"])
                dk, dv = torch.empty_like(t["k"]), torch.empty_like(t["v"])
                ws = torch.empty(fa.fa_backward_gqa_workspace_size(B, H, w.kv_heads, N, d), dtype=torch.uint8,
                                 device=dev)
                bwd = fa.fa_backward_gqa if grouped else fa.fa_backward
                bwd(t["q"], t["k"], t["v"], o, t["do"], lse, dq, dk, dv, w.scale, w.causal, ws,
                    kv_len=t["kv_len"], stream=stream)
                args = (t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(), t["do"].data_ptr(),
                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, w.kv_heads, N, d, w.scale,
                        int(w.causal), kvp, ws.data_ptr(), ws.numel(), sp)

                def call():
                    lib.fa_backward_gqa(*args)
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            # at least `iters` calls and about 30 ms of timed work per entry
            t0 = time.perf_counter()
            call()
            torch.cuda.synchronize()
            n_it = max(iters, int(0.03 / max(time.perf_counter() - t0, 1e-6)))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n_it):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n_it
            f = w.fwd_flops() * (1.0 if direction == "fwd" else 2.5)
            tf = f / (ms * 1e-3) / 1e12
            res[direction] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                              "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                              "alg_gbs": round(_alg_bytes(B, H, N, d, direction, w.kv_heads) / (ms * 1e-3) / 1e9, 1)}
            if name in COLD_WORKLOADS:
                # cold caches: before each timed call, overwrite a buffer twice the size of
                # the 256 MB MALL (and so every L2); the median of single-call event times
                cold = []
                for _ in range(11):
                    flush.fill_(1.0)
                    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    c0.record(stream)
                    call()
                    c1.record(stream)
                    torch.cuda.synchronize()
                    cold.append(c0.elapsed_time(c1))
                cms = sorted(cold)[len(cold) // 2]
                res[direction]["cold_ms"] = round(cms, 4)
                res[direction]["cold_alg_gbs"] = round(
                    _alg_bytes(B, H, N, d, direction, w.kv_heads) / (cms * 1e-3) / 1e9, 1)
        if name in ("tiny", "bert_large", "gpt2"):
            res["step"] = time_step_graph(lib, torch, dev, t, w)
        if name == "long_64k":
            res["query_shards"] = time_query_shards(lib, torch, stream, t, w)
        if name.startswith("sweep_n") or name == "long_64k":
            # the FP8 forward on the same inputs (block quantisation + incoherent processing)
            res["fwd_fp8"] = {k: v for k, v in run_fp8(fa, wl, torch, dev, stream, t, w, iters)[
                f"fwd_fp8_{'causal' if w.causal else 'full'}"].items()}
        print(json.dumps({"sweep": res}), file=sys.stderr, flush=True)
        out.append(res)
        del t, o, lse
        torch.cuda.empty_cache()
    return out


def time_query_shards(lib, torch, stream, t, w, gpus=8, iters=5):
    """One GPU's share of the causal forward split by query rows over `gpus` GPUs that each
    hold all keys and values (fa_forward_offset; the all-gather of K and V is not part of
    it): contiguous shares of N/gpus rows, and the zig-zag assignment (2*gpus pieces, GPU g
    takes pieces g and 2*gpus-1-g, which balances the causal work).  Returns each GPU's
    time, the slowest one, and the whole problem's FLOPs over that time (the rate the
    GPUs would reach together if the exchange hides behind the compute)."""
    B, H, N, d = w.shape
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=t["q"].device)
    sp = stream.cuda_stream

    def piece_ms(r0, r1):
        q = t["q"][:, :, r0:r1].contiguous()
        args = (q.data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, r1 - r0, N,
                d, w.scale, int(w.causal), r0, None, sp)
        st = lib.fa_forward_offset(*args)
        if st != 0:
            raise RuntimeError(f"fa_forward_offset returned {st}")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            lib.fa_forward_offset(*args)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    n = N // gpus
    contiguous = [piece_ms(g * n, (g + 1) * n) for g in range(gpus)]
    h = n // 2
    pieces = [piece_ms(p * h, (p + 1) * h) for p in range(2 * gpus)]
    zigzag = [pieces[g] + pieces[2 * gpus - 1 - g] for g in range(gpus)]
    out = {"gpus": gpus, "rows_per_gpu": n}
    for name, per in (("contiguous", contiguous), ("zigzag", zigzag)):
        worst = max(per)
        out[name] = {"per_gpu_ms": [round(x, 4) for x in per], "max_ms": round(worst, 4),
                     "tflops_all_gpus": round(w.fwd_flops() / (worst * 1e-3) / 1e12, 1)}
    return out


def time_step_graph(lib, torch, dev, t, w, min_iters=20):
    """One forward + backward step of a small workload, timed as back-to-back direct C-ABI
    calls and as replays of a HIP graph that captured the same calls (the host cost of
    launching is what differs at these sizes).  Both on one side stream with HIP events;
    ms per step."""
    B, H, N, d = w.shape
    gs = torch.cuda.Stream(device=dev)
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    ws = torch.empty(lib.fa_backward_gqa_workspace_size(B, H, w.kv_heads, N, d), dtype=torch.uint8, device=dev)
    kvp = None if t["kv_len"] is None else t["kv_len"].data_ptr()
    sp = gs.cuda_stream
    fargs = (t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
             w.kv_heads, N, d, w.scale, int(w.causal), kvp, sp)
    bargs = (t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(), t["do"].data_ptr(),
             lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, w.kv_heads, N, d, w.scale,
             int(w.causal), kvp, ws.data_ptr(), ws.numel(), sp)

    def step():
        if lib.fa_forward_gqa(*fargs) != 0 or lib.fa_backward_gqa(*bargs) != 0:
            raise RuntimeError("step launch failed")

    gs.wait_stream(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        step()
    torch.cuda.synchronize()
    out = {}
    for kind in ("eager", "graph"):
        run = step if kind == "eager" else g.replay
        with torch.cuda.stream(gs):
            for _ in range(3):
                run()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run()
            torch.cuda.synchronize()
            n_it = max(min_iters, int(0.03 / max(time.perf_counter() - t0, 1e-6)))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(gs)
            for _ in range(n_it):
                run()
            e1.record(gs)
            torch.cuda.synchronize()
        out[f"{kind}_ms"] = round(e0.elapsed_time(e1) / n_it, 4)
    del g
    return out


def _oracle_task_init():
    """Worker initialiser of the CPU baseline: BLAS on one thread per worker process."""
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:  # threadpoolctl missing: OPENBLAS_NUM_THREADS=1 was set before spawning
        pass


def _oracle_task(task):
    """One task of the CPU baseline: the fp64 oracle's forward, then backward, of one head
    under one mask mode.  Returns (forward seconds, backward seconds)."""
    q_bits, k_bits, v_bits, do_bits, scale, causal = task
    from oracle import ref
    from exact_io_aware_19_amd import workloads as wl

    qh, kh, vh, doh = (wl.bf16_bits_to_f64(x)[None, None] for x in (q_bits, k_bits, v_bits, do_bits))
    t0 = time.perf_counter()
    ref.attention_forward(qh, kh, vh, scale, causal=causal)
    t1 = time.perf_counter()
    ref.attention_backward(qh, kh, vh, doh, scale, causal=causal)
    return t1 - t0, time.perf_counter() - t1


def cpu_worker_count():
    """One worker per host core this process may run on, at most 16 (the host share of one
    GPU on the machines the bench runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(inp, shape, heads):
    """The fp64 oracle as it stands, on `heads` (b, h) heads of the bench workload, both
    mask modes, forward + backward, on a process pool of one single-threaded-BLAS worker
    per host core; FLOPs counted with the same convention as the GPU line.  Must run
    before this process touches the GPU: the workers are spawned (fresh interpreters)."""
    import concurrent.futures
    import multiprocessing

    B, H, N, d = shape
    scale = 1.0 / math.sqrt(d)
    workers = cpu_worker_count()
    tasks = [(inp.q[b, h], inp.k[b, h], inp.v[b, h], inp.do[b, h], scale, causal)
             for b, h in heads for causal in (False, True)]
    flops = sum(3.5 * fwd_flops(1, 1, N, d, t[5]) for t in tasks)
    saved = {k: os.environ.get(k) for k in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS")}
    os.environ.update({k: "1" for k in saved})
    try:
        ctx = multiprocessing.get_context("spawn")
        with concurrent.futures.ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                                                    initializer=_oracle_task_init) as pool:
            # start every worker and import the oracle before the clock starts
            tiny = (inp.q[0, 0, :8], inp.k[0, 0, :8], inp.v[0, 0, :8], inp.do[0, 0, :8], scale, False)
            list(pool.map(_oracle_task, [tiny] * workers))
            t0 = time.perf_counter()
            res = list(pool.map(_oracle_task, tasks))
            wall = time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    t_fwd = sum(r[0] for r in res)
    t_bwd = sum(r[1] for r in res)
    blas = None
    try:
        from threadpoolctl import threadpool_info

        blas = ",".join(sorted({str(i.get("internal_api")) for i in threadpool_info() if i.get("user_api") == "blas"}))
    except Exception:
        pass
    full_tasks = 2 * B * H  # every head, both mask modes: the whole step
    return {
        "value": round(flops / wall / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{len(heads)} of {B * H} heads of (B={B},H={H},N={N},d={d}), no mask and causal, forward+backward "
                  f"in numpy fp64; {len(tasks)} tasks on {workers} single-threaded-BLAS worker processes; "
                  f"{wall:.1f} s wall",
        "seconds": round(wall, 2),
        "worker_forward_seconds": round(t_fwd, 2),
        "worker_backward_seconds": round(t_bwd, 2),
        "full_step_seconds_extrapolated": round(wall * full_tasks / len(tasks), 1),
        "host_cpus": os.cpu_count(),
        "blas": blas or None,
    }


def summarize_pmc(fetch_csv, write_csv, out_md, by_grid=False):
    """HBM bytes per launch of every kernel of the bench step from two rocprofv3 --pmc
    runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the last ten plain copies (bench.py --copy-calibration), whose
    bytes are known.  by_grid: one row per kernel and grid size (workgroups), for runs
    that launch one kernel on several workload shapes (--sweep)."""

    def load(path, counter):
        rows = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    name = r["Kernel_Name"]
                    if by_grid and "fa355" in name:
                        wg = max(1, int(r["Workgroup_Size"]))
                        bare = name.replace("void ", "", 1).replace("fa355::(anonymous namespace)::", "").split("(")[0]
                        name = "fa355::(anonymous namespace)::%s grid=%d" % (bare, int(r["Grid_Size"]) // wg)
                    rows.append((int(r["Dispatch_Id"]), name, float(r["Counter_Value"])))
        return sorted(rows)

    out = {}
    cal = {}
    kib = COPY_CAL_MIB * 1024  # KiB each calibration copy reads and writes
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = load(path, counter)
        copies = [v for _, name, v in rows if "copyBuffer" in name][-10:]
        if len(copies) < 10:
            raise SystemExit(f"{path}: fewer than 10 copy dispatches (run bench.py with --copy-calibration)")
        cal[counter] = sum(copies) / len(copies)  # KiB per copy
        per = {}
        for _, name, v in rows:
            if "fa355" in name:
                key = name.replace("void ", "", 1) if name.startswith("void ") else name
                key = key.replace("fa355::(anonymous namespace)::", "").replace("fa355::", "").split("(")[0]
                if key.startswith(("fa_", "fp8_")):  # attention kernels, not the machine microbenchmarks
                    per.setdefault(key, []).append(v)
        out[counter] = {kname: sum(vs) / len(vs) for kname, vs in per.items()}
    m = re.search(r"--copy-calibration (\d+)", " ".join(sys.argv))
    sweep = " --sweep --no-machine" if by_grid else ""
    fdir = os.path.relpath(os.path.dirname(os.path.abspath(fetch_csv)), ROOT)
    wdir = os.path.relpath(os.path.dirname(os.path.abspath(write_csv)), ROOT)
    lines = [
        "# HBM traffic per launch, attention fwd/bwd, "
        + ("every workload of the sweep (one row per kernel and grid)" if by_grid else "B=2 H=16 N=8192 d=128"),
        "",
        "Commands (each on one MI355X, from the repository root, one counter per run):",
        "",
        "    rocprofv3 --pmc FETCH_SIZE -f csv -d %s -o p -- python bench.py --steps 2 --warmup 1 --cpu-heads 0 --copy-calibration%s" % (fdir, sweep),
        "    rocprofv3 --pmc WRITE_SIZE -f csv -d %s -o p -- python bench.py --steps 2 --warmup 1 --cpu-heads 0 --copy-calibration%s" % (wdir, sweep),
        "    python bench.py%s --summarize-pmc %s %s %s"
        % (" --pmc-by-grid" if by_grid else "", os.path.relpath(os.path.abspath(fetch_csv), ROOT),
           os.path.relpath(os.path.abspath(write_csv), ROOT), os.path.relpath(out_md, ROOT)),
        "",
        "Calibration: the last ten dispatches of the plain %d MiB device copy read and write" % COPY_CAL_MIB,
        "%d bytes each; the counters read %.0f KiB (FETCH_SIZE) and %.0f KiB (WRITE_SIZE)," % (COPY_CAL_MIB << 20, cal["FETCH_SIZE"], cal["WRITE_SIZE"]),
        "so bytes = counter KiB x %.4f x 1024 (fetch) and x %.4f x 1024 (write)." % (kib / cal["FETCH_SIZE"], kib / cal["WRITE_SIZE"]),
        "",
        "kernel_source_sha: " + kernel_source_hash(),
        "",
        "| kernel | HBM bytes per launch | fetch bytes | write bytes |",
        "|---|---|---|---|",
    ]
    for kname in sorted(out["FETCH_SIZE"]):
        fb = out["FETCH_SIZE"][kname] * 1024 * kib / cal["FETCH_SIZE"]
        wb = out["WRITE_SIZE"].get(kname, 0.0) * 1024 * kib / cal["WRITE_SIZE"]
        shown = kname.replace("void ", "", 1).replace("fa355::(anonymous namespace)::", "")
        lines.append("| %s | %.0f | %.0f | %.0f |" % (shown, fb + wb, fb, wb))
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30, help="timed steps (default 30: about 200 ms of timed work)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--n", type=int, default=8192, help="sequence length of the bench workload (default 8192)")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="heads in the oracle CPU-baseline sample, each under both masks (0 = skip)")
    ap.add_argument("--sweep", action="store_true", help="also time every workload of the sweep (stderr)")
    ap.add_argument("--no-fp8", dest="fp8", action="store_false",
                    help="skip the FP8 forward (timed after the bf16 step, reported under detail)")
    ap.add_argument("--fp8-iters", type=int, default=20, help="timed iterations of the FP8 forward (default 20)")
    ap.add_argument("--clock-steps", type=int, default=20,
                    help="untimed steps after the timed ones during which the gfx clock and board power are sampled "
                         "(default 20; only when --steps >= 10; 0: none)")
    ap.add_argument("--no-machine", dest="machine", action="store_false",
                    help="skip the machine microbenchmarks (sustained MFMA, exp, LDS, atomic rates)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run 10 plain device copies of {COPY_CAL_MIB} MiB (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--pmc-by-grid", action="store_true",
                    help="with --summarize-pmc: one row per kernel and grid size (for --sweep runs)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc counter CSVs and exit")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, by_grid=args.pmc_by_grid)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    # the CPU baseline first: its worker processes are spawned before this process
    # initialises the GPU
    cpu = None
    if args.cpu_heads > 0:
        import numpy as np

        from exact_io_aware_19_amd import workloads as wl

        inp = wl.generate(bench_workload(args.n), with_do=True)
        rng = np.random.default_rng(12345)
        B, H = inp.q.shape[:2]
        heads = [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(args.cpu_heads)]
        cpu = cpu_baseline(inp, inp.q.shape, heads)
        del inp
    value, wall, detail, roofline, shape, inp, _ = run_gpu(args)
    B, H, N, d = shape
    if args.machine:
        import torch

        detail["machine"] = m = run_machine(torch, torch.device("cuda:0"), torch.cuda.current_stream())
        # the dominant kernel against the MFMA rate the chip sustains, beside the data-sheet peak
        roofline["frac_of_sustained_mfma"] = round(roofline["achieved"] / m["mfma_bf16_tflops"], 4)
    if args.copy_calibration:  # last: no copy may follow the calibration copies
        import torch

        roofline["copy_calibration"] = copy_calibration(torch)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) fp32 rounded to bf16",
        "value_basis": "FLOPs of the timed steps / wall time of the timed region (mean over the steps); "
                       "detail.step_kernels_ms_median is the median step",
        "config": {"workload": f"large-head attention fwd+bwd, no mask and causal", "B": B, "H": H, "N": N, "d": d,
                   "scale": round(1.0 / math.sqrt(d), 8), "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2)},
        "detail": detail,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "env": run_env(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
