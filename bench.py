#!/usr/bin/env python3
"""Throughput bench for the exact-attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
fa_forward + fa_backward with no mask, then fa_forward + fa_backward with the causal
mask, on the large-head workload (B=2, H=16, N=8192, d=128, bf16 ~ N(0,1), scale
1/sqrt(128); the N >= 4096, d = 128 regime the throughput target is quoted on).

FLOP convention: forward 4*B*H*N^2*d, halved when causal; backward 2.5x the forward.
`value` = total FLOPs of the K timed steps / their wall time (inputs resident in HBM).

Printed JSON line (rank 0 only):
  metric, value (TFLOP/s), unit, n_gpus, steps, warmup, ms_per_step, higher_is_better,
  scaling, vs_baseline, dtype, data, config, detail (per call: TFLOP/s, % of the bf16
  dense peak), roofline (dominant launch, HIP events on the launch stream) and
  cpu_baseline (the fp64 oracle on a bounded sample, host cores of this machine).

Options: --sweep prints one extra line per workload of the sweep to stderr.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s (bf16, causal & non) + % of MI355X bf16 MFMA peak"


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def _alg_bytes(B, H, N, d, direction):
    """Algorithmic HBM bytes of one call: fwd reads Q,K,V and writes O (bf16) + LSE (fp32);
    bwd reads Q,K,V,O,dO (bf16) + LSE, writes dQ,dK,dV (bf16), writes and reads D (fp32)."""
    rows = B * H * N
    if direction == "fwd":
        return 8.0 * rows * d + 4.0 * rows
    return 16.0 * rows * d + 12.0 * rows


def run_gpu(args):
    import torch
    import exact_io_aware_19_amd as fa
    from exact_io_aware_19_amd import workloads as wl

    dev = torch.device("cuda:0")
    B, H, N, d = 2, 16, args.n, 128
    scale = 1.0 / math.sqrt(d)
    w = wl.Workload(f"sweep_n{N}", B, H, N, d, False, scale, 1040 + int(math.log2(N)))
    inp = wl.generate(w, with_do=True)
    t = inp.to_torch(dev)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = {m: torch.empty_like(q) for m in (False, True)}
    lse = {m: torch.empty((B, H, N), dtype=torch.float32, device=dev) for m in (False, True)}
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_backward_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    calls = [("fwd", False), ("bwd", False), ("fwd", True), ("bwd", True)]
    ev = {c: [] for c in calls}

    def step(record):
        for c in calls:
            direction, causal = c
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            if direction == "fwd":
                fa.fa_forward(q, k, v, o[causal], lse[causal], scale, causal, stream=stream)
            else:
                fa.fa_backward(q, k, v, o[causal], do, lse[causal], dq, dk, dv, scale, causal, ws, stream=stream)
            if record:
                e1.record(stream)
                ev[c].append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    step_flops = 0.0
    detail = {}
    for c in calls:
        direction, causal = c
        f = fwd_flops(B, H, N, d, causal) * (1.0 if direction == "fwd" else 2.5)
        step_flops += f
        ms = sum(a.elapsed_time(b) for a, b in ev[c]) / len(ev[c])
        tf = f / (ms * 1e-3) / 1e12
        detail[f"{direction}_{'causal' if causal else 'full'}"] = {
            "ms": round(ms, 4),
            "tflops": round(tf, 1),
            "pct_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
            "alg_gbs": round(_alg_bytes(B, H, N, d, direction) / (ms * 1e-3) / 1e9, 1),
        }
    value = step_flops * args.steps / wall / 1e12
    # dominant launch = the call with the largest share of the step time
    dom = max(detail, key=lambda kname: detail[kname]["ms"])
    dd = detail[dom]
    roofline = {
        "bound": "mfma",
        "achieved": dd["tflops"],
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(dd["tflops"] / PEAK_BF16_TFLOPS, 4),
        "traffic": None,
        "launch": dom,
        "launch_kernels": (["fa_fwd_kernel"] if dom.startswith("fwd") else ["fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel"]),
    }
    sweep = []
    if args.sweep:
        sweep = run_sweep(fa, wl, torch, dev, stream)
    return value, wall, detail, roofline, (B, H, N, d), inp, sweep


def run_sweep(fa, wl, torch, dev, stream, iters=10):
    out = []
    for name in ["tiny", "bert_large", "gpt2"] + [f"sweep_n{n}_{m}" for n in (2048, 4096, 8192, 16384)
                                                   for m in ("full", "causal")] + ["long_64k"]:
        w = wl.get_workload(name)
        inp = wl.generate(w)
        t = inp.to_torch(dev)
        B, H, N, d = w.shape
        o = torch.empty_like(t["q"])
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        res = {"workload": name}
        for direction in (("fwd", "bwd") if w.backward else ("fwd",)):
            if direction == "fwd":
                def call():
                    fa.fa_forward(t["q"], t["k"], t["v"], o, lse, w.scale, w.causal, kv_len=t["kv_len"], stream=stream)
            else:
                dq, dk, dv = (torch.empty_like(t["q"]) for _ in range(3))
                ws = torch.empty(fa.fa_backward_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev)

                def call():
                    fa.fa_backward(t["q"], t["k"], t["v"], o, t["do"], lse, dq, dk, dv, w.scale, w.causal, ws,
                                   kv_len=t["kv_len"], stream=stream)
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(iters):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / iters
            f = w.fwd_flops() * (1.0 if direction == "fwd" else 2.5)
            tf = f / (ms * 1e-3) / 1e12
            res[direction] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                              "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                              "alg_gbs": round(_alg_bytes(B, H, N, d, direction) / (ms * 1e-3) / 1e9, 1)}
        print(json.dumps({"sweep": res}), file=sys.stderr, flush=True)
        out.append(res)
        del t, o, lse
        torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, shape, heads):
    """The fp64 oracle as it stands, on `heads` (b, h) heads of the bench workload, both
    mask modes, forward + backward; FLOPs counted with the same convention."""
    from oracle import ref
    from exact_io_aware_19_amd import workloads as wl

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default is one thread per core
        threads = os.cpu_count() or 1
    B, H, N, d = shape
    scale = 1.0 / math.sqrt(d)
    flops = 0.0
    t0 = time.perf_counter()
    for b, h in heads:
        qh, kh, vh, doh = (wl.bf16_bits_to_f64(getattr(inp, n)[b, h])[None, None] for n in ("q", "k", "v", "do"))
        for causal in (False, True):
            ref.attention_forward(qh, kh, vh, scale, causal=causal)
            ref.attention_backward(qh, kh, vh, doh, scale, causal=causal)
            flops += 3.5 * fwd_flops(1, 1, N, d, causal)
    sec = time.perf_counter() - t0
    return {
        "value": round(flops / sec / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(heads)} of {B * H} heads of (B={B},H={H},N={N},d={d}), no mask and causal, "
                  f"forward+backward in numpy fp64; {sec:.1f} s",
        "seconds": round(sec, 2),
        "host_cpus": os.cpu_count(),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--n", type=int, default=8192, help="sequence length of the bench workload (default 8192)")
    ap.add_argument("--cpu-heads", type=int, default=3, help="heads in the oracle CPU-baseline sample (0 = skip)")
    ap.add_argument("--sweep", action="store_true", help="also time every workload of the sweep (stderr)")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    value, wall, detail, roofline, shape, inp, _ = run_gpu(args)
    B, H, N, d = shape
    cpu = None
    if args.cpu_heads > 0:
        import numpy as np

        rng = np.random.default_rng(12345)
        heads = [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(args.cpu_heads)]
        cpu = cpu_baseline(inp, shape, heads)
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
        "config": {"workload": f"large-head attention fwd+bwd, no mask and causal", "B": B, "H": H, "N": N, "d": d,
                   "scale": round(1.0 / math.sqrt(d), 8), "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2)},
        "detail": detail,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
