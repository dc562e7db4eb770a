"""CPU tests of the bench's host logic: the FLOP and byte conventions, the HBM-traffic
summary built from rocprofv3 counter CSVs (calibration by the plain copies, per-kernel and
per-grid rows), the staleness check of the committed traffic figure, the refusal of more
than one GPU, and the clock/power sampler's parsing of sysfs."""

import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_flop_convention():
    # forward 4 B H N^2 d, halved when causal; the backward is 2.5x that (applied by callers)
    assert bench.fwd_flops(2, 16, 8192, 128, False) == 4.0 * 2 * 16 * 8192**2 * 128
    assert bench.fwd_flops(2, 16, 8192, 128, True) == 2.0 * 2 * 16 * 8192**2 * 128
    assert bench.KERNEL_FLOP_SHARE["dq"] + bench.KERNEL_FLOP_SHARE["dkdv"] == 2.5


def test_algorithmic_bytes():
    B, H, N, d = 2, 3, 100, 64
    rows = B * H * N
    # forward: Q, K, V read and O written in bf16, LSE fp32
    assert bench._alg_bytes(B, H, N, d, "fwd") == 4 * rows * d * 2 + 4 * rows
    # backward: Q, K, V, O, dO read and dQ, dK, dV written in bf16; LSE read; D written, read
    assert bench._alg_bytes(B, H, N, d, "bwd") == 8 * rows * d * 2 + 12 * rows
    # grouped K/V heads: K, V (and dK, dV) count the K/V heads only
    kv_rows = B * 1 * N
    assert bench._alg_bytes(B, H, N, d, "fwd", hkv=1) == 2 * rows * d * 2 + 2 * kv_rows * d * 2 + 4 * rows


def _write_counters(path, counter, rows):
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i, (name, grid, wg, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid, "Workgroup_Size": wg,
                        "Counter_Name": counter, "Counter_Value": value})


KERN_A = "void fa355::(anonymous namespace)::fa_fwd_kernel<128, 64, false, false>(fa355::FwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _table(md):
    with open(md) as f:
        return {line.split("|")[1].strip(): [float(x) for x in line.split("|")[2:5]]
                for line in f if line.startswith("| ") and not line.startswith("| kernel") and "---" not in line}


def test_summarize_pmc_calibrates_with_the_last_ten_copies(tmp_path):
    cal_kib = bench.COPY_CAL_MIB * 1024
    # an early copy with a different reading must be ignored; the last ten read half the
    # bytes on FETCH_SIZE (factor 2) and all of them on WRITE_SIZE (factor 1)
    fetch = [(COPY, 1, 1, 1.0), (KERN_A, 1024 * 512, 512, 1000.0), (KERN_A, 1024 * 512, 512, 3000.0)]
    fetch += [(COPY, 1, 1, cal_kib / 2)] * 10
    write = [(COPY, 1, 1, 5.0), (KERN_A, 1024 * 512, 512, 100.0), (KERN_A, 1024 * 512, 512, 300.0)]
    write += [(COPY, 1, 1, cal_kib)] * 10
    fcsv, wcsv, md = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.md"
    _write_counters(fcsv, "FETCH_SIZE", fetch)
    _write_counters(wcsv, "WRITE_SIZE", write)
    assert bench.summarize_pmc(str(fcsv), str(wcsv), str(md)) == 0
    rows = _table(md)
    total, fb, wb = rows["fa_fwd_kernel<128, 64, false, false>"]
    # mean of the kernel's two dispatches (2000 KiB fetch, 200 KiB write), scaled by the
    # calibration
    assert fb == pytest.approx(2000 * 1024 * 2)
    assert wb == pytest.approx(200 * 1024)
    assert total == pytest.approx(fb + wb)
    assert "kernel_source_sha: " + bench.kernel_source_hash() in md.read_text()


def test_summarize_pmc_by_grid_keeps_shapes_apart(tmp_path):
    cal_kib = bench.COPY_CAL_MIB * 1024
    fetch = [(KERN_A, 256 * 512, 512, 10.0), (KERN_A, 1024 * 512, 512, 40.0)] + [(COPY, 1, 1, cal_kib)] * 10
    write = [(KERN_A, 256 * 512, 512, 1.0), (KERN_A, 1024 * 512, 512, 4.0)] + [(COPY, 1, 1, cal_kib)] * 10
    fcsv, wcsv, md = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.md"
    _write_counters(fcsv, "FETCH_SIZE", fetch)
    _write_counters(wcsv, "WRITE_SIZE", write)
    assert bench.summarize_pmc(str(fcsv), str(wcsv), str(md), by_grid=True) == 0
    rows = _table(md)
    assert rows["fa_fwd_kernel<128, 64, false, false> grid=256"][1] == pytest.approx(10 * 1024)
    assert rows["fa_fwd_kernel<128, 64, false, false> grid=1024"][1] == pytest.approx(40 * 1024)


def test_summarize_pmc_needs_the_calibration_copies(tmp_path):
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counters(fcsv, "FETCH_SIZE", [(KERN_A, 512, 512, 1.0)])
    _write_counters(wcsv, "WRITE_SIZE", [(KERN_A, 512, 512, 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(fcsv), str(wcsv), str(tmp_path / "t.md"))


def test_traffic_figure_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    md = tmp_path / "t.md"
    md.write_text("kernel_source_sha: %s\n\n| k<1> | 123 | 100 | 23 |\n" % bench.kernel_source_hash())
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(md))
    assert bench.read_traffic("k<1>") == 123.0
    assert bench.read_traffic("other") is None
    md.write_text("kernel_source_sha: 0000000000000000\n\n| k<1> | 123 | 100 | 23 |\n")
    assert bench.read_traffic("k<1>") is None


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_cpu_baseline_runs_a_spawned_single_threaded_pool():
    """The CPU baseline leg on a small sample: one spawned worker per host core (at most
    16), each with single-threaded BLAS, both mask modes per head; the line's fields."""
    import bench
    from exact_io_aware_19_amd import workloads as wl

    w = wl.Workload("small", 1, 2, 256, 64, False, 0.125, 77)
    inp = wl.generate(w, with_do=True)
    out = bench.cpu_baseline(inp, inp.q.shape, [(0, 0), (0, 1)])
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s" and out["value"] > 0
    assert out["cores"] == bench.cpu_worker_count() <= 16
    assert "4 tasks" in out["sample"]
    assert out["full_step_seconds_extrapolated"] == round(out["seconds"] * 4 / 4, 1)


def test_current_sclk_is_the_marked_line():
    # a live reading (as MI355X reports it) and a marked DPM level
    assert bench.parse_current_sclk_mhz("S: 1843Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == 1843
    assert bench.parse_current_sclk_mhz("0: 500Mhz\n1: 2100Mhz *\n2: 2400Mhz\n") == 2100
    assert bench.parse_current_sclk_mhz("0: 500Mhz\n1: 2400Mhz\n") is None


def test_clock_sampler_summarises_sysfs(tmp_path):
    dev = tmp_path / "device"
    (dev / "hwmon" / "hwmon3").mkdir(parents=True)
    (dev / "pp_dpm_sclk").write_text("S: 1790Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    (dev / "hwmon" / "hwmon3" / "power1_input").write_text("1375000000\n")
    (dev / "hwmon" / "hwmon3" / "power1_cap").write_text("1400000000\n")
    (dev / "hwmon" / "hwmon3" / "temp2_label").write_text("junction\n")
    (dev / "hwmon" / "hwmon3" / "temp2_input").write_text("81000\n")
    (dev / "hwmon" / "hwmon3" / "temp3_label").write_text("mem\n")
    (dev / "hwmon" / "hwmon3" / "temp3_input").write_text("60000\n")
    s = bench.ClockSampler(str(dev), period_s=0.001).start()
    import time

    time.sleep(0.05)
    out = s.stop()
    assert out["samples"] >= 1
    assert out["sclk_mhz_median"] == out["sclk_mhz_min"] == out["sclk_mhz_max"] == 1790
    assert out["power_w_median"] == 1375.0 and out["power_cap_w"] == 1400.0
    assert out["junction_c_median"] == out["junction_c_max"] == 81.0
    # no sysfs directory: no summary, and no thread started
    assert bench.ClockSampler(None).start().stop() is None
