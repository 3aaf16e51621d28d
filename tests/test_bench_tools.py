"""CPU checks of bench.py's own arithmetic and summaries: the algorithmic bytes and FLOPs against the
figures the configurations are quoted with, the cold-cache rotation, the rocprofv3 summaries on small
CSV fixtures written here, and the source-hash key of the committed traffic records."""
import argparse
import csv
import json
import math

import pytest

import bench


def test_algorithmic_bytes_and_flops_of_the_configurations():
    # A bf16 read once + B codes + B scale bytes + C bf16 written once; the quantised A is not counted.
    assert bench.alg_bytes(4, 256, 512) == 75_776
    assert bench.alg_bytes(16, 2112, 7168) == 8_339_456
    assert bench.alg_bytes(64, 7168, 2048) == 8_978_432
    assert bench.alg_bytes(4096, 4096, 7168) == 107_872_256
    assert bench.alg_bytes(256, 4096, 7168) == 3_670_016 + 14_680_064 + 917_504 + 2_097_152  # mid: A, B, scales, C
    assert bench.alg_flops(4096, 4096, 7168) == 240_518_168_576
    # Grouped (N 4096, K 7168): 124 780 544 B for the eight B matrices plus 22 528 B per row of A and C.
    Ms = [448, 384, 704, 384, 1024, 128, 256, 640]
    assert sum(bench.alg_bytes(m, 4096, 7168) for m in Ms) == 124_780_544 + 22_528 * sum(Ms)
    # RMSNorm + quantisation: x read once, w, codes and scale bytes written once.
    assert bench.rms_bytes(4096, 7168) == 74_332_160


def test_roofline_peaks():
    assert bench.HBM_PEAK_GBS == 8000.0
    assert bench.FP4_PEAK_TFLOPS == 10100.0
    # The square's floors: 13.5 us of HBM, 23.8 us of matrix work (so it is matrix-bound).
    assert bench.alg_bytes(4096, 4096, 7168) / (bench.HBM_PEAK_GBS * 1e9) == pytest.approx(13.48e-6, rel=1e-3)
    assert bench.alg_flops(4096, 4096, 7168) / (bench.FP4_PEAK_TFLOPS * 1e12) == pytest.approx(23.81e-6, rel=1e-3)


@pytest.mark.parametrize("set_bytes", [75_776, 8_339_456 + 2 * 16 * 2112, 107_872_256, 650_000_000])
def test_cold_rotation_covers_twice_the_infinity_cache(set_bytes):
    args = argparse.Namespace(warm_cache=False)
    R = bench.n_sets(args, set_bytes)
    assert R * set_bytes >= bench.ROTATE_BYTES and (R - 1) * set_bytes < bench.ROTATE_BYTES or R == 1
    assert bench.ROTATE_BYTES >= 2 * (256 << 20)
    assert bench.cache_label(args, R, set_bytes).startswith("cold" if R > 1 else "warm")
    assert bench.n_sets(argparse.Namespace(warm_cache=True), set_bytes) == 1


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _trace_row(name, start_ns, dur_ns, grid_x, wg_x):
    return {"Kernel_Name": name, "Start_Timestamp": start_ns, "End_Timestamp": start_ns + dur_ns,
            "Grid_Size_X": grid_x, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
            "Workgroup_Size_X": wg_x, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1}


def _table(out):
    rows = {}
    for line in out.splitlines():
        cells = [c.strip() for c in line.strip("|").split("|")]
        if len(cells) == 10 and cells[2].isdigit():
            rows[(cells[0], int(cells[1]))] = [int(cells[2])] + [float(c) for c in cells[3:]]
    return rows


def test_summarize_stats_per_kernel_and_grid(tmp_path, capsys):
    rows = [_trace_row("gemm_tiled", 1000 * i, 70_000 + 1000 * i, 256 * 512, 512) for i in range(10)]
    rows += [_trace_row("gemm_tiled", 500_000 + i, 5_000, 8 * 512, 512) for i in range(4)]  # another grid
    rows += [_trace_row("other", 900_000, 1_000, 64, 64)]
    _write_csv(tmp_path / "run_kernel_trace.csv", rows)
    bench.summarize_stats(str(tmp_path))
    t = _table(capsys.readouterr().out)
    calls, avg, p10, med, p90, lo, hi, share = t[("gemm_tiled", 256)]
    assert calls == 10 and lo == 70.0 and hi == 79.0
    assert avg == pytest.approx(74.5) and med == pytest.approx(74.5)
    assert t[("gemm_tiled", 8)][0] == 4 and t[("other", 1)][0] == 1
    total = sum(70 + i for i in range(10)) + 4 * 5 + 1
    assert share == pytest.approx(100 * sum(70 + i for i in range(10)) / total, abs=0.05)
    # --select keeps dispatches A..B-1 of each kernel and grid, in start order.
    bench.summarize_stats(str(tmp_path), "2:5")
    t = _table(capsys.readouterr().out)
    assert t[("gemm_tiled", 256)][0] == 3 and t[("gemm_tiled", 256)][5] == 72.0 and t[("gemm_tiled", 256)][6] == 74.0
    assert t[("gemm_tiled", 8)][0] == 2 and ("other", 1) not in t


def _pmc_rows(name, counter, values):
    return [{"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v} for v in values]


def test_summarize_pmc_scales_by_the_copy_calibration(tmp_path, capsys):
    work, copy = tmp_path / "w", tmp_path / "c"
    (work / "FETCH_SIZE").mkdir(parents=True)
    (work / "WRITE_SIZE").mkdir()
    (copy / "FETCH_SIZE").mkdir(parents=True)
    (copy / "WRITE_SIZE").mkdir()
    _write_csv(work / "FETCH_SIZE" / "run_counter_collection.csv", _pmc_rows("gemm_tiled_kernel", "FETCH_SIZE", [100.0, 300.0]))
    _write_csv(work / "WRITE_SIZE" / "run_counter_collection.csv", _pmc_rows("gemm_tiled_kernel", "WRITE_SIZE", [50.0]))
    kib = bench.COPY_BYTES / 1024
    # The counters read the copy as half (fetch) and twice (write) its size: factors 2 and 1/2.
    _write_csv(copy / "FETCH_SIZE" / "run_counter_collection.csv", _pmc_rows("elementwise copy", "FETCH_SIZE", [kib / 2]))
    _write_csv(copy / "WRITE_SIZE" / "run_counter_collection.csv", _pmc_rows("elementwise copy", "WRITE_SIZE", [kib * 2]))
    bench.summarize_pmc(str(work), str(copy), "gemm_tiled")
    rec = json.loads(capsys.readouterr().out)
    assert rec["FETCH_SIZE"]["kib_per_dispatch"] == 200.0 and rec["FETCH_SIZE"]["copy_factor"] == pytest.approx(2.0)
    assert rec["WRITE_SIZE"]["copy_factor"] == pytest.approx(0.5)
    assert rec["bytes_per_launch"] == round((200.0 * 2.0 + 50.0 * 0.5) * 1024)
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()


@pytest.mark.parametrize("name", ["square", "skinny", "stress", "grouped", "grouped_decode", "mid", "rmsnorm",
                                  "grouped_mnk", "nvfp4_grouped", "square_unfused"])
def test_committed_traffic_records_match_the_sources(name, monkeypatch):
    b = bench.recorded_traffic(name)
    assert b is not None and b > 0, f"profiles/traffic_{name}.json is stale or missing"
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources=None: "0" * 16)
    assert bench.recorded_traffic(name) is None
