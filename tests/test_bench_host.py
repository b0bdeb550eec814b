"""Host-side logic of bench.py: the percentile helper, the reading of
rocprofv3 trace and counter CSVs, the source-hash gate on the committed
profile summaries, the algorithmic byte counts per launch, and the refusal of
more than one GPU. Nothing here touches a GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

import bench

KERNEL_M1 = "void skinny::mmvq_q4_0_kernel<1, 2>(unsigned char const*, ...)"
COPY = "__amd_rocclr_copyBuffer"


def test_launch_stats_nearest_rank():
    st = bench.launch_stats([float(v) for v in range(11, 0, -1)])
    assert st == {"median_us": 6.0, "p10_us": 2.0, "p90_us": 10.0, "sweeps": 11}
    one = bench.launch_stats([3.25])
    assert one["median_us"] == one["p10_us"] == one["p90_us"] == 3.25


def test_byte_counts_match_block_sizes():
    # Q4_0: 32 four-bit codes + one binary16 scale = 18 bytes per 32 weights;
    # Q8_1: 32 int8 codes + binary16 d and s = 36 bytes per 32 activations;
    # Q4_K: 144 bytes per 256; Q6_K: 210 bytes per 256; NVFP4: 8 bytes of
    # codes + one E4M3 scale per 16 values, plus the tensor's fp32 scale;
    # FP8: one byte a weight + an fp32 scale a row.
    M, K, N = 3, 4096, 1024
    out_f32 = 4 * M * N
    assert bench.q4_bytes(M, K, N) == N * K // 32 * 18 + M * K // 32 * 36 + out_f32
    assert bench.quant_bytes(M, K) == 4 * M * K + M * K // 32 * 36
    assert bench.q4_k_bytes(M, K, N) == N * K // 256 * 144 + M * K // 32 * 36 + out_f32
    # the Q6_K kernel reads only d of each Q8_1 block, not s
    assert bench.q6_k_bytes(M, K, N) == N * K // 256 * 210 + M * K // 32 * 34 + out_f32
    # IQ4_XS: 128 bytes of indices + an 8-byte header per 256 weights; the
    # kernel reads only d of each Q8_1 block
    assert bench.iq4_xs_bytes(M, K, N) == N * K // 256 * 136 + M * K // 32 * 34 + out_f32
    assert bench.nvfp4_bytes(M, K, N) == N * K // 16 * 9 + 4 + 2 * M * K + 2 * M * N
    assert bench.fp8_bytes(M, K, N) == N * K + 4 * N + 2 * M * K + 2 * M * N


def _sweep_rows(t0, dur_ns):
    """One Llama-2-7B decode sweep at M = 1 as kernel-trace rows: 32 layers
    of the four GEMVs, then lm_head, each launch dur_ns long."""
    rows = []
    shapes = [n for _ in range(32) for _, _, n in bench.LLAMA] + [bench.LM_HEAD[2]]
    t = t0
    for n in shapes:
        rows.append({"Kernel_Name": KERNEL_M1, "Grid_Size": str(64 * (n // 2)),
                     "Start_Timestamp": str(t), "End_Timestamp": str(t + dur_ns)})
        t += dur_ns + 100
    return rows, t


def test_sweep_launch_stats_finds_whole_sweeps_only():
    a, t = _sweep_rows(1000, 7000)
    # a partial sweep and unrelated launches between whole sweeps are skipped
    partial, t = _sweep_rows(t + 50, 9000)
    partial = partial[:40]
    t = int(partial[-1]["End_Timestamp"]) + 100
    other = [{"Kernel_Name": "void skinny::quantize_q8_1_kernel<1>(float const*)",
              "Grid_Size": "64", "Start_Timestamp": str(t), "End_Timestamp": str(t + 500)}]
    b, _ = _sweep_rows(t + 1000, 6000)
    rows = b + other + partial + a          # the trace need not be in time order
    durs = bench.sweep_launch_stats(rows)
    assert durs == [7000.0, 6000.0]


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _pmc_rows(copy_kib, kernel_kib, grid):
    """Counter rows of one run: the calibration copy, then one launch of the
    dominant kernel, each counter split over two XCD rows as rocprofv3 does."""
    rows = []
    for disp, (name, g, kib) in enumerate([(COPY, 4096, copy_kib), (KERNEL_M1, grid, kernel_kib)]):
        for half in (0.25, 0.75):
            rows.append({"Dispatch_Id": str(disp + 1), "Kernel_Name": name, "Grid_Size": str(g),
                         "Counter_Name": "X", "Counter_Value": repr(kib * half)})
    return rows


def test_summarize_pmc_scales_by_the_calibration_copy(tmp_path, capsys, monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h")
    grid = 64 * (4096 // 2)                 # o_proj of the sweep at M = 1
    calib_kib = bench.CALIB_BYTES / 1024
    # the copy's counters read 2x (fetch) and 1x (write) its true size
    _write_csv(str(tmp_path / "f" / "run" / "x_counter_collection.csv"),
               _pmc_rows(2 * calib_kib, 20000.0, grid))
    _write_csv(str(tmp_path / "w" / "run" / "x_counter_collection.csv"),
               _pmc_rows(calib_kib, 16.0, grid))
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"))
    out = capsys.readouterr().out
    assert "FETCH_SIZE scale 0.5000, WRITE_SIZE scale 1.0000" in out
    line = [ln for ln in out.splitlines() if ln.startswith("TRAFFIC_JSON ")]
    d = json.loads(line[0][len("TRAFFIC_JSON "):])
    assert d["source_sha256"] == "h"
    assert d["traffic_bytes_per_launch"] == pytest.approx(20000.0 * 1024 * 0.5 + 16.0 * 1024)


def test_summarize_pmc_rejects_mismatched_runs(tmp_path):
    grid = 64 * (4096 // 2)
    _write_csv(str(tmp_path / "f" / "a_counter_collection.csv"), _pmc_rows(1.0, 1.0, grid))
    _write_csv(str(tmp_path / "w" / "a_counter_collection.csv"), _pmc_rows(1.0, 1.0, grid)[:2])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"))


def test_committed_profiles_are_gated_by_the_kernel_source(monkeypatch):
    # the committed summaries were taken on the kernel sources as they stand
    trace = bench.committed_trace()
    traffic = bench.committed_traffic()
    assert trace is not None and trace["sweeps"] >= 10
    assert 1.0 < trace["p10_us"] <= trace["median_us"] <= trace["p90_us"] < 50.0
    assert traffic is not None
    # about the algorithmic bytes of one average sweep launch
    shapes = [n for _ in range(32) for _, _, n in bench.LLAMA] + [bench.LM_HEAD[2]]
    algo = sum(bench.q4_bytes(1, k, n) for _ in range(32) for _, k, n in bench.LLAMA)
    algo = (algo + bench.q4_bytes(1, bench.LM_HEAD[1], bench.LM_HEAD[2])) / len(shapes)
    assert 0.9 * algo < traffic < 1.2 * algo
    # a different source hash voids both
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.committed_trace() is None
    assert bench.committed_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
