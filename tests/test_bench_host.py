"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal, the
PMC summary with its copy-kernel calibration, the traffic record's source
hash check and the split's flop count."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _pmc_dir(tmp_path, name, counter, rows):
    d = tmp_path / name
    d.mkdir()
    with open(d / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})
    return str(d)


def test_summarize_pmc_calibrates_against_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_file", lambda wl: str(tmp_path / "traffic.json"))
    kib = bench.CALIB_BYTES / 1024
    # the copy reads half its bytes on FETCH_SIZE (factor 2) and all of them on WRITE_SIZE
    f = _pmc_dir(tmp_path, "f", "FETCH_SIZE", [("copyBuffer(...)", kib / 2), ("qgemm_pipe_kernel<...>", 1000.0),
                                               ("qgemm_pipe_kernel<...>", 1200.0)])
    w = _pmc_dir(tmp_path, "w", "WRITE_SIZE", [("copyBuffer(...)", kib), ("qgemm_pipe_kernel<...>", 500.0)])
    bench.summarize_pmc(f, w, "attn_proj_w4a4")
    rec = json.load(open(tmp_path / "traffic.json"))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes_per_launch"] == int(1100.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == 500 * 1024
    assert rec["gemm_source_hash"] == bench.gemm_source_hash("attn_proj_w4a4")
    assert rec["n_dispatches"] == [2, 1]


def test_load_traffic_rejects_a_stale_source_hash(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda wl: str(path))
    assert bench.load_traffic("attn_proj_w4a4") is None
    json.dump({"bytes_per_launch": 123, "gemm_source_hash": "not-this-source"}, open(path, "w"))
    assert bench.load_traffic("attn_proj_w4a4") is None
    json.dump({"bytes_per_launch": 123, "gemm_source_hash": bench.gemm_source_hash("attn_proj_w4a4")}, open(path, "w"))
    assert bench.load_traffic("attn_proj_w4a4") == 123


def test_committed_traffic_records_match_the_sources():
    for wl in ("attn_proj_w4a4", "attn_proj_w4a4_fp6", "ffdown_w8a8", "svdq_gateup", "svdq_gateup_fp6",
               "attn_proj_mxfp4", "attn_proj_mxfp8", "svdq_gateup_mxfp4"):
        assert bench.load_traffic(wl) is not None, wl


@pytest.mark.parametrize("q", [0, 2])
def test_split_flops(q):
    N, K, r, l = 40960, 5120, 32, 40
    # sketch product, 2 per power iteration, the final B^T, and the residual
    per_fit = 2 * N * K * l + q * 2 * (2 * N * K * l) + 2 * N * K * l + 2 * N * K * r
    assert bench._split_flops(N, K, r, l, q, 3) == 3 * per_fit


def test_warmup_is_a_floor_and_steps_are_exact():
    a = bench._parse(["--steps", "20", "--warmup", "5"])
    assert a.steps == 20 and a.warmup == 5      # at least 5 steps, and at least WARMUP_S of them
    assert bench.WARMUP_S >= 0.5
    d = bench._parse([])
    assert d.steps == 200 and d.warmup == 20
    s = bench._parse(["--workload", "stack"])
    assert s.steps == 3 and s.warmup == 1


def test_gemm_only_launch_count():
    assert bench.launch_count(0.07) == bench.GEMM_LAUNCHES    # headline GEMM: 100 launches a repeat
    assert bench.launch_count(1.6) == 31                      # about 50 ms a repeat
    assert bench.launch_count(150.0) == 2                     # the stack: at least 2
