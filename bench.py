"""Benchmark of the rotated low-bit quantized linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: one DiT attention projection at 1024x1024 -- X bf16 [4096 x 5120]
~ N(0,1) with 1% outlier channels x30, W [5120 x 5120] ~ N(0, 0.02) packed
int4 with the group-256 rotation, per-token activation / per-output-channel
weight scales, bf16 out.  Inputs and packed weights are resident in HBM
before timing.  One step = the layer's online path: rotate + quantize the
activations (rotate_quantize_act), then the W4A4 GEMM with its dequant
epilogue (qgemm_w4a4).  Weight packing is offline and timed separately.

Prints ONE JSON line.  `value` is the effective integer throughput of a
whole step, 2*M*N*K / step time, in TOP/s (eager launches, K steps between
two synchronizations).  `roofline` describes the GEMM kernel (the dominant
kernel): its average duration is measured inside the timed region with HIP
events that bracket each GEMM launch on the stream it runs on.
`cpu_baseline` times the CPU oracle on a bounded row sample.

Profiling helpers (used to make the summaries under profiles/):
    --calib-copy            also run a plain 256 MiB device copy (a kernel of
                            known traffic, to calibrate FETCH_SIZE/WRITE_SIZE)
    --summarize-pmc F W     read two rocprofv3 --pmc output dirs (FETCH_SIZE
                            run, WRITE_SIZE run) of this benchmark with
                            --calib-copy and write the GEMM's calibrated HBM
                            traffic per launch to profiles/
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_MFMA_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qgemm_w4a4_4096x5120x5120_traffic.json")
GEMM_SOURCES = ["rotated_bit_quantized_rotate_amd/csrc/qgemm_pipe.hip"]
CALIB_BYTES = 256 << 20


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time of the oracle baseline sample")
    p.add_argument("--calib-copy", action="store_true")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    return p.parse_args()


def cpu_baseline(wl, target_s=12.0):
    """The oracle as it stands, on a row sample of X against the full weights
    (weights quantized beforehand, like the GPU step): rotate + quantize the
    rows, exact integer product via float64 BLAS, dequant, bf16 rounding.
    A 64-row probe sizes the sample to about `target_s` seconds."""
    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    qw = O.quantize_weights(wl.w, wl.w_bits, wl.scale_mode)

    def run(rows):
        xs = np.ascontiguousarray(wl.x[:rows])
        t0 = time.perf_counter()
        qa = O.quantize_activations(xs, wl.a_bits, wl.scale_mode)
        y = O.linear_fp64(qa, qw)
        O.f64_to_bf16_bits(y)
        return time.perf_counter() - t0

    probe = run(64)
    rows = int(min(wl.M, max(64, 64 * target_s / max(probe, 1e-3))))
    dt = run(rows)
    ops = 2.0 * rows * wl.N * wl.K
    return {"value": round(ops / dt / 1e12, 4), "unit": "TOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of {wl.M} rows of X against all {wl.N} outputs (weights "
                      f"pre-quantized): rotate+quantize, exact integer GEMM via float64 BLAS, "
                      f"dequant, bf16 rounding; {dt:.2f} s wall on {threads} BLAS threads"}


def _read_pmc(dirname, counter):
    """{kernel short name: [values]} from a rocprofv3 counter_collection.csv."""
    out = {}
    for f in glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("qgemm" if "qgemm_pipe_kernel" in name else
                   "copy" if ("copyBuffer" in name or "copy" in name.lower()) else
                   re.sub(r"\(.*", "", name)[:40])
            out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def summarize_pmc(fetch_dir, write_dir):
    f = _read_pmc(fetch_dir, "FETCH_SIZE")
    w = _read_pmc(write_dir, "WRITE_SIZE")
    kib = 1024.0
    copy_f = np.mean(f["copy"]) * kib
    copy_w = np.mean(w["copy"]) * kib
    f_scale = CALIB_BYTES / copy_f
    w_scale = CALIB_BYTES / copy_w
    gf = np.mean(f["qgemm"]) * kib * f_scale
    gw = np.mean(w["qgemm"]) * kib * w_scale
    rec = {"kernel": "qgemm_w4a4 (qgemm_pipe_kernel 256x320)", "workload": "M=4096 N=5120 K=5120",
           "fetch_bytes_per_launch": int(gf), "write_bytes_per_launch": int(gw),
           "bytes_per_launch": int(gf + gw),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "copy_kib_fetch": round(copy_f / kib, 1), "copy_kib_write": round(copy_w / kib, 1),
           "gemm_source_hash": gemm_source_hash(),
           "n_dispatches": [len(f["qgemm"]), len(w["qgemm"])]}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def load_traffic():
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if rec.get("gemm_source_hash") != gemm_source_hash():
        return None                      # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


def main():
    args = _parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import rotated_bit_quantized_rotate_amd as Q
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if not Q.device_supported(0):
        raise SystemExit("device 0 is not gfx950")

    wl = W.attn_proj_w4a4()
    M, N, K = wl.M, wl.N, wl.K

    def to_dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x = to_dev_bf16(wl.x)
    w = to_dev_bf16(wl.w)
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    sa = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    # offline weight preparation (not part of a step)
    wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    sw = torch.empty((N,), dtype=torch.float32, device=dev)
    Q.pack_weight_int4(w, packed=wq, scales=sw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        Q.pack_weight_int4(w, packed=wq, scales=sw)
    e1.record()
    torch.cuda.synchronize()
    pack_ms = e0.elapsed_time(e1) / 10

    def prologue():
        Q.rotate_quantize_act(x, bits=4, scale_mode="row", codes=codes, scales=sa)

    def gemm():
        Q.qgemm_w4a4(codes, sa, wq, sw, K, out=out)

    for _ in range(args.warmup):
        prologue()
        gemm()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, synchronized on both sides.
    # Events bracket the prologue and the GEMM of every step on the stream
    # the kernels run on (the current torch stream).
    n = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * n + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for s in range(n):
        prologue()
        ev[3 * s + 1].record()
        gemm()
        ev[3 * s + 2].record()
        ev[3 * s + 3].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    step_ms = ev[0].elapsed_time(ev[3 * n]) / n
    gemm_ms = float(np.mean([ev[3 * s + 1].elapsed_time(ev[3 * s + 2]) for s in range(n)]))
    pro_ms = float(np.mean([(ev[3 * s].elapsed_time(ev[3 * s + 1])) for s in range(n)]))

    # ---- the same step replayed from a HIP graph (no host launch cost)
    graph_step_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            prologue()
            gemm()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            prologue()
            gemm()
        for _ in range(5):
            g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_step_ms = e0.elapsed_time(e1) / n
    except Exception as exc:  # graph capture is an extra figure only
        print(f"graph replay skipped: {exc}", file=sys.stderr)

    if args.calib_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    ops = 2.0 * M * N * K
    value = ops / (step_ms * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    pro_bytes = M * K * 2 + M * K + M * 4          # bf16 in, int8 codes + scales out
    gemm_bytes = M * K + N * K // 2 + M * 4 + N * 4 + M * N * 2

    rec = {
        "metric": "effective int TOPS + % int8 MFMA peak, W4A4 rotated GEMM M=4096 K=N=5120",
        "value": round(value, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 MFMA (int4 codes), int32 accumulate, bf16 out",
        "data": "synthetic",
        "config": {"workload": "W4A4 rotated linear, DiT attention projection at 1024^2: "
                               "X bf16 [4096x5120] N(0,1) + 1% outlier channels x30, "
                               "W [5120x5120] packed int4, group-256 Hadamard, per-token / "
                               "per-row scales, bf16 out",
                   "M": M, "N": N, "K": K, "global_batch": M, "parallelism": "single GPU"},
        "pct_int8_peak_step": round(100.0 * value / INT8_MFMA_PEAK_TOPS, 2),
        "gemm_only": {"ms": round(gemm_ms, 5), "tops": round(gemm_tops, 2),
                      "pct_int8_peak": round(100.0 * gemm_tops / INT8_MFMA_PEAK_TOPS, 2)},
        "prologue": {"ms": round(pro_ms, 5),
                     "gbs": round(pro_bytes / (pro_ms * 1e-3) / 1e9, 1),
                     "pct_hbm_peak": round(100.0 * pro_bytes / (pro_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
        "graph_step_ms": None if graph_step_ms is None else round(graph_step_ms, 5),
        "graph_step_tops": None if graph_step_ms is None else round(ops / (graph_step_ms * 1e-3) / 1e12, 2),
        "weight_prep_ms": round(pack_ms, 5),
        "wall_ms_timed_region": round(wall_ms, 3),
        "roofline": {"bound": "mfma", "kernel": "qgemm_w4a4",
                     "achieved": round(gemm_tops, 2), "peak": INT8_MFMA_PEAK_TOPS,
                     "unit": "TOP/s", "frac": round(gemm_tops / INT8_MFMA_PEAK_TOPS, 4),
                     "traffic": load_traffic(), "algorithmic_bytes": gemm_bytes},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
