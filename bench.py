"""Benchmark of the rotated low-bit quantized linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: one DiT attention projection at 1024x1024 -- X bf16 [4096 x 5120]
~ N(0,1) with 1% outlier channels x30, W [5120 x 5120] ~ N(0, 0.02) packed
int4 with the group-256 rotation, per-token activation / per-output-channel
weight scales, bf16 out.  Inputs and packed weights are resident in HBM
before timing.  One step = the layer's online path: rotate + quantize the
activations (rotate_quantize_act) then the W4A4 GEMM with its dequant
epilogue (qgemm_w4a4).  Weight packing is offline and timed separately.

Prints ONE JSON line.  `value` is the effective integer throughput of a
whole step, 2*M*N*K / step time, in TOP/s.  `roofline` describes the GEMM
kernel (the dominant kernel) against the int8 MFMA peak, timed with HIP
events on the stream the kernels run on.  `cpu_baseline` times the CPU oracle
on a bounded row sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_MFMA_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time of the oracle baseline sample")
    return p.parse_args()


def _event_time_ms(fn, iters, torch):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


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
    return {"value": ops / dt / 1e12, "unit": "TOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {wl.M} rows of X (all {wl.N} outputs), weights pre-quantized; "
                      f"{dt:.2f} s wall"}


def main():
    args = _parse()
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
    pack_ms = _event_time_ms(lambda: Q.pack_weight_int4(w, packed=wq, scales=sw), 10, torch)

    def prologue():
        Q.rotate_quantize_act(x, bits=4, scale_mode="row", codes=codes, scales=sa)

    def gemm():
        Q.qgemm_w4a4(codes, sa, wq, sw, K, out=out)

    def step():
        prologue()
        gemm()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronized on both sides
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    step_ms = start.elapsed_time(end) / args.steps

    # per-kernel averages (HIP events on the kernels' stream)
    reps = max(20, args.steps)
    gemm_ms = _event_time_ms(gemm, reps, torch)
    pro_ms = _event_time_ms(prologue, reps, torch)

    ops = 2.0 * M * N * K
    value = ops / (step_ms * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    pro_bytes = M * K * 2 + M * K + M * 4          # bf16 in, int8 codes + scales out
    gemm_bytes = M * K + N * K // 2 + M * 4 + N * 4 + M * N * 2

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "qgemm_w4a4_4096x5120x5120_traffic.json")
    if os.path.exists(tfile):
        try:
            traffic = json.load(open(tfile)).get("bytes_per_launch")
        except Exception:
            traffic = None

    rec = {
        "metric": "effective int TOPS + % int8 MFMA peak, W4A4 rotated GEMM M=4096 K=N=5120",
        "value": round(value, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
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
        "weight_prep_ms": round(pack_ms, 5),
        "wall_ms_timed_region": round(wall_ms, 3),
        "roofline": {"bound": "mfma", "kernel": "qgemm_w4a4",
                     "achieved": round(gemm_tops, 2), "peak": INT8_MFMA_PEAK_TOPS,
                     "unit": "TOP/s", "frac": round(gemm_tops / INT8_MFMA_PEAK_TOPS, 4),
                     "traffic": traffic, "algorithmic_bytes": gemm_bytes},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
