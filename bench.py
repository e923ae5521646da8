"""Benchmark of the rotated low-bit quantized linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload attn_proj_w4a4|attn_proj_w4a4_fp6|ffdown_w8a8|svdq_gateup|
                                svdq_gateup_fp6|svdq_split_gateup|stack|stack_fp6|stack_fused|
                                stack_fused_fp6|stack_grouped]

Default workload (the headline line): one DiT attention projection at
1024x1024 -- X bf16 [4096 x 5120] ~ N(0,1) with 1% outlier channels x30,
W [5120 x 5120] ~ N(0, 0.02) packed int4 with the group-256 rotation,
per-token activation / per-output-channel weight scales, bf16 out.

Other workloads (separate runs, same JSON shape):
  ffdown_w8a8   W8A8 ff.down, X [4096 x 20480] post-SwiGLU-like, W int8 per
                row [5120 x 20480], gated residual onto bf16 [4096 x 5120]
  svdq_gateup   group-64 W4A4 gate|up [40960 x 5120] + bf16 rank-32
                low-rank branch, SwiGLU out [4096 x 20480]
  svdq_gateup_fp6  the same layer with the codes in the FP6 e2m3 layout on
                the FP6 matrix instruction (bit-identical output)
  attn_proj_w4a4_fp6  the headline projection on the FP6 instruction
  stack         the 224 linears of a 28-block DiT at 2048x2048 (16384
                tokens): 128 W4A4 + 96 W8A8, every activation resident
  stack_fp6     the stack with its 128 W4A4 layers' INT4 codes in the FP6 layout
                on the FP6 matrix instruction (same outputs bit for bit)
  stack_fused   the same 224 linears with each block's RMSNorm + modulation
                fused into its prologues and one prepared activation per
                shared input and precision (Q|gate int4, K|V int8, gate|up):
                5 prologues per block instead of 8
  stack_fused_fp6  stack_fused with the W4A4 layers on the FP6 instruction
  stack_grouped stack_fused with each block's Q|K|V|gate projections in one
                grouped launch (sigmoid on the gate; K, V in INT8) and its
                gate|up projections in another: 4 GEMM launches per block

Inputs and prepared weights are resident in HBM before timing.  One step is
the layer's online path: rotate + quantize the activations
(rotate_quantize_act, which also forms X @ L1 for the low-rank branch), then
the quantized GEMM with its fused epilogue.  Weight preparation (rotation,
quantization, int4 packing) is offline and timed separately.

Prints ONE JSON line.  `value` is the effective integer throughput of a whole
step, 2*M*N*K / step time, in TOP/s (eager launches, K steps between two
synchronizations, with one HIP event before and one after).  `roofline`
describes the GEMM kernel (the dominant kernel): its time is the median of 5
repeats of back-to-back GEMM launches on codes already in HBM (HIP events on
the launch stream); the step minus the prologues run alone is reported beside
it.  The group-64 layers are bound by their per-group fp32 rescale, so their
roofline is the VALU's (`bound` "alu": algorithmic rescale instructions
against the fp32 issue rate), with the int8-MFMA fraction kept beside it.  A
second run of the K steps with a HIP event after every launch gives the
per-kernel breakdown
reported beside it (`*_with_kernel_events`); those events add a gap of a
few microseconds at each kernel boundary.  `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload.

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
FP6_MFMA_PEAK_TOPS = 10100.0     # MI355X dense FP6 / FP4 MFMA, 10.1 PFLOP/s
FP4_MFMA_PEAK_TOPS = 10100.0
FP8_MFMA_PEAK_TOPS = 5000.0      # MI355X dense FP8 MFMA, 5.0 PFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector FMA: 256 CUs x 128 lanes x 2 x 2.4 GHz
# fp32 VALU instructions without packed fp32 (which this library never emits):
# 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz (a wave64 instruction
# occupies its SIMD for 4 clocks), in lane-instructions per second
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
CALIB_BYTES = 256 << 20
CSRC = "rotated_bit_quantized_rotate_amd/csrc/"
HEADLINE_METRIC = "effective int TOPS + % int8 MFMA peak, W4A4 rotated GEMM M=4096 K=N=5120"

# workload -> (GEMM kernel label, shape tag, sources whose text defines that kernel)
GEMM_KERNELS = {
    "attn_proj_w4a4": ("qgemm_w4a4", "4096x5120x5120", ["qgemm_pipe.hip"]),
    "attn_proj_w4a4_fp6": ("qgemm_w4a4_fp6", "4096x5120x5120", ["qgemm_pipe.hip"]),
    "attn_proj_mxfp4": ("qgemm_mx_fp4", "4096x5120x5120", ["qgemm_pipe.hip"]),
    "attn_proj_mxfp8": ("qgemm_mx_fp8", "4096x5120x5120", ["qgemm_pipe.hip"]),
    "svdq_gateup_mxfp4": ("qgemm_mx_lowrank_fp4", "4096x5120x40960", ["qgemm_pipe.hip"]),
    "svdq_split_gateup": ("svdq_split", "40960x5120_r32", ["svdq_split.hip"]),
    "ffdown_w8a8": ("qgemm_w8a8", "4096x20480x5120", ["qgemm_pipe.hip"]),
    "svdq_gateup": ("qgemm_w4a4_lowrank", "4096x5120x40960", ["qgemm_pipe.hip"]),
    "svdq_gateup_fp6": ("qgemm_w4a4_lowrank_fp6", "4096x5120x40960", ["qgemm_pipe.hip"]),
    "stack": ("qgemm_stack", "224x16384", ["qgemm_pipe.hip"]),
    "stack_fused": ("qgemm_stack_fused", "224x16384", ["qgemm_pipe.hip"]),
    "stack_fp6": ("qgemm_stack_fp6", "224x16384", ["qgemm_pipe.hip"]),
    "stack_fused_fp6": ("qgemm_stack_fused_fp6", "224x16384", ["qgemm_pipe.hip"]),
    "stack_grouped": ("qgemm_stack_grouped", "224x16384", ["qgemm_pipe.hip"]),
}


def traffic_file(workload):
    label, shape, _ = GEMM_KERNELS[workload]
    return os.path.join(ROOT, "profiles", f"{label}_{shape}_traffic.json")


def gemm_source_hash(workload="attn_proj_w4a4") -> str:
    h = hashlib.sha256()
    for f in GEMM_KERNELS[workload][2]:
        with open(os.path.join(ROOT, CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


WARMUP_S = 0.5       # warm-up floor, seconds of steps (clocks settle only under sustained load)
GEMM_REPEATS = 5     # GEMM-only: median of this many repeats ...
GEMM_LAUNCHES = 100  # ... of this many back-to-back launches (after 10 untimed ones)
COLD_LAUNCHES = 20   # cold-cache variant: launches, each after a 512 MiB write
FLUSH_BYTES = 512 << 20


def _parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default 200; 3 for the stack)")
    p.add_argument("--warmup", type=int, default=None,
                   help="minimum untimed warm-up steps (default 20; 1 for the stack); warm-up always "
                        "lasts at least 0.5 s of steps")
    p.add_argument("--workload", default="attn_proj_w4a4", choices=sorted(GEMM_KERNELS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--no-other-gemms", action="store_true",
                   help="headline workload: skip the GEMM-only figures of the W8A8 and SVDQuant layers")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time of the oracle baseline sample")
    p.add_argument("--calib-copy", action="store_true")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    a = p.parse_args(argv)
    stack = a.workload.startswith("stack")
    if a.steps is None:
        a.steps = 3 if stack else (20 if a.workload.startswith("svdq_split") else 200)
    if a.warmup is None:
        a.warmup = 1 if stack else 20
    return a


# ---------------------------------------------------------------- CPU oracle --
def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, target_s=12.0, one_thread_s=3.0):
    """The oracle as it stands, on a row sample of X against the full weights
    (weights quantized beforehand, like the GPU step): rotate + quantize the
    rows, exact integer product via float64 BLAS (per 64-group for group-64
    scales), dequant, low-rank branch, epilogue, bf16 rounding.  A 64-row
    probe sizes the sample to about `target_s` seconds; when the whole
    workload takes less, it is run repeatedly and the total time is used.
    A second, smaller sample runs with BLAS limited to one thread."""
    import oracle as O

    threads = _blas_threads()
    qw = O.quantize_weights(wl.w, wl.w_bits, wl.scale_mode)
    res = O.bf16_bits_to_f64(wl.residual) if wl.residual is not None else None
    gate = O.bf16_bits_to_f64(wl.gate) if wl.gate is not None else None

    def run(rows):
        xs = np.ascontiguousarray(wl.x[:rows])
        t0 = time.perf_counter()
        qa = O.quantize_activations(xs, wl.a_bits, wl.scale_mode)
        y = O.linear_fp64(qa, qw, xs, wl.l1, wl.l2)
        out = O.epilogue(y, wl.epilogue, None if res is None else res[:rows], gate)
        O.f64_to_bf16_bits(out)
        return time.perf_counter() - t0

    def sample(target):
        probe = run(64)
        rows = int(min(wl.M, max(64, 64 * target / max(probe, 1e-3))))
        reps = 1
        if rows == wl.M:
            first = run(rows)
            reps = max(1, int(round((target - first) / max(first, 1e-3))))
        t = sum(run(rows) for _ in range(reps))
        return rows, reps, t

    rows, reps, t = sample(target_s)
    ops = 2.0 * rows * wl.N * wl.K * reps
    what = f"{rows} of {wl.M} rows of X" + (f", whole workload x{reps}" if rows == wl.M else "")
    rec = {"value": round(ops / t / 1e12, 4), "unit": "TOP/s", "cores": int(threads),
           "kind": "oracle", "cpu_model": _cpu_model(),
           "sample": f"{what} against all {wl.N} outputs (weights pre-quantized): "
                     f"rotate+quantize, exact integer GEMM via float64 BLAS, dequant, "
                     + (f"rank-{wl.l1.shape[1]} branch, " if wl.l1 is not None else "")
                     + f"{wl.epilogue} epilogue, bf16 rounding; {t:.2f} s wall on {threads} "
                     f"BLAS threads"}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            r1, n1, t1 = sample(one_thread_s)
        rec["one_thread"] = {"value": round(2.0 * r1 * wl.N * wl.K * n1 / t1 / 1e12, 5), "unit": "TOP/s",
                             "sample": f"{r1} rows x{n1}, {t1:.2f} s wall on 1 BLAS thread"}
    except ImportError:
        rec["one_thread"] = None
    return rec


# ------------------------------------------------------------ PMC traffic --
def _read_pmc(dirname, counter):
    """{kernel class: [values]} from a rocprofv3 counter_collection.csv."""
    out = {}
    for f in glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("qgemm" if "qgemm" in name else
                   "copy" if ("copyBuffer" in name or "copy" in name.lower()) else
                   re.sub(r"\(.*", "", name)[:40])
            out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def summarize_pmc(fetch_dir, write_dir, workload):
    f = _read_pmc(fetch_dir, "FETCH_SIZE")
    w = _read_pmc(write_dir, "WRITE_SIZE")
    kib = 1024.0
    # the calibration copies are the run's largest device copies; smaller
    # ones (input uploads) must not dilute the factor
    copy_f = np.max(f["copy"]) * kib
    copy_w = np.max(w["copy"]) * kib
    f_scale = CALIB_BYTES / copy_f
    w_scale = CALIB_BYTES / copy_w
    gf = np.mean(f["qgemm"]) * kib * f_scale
    gw = np.mean(w["qgemm"]) * kib * w_scale
    label, shape, _ = GEMM_KERNELS[workload]
    rec = {"kernel": label, "workload": shape,
           "fetch_bytes_per_launch": int(gf), "write_bytes_per_launch": int(gw),
           "bytes_per_launch": int(gf + gw),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "copy_kib_fetch": round(copy_f / kib, 1), "copy_kib_write": round(copy_w / kib, 1),
           "gemm_source_hash": gemm_source_hash(workload),
           "n_dispatches": [len(f["qgemm"]), len(w["qgemm"])]}
    path = traffic_file(workload)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def load_traffic(workload):
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    if rec.get("gemm_source_hash") != gemm_source_hash(workload):
        return None                      # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


# -------------------------------------------------------------- workloads --
class Case:
    """One benchmark workload: prepared device tensors and the launches of a
    step, in order, each tagged "prologue" or "gemm"."""

    def __init__(self):
        self.launches = []        # [(tag, fn)]
        self.ops = 0              # 2*M*N*K summed over the step's GEMMs
        self.gemm_bytes = 0       # algorithmic HBM bytes of the step's GEMMs
        self.pro_bytes = 0        # algorithmic HBM bytes of the step's prologues
        self.gemm_launches = 0
        self.prep_ms = 0.0
        self.metric = ""
        self.config = {}
        self.dtype = ""
        self.wl = None            # host workload for the CPU baseline
        self.peak = INT8_MFMA_PEAK_TOPS   # dense matrix peak of the GEMM's instruction
        # VALU-bound GEMMs (group-64 rescale): algorithmic fp32 VALU lane-
        # instructions per launch; the roofline is then the VALU's
        self.valu_ops = 0
        self.bound = "mfma"
        self.cpu_fn = None        # custom CPU baseline (else the linear's oracle on case.wl)
        self.unit = "TOP/s"
        # low-rank layers: (the prologue without X @ L1, the GEMM without the
        # branch), the same launches otherwise, to report the branch's cost
        self.branch = None


def _bf16_dev(bits, dev):
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)


def _timed_prep(fn):
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def case_attn(Q, W, dev):
    import torch
    wl = W.attn_proj_w4a4()
    M, N, K = wl.M, wl.N, wl.K
    x, w = _bf16_dev(wl.x, dev), _bf16_dev(wl.w, dev)
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    sa = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    sw = torch.empty((N,), dtype=torch.float32, device=dev)
    c = Case()
    c.prep_ms = _timed_prep(lambda: Q.pack_weight_int4(w, packed=wq, scales=sw))
    c.launches = [
        ("prologue", lambda: Q.rotate_quantize_act(x, bits=4, scale_mode="row", codes=codes, scales=sa)),
        ("gemm", lambda: Q.qgemm_w4a4(codes, sa, wq, sw, K, out=out)),
    ]
    c.ops = wl.int_ops
    c.gemm_launches = 1
    c.pro_bytes = M * K * 2 + M * K + M * 4
    c.gemm_bytes = M * K + N * K // 2 + M * 4 + N * 4 + M * N * 2
    c.metric = HEADLINE_METRIC
    c.dtype = "int8 MFMA (int4 codes), int32 accumulate, bf16 out"
    c.config = {"workload": "W4A4 rotated linear, DiT attention projection at 1024^2: "
                            "X bf16 [4096x5120] N(0,1) + 1% outlier channels x30, "
                            "W [5120x5120] packed int4, group-256 Hadamard, per-token / "
                            "per-row scales, bf16 out",
                "M": M, "N": N, "K": K, "global_batch": M, "parallelism": "single GPU"}
    c.wl = wl
    return c


def case_attn_fp6(Q, W, dev):
    """The attention projection with the int4 codes in the FP6 e2m3 layout,
    multiplied on the FP6 matrix instruction (same codes, same output)."""
    import torch
    wl = W.attn_proj_w4a4()
    M, N, K = wl.M, wl.N, wl.K
    x, w = _bf16_dev(wl.x, dev), _bf16_dev(wl.w, dev)
    codes = torch.empty((M, K // 4 * 3), dtype=torch.uint8, device=dev)
    sa = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wq = torch.empty((N, K // 4 * 3), dtype=torch.uint8, device=dev)
    sw = torch.empty((N,), dtype=torch.float32, device=dev)
    c = Case()
    c.prep_ms = _timed_prep(lambda: Q.pack_weight_fp6(w, packed=wq, scales=sw))
    c.launches = [
        ("prologue", lambda: Q.rotate_quantize_act(x, bits=4, scale_mode="row", layout="fp6", codes=codes,
                                                   scales=sa)),
        ("gemm", lambda: Q.qgemm_w4a4_fp6(codes, sa, wq, sw, K, out=out)),
    ]
    c.ops = wl.int_ops
    c.gemm_launches = 1
    c.pro_bytes = M * K * 2 + M * K // 4 * 3 + M * 4
    c.gemm_bytes = (M + N) * K // 4 * 3 + M * 4 + N * 4 + M * N * 2
    c.metric = "effective int TOPS, W4A4 rotated GEMM M=4096 K=N=5120 on the FP6 matrix instruction (experiment)"
    c.dtype = "fp6 e2m3 MFMA (exact int4 codes), fp32 accumulate (exact), bf16 out"
    c.peak = FP6_MFMA_PEAK_TOPS
    c.config = {"workload": "W4A4 rotated linear, DiT attention projection at 1024^2, int4 codes stored as "
                            "FP6 e2m3: X bf16 [4096x5120] N(0,1) + 1% outlier channels x30, W [5120x5120], "
                            "group-256 Hadamard, per-token / per-row scales, bf16 out",
                "M": M, "N": N, "K": K, "global_batch": M, "parallelism": "single GPU"}
    c.wl = wl
    return c


def mx_cpu_baseline(wl, fmt, target_s=12.0, one_thread_s=3.0):
    """The MX oracle on a row sample of X against the pre-quantized weights:
    rotate, block-quantize, the block-scaled product (float64 BLAS per
    32-channel block), the low-rank branch and epilogue when the workload
    has them, bf16 rounding."""
    import oracle as O

    threads = _blas_threads()
    qw = O.quantize_mx(wl.w, fmt)
    l1 = None if wl.l1 is None else O.bf16_bits_to_f64(wl.l1)
    l2 = None if wl.l2 is None else O.bf16_bits_to_f64(wl.l2)

    def run(rows):
        xs = np.ascontiguousarray(wl.x[:rows])
        t0 = time.perf_counter()
        qa = O.quantize_mx(xs, fmt)
        y = O.mx_gemm(qa, qw)
        if l1 is not None:
            y = y + (O.bf16_bits_to_f64(xs) @ l1) @ l2
        O.f64_to_bf16_bits(O.epilogue(y, wl.epilogue))
        return time.perf_counter() - t0

    def sample(target):
        probe = run(16)
        rows = int(min(wl.M, max(16, 16 * target / max(probe, 1e-3))))
        return rows, run(rows)

    rows, t = sample(target_s)
    rec = {"value": round(2.0 * rows * wl.N * wl.K / t / 1e12, 5), "unit": "TOP/s", "cores": int(threads),
           "kind": "oracle", "cpu_model": _cpu_model(),
           "sample": f"{rows} of {wl.M} rows of X against all {wl.N} outputs (weights pre-quantized): rotate, "
                     f"MX {fmt} block quantization, block-scaled product via float64 BLAS per 32-channel "
                     f"block{', rank-%d branch' % wl.l1.shape[1] if wl.l1 is not None else ''}, {wl.epilogue} "
                     f"epilogue, bf16 rounding; {t:.2f} s wall on {threads} BLAS threads"}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            r1, t1 = sample(one_thread_s)
        rec["one_thread"] = {"value": round(2.0 * r1 * wl.N * wl.K / t1 / 1e12, 6), "unit": "TOP/s",
                             "sample": f"{r1} rows, {t1:.2f} s wall on 1 BLAS thread"}
    except ImportError:
        rec["one_thread"] = None
    return rec


def case_attn_mx(Q, W, dev, fmt="fp4"):
    """The attention projection in the OCP MX block formats on gfx950's
    block-scaled matrix instruction: both operands rotated and quantized to
    32-element blocks with an E8M0 scale (MXFP4: E2M1 elements, the
    counterpart of the pages' NVFP4 build; MXFP8: E4M3, their mxfp8 build)."""
    import torch
    wl = W.attn_proj_w4a4()
    M, N, K = wl.M, wl.N, wl.K
    eb = K // 2 if fmt == "fp4" else K          # element bytes per row
    x, w = _bf16_dev(wl.x, dev), _bf16_dev(wl.w, dev)
    codes = torch.empty((M, eb), dtype=torch.uint8, device=dev)
    sa = torch.empty((K // 128, M, 4), dtype=torch.uint8, device=dev)
    wq = torch.empty((N, eb), dtype=torch.uint8, device=dev)
    sw = torch.empty((K // 128, N, 4), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    c = Case()
    c.prep_ms = _timed_prep(lambda: Q.rotate_quantize_mx(w, fmt=fmt, codes=wq, scales=sw))
    c.launches = [
        ("prologue", lambda: Q.rotate_quantize_mx(x, fmt=fmt, codes=codes, scales=sa)),
        ("gemm", lambda: Q.qgemm_mx(codes, sa, wq, sw, K, fmt=fmt, out=out)),
    ]
    c.ops = wl.int_ops
    c.gemm_launches = 1
    c.pro_bytes = M * K * 2 + M * eb + M * K // 32
    c.gemm_bytes = (M + N) * (eb + K // 32) + M * N * 2
    name = "MXFP4" if fmt == "fp4" else "MXFP8"
    c.metric = (f"effective TOPS + % {'FP4' if fmt == 'fp4' else 'FP8'} MFMA peak, {name} rotated GEMM "
                f"M=4096 K=N=5120 (block-scaled matrix instruction)")
    c.dtype = (f"{'fp4 e2m1' if fmt == 'fp4' else 'fp8 e4m3'} elements x E8M0 block-32 scales (MX), "
               "fp32 accumulate, bf16 out")
    c.peak = FP4_MFMA_PEAK_TOPS if fmt == "fp4" else FP8_MFMA_PEAK_TOPS
    c.config = {"workload": f"{name} rotated linear, DiT attention projection at 1024^2: X bf16 [4096x5120] "
                            "N(0,1) + 1% outlier channels x30, W [5120x5120], group-256 Hadamard, OCP MX "
                            "blocks of 32 with E8M0 scales on both operands, bf16 out",
                "M": M, "N": N, "K": K, "global_batch": M, "parallelism": "single GPU"}
    c.wl = wl
    c.cpu_fn = lambda s: mx_cpu_baseline(wl, fmt, s)
    return c


def case_svdq_mx(Q, W, dev):
    """The SVDQuant gate|up layer in MXFP4 -- the pages' NVFP4 r32 build on
    gfx950's block-scaled FP4 instruction: the same X, W, rank-32 factors and
    SwiGLU as the INT4 group-64 workload, W and X as MXFP4 blocks."""
    import torch
    wl = W.svdq_gateup()
    M, N, K = wl.M, wl.N, wl.K
    r = wl.l1.shape[1]
    x, w = _bf16_dev(wl.x, dev), _bf16_dev(wl.w, dev)
    l1, l2 = _bf16_dev(wl.l1, dev), _bf16_dev(np.ascontiguousarray(wl.l2.T), dev)  # L2 transposed, [N, r]
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sa = torch.empty((K // 128, M, 4), dtype=torch.uint8, device=dev)
    lr = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    sw = torch.empty((K // 128, N, 4), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
    c = Case()
    c.prep_ms = _timed_prep(lambda: Q.rotate_quantize_mx(w, fmt="fp4", codes=wq, scales=sw))
    c.launches = [
        ("prologue", lambda: Q.rotate_quantize_mx(x, fmt="fp4", codes=codes, scales=sa, l1=l1, lr=lr)),
        ("gemm", lambda: Q.qgemm_mx_lowrank(codes, sa, wq, sw, K, fmt="fp4", lr=lr, l2=l2, epilogue="swiglu",
                                            out=out)),
    ]
    out0 = torch.empty_like(out)
    c.branch = (
        lambda: Q.rotate_quantize_mx(x, fmt="fp4", codes=codes, scales=sa),
        lambda: Q.qgemm_mx_lowrank(codes, sa, wq, sw, K, fmt="fp4", epilogue="swiglu", out=out0))
    c.ops = wl.int_ops
    c.gemm_launches = 1
    c.pro_bytes = M * K * 2 + K * r * 2 + M * K // 2 + M * K // 32 + M * r * 2
    c.gemm_bytes = (M + N) * (K // 2 + K // 32) + M * r * 2 + r * N * 2 + M * (N // 2) * 2
    c.metric = ("effective TOPS + % FP4 MFMA peak, MXFP4 SVDQuant gate|up GEMM + rank-32 low-rank + SwiGLU "
                "M=4096 K=5120 N=40960 (block-scaled matrix instruction)")
    c.dtype = "fp4 e2m1 elements x E8M0 block-32 scales (MX), fp32 accumulate, bf16 rank-32 branch, bf16 out"
    c.peak = FP4_MFMA_PEAK_TOPS
    c.config = {"workload": "SVDQuant fused gate|up in MXFP4 (the NVFP4 r32 build on gfx950): X bf16 [4096x5120], "
                            "W [40960x5120] MXFP4 with group-256 Hadamard, bf16 rank-32 L1 [5120x32] / "
                            "L2 [32x40960], SwiGLU -> bf16 [4096x20480]",
                "M": M, "N": N, "K": K, "rank": r, "global_batch": M, "parallelism": "single GPU"}
    c.wl = wl
    c.cpu_fn = lambda s: mx_cpu_baseline(wl, "fp4", s)
    return c


SPLIT_RANK, SPLIT_OVER, SPLIT_POWER, SPLIT_REFINE = 32, 8, 2, 2


def _split_flops(N, K, r, l, q, iters):
    """fp32 multiply-adds x 2 of the split's large products per call: the
    sketch product, 2 per power iteration, the final B^T, and the residual."""
    return 2.0 * N * K * (l * (2 + 2 * q) + r) * iters


def case_svdq_split(Q, W, dev):
    """The offline SVDQuant split of the gate|up weight [40960 x 5120]: rank 32,
    oversampling 8, 2 power iterations, activation-aware with synthetic
    channel RMS, 2 refinement iterations (3 fits), group-64 residual."""
    import torch
    wl = W.svdq_gateup()
    N, K = wl.w.shape
    r, l = SPLIT_RANK, SPLIT_RANK + SPLIT_OVER
    w = _bf16_dev(wl.w, dev)
    omega = torch.from_numpy(W.gaussian_sketch(K, l, 0)).to(dev)
    rms_h = W.act_rms(K, 1)
    rms = torch.from_numpy(rms_h).to(dev)
    ws = torch.empty(Q.svdq_split_workspace_bytes(N, K, r, SPLIT_OVER, "group64"), dtype=torch.uint8, device=dev)
    c = Case()
    c.launches = [("gemm", lambda: Q.svdq_split(w, omega, r, SPLIT_OVER, SPLIT_POWER, SPLIT_REFINE, "group64",
                                                act_rms=rms, workspace=ws))]
    iters = SPLIT_REFINE + 1
    c.ops = _split_flops(N, K, r, l, SPLIT_POWER, iters)
    c.gemm_launches = 1
    c.gemm_bytes = N * K * 2 + K * l * 4 + K * 4 + K * r * 2 + r * N * 2 + N * K // 2 + N * (K // 64) * 4
    c.metric = ("offline SVDQuant split of the gate|up weight [40960x5120], rank 32, 3 fits: effective fp32 "
                "TFLOP/s of its products (ms_per_step = one split)")
    c.dtype = "fp32 (products, CholeskyQR2 and Jacobi in fp64), bf16 factors, int4 residual"
    c.peak = FP32_VECTOR_PEAK_TFLOPS
    c.bound = "alu"
    c.unit = "TFLOP/s"
    c.config = {"workload": "SVDQuant split: W bf16 [40960x5120] N(0, 0.02), Gaussian sketch [5120x40] (seed 0), "
                            "synthetic log-normal channel RMS with 1% outlier channels x30 (seed 1); rank 32, "
                            "oversample 8, 2 power iterations, 2 refinement iterations, group-64 INT4 residual",
                "N": N, "K": K, "rank": r, "iterations": iters, "parallelism": "single GPU"}

    def cpu(target_s):
        import oracle as O
        threads = _blas_threads()
        om = W.gaussian_sketch(K, l, 0)

        def run(rows):
            t0 = time.perf_counter()
            O.svdq_split(wl.w[:rows], om, r, SPLIT_POWER, SPLIT_REFINE, "group64", act_rms=rms_h)
            return time.perf_counter() - t0

        probe = run(512)
        rows = int(min(N, max(512, 512 * target_s / max(probe, 1e-3))) // 16 * 16)
        t = run(rows)
        ops = _split_flops(rows, K, r, l, SPLIT_POWER, iters)
        return {"value": round(ops / t / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
                "sample": f"the oracle's split of the first {rows} of {N} weight rows (same rank, sketch, "
                          f"power and refinement iterations, act-aware, group-64): {t:.2f} s wall on {threads} "
                          f"BLAS threads"}
    c.cpu_fn = cpu
    return c


def case_ffdown(Q, W, dev):
    import torch
    wl = W.ffdown_w8a8()
    M, N, K = wl.M, wl.N, wl.K
    x, w = _bf16_dev(wl.x, dev), _bf16_dev(wl.w, dev)
    res, gate = _bf16_dev(wl.residual, dev), _bf16_dev(wl.gate, dev)
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    sa = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    sw = torch.empty((N,), dtype=torch.float32, device=dev)
    c = Case()
    c.prep_ms = _timed_prep(lambda: Q.rotate_quantize_act(w, bits=8, scale_mode="row", codes=wq,
                                                          scales=sw))
    c.launches = [
        ("prologue", lambda: Q.rotate_quantize_act(x, bits=8, scale_mode="row", codes=codes, scales=sa)),
        ("gemm", lambda: Q.qgemm_w8a8(codes, sa, wq, sw, residual=res, gate=gate,
                                      epilogue="gated_residual", out=out)),
    ]
    c.ops = wl.int_ops
    c.gemm_launches = 1
    c.pro_bytes = M * K * 2 + M * K + M * 4
    c.gemm_bytes = M * K + N * K + M * 4 + N * 4 + N * 2 + 2 * M * N * 2
    c.metric = ("effective int TOPS + % int8 MFMA peak, W8A8 rotated GEMM + gated residual "
                "M=4096 K=20480 N=5120")
    c.dtype = "int8 MFMA, int32 accumulate, bf16 out"
    c.config = {"workload": "W8A8 protected ff.down: X bf16 [4096x20480] = silu(a)*b, W int8 per-row "
                            "[5120x20480], group-256 Hadamard, per-token int8, gated residual onto "
                            "bf16 [4096x5120]",
                "M": M, "N": N, "K": K, "global_batch": M, "parallelism": "single GPU"}
    c.wl = wl
    return c


def case_svdq(Q, W, dev, fp6=False):
    """The SVDQuant gate|up layer; fp6: the same codes in the FP6 e2m3 layout
    on the FP6 matrix instruction, one instruction per 64-channel group."""
    import torch
    wl = W.svdq_gateup()
    M, N, K = wl.M, wl.N, wl.K
    r = wl.l1.shape[1]
    x, w = _bf16_dev(wl.x, dev), _bf16_dev(wl.w, dev)
    l1, l2 = _bf16_dev(wl.l1, dev), _bf16_dev(np.ascontiguousarray(wl.l2.T), dev)  # L2 transposed, [N, r]
    acols, wcols = (K // 4 * 3, K // 4 * 3) if fp6 else (K, K // 2)
    codes = torch.empty((M, acols), dtype=torch.uint8 if fp6 else torch.int8, device=dev)
    sa = torch.empty((K // 64, M), dtype=torch.float32, device=dev).t()  # group-major group-64 scales
    lr = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
    wq = torch.empty((N, wcols), dtype=torch.uint8, device=dev)
    sw = torch.empty((K // 64, N), dtype=torch.float32, device=dev).t()
    layout = "fp6" if fp6 else "i8"
    pack = Q.pack_weight_fp6 if fp6 else Q.pack_weight_int4
    c = Case()
    c.prep_ms = _timed_prep(lambda: pack(w, scale_mode="group64", packed=wq, scales=sw))
    c.launches = [
        ("prologue", lambda: Q.rotate_quantize_act(x, bits=4, scale_mode="group64", layout=layout, codes=codes,
                                                   scales=sa, l1=l1, lr=lr)),
        ("gemm", (lambda: Q.qgemm_w4a4_fp6_lowrank(codes, sa, wq, sw, K, lr=lr, l2=l2, epilogue="swiglu",
                                                   out=out)) if fp6 else
                 (lambda: Q.qgemm_w4a4_lowrank(codes, sa, wq, sw, K, lr=lr, l2=l2, epilogue="swiglu", out=out))),
    ]
    out0 = torch.empty_like(out)
    c.branch = (
        lambda: Q.rotate_quantize_act(x, bits=4, scale_mode="group64", layout=layout, codes=codes, scales=sa),
        (lambda: Q.qgemm_w4a4_fp6_lowrank(codes, sa, wq, sw, K, epilogue="swiglu", out=out0)) if fp6 else
        (lambda: Q.qgemm_w4a4_lowrank(codes, sa, wq, sw, K, epilogue="swiglu", out=out0)))
    c.ops = wl.int_ops
    c.gemm_launches = 1
    # the rescale of every output and 64-channel group: convert the int32
    # partial, form s_a * s_w, fma (3); the FP6 instruction's partial is
    # already fp32 (2)
    c.valu_ops = M * N * (K // 64) * (2 if fp6 else 3)
    c.pro_bytes = M * K * 2 + K * r * 2 + M * acols + M * (K // 64) * 4 + M * r * 2
    c.gemm_bytes = (M * acols + N * wcols + M * (K // 64) * 4 + N * (K // 64) * 4 + M * r * 2
                    + r * N * 2 + M * (N // 2) * 2)
    if fp6:
        c.metric = ("effective int TOPS, group-64 W4A4 GEMM + rank-32 low-rank + SwiGLU M=4096 K=5120 N=40960 "
                    "on the FP6 matrix instruction (experiment)")
        c.dtype = "fp6 e2m3 MFMA (exact int4 codes), exact fp32 per-64 partials, fp32 rescale, bf16 out"
        c.peak = FP6_MFMA_PEAK_TOPS
    else:
        c.metric = ("effective int TOPS + % int8 MFMA peak, group-64 W4A4 GEMM + rank-32 low-rank + SwiGLU "
                    "M=4096 K=5120 N=40960")
        c.dtype = "int8 MFMA (int4 codes), int32 per-64 partials, fp32 rescale, bf16 out"
    c.config = {"workload": "SVDQuant fused gate|up: X bf16 [4096x5120], W int4 group-64 [40960x5120]"
                            + (" stored as FP6 e2m3" if fp6 else "")
                            + ", bf16 rank-32 L1 [5120x32] / L2 [32x40960], SwiGLU -> bf16 [4096x20480]",
                "M": M, "N": N, "K": K, "rank": r, "global_batch": M, "parallelism": "single GPU"}
    c.wl = wl
    return c


def case_stack(Q, W, dev, fp6=False):
    """224 linears of the 28-block stack at 2048^2.  Activations for every
    layer are drawn on the device (torch generator seeded 2l+1, N(0,1)) and
    kept resident; weights (seeded 2l, N(0,0.02)) are prepared offline and the
    bf16 copies freed.  One codes buffer and one output buffer are reused.
    fp6: the 128 W4A4 layers hold the same INT4 codes in the FP6 layout and
    run on the FP6 matrix instruction (same outputs bit for bit)."""
    import torch
    M = 16384
    layers = W.stack_layers()
    g = torch.Generator(device=dev)
    maxk = max(k for _, _, _, k, _ in layers)
    maxn = max(n for _, _, n, _, _ in layers)
    codes = torch.empty((M * maxk,), dtype=torch.int8, device=dev)
    codes6 = torch.empty((M * maxk // 4 * 3,), dtype=torch.uint8, device=dev) if fp6 else None
    sa = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M * maxn,), dtype=torch.bfloat16, device=dev)
    c = Case()
    prep = 0.0
    n4 = 0
    for li, (b, name, n, k, bits) in enumerate(layers):
        g.manual_seed(2 * li)
        w = (torch.randn((n, k), generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        g.manual_seed(2 * li + 1)
        x = torch.randn((M, k), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        sw = torch.empty((n,), dtype=torch.float32, device=dev)
        cd = codes[: M * k].view(M, k)
        o = out[: M * n].view(M, n)
        if bits == 4 and fp6:
            wq = torch.empty((n, k // 4 * 3), dtype=torch.uint8, device=dev)
            c6 = codes6[: M * k // 4 * 3].view(M, k // 4 * 3)
            prep += _timed_prep(lambda: Q.pack_weight_fp6(w, packed=wq, scales=sw))
            c.launches.append(("prologue", lambda x=x, c6=c6: Q.rotate_quantize_act(
                x, bits=4, scale_mode="row", layout="fp6", codes=c6, scales=sa)))
            c.launches.append(("gemm", lambda c6=c6, wq=wq, sw=sw, o=o, k=k: Q.qgemm_w4a4_fp6(
                c6, sa, wq, sw, k, out=o)))
            c.gemm_bytes += (M + n) * k // 4 * 3
            n4 += 1
        elif bits == 4:
            wq = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
            prep += _timed_prep(lambda: Q.pack_weight_int4(w, packed=wq, scales=sw))
            c.launches.append(("prologue", lambda x=x, cd=cd: Q.rotate_quantize_act(
                x, bits=4, scale_mode="row", codes=cd, scales=sa)))
            c.launches.append(("gemm", lambda cd=cd, wq=wq, sw=sw, o=o, k=k: Q.qgemm_w4a4(
                cd, sa, wq, sw, k, out=o)))
            c.gemm_bytes += M * k + n * k // 2
            n4 += 1
        else:
            wq = torch.empty((n, k), dtype=torch.int8, device=dev)
            prep += _timed_prep(lambda: Q.rotate_quantize_act(w, bits=8, scale_mode="row", codes=wq,
                                                              scales=sw))
            c.launches.append(("prologue", lambda x=x, cd=cd: Q.rotate_quantize_act(
                x, bits=8, scale_mode="row", codes=cd, scales=sa)))
            c.launches.append(("gemm", lambda cd=cd, wq=wq, sw=sw, o=o: Q.qgemm_w8a8(
                cd, sa, wq, sw, out=o)))
            c.gemm_bytes += M * k + n * k
        del w
        c.ops += 2 * M * n * k
        c.pro_bytes += M * k * 2 + M * k + M * 4
        c.gemm_bytes += M * 4 + n * 4 + M * n * 2
        c.gemm_launches += 1
    torch.cuda.synchronize()
    c.prep_ms = prep
    c.metric = ("effective int TOPS + % int8 MFMA peak, mixed 224-linear DiT stack at 2048^2 "
                "(16384 tokens, 128 W4A4 + 96 W8A8)" + (", W4A4 layers on the FP6 instruction" if fp6 else ""))
    c.dtype = ("FP6 e2m3 MFMA (exact int4 codes) for W4A4, int8 MFMA for W8A8, bf16 out" if fp6 else
               "int8 MFMA (int4/int8 codes), int32 accumulate, bf16 out")
    c.config = {"workload": "28-block DiT linear stack at 2048^2: 16384 tokens, d=5120, ffn=20480, "
                            f"{len(layers)} linears ({n4} W4A4, {len(layers) - n4} W8A8), per-token / "
                            "per-row scales, group-256 Hadamard, bf16 out, every activation resident"
                            + ("; W4A4 codes in the FP6 layout on the FP6 instruction" if fp6 else ""),
                "M": M, "layers": len(layers), "global_batch": M, "parallelism": "single GPU"}
    return c


def case_stack_fused(Q, W, dev, grouped=False, fp6=False):
    """The stack's 224 linears (same weights) as a DiT block runs them when
    the block's RMSNorm + modulation live in the quantization prologue and one
    prepared activation serves every projection of the same input (model card
    "Krea 2 Turbo OrbitQuant W4A4", section "Fused transformer (OrbitQuant
    0.11)").  Per block, four resident inputs (torch generator, N(0,1)):
    the attention input (seed of wq's input), the wo input, the MLP input and
    the down input (seeds of wo's, mlp_gate's and mlp_down's inputs); the
    attention and MLP inputs go through rmsnorm_rotate_quantize_act with
    synthetic adaLN vectors (gamma ~ 1 + 0.1 N, scale ~ 0.2 N, shift ~ 0.1 N,
    seeds 10^7 + 8 b + i).  The attention input is prepared once as int4
    codes (wq, attn_gate) and once as int8 codes (wk, wv); the MLP input once
    (mlp_gate, mlp_up).  grouped: the block's Q|K|V|gate projections run as
    one grouped launch (sigmoid on the gate) and gate|up as another.  fp6:
    the W4A4 layers' codes in the FP6 layout on the FP6 instruction (same
    outputs bit for bit; separate launches)."""
    import torch
    M = 16384
    layers = W.stack_layers()
    g = torch.Generator(device=dev)
    maxk = max(k for _, _, _, k, _ in layers)
    maxn = max(n for _, _, n, _, _ in layers)
    assert not (fp6 and grouped), "the grouped GEMM takes int8-MFMA operands"
    codes = {4: torch.empty((M * maxk // 4 * 3 if fp6 else M * maxk,), dtype=torch.uint8 if fp6 else torch.int8,
                            device=dev),
             8: torch.empty((M * maxk,), dtype=torch.int8, device=dev)}
    sa = {4: torch.empty((M,), dtype=torch.float32, device=dev),
          8: torch.empty((M,), dtype=torch.float32, device=dev)}
    # grouped launches write every segment at once: room for gate|up side by side
    out = torch.empty((M * maxn * (2 if grouped else 1),), dtype=torch.bfloat16, device=dev)
    c = Case()
    prep = 0.0
    n4 = 0
    names = [nm for nm, _, _ in W.STACK_BLOCK]

    def rnd(seed, shape, std=1.0, mean=0.0):
        g.manual_seed(seed)
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std + mean).to(torch.bfloat16)

    def prologue(x, bits, norm):
        f6 = fp6 and bits == 4
        kc = x.shape[1] // 4 * 3 if f6 else x.shape[1]
        cd = codes[bits][: M * kc].view(M, kc)
        lay = "fp6" if f6 else "i8"
        if norm is None:
            fn = lambda: Q.rotate_quantize_act(x, bits=bits, scale_mode="row", layout=lay, codes=cd,
                                               scales=sa[bits])
        else:
            fn = lambda: Q.rmsnorm_rotate_quantize_act(x, *norm, eps=1e-6, bits=bits, scale_mode="row",
                                                       layout=lay, codes=cd, scales=sa[bits])
        c.launches.append(("prologue", fn))
        c.pro_bytes += M * x.shape[1] * 3 + M * 4

    for b in range(W.STACK_BLOCKS):
        base = 8 * b
        x_attn = rnd(2 * (base + names.index("wq")) + 1, (M, 5120))
        x_o = rnd(2 * (base + names.index("wo")) + 1, (M, 6144))
        x_mlp = rnd(2 * (base + names.index("mlp_gate")) + 1, (M, 5120))
        x_down = rnd(2 * (base + names.index("mlp_down")) + 1, (M, 20480))
        norm_attn = (rnd(10 ** 7 + base, (5120,), 0.1, 1.0), rnd(10 ** 7 + base + 1, (5120,), 0.2),
                     rnd(10 ** 7 + base + 2, (5120,), 0.1))
        norm_mlp = (rnd(10 ** 7 + base + 3, (5120,), 0.1, 1.0), rnd(10 ** 7 + base + 4, (5120,), 0.2),
                    rnd(10 ** 7 + base + 5, (5120,), 0.1))
        # prepared weights of the block's 8 linears (the stack's seeds and preparation)
        lw = {}
        for i, (name, n, k) in enumerate(W.STACK_BLOCK):
            li = base + i
            bits = W.stack_precision(b, name)
            w = rnd(2 * li, (n, k), 0.02)
            sw = torch.empty((n,), dtype=torch.float32, device=dev)
            if bits == 4 and fp6:
                wq = torch.empty((n, k // 4 * 3), dtype=torch.uint8, device=dev)
                prep += _timed_prep(lambda: Q.pack_weight_fp6(w, packed=wq, scales=sw))
                n4 += 1
            elif bits == 4:
                wq = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
                prep += _timed_prep(lambda: Q.pack_weight_int4(w, packed=wq, scales=sw))
                n4 += 1
            else:
                wq = torch.empty((n, k), dtype=torch.int8, device=dev)
                prep += _timed_prep(lambda: Q.rotate_quantize_act(w, bits=8, scale_mode="row", codes=wq,
                                                                  scales=sw))
            del w
            lw[name] = (wq, sw, n, k, bits)

        def gemm(name):
            wq, sw, n, k, bits = lw[name]
            o = out[: M * n].view(M, n)
            if bits == 4 and fp6:
                c6 = codes[4][: M * k // 4 * 3].view(M, k // 4 * 3)
                c.launches.append(("gemm", lambda: Q.qgemm_w4a4_fp6(c6, sa[4], wq, sw, k, out=o)))
                c.ops += 2 * M * n * k
                c.gemm_bytes += (M + n) * k // 4 * 3 + M * 4 + n * 4 + M * n * 2  # FP6: 3/4 byte per code
                c.gemm_launches += 1
                return
            cd = codes[bits][: M * k].view(M, k)
            if bits == 4:
                fn = lambda: Q.qgemm_w4a4(cd, sa[4], wq, sw, k, out=o)
                c.gemm_bytes += n * k // 2
            else:
                fn = lambda: Q.qgemm_w8a8(cd, sa[8], wq, sw, out=o)
                c.gemm_bytes += n * k
            c.launches.append(("gemm", fn))
            c.ops += 2 * M * n * k
            c.gemm_bytes += M * k + M * 4 + n * 4 + M * n * 2
            c.gemm_launches += 1

        def grouped_gemm(parts):
            segs, off = [], 0
            for name, epi in parts:
                wq, sw, n, k, bits = lw[name]
                o = out[off: off + M * n].view(M, n)
                off += M * n
                segs.append(dict(w=wq, sw=sw, bits=bits, epilogue=epi, out=o))
                c.ops += 2 * M * n * k
                c.gemm_bytes += (n * k // 2 if bits == 4 else n * k) + n * 4 + M * n * 2
            k = lw[parts[0][0]][3]
            bits_used = {lw[nm][4] for nm, _ in parts}
            c.gemm_bytes += sum(M * k + M * 4 for _ in bits_used)
            a4 = codes[4][: M * k].view(M, k) if 4 in bits_used else None
            a8 = codes[8][: M * k].view(M, k) if 8 in bits_used else None
            c.launches.append(("gemm", lambda: Q.qgemm_grouped(a4, sa[4] if a4 is not None else None, a8,
                                                               sa[8] if a8 is not None else None, k, segs)))
            c.gemm_launches += 1

        if grouped:
            prologue(x_attn, 4, norm_attn)
            prologue(x_attn, 8, norm_attn)
            grouped_gemm([("wq", "bf16"), ("wk", "bf16"), ("wv", "bf16"), ("attn_gate", "sigmoid")])
        else:
            prologue(x_attn, 4, norm_attn)
            gemm("wq")
            gemm("attn_gate")
            prologue(x_attn, 8, norm_attn)
            gemm("wk")
            gemm("wv")
        prologue(x_o, lw["wo"][4], None)
        gemm("wo")
        prologue(x_mlp, 4, norm_mlp)
        if grouped:
            grouped_gemm([("mlp_gate", "bf16"), ("mlp_up", "bf16")])
        else:
            gemm("mlp_gate")
            gemm("mlp_up")
        prologue(x_down, lw["mlp_down"][4], None)
        gemm("mlp_down")
    torch.cuda.synchronize()
    c.prep_ms = prep
    c.metric = ("effective int TOPS + % int8 MFMA peak, mixed 224-linear DiT stack at 2048^2 "
                "(16384 tokens, 128 W4A4 + 96 W8A8), norm fused + prepared activations reused"
                + (" + grouped Q|K|V|gate and gate|up GEMMs" if grouped else "")
                + (", W4A4 layers on the FP6 instruction" if fp6 else ""))
    c.dtype = ("FP6 e2m3 MFMA (exact int4 codes) for W4A4, int8 MFMA for W8A8, bf16 out" if fp6 else
               "int8 MFMA (int4/int8 codes), int32 accumulate, bf16 out")
    c.config = {"workload": "28-block DiT linear stack at 2048^2: 16384 tokens, d=5120, ffn=20480, "
                            f"{len(layers)} linears ({n4} W4A4, {len(layers) - n4} W8A8), per-token / "
                            "per-row scales, group-256 Hadamard, bf16 out; RMSNorm + adaLN modulation fused "
                            "into the attention and MLP prologues, one prepared activation per shared input "
                            "and precision (5 prologues per block)"
                            + ("; Q|K|V|gate (sigmoid gate, K/V INT8) and gate|up as grouped launches "
                               "(4 GEMM launches per block)" if grouped else "")
                            + ("; W4A4 codes in the FP6 layout on the FP6 instruction" if fp6 else "")
                            + ", every input resident",
                "M": M, "layers": len(layers), "prologues": 5 * W.STACK_BLOCKS, "global_batch": M,
                "parallelism": "single GPU"}
    return c


CASES = {"attn_proj_w4a4": case_attn, "attn_proj_w4a4_fp6": case_attn_fp6, "svdq_split_gateup": case_svdq_split,
         "attn_proj_mxfp4": lambda Q, W, dev: case_attn_mx(Q, W, dev, "fp4"),
         "attn_proj_mxfp8": lambda Q, W, dev: case_attn_mx(Q, W, dev, "fp8"),
         "svdq_gateup_mxfp4": case_svdq_mx,
         "ffdown_w8a8": case_ffdown, "svdq_gateup": case_svdq,
         "svdq_gateup_fp6": lambda Q, W, dev: case_svdq(Q, W, dev, fp6=True),
         "stack": case_stack, "stack_fp6": lambda Q, W, dev: case_stack(Q, W, dev, fp6=True),
         "stack_fused": case_stack_fused,
         "stack_fused_fp6": lambda Q, W, dev: case_stack_fused(Q, W, dev, fp6=True),
         "stack_grouped": lambda Q, W, dev: case_stack_fused(Q, W, dev, grouped=True)}


# ------------------------------------------------------------------- main --
def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_back_to_back(fns, launches=GEMM_LAUNCHES, repeats=GEMM_REPEATS, warm=10):
    """Median over `repeats` of the time per pass of `fns` (a list of
    launches run in order), each repeat `launches` passes back to back
    between two events on the current stream, after `warm` untimed passes.
    Returns (median ms per pass, every repeat's ms per pass)."""
    import torch
    for _ in range(warm):
        for fn in fns:
            fn()
    per = []
    for _ in range(repeats):
        e0, e1 = _events()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(launches):
            for fn in fns:
                fn()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / launches)
    return float(np.median(per)), per


def time_cold(fns, dev, launches=COLD_LAUNCHES):
    """Median time of one pass of `fns` right after a 512 MiB device write
    (more than L2 and the 256 MB MALL hold), events around the pass only."""
    import torch
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    per = []
    for _ in range(launches):
        flush.fill_(1)
        e0, e1 = _events()
        e0.record()
        for fn in fns:
            fn()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    del flush
    return float(np.median(per))


def launch_count(pass_ms, target_ms=50.0):
    """Passes per repeat: GEMM_LAUNCHES, fewer for long passes (a repeat of
    about target_ms, at least 2)."""
    return int(max(2, min(GEMM_LAUNCHES, round(target_ms / max(pass_ms, 1e-6)))))


def gemm_only_record(case, ops, dev, cold=True):
    """GEMM-only figures of a case: back-to-back launches of its GEMMs on
    the codes its prologues left in HBM (median of 5 repeats of 100 passes,
    fewer passes when one pass is long; the stack's 224 GEMMs form one
    pass), and a cold-cache variant for single-GEMM cases."""
    import torch
    fns = [fn for tag, fn in case.launches if tag == "gemm"]
    for tag, fn in case.launches:      # leave valid codes in place
        fn()
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for fn in fns:
        fn()
    e1.record()
    torch.cuda.synchronize()
    passes = launch_count(e0.elapsed_time(e1))
    stack = len(fns) > 8
    ms, reps = time_back_to_back(fns, launches=passes, warm=min(10, passes))
    rec = {"ms": round(ms, 5), "ms_per_launch": round(ms / case.gemm_launches, 5),
           "repeats_ms": [round(v, 5) for v in reps], "passes_per_repeat": passes,
           "tops": round(ops / (ms * 1e-3) / 1e12, 2),
           "gbs": round(case.gemm_bytes / (ms * 1e-3) / 1e9, 1)}
    if case.bound == "mfma":
        rec["pct_int8_peak"] = round(100.0 * ops / (ms * 1e-3) / 1e12 / INT8_MFMA_PEAK_TOPS, 2)
        if case.peak != INT8_MFMA_PEAK_TOPS:
            rec["pct_own_peak"] = round(100.0 * ops / (ms * 1e-3) / 1e12 / case.peak, 2)
    if case.valu_ops:   # VALU-bound group-64 rescale: fraction of the fp32 VALU issue rate
        rec["pct_valu_peak"] = round(100.0 * case.valu_ops / case.gemm_launches / (rec["ms_per_launch"] * 1e-3)
                                     / 1e12 / VALU_PEAK_TOPS, 2)
    if cold and not stack:
        cms = time_cold(fns, dev)
        rec["cold_ms"] = round(cms, 5)
        rec["cold_tops"] = round(ops / (cms * 1e-3) / 1e12, 2)
    return rec


def main(argv=None):
    args = _parse(argv)
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import rotated_bit_quantized_rotate_amd as Q
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if not Q.device_supported(0):
        raise SystemExit("device 0 is not gfx950")

    case = CASES[args.workload](Q, W, dev)
    L = len(case.launches)
    stack = args.workload.startswith("stack")

    def step():
        for _, fn in case.launches:
            fn()

    # ---- warm-up: at least `warmup` steps and at least WARMUP_S seconds
    w, t_w = 0, time.perf_counter()
    while w < args.warmup or time.perf_counter() - t_w < WARMUP_S:
        step()
        w += 1
        if w % (1 if stack else 16) == 0:
            torch.cuda.synchronize()  # keep the host within a few steps of the GPU
    torch.cuda.synchronize()
    warmup_s = time.perf_counter() - t_w

    # ---- timed region: exactly `steps` steps, synchronized on both sides,
    # one event before and one after on the stream the kernels run on (the
    # current torch stream).  This is the step time `value` reports.
    n = args.steps
    e_start, e_end = _events()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record()
    for s in range(n):
        step()
    e_end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    step_ms = e_start.elapsed_time(e_end) / n

    # ---- GEMM-only: back-to-back launches on the prepared codes (the
    # roofline's kernel time), and a cold-cache variant
    ops = float(case.ops)
    gemm = gemm_only_record(case, ops, dev)
    gemm_ms = gemm["ms"]

    # ---- per-kernel breakdown: the `steps` steps again with an event after
    # every launch (each event adds a small gap at the kernel boundary)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(L * n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for s in range(n):
        for i, (_, fn) in enumerate(case.launches):
            fn()
            ev[s * L + i + 1].record()
    torch.cuda.synchronize()
    step_events_ms = ev[0].elapsed_time(ev[L * n]) / n
    t_tag = {"prologue": 0.0, "gemm": 0.0}
    for s in range(n):
        for i, (tag, _) in enumerate(case.launches):
            t_tag[tag] += ev[s * L + i].elapsed_time(ev[s * L + i + 1])
    gemm_ev_ms = t_tag["gemm"] / n
    pro_ev_ms = t_tag["prologue"] / n

    # ---- the step's prologues alone, back to back (median of 5 repeats):
    # their time per step, and the step minus it (the GEMM share of a step)
    pro_fns = [fn for tag, fn in case.launches if tag == "prologue"]
    pro_ms = time_back_to_back(pro_fns, launches=1 if stack else 50, warm=2)[0] if pro_fns else 0.0

    # ---- the step, median of 5 repeats of the same K steps
    step_med_ms = time_back_to_back([step], launches=n, warm=0)[0]

    # ---- the same step replayed from a HIP graph (no host launch cost)
    graph_step_ms = None
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                step()
            for _ in range(2):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = _events()
            e0.record()
            for _ in range(n):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            graph_step_ms = e0.elapsed_time(e1) / n
        except Exception as exc:  # graph capture is an extra figure only
            print(f"graph replay skipped: {exc}", file=sys.stderr)

    # ---- the other single-layer GEMMs, GEMM-only, in the same process
    other = None
    if args.workload == "attn_proj_w4a4" and not args.no_other_gemms:
        other = {}
        for name in ("attn_proj_w4a4_fp6", "ffdown_w8a8", "svdq_gateup", "svdq_gateup_fp6", "attn_proj_mxfp4",
                     "svdq_gateup_mxfp4", "stack", "stack_fp6"):
            oc = CASES[name](Q, W, dev)
            rec = gemm_only_record(oc, float(oc.ops), dev)
            rec["workload"] = oc.config["workload"]
            other[name] = rec
            del oc
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    if args.calib_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    value = ops / (step_ms * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    sub_ms = step_ms - pro_ms
    label = GEMM_KERNELS[args.workload][0]
    traffic = load_traffic(args.workload)
    rec = {
        "metric": case.metric,
        "value": round(value, 2),
        "unit": case.unit,
        "n_gpus": 1,
        "steps": n,
        "warmup": w,
        "warmup_s": round(warmup_s, 3),
        "ms_per_step": round(step_ms, 5),
        "ms_per_step_median5": round(step_med_ms, 5),
        "ms_per_step_with_kernel_events": round(step_events_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": case.config,
        "pct_int8_peak_step": round(100.0 * value / INT8_MFMA_PEAK_TOPS, 2) if case.bound == "mfma" else None,
        "gemm_only": gemm,
        "gemm_step_minus_prologue": {"ms": round(sub_ms, 5), "ms_per_launch": round(sub_ms / case.gemm_launches, 5),
                                     "ms_per_launch_with_kernel_events": round(gemm_ev_ms / case.gemm_launches, 5),
                                     "tops": round(ops / (sub_ms * 1e-3) / 1e12, 2) if sub_ms > 0 else None},
        "prologue": None if pro_ms <= 0 else {
            "ms": round(pro_ms, 5),
            "ms_with_kernel_events": round(pro_ev_ms, 5),
            "gbs": round(case.pro_bytes / (pro_ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * case.pro_bytes / (pro_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
        "graph_step_ms": None if graph_step_ms is None else round(graph_step_ms, 5),
        "graph_step_tops": None if graph_step_ms is None else round(ops / (graph_step_ms * 1e-3) / 1e12, 2),
        "weight_prep_ms": round(case.prep_ms, 5),
        "wall_ms_timed_region": round(wall_ms, 3),
        "roofline": {"bound": case.bound, "kernel": label,
                     "achieved": round(gemm_tops, 2), "peak": case.peak,
                     "unit": case.unit, "frac": round(gemm_tops / case.peak, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": int(case.gemm_bytes // case.gemm_launches),
                     "timing": "GEMM-only: median of 5 repeats of back-to-back launches, HIP events on the "
                               "launch stream"},
    }
    if case.valu_ops:
        # the group-64 rescale bounds these kernels (VALU busy 94 % on INT8 by
        # the counters): the roofline is the fp32 VALU's issue rate
        achieved = case.valu_ops / case.gemm_launches / (gemm["ms_per_launch"] * 1e-3) / 1e12
        rec["roofline"] = {"bound": "alu", "kernel": label,
                           "achieved": round(achieved, 2), "peak": round(VALU_PEAK_TOPS, 2),
                           "unit": "T VALU lane-instructions/s", "frac": round(achieved / VALU_PEAK_TOPS, 4),
                           "valu_ops_per_launch": int(case.valu_ops // case.gemm_launches),
                           "traffic": traffic,
                           "algorithmic_bytes": int(case.gemm_bytes // case.gemm_launches),
                           "timing": rec["roofline"]["timing"],
                           "mfma_frac": rec["roofline"]["frac"]}
    if case.branch is not None:
        # the low-rank branch's share: the prologue and the GEMM timed again
        # without it (same codes, tiles and epilogue), back to back
        pro0_ms = time_back_to_back([case.branch[0]], launches=50, warm=2)[0]
        g0_ms = time_back_to_back([case.branch[1]], launches=gemm["passes_per_repeat"],
                                  warm=min(10, gemm["passes_per_repeat"]))[0]
        down, up = pro_ms - pro0_ms, gemm["ms"] - g0_ms
        rec["lowrank_branch"] = {
            "down_ms": round(down, 5), "up_ms": round(up, 5),
            "prologue_without_ms": round(pro0_ms, 5), "gemm_without_ms": round(g0_ms, 5),
            "pct_of_step": round(100.0 * (down + up) / step_ms, 2),
            "method": "X @ L1: prologue with it minus without; lr @ L2: GEMM with it minus without "
                      "(medians of back-to-back launches)"}
    if other is not None:
        rec["other_gemms"] = other
    if not args.no_cpu_baseline and case.cpu_fn is not None:
        rec["cpu_baseline"] = case.cpu_fn(args.cpu_seconds)
    elif not args.no_cpu_baseline and case.wl is not None:
        rec["cpu_baseline"] = cpu_baseline(case.wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
