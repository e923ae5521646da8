"""Build libqlinear.so (HIP kernels + C ABI) in-tree for gfx950.

    python -m rotated_bit_quantized_rotate_amd.build      # or build() from Python

Each .hip file under csrc/ is compiled with hipcc for --offload-arch=gfx950
into _build/, then linked into rotated_bit_quantized_rotate_amd/libqlinear.so.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libqlinear.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["qlinear_api.hip", "rotate_quant.hip", "mx_quant.hip", "qgemm_pipe.hip", "svdq_split.hip"]

# Packed-FP32 VALU forms are disabled for device code; the host pass warns
# that it does not know the feature, which is harmless.
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    h = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return h


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines()
                    if "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link libqlinear.so.
    Always recompiles.  Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2) // 2))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    _check_stubs(tmp)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _check_stubs(lib: str) -> None:
    """Fail if a kernel's host launch stub is referenced but not defined:
    the host compilation pass can drop a kernel template it fails to
    instantiate without an error, which would only show up when the library
    is loaded."""
    nm = shutil.which("nm") or "/usr/bin/nm"
    r = subprocess.run([nm, "-u", lib], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        raise RuntimeError(f"{len(missing)} kernel launch stubs are undefined in {lib}, e.g. {missing[0]}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
