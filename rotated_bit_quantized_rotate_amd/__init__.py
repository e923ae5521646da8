"""Rotated low-bit quantized linear for AMD MI355X (gfx950).

The computation lives in libqlinear.so (hand-written HIP kernels behind the C
ABI declared in include/qlinear.h); this package is its thin Python binding
(``_lib``) plus the in-tree build script (``build``).
"""

from ._lib import (  # noqa: F401
    QLinearError,
    device_supported,
    group64_scales,
    lib,
    pack_weight_fp6,
    pack_weight_int4,
    qgemm_grouped,
    qgemm_mx,
    qgemm_mx_lowrank,
    qgemm_w4a4,
    qgemm_w4a4_fp6,
    qgemm_w4a4_fp6_lowrank,
    qgemm_w4a4_lowrank,
    qgemm_w8a8,
    rmsnorm_rotate_quantize_act,
    rotate_quantize_act,
    rotate_quantize_mx,
    status_string,
    svdq_split,
    svdq_split_noalloc,
    svdq_split_noalloc_max_bytes,
    svdq_split_workspace_bytes,
)
