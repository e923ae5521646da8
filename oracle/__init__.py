"""CPU oracle for the rotated low-bit quantized linear -- TEST INFRASTRUCTURE.

Only the test suite, the package's smoke entry and the benchmark's CPU
baseline leg may import this package.  The library (HIP kernels behind the C
ABI and its Python binding) never imports, links or calls anything here, and
this package imports nothing from the library: the two share no code.  The
seeded input generators live in their own module (``workloads``) and hold none
of the method's arithmetic.

The oracle is plain NumPy: bf16 inputs are widened exactly to float64, the
rotation is an explicit matrix product with the closed-form 256x256 regular
Hadamard matrix, the integer contraction is exact, and the epilogues run in
float64 before one round-to-nearest-even cast to bfloat16.  The quantization
follows its definition in float64: absmax of the exactly rotated values,
scale = absmax / qmax rounded once to float32, code = round-half-even of
x' * qmax / absmax.

Sources (web pages; cited by title and section):
  [OrbitQuant]  model card "Krea 2 Turbo OrbitQuant W4A4" -- sections
                "Fused transformer (OrbitQuant 0.11)", "What is quantized",
                "Latency and VRAM".
  [INT4-mixed]  model card "Krea-2 Turbo -- INT4 tensorwise W4A4 (+ConvRot,
                mixed int8 fallback)" -- introduction.
  [SVDQ-Comfy]  README "Krea-2-SVDQuant-ComfyUI" -- sections "Why this
                exists", "Low-rank refinement", "LoRA".
  [NunchakuLite] model card "Krea 2 Turbo Nunchaku Lite INT4 r32" -- intro.
  [lab]         research log "lab" -- Studies 1-4.

The offline low-rank split (svdq_split_ref) follows [SVDQ-Comfy], sections on
reproducible builds, "Activation-aware branch" and "Low-rank refinement, and
what the objective actually is"; its randomized SVD is Halko, Martinsson and
Tropp's randomized subspace iteration (2011).

The MX block-scaled variant (mx_ref) stands in for the NVFP4 build of
[NunchakuLite] "Benchmark" and the mxfp8 build of [lab] Study 1; the block
formats follow the OCP Microscaling Formats (MX) Specification v1.0.

Parity status of each function is pinned by the ``-m "not gpu"`` tests:
closed forms and Kronecker construction (Hadamard), involution (rotation),
error bounds and ties (quantizer), documented byte example (packing),
brute-force integer loops (GEMM), grid-exact end-to-end reconstruction
(whole linear), the low-rank identity, textbook SiLU values, and for the
fused RMSNorm + modulation prologue closed forms (unit mean square, eps
inside the root), scale invariance, a worked modulation example, brute-force
loops and the reduction to the plain prologue when the norm is the identity, and for the
FP6 (e2m3) code layout the format's constants, hand-derived bit patterns, a
worked packing example and exact float32 summation at the largest K; for the
low-rank split the weight normalization in closed form, exact recovery of low-rank
matrices, agreement with the full SVD under fast spectral decay, the plain split
rebuilt from a full SVD, best-kept refinement, zero and scale-invariance cases; for the MX
formats the element tables decoded from the bit fields, E4M3 rounding against torch's
float8_e4m3fn cast, hand-worked blocks, the block error bound and exact rational
products on tiny inputs.  No function
here is "parity unpinned".
"""

from .qlinear_ref import *  # noqa: F401,F403
from .qlinear_ref import __all__ as _q_all
from .svdq_split_ref import *  # noqa: F401,F403
from .svdq_split_ref import __all__ as _s_all
from .mx_ref import *  # noqa: F401,F403
from .mx_ref import __all__ as _m_all

__all__ = list(_q_all) + list(_s_all) + list(_m_all)
