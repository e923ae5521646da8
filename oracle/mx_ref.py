"""Reference (oracle) implementation of the MX block-scaled rotated linear.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the pages say.  Model card "Krea 2 Turbo Nunchaku Lite INT4 r32",
section "Benchmark": next to the INT4 build stands an NVFP4 build (4-bit
floating-point weights and activations with small-block scales) that runs
faster on GPUs with native FP4 matrix hardware; research log "lab", Study 1
and Study 2: an mxfp8 build (8-bit floats with block scales) measured next to
the INT8 rotation build.  The pages name the formats but do not define them.

What is computed here.  The block formats come from the Open Compute
Project's "OCP Microscaling Formats (MX) Specification", version 1.0: a block
of 32 consecutive elements along K shares one scale X = 2^e stored as an
E8M0 byte (e + 127, e in [-127, 127]); elements are FP4 E2M1 (MXFP4) or
FP8 E4M3 (MXFP8).  Converting a block V of wider values: e = floor(log2
max|V|) - emax_elem (emax_elem = 2 for E2M1, 8 for E4M3), clamped to the
E8M0 range, and each element is V_i / X rounded to the nearest value of the
element format, ties to the even code, saturating at the largest finite
magnitude (6 for E2M1, 448 for E4M3).  NVFP4 (16-element blocks, E4M3
scales) has no matrix instruction on gfx950; MXFP4 is the block-scaled FP4
that the hardware multiplies natively, so it stands in for the pages' NVFP4
build.  The rotation is the same group-256 regular Hadamard as the integer
path (optional).

Readings where the definition leaves a choice open:
  * an all-zero block gets e = -127 (E8M0 byte 0) and zero elements;
  * a zero element (also a negative value that rounds to zero) is stored as
    the +0 pattern;
  * the product of two MX operands is sum_b 2^(ea_b + ew_b) * sum_{k in b}
    Pa_k Pw_k over the K/32 blocks (the dot product of the MX definition),
    formed here exactly up to the final float64 additions.

Notation: X activations [M, K], W weights [N, K]; y = X W^T [M, N].
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from .qlinear_ref import bf16_bits_to_f64, epilogue, f64_to_bf16_bits, rotate

__all__ = [
    "MX_BLOCK", "MX_FORMATS", "MXFormat", "MXResult",
    "mx_element_magnitudes", "mx_round_element", "mx_shared_exponent", "mx_ratio",
    "mx_quantize", "mx_dequantize", "mx_pack", "mx_unpack",
    "mx_gemm", "mx_gemm_exact", "quantize_mx", "mx_linear",
]

MX_BLOCK = 32          # elements per shared scale
E8M0_MIN, E8M0_MAX = -127, 127


class MXFormat:
    """An element format: sign, `ebits` exponent bits with `bias`, `mbits`
    mantissa bits, subnormals at exponent field 0.  `maxcode` is the largest
    magnitude code of a finite value (E4M3 keeps no infinities and uses only
    its all-ones pattern for NaN)."""

    def __init__(self, name, ebits, mbits, bias, maxcode):
        self.name, self.ebits, self.mbits, self.bias, self.maxcode = name, ebits, mbits, bias, maxcode
        self.width = 1 + ebits + mbits
        self.sign_bit = 1 << (ebits + mbits)

    @property
    def emax(self) -> int:
        """Exponent of the largest normal binade."""
        return (self.maxcode >> self.mbits) - self.bias

    @property
    def max_value(self) -> float:
        return float(mx_element_magnitudes(self)[-1])


MX_FORMATS = {
    "fp4": MXFormat("e2m1", ebits=2, mbits=1, bias=1, maxcode=0b111),
    "fp8": MXFormat("e4m3", ebits=4, mbits=3, bias=7, maxcode=0b1111110),
}


def _fmt(fmt) -> MXFormat:
    return MX_FORMATS[fmt] if isinstance(fmt, str) else fmt


def mx_element_magnitudes(fmt) -> np.ndarray:
    """Magnitudes of magnitude codes 0 .. maxcode, decoded from the bit
    fields: exponent field E, mantissa field m; E = 0 is subnormal,
    m / 2^mbits * 2^(1 - bias); otherwise (1 + m / 2^mbits) * 2^(E - bias).
    Increasing in the code."""
    f = _fmt(fmt)
    out = []
    for c in range(f.maxcode + 1):
        E, m = c >> f.mbits, c & ((1 << f.mbits) - 1)
        if E == 0:
            out.append(m / (1 << f.mbits) * 2.0 ** (1 - f.bias))
        else:
            out.append((1 + m / (1 << f.mbits)) * 2.0 ** (E - f.bias))
    return np.array(out, dtype=np.float64)


def mx_round_element(v, fmt) -> np.ndarray:
    """Round float64 values v (already divided by the block scale) to the
    element format: nearest magnitude, a tie to the even magnitude code,
    magnitudes at or beyond the largest finite value saturate to it.
    Returns the element bit patterns (uint8; sign in the top bit of the
    element, +0 for every zero)."""
    f = _fmt(fmt)
    grid = mx_element_magnitudes(f)
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    # lo: largest grid index with grid[lo] <= a (a >= 0 = grid[0])
    lo = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, f.maxcode)
    hi = np.minimum(lo + 1, f.maxcode)
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    up = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    mag = np.where(up & (hi > lo), hi, lo)
    mag = np.where(a >= grid[-1], f.maxcode, mag)           # saturation
    sign = (v < 0) & (mag > 0)
    return (mag + sign * f.sign_bit).astype(np.uint8)


def _element_value(codes, fmt) -> np.ndarray:
    f = _fmt(fmt)
    codes = np.asarray(codes, dtype=np.int64)
    mag = mx_element_magnitudes(f)[codes & (f.sign_bit - 1)]
    return np.where(codes & f.sign_bit, -mag, mag)


def mx_shared_exponent(amax, fmt) -> np.ndarray:
    """e = floor(log2 amax) - emax_elem, clamped to [-127, 127]; -127 for an
    all-zero block.  floor(log2 amax) is read off the float64 exponent
    exactly (frexp: amax = m 2^k with 1/2 <= m < 1, so it is k - 1)."""
    f = _fmt(fmt)
    amax = np.asarray(amax, dtype=np.float64)
    _, k = np.frexp(amax)
    e = (k.astype(np.int64) - 1) - f.emax
    e = np.where(amax > 0, e, E8M0_MIN)
    return np.clip(e, E8M0_MIN, E8M0_MAX).astype(np.int64)


def _blocks(x: np.ndarray) -> np.ndarray:
    R, K = x.shape
    if K % MX_BLOCK:
        raise ValueError(f"MX blocks need K % {MX_BLOCK} == 0, got K={K}")
    return x.reshape(R, K // MX_BLOCK, MX_BLOCK)


def mx_ratio(x: np.ndarray, fmt) -> np.ndarray:
    """V / X for every element of x [R, K] (float64, exact: X is a power of
    two): the value that mx_round_element rounds."""
    xb = _blocks(np.asarray(x, dtype=np.float64))
    e = mx_shared_exponent(np.abs(xb).max(axis=2), fmt)
    return np.ldexp(xb, -e[:, :, None]).reshape(x.shape)


class MXResult:
    """One MX-quantized operand: element bit patterns [R, K] (uint8), block
    exponents [R, K/32] (int64), the format name, and the pre-quantization
    float64 values (after the rotation, if any)."""

    def __init__(self, codes, exps, fmt, values):
        self.codes, self.exps, self.fmt, self.values = codes, exps, fmt, values

    def elements(self) -> np.ndarray:
        """Signed element values (before the block scale), float64."""
        return _element_value(self.codes, self.fmt)

    def dequant(self) -> np.ndarray:
        return mx_dequantize(self.codes, self.exps, self.fmt)


def mx_quantize(x: np.ndarray, fmt) -> MXResult:
    """Block-quantize x [R, K] (float64) to MX: per 32-element block along K,
    the shared exponent from the block's absolute maximum, then every
    element V / 2^e rounded to the element format."""
    x = np.asarray(x, dtype=np.float64)
    xb = _blocks(x)
    e = mx_shared_exponent(np.abs(xb).max(axis=2), fmt)
    codes = mx_round_element(np.ldexp(xb, -e[:, :, None]), fmt).reshape(x.shape)
    return MXResult(codes, e, fmt if isinstance(fmt, str) else fmt.name, x)


def mx_dequantize(codes, exps, fmt) -> np.ndarray:
    codes = np.asarray(codes)
    R, K = codes.shape
    vals = _element_value(codes, fmt).reshape(R, K // MX_BLOCK, MX_BLOCK)
    return np.ldexp(vals, np.asarray(exps, np.int64)[:, :, None]).reshape(R, K)


def mx_pack(q: MXResult):
    """Storage layout: element bytes (FP8: one byte per element; FP4: element
    2i in the low nibble and 2i + 1 in the high nibble of byte i) and the
    E8M0 scale bytes e + 127, row-major [R, K/32]."""
    f = _fmt(q.fmt)
    c = np.asarray(q.codes, np.uint8)
    if f.width == 4:
        data = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    else:
        data = c.copy()
    return data, (np.asarray(q.exps) + 127).astype(np.uint8)


def mx_unpack(data, scale_bytes, fmt):
    """Inverse of mx_pack: (codes [R, K], exps [R, K/32])."""
    f = _fmt(fmt)
    data = np.asarray(data, np.uint8)
    if f.width == 4:
        R, H = data.shape
        codes = np.empty((R, 2 * H), np.uint8)
        codes[:, 0::2] = data & 0xF
        codes[:, 1::2] = data >> 4
    else:
        codes = data.copy()
    return codes, np.asarray(scale_bytes, np.int64) - 127


def mx_gemm(qa: MXResult, qw: MXResult) -> np.ndarray:
    """y[m, n] = sum_b 2^(ea[m,b] + ew[n,b]) * sum_{k in block b} Pa[m,k] Pw[n,k].
    Each block's element dot product is exact in float64 (products of
    E2M1 / E4M3 values have at most 8 significant bits, 32 of them sum
    exactly), and so is its power-of-two scaling; only the additions over
    the K/32 blocks round (in float64)."""
    pa = _blocks(qa.elements())
    pw = _blocks(qw.elements())
    M, NB, _ = pa.shape
    y = np.zeros((M, pw.shape[0]))
    for b in range(NB):
        part = pa[:, b, :] @ pw[:, b, :].T
        y += np.ldexp(part, qa.exps[:, b][:, None] + qw.exps[:, b][None, :])
    return y


def mx_gemm_exact(qa: MXResult, qw: MXResult):
    """The same product in exact rational arithmetic (Python loops; tiny
    inputs only): a list of rows of Fractions."""
    pa, pw = qa.elements(), qw.elements()
    M, K = pa.shape
    N = pw.shape[0]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                b = k // MX_BLOCK
                s += (Fraction(pa[m, k]) * Fraction(pw[n, k])
                      * Fraction(2) ** int(qa.exps[m, b] + qw.exps[n, b]))
            row.append(s)
        out.append(row)
    return out


def quantize_mx(x_bits, fmt, rotate_on: bool = True) -> MXResult:
    """bf16 bits [R, K] -> optional group-256 rotation -> MX quantization.
    Serves the online activation prologue and the offline weight packing
    alike (both operands use the same block quantizer)."""
    x = bf16_bits_to_f64(x_bits)
    return mx_quantize(rotate(x) if rotate_on else x, fmt)


def mx_linear(x_bits, w_bits, fmt, rotate_on: bool = True, bias_bits=None, epi: str = "bf16",
              residual_bits=None, gate_bits=None, l1_bits=None, l2_bits=None):
    """End-to-end MX linear.  Returns (out_bf16_bits, y_fp64, qa, qw), y the
    product plus bias (plus the low-rank branch) before the epilogue.

    With l1_bits [K, r] / l2_bits [r, N] this is the SVDQuant layer in MX
    form -- the pages' "NVFP4 r32" build (model card "Krea 2 Turbo Nunchaku
    Lite INT4 r32", section "Benchmark": an FP4 build with a rank-32 branch;
    README "Krea-2-SVDQuant-ComfyUI", section "Low-rank refinement": W is a
    quantized part plus a small full-precision product): the branch
    (X L1) L2 is added with the unrotated bf16 X, as in the integer layer."""
    qa = quantize_mx(x_bits, fmt, rotate_on)
    qw = quantize_mx(w_bits, fmt, rotate_on)
    y = mx_gemm(qa, qw)
    if bias_bits is not None:
        y = y + bf16_bits_to_f64(bias_bits)[None, :]
    if l1_bits is not None and l2_bits is not None and np.asarray(l1_bits).shape[1] > 0:
        x = bf16_bits_to_f64(x_bits)
        y = y + (x @ bf16_bits_to_f64(l1_bits)) @ bf16_bits_to_f64(l2_bits)
    res = bf16_bits_to_f64(residual_bits) if residual_bits is not None else None
    gate = bf16_bits_to_f64(gate_bits) if gate_bits is not None else None
    return f64_to_bf16_bits(epilogue(y, epi, res, gate)), y, qa, qw
