"""Reference (oracle) implementation of the rotated low-bit quantized linear.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Slow, plain and
literal: every step is written the way the method defines it, with NumPy
library primitives (matmul, rint) as the only building blocks.

Notation: X activations [M, K], W weights [N, K] (out x in, the layout of a
torch Linear), y = X W^T [M, N].  H is the 256x256 regular Hadamard matrix,
Hn = H / 16 its orthonormal (and self-inverse) version.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "GROUP", "QMAX", "SCALE_MODES",
    "bf16_bits_to_f64", "f64_to_bf16_bits", "bf16_round",
    "regular_hadamard_256", "rotate",
    "quantize", "code_ratio", "dequantize",
    "pack_int4", "unpack_int4",
    "fp6_e2m3_value", "fp6_e2m3_encode", "pack_fp6", "unpack_fp6",
    "int_gemm", "int_gemm_grouped",
    "silu", "sigmoid", "epilogue",
    "QuantResult", "quantize_activations", "quantize_weights",
    "rmsnorm_modulate", "quantize_activations_norm",
    "linear_fp64", "linear",
]

GROUP = 256                      # rotation group size along K
QMAX = {4: 7, 8: 127}            # symmetric code range +-qmax
SCALE_MODES = ("tensor", "row", "group64")


# --------------------------------------------------------------------------
# bfloat16 <-> float64
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values (bf16 is the top half of
    a float32, so the widening is exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):     # NaN payloads widen as NaN
        return b.view(np.float32).astype(np.float64)


_BF16_MAX = float(np.frombuffer(np.uint32(0x7F7F0000).tobytes(), np.float32)[0])


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even),
    returned as float64.  bfloat16 keeps 8 significant bits and float32's
    exponent range; its smallest subnormal step is 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    xf = x[finite]
    _, e = np.frexp(xf)                     # xf = m * 2^e, 0.5 <= |m| < 1
    step_exp = np.maximum(e - 8, -133)      # exponent of one unit in the last place
    q = np.ldexp(np.rint(np.ldexp(xf, -step_exp)), step_exp)
    # Above the largest finite bf16 the value rounds to infinity (the tie
    # point itself rounds to the even neighbour, which is infinity).
    q = np.where(np.abs(q) > _BF16_MAX, np.copysign(np.inf, xf), q)
    out[finite] = q
    out[~finite] = x[~finite]
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, one round-to-nearest-even."""
    r = bf16_round(x).astype(np.float32)    # exact: r is a bf16 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# Rotation: group-256 regular Hadamard ([INT4-mixed] introduction names a
# group-256 regular-Hadamard rotation applied to weights offline and to
# activations online; [SVDQ-Comfy] "Why this exists" says the group-wise
# Hadamard rotation spreads outliers without calibration).
# --------------------------------------------------------------------------

def regular_hadamard_256() -> np.ndarray:
    """The 256x256 regular Hadamard matrix H = H4 (x) H4 (x) H4 (x) H4 with
    H4 = J - 2I (every entry +1 except -1 on the diagonal).

    Closed form: write i and j in base 4 (four digits each); H[i, j] = -1 to
    the power of the number of digit positions where i and j agree.  H is
    symmetric, H H^T = 256 I and every row and column sums to 16, which is
    what "regular" means.  Returned as int64."""
    idx = np.arange(GROUP)
    agree = np.zeros((GROUP, GROUP), dtype=np.int64)
    for d in range(4):
        digit = (idx >> (2 * d)) & 3
        agree += digit[:, None] == digit[None, :]
    return np.where(agree % 2 == 0, 1, -1).astype(np.int64)


def rotate(x: np.ndarray) -> np.ndarray:
    """x [R, K] float64 -> x multiplied on the right by blockdiag(H/16, ...):
    every aligned, contiguous group of 256 channels along K is rotated by the
    orthonormal Hn = H/16.  K must be a multiple of 256.  For bf16 inputs the
    result is exact in float64 (at most ~45 significant bits are needed)."""
    x = np.asarray(x, dtype=np.float64)
    R, K = x.shape
    if K % GROUP:
        raise ValueError(f"rotation needs K % {GROUP} == 0, got K={K}")
    hn = regular_hadamard_256().astype(np.float64) / 16.0
    return (x.reshape(R, K // GROUP, GROUP) @ hn).reshape(R, K)


# --------------------------------------------------------------------------
# Symmetric quantization ([INT4-mixed] introduction: signed INT4 weights,
# activations quantized dynamically at run time; [OrbitQuant] "What is
# quantized": per-row INT8 weights with INT8 activations for ff.down;
# [NunchakuLite] introduction: INT4 with group size 64).
# --------------------------------------------------------------------------

def _units(x: np.ndarray, mode: str) -> np.ndarray:
    R, K = x.shape
    if mode == "tensor":
        return x.reshape(1, R * K)
    if mode == "row":
        return x.reshape(R, K)
    if mode == "group64":
        if K % 64:
            raise ValueError("group64 needs K % 64 == 0")
        return x.reshape(R * (K // 64), 64)
    raise ValueError(f"unknown scale mode {mode!r}")


def _scale_shape(R: int, K: int, mode: str):
    return {"tensor": (1,), "row": (R,), "group64": (R, K // 64)}[mode]


def _f32_quotient(a: np.ndarray, qmax: int) -> np.ndarray:
    """a / qmax rounded once to float32 (round half to even), for float64 a.

    The float64 quotient, cast to float32, is that correctly rounded value:
    double rounding could differ only if the float64 rounding moved an
    inexact quotient onto a float32 midpoint.  It cannot: a is a multiple of
    its float64 ulp u_a, a midpoint m is a multiple of a much larger power of
    two, so a nonzero a - qmax m is at least u_a and the quotient misses m by
    at least u_a / qmax, which (qmax = 7 or 127, just below a power of two)
    exceeds half a float64 ulp of the quotient."""
    return (np.asarray(a, dtype=np.float64) / qmax).astype(np.float32)


def code_ratio(xr: np.ndarray, bits: int, mode: str) -> np.ndarray:
    """The unrounded code t = x' * qmax / a of every element of xr [R, K]
    (already rotated values), a = max |x'| over the element's unit (whole
    tensor, one row, or one row x 64-channel group), in float64; 0 where the
    unit is all zero.  The code is rne(t) (see quantize)."""
    qmax = QMAX[bits]
    R, K = xr.shape
    x = np.asarray(xr, dtype=np.float64)
    u = _units(x, mode)
    a = np.abs(u).max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(a[:, None] > 0, u * qmax / a[:, None], 0.0)
    return t.reshape(R, K)


def quantize(xr: np.ndarray, bits: int, mode: str):
    """Dynamic symmetric quantization of (already rotated) values xr [R, K].

    Per unit (whole tensor, one row, or one row x 64-channel group):
      a     = max |x'|                              (absmax of the unit)
      s     = a / qmax, rounded once to float32     (the stored scale)
      q     = clamp(rne(x' * qmax / a), +-qmax)     (the code; 0 when a == 0)
    with qmax = 7 (int4) or 127 (int8), round-half-to-even, and -qmax-1 never
    produced.  Everything before the float32 scale is float64: the rotated
    values are exact, a is exact, and x' * qmax / a is the float64 quotient.

    Returns (codes int8 [R, K], scales float32 of shape [1] | [R] | [R, K/64])."""
    qmax = QMAX[bits]
    R, K = xr.shape
    u = _units(np.asarray(xr, dtype=np.float64), mode)
    a = np.abs(u).max(axis=1)
    scale = _f32_quotient(a, qmax)
    q = np.clip(np.rint(code_ratio(xr, bits, mode)), -qmax, qmax).astype(np.int8)
    return q, scale.reshape(_scale_shape(R, K, mode))


def _expand_scale(scale: np.ndarray, R: int, K: int, mode: str) -> np.ndarray:
    s = np.asarray(scale, dtype=np.float64)
    if mode == "tensor":
        return np.full((R, K), s.reshape(-1)[0])
    if mode == "row":
        return np.repeat(s.reshape(R, 1), K, axis=1)
    return np.repeat(s.reshape(R, K // 64), 64, axis=1)


def dequantize(q: np.ndarray, scale: np.ndarray, mode: str) -> np.ndarray:
    """codes * scale, broadcast per unit, in float64 (exact)."""
    R, K = q.shape
    return q.astype(np.float64) * _expand_scale(scale, R, K, mode)


# --------------------------------------------------------------------------
# INT4 packing ([INT4-mixed] introduction: packed signed INT4 weights, two
# values per byte).  The byte order is this library's documented layout:
# within each run of 8 consecutive K positions 8c..8c+7, byte 4c+j (j=0..3)
# holds position 8c+j in its low nibble and 8c+j+4 in its high nibble, each
# as a 4-bit two's-complement value.
# --------------------------------------------------------------------------

def pack_int4(q: np.ndarray) -> np.ndarray:
    """int8 codes [R, K] (values in -8..7, K % 8 == 0) -> uint8 [R, K/2]."""
    R, K = q.shape
    if K % 8:
        raise ValueError("int4 packing needs K % 8 == 0")
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8).reshape(R, K // 8, 2, 4)
    low = nib[:, :, 0, :]     # positions 8c + j
    high = nib[:, :, 1, :]    # positions 8c + 4 + j
    return (low | (high << 4)).reshape(R, K // 2)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    """uint8 [R, K/2] -> int8 codes [R, K]; inverse of pack_int4."""
    R, KH = p.shape
    b = np.asarray(p, dtype=np.uint8).reshape(R, KH // 4, 1, 4)
    nib = np.concatenate([b & 0xF, b >> 4], axis=2).astype(np.int16)
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8).reshape(R, KH * 2)


# --------------------------------------------------------------------------
# Exact integer contraction ([SVDQ-Comfy] "Why this exists": the speed comes
# from running the matmul on integer units with activations quantized too;
# [lab] Study 2/3: the fused low-bit multiply is the lever).
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# FP6 (e2m3) code layout -- an alternative encoding of the same int4 codes
# for gfx950's FP6 matrix instructions.  Every integer -7..7 is exactly an
# e2m3 value (sign bit, 2 exponent bits with bias 1, 3 mantissa bits: the
# FP6 E2M3 element of the OCP microscaling formats), so the encoding changes
# no code and no product; products of two codes are integers of magnitude
# <= 49 and their sums stay exact in float32 while 49 K < 2^24.
# Layout (this library's own): a row of K codes is K/128 blocks of 96 bytes.
# In block b, sub-block g (0..3) holds channels 128b + 32g + i (i = 0..31)
# as the 192-bit little-endian integer v_g with channel i in bits 6i..6i+5;
# bytes 16g..16g+15 of the block are the low 16 bytes of v_g and bytes
# 64 + 8g .. 64 + 8g + 7 its high 8 bytes.
# --------------------------------------------------------------------------

def fp6_e2m3_value(bits) -> np.ndarray:
    """Decode 6-bit e2m3 patterns to float64 from the format's definition:
    sign = bit 5, exponent e = bits 4..3, mantissa m = bits 2..0;
    e == 0: (-1)^s * m / 8 (subnormal); else (-1)^s * 2^(e-1) * (1 + m/8)."""
    b = np.asarray(bits, dtype=np.int64)
    s = np.where((b >> 5) & 1, -1.0, 1.0)
    e = (b >> 3) & 3
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0, np.ldexp(1.0 + m / 8.0, (e - 1).astype(np.int64)))
    return s * mag


def fp6_e2m3_encode(q: np.ndarray) -> np.ndarray:
    """int codes -7..7 -> their exact e2m3 bit patterns, found by searching
    all 64 patterns with the decoder (zero takes the +0 pattern)."""
    q = np.asarray(q, dtype=np.int64)
    if np.abs(q).max(initial=0) > 7:
        raise ValueError("FP6 codes hold -7..7")
    vals = fp6_e2m3_value(np.arange(64))
    out = np.zeros(q.shape, dtype=np.int64)
    for code in range(-7, 8):
        out[q == code] = np.nonzero(vals == code)[0].min()
    return out


def pack_fp6(q: np.ndarray) -> np.ndarray:
    """int8 codes [R, K] (-7..7, K % 128 == 0) -> uint8 [R, 3K/4] in the FP6 layout."""
    q = np.asarray(q)
    R, K = q.shape
    if K % 128:
        raise ValueError("FP6 layout needs K % 128 == 0")
    pat = fp6_e2m3_encode(q).reshape(R, K // 128, 4, 32)
    # bit 6i + b of v_g is bit b of channel i's pattern
    bits = ((pat[..., None] >> np.arange(6)) & 1).astype(np.uint8).reshape(R, K // 128, 4, 192)
    v = np.packbits(bits, axis=-1, bitorder="little")          # [R, K/128, 4, 24] little-endian bytes
    blk = np.concatenate([v[..., :16].reshape(R, K // 128, 64),  # low 16 bytes of v_0..v_3
                          v[..., 16:].reshape(R, K // 128, 32)], axis=-1)  # then their high 8 bytes
    return blk.reshape(R, K // 128 * 96)


def unpack_fp6(p: np.ndarray) -> np.ndarray:
    """uint8 [R, 3K/4] in the FP6 layout -> int8 codes [R, K]."""
    p = np.asarray(p, dtype=np.uint8)
    R, nb = p.shape
    blk = p.reshape(R, nb // 96, 96)
    v = np.concatenate([blk[..., :64].reshape(R, nb // 96, 4, 16),
                        blk[..., 64:].reshape(R, nb // 96, 4, 8)], axis=-1)    # [R, K/128, 4, 24]
    bits = np.unpackbits(v, axis=-1, bitorder="little").reshape(R, nb // 96, 4, 32, 6)
    pat = (bits.astype(np.int64) << np.arange(6)).sum(axis=-1)
    return fp6_e2m3_value(pat).astype(np.int8).reshape(R, nb // 96 * 128)


def int_gemm(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qa[m, k] * qw[n, k], exactly, as int64.  Formed by a
    float64 BLAS product of the integer matrices, which is exact because every
    partial sum stays far below 2^53 (|acc| <= K * 127^2)."""
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    assert qa.shape[1] == qw.shape[1]
    assert qa.shape[1] * 127 * 127 < 2 ** 53
    return (qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)


def int_gemm_grouped(qa: np.ndarray, qw: np.ndarray, group: int = 64) -> np.ndarray:
    """One exact integer partial per K-group: acc[g, m, n] over k in group g."""
    K = qa.shape[1]
    G = K // group
    return np.stack([int_gemm(qa[:, g * group:(g + 1) * group],
                              qw[:, g * group:(g + 1) * group]) for g in range(G)])


# --------------------------------------------------------------------------
# Epilogues ([OrbitQuant] "Fused transformer": SwiGLU over a gate|up GEMM and
# gated residual updates happen in GEMM epilogues).
# --------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU, z * sigmoid(z), in float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic sigmoid 1 / (1 + exp(-z)), in float64: the attention gate of
    [OrbitQuant] "Fused transformer (OrbitQuant 0.11)" (the grouped
    Q|K|V|gate GEMM applies it in its epilogue)."""
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def epilogue(y: np.ndarray, kind: str, residual=None, gate=None) -> np.ndarray:
    """Apply the output epilogue to the float64 GEMM result y [M, N]:
      "bf16"           -> y
      "swiglu"         -> silu(y[:, :F]) * y[:, F:], F = N / 2 (first half of
                          the output columns is the gate, second half up)
      "gated_residual" -> residual + gate[n] * y
      "sigmoid"        -> sigmoid(y) (the attention gate projection)
    Returns float64 (round with f64_to_bf16_bits)."""
    if kind == "bf16":
        return y
    if kind == "sigmoid":
        return sigmoid(y)
    if kind == "swiglu":
        F = y.shape[1] // 2
        return silu(y[:, :F]) * y[:, F:]
    if kind == "gated_residual":
        return np.asarray(residual, np.float64) + np.asarray(gate, np.float64)[None, :] * y
    raise ValueError(kind)


# --------------------------------------------------------------------------
# Whole linear layer.
# --------------------------------------------------------------------------

class QuantResult:
    """Codes and scales of one quantized operand."""

    def __init__(self, codes, scales, bits, mode, rotated):
        self.codes = codes        # int8 [R, K]
        self.scales = scales      # float32 [1] | [R] | [R, K/64]
        self.bits = bits
        self.mode = mode
        self.rotated = rotated    # float64 [R, K] rotated values (pre-quantization)

    def dequant(self) -> np.ndarray:
        return dequantize(self.codes, self.scales, self.mode)


def quantize_activations(x_bits, bits: int, mode: str, rotate_on: bool = True) -> QuantResult:
    """Online activation prologue: bf16 -> rotate (optional) -> quantize."""
    x = bf16_bits_to_f64(x_bits)
    xr = rotate(x) if rotate_on else x
    q, s = quantize(xr, bits, mode)
    return QuantResult(q, s, bits, mode, xr)


def rmsnorm_modulate(x_bits, gamma_bits=None, scale_bits=None, shift_bits=None, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm followed by the adaLN modulation of a DiT block input, float64.

    [OrbitQuant] "Fused transformer (OrbitQuant 0.11)": the block's RMSNorm
    and modulation run inside the activation quantization prologues.  The page
    names the two steps, not their formula; the reading taken is the usual one
    for a batch-1 block (per-channel modulation vectors):

        r[m]    = 1 / sqrt(mean_k x[m, k]^2 + eps)
        h[m, k] = x[m, k] * r[m] * gamma[k] * (1 + scale[k]) + shift[k]

    x_bits: bf16 bits [M, K]; gamma, scale, shift: bf16 bits [K] or None
    (meaning 1, 0 and 0).  eps > 0."""
    x = bf16_bits_to_f64(x_bits)
    M, K = x.shape
    gamma = np.ones(K) if gamma_bits is None else bf16_bits_to_f64(gamma_bits).reshape(K)
    scale = np.zeros(K) if scale_bits is None else bf16_bits_to_f64(scale_bits).reshape(K)
    shift = np.zeros(K) if shift_bits is None else bf16_bits_to_f64(shift_bits).reshape(K)
    ms = np.mean(x * x, axis=1)                       # mean square of each row
    r = 1.0 / np.sqrt(ms + eps)
    return x * r[:, None] * (gamma * (1.0 + scale))[None, :] + shift[None, :]


def quantize_activations_norm(x_bits, gamma_bits, scale_bits, shift_bits, eps: float, bits: int, mode: str,
                              rotate_on: bool = True) -> QuantResult:
    """The prologue with the norm fused in front: h = rmsnorm_modulate(x, ...)
    (never rounded to bf16), then rotate and quantize h exactly as
    quantize_activations does for x."""
    h = rmsnorm_modulate(x_bits, gamma_bits, scale_bits, shift_bits, eps)
    hr = rotate(h) if rotate_on else h
    q, s = quantize(hr, bits, mode)
    return QuantResult(q, s, bits, mode, hr)


def quantize_weights(w_bits, bits: int, mode: str, rotate_on: bool = True) -> QuantResult:
    """Offline weight preparation: the same rotation along K and the same
    symmetric quantizer, applied to the rows of W [N, K]."""
    return quantize_activations(w_bits, bits, mode, rotate_on)


def _scale_col(q: QuantResult) -> np.ndarray:
    """Per-row scale as a float64 column [R, 1] (tensor or row mode)."""
    R = q.codes.shape[0]
    s = np.asarray(q.scales, np.float64).reshape(-1)
    return (np.full(R, s[0]) if q.mode == "tensor" else s).reshape(R, 1)


def linear_fp64(qa: QuantResult, qw: QuantResult, x_bits=None, l1_bits=None, l2_bits=None,
                bias_bits=None) -> np.ndarray:
    """Dequantized product before the epilogue, float64.

    The layer accumulates the codes exactly in integers and only then
    dequantizes ([OrbitQuant] "Fused transformer": integer GEMMs with the
    scaling and the rest of the output work in their epilogues), so y is
    formed from the exact integer product:
      tensor / row scales:  y = acc * s_a[m] * s_w[n]
      group-64 scales:      y = sum_g acc_g * (s_a[m, g] * s_w[n, g])
    which equals deq(A) deq(W)^T mathematically; an exactly-zero accumulator
    gives an exactly-zero y.  Optional bias[n] is added, and the low-rank
    branch adds (X L1) L2 with the unrotated bf16 X ([SVDQ-Comfy] "Low-rank
    refinement": W is split into a quantized part plus a small
    full-precision product; "LoRA": the branch is applied as a parallel
    low-rank product, (W + BA)x = Wx + B(Ax))."""
    if (qa.mode == "group64") != (qw.mode == "group64"):
        raise ValueError("group-64 scales must be used on both operands")
    if qa.mode == "group64":
        K = qa.codes.shape[1]
        sa = np.asarray(qa.scales, np.float64)
        sw = np.asarray(qw.scales, np.float64)
        y = np.zeros((qa.codes.shape[0], qw.codes.shape[0]))
        for g in range(K // 64):
            sl = slice(64 * g, 64 * g + 64)
            acc_g = int_gemm(qa.codes[:, sl], qw.codes[:, sl]).astype(np.float64)
            y += acc_g * (sa[:, g][:, None] * sw[:, g][None, :])
    else:
        acc = int_gemm(qa.codes, qw.codes).astype(np.float64)
        y = acc * _scale_col(qa) * _scale_col(qw).T
    if bias_bits is not None:
        y = y + bf16_bits_to_f64(bias_bits)[None, :]
    if l1_bits is not None and l2_bits is not None and np.asarray(l1_bits).shape[1] > 0:
        x = bf16_bits_to_f64(x_bits)
        y = y + (x @ bf16_bits_to_f64(l1_bits)) @ bf16_bits_to_f64(l2_bits)
    return y


def linear(x_bits, w_bits, a_bits: int, w_bits_n: int, mode: str, epi: str = "bf16",
           rotate_on: bool = True, l1_bits=None, l2_bits=None, bias_bits=None,
           residual_bits=None, gate_bits=None):
    """End-to-end rotated low-bit linear.  Returns (out_bf16_bits, y_fp64,
    activation QuantResult, weight QuantResult)."""
    qa = quantize_activations(x_bits, a_bits, mode, rotate_on)
    qw = quantize_weights(w_bits, w_bits_n, mode, rotate_on)
    y = linear_fp64(qa, qw, x_bits, l1_bits, l2_bits, bias_bits)
    res = bf16_bits_to_f64(residual_bits) if residual_bits is not None else None
    gate = bf16_bits_to_f64(gate_bits) if gate_bits is not None else None
    out = epilogue(y, epi, res, gate)
    return f64_to_bf16_bits(out), y, qa, qw
