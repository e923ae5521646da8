"""Acceptance checks of the HIP path against the oracle, with tolerances
derived from the kernels' float32 arithmetic.

The oracle quantizes by the definition in float64; the kernels rotate in
float32 and take the code from a float32 product.  Their codes may therefore
differ from the oracle's only where the exact quotient t = x' * qmax / a sits
within the kernels' error of a rounding tie, and their scales only by the
error of the float32 absmax.  Both errors have rigorous bounds:

Rotation.  The kernels form z = H x (x' = z / 16) with four radix-4 stages.
A stage output is the sum of the four values that differ in one base-4 digit
(three float32 additions) minus twice the value itself (one rounding, the
doubling is exact), so it carries a local error of at most 5 u S with S the
sum of |inputs| of that butterfly (u = 2^-24).  The transform's entries are
+-1, so errors travel to later stages with coefficient magnitude one, and at
every stage the butterflies feeding one output partition the 256 inputs of
the group.  Hence |z_gpu - z| <= 4 * 5 u * ||x_g||_1 per 256-channel group,
i.e. |x'_gpu - x'| <= 20 u ||x_g||_1 / 16.  Errors already in the inputs
(the fused norm) add their sum over the group.

Code.  With B_i the bound of element i and B the largest over its unit,
a_gpu = max |x'_gpu| is within B of a, the float32 reciprocal and product add
two roundings, so the kernel's pre-rounding value is within
  delta_i = qmax (B_i + B) / (a - B) + 4 u qmax
of t_i.  A code may differ from rne(t_i) only if |code - t_i| <= 1/2 + delta_i
(a near-tie); every code is checked against that, and the flips also against
the 1e-4 budget.

Scale.  s_gpu = fl32(a_gpu / qmax) (the 1/16 is exact), so
|s_gpu - a / qmax| <= B / qmax + half an ulp of s.

Outputs.  The dequantized product of the same codes is checked element by
element: the kernel's float32 epilogue (scale products, group-64 partial
sums, the bf16 low-rank intermediate, the SwiGLU / sigmoid / residual
arithmetic) is bounded per element, and the bf16 output may differ from the
rounded oracle value by that bound plus one bf16 ulp.
"""

from __future__ import annotations

import numpy as np

import oracle as O

U = 2.0 ** -24          # float32 unit roundoff
BF16_U = 2.0 ** -8      # bf16 unit roundoff: 8 significant bits, |fl(x) - x| <= 2^-8 |x|
FLIP_BUDGET = 1e-4


# ------------------------------------------------------------ prologue ----

def rotation_error_bound(x_abs: np.ndarray, pre_err=None, rotate: bool = True) -> np.ndarray:
    """Per-element bound on |x'_gpu - x'| (rotated-value units) for inputs
    with magnitudes x_abs [R, K] and input errors pre_err (None: exact bf16
    inputs)."""
    x_abs = np.abs(np.asarray(x_abs, np.float64))
    R, K = x_abs.shape
    pe = np.zeros_like(x_abs) if pre_err is None else np.asarray(pre_err, np.float64)
    if not rotate:
        return pe.copy()
    g1 = x_abs.reshape(R, K // 256, 256).sum(axis=2)
    ge = pe.reshape(R, K // 256, 256).sum(axis=2)
    b = (20.0 * U * g1 + ge) / 16.0
    return np.repeat(b, 256, axis=1)


def norm_input_error(x_bits, gamma_bits, scale_bits, shift_bits, eps: float):
    """The fused RMSNorm + modulation prologue's input to the rotation:
    (h float64 [M, K] from the oracle, bound on |h_gpu - h|).

    The kernel sums the K squares of a row in float32 in chains of at most
    K/16 + 20 additions (lane, 16-lane row, row slots), so the sum carries a
    relative error of at most n u; r = 1 / sqrt(sum / K + eps) then adds three
    roundings and halves the sum's error: |r_gpu / r - 1| <= (n/2 + 3) u.
    g = gamma (1 + scale) has two roundings, x r one, and h = fma(x r, g,
    shift) one more relative to h."""
    h = O.rmsnorm_modulate(x_bits, gamma_bits, scale_bits, shift_bits, eps)
    x = O.bf16_bits_to_f64(x_bits)
    M, K = x.shape
    g = np.ones(K) if gamma_bits is None else O.bf16_bits_to_f64(gamma_bits).reshape(K)
    sc = np.zeros(K) if scale_bits is None else O.bf16_bits_to_f64(scale_bits).reshape(K)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    xrg = np.abs(x * r[:, None] * (g * (1.0 + sc))[None, :])
    n = K / 16 + 20
    dr = (n / 2 + 3) * U
    return h, xrg * (dr + 4 * U) + U * np.abs(h)


def _unit_view(a: np.ndarray, mode: str) -> np.ndarray:
    R, K = a.shape
    return {"tensor": a.reshape(1, R * K), "row": a, "group64": a.reshape(R * (K // 64), 64)}[mode]


def check_codes(got_codes, got_scales, xr, bound, bits: int, mode: str, budget: float = FLIP_BUDGET,
                rows=None):
    """Check GPU codes [R', K] and scales against the oracle's definition on
    the rotated values xr [R, K] (float64) with per-element error bound
    `bound` [R, K].  rows: the rows of xr the GPU arrays hold (None: all);
    units are always formed on the full xr (tensor mode needs every row).
    Returns {"flips", "flip_frac", "scale_ulp_max", "scale_ulp_bound"}."""
    qmax = O.QMAX[bits]
    xr = np.asarray(xr, np.float64)
    R, K = xr.shape
    t = O.code_ratio(xr, bits, mode)
    ref = np.clip(np.rint(t), -qmax, qmax)
    uv = _unit_view(np.abs(xr), mode)
    a = uv.max(axis=1)
    bu = _unit_view(np.asarray(bound, np.float64), mode).max(axis=1)
    # per element: its unit's a and B
    nun = uv.shape[1]
    a_el = np.repeat(a, nun).reshape(R, K)
    bu_el = np.repeat(bu, nun).reshape(R, K)
    with np.errstate(divide="ignore", invalid="ignore"):
        delta = np.where(a_el > bu_el, qmax * (np.asarray(bound) + bu_el) / (a_el - bu_el) + 4 * U * qmax, np.inf)
    sel = np.arange(R) if rows is None else np.asarray(rows)
    got = np.asarray(got_codes).astype(np.float64)
    assert got.shape == (len(sel), K), (got.shape, len(sel), K)
    t_s, ref_s, d_s = t[sel], ref[sel], delta[sel]
    assert np.abs(got).max(initial=0) <= qmax, "code outside +-qmax"
    far = np.abs(got - t_s) > 0.5 + d_s
    if far.any():
        i = np.argwhere(far)[0]
        raise AssertionError(f"{int(far.sum())} codes are not near-ties: first at {i.tolist()}: "
                             f"gpu {got[tuple(i)]:.0f}, exact quotient {t_s[tuple(i)]:.9f}, window {d_s[tuple(i)]:.2e}")
    flips = int((got != ref_s).sum())
    frac = flips / got.size if got.size else 0.0
    assert frac <= budget, f"flip fraction {frac:.2e} > {budget:.0e}"
    # scales
    s_exact = a / qmax
    s_bound = bu / qmax
    gs = np.asarray(got_scales, np.float64)
    if mode == "tensor":
        unit_idx = np.zeros(1, dtype=np.int64)
        gs = gs.reshape(1)
    elif mode == "row":
        unit_idx = sel
        gs = gs.reshape(len(sel))
    else:
        unit_idx = (sel[:, None] * (K // 64) + np.arange(K // 64)[None, :]).reshape(-1)
        gs = gs.reshape(-1)
    se = s_exact[unit_idx]
    sb = s_bound[unit_idx]
    ulp = np.ldexp(1.0, np.frexp(np.maximum(se, 1e-38).astype(np.float32))[1] - 24)
    err = np.abs(gs - se)
    bad = err > sb + 0.5 * ulp * (1 + 1e-9) + ulp * 1e-3
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError(f"{int(bad.sum())} scales off: unit {int(unit_idx[i])}: gpu {gs[i]!r}, "
                             f"exact {se[i]!r}, bound {sb[i]:.3e}")
    zero = se == 0
    assert (gs[zero] == 0).all(), "an all-zero unit must have scale 0"
    with np.errstate(divide="ignore", invalid="ignore"):
        ulps = np.where(zero, 0.0, err / ulp)
        ulpb = np.where(zero, 0.0, sb / ulp + 0.5)
    return {"flips": flips, "flip_frac": frac, "scale_ulp_max": float(ulps.max(initial=0.0)),
            "scale_ulp_bound": float(ulpb.max(initial=0.0))}


# ------------------------------------------------------------- outputs ----

def _bf16_ulp(v):
    v = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.frexp(v)[1] - 8)


def dequant_product_bound(qa: "O.QuantResult", qw: "O.QuantResult", post_packed: bool = True):
    """(y float64 [M, N] of the same codes, bound on |y_gpu - y| from the
    kernel's float32 dequantization).  Tensor / row scales: y_gpu =
    fl(fl(fl(acc) * fl(s_a / 16^p)) * s_w): at most 4 roundings relative to
    |y|.  Group-64 scales: y_gpu accumulates the K/64 terms
    fl(part_g) * fl(s_a s_w) with fused multiply-adds in group order, at most
    (K/64 + 3) u relative to the sum of the terms' magnitudes."""
    y = O.linear_fp64(qa, qw)
    if qa.mode == "group64":
        K = qa.codes.shape[1]
        G = K // 64
        aq = O.QuantResult(np.abs(qa.codes), np.abs(qa.scales), qa.bits, qa.mode, None)
        mag = np.zeros_like(y)
        sa = np.asarray(qa.scales, np.float64)
        sw = np.asarray(qw.scales, np.float64)
        for g in range(G):
            sl = slice(64 * g, 64 * g + 64)
            acc = np.abs(O.int_gemm(qa.codes[:, sl], qw.codes[:, sl])).astype(np.float64)
            mag += acc * (sa[:, g][:, None] * sw[:, g][None, :])
        del aq
        return y, (G + 3) * U * mag
    return y, 5 * U * np.abs(y)


def linear_bound(qa: "O.QuantResult", qw: "O.QuantResult", x_bits=None, l1_bits=None, l2_bits=None,
                 bias_bits=None):
    """(y float64 [M, N] = dequantized product + bias + low-rank branch, as
    the oracle's linear_fp64, and the bound on the kernel's float32 y): the
    product's bound, the branch's bound, and three more roundings of the
    additions relative to the magnitudes added."""
    y, dy = dequant_product_bound(qa, qw)
    mag = np.abs(y)
    if bias_bits is not None:
        b = O.bf16_bits_to_f64(bias_bits)[None, :]
        y = y + b
        mag = mag + np.abs(b)
    if l1_bits is not None and np.asarray(l1_bits).shape[1] > 0:
        br, dbr = lowrank_bound(x_bits, l1_bits, l2_bits)
        y = y + br
        dy = dy + dbr
        mag = mag + np.abs(br)
    return y, dy + 3 * U * mag


def lowrank_bound(x_bits, l1_bits, l2_bits):
    """(branch (X L1) L2 float64, bound on the kernel's branch error): lr is
    accumulated in float32 over K (at most K/8 + 4 roundings relative to
    sum |x l1|, a loose bound for the matrix instruction's summation) and
    stored as bf16 (half a bf16 ulp); lr L2 accumulates in float32 over the
    rank."""
    x = O.bf16_bits_to_f64(x_bits)
    l1 = O.bf16_bits_to_f64(l1_bits)
    l2 = O.bf16_bits_to_f64(l2_bits)
    K = x.shape[1]
    r = l1.shape[1]
    lr = x @ l1
    lr_err = BF16_U * np.abs(lr) + (K / 8 + 4) * U * (np.abs(x) @ np.abs(l1))
    lr_err = lr_err * (1 + BF16_U) + BF16_U * 2.0 ** -126
    br = lr @ l2
    return br, lr_err @ np.abs(l2) + (r + 4) * U * (np.abs(lr) @ np.abs(l2))


def epilogue_with_bound(y, dy, kind: str, residual=None, gate=None):
    """Apply the epilogue to y (float64) and carry the bound dy through it,
    plus the kernel's float32 evaluation of the epilogue (16 u relative for
    SiLU / sigmoid with the hardware exponential and a division; 2 roundings
    for the residual update)."""
    if kind in ("bf16", "f32"):
        return y, dy
    if kind == "sigmoid":
        out = O.sigmoid(y)
        return out, 0.25 * dy + 16 * U * np.abs(out)
    if kind == "swiglu":
        F = y.shape[1] // 2
        g, u = y[:, :F], y[:, F:]
        dg, du = dy[:, :F], dy[:, F:]
        out = O.silu(g) * u
        return out, 1.1 * np.abs(u) * dg + np.abs(O.silu(g)) * du + 1.1 * dg * du + 16 * U * np.abs(out)
    if kind == "gated_residual":
        res = np.asarray(residual, np.float64)
        gt = np.asarray(gate, np.float64)[None, :]
        out = res + gt * y
        return out, np.abs(gt) * dy + 2 * U * (np.abs(res) + np.abs(gt * y))
    raise ValueError(kind)


def assert_outputs_close(got, want, bound, bf16: bool = True, what: str = ""):
    """Element-wise: |got - round(want)| <= bound + one bf16 ulp (bf16
    outputs) or <= bound + half a float32 ulp (float32 outputs)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    bound = np.asarray(bound, np.float64)
    if bf16:
        ref = O.bf16_round(want)
        tol = bound + _bf16_ulp(np.abs(want) + bound)
    else:
        ref = want
        tol = bound + np.ldexp(1.0, np.frexp(np.maximum(np.abs(want) + bound, 2.0 ** -126))[1] - 24)
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs off; first at {i.tolist()}: "
                             f"got {got[tuple(i)]!r}, want {ref[tuple(i)]!r}, tol {tol[tuple(i)]:.3e}")
    return float((err / np.maximum(tol, 1e-300)).max(initial=0.0))


# ------------------------------------------------------------ MX blocks ----
#
# MX block quantization (oracle.mx_ref).  The kernels take the block
# exponent from their float32 block maximum and divide by it exactly, so with
# B_i the bound on |x'_gpu - x'_i| and B the largest over the block:
#   * the exponent can differ from the oracle's only if [a - B, a + B]
#     straddles a power of two: e_gpu lies between the exponents of a - B
#     and a + B;
#   * given e_gpu, the element's pre-rounding value is within B_i / 2^e_gpu
#     of x'_i / 2^e_gpu, and rounding is monotone, so the code lies between
#     the roundings of the two ends of that interval.
# Unrotated bf16 inputs have B = 0: both decisions are the oracle's exactly.

def mx_values(codes, fmt):
    """Signed element values of element bit patterns."""
    f = O.MX_FORMATS[fmt]
    codes = np.asarray(codes, np.int64)
    mags = O.mx_element_magnitudes(fmt)[codes & (f.sign_bit - 1)]
    return np.where(codes & f.sign_bit, -mags, mags)


def check_mx(got_codes, got_exps, xr, bound, fmt: str, budget: float = FLIP_BUDGET, rows=None):
    """Check GPU MX element codes [R', K] (unpacked) and block exponents
    [R', K/32] against the oracle's definition on rotated values xr [R, K]
    with per-element error bound `bound`.  Returns {"exp_flips",
    "code_flips", "flip_frac"}: decisions that differ from the oracle's own
    (all of them inside the near-tie windows above)."""
    xr = np.asarray(xr, np.float64)
    R, K = xr.shape
    sel = np.arange(R) if rows is None else np.asarray(rows)
    xs = xr[sel]
    bs = np.asarray(bound, np.float64)[sel]
    nb = K // O.MX_BLOCK
    gc = np.asarray(got_codes)
    ge = np.asarray(got_exps, np.int64)
    assert gc.shape == xs.shape and ge.shape == (len(sel), nb), (gc.shape, ge.shape)
    a = np.abs(xs).reshape(-1, nb, 32).max(axis=2)
    bb = bs.reshape(-1, nb, 32).max(axis=2)
    ref = O.mx_quantize(xs, fmt)
    e_lo = O.mx_shared_exponent(np.maximum(a - bb, 0.0), fmt)
    e_hi = O.mx_shared_exponent(a + bb, fmt)
    bad = (ge < e_lo) | (ge > e_hi)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{int(bad.sum())} block exponents outside the window: first {list(i)}: gpu {ge[i]}, "
                             f"oracle {ref.exps[i]}, block max {a[i]!r} +- {bb[i]:.3e}")
    sh = np.repeat(ge, 32, axis=1)
    t = np.ldexp(xs, -sh)
    d = np.ldexp(bs, -sh)
    lo = mx_values(O.mx_round_element(t - d, fmt), fmt)
    hi = mx_values(O.mx_round_element(t + d, fmt), fmt)
    gv = mx_values(gc, fmt)
    far = (gv < lo) | (gv > hi)
    if far.any():
        i = tuple(np.argwhere(far)[0])
        raise AssertionError(f"{int(far.sum())} MX codes outside their rounding window: first {list(i)}: gpu "
                             f"{int(gc[i]):#x} ({gv[i]}), value / scale {t[i]!r} +- {d[i]:.3e}")
    f = O.MX_FORMATS[fmt]
    zero_neg = (gc & (f.sign_bit - 1)) == 0
    assert not (gc[zero_neg] & f.sign_bit).any(), "a zero element carries the sign bit"
    code_flips = int((gc != ref.codes).sum())
    frac = code_flips / gc.size if gc.size else 0.0
    assert frac <= budget, f"MX code flip fraction {frac:.2e} > {budget:.0e}"
    return {"exp_flips": int((ge != ref.exps).sum()), "code_flips": code_flips, "flip_frac": frac}


MX_ALIGN_BITS = 13      # FP8 products kept down to 2^-13 of the group's largest (measured)


def mx_product_bound(qa: "O.MXResult", qw: "O.MXResult"):
    """(y = the oracle's MX product of these codes, bound on the kernel's
    float32 result).

    Measured on gfx950 (in-bounds probes of the block-scaled 16x16x128
    instruction): inside a small group of adjacent elements (two neighbours
    interact, elements 16 apart do not) each product is truncated toward
    zero to a multiple of 2^(E - 13), E the binade of the group's largest
    product; group sums, block scales and the sums over blocks and over the
    K/128 chained instructions are exact to float32 or better.  FP4 products
    are multiples of 1/4 no larger than 36, so nothing is truncated; FP8
    products span 36 binades.  Bound: for FP8, per 16-element chunk (which
    contains the group), 16 products times the grid step of the chunk's
    largest possible product (max|a| * max|w| over the chunk), times the
    block scales; plus (127 + K/128) u times the sum of the products'
    magnitudes for the float32 additions in any order, plus the float32
    underflow step per addition."""
    y = O.mx_gemm(qa, qw)
    f = O.MX_FORMATS[qa.fmt]
    qa_abs = O.MXResult(np.asarray(qa.codes) & (f.sign_bit - 1), qa.exps, qa.fmt, None)
    qw_abs = O.MXResult(np.asarray(qw.codes) & (f.sign_bit - 1), qw.exps, qw.fmt, None)
    mag = O.mx_gemm(qa_abs, qw_abs)
    K = np.asarray(qa.codes).shape[1]
    n = 127 + K / 128
    bound = n * U * mag + K * 2.0 ** -149
    if qa.fmt == "fp8":
        M, N = y.shape
        am = np.abs(qa.elements()).reshape(M, K // 16, 16).max(axis=2)
        wm = np.abs(qw.elements()).reshape(N, K // 16, 16).max(axis=2)
        for c in range(K // 16):
            top = am[:, c][:, None] * wm[:, c][None, :]
            with np.errstate(divide="ignore"):
                e = np.floor(np.log2(np.where(top > 0, top, 1.0)))
            step = np.where(top > 0, np.ldexp(1.0, (e - MX_ALIGN_BITS).astype(np.int64)), 0.0)
            sc = qa.exps[:, c // 2][:, None] + qw.exps[:, c // 2][None, :]
            bound = bound + 16 * np.ldexp(step, sc)
    return y, bound


def mx_linear_bound(qa: "O.MXResult", qw: "O.MXResult", bias_bits=None):
    """(y + bias, bound): the product's bound plus the bias addition's
    rounding."""
    y, dy = mx_product_bound(qa, qw)
    mag = np.abs(y)
    if bias_bits is not None:
        b = O.bf16_bits_to_f64(bias_bits)[None, :]
        y = y + b
        mag = mag + np.abs(b)
    return y, dy + 2 * U * mag
