"""CPU checks of the GPU acceptance checks (tests/parity_checks.py).

The kernels' float32 arithmetic is emulated here in NumPy float32 (radix-4
butterflies, float32 absmax, reciprocal and product, float32 group-64
accumulation): such results must pass the checks, whose tolerances are
derived from that arithmetic, and planted mistakes (a flip away from a tie,
an off scale, a wrong output) must fail them.  This keeps the tolerances
honest without a GPU."""

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import parity_checks as P

F = np.float32


def _fp32_rotate(v):
    """z = H v in float32, one radix-4 digit at a time: s = (a + b) + (c + d),
    out = s - 2 v (the doubling is exact, one rounding)."""
    v = np.asarray(v, F)
    R, K = v.shape
    t = v.reshape(R, K // 256, 4, 4, 4, 4)
    for ax in (5, 4, 3, 2):                      # digits d0, d1, d2, d3
        a, b, c, d = (np.take(t, i, axis=ax) for i in range(4))
        s = (a + b) + (c + d)
        t = np.stack([s - F(2) * x for x in (a, b, c, d)], axis=ax)
    return t.reshape(R, K)


def _fp32_quantize(v, bits, mode, rotate=True):
    qmax = F(O.QMAX[bits])
    z = _fp32_rotate(v) if rotate else np.asarray(v, F)
    R, K = z.shape
    u = P._unit_view(z, mode)
    am = np.abs(u).max(axis=1).astype(F)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.where(am > 0, qmax / am, F(0)).astype(F)
        if rotate:
            prod = (u * inv[:, None]).astype(F)
        else:   # unrotated bf16 inputs: the correctly rounded quotient (x qmax) / amax
            prod = np.where(am[:, None] > 0, (u * qmax) / am[:, None], F(0)).astype(F)
    codes = np.rint(prod).astype(np.int8).reshape(R, K)
    post = F(1 / 16) if rotate else F(1)
    scales = ((am / qmax).astype(F) * post).astype(F)
    shape = {"tensor": (1,), "row": (R,), "group64": (R, K // 64)}[mode]
    return codes, scales.reshape(shape)


CASES = [(4, "row"), (8, "row"), (4, "group64"), (4, "tensor"), (8, "tensor")]


@pytest.mark.parametrize("bits,mode", CASES)
def test_float32_kernel_arithmetic_passes(bits, mode):
    rng = np.random.default_rng(bits * 7 + len(mode))
    x = rng.standard_normal((96, 1536)).astype(np.float32)
    x, _ = W.with_outlier_channels(rng, x, 15, 30.0)
    xb = W.to_bf16_bits(x)
    xf = O.bf16_bits_to_f64(xb)
    codes, scales = _fp32_quantize(xf.astype(F), bits, mode)
    xr = O.rotate(xf)
    st = P.check_codes(codes, scales, xr, P.rotation_error_bound(xf), bits, mode)
    assert st["scale_ulp_max"] <= st["scale_ulp_bound"]


def test_float32_unrotated_and_norm_inputs_pass():
    rng = np.random.default_rng(3)
    M, K = 40, 1024
    x = (rng.standard_normal((M, K)) * rng.uniform(0.05, 20, (M, 1))).astype(np.float32)
    xb = W.to_bf16_bits(x)
    g = W.to_bf16_bits(1 + 0.1 * rng.standard_normal(K))
    sc = W.to_bf16_bits(0.2 * rng.standard_normal(K))
    sh = W.to_bf16_bits(0.1 * rng.standard_normal(K))
    xf = O.bf16_bits_to_f64(xb)
    codes, scales = _fp32_quantize(xf.astype(F), 4, "row", rotate=False)
    P.check_codes(codes, scales, xf, P.rotation_error_bound(xf, None, rotate=False), 4, "row", budget=0.0)
    # the norm in float32, as the kernel orders it
    h, herr = P.norm_input_error(xb, g, sc, sh, 1e-5)
    xs = xf.astype(F)
    ss = np.zeros(M, F)
    for k in range(K):
        ss = (ss + xs[:, k] * xs[:, k]).astype(F)
    r = (F(1) / np.sqrt((ss / F(K) + F(1e-5)).astype(F))).astype(F)
    gg = (O.bf16_bits_to_f64(g).astype(F) * (F(1) + O.bf16_bits_to_f64(sc).astype(F))).astype(F)
    hg = ((xs * r[:, None]).astype(F) * gg[None, :] + O.bf16_bits_to_f64(sh).astype(F)[None, :]).astype(F)
    assert (np.abs(hg - h) <= herr).all()
    for bits, mode in [(8, "row"), (4, "group64")]:
        codes, scales = _fp32_quantize(hg, bits, mode)
        P.check_codes(codes, scales, O.rotate(h), P.rotation_error_bound(h, herr), bits, mode)


def test_rotation_bound_holds_for_float32_butterflies():
    rng = np.random.default_rng(4)
    for scale in (1e-3, 1.0, 300.0):
        x = O.bf16_bits_to_f64(W.to_bf16_bits((rng.standard_normal((64, 2048)) * scale).astype(np.float32)))
        x[:, ::97] *= 60
        x = O.bf16_bits_to_f64(W.to_bf16_bits(x.astype(np.float32)))
        z32 = _fp32_rotate(x.astype(F)).astype(np.float64) / 16
        assert (np.abs(z32 - O.rotate(x)) <= P.rotation_error_bound(x)).all()


def _case(seed=5, bits=4, mode="row"):
    rng = np.random.default_rng(seed)
    x = O.bf16_bits_to_f64(W.to_bf16_bits(rng.standard_normal((64, 1024)).astype(np.float32)))
    codes, scales = _fp32_quantize(x.astype(F), bits, mode)
    return x, O.rotate(x), codes, scales


def test_planted_flip_away_from_a_tie_fails():
    x, xr, codes, scales = _case()
    t = O.code_ratio(xr, 4, "row")
    i = np.argwhere(np.abs(t - np.rint(t)) < 0.3)[0]
    bad = codes.copy()
    bad[tuple(i)] += 1 if bad[tuple(i)] < 7 else -1
    with pytest.raises(AssertionError, match="not near-ties"):
        P.check_codes(bad, scales, xr, P.rotation_error_bound(x), 4, "row")


def test_planted_flips_over_budget_fail():
    x, xr, codes, scales = _case(6, 8, "row")
    # move every code whose quotient lies within the window of a tie to the
    # other side: all are near-ties, but far more than the budget allows
    t = O.code_ratio(xr, 8, "row")
    near = np.abs(np.abs(t - np.floor(t)) - 0.5) < 2e-2
    assert near.sum() > 1e-4 * t.size
    bad = codes.copy()
    other = np.where(np.rint(t) == np.floor(t), np.floor(t) + 1, np.floor(t))
    bad[near] = other[near]
    with pytest.raises(AssertionError):
        P.check_codes(bad, scales, xr, P.rotation_error_bound(x) * 1e4, 8, "row")


@pytest.mark.parametrize("mode", ["row", "group64", "tensor"])
def test_planted_scale_error_fails(mode):
    x, xr, codes, scales = _case(7, 4, mode)
    bad = scales.copy().reshape(-1)
    bad[0] = np.nextafter(np.nextafter(bad[0], F(np.inf)), F(np.inf)) * F(1 + 2 ** -12)
    with pytest.raises(AssertionError, match="scales off"):
        P.check_codes(codes, bad.reshape(scales.shape), xr, P.rotation_error_bound(x), 4, mode)


def _fp32_group_epilogue(qa, qw):
    """y = sum_g fl(part_g) * fl(s_a s_w), accumulated in group order with a
    fused multiply-add (product exact, one float32 rounding per step)."""
    K = qa.codes.shape[1]
    sa = np.asarray(qa.scales, F)
    sw = np.asarray(qw.scales, F)
    y = np.zeros((qa.codes.shape[0], qw.codes.shape[0]), F)
    for g in range(K // 64):
        sl = slice(64 * g, 64 * g + 64)
        part = O.int_gemm(qa.codes[:, sl], qw.codes[:, sl]).astype(F)
        s = (sa[:, g][:, None] * sw[:, g][None, :]).astype(F)
        y = (part.astype(np.float64) * s.astype(np.float64) + y.astype(np.float64)).astype(F)
    return y


def test_group64_float32_epilogue_passes_and_planted_error_fails():
    rng = np.random.default_rng(8)
    xb = W.to_bf16_bits(rng.standard_normal((48, 2048)).astype(np.float32))
    wb = W.to_bf16_bits((0.02 * rng.standard_normal((80, 2048))).astype(np.float32))
    qa = O.quantize_activations(xb, 4, "group64")
    qw = O.quantize_weights(wb, 4, "group64")
    y32 = _fp32_group_epilogue(qa, qw)
    y, dy = P.linear_bound(qa, qw)
    got = O.bf16_round(y32.astype(np.float64))
    P.assert_outputs_close(got, y, dy)
    bad = got.copy()
    bad[3, 5] = O.bf16_round(bad[3, 5] * (1 + 3 * 2.0 ** -8))
    with pytest.raises(AssertionError):
        P.assert_outputs_close(bad, y, dy)


def test_swiglu_and_residual_bounds_cover_float32_evaluation():
    rng = np.random.default_rng(9)
    y = rng.standard_normal((32, 64)) * 3
    y32 = y.astype(F)
    dy = np.abs(y32.astype(np.float64) - y)
    out, d = P.epilogue_with_bound(y, dy, "swiglu")
    g, u = y32[:, :32], y32[:, 32:]
    o32 = (g / (F(1) + np.exp(-g)) * u).astype(F)
    P.assert_outputs_close(O.bf16_round(o32.astype(np.float64)), out, d)
    res = rng.standard_normal((32, 64))
    gate = rng.standard_normal(64)
    out, d = P.epilogue_with_bound(y, dy, "gated_residual", res, gate)
    o32 = (res.astype(F) + gate.astype(F)[None, :] * y32).astype(F)
    P.assert_outputs_close(O.bf16_round(o32.astype(np.float64)), out, d)


# ---------------------------------------------------------------- MX --------

def _fp32_mx(v, fmt, rotate=True):
    """The MX kernel's arithmetic: z = H x in float32, the block maximum in
    float32, its exponent, an exact division by the power of two, then the
    element rounding (the hardware conversion rounds exactly representable
    float32 values to nearest even, saturating)."""
    z = _fp32_rotate(v) if rotate else np.asarray(v, F)
    R, K = z.shape
    zb = z.reshape(R, K // 32, 32)
    m = np.abs(zb).max(axis=2)
    _, k = np.frexp(m)
    off = 4 if rotate else 0
    e = np.where(m > 0, k.astype(np.int64) - 1 - O.MX_FORMATS[fmt].emax - off, -127)
    e = np.clip(e, -127, 127)
    s = np.ldexp(zb.astype(np.float64), -(e + off)[:, :, None])
    return O.mx_round_element(s, fmt).reshape(R, K), e


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_mx_float32_kernel_arithmetic_passes(fmt):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 1024)) * rng.uniform(0.01, 50, (64, 1))).astype(np.float32)
    x, _ = W.with_outlier_channels(rng, x, 10, 30.0)
    xf = O.bf16_bits_to_f64(W.to_bf16_bits(x))
    codes, e = _fp32_mx(xf, fmt)
    st = P.check_mx(codes, e, O.rotate(xf), P.rotation_error_bound(xf), fmt)
    assert st["exp_flips"] <= 1
    codes, e = _fp32_mx(xf, fmt, rotate=False)
    st = P.check_mx(codes, e, xf, P.rotation_error_bound(xf, None, rotate=False), fmt, budget=0.0)
    assert st["code_flips"] == 0 and st["exp_flips"] == 0


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_mx_planted_mistakes_fail(fmt):
    rng = np.random.default_rng(12)
    xf = O.bf16_bits_to_f64(W.to_bf16_bits(rng.standard_normal((8, 256)).astype(np.float32)))
    bound = P.rotation_error_bound(xf, None, rotate=False)
    codes, e = _fp32_mx(xf, fmt, rotate=False)
    P.check_mx(codes, e, xf, bound, fmt, budget=0.0)
    bad_e = e.copy()
    bad_e[3, 2] += 1                                       # a block exponent one too large
    with pytest.raises(AssertionError, match="exponents"):
        P.check_mx(codes, bad_e, xf, bound, fmt, budget=1.0)
    f = O.MX_FORMATS[fmt]
    bad = codes.copy()
    mag = bad & (f.sign_bit - 1)
    i = np.argwhere((mag > 1) & (mag < f.maxcode - 1))[0]  # a mid-grid code, one step up
    bad[tuple(i)] += 1
    with pytest.raises(AssertionError, match="rounding window"):
        P.check_mx(bad, e, xf, bound, fmt, budget=1.0)
    neg0 = codes.copy()
    j = np.argwhere(neg0 == 0)
    if len(j):
        neg0[tuple(j[0])] = f.sign_bit                     # -0 instead of +0
        with pytest.raises(AssertionError, match="sign bit"):
            P.check_mx(neg0, e, xf, bound, fmt, budget=1.0)


def test_mx_exponent_window_at_a_power_of_two():
    # a block maximum just below 4 with an error bound that reaches past it:
    # both exponents are acceptable, each with the codes it implies
    x = np.zeros((1, 32))
    x[0, 0] = 4.0 * (1 - 2.0 ** -30)
    x[0, 1] = 1.3
    bound = np.full_like(x, 2.0 ** -26)
    q = O.mx_quantize(x, "fp4")
    assert q.exps[0, 0] == -1
    P.check_mx(q.codes, q.exps, x, bound, "fp4", budget=1.0)
    up = O.mx_quantize(x * (1 + 2.0 ** -28), "fp4")       # the neighbour past the power of two
    assert up.exps[0, 0] == 0
    st = P.check_mx(up.codes, up.exps, x, bound, "fp4", budget=1.0)
    assert st["exp_flips"] == 1
    with pytest.raises(AssertionError):
        P.check_mx(up.codes, up.exps, x, np.zeros_like(x), "fp4", budget=1.0)


def test_mx_product_bound_catches_a_wrong_block_scale():
    rng = np.random.default_rng(13)
    qa = O.mx_quantize(rng.standard_normal((8, 512)), "fp4")
    qw = O.mx_quantize(rng.standard_normal((16, 512)) * 0.02, "fp4")
    y, dy = P.mx_product_bound(qa, qw)
    got = y.astype(np.float32).astype(np.float64)
    P.assert_outputs_close(got, y, dy, bf16=False, what="fp32 rounding")
    wrong = qa.exps.copy()
    wrong[0, 5] += 1
    y2 = O.mx_gemm(O.MXResult(qa.codes, wrong, "fp4", None), qw)
    with pytest.raises(AssertionError):
        P.assert_outputs_close(y2, y, dy, bf16=False, what="wrong scale")


def test_mx_fp8_group_truncation_within_bound():
    # the FP8 instruction's measured arithmetic: products truncated toward
    # zero to 2^(E - 13) inside groups of adjacent elements (emulated with
    # groups of 8, larger than any measured interaction), then exact sums
    rng = np.random.default_rng(14)
    qa = O.mx_quantize(rng.standard_normal((6, 512)) * np.exp(rng.uniform(-3, 3, (6, 512))), "fp8")
    qw = O.mx_quantize(rng.standard_normal((10, 512)), "fp8")
    y, dy = P.mx_product_bound(qa, qw)
    pa, pw = qa.elements(), qw.elements()
    got = np.zeros_like(y)
    for m in range(6):
        for n in range(10):
            p = pa[m] * pw[n]
            tot = 0.0
            for g in range(0, 512, 8):
                grp = p[g:g + 8]
                top = np.abs(grp).max()
                if top > 0:
                    step = 2.0 ** (np.floor(np.log2(top)) - 13)
                    grp = np.trunc(grp / step) * step
                b = g // 32
                tot += grp.sum() * 2.0 ** (qa.exps[m, b] + qw.exps[n, b])
            got[m, n] = np.float32(tot)
    P.assert_outputs_close(got, y, dy, bf16=False, what="truncated groups")
    # a grid one binade coarser than the bound allows fails somewhere
    bad = got + 40 * dy
    with pytest.raises(AssertionError):
        P.assert_outputs_close(bad, y, dy, bf16=False, what="too coarse")


def test_bf16_unit_roundoff_is_tight():
    # |bf16(x) - x| <= BF16_U |x| for every x, and the worst case comes close
    # to it (a value just above 1 + 2^-8 rounds down by almost 2^-8 of itself)
    rng = np.random.default_rng(15)
    x = np.concatenate([rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000)),
                        [1 + 2.0 ** -8 - 2.0 ** -30, 0.5455]])
    rel = np.abs(O.bf16_round(x) - x) / np.abs(x)
    assert rel.max() <= P.BF16_U
    assert rel.max() > 0.99 * P.BF16_U / (1 + 2.0 ** -8)
