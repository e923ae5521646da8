"""Pins of the MX block-scaled oracle (oracle.mx_ref) to facts outside it:
the element tables of the OCP MX v1.0 formats, an independent library
conversion (torch's float8_e4m3fn cast), hand-worked blocks, the error bound
the definition implies, and exact rational arithmetic on tiny products."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def test_e2m1_table():
    # FP4 E2M1: the eight magnitudes listed for the format
    assert O.mx_element_magnitudes("fp4").tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    f = O.MX_FORMATS["fp4"]
    assert f.emax == 2 and f.max_value == 6.0 and f.sign_bit == 8


def test_e4m3_table_matches_torch_decoding():
    mags = O.mx_element_magnitudes("fp8")
    assert len(mags) == 127                       # 0x00 .. 0x7E; 0x7F is NaN
    ref = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(mags, ref)
    f = O.MX_FORMATS["fp8"]
    assert f.emax == 8 and f.max_value == 448.0
    assert mags[1] == 2.0 ** -9 and mags[8] == 2.0 ** -6   # smallest subnormal, smallest normal


@pytest.mark.parametrize("v, code", [
    (0.0, 0), (0.2, 0), (0.25, 0), (0.26, 1),      # 0.25 ties to 0 (code 0 even)
    (0.5, 1), (0.75, 2), (0.74, 1),                # 0.75 ties up to 1.0 (code 2)
    (1.25, 2), (1.26, 3), (1.75, 4), (1.74, 3),
    (2.5, 4), (2.51, 5), (3.5, 6), (3.49, 5),
    (5.0, 6), (5.01, 7), (6.0, 7), (7.99, 7), (100.0, 7),   # saturation at 6
    (-0.2, 0), (-0.3, 9), (-5.5, 15), (-1e9, 15),            # sign bit 8; -0 stored as +0
])
def test_e2m1_rounding_hand_worked(v, code):
    assert int(O.mx_round_element(np.array([v]), "fp4")[0]) == code


def test_e4m3_rounding_matches_torch_cast_in_range():
    # every representable value, every midpoint, and points a quarter step either side
    mags = O.mx_element_magnitudes("fp8")
    mids = (mags[:-1] + mags[1:]) / 2
    steps = np.diff(mags)
    pts = np.concatenate([mags, mids, mids - steps / 4, mids + steps / 4])
    rng = np.random.default_rng(0)
    pts = np.concatenate([pts, rng.uniform(0, 448, 20000), np.exp(rng.uniform(-12, 6, 20000))])
    pts = pts[pts <= 448.0]
    v = np.concatenate([pts, -pts])
    ours = O.mx_round_element(v, "fp8")
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref = np.where((ref & 0x7F) == 0, 0, ref)      # the oracle stores every zero as +0
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_where_the_cast_overflows():
    v = np.array([448.0, 449.0, 464.0, 480.0, 1e6, -1e30])
    assert O.mx_round_element(v, "fp8").tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


@pytest.mark.parametrize("amax, e4, e8", [
    (6.5, 0, -6), (8.0, 1, -5), (7.99, 0, -6), (4.0, 0, -6), (3.99, -1, -7),
    (1.0, -2, -8), (0.3, -4, -10), (448.0, 6, 0), (512.0, 7, 1),
    (0.0, -127, -127), (2.0 ** -140, -127, -127), (2.0 ** 200, 127, 127),
])
def test_shared_exponent_hand_worked(amax, e4, e8):
    assert int(O.mx_shared_exponent(np.array([amax]), "fp4")[0]) == e4
    assert int(O.mx_shared_exponent(np.array([amax]), "fp8")[0]) == e8


def test_hand_worked_fp4_block():
    blk = np.zeros(32)
    blk[:8] = [6.5, 0.3, -1.1, 0.25, 0.75, 2.5, -3.5, 5.0]
    q = O.mx_quantize(blk[None, :], "fp4")
    assert q.exps.tolist() == [[0]]                # floor(log2 6.5) - 2 = 0: X = 1
    assert q.codes[0, :8].tolist() == [7, 1, 10, 0, 2, 4, 14, 6]
    assert q.dequant()[0, :8].tolist() == [6.0, 0.5, -1.0, 0.0, 1.0, 2.0, -4.0, 4.0]
    data, sb = O.mx_pack(q)
    assert data[0, :4].tolist() == [0x17, 0x0A, 0x42, 0x6E] and sb.tolist() == [[127]]
    codes, exps = O.mx_unpack(data, sb, "fp4")
    assert np.array_equal(codes, q.codes) and np.array_equal(exps, q.exps)


def test_hand_worked_scaled_blocks():
    # block 0: amax 12 -> e = 3 - 2 = 1, X = 2; block 1 all zero; block 2: amax 0.1 -> e = -4 - 2 = -6
    x = np.zeros((1, 96))
    x[0, 0], x[0, 1], x[0, 2] = 12.0, -3.0, 0.4
    x[0, 64], x[0, 65] = 0.1, -0.03
    q = O.mx_quantize(x, "fp4")
    assert q.exps.tolist() == [[1, -127, -6]]
    # 12/2 = 6 (code 7); -3/2 = -1.5 (code 3, negative 11); 0.4/2 = 0.2 -> 0
    assert q.codes[0, :3].tolist() == [7, 11, 0]
    # 0.1 * 64 = 6.4 -> 6 (saturated); -0.03 * 64 = -1.92 -> -2 (code 4 + 8)
    assert q.codes[0, 64:66].tolist() == [7, 12]
    assert not q.codes[0, 32:64].any()
    _, sb = O.mx_pack(q)
    assert sb.tolist() == [[128, 0, 121]]


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_block_error_bound_and_normalization(fmt):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    q = O.mx_quantize(x, fmt)
    f = O.MX_FORMATS[fmt]
    t = O.mx_ratio(x, fmt)                           # V / X
    amax_t = np.abs(t).reshape(64, -1, 32).max(axis=2)
    # the block maximum lands in the top binade: [2^emax, 2^(emax+1))
    assert np.all(amax_t >= 2.0 ** f.emax) and np.all(amax_t < 2.0 ** (f.emax + 1))
    p = q.elements()
    mags = O.mx_element_magnitudes(fmt)
    sat = np.abs(t) >= f.max_value
    # unsaturated: within half a grid step of the rounded value (the step at
    # the larger neighbour bounds it); saturated: the largest magnitude
    idx = np.abs(q.codes.astype(np.int64)) & (f.sign_bit - 1)
    step = np.diff(np.append(mags, mags[-1] * 2))[np.minimum(idx, f.maxcode)]
    step_below = np.diff(np.insert(mags, 0, 0.0))[idx]
    half = np.maximum(step, step_below) / 2
    assert np.all(np.abs(t - p)[~sat] <= half[~sat])
    assert np.all(np.abs(p[sat]) == f.max_value) and np.all(np.sign(p[sat]) == np.sign(t[sat]))
    # relative error of the whole block stays within the format's precision
    err = np.abs(q.dequant() - x).reshape(64, -1, 32).max(axis=2)
    amax = np.abs(x).reshape(64, -1, 32).max(axis=2)
    assert np.all(err <= amax * (0.25 if fmt == "fp4" else 0.125))   # saturation: (2^(emax+1) - max) / 2^(emax+1)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_gemm_against_exact_rationals(fmt):
    rng = np.random.default_rng(2)
    xa = rng.standard_normal((3, 64)) * np.array([[1.0], [1e-3], [40.0]]) * np.repeat([1.0, 16.0], 32)
    xw = rng.standard_normal((2, 64)) * np.array([[0.02], [7.0]]) * np.repeat([3.0, 0.1], 32)
    xa[1, 32:] = 0.0                                  # an all-zero block
    qa, qw = O.mx_quantize(xa, fmt), O.mx_quantize(xw, fmt)
    # distinct scales per row and block, so a transposed or misaligned
    # scale would change the sum
    assert len(set(qa.exps.ravel().tolist())) >= 4 and len(set(qw.exps.ravel().tolist())) >= 3
    y = O.mx_gemm(qa, qw)
    ex = O.mx_gemm_exact(qa, qw)
    for m in range(3):
        for n in range(2):
            assert Fraction(float(y[m, n])) == ex[m][n]   # exact: 2 blocks, no rounding


def test_gemm_equals_dequantized_product():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 512))
    w = rng.standard_normal((8, 512)) * 0.02
    qa, qw = O.mx_quantize(x, "fp4"), O.mx_quantize(w, "fp4")
    assert np.allclose(O.mx_gemm(qa, qw), qa.dequant() @ qw.dequant().T, rtol=1e-12, atol=1e-15)


def test_linear_rotation_matches_rotating_first():
    rng = np.random.default_rng(4)
    xb = O.f64_to_bf16_bits(rng.standard_normal((8, 256)))
    wb = O.f64_to_bf16_bits(rng.standard_normal((16, 256)) * 0.02)
    out, y, qa, qw = O.mx_linear(xb, wb, "fp4", rotate_on=True)
    assert np.array_equal(qa.values, O.rotate(O.bf16_bits_to_f64(xb)))
    ref = O.mx_quantize(O.rotate(O.bf16_bits_to_f64(wb)), "fp4")
    assert np.array_equal(qw.codes, ref.codes) and np.array_equal(qw.exps, ref.exps)
    # the rotation cancels (Hn Hn^T = I): y - x w^T = dA Wr^T + Ar dW^T + dA dW^T
    # with the rotated operands Ar, Wr and their quantization errors dA, dW
    exact = O.bf16_bits_to_f64(xb) @ O.bf16_bits_to_f64(wb).T
    ar, wr = qa.values, qw.values
    da, dw = qa.dequant() - ar, qw.dequant() - wr
    nrm = np.linalg.norm
    bound = nrm(da) * nrm(wr, 2) + nrm(ar, 2) * nrm(dw) + nrm(da) * nrm(dw)
    assert nrm(y - exact) <= bound * (1 + 1e-9)
    assert np.allclose(ar @ wr.T, exact, rtol=0, atol=1e-12)


def test_lowrank_branch_adds_the_exact_factor_product():
    # the branch is (X L1) L2 on the unrotated input: brute-force sums on a tiny case
    rng = np.random.default_rng(5)
    xb = O.f64_to_bf16_bits(rng.standard_normal((3, 256)))
    wb = O.f64_to_bf16_bits(rng.standard_normal((32, 256)) * 0.02)
    l1 = O.f64_to_bf16_bits(rng.standard_normal((256, 16)) * 0.1)
    l2 = O.f64_to_bf16_bits(rng.standard_normal((16, 32)) * 0.1)
    _, y0, _, _ = O.mx_linear(xb, wb, "fp4")
    _, y1, _, _ = O.mx_linear(xb, wb, "fp4", l1_bits=l1, l2_bits=l2)
    x, a, b = O.bf16_bits_to_f64(xb), O.bf16_bits_to_f64(l1), O.bf16_bits_to_f64(l2)
    for m in range(3):
        for n in (0, 17, 31):
            br = sum(sum(x[m, k] * a[k, r] for k in range(256)) * b[r, n] for r in range(16))
            assert abs((y1 - y0)[m, n] - br) <= 1e-12 * (1 + abs(br))
    # rank 0 is the plain layer; SwiGLU pairs the first half (gate) with the second (up)
    _, y2, _, _ = O.mx_linear(xb, wb, "fp4", l1_bits=l1[:, :0], l2_bits=l2[:0])
    assert np.array_equal(y2, y0)
    out, y3, _, _ = O.mx_linear(xb, wb, "fp4", epi="swiglu", l1_bits=l1, l2_bits=l2)
    g, u = y3[:, :16], y3[:, 16:]
    assert np.array_equal(out, O.f64_to_bf16_bits(g / (1 + np.exp(-g)) * u))
