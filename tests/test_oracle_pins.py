"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks one oracle function against a closed form, an independent
construction, an invariant, a brute-force loop or a worked example, chosen so
that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, a wrong rounding mode) fails at least one of them.
"""

import itertools

import numpy as np
import pytest
import torch

import oracle as O
from workloads import to_bf16_bits, tiny_w4a4


# ---------------------------------------------------------------- Hadamard --

def _kron_h256(golden):
    h4 = np.array([[int(v) for v in ln.split()] for ln in golden("regular_hadamard_4.txt")])
    h = h4
    for _ in range(3):
        h = np.kron(h, h4)
    return h4, h


def test_h4_block_is_regular_hadamard(golden):
    h4, _ = _kron_h256(golden)
    assert (h4 @ h4.T == 4 * np.eye(4, dtype=int)).all()
    assert (h4.sum(axis=1) == 2).all()


def test_hadamard_closed_form_equals_kronecker_power(golden):
    _, hk = _kron_h256(golden)
    assert (O.regular_hadamard_256() == hk).all()


def test_hadamard_orthogonal_symmetric_regular():
    h = O.regular_hadamard_256()
    assert set(np.unique(h)) == {-1, 1}
    assert (h == h.T).all()
    assert (h @ h.T == 256 * np.eye(256, dtype=np.int64)).all()
    assert (h.sum(axis=0) == 16).all() and (h.sum(axis=1) == 16).all()


def test_constant_vector_is_fixed_and_one_hot_spreads():
    # Regularity: the constant vector is an eigenvector of H/16 with eigenvalue 1.
    ones = np.ones((1, 256))
    assert (O.rotate(ones) == ones).all()
    # A single outlier of size 20 spreads to +-20/16 in all 256 slots.
    e = np.zeros((1, 256))
    e[0, 37] = 20.0
    r = O.rotate(e)
    assert np.allclose(np.abs(r), 20.0 / 16.0, rtol=0, atol=0)


# ---------------------------------------------------------------- rotation --

def _bf16_vals(rng, shape, scale=1.0):
    return O.bf16_bits_to_f64(to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32)))


def test_rotation_is_exact_involution():
    rng = np.random.default_rng(1)
    x = _bf16_vals(rng, (8, 1024))
    x[:, 5] *= 30
    assert (O.rotate(O.rotate(x)) == x).all()


def test_rotation_matches_radix4_digit_transform():
    # Independent derivation: view each group as a 4x4x4x4 tensor over the
    # base-4 digits of the channel index and apply H4/2 along every axis.
    rng = np.random.default_rng(2)
    x = _bf16_vals(rng, (3, 512))
    h4 = np.ones((4, 4)) - 2 * np.eye(4)
    t = x.reshape(3, 2, 4, 4, 4, 4)
    for ax in range(2, 6):
        t = np.moveaxis(np.tensordot(t, h4 / 2, axes=([ax], [0])), -1, ax)
    assert np.array_equal(t.reshape(3, 512), O.rotate(x))


def test_rotation_is_only_along_aligned_groups():
    rng = np.random.default_rng(3)
    x = _bf16_vals(rng, (2, 512))
    r = O.rotate(x)
    x2 = x.copy()
    x2[:, 300] += 1.0          # a change in group 1 must leave group 0 alone
    r2 = O.rotate(x2)
    assert (r2[:, :256] == r[:, :256]).all() and not (r2[:, 256:] == r[:, 256:]).all()
    with pytest.raises(ValueError):
        O.rotate(np.zeros((1, 320)))


def test_rotation_preserves_products():
    rng = np.random.default_rng(4)
    x = _bf16_vals(rng, (16, 768))
    w = _bf16_vals(rng, (12, 768), 0.02)
    ref = x @ w.T
    got = O.rotate(x) @ O.rotate(w).T
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


# --------------------------------------------------------------- quantizer --

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("mode", ["tensor", "row", "group64"])
def test_quantizer_error_bound_range_and_sign(bits, mode):
    rng = np.random.default_rng(5)
    x = _bf16_vals(rng, (6, 512))
    x[:, 7] *= 25
    xr = O.rotate(x)
    q, s = O.quantize(xr, bits, mode)
    qmax = O.QMAX[bits]
    deq = O.dequantize(q, s, mode)
    smat = O.dequantize(np.ones_like(q), s, mode)
    # |x - s q| <= s/2 up to the float32 rounding of the scale.
    assert (np.abs(xr - deq) <= smat * (0.5 + 1e-5) + 1e-30).all()
    assert np.abs(q).max() <= qmax
    # Each unit's absmax maps to +-qmax exactly.
    units = {"tensor": q.reshape(1, -1), "row": q, "group64": q.reshape(-1, 64)}[mode]
    assert (np.abs(units).max(axis=1) == qmax).all()
    nz = q != 0
    assert (np.sign(q[nz]) == np.sign(xr[nz])).all()


def test_quantizer_zero_unit_and_ties_to_even():
    # rotate off: one row whose absmax is 7, so the reciprocal is exactly 1
    x = np.array([[7.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 6.5] + [0.0] * 56,
                  [0.0] * 64])
    q, s = O.quantize(x, 4, "row")
    assert q[0, :8].tolist() == [7, 2, 4, -2, 0, 2, 0, 6]
    assert s[0] == np.float32(1.0)
    assert s[1] == 0 and (q[1] == 0).all()


def test_quantizer_scale_is_float32_absmax_over_qmax():
    x = np.zeros((1, 64))
    x[0, 3] = -3.0
    q, s = O.quantize(x, 8, "row")
    assert s.dtype == np.float32 and s[0] == np.float32(3.0 / 127)
    assert q[0, 3] == -127


def test_code_is_float64_quotient_not_float32_reciprocal_product():
    """The code is round-half-even of the quotient x' * qmax / a.  Here
    x' * 7 / 1 = 3.5 - 2^-28 exactly up to float64 rounding, which lies
    below the tie, so the code is 3.  Rounding x' to float32 first (it
    becomes 0.5) and multiplying by a float32 reciprocal gives exactly 3.5,
    which ties to the even 4: the two recipes part at this near-tie, and the
    definition decides."""
    t = (3.5 - 2.0 ** -28) / 7.0
    x = np.array([[1.0, t, -t, 0.0] + [0.0] * 60])
    q, s = O.quantize(x, 4, "row")
    assert q[0, :4].tolist() == [7, 3, -3, 0]
    assert s[0] == np.float32(1.0 / 7.0)
    f32 = np.rint(np.float32(t) * np.float32(7.0))   # the float32 recipe lands on the tie
    assert f32 == 4.0
    assert np.allclose(O.code_ratio(x, 4, "row")[0, :3], [7.0, 3.5 - 2.0 ** -28, -(3.5 - 2.0 ** -28)],
                       rtol=0, atol=1e-15)


def test_scale_is_the_correctly_rounded_float32_quotient():
    """s = a / qmax rounded once to float32, checked against exact rational
    arithmetic (round half to even on the exact quotient), including an
    exact float32 midpoint and random float64 absmax values."""
    from fractions import Fraction

    def exact_f32(a, qmax):
        v = Fraction(a) / qmax
        f = np.float32(float(v))
        cands = sorted({f, np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))},
                       key=lambda c: (abs(Fraction(float(c)) - v), int(np.float32(c).view(np.uint32)) & 1))
        return cands[0]

    rng = np.random.default_rng(12)
    vals = list(np.ldexp(rng.random(400) + 0.5, rng.integers(-30, 30, 400)))
    vals += [7.0 * (1.0 + 2.0 ** -24), 127.0 * (1.0 + 3 * 2.0 ** -24), 7.0, 127.0 * 2.0 ** -20]
    for qmax in (7, 127):
        for a in vals:
            x = np.zeros((1, 64))
            x[0, 5] = a
            _, s = O.quantize(x, 4 if qmax == 7 else 8, "row")
            assert s[0] == exact_f32(a, qmax), (a, qmax)
    # a / 7 = 1 + 2^-24 exactly: a float32 midpoint, which rounds to the even 1.0
    x = np.zeros((1, 64))
    x[0, 0] = 7.0 * (1.0 + 2.0 ** -24)
    assert O.quantize(x, 4, "row")[1][0] == np.float32(1.0)


def test_rotation_lowers_outlier_quantization_error():
    # The pages' reason for the rotation: outlier channels wreck a shared
    # scale unless they are spread first.  Holds on every seed of the tiny
    # tensorwise workload.
    for seed in range(10):
        wl = tiny_w4a4(seed)
        x = O.bf16_bits_to_f64(wl.x)
        err = {}
        for rot in (True, False):
            xr = O.rotate(x) if rot else x
            q, s = O.quantize(xr, 4, "tensor")
            d = O.dequantize(q, s, "tensor")
            d = O.rotate(d) if rot else d
            err[rot] = np.linalg.norm(d - x) / np.linalg.norm(x)
        assert err[True] < err[False]


# ----------------------------------------------------------------- packing --

def test_pack_layout_worked_example(golden):
    for ln in golden("int4_pack_layout.txt"):
        codes, hexes = ln.split("|")
        q = np.array([[int(v) for v in codes.split()]], dtype=np.int8)
        want = np.array([[int(h, 16) for h in hexes.split()]], dtype=np.uint8)
        assert (O.pack_int4(q) == want).all(), ln
        assert (O.unpack_int4(want) == q).all(), ln


def test_pack_roundtrip_random():
    rng = np.random.default_rng(6)
    q = rng.integers(-8, 8, size=(5, 256)).astype(np.int8)
    p = O.pack_int4(q)
    assert p.shape == (5, 128) and p.dtype == np.uint8
    assert (O.unpack_int4(p) == q).all()


# ------------------------------------------------------------ integer GEMM --

def _brute_gemm(qa, qw):
    M, K = qa.shape
    N = qw.shape[0]
    out = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        for n in range(N):
            out[m, n] = sum(int(qa[m, k]) * int(qw[n, k]) for k in range(K))
    return out


@pytest.mark.parametrize("qmax", [7, 127])
def test_int_gemm_equals_brute_force(qmax):
    rng = np.random.default_rng(7)
    for M, N, K in [(1, 1, 64), (3, 5, 128), (7, 4, 256)]:
        qa = rng.integers(-qmax, qmax + 1, size=(M, K)).astype(np.int8)
        qw = rng.integers(-qmax, qmax + 1, size=(N, K)).astype(np.int8)
        assert (O.int_gemm(qa, qw) == _brute_gemm(qa, qw)).all()


def test_int_gemm_closed_forms_and_bound():
    K = 5120
    ones = np.ones((2, K), dtype=np.int8)
    assert (O.int_gemm(ones, ones) == K).all()
    full = np.full((1, K), 127, dtype=np.int8)
    assert O.int_gemm(full, -full)[0, 0] == -K * 127 * 127
    assert K * 127 * 127 < 2 ** 31           # int32 accumulators suffice at K=5120
    assert 20480 * 127 * 127 < 2 ** 31        # and at the ff.down K=20480


def test_grouped_partials_sum_to_total():
    rng = np.random.default_rng(8)
    qa = rng.integers(-7, 8, size=(4, 256)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(3, 256)).astype(np.int8)
    g = O.int_gemm_grouped(qa, qw, 64)
    assert g.shape == (4, 4, 3)
    assert (g.sum(axis=0) == O.int_gemm(qa, qw)).all()
    assert (g[1] == _brute_gemm(qa[:, 64:128], qw[:, 64:128])).all()


# ------------------------------------------------------------- dequantize --

def test_dequant_product_matches_scaled_accumulator():
    rng = np.random.default_rng(9)
    x = _bf16_vals(rng, (5, 256))
    w = _bf16_vals(rng, (3, 256), 0.02)
    qa = O.QuantResult(*O.quantize(O.rotate(x), 4, "row"), 4, "row", None)
    qw = O.QuantResult(*O.quantize(O.rotate(w), 4, "row"), 4, "row", None)
    acc = _brute_gemm(qa.codes, qw.codes)
    want = np.array([[acc[m, n] * float(qa.scales[m]) * float(qw.scales[n])
                      for n in range(3)] for m in range(5)])
    got = O.linear_fp64(qa, qw)
    assert np.allclose(got, want, rtol=1e-14, atol=0)


def test_zero_accumulator_gives_exact_zero():
    # Codes whose integer product is 0 must dequantize to exactly 0, whatever
    # the scales (the integer sum is exact; scaling happens afterwards).
    qa = np.zeros((2, 256), np.int8)
    qw = np.zeros((3, 256), np.int8)
    qa[0, :4] = [3, -5, 7, 1]
    qw[0, :4] = [5, 3, 0, 0]                 # 15 - 15 = 0
    qw[1, :4] = [1, 1, 1, -3]                # 3 - 5 + 7 - 3 = 2
    for mode, sa, sw in [("row", np.float32([0.1234567, 3.3]), np.float32([0.0771, 1.7, 2.9])),
                         ("tensor", np.float32([0.1234567]), np.float32([0.0771]))]:
        a = O.QuantResult(qa, sa, 4, mode, None)
        w = O.QuantResult(qw, sw, 4, mode, None)
        y = O.linear_fp64(a, w)
        assert y[0, 0] == 0.0 and y[0, 2] == 0.0 and y[1].tolist() == [0.0, 0.0, 0.0]
        assert y[0, 1] == 2 * float(sa[0]) * float(sw[1 if mode == "row" else 0])
    g = O.QuantResult(qa, np.full((2, 4), 0.3, np.float32), 4, "group64", None)
    gw = O.QuantResult(qw, np.full((3, 4), 0.7, np.float32), 4, "group64", None)
    assert O.linear_fp64(g, gw)[0, 0] == 0.0


def test_group64_dequant_matches_per_group_loop():
    rng = np.random.default_rng(10)
    x = _bf16_vals(rng, (3, 256))
    w = _bf16_vals(rng, (2, 256), 0.02)
    qa = O.QuantResult(*O.quantize(O.rotate(x), 4, "group64"), 4, "group64", None)
    qw = O.QuantResult(*O.quantize(O.rotate(w), 4, "group64"), 4, "group64", None)
    want = np.zeros((3, 2))
    for m, n, g in itertools.product(range(3), range(2), range(4)):
        sl = slice(64 * g, 64 * g + 64)
        acc = int(np.dot(qa.codes[m, sl].astype(np.int64), qw.codes[n, sl].astype(np.int64)))
        want[m, n] += acc * float(qa.scales[m, g]) * float(qw.scales[n, g])
    assert np.allclose(O.linear_fp64(qa, qw), want, rtol=1e-14, atol=0)


# --------------------------------------------------- grid-exact end to end --

def _grid_rows(rng, R, K, c, qmax, span):
    """Rows whose rotated image lies on the quantization grid c*{-qmax..qmax}:
    every aligned ``span`` channels hold one +-qmax*c entry (so every scale
    unit sees the same absmax) and one smaller grid entry, zeros elsewhere.
    Sparse enough that the rotated rows are exact bf16 values."""
    xr = np.zeros((R, K))
    for r in range(R):
        for g in range(K // span):
            pos = rng.choice(span, size=2, replace=False) + span * g
            xr[r, pos[0]] = c * qmax * rng.choice([-1, 1])
            xr[r, pos[1]] = c * rng.integers(-qmax + 1, qmax)
    return xr


@pytest.mark.parametrize("bits,mode,span", [(4, "row", 64), (4, "tensor", 64),
                                            (4, "group64", 64), (8, "row", 256),
                                            (8, "tensor", 256)])
def test_grid_inputs_reproduce_exact_matmul(bits, mode, span):
    """If the rotated operands already lie on their quantization grids, the
    whole quantized linear must equal the exact product X W^T: this pins the
    rotation direction, the scale, the codes, the integer product and the
    dequantization together."""
    rng = np.random.default_rng(11)
    qmax = O.QMAX[bits]
    M, N, K = 4, 6, 512
    xr = _grid_rows(rng, M, K, 2.0 ** -6, qmax, span)
    wr = _grid_rows(rng, N, K, 2.0 ** -9, qmax, span)
    x = O.rotate(xr)          # rotation is its own inverse: rotate(x) == xr
    w = O.rotate(wr)
    assert (O.bf16_round(x) == x).all() and (O.bf16_round(w) == w).all()
    xb = O.f64_to_bf16_bits(x)
    wb = O.f64_to_bf16_bits(w)
    out, y, qa, qw = O.linear(xb, wb, bits, bits, mode)
    assert (qa.codes == np.rint(xr / 2.0 ** -6)).all()
    assert (qw.codes == np.rint(wr / 2.0 ** -9)).all()
    assert np.array_equal(y, x @ w.T)
    assert (out == O.f64_to_bf16_bits(x @ w.T)).all()


# ---------------------------------------------------------------- low rank --

def test_low_rank_branch_identity():
    rng = np.random.default_rng(13)
    M, N, K, r = 5, 8, 256, 16
    xb = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wb = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    l1 = to_bf16_bits((rng.standard_normal((K, r)) * 0.02).astype(np.float32))
    l2 = to_bf16_bits((rng.standard_normal((r, N)) * 0.02).astype(np.float32))
    qa = O.quantize_activations(xb, 4, "group64")
    qw = O.quantize_weights(wb, 4, "group64")
    base = O.linear_fp64(qa, qw)
    with_branch = O.linear_fp64(qa, qw, xb, l1, l2)
    x = O.bf16_bits_to_f64(xb)
    # (W + L2^T L1^T)-style merged form: X (L1 L2) == (X L1) L2
    merged = base + x @ (O.bf16_bits_to_f64(l1) @ O.bf16_bits_to_f64(l2))
    assert np.allclose(with_branch, merged, rtol=1e-12, atol=1e-15)
    # rank 0 reduces to the plain quantized product
    empty1 = np.zeros((K, 0), np.uint16)
    empty2 = np.zeros((0, N), np.uint16)
    assert (O.linear_fp64(qa, qw, xb, empty1, empty2) == base).all()


# --------------------------------------------------------------- epilogues --

def test_silu_textbook_values(golden):
    for ln in golden("silu_values.txt"):
        z, v = (float(t) for t in ln.split())
        assert O.silu(np.array([z]))[0] == pytest.approx(v, rel=1e-15, abs=1e-300)


def test_swiglu_pairs_first_half_gate_with_second_half_up():
    y = np.array([[1.0, 2.0, 3.0, 4.0]])
    out = O.epilogue(y, "swiglu")
    assert out.shape == (1, 2)
    assert np.allclose(out, [[O.silu(np.array([1.0]))[0] * 3.0, O.silu(np.array([2.0]))[0] * 4.0]])


def test_gated_residual_special_cases():
    rng = np.random.default_rng(14)
    y = rng.standard_normal((3, 4))
    res = rng.standard_normal((3, 4))
    assert (O.epilogue(y, "gated_residual", res, np.zeros(4)) == res).all()
    assert (O.epilogue(y, "gated_residual", np.zeros((3, 4)), np.ones(4)) == y).all()
    gate = np.array([0.0, 1.0, 2.0, -1.0])
    assert np.allclose(O.epilogue(y, "gated_residual", res, gate), res + y * gate[None, :])


# ------------------------------------------------------------ bf16 casting --

def test_bf16_rounding_worked_examples(golden):
    for ln in golden("bf16_rounding.txt"):
        f32_hex, bf_hex = ln.split()
        f = np.array([int(f32_hex, 16)], dtype=np.uint32).view(np.float32).astype(np.float64)
        assert int(O.f64_to_bf16_bits(f)[0]) == int(bf_hex, 16), ln


def test_bf16_rounding_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(15)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(f.astype(np.float64))
    assert (got == want).all()


def test_bf16_widening_is_exact():
    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    assert (O.f64_to_bf16_bits(v[fin]) == bits[fin]).all()


# ------------------------------------------- RMSNorm + modulation prologue --

def test_rmsnorm_gives_unit_mean_square_without_eps():
    # with eps = 0 and no modulation every row of h has mean square exactly 1
    rng = np.random.default_rng(21)
    x = to_bf16_bits(rng.normal(size=(5, 512)) * rng.uniform(0.1, 30.0, size=(5, 1)))
    h = O.rmsnorm_modulate(x, eps=0.0)
    assert np.allclose(np.mean(h * h, axis=1), 1.0, rtol=0, atol=1e-12)


def test_rmsnorm_eps_sits_inside_the_root_next_to_the_mean():
    # a constant row c: mean square c^2, so h = c / sqrt(c^2 + eps); c = 3, eps = 7 -> 3/4 exactly
    x = to_bf16_bits(np.full((2, 256), 3.0))
    h = O.rmsnorm_modulate(x, eps=7.0)
    assert np.array_equal(h, np.full((2, 256), 0.75))
    # mean (not sum) of squares: K = 256 constant channels of 1 with eps = 3 -> 1/2
    h1 = O.rmsnorm_modulate(to_bf16_bits(np.ones((1, 256))), eps=3.0)
    assert np.array_equal(h1, np.full((1, 256), 0.5))


def test_rmsnorm_is_scale_invariant_without_eps():
    rng = np.random.default_rng(22)
    xf = rng.normal(size=(3, 256))
    a = O.rmsnorm_modulate(to_bf16_bits(xf), eps=0.0)
    b = O.rmsnorm_modulate(to_bf16_bits(xf * 8.0), eps=0.0)   # power of two: the bf16 inputs scale exactly
    assert np.allclose(a, b, rtol=1e-15, atol=0)


def test_modulation_worked_example():
    # x = (1, -1, 1, -1) has mean square 1, so with eps = 0 the norm is the identity and
    # h = x * gamma * (1 + scale) + shift:
    #   gamma = (2, 1, 1, 1), scale = (0, 1, -0.5, 0), shift = (0, 0, 0, 0.25) -> (2, -2, 0.5, -0.75)
    x = to_bf16_bits(np.array([[1.0, -1.0, 1.0, -1.0]]))
    g = to_bf16_bits(np.array([2.0, 1.0, 1.0, 1.0]))
    s = to_bf16_bits(np.array([0.0, 1.0, -0.5, 0.0]))
    t = to_bf16_bits(np.array([0.0, 0.0, 0.0, 0.25]))
    assert np.array_equal(O.rmsnorm_modulate(x, g, s, t, eps=0.0), np.array([[2.0, -2.0, 0.5, -0.75]]))


def test_rmsnorm_modulate_matches_brute_force_loops():
    # per-row factor, per-channel vectors (a transposed broadcast fails: M != K and the vectors differ)
    rng = np.random.default_rng(23)
    M, K, eps = 3, 8, 0.25
    xb = to_bf16_bits(rng.normal(size=(M, K)))
    gb, sb, tb = (to_bf16_bits(rng.normal(size=K)) for _ in range(3))
    x, g, s, t = (O.bf16_bits_to_f64(v) for v in (xb, gb, sb, tb))
    want = np.zeros((M, K))
    for m in range(M):
        acc = 0.0
        for k in range(K):
            acc += x[m, k] * x[m, k]
        r = 1.0 / np.sqrt(acc / K + eps)
        for k in range(K):
            want[m, k] = x[m, k] * r * g[k] * (1.0 + s[k]) + t[k]
    assert np.allclose(O.rmsnorm_modulate(xb, gb, sb, tb, eps=eps), want, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("bits,mode", [(4, "row"), (8, "group64"), (4, "tensor")])
def test_norm_prologue_reduces_to_the_plain_prologue_when_the_norm_is_identity(bits, mode):
    # rows of +-1 have mean square 1: with eps = 0 and no modulation h == x, so the fused
    # prologue must give the plain prologue's codes and scales bit for bit
    rng = np.random.default_rng(24)
    x = to_bf16_bits(np.where(rng.random((4, 512)) < 0.5, -1.0, 1.0))
    a = O.quantize_activations_norm(x, None, None, None, 0.0, bits, mode)
    b = O.quantize_activations(x, bits, mode)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)


# ------------------------------------------------------ sigmoid gate epilogue --

def test_sigmoid_closed_form_values(golden):
    for ln in golden("sigmoid_values.txt"):
        z, want = (float(v) for v in ln.split())
        assert abs(float(O.sigmoid(np.array([z]))[0]) - want) <= 1e-15


def test_sigmoid_symmetry_range_and_silu_relation():
    z = np.linspace(-30, 30, 1201)
    s = O.sigmoid(z)
    assert np.allclose(s + O.sigmoid(-z), 1.0, rtol=0, atol=1e-15)       # sigma(-z) = 1 - sigma(z)
    assert ((s > 0) & (s < 1)).all() and (np.diff(s) > 0).all()           # increasing into (0, 1)
    assert np.allclose(O.silu(z), z * s, rtol=1e-15, atol=1e-300)         # silu(z) = z sigma(z)
    y = np.array([[0.0, 1.0986122886681098]])
    assert np.allclose(O.epilogue(y, "sigmoid"), [[0.5, 0.75]], rtol=0, atol=1e-15)


# ---- FP6 (e2m3) code layout -------------------------------------------------
# The FP6 E2M3 element of the OCP microscaling formats: largest normal 7.5,
# smallest normal 1.0, smallest subnormal 0.125, 0.875 the largest subnormal;
# bit 5 is the sign.

def test_fp6_decoder_format_constants():
    v = O.fp6_e2m3_value(np.arange(64))
    assert v[0] == 0.0 and v[1] == 0.125 and v[7] == 0.875 and v[8] == 1.0 and v[31] == 7.5
    assert v[32] == 0.0 and np.signbit(v[32]) and v[63] == -7.5
    assert np.array_equal(v[32:], -v[:32])
    assert np.all(np.diff(v[:32]) > 0)                 # magnitudes strictly increase with the pattern
    assert np.abs(v).max() == 7.5


def test_fp6_codes_are_exact_and_hand_derived():
    # patterns of |c| = 0..7 worked out by hand from the definition
    hand = {0: 0, 1: 8, 2: 16, 3: 20, 4: 24, 5: 26, 6: 28, 7: 30}
    q = np.arange(-7, 8).reshape(1, 15)
    q = np.concatenate([q, np.zeros((1, 128 - 15), dtype=q.dtype)], axis=1).astype(np.int8)
    packed = O.pack_fp6(q)
    v0 = int.from_bytes(bytes(packed[0, 0:16]) + bytes(packed[0, 64:72]), "little")
    for i, c in enumerate(range(-7, 8)):
        pat = (v0 >> (6 * i)) & 63
        assert pat == hand[abs(c)] + (32 if c < 0 else 0), c
        assert O.fp6_e2m3_value(pat) == c


def test_fp6_pack_golden_example(golden):
    q = np.zeros((1, 128), dtype=np.int8)
    q[0, 0], q[0, 1], q[0, 32], q[0, 63] = 1, -7, 3, 7
    want = np.zeros(96, dtype=np.uint8)
    for line in golden("fp6_pack_example.txt"):
        i, v = map(int, line.split())
        want[i] = v
    got = O.pack_fp6(q)
    assert got.shape == (1, 96)
    assert np.array_equal(got[0], want)
    assert np.array_equal(O.unpack_fp6(got), q)


def test_fp6_round_trip_and_rejects():
    rng = np.random.default_rng(11)
    q = rng.integers(-7, 8, size=(5, 384)).astype(np.int8)
    assert np.array_equal(O.unpack_fp6(O.pack_fp6(q)), q)
    with pytest.raises(ValueError):
        O.pack_fp6(np.full((1, 128), 8, dtype=np.int8))
    with pytest.raises(ValueError):
        O.pack_fp6(np.zeros((1, 96), dtype=np.int8))


def test_fp6_products_sum_exactly_in_float32():
    # decoded products are integers <= 49 in magnitude; a float32 running sum
    # over K = 5120 stays below 2^24 and so equals the exact integer dot
    # product, including the all-extreme row
    rng = np.random.default_rng(12)
    K = 5120
    a = rng.integers(-7, 8, size=(3, K)).astype(np.int8)
    w = rng.integers(-7, 8, size=(2, K)).astype(np.int8)
    a[0] = 7
    w[0] = 7
    w[1, ::2] = -7
    da = O.fp6_e2m3_value(O.fp6_e2m3_encode(a)).astype(np.float32)
    dw = O.fp6_e2m3_value(O.fp6_e2m3_encode(w)).astype(np.float32)
    exact = O.int_gemm(a, w)
    for i in range(3):
        for j in range(2):
            s = np.float32(0)
            for k in range(0, K, 128):             # one 128-channel block per step, as the matrix core does
                s = np.float32(s + np.float32(np.dot(da[i, k:k + 128].astype(np.float64), dw[j, k:k + 128])))
            assert int(s) == exact[i, j]
    assert exact[0, 0] == 49 * K
