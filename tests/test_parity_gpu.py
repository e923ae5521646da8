"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Acceptance (tolerances derived in tests/parity_checks.py from the kernels'
float32 arithmetic):
  * activation / weight codes: every code equals round-half-even of the
    oracle's exact quotient x' * qmax / absmax unless that quotient lies
    within the kernels' float32 error of a rounding tie, where a +-1 flip is
    allowed; flips stay at or below 1e-4 of the codes.  Unrotated bf16
    inputs take the exact decision (no flips at all);
  * scales within the float32 absmax error bound of absmax / qmax (plus
    half an ulp), reported in ulps;
  * int32 accumulators bit-exact when both sides consume the same codes;
  * outputs element by element against the oracle's dequantized product of
    the same codes, within the kernel's float32 epilogue bound plus one bf16
    ulp -- at full size on sampled rows too;
  * final bf16 outputs within 1e-2 relative Frobenius error of the oracle's
    own end-to-end result.
Inputs are the seeded synthetic workloads; sizes span several tiles of
each kernel configuration plus ragged tails.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import parity_checks as P
from tests.helpers import (bf16_bits, bf16_ulp_diff, ensure_built, pair_w4, rel_fro, to_dev, to_dev_bf16, to_dev_scales,
                           to_dev_l2, unpair_w4)

pytestmark = pytest.mark.gpu

FLIP_BUDGET = P.FLIP_BUDGET
REL_FRO = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch

    ensure_built()
    import rotated_bit_quantized_rotate_amd as Q

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert Q.device_supported(0), "device is not gfx950"
    return Q


@pytest.fixture(scope="module")
def Q(_lib):
    return _lib


def _rand_bf16(seed, shape, std=1.0, outliers=0, factor=30.0):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    if outliers:
        a, _ = W.with_outlier_channels(rng, a, outliers, factor)
    return W.to_bf16_bits(a)


def _check_prologue(got_codes, got_scales, xb, bits, mode, rotate=True, budget=None, rows=None):
    """GPU codes and scales of bf16 input xb against the oracle's definition;
    unrotated inputs must match exactly (budget 0)."""
    x = O.bf16_bits_to_f64(xb)
    xr = O.rotate(x) if rotate else x
    if budget is None:
        budget = FLIP_BUDGET if rotate else 0.0
    return P.check_codes(got_codes, got_scales, xr, P.rotation_error_bound(x, None, rotate), bits, mode,
                         budget, rows)


# --------------------------------------------------------------- prologue --

@pytest.mark.parametrize("M,K", [(1, 256), (37, 512), (300, 5120), (5, 20480), (16, 1536), (33, 6144)])
@pytest.mark.parametrize("bits,mode", [(4, "row"), (8, "row"), (4, "group64"), (4, "tensor"),
                                       (8, "tensor")])
def test_rotate_quantize_matches_oracle(Q, M, K, bits, mode):
    import torch

    xb = _rand_bf16(M * 7 + K, (M, K), outliers=max(1, K // 100))
    x = to_dev_bf16(xb)
    codes, scales, _ = Q.rotate_quantize_act(x, bits=bits, scale_mode=mode, layout="i8", rotate=True)
    torch.cuda.synchronize()
    st = _check_prologue(codes.cpu().numpy(), scales.cpu().numpy(), xb, bits, mode)
    print(f"flips {st['flip_frac']:.2e}, scale ulps {st['scale_ulp_max']:.1f} (bound {st['scale_ulp_bound']:.1f})")


@pytest.mark.parametrize("mode", ["row", "group64", "tensor"])
def test_packed_layout_and_no_rotation(Q, mode):
    import torch

    M, K = 70, 1024
    xb = _rand_bf16(3, (M, K), outliers=8)
    x = to_dev_bf16(xb)
    for rot in (True, False):
        packed, scales, _ = Q.rotate_quantize_act(x, bits=4, scale_mode=mode, layout="packed", rotate=rot)
        torch.cuda.synchronize()
        got = O.unpack_int4(packed.cpu().numpy())
        # no rotation: the decision is the exact quotient's, no flips allowed
        _check_prologue(got, scales.cpu().numpy(), xb, 4, mode, rotate=rot)


def _exact_tie_rows(bits, M, K, seed):
    """bf16 rows full of exact ties x * qmax / absmax = k + 1/2.  int4: the
    absmax is 7 c 2^e with c odd, so x = (2k + 1) c 2^(e-1) is a bf16 value;
    int8: x = +-absmax / 2 gives the tie 63.5 for any absmax."""
    rng = np.random.default_rng(seed)
    qmax = O.QMAX[bits]
    x = np.zeros((M, K), np.float64)
    for m in range(M):
        e = float(2.0 ** rng.integers(-6, 6))
        if bits == 4:
            c = int(rng.choice([3, 5, 9, 11, 13, 15, 17, 19]))    # (2k + 1) c < 256
            amax = 7 * c * e
            k = rng.integers(0, 7, size=K)
            x[m] = (2 * k + 1) * c * e / 2
        else:
            amax = float(rng.integers(129, 256)) * e / 2
            x[m] = amax / 2
        x[m, 0] = amax
        x[m, 1::3] *= -1
    assert np.array_equal(O.bf16_bits_to_f64(W.to_bf16_bits(x.astype(np.float32))), x)
    return W.to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("bits", [4, 8])
def test_unrotated_exact_ties_follow_the_definition(Q, bits):
    """Unrotated bf16 inputs hit exact ties x * qmax / absmax = k + 1/2; the
    codes must round them to even, as the definition does, with no flips.
    (A float32 reciprocal product breaks a share of these ties the other
    way; the host checks that the case really contains such ties.)"""
    import torch

    M, K = 64, 512
    xb = _exact_tie_rows(bits, M, K, 40 + bits)
    x = O.bf16_bits_to_f64(xb)
    t = O.code_ratio(x, bits, "row")
    assert (np.abs(t - np.floor(t)) == 0.5).mean() > 0.5          # mostly exact ties
    qmax = np.float32(O.QMAX[bits])
    inv = (qmax / np.abs(x).max(axis=1).astype(np.float32)).astype(np.float32)
    recip = np.rint((x.astype(np.float32) * inv[:, None]).astype(np.float32))
    assert (recip != np.rint(t)).sum() > 0                         # the product recipe breaks some
    codes, scales, _ = Q.rotate_quantize_act(to_dev_bf16(xb), bits=bits, scale_mode="row", rotate=False)
    torch.cuda.synchronize()
    _check_prologue(codes.cpu().numpy(), scales.cpu().numpy(), xb, bits, "row", rotate=False)


def test_prologue_degenerate_rows(Q):
    import torch

    M, K = 6, 512
    xb = _rand_bf16(4, (M, K))
    xb[1] = 0                                  # all-zero row: scale 0, codes 0
    xb[2] = 0
    xb[2, 17] = W.to_bf16_bits(np.array([1000.0], np.float32))[0]   # one huge outlier
    xb[3, :256] = 0                            # all-zero 64-groups
    x = to_dev_bf16(xb)
    for bits, mode in [(4, "row"), (8, "row"), (4, "group64"), (8, "tensor")]:
        codes, scales, _ = Q.rotate_quantize_act(x, bits=bits, scale_mode=mode)
        torch.cuda.synchronize()
        _check_prologue(codes.cpu().numpy(), scales.cpu().numpy(), xb, bits, mode)
        c = codes.cpu().numpy()
        assert (c[1] == 0).all()
        if mode == "row":
            # one outlier spreads to +-1000/16 over its group: exactly +-qmax there
            assert (np.abs(c[2, :256]) == O.QMAX[bits]).all() and (c[2, 256:] == 0).all()
            assert float(scales.cpu().numpy()[1]) == 0.0


def test_prologue_empty_input(Q):
    import torch

    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    codes, scales, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row")
    torch.cuda.synchronize()
    assert codes.shape == (0, 256)


def test_prologue_strided_rows(Q):
    import torch

    M, K, ld = 9, 512, 768
    xb = _rand_bf16(5, (M, ld))
    x = to_dev_bf16(xb)[:, :K]
    codes, scales, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row")
    torch.cuda.synchronize()
    _check_prologue(codes.cpu().numpy(), scales.cpu().numpy(), np.ascontiguousarray(xb[:, :K]), 4, "row")



# ------------------------------------ RMSNorm + modulation fused prologue --
# h = x * r * g + shift is formed in float32; the bound on |h_gpu - h| (the
# float32 sum of squares, the root, the modulation) joins the rotation's in
# the near-tie windows and the scale bound (tests/parity_checks.py).


def _norm_inputs(seed, M, K, vectors=True, row_spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x, _ = W.with_outlier_channels(rng, x, max(1, K // 100), 30.0)
    if row_spread:
        x *= rng.uniform(0.05, 20.0, size=(M, 1)).astype(np.float32)
    g = W.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(K)) if vectors else None
    sc = W.to_bf16_bits(0.2 * rng.standard_normal(K)) if vectors else None
    sh = W.to_bf16_bits(0.1 * rng.standard_normal(K)) if vectors else None
    return W.to_bf16_bits(x), g, sc, sh


def _dev_vec(v):
    return None if v is None else to_dev_bf16(v)


def _check_norm(got_codes, got_scales, xb, g, sc, sh, eps, bits, mode, rotate=True):
    h, herr = P.norm_input_error(xb, g, sc, sh, eps)
    hr = O.rotate(h) if rotate else h
    return P.check_codes(got_codes, got_scales, hr, P.rotation_error_bound(h, herr, rotate), bits, mode)


@pytest.mark.parametrize("M,K", [(1, 256), (37, 1536), (300, 5120), (9, 8192)])
@pytest.mark.parametrize("bits,mode", [(4, "row"), (8, "row"), (4, "group64"), (4, "tensor")])
def test_rmsnorm_prologue_matches_oracle(Q, M, K, bits, mode):
    import torch

    eps = 1e-5
    xb, g, sc, sh = _norm_inputs(M * 11 + K, M, K)
    codes, scales = Q.rmsnorm_rotate_quantize_act(to_dev_bf16(xb), _dev_vec(g), _dev_vec(sc), _dev_vec(sh),
                                                  eps=eps, bits=bits, scale_mode=mode)
    torch.cuda.synchronize()
    _check_norm(codes.cpu().numpy(), scales.cpu().numpy(), xb, g, sc, sh, eps, bits, mode)



@pytest.mark.parametrize("bits,mode", [(4, "row"), (8, "row"), (4, "group64")])
def test_rmsnorm_prologue_full_size_sampled_rows(Q, bits, mode):
    """The stack's normed prologue at its real size (16384 x 5120): the grid
    is capped, so each workgroup loops over several row blocks (the
    double-buffered row reductions); rows are independent, so the oracle
    checks a sample of them."""
    import torch

    M, K = 16384, 5120
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32)
    x *= torch.rand((M, 1), generator=g, device="cuda") * 10 + 0.1
    x = x.to(torch.bfloat16)
    gam = (1.0 + 0.1 * torch.randn((K,), generator=g, device="cuda")).to(torch.bfloat16)
    sc = (0.2 * torch.randn((K,), generator=g, device="cuda")).to(torch.bfloat16)
    sh = (0.1 * torch.randn((K,), generator=g, device="cuda")).to(torch.bfloat16)
    codes, scales = Q.rmsnorm_rotate_quantize_act(x, gam, sc, sh, eps=1e-6, bits=bits, scale_mode=mode)
    torch.cuda.synchronize()
    ri = torch.as_tensor(_sample_rows(M, 64), device="cuda")
    xb = bf16_bits(x[ri])
    _check_norm(codes[ri].cpu().numpy(), scales[ri].cpu().numpy(), xb, bf16_bits(gam), bf16_bits(sc),
                bf16_bits(sh), 1e-6, bits, mode)

def test_rmsnorm_prologue_eps_and_absent_vectors(Q):
    import torch

    # small rows next to a large eps: eps dominates r, so a misplaced eps would show
    M, K, eps = 40, 1024, 4.0
    xb, _, _, _ = _norm_inputs(31, M, K, vectors=False, row_spread=False)
    xb = W.to_bf16_bits(O.bf16_bits_to_f64(xb) * 0.25)
    for bits, mode in [(4, "row"), (8, "group64")]:
        codes, scales = Q.rmsnorm_rotate_quantize_act(to_dev_bf16(xb), eps=eps, bits=bits, scale_mode=mode)
        torch.cuda.synchronize()
        _check_norm(codes.cpu().numpy(), scales.cpu().numpy(), xb, None, None, None, eps, bits, mode)


@pytest.mark.parametrize("rot", [True, False])
def test_rmsnorm_prologue_packed_layout(Q, rot):
    import torch

    M, K = 70, 2048
    xb, g, sc, sh = _norm_inputs(32, M, K)
    packed, scales = Q.rmsnorm_rotate_quantize_act(to_dev_bf16(xb), _dev_vec(g), _dev_vec(sc), _dev_vec(sh),
                                                   eps=1e-6, bits=4, scale_mode="row", layout="packed",
                                                   rotate=rot)
    torch.cuda.synchronize()
    _check_norm(O.unpack_int4(packed.cpu().numpy()), scales.cpu().numpy(), xb, g, sc, sh, 1e-6, 4, "row", rot)


def test_rmsnorm_prologue_zero_rows_strided_and_empty(Q):
    import torch

    M, K, ld = 12, 512, 768
    rng = np.random.default_rng(33)
    xfull = W.to_bf16_bits(rng.standard_normal((M, ld)).astype(np.float32))
    xfull[2] = 0                     # zero row: h = shift (r = 1/sqrt(eps))
    xfull[5] = 0
    sh = W.to_bf16_bits(0.5 * rng.standard_normal(K))
    x = to_dev_bf16(xfull)[:, :K]
    xb = np.ascontiguousarray(xfull[:, :K])
    for shift in (sh, None):
        codes, scales = Q.rmsnorm_rotate_quantize_act(x, mod_shift=_dev_vec(shift), eps=1e-6, bits=4,
                                                      scale_mode="row")
        torch.cuda.synchronize()
        _check_norm(codes.cpu().numpy(), scales.cpu().numpy(), xb, None, None, shift, 1e-6, 4, "row")
        if shift is None:            # zero rows stay zero: scale 0, codes 0
            assert (codes.cpu().numpy()[[2, 5]] == 0).all() and (scales.cpu().numpy()[[2, 5]] == 0).all()
    empty = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    c, s_ = Q.rmsnorm_rotate_quantize_act(empty, eps=1e-6)
    torch.cuda.synchronize()
    assert c.shape == (0, K)


def test_rmsnorm_prologue_reused_by_two_gemms(Q):
    """One prepared activation feeds two projections of the same input (as
    Q|K|V|gate or gate|up share it): each GEMM output matches the oracle's
    linear of the normalized input."""
    import torch

    M, K, N1, N2 = 200, 1536, 384, 1024
    xb, g, sc, sh = _norm_inputs(34, M, K)
    codes, scales = Q.rmsnorm_rotate_quantize_act(to_dev_bf16(xb), _dev_vec(g), _dev_vec(sc), _dev_vec(sh),
                                                  eps=1e-6, bits=4, scale_mode="row")
    qa = O.quantize_activations_norm(xb, g, sc, sh, 1e-6, 4, "row", True)
    rng = np.random.default_rng(35)
    for N in (N1, N2):
        wb = W.to_bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
        wp, sw = Q.pack_weight_int4(to_dev_bf16(wb), scale_mode="row")
        out = Q.qgemm_w4a4(codes, scales, wp, sw, K)
        torch.cuda.synchronize()
        qw = O.quantize_weights(wb, 4, "row", True)
        want = O.linear_fp64(qa, qw)
        assert rel_fro(O.bf16_bits_to_f64(bf16_bits(out)), want) <= REL_FRO


@pytest.mark.parametrize("rank", [16, 32, 64, 128])
@pytest.mark.parametrize("mode", ["group64", "row"])
def test_lowrank_down_projection(Q, rank, mode):
    """lr = X @ L1 next to the quantization pass (its own launch, which
    re-reads X), with group-64 and row scales: 130 rows are nine 16-row
    blocks, the last with 2 rows."""
    import torch

    M, K = 130, 1024
    xb = _rand_bf16(6, (M, K))
    l1b = _rand_bf16(7, (K, rank), 0.02)
    _, _, lr = Q.rotate_quantize_act(to_dev_bf16(xb), bits=4, scale_mode=mode,
                                     l1=to_dev_bf16(l1b))
    torch.cuda.synchronize()
    want = O.bf16_bits_to_f64(xb) @ O.bf16_bits_to_f64(l1b)
    got = O.bf16_bits_to_f64(bf16_bits(lr))
    assert rel_fro(got, want) < 4e-3
    assert bf16_ulp_diff(bf16_bits(lr), O.f64_to_bf16_bits(want)).max() <= 1


# ------------------------------------------------------------ weight pack --

@pytest.mark.parametrize("mode", ["row", "tensor", "group64"])
def test_pack_weight_int4_matches_oracle(Q, mode):
    import torch

    N, K = 272, 1024
    wb = _rand_bf16(8, (N, K), 0.02)
    packed, scales = Q.pack_weight_int4(to_dev_bf16(wb), scale_mode=mode)
    torch.cuda.synchronize()
    got = O.unpack_int4(unpair_w4(packed.cpu().numpy()))
    _check_prologue(got, scales.cpu().numpy(), wb, 4, mode)


# -------------------------------------------------- exact integer product --

# The small shapes run the 256 x 256-tile kernels; (4059, 5104, 512) needs
# more than 256 such tiles but only 256 of 256 x 320, so it runs the wide
# kernels, with ragged tails in both M and N.
GEMM_SHAPES = [(1, 16, 256), (130, 272, 512), (257, 400, 1024), (128, 128, 256), (300, 656, 768),
               (4059, 5104, 512)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("a_layout", ["i8", "packed"])
def test_w4a4_int32_bit_exact(Q, M, N, K, a_layout):
    import torch

    rng = np.random.default_rng(M + N + K)
    qa = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    a = to_dev(O.pack_int4(qa) if a_layout == "packed" else qa)
    w = to_dev(pair_w4(O.pack_int4(qw)))
    one_a = torch.ones(M, dtype=torch.float32, device="cuda")
    one_w = torch.ones(N, dtype=torch.float32, device="cuda")
    out = Q.qgemm_w4a4(a, one_a, w, one_w, K, a_layout=a_layout, epilogue="i32")
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.int64), O.int_gemm(qa, qw))


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES + [(64, 64, 20480)])
def test_w8a8_int32_bit_exact(Q, M, N, K):
    import torch

    rng = np.random.default_rng(M * N + K)
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    one_a = torch.ones(M, dtype=torch.float32, device="cuda")
    one_w = torch.ones(N, dtype=torch.float32, device="cuda")
    out = Q.qgemm_w8a8(to_dev(qa), one_a, to_dev(qw), one_w, epilogue="i32")
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.int64), O.int_gemm(qa, qw))


def test_int32_extremes(Q):
    """All codes at +-qmax: the largest accumulators the layer can produce."""
    import torch

    M, N, K = 32, 32, 20480
    qa = np.full((M, K), 127, np.int8)
    qw = np.full((N, K), -127, np.int8)
    qw[::2] = 127
    ones = torch.ones(max(M, N), dtype=torch.float32, device="cuda")
    out = Q.qgemm_w8a8(to_dev(qa), ones[:M], to_dev(qw), ones[:N], epilogue="i32")
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.int64), O.int_gemm(qa, qw))
    qa4 = np.full((M, 5120), -7, np.int8)
    qw4 = np.full((N, 5120), 7, np.int8)
    out = Q.qgemm_w4a4(to_dev(O.pack_int4(qa4)), ones[:M], to_dev(pair_w4(O.pack_int4(qw4))), ones[:N], 5120,
                       a_layout="packed", epilogue="i32")
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == -49 * 5120).all()


def test_group64_unit_scales_exact(Q):
    """Group-64 with all scales 1: the per-group fp32 sum of exact int32
    partials is exact (|sum| < 2^24), so the float output equals the
    integer product bit for bit."""
    import torch

    M, N, K = 130, 144, 1024
    rng = np.random.default_rng(9)
    qa = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sa = Q.group64_scales(torch.ones((M, K // 64), dtype=torch.float32, device="cuda"))
    sw = Q.group64_scales(torch.ones((N, K // 64), dtype=torch.float32, device="cuda"))
    out = Q.qgemm_w4a4_lowrank(to_dev(qa), sa, to_dev(pair_w4(O.pack_int4(qw))), sw, K, epilogue="f32")
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), O.int_gemm(qa, qw).astype(np.float64))


@pytest.mark.parametrize("a_layout", ["i8", "packed"])
def test_group64_pow2_scales_exact(Q, a_layout):
    """Group-64 with power-of-two scales 2^-e that differ per row and group:
    every term acc_g * s_a * s_w is a multiple of 2^-6 below 2^18 and the
    sum stays below 2^24, so the fp32 result is exact in any order and must
    equal the oracle's dequantized product bit for bit.  A scale applied to
    the wrong row, column or group changes the result."""
    import torch

    M, N, K = 200, 272, 1024
    rng = np.random.default_rng(11)
    qa = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sa_h = np.ldexp(1.0, -rng.integers(0, 4, size=(M, K // 64))).astype(np.float32)
    sw_h = np.ldexp(1.0, -rng.integers(0, 4, size=(N, K // 64))).astype(np.float32)
    a = to_dev(O.pack_int4(qa) if a_layout == "packed" else qa)
    out = Q.qgemm_w4a4_lowrank(a, to_dev_scales(sa_h), to_dev(pair_w4(O.pack_int4(qw))), to_dev_scales(sw_h), K,
                               a_layout=a_layout, epilogue="f32")
    torch.cuda.synchronize()
    ref_a = O.QuantResult(qa, sa_h, 4, "group64", None)
    ref_w = O.QuantResult(qw, sw_h, 4, "group64", None)
    want = O.linear_fp64(ref_a, ref_w)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), want)


# ---------------------------------------------- dequant epilogues (same codes) --

def _assert_bf16_close(got_bits, want_f64, bound):
    """got (bf16 bits) within one bf16 ulp of the rounded oracle value plus
    the kernel's float32 bound (tests/parity_checks.py)."""
    P.assert_outputs_close(O.bf16_bits_to_f64(got_bits), want_f64, bound)


def _upload_quant(ref, packed, weight=False):
    """Codes (packed int4 or int8 containers) and scales on the device;
    packed weights in the library's paired-row order."""
    codes = O.pack_int4(ref.codes) if packed else ref.codes
    if packed and weight:
        codes = pair_w4(codes)
    return to_dev(codes), to_dev_scales(ref.scales)


@pytest.mark.parametrize("mode", ["row", "tensor"])
def test_w4a4_bf16_epilogue_same_codes(Q, mode):
    import torch

    M, N, K = 257, 400, 1024
    xb = _rand_bf16(10, (M, K), outliers=10)
    wb = _rand_bf16(11, (N, K), 0.02)
    bias = _rand_bf16(12, (N,), 0.1)
    qa = O.quantize_activations(xb, 4, mode)
    qw = O.quantize_weights(wb, 4, mode)
    a, sa = _upload_quant(qa, False)
    w, sw = _upload_quant(qw, True, weight=True)
    for bb in (None, bias):
        out = Q.qgemm_w4a4(a, sa, w, sw, K, a_scale_mode=mode, w_scale_mode=mode,
                           bias=None if bb is None else to_dev_bf16(bb))
        torch.cuda.synchronize()
        y, dy = P.linear_bound(qa, qw, bias_bits=bb)
        got = bf16_bits(out)
        assert rel_fro(O.bf16_bits_to_f64(got), y) < REL_FRO
        _assert_bf16_close(got, y, dy)


def test_w8a8_gated_residual_same_codes(Q):
    import torch

    M, N, K = 200, 272, 2048
    xb = _rand_bf16(13, (M, K))
    wb = _rand_bf16(14, (N, K), 0.01)
    res = _rand_bf16(15, (M, N))
    gate = _rand_bf16(16, (N,))
    qa = O.quantize_activations(xb, 8, "row")
    qw = O.quantize_weights(wb, 8, "row")
    a, sa = _upload_quant(qa, False)
    w, sw = _upload_quant(qw, False)
    y, dy = P.linear_bound(qa, qw)
    ref, dref = P.epilogue_with_bound(y, dy, "gated_residual", O.bf16_bits_to_f64(res), O.bf16_bits_to_f64(gate))
    # out-of-place
    out = Q.qgemm_w8a8(a, sa, w, sw, residual=to_dev_bf16(res), gate=to_dev_bf16(gate),
                       epilogue="gated_residual")
    torch.cuda.synchronize()
    _assert_bf16_close(bf16_bits(out), ref, dref)
    # in place: h += gate * y
    h = to_dev_bf16(res)
    Q.qgemm_w8a8(a, sa, w, sw, residual=h, gate=to_dev_bf16(gate), epilogue="gated_residual", out=h)
    torch.cuda.synchronize()
    _assert_bf16_close(bf16_bits(h), ref, dref)
    # residual 0, gate 1: the plain epilogue, so the residual cannot mask the product
    z = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    ones = to_dev_bf16(W.to_bf16_bits(np.ones(N, np.float32)))
    out = Q.qgemm_w8a8(a, sa, w, sw, residual=z, gate=ones, epilogue="gated_residual")
    plain = Q.qgemm_w8a8(a, sa, w, sw, epilogue="bf16")
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), bf16_bits(plain))
    _assert_bf16_close(bf16_bits(plain), y, dy)


def _sample_rows(M, n=48):
    rng = np.random.default_rng(M)
    return np.unique(np.concatenate([np.arange(8), M - 1 - np.arange(8), rng.choice(M, n, replace=False)]))


@pytest.mark.parametrize("w8,N", [(False, 5104), (True, 5104), (True, 1520)])
def test_wide_tile_staged_epilogue_ragged(Q, w8, N):
    """The 256 x 320 tiles (N = 5104: chosen once a shape needs more than 256
    tiles of 256 x 256) and the int8-weight 256 x 192 tiles (N = 1520: 8 tile
    columns, the last 176 wide) with ragged M and N, a strided output (ldo >
    N) and the LDS-staged bf16 and gated-residual epilogues, against the
    oracle's dequantized product on sampled rows."""
    import torch

    M, K = 4059, 512
    rng = np.random.default_rng(21)
    qmax = 127 if w8 else 7
    qa = rng.integers(-qmax, qmax + 1, size=(M, K)).astype(np.int8)
    qw = rng.integers(-qmax, qmax + 1, size=(N, K)).astype(np.int8)
    sa_h = (rng.random(M, dtype=np.float32) * 0.02 + 0.01).astype(np.float32)
    sw_h = (rng.random(N, dtype=np.float32) * 0.02 + 0.01).astype(np.float32)
    rows = _sample_rows(M)
    y, dy = P.linear_bound(O.QuantResult(qa[rows], sa_h[rows], 8 if w8 else 4, "row", None),
                           O.QuantResult(qw, sw_h, 8 if w8 else 4, "row", None))
    big = torch.zeros((M, N + 16), dtype=torch.bfloat16, device="cuda")
    out = big[:, :N]
    a, w, sa, sw = to_dev(qa), to_dev(qw if w8 else pair_w4(O.pack_int4(qw))), to_dev_scales(sa_h), to_dev_scales(sw_h)
    if w8:
        Q.qgemm_w8a8(a, sa, w, sw, epilogue="bf16", out=out)
    else:
        Q.qgemm_w4a4(a, sa, w, sw, K, epilogue="bf16", out=out)
    torch.cuda.synchronize()
    _assert_bf16_close(bf16_bits(out)[rows], y, dy)
    assert not big[:, N:].any().item(), "store past the row end"
    if not w8:
        return
    res_h = _rand_bf16(22, (M, N))
    gate_h = _rand_bf16(23, (N,))
    res = to_dev_bf16(res_h)
    Q.qgemm_w8a8(a, sa, w, sw, residual=res, gate=to_dev_bf16(gate_h), epilogue="gated_residual", out=res)
    torch.cuda.synchronize()
    ref, dref = P.epilogue_with_bound(y, dy, "gated_residual", O.bf16_bits_to_f64(res_h)[rows],
                                      O.bf16_bits_to_f64(gate_h))
    _assert_bf16_close(bf16_bits(res)[rows], ref, dref)
    # gate 0 returns the residual bit for bit, except that a residual of -0
    # comes back as +0 (IEEE: -0 + 0*y = +0 for y >= 0), as in the oracle
    zero_gate = torch.zeros(N, dtype=torch.bfloat16, device="cuda")
    out0 = Q.qgemm_w8a8(a, sa, w, sw, residual=to_dev_bf16(res_h), gate=zero_gate, epilogue="gated_residual")
    torch.cuda.synchronize()
    got0 = bf16_bits(out0)
    both_zero = ((got0 & 0x7FFF) == 0) & ((res_h & 0x7FFF) == 0)
    bad = np.argwhere((got0 != res_h) & ~both_zero)
    assert bad.size == 0, (f"{len(bad)} outputs differ from the residual, first at {bad[:4].tolist()}: "
                           f"{got0[tuple(bad[0])]:#06x} vs {res_h[tuple(bad[0])]:#06x}")


def _lowrank_same_codes(Q, M, F, K, rank, mode, epi, seed, a_layout="i8"):
    """One low-rank GEMM on the oracle's codes and an uploaded bf16 lr; the
    expected value is the oracle's dequantized product plus lr L2 (lr taken
    as the given bf16 tensor), through the epilogue, element by element."""
    import torch

    N = 2 * F
    xb = _rand_bf16(seed, (M, K), outliers=max(1, K // 100))
    wb = _rand_bf16(seed + 1, (N, K), 0.02)
    qa = O.quantize_activations(xb, 4, mode)
    qw = O.quantize_weights(wb, 4, mode)
    a, sa = _upload_quant(qa, a_layout == "packed")
    w, sw = _upload_quant(qw, True, weight=True)
    lrb = _rand_bf16(seed + 2, (M, max(rank, 16)), 0.5)[:, :rank]
    l2b = _rand_bf16(seed + 3, (max(rank, 16), N), 0.05)[:rank]
    lr = to_dev_bf16(np.ascontiguousarray(lrb)) if rank else None
    l2 = to_dev_l2(l2b) if rank else None
    out = Q.qgemm_w4a4_lowrank(a, sa, w, sw, K, lr=lr, l2=l2, a_scale_mode=mode, w_scale_mode=mode,
                               a_layout=a_layout, epilogue=epi)
    torch.cuda.synchronize()
    y, dy = P.linear_bound(qa, qw)
    if rank:
        lrf, l2f = O.bf16_bits_to_f64(lrb), O.bf16_bits_to_f64(l2b)
        br = lrf @ l2f
        y = y + br
        dy = dy + (rank + 4) * P.U * (np.abs(lrf) @ np.abs(l2f)) + 3 * P.U * np.abs(br)
    want, dw = P.epilogue_with_bound(y, dy, epi)
    got = out.cpu().numpy().astype(np.float64) if epi == "f32" else O.bf16_bits_to_f64(bf16_bits(out))
    P.assert_outputs_close(got, want, dw, bf16=epi != "f32", what=f"{mode} r{rank} {epi}")
    assert rel_fro(got, want) < REL_FRO


@pytest.mark.parametrize("rank", [0, 16, 48, 64, 128])
@pytest.mark.parametrize("mode", ["row", "tensor", "group64"])
@pytest.mark.parametrize("epi", ["bf16", "swiglu", "f32"])
def test_lowrank_gemm_same_codes(Q, rank, mode, epi):
    """Every scale mode, rank (a partial last 32-rank block at 16 and 48,
    several blocks at 64 and 128) and epilogue of the low-rank GEMM, with
    ragged M and N, element by element against the oracle."""
    _lowrank_same_codes(Q, 139, 176, 1024, rank, mode, epi, 100 + rank)


@pytest.mark.parametrize("mode", ["row", "group64"])
def test_lowrank_gemm_packed_activations(Q, mode):
    _lowrank_same_codes(Q, 300, 160, 768, 32, mode, "swiglu", 7, a_layout="packed")


def test_group64_lowrank_with_device_lr(Q):
    """The branch with lr from the prologue (X L1 on the device) against the
    oracle's fp64 branch: the bound carries the bf16 rounding of lr."""
    import torch

    M, F, K, rank = 130, 160, 1024, 32
    N = 2 * F
    xb = _rand_bf16(17, (M, K))
    wb = _rand_bf16(18, (N, K), 0.02)
    l1 = _rand_bf16(19, (K, rank), 0.02)
    l2 = _rand_bf16(20, (rank, N), 0.02)
    qa = O.quantize_activations(xb, 4, "group64")
    qw = O.quantize_weights(wb, 4, "group64")
    a, sa = _upload_quant(qa, False)
    w, sw = _upload_quant(qw, True, weight=True)
    _, _, lr = Q.rotate_quantize_act(to_dev_bf16(xb), bits=4, scale_mode="group64", l1=to_dev_bf16(l1))
    for epi in ("swiglu", "bf16"):
        out = Q.qgemm_w4a4_lowrank(a, sa, w, sw, K, lr=lr, l2=to_dev_l2(l2), epilogue=epi)
        torch.cuda.synchronize()
        y, dy = P.linear_bound(qa, qw, xb, l1, l2)
        want, dw = P.epilogue_with_bound(y, dy, epi)
        _assert_bf16_close(bf16_bits(out), want, dw)


# ------------------------------------------------- end to end, per workload --

def _e2e(Q, wl, rows=None, wrows=None):
    """Run the whole GPU path (prologue, weight prep, GEMM + epilogue) on the
    full workload.  On `rows` (all if None) and weight rows `wrows` (all if
    None; the gate|up pairs for SwiGLU):
      * activation and weight codes and scales against the oracle's
        definition (near-tie flips only, within the budget);
      * the output element by element against the oracle's dequantized
        product of the GPU's own (just validated) codes, through the
        epilogue, within the kernel's float32 bound plus one bf16 ulp;
      * the output against the oracle's own end to end result within 1e-2
        relative Frobenius error."""
    import torch

    x = to_dev_bf16(wl.x)
    w = to_dev_bf16(wl.w)
    mode = wl.scale_mode
    rank = 0 if wl.l1 is None else wl.l1.shape[1]
    l1 = to_dev_bf16(wl.l1) if rank else None
    a_codes, sa, lr = Q.rotate_quantize_act(x, bits=wl.a_bits, scale_mode=mode, l1=l1)
    if wl.w_bits == 4:
        wq, sw = Q.pack_weight_int4(w, scale_mode=mode)
    else:
        wq, sw, _ = Q.rotate_quantize_act(w, bits=8, scale_mode=mode)
    if wl.epilogue == "gated_residual":
        out = Q.qgemm_w8a8(a_codes, sa, wq, sw, residual=to_dev_bf16(wl.residual),
                           gate=to_dev_bf16(wl.gate), epilogue="gated_residual")
    elif wl.w_bits == 8:
        out = Q.qgemm_w8a8(a_codes, sa, wq, sw, a_scale_mode=mode, w_scale_mode=mode)
    elif mode == "group64" or rank:
        out = Q.qgemm_w4a4_lowrank(a_codes, sa, wq, sw, wl.K, lr=lr,
                                   l2=to_dev_l2(wl.l2) if rank else None,
                                   a_scale_mode=mode, w_scale_mode=mode, epilogue=wl.epilogue)
    else:
        out = Q.qgemm_w4a4(a_codes, sa, wq, sw, wl.K, a_scale_mode=mode, w_scale_mode=mode)
    torch.cuda.synchronize()

    rsel = np.arange(wl.M) if rows is None else np.sort(np.asarray(rows))
    if wl.epilogue == "swiglu":
        F = wl.N // 2
        fsel = np.arange(F) if wrows is None else np.sort(np.asarray(wrows))
        nsel = np.concatenate([fsel, F + fsel])
    else:
        nsel = np.arange(wl.N) if wrows is None else np.sort(np.asarray(wrows))
    xs = np.ascontiguousarray(wl.x[rsel])
    wsb = np.ascontiguousarray(wl.w[nsel])

    # codes and scales, activations and weights (tensor units need every row)
    ga = a_codes.cpu().numpy()[rsel]
    gsa = sa.cpu().numpy()
    if wl.w_bits == 4:
        gw = O.unpack_int4(unpair_w4(wq.cpu().numpy())[nsel])
    else:
        gw = wq[torch.as_tensor(nsel, device=wq.device)].cpu().numpy()
    gsw = sw.cpu().numpy()
    if mode == "tensor":
        sta = _check_prologue(ga, gsa, wl.x, wl.a_bits, mode, rows=rsel)
        stw = _check_prologue(gw, gsw, wl.w, wl.w_bits, mode, rows=nsel)
    else:
        gsa, gsw = gsa[rsel], gsw[nsel]
        sta = _check_prologue(ga, gsa, xs, wl.a_bits, mode)
        stw = _check_prologue(gw, gsw, wsb, wl.w_bits, mode)

    # element by element on the GPU's own codes
    qa_g = O.QuantResult(ga, gsa, wl.a_bits, mode, None)
    qw_g = O.QuantResult(gw, gsw, wl.w_bits, mode, None)
    l2s = np.ascontiguousarray(wl.l2[:, nsel]) if rank else None
    y, dy = P.linear_bound(qa_g, qw_g, xs, wl.l1 if rank else None, l2s)
    if wl.epilogue == "gated_residual":
        res = O.bf16_bits_to_f64(wl.residual[np.ix_(rsel, nsel)])
        gate = O.bf16_bits_to_f64(wl.gate[nsel])
        want, dw = P.epilogue_with_bound(y, dy, "gated_residual", res, gate)
        got = bf16_bits(out)[np.ix_(rsel, nsel)]
    elif wl.epilogue == "swiglu":
        want, dw = P.epilogue_with_bound(y, dy, "swiglu")
        got = bf16_bits(out)[np.ix_(rsel, nsel[:len(nsel) // 2])]
    else:
        want, dw = y, dy
        got = bf16_bits(out)[np.ix_(rsel, nsel)]
    worst = P.assert_outputs_close(O.bf16_bits_to_f64(got), want, dw, what=wl.name)

    # against the oracle's own end-to-end result (its own codes)
    qa = O.quantize_activations(xs if mode != "tensor" else wl.x, wl.a_bits, mode)
    qw = O.quantize_weights(wsb if mode != "tensor" else wl.w, wl.w_bits, mode)
    if mode == "tensor":
        qa = O.QuantResult(qa.codes[rsel], qa.scales, qa.bits, mode, None)
        qw = O.QuantResult(qw.codes[nsel], qw.scales, qw.bits, mode, None)
    y_o = O.linear_fp64(qa, qw, xs, wl.l1 if rank else None, l2s)
    if wl.epilogue == "gated_residual":
        ref = O.epilogue(y_o, "gated_residual", res, gate)
    else:
        ref = O.epilogue(y_o, wl.epilogue)
    err = rel_fro(O.bf16_bits_to_f64(got), O.bf16_bits_to_f64(O.f64_to_bf16_bits(ref)))
    assert err < REL_FRO, f"{wl.name}: rel Frobenius {err:.3e}"
    print(f"{wl.name}: act flips {sta['flip_frac']:.2e} scale ulps {sta['scale_ulp_max']:.1f}/"
          f"{sta['scale_ulp_bound']:.1f}; weight flips {stw['flip_frac']:.2e} scale ulps "
          f"{stw['scale_ulp_max']:.1f}/{stw['scale_ulp_bound']:.1f}; outputs at {worst:.2f} of their bound; "
          f"rel_fro {err:.2e}", flush=True)
    return err, sta["flip_frac"]


def test_e2e_tiny_tensorwise(Q):
    err, frac = _e2e(Q, W.tiny_w4a4(0))
    assert err < 2e-3


def test_e2e_attention_projection_reduced(Q):
    wl = W.attn_proj_w4a4(M=520, N=656)
    _e2e(Q, wl)


def test_e2e_attention_projection_full_size(Q):
    """The benchmarked shape M=4096, K=N=5120: every output row the oracle
    checks is one of 64 sampled rows (all 5120 columns)."""
    wl = W.attn_proj_w4a4()
    rows = np.random.default_rng(0).choice(wl.M, 64, replace=False)
    _e2e(Q, wl, rows=rows)


def test_e2e_ffdown_w8a8_reduced(Q):
    wl = W.ffdown_w8a8(M=200, K=4096, N=272)
    _e2e(Q, wl)


def test_e2e_ffdown_w8a8_full_size(Q):
    wl = W.ffdown_w8a8()
    rng = np.random.default_rng(1)
    _e2e(Q, wl, rows=rng.choice(wl.M, 16, replace=False), wrows=rng.choice(wl.N, 512, replace=False))


def test_e2e_svdq_gateup_reduced(Q):
    wl = W.svdq_gateup(M=130, K=1024, F=160)
    _e2e(Q, wl)


def test_e2e_svdq_gateup_full_size(Q):
    wl = W.svdq_gateup()
    rng = np.random.default_rng(2)
    _e2e(Q, wl, rows=rng.choice(wl.M, 16, replace=False),
         wrows=rng.choice(wl.N // 2, 256, replace=False))


@pytest.mark.parametrize("index", [0, 1, 4, 5, 7, 7 + 8 * 15])
def test_e2e_stack_layer_shapes(Q, index):
    """One layer of each distinct shape/precision of the 224-linear stack at
    16384 tokens (sampled rows)."""
    wl = W.stack_layer(index)
    rng = np.random.default_rng(index)
    _e2e(Q, wl, rows=rng.choice(wl.M, 8, replace=False), wrows=rng.choice(wl.N, 384, replace=False))


def test_gemm_empty_inputs(Q):
    """M = 0: every GEMM entry point returns an empty output and launches nothing."""
    import torch

    N, K, r = 320, 512, 16
    d = "cuda"
    w4 = torch.zeros((N, K // 2), dtype=torch.uint8, device=d)
    w8 = torch.zeros((N, K), dtype=torch.int8, device=d)
    w6 = torch.zeros((N, K // 4 * 3), dtype=torch.uint8, device=d)
    sw = torch.ones(N, dtype=torch.float32, device=d)
    swg = Q.group64_scales(torch.ones((N, K // 64), dtype=torch.float32, device=d))
    a8 = torch.empty((0, K), dtype=torch.int8, device=d)
    sa = torch.empty((0,), dtype=torch.float32, device=d)
    outs = [
        Q.qgemm_w4a4(a8, sa, w4, sw, K),
        Q.qgemm_w8a8(a8, sa, w8, sw, residual=torch.empty((0, N), dtype=torch.bfloat16, device=d),
                     gate=torch.ones(N, dtype=torch.bfloat16, device=d), epilogue="gated_residual"),
        Q.qgemm_w4a4_lowrank(a8, torch.empty((0, K // 64), dtype=torch.float32, device=d), w4, swg, K,
                             lr=torch.empty((0, r), dtype=torch.bfloat16, device=d),
                             l2=torch.zeros((N, r), dtype=torch.bfloat16, device=d)),
        Q.qgemm_w4a4_fp6(torch.empty((0, K // 4 * 3), dtype=torch.uint8, device=d), sa, w6, sw, K),
    ]
    torch.cuda.synchronize()
    assert [tuple(o.shape) for o in outs] == [(0, N), (0, N), (0, N // 2), (0, N)]


def test_deterministic_outputs(Q):
    import torch

    wl = W.attn_proj_w4a4(M=300, N=400)
    x = to_dev_bf16(wl.x)
    w = to_dev_bf16(wl.w)
    outs = []
    for _ in range(2):
        a, sa, _ = Q.rotate_quantize_act(x, bits=4)
        wq, sw = Q.pack_weight_int4(w)
        outs.append(bf16_bits(Q.qgemm_w4a4(a, sa, wq, sw, wl.K)))
        torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])


# ------------------------------------------- grouped Q|K|V|gate GEMM (F2) --

def _prep_weight(Q, wb, bits):
    import torch

    w = to_dev_bf16(wb)
    if bits == 4:
        return Q.pack_weight_int4(w, scale_mode="row")
    wq = torch.empty(wb.shape, dtype=torch.int8, device="cuda")
    sw = torch.empty((wb.shape[0],), dtype=torch.float32, device="cuda")
    Q.rotate_quantize_act(w, bits=8, scale_mode="row", codes=wq, scales=sw)
    return wq, sw


def _qkvg(M, K, dims, seed):
    """Activations and the four projections (q int4, k int8, v int8, gate int4 + sigmoid)."""
    rng = np.random.default_rng(seed)
    xb = W.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    specs = [("q", dims[0], 4, "bf16"), ("k", dims[1], 8, "bf16"), ("v", dims[2], 8, "bf16"),
             ("gate", dims[3], 4, "sigmoid")]
    ws = {name: W.to_bf16_bits((0.02 * rng.standard_normal((n, K))).astype(np.float32))
          for name, n, _, _ in specs}
    return xb, specs, ws


@pytest.mark.parametrize("M,K,dims", [(300, 1536, (384, 96, 96, 384)), (64, 256, (320, 16, 48, 640)),
                                      (515, 1024, (640, 160, 160, 640))])
def test_grouped_qkvg_matches_oracle_and_separate_launches(Q, M, K, dims):
    import torch

    xb, specs, ws = _qkvg(M, K, dims, seed=M + K)
    x = to_dev_bf16(xb)
    a4, sa4, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row")
    a8, sa8, _ = Q.rotate_quantize_act(x, bits=8, scale_mode="row")
    prep = {name: _prep_weight(Q, ws[name], bits) for name, _, bits, _ in specs}
    segs = [dict(w=prep[name][0], sw=prep[name][1], bits=bits, epilogue=epi) for name, _, bits, epi in specs]
    outs = Q.qgemm_grouped(a4, sa4, a8, sa8, K, segs)
    torch.cuda.synchronize()
    qa = {4: O.quantize_activations(xb, 4, "row", True), 8: O.quantize_activations(xb, 8, "row", True)}
    for (name, n, bits, epi), out in zip(specs, outs):
        wq, sw = prep[name]
        # the same product through the single-projection entry point, on the same codes: bit-exact
        if bits == 4:
            sep = Q.qgemm_w4a4(a4, sa4, wq, sw, K, epilogue=epi)
        else:
            sep = Q.qgemm_w8a8(a8, sa8, wq, sw, epilogue=epi)
        torch.cuda.synchronize()
        assert torch.equal(out, sep), name
        # and against the oracle
        qw = O.quantize_weights(ws[name], bits, "row", True)
        want = O.epilogue(O.linear_fp64(qa[bits], qw), epi)
        assert rel_fro(O.bf16_bits_to_f64(bf16_bits(out)), want) <= REL_FRO, name


@pytest.mark.parametrize("bits", [4, 8])
def test_sigmoid_epilogue_same_codes(Q, bits):
    """The sigmoid epilogue element by element, from the oracle's own codes."""
    import torch

    M, N, K = 130, 640, 1024
    rng = np.random.default_rng(41 + bits)
    xb = W.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wb = W.to_bf16_bits((0.05 * rng.standard_normal((N, K))).astype(np.float32))
    qa = O.quantize_activations(xb, bits, "row", True)
    qw = O.quantize_weights(wb, bits, "row", True)
    a = to_dev(qa.codes)
    sa = to_dev_scales(qa.scales)
    sw = to_dev_scales(qw.scales)
    if bits == 4:
        out = Q.qgemm_w4a4(a, sa, to_dev(pair_w4(O.pack_int4(qw.codes))), sw, K, epilogue="sigmoid")
    else:
        out = Q.qgemm_w8a8(a, sa, to_dev(qw.codes), sw, epilogue="sigmoid")
    torch.cuda.synchronize()
    want, dw = P.epilogue_with_bound(*P.linear_bound(qa, qw), "sigmoid")
    _assert_bf16_close(bf16_bits(out), want, dw)


def test_grouped_stack_block_full_size(Q):
    """One block's attention projections of the 2048^2 stack (16384 tokens, K = 5120:
    q and gate [6144] int4, k and v [1536] int8) in one grouped launch: every
    output equals the separate launches, and sampled rows match the oracle."""
    import torch

    M, K = 16384, 5120
    g = torch.Generator(device="cuda")
    g.manual_seed(91)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    a4, sa4, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row")
    a8, sa8, _ = Q.rotate_quantize_act(x, bits=8, scale_mode="row")
    specs = [("q", 6144, 4, "bf16"), ("k", 1536, 8, "bf16"), ("v", 1536, 8, "bf16"), ("gate", 6144, 4, "sigmoid")]
    wsb, prep = {}, {}
    for name, n, bits, _ in specs:
        w = (0.02 * torch.randn((n, K), generator=g, device="cuda", dtype=torch.float32)).to(torch.bfloat16)
        wsb[name] = bf16_bits(w)
        prep[name] = _prep_weight(Q, wsb[name], bits)
    segs = [dict(w=prep[nm][0], sw=prep[nm][1], bits=b, epilogue=e) for nm, _, b, e in specs]
    outs = Q.qgemm_grouped(a4, sa4, a8, sa8, K, segs)
    torch.cuda.synchronize()
    ri = torch.as_tensor(_sample_rows(M, 32), device="cuda")
    xs = bf16_bits(x[ri])
    qa = {4: O.quantize_activations(xs, 4, "row", True), 8: O.quantize_activations(xs, 8, "row", True)}
    for (name, n, bits, epi), out in zip(specs, outs):
        wq, sw = prep[name]
        sep = (Q.qgemm_w4a4(a4, sa4, wq, sw, K, epilogue=epi) if bits == 4
               else Q.qgemm_w8a8(a8, sa8, wq, sw, epilogue=epi))
        torch.cuda.synchronize()
        assert torch.equal(out, sep), name
        del sep
        cols = np.sort(np.random.default_rng(n).choice(n, 192, replace=False))
        qw = O.quantize_weights(wsb[name][cols], bits, "row", True)      # weight rows are independent
        want = O.epilogue(O.linear_fp64(qa[bits], qw), epi)
        got = bf16_bits(out[ri][:, torch.as_tensor(cols, device="cuda")])
        assert rel_fro(O.bf16_bits_to_f64(got), want) <= REL_FRO, name
