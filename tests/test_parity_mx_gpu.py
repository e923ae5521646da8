"""GPU parity of the MX block-scaled path (rotate_quantize_mx, qgemm_mx)
against the oracle (oracle.mx_ref), through the C ABI.

Acceptance (windows derived in tests/parity_checks.py):
  * block exponents and element codes: the oracle's decision on the exactly
    rotated values, except where the kernel's float32 rotation error puts a
    block maximum across a power of two or an element across a rounding
    boundary; decisions that differ stay at or below 1e-4 of the codes.
    Unrotated bf16 inputs take the exact decisions (no differences at all);
  * GEMM outputs element by element against the oracle's MX product of the
    same codes, within the float32 accumulation bound plus one bf16 ulp;
  * end-to-end bf16 outputs within 1e-2 relative Frobenius error of the
    oracle's own result;
  * at the full attention-projection size (4096 x 5120 x 5120) on sampled
    rows.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import parity_checks as P
from tests.helpers import bf16_bits, ensure_built, rel_fro, to_dev, to_dev_bf16, to_dev_l2

pytestmark = pytest.mark.gpu

REL_FRO = 1e-2


@pytest.fixture(scope="module")
def Q():
    import torch

    ensure_built()
    import rotated_bit_quantized_rotate_amd as Q

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert Q.device_supported(0), "device is not gfx950"
    return Q


def _rand_bf16(seed, shape, std=1.0, outliers=0, factor=30.0, row_spread=False):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    if row_spread:
        a *= np.exp(rng.uniform(-6, 6, (shape[0], 1))).astype(np.float32)
    if outliers:
        a, _ = W.with_outlier_channels(rng, a, outliers, factor)
    return W.to_bf16_bits(a)


def _gpu_mx(Q, xb, fmt, rotate):
    import torch

    codes, scales = Q.rotate_quantize_mx(to_dev_bf16(xb), fmt=fmt, rotate=rotate)
    torch.cuda.synchronize()
    return codes, scales


def _rowmajor(scales):
    """Stage-major scale bytes [K/128, R, 4] -> row-major [R, K/32]."""
    s = np.asarray(scales.cpu().numpy() if hasattr(scales, "cpu") else scales)
    return np.ascontiguousarray(s.transpose(1, 0, 2).reshape(s.shape[1], -1))


def _unpack(codes, scales, fmt):
    return O.mx_unpack(codes.cpu().numpy(), _rowmajor(scales), fmt)


def _check(codes, exps, xb, fmt, rotate, rows=None):
    x = O.bf16_bits_to_f64(xb)
    xr = O.rotate(x) if rotate else x
    budget = P.FLIP_BUDGET if rotate else 0.0
    return P.check_mx(codes, exps, xr, P.rotation_error_bound(x, None, rotate), fmt, budget, rows)


# --------------------------------------------------------------- prologue --

@pytest.mark.parametrize("M,K", [(1, 256), (37, 512), (300, 5120), (5, 20480), (33, 6144)])
@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("rotate", [True, False])
def test_mx_quantize_matches_oracle(Q, M, K, fmt, rotate):
    xb = _rand_bf16(M * 3 + K, (M, K), outliers=max(1, K // 100), row_spread=True)
    codes, scales = _gpu_mx(Q, xb, fmt, rotate)
    assert codes.shape == (M, K // 2 if fmt == "fp4" else K) and scales.shape == (K // 128, M, 4)
    c, e = _unpack(codes, scales, fmt)
    st = _check(c, e, xb, fmt, rotate)
    print(f"exp flips {st['exp_flips']}, code flips {st['code_flips']} ({st['flip_frac']:.2e})")


def _edge_rows(fmt, K, seed):
    """Unrotated rows that exercise every decision: element-grid ties at
    several block scales, saturation (block maxima in [max, 2^(emax+1)) of
    the scale), all-zero blocks, negative values that round to zero, a wide
    range of block scales along one row, and a block whose maximum is an
    exact power of two."""
    rng = np.random.default_rng(seed)
    f = O.MX_FORMATS[fmt]
    mags = O.mx_element_magnitudes(fmt)
    mids = (mags[:-1] + mags[1:]) / 2
    rows = []
    # ties: a block of midpoints with its maximum fixing the scale 2^s
    for s in (-20, -3, 0, 5, 30):
        r = np.zeros(K)
        for b in range(K // 32):
            blk = rng.choice(mids, 32) * rng.choice([-1.0, 1.0], 32)
            blk[0] = 2.0 ** (f.emax + 1) * (1 - 2.0 ** -7)    # largest bf16 below the next binade
            r[32 * b:32 * b + 32] = np.ldexp(blk, s + (b % 5) - 2)
        rows.append(r)
    # saturation and zeros
    r = np.zeros(K)
    for b in range(K // 32):
        if b % 3 == 0:
            continue                                       # all-zero block
        blk = rng.uniform(-1, 1, 32) * mags[-1]
        blk[b % 32] = (mags[-1] + (2.0 ** (f.emax + 1) - mags[-1]) * rng.uniform(0, 1)) * (-1) ** b
        r[32 * b:32 * b + 32] = blk
    rows.append(r)
    # negative values below half the smallest step next to a large value
    r = np.zeros(K)
    for b in range(K // 32):
        blk = -rng.uniform(0, mags[1] / 2, 32) * 2.0 ** (f.emax - 1)
        blk[0] = 2.0 ** f.emax * 1.5
        r[32 * b:32 * b + 32] = blk * 2.0 ** (b % 7 - 3)
    rows.append(r)
    # block maxima at exact powers of two, and wide dynamic range
    r = rng.standard_normal(K)
    for b in range(K // 32):
        r[32 * b:32 * b + 32] *= 2.0 ** ((b * 37) % 200 - 100)
        r[32 * b + 7] = 2.0 ** ((b * 37) % 200 - 98)
    rows.append(r)
    xb = O.f64_to_bf16_bits(np.array(rows))
    return xb


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_mx_quantize_edge_values_exact(Q, fmt):
    xb = _edge_rows(fmt, 1024, 5)
    codes, scales = _gpu_mx(Q, xb, fmt, rotate=False)
    c, e = _unpack(codes, scales, fmt)
    ref = O.quantize_mx(xb, fmt, rotate_on=False)
    np.testing.assert_array_equal(e, ref.exps)
    np.testing.assert_array_equal(c, ref.codes)
    data, sb = O.mx_pack(ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), data)       # the byte layout too
    np.testing.assert_array_equal(_rowmajor(scales), sb)
    # stage-major: slice s holds row r's blocks 4s .. 4s+3 at [s, r, :]
    np.testing.assert_array_equal(scales.cpu().numpy()[1, 3], sb[3, 4:8])


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_mx_quantize_strided_rows_and_empty(Q, fmt):
    import torch

    M, K, ldx = 19, 768, 1024
    xb = _rand_bf16(7, (M, ldx), outliers=4)
    full = to_dev_bf16(xb)
    codes, scales = Q.rotate_quantize_mx(full[:, :K], fmt=fmt, rotate=True)
    torch.cuda.synchronize()
    c, e = _unpack(codes, scales, fmt)
    _check(c, e, xb[:, :K].copy(), fmt, True)
    empty = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    codes, scales = Q.rotate_quantize_mx(empty, fmt=fmt)
    assert codes.shape[0] == 0 and scales.shape[1] == 0


# ------------------------------------------------------------------- GEMM --

def _mx_pair(Q, M, N, K, fmt, seed, rotate=True):
    xb = _rand_bf16(seed, (M, K), outliers=max(1, K // 100))
    wb = _rand_bf16(seed + 1, (N, K), std=0.02)
    ca, sa = _gpu_mx(Q, xb, fmt, rotate)
    cw, sw = _gpu_mx(Q, wb, fmt, rotate)
    a_c, a_e = _unpack(ca, sa, fmt)
    w_c, w_e = _unpack(cw, sw, fmt)
    qa = O.MXResult(a_c, a_e, fmt, None)
    qw = O.MXResult(w_c, w_e, fmt, None)
    return xb, wb, (ca, sa, cw, sw), qa, qw


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("M,N,K", [(1, 16, 256), (100, 272, 1024), (300, 640, 512), (513, 336, 2048),
                                   (256, 1280, 5120)])
@pytest.mark.parametrize("epi", ["bf16", "f32"])
def test_mx_gemm_same_codes(Q, fmt, M, N, K, epi):
    import torch

    xb, wb, (ca, sa, cw, sw), qa, qw = _mx_pair(Q, M, N, K, fmt, seed=M + N + K)
    bias = W.to_bf16_bits(np.random.default_rng(1).standard_normal(N).astype(np.float32) * 0.1)
    out = Q.qgemm_mx(ca, sa, cw, sw, K, fmt=fmt, bias=to_dev_bf16(bias), epilogue=epi)
    torch.cuda.synchronize()
    y, dy = P.mx_linear_bound(qa, qw, bias)
    got = bf16_bits(out).astype(np.uint16) if epi == "bf16" else out.cpu().numpy()
    got = O.bf16_bits_to_f64(got) if epi == "bf16" else got.astype(np.float64)
    r = P.assert_outputs_close(got, y, dy, bf16=epi == "bf16", what=f"{fmt} {epi}")
    print(f"worst error / tolerance {r:.3f}")


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_mx_gemm_wide_tiles_ragged(Q, fmt):
    """A grid where 256 x 320 tiles save a wave over 256 x 256 (16 x 16
    against 16 x 20 tiles), so the wide configuration runs, with ragged M
    and N tails; sampled rows (the last tile row included) against the
    oracle's product of the GPU's codes, every column."""
    import torch

    M, N, K = 4000, 5104, 512
    xb, wb, (ca, sa, cw, sw), qa, qw = _mx_pair(Q, M, N, K, fmt, seed=11)
    out = Q.qgemm_mx(ca, sa, cw, sw, K, fmt=fmt)
    torch.cuda.synchronize()
    rows = np.array([0, 17, 255, 256, 2100, 3839, 3840, 3998, 3999])
    qa_rows = O.MXResult(qa.codes[rows], qa.exps[rows], fmt, None)
    y, dy = P.mx_linear_bound(qa_rows, qw)
    got = O.bf16_bits_to_f64(bf16_bits(out[rows]))
    r = P.assert_outputs_close(got, y, dy, what=f"{fmt} wide tiles")
    print(f"worst error / tolerance {r:.3f}")


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("epi", ["sigmoid", "gated_residual", "swiglu"])
def test_mx_gemm_epilogues(Q, fmt, epi):
    import torch

    M, N, K = 260, 640, 1024
    xb, wb, (ca, sa, cw, sw), qa, qw = _mx_pair(Q, M, N, K, fmt, seed=41)
    rng = np.random.default_rng(2)
    res = gate = None
    cols = N // 2 if epi == "swiglu" else N
    if epi == "gated_residual":
        res = W.to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
        gate = W.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    out = Q.qgemm_mx(ca, sa, cw, sw, K, fmt=fmt, epilogue=epi,
                     residual=None if res is None else to_dev_bf16(res),
                     gate=None if gate is None else to_dev_bf16(gate))
    torch.cuda.synchronize()
    assert out.shape == (M, cols)
    y, dy = P.mx_linear_bound(qa, qw)
    want, dwant = P.epilogue_with_bound(y, dy, epi, None if res is None else O.bf16_bits_to_f64(res),
                                        None if gate is None else O.bf16_bits_to_f64(gate))
    P.assert_outputs_close(O.bf16_bits_to_f64(bf16_bits(out)), want, dwant, what=f"{fmt} {epi}")


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_mx_gated_residual_in_place(Q, fmt):
    import torch

    M, N, K = 64, 256, 512
    xb, wb, (ca, sa, cw, sw), qa, qw = _mx_pair(Q, M, N, K, fmt, seed=43)
    rng = np.random.default_rng(3)
    res = W.to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    gate = W.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    h = to_dev_bf16(res)
    Q.qgemm_mx(ca, sa, cw, sw, K, fmt=fmt, epilogue="gated_residual", residual=h, gate=to_dev_bf16(gate), out=h)
    torch.cuda.synchronize()
    y, dy = P.mx_linear_bound(qa, qw)
    want, dwant = P.epilogue_with_bound(y, dy, "gated_residual", O.bf16_bits_to_f64(res), O.bf16_bits_to_f64(gate))
    P.assert_outputs_close(O.bf16_bits_to_f64(bf16_bits(h)), want, dwant, what="in place")


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("rotate", [True, False])
def test_mx_linear_end_to_end(Q, fmt, rotate):
    import torch

    M, N, K = 320, 640, 2048
    xb = _rand_bf16(51, (M, K), outliers=20)
    wb = _rand_bf16(52, (N, K), std=0.02)
    ca, sa = _gpu_mx(Q, xb, fmt, rotate)
    cw, sw = _gpu_mx(Q, wb, fmt, rotate)
    out = Q.qgemm_mx(ca, sa, cw, sw, K, fmt=fmt)
    torch.cuda.synchronize()
    ref_bits, y, qa, qw = O.mx_linear(xb, wb, fmt, rotate_on=rotate)
    e = rel_fro(O.bf16_bits_to_f64(bf16_bits(out)), O.bf16_bits_to_f64(ref_bits))
    exact = O.bf16_bits_to_f64(xb) @ O.bf16_bits_to_f64(wb).T
    q_err = rel_fro(y, exact)
    print(f"rel Frobenius vs oracle {e:.2e}; MX quantization error vs unquantized {q_err:.3f}")
    assert e <= REL_FRO


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_mx_full_size_sampled_rows(Q, fmt):
    """The attention projection at its full size (X [4096 x 5120] with 1 %
    outlier channels x30, W [5120 x 5120]) in the launch configuration the
    benchmark times; codes of sampled rows against the definition, and their
    outputs against the oracle's product of the GPU's codes."""
    import torch

    wl = W.attn_proj_w4a4()
    M, K = wl.x.shape
    N = wl.w.shape[0]
    ca, sa = _gpu_mx(Q, wl.x, fmt, True)
    cw, sw = _gpu_mx(Q, wl.w, fmt, True)
    out = Q.qgemm_mx(ca, sa, cw, sw, K, fmt=fmt)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 2047, 3000, 4094, 4095])
    xs = wl.x[rows]
    a_c, a_e = O.mx_unpack(ca[rows].cpu().numpy(), _rowmajor(sa)[rows], fmt)
    st = _check(a_c, a_e, xs, fmt, True)
    w_c, w_e = _unpack(cw, sw, fmt)
    stw = _check(w_c, w_e, wl.w, fmt, True)
    print(f"activation rows: {st}; weights: {stw}")
    y, dy = P.mx_linear_bound(O.MXResult(a_c, a_e, fmt, None), O.MXResult(w_c, w_e, fmt, None))
    got = O.bf16_bits_to_f64(bf16_bits(out[rows]))
    P.assert_outputs_close(got, y, dy, what=f"{fmt} full size")


# ------------------------------------------------------- low-rank branch --

def _lowrank_case(Q, M, N, K, r, fmt, seed):
    import torch

    xb = _rand_bf16(seed, (M, K), outliers=max(1, K // 100))
    wb = _rand_bf16(seed + 1, (N, K), std=0.02)
    l1 = _rand_bf16(seed + 2, (K, r), std=0.02)
    l2 = _rand_bf16(seed + 3, (r, N), std=0.02)
    ca, sa, lr = Q.rotate_quantize_mx(to_dev_bf16(xb), fmt=fmt, l1=to_dev_bf16(l1))
    cw, sw = Q.rotate_quantize_mx(to_dev_bf16(wb), fmt=fmt)
    torch.cuda.synchronize()
    return xb, wb, l1, l2, (ca, sa, cw, sw, lr)


def _lowrank_want(xb, l1, l2, ca, sa, cw, sw, fmt, epi, rows=None):
    a_c, a_e = O.mx_unpack(ca.cpu().numpy(), _rowmajor(sa), fmt)
    w_c, w_e = _unpack(cw, sw, fmt)
    if rows is not None:
        a_c, a_e, xb = a_c[rows], a_e[rows], xb[rows]
    y, dy = P.mx_linear_bound(O.MXResult(a_c, a_e, fmt, None), O.MXResult(w_c, w_e, fmt, None))
    br, dbr = P.lowrank_bound(xb, l1, l2)
    y2 = y + br
    dy2 = dy + dbr + 3 * P.U * (np.abs(y) + np.abs(br))
    return P.epilogue_with_bound(y2, dy2, epi)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("r", [16, 32, 64, 128])
@pytest.mark.parametrize("epi", ["bf16", "swiglu", "f32"])
def test_mx_lowrank_gemm(Q, fmt, r, epi):
    import torch

    M, N, K = 300, 640, 1024
    xb, wb, l1, l2, (ca, sa, cw, sw, lr) = _lowrank_case(Q, M, N, K, r, fmt, seed=61 + r)
    # the down-projection is the unrotated x @ l1, rounded once to bf16
    lr_want = O.bf16_bits_to_f64(xb) @ O.bf16_bits_to_f64(l1)
    lr_bound = P.BF16_U * np.abs(lr_want) + (K / 8 + 4) * P.U * (np.abs(O.bf16_bits_to_f64(xb)) @
                                                                  np.abs(O.bf16_bits_to_f64(l1)))
    lr_got = O.bf16_bits_to_f64(bf16_bits(lr))
    assert np.all(np.abs(lr_got - lr_want) <= lr_bound + 2.0 ** -133)
    out = Q.qgemm_mx_lowrank(ca, sa, cw, sw, K, fmt=fmt, lr=lr, l2=to_dev_l2(l2), epilogue=epi)
    torch.cuda.synchronize()
    want, bound = _lowrank_want(xb, l1, l2, ca, sa, cw, sw, fmt, epi)
    got = out.cpu().numpy().astype(np.float64) if epi == "f32" else O.bf16_bits_to_f64(bf16_bits(out))
    r_ = P.assert_outputs_close(got, want, bound, bf16=epi != "f32", what=f"{fmt} rank {r} {epi}")
    print(f"worst error / tolerance {r_:.3f}")


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_mx_lowrank_rank0_equals_plain(Q, fmt):
    import torch

    M, N, K = 128, 256, 512
    xb, wb, l1, l2, (ca, sa, cw, sw, lr) = _lowrank_case(Q, M, N, K, 16, fmt, seed=71)
    a = Q.qgemm_mx_lowrank(ca, sa, cw, sw, K, fmt=fmt, epilogue="bf16")
    b = Q.qgemm_mx(ca, sa, cw, sw, K, fmt=fmt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_mx_svdq_gateup_full_size_sampled_rows(Q):
    """The SVDQuant gate|up layer at its full size in MXFP4 (X [4096 x 5120],
    W [40960 x 5120], rank-32 L1 / L2, SwiGLU -> [4096 x 20480]) in the
    launch configuration the benchmark times; sampled rows against the
    oracle's product of the GPU's codes, sampled weight rows against the
    quantizer's definition."""
    import torch

    wl = W.svdq_gateup()
    M, K = wl.x.shape
    N = wl.w.shape[0]
    ca, sa, lr = Q.rotate_quantize_mx(to_dev_bf16(wl.x), fmt="fp4", l1=to_dev_bf16(wl.l1))
    cw, sw = Q.rotate_quantize_mx(to_dev_bf16(wl.w), fmt="fp4")
    out = Q.qgemm_mx_lowrank(ca, sa, cw, sw, K, fmt="fp4", lr=lr, l2=to_dev_l2(wl.l2), epilogue="swiglu")
    torch.cuda.synchronize()
    rows = np.array([0, 255, 2048, 4095])
    want, bound = _lowrank_want(wl.x, wl.l1, wl.l2, ca, sa, cw, sw, "fp4", "swiglu", rows=rows)
    got = O.bf16_bits_to_f64(bf16_bits(out[rows]))
    P.assert_outputs_close(got, want, bound, what="MXFP4 SVDQuant gate|up")
    wsel = np.random.default_rng(0).choice(N, 64, replace=False)
    w_c, w_e = _unpack(cw, sw, "fp4")
    st = _check(w_c[wsel], w_e[wsel], wl.w[wsel], "fp4", True)
    print(f"weights (64 sampled rows): {st}")
