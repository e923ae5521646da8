"""GPU parity of the FP6 (e2m3) experiment: the prologue's FP6 code layout,
the FP6 weight packer and the W4A4 GEMM on the FP6 matrix instruction.

The FP6 path stores the same int4 codes in another layout and multiplies
them on another instruction, so the bar is exactness:
  * codes written in the FP6 layout equal the oracle's FP6 packing of the
    codes the same kernel writes in the int8 layout, byte for byte, and the
    scales are identical; those codes meet the usual flip budget against
    the oracle's own quantization;
  * the exact-sum output (I32) equals the oracle's integer product;
  * every float epilogue equals the INT4 path's output on the same codes
    bit for bit (the fp32 sums of the FP6 products are exact integers), and
    the oracle's dequantized product through the epilogue element by
    element (tolerances from tests/parity_checks.py).
Sizes span the 256 x 256 and 256 x 320 tile kernels with ragged tails, and
the full 4096 x 5120 x 5120 attention projection.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import parity_checks as P
from tests.helpers import (bf16_bits, ensure_built, pair_w4, quad_fp6, to_dev, to_dev_bf16, to_dev_l2, to_dev_scales,
                           unpair_w4, unquad_fp6)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import torch

    ensure_built()
    import rotated_bit_quantized_rotate_amd as Q

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert Q.device_supported(0), "device is not gfx950"
    return Q


def _rand_bf16(seed, shape, std=1.0, outliers=0, factor=30.0):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    if outliers:
        a, _ = W.with_outlier_channels(rng, a, outliers, factor)
    return W.to_bf16_bits(a)


# ------------------------------------------------------------ prologue ------

@pytest.mark.parametrize("M,K", [(1, 256), (37, 512), (300, 5120), (5, 20480), (33, 6144)])
@pytest.mark.parametrize("mode", ["row", "tensor", "group64"])
def test_prologue_fp6_layout(Q, M, K, mode):
    import torch

    xb = _rand_bf16(M * 3 + K, (M, K), outliers=max(1, K // 100))
    x = to_dev_bf16(xb)
    c8, s8, _ = Q.rotate_quantize_act(x, bits=4, scale_mode=mode, layout="i8")
    c6, s6, _ = Q.rotate_quantize_act(x, bits=4, scale_mode=mode, layout="fp6")
    torch.cuda.synchronize()
    assert tuple(c6.shape) == (M, K // 4 * 3)
    codes = c8.cpu().numpy()
    assert np.array_equal(unquad_fp6(c6.cpu().numpy()), O.pack_fp6(codes))
    assert torch.equal(s6, s8)
    xf = O.bf16_bits_to_f64(xb)
    P.check_codes(O.unpack_fp6(unquad_fp6(c6.cpu().numpy())), s6.cpu().numpy(), O.rotate(xf), P.rotation_error_bound(xf),
                  4, mode)


def test_prologue_fp6_extreme_codes_and_strides(Q):
    """Rows that quantize to every code -7..7 (including the absmax ones),
    zero rows, and a strided input."""
    import torch

    M, K = 64, 1024
    rng = np.random.default_rng(5)
    xf = rng.standard_normal((M, K), dtype=np.float32)
    xf[3] = 0.0
    xf[7] = np.tile(np.arange(-7, 8, dtype=np.float32), K // 15 + 1)[:K]
    big = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    big[:, :K] = torch.from_numpy(xf).to(torch.bfloat16).cuda()
    x = big[:, :K]
    for rot in (True, False):
        c8, s8, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row", layout="i8", rotate=rot)
        c6, s6, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row", layout="fp6", rotate=rot)
        torch.cuda.synchronize()
        codes = c8.cpu().numpy()
        assert np.array_equal(unquad_fp6(c6.cpu().numpy()), O.pack_fp6(codes))
        assert torch.equal(s6, s8)
        if not rot:
            assert set(np.unique(codes[7])) == set(range(-7, 8))
        assert not codes[3].any()


def test_rmsnorm_prologue_fp6_layout(Q):
    import torch

    M, K = 300, 5120
    xb = _rand_bf16(41, (M, K), outliers=20)
    g = to_dev_bf16(_rand_bf16(42, (K,), 0.3))
    sc = to_dev_bf16(_rand_bf16(43, (K,), 0.1))
    sh = to_dev_bf16(_rand_bf16(44, (K,), 0.1))
    x = to_dev_bf16(xb)
    c8, s8 = Q.rmsnorm_rotate_quantize_act(x, g, sc, sh, eps=1e-6, bits=4, layout="i8")
    c6, s6 = Q.rmsnorm_rotate_quantize_act(x, g, sc, sh, eps=1e-6, bits=4, layout="fp6")
    torch.cuda.synchronize()
    assert np.array_equal(unquad_fp6(c6.cpu().numpy()), O.pack_fp6(c8.cpu().numpy()))
    assert torch.equal(s6, s8)


@pytest.mark.parametrize("mode", ["row", "tensor", "group64"])
def test_pack_weight_fp6(Q, mode):
    import torch

    N, K = 272, 1024
    wb = _rand_bf16(8, (N, K), 0.02)
    w = to_dev_bf16(wb)
    p4, s4 = Q.pack_weight_int4(w, scale_mode=mode)
    p6, s6 = Q.pack_weight_fp6(w, scale_mode=mode)
    torch.cuda.synchronize()
    assert np.array_equal(unquad_fp6(p6.cpu().numpy()), O.pack_fp6(O.unpack_int4(unpair_w4(p4.cpu().numpy()))))
    assert torch.equal(s6, s4)


# ---------------------------------------------------------------- GEMM ------

# 256 x 256 tiles for the small shapes; (4059, 5104, 512) needs more than 256
# of them and runs the 256 x 320 kernels, with ragged M and N.
FP6_SHAPES = [(1, 16, 256), (130, 272, 512), (257, 400, 1024), (128, 128, 256), (300, 656, 768),
              (4059, 5104, 512), (64, 64, 20480)]


@pytest.mark.parametrize("M,N,K", FP6_SHAPES)
def test_fp6_exact_sum_matches_oracle(Q, M, N, K):
    import torch

    rng = np.random.default_rng(M * 5 + N + K)
    qa = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    a, w = to_dev(quad_fp6(O.pack_fp6(qa))), to_dev(quad_fp6(O.pack_fp6(qw)))
    one_a = torch.ones(M, dtype=torch.float32, device="cuda")
    one_w = torch.ones(N, dtype=torch.float32, device="cuda")
    out = Q.qgemm_w4a4_fp6(a, one_a, w, one_w, K, epilogue="i32")
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.int64), O.int_gemm(qa, qw))


def test_fp6_exact_sum_extremes(Q):
    """All codes +-7 at K = 20480: sums of +-49 K = +-1003520, still exact."""
    import torch

    M, N, K = 32, 48, 20480
    qa = np.full((M, K), 7, dtype=np.int8)
    qa[1::2] = -7
    qw = np.full((N, K), 7, dtype=np.int8)
    qw[:, ::2] = -7
    qw[5] = 7
    one_a = torch.ones(M, dtype=torch.float32, device="cuda")
    one_w = torch.ones(N, dtype=torch.float32, device="cuda")
    out = Q.qgemm_w4a4_fp6(to_dev(quad_fp6(O.pack_fp6(qa))), one_a, to_dev(quad_fp6(O.pack_fp6(qw))), one_w, K, epilogue="i32")
    torch.cuda.synchronize()
    want = O.int_gemm(qa, qw)
    assert np.array_equal(out.cpu().numpy().astype(np.int64), want)
    assert want[0, 5] == 49 * K and want[1, 5] == -49 * K


def _same_codes_pair(M, N, K, seed, mode):
    """Quantized operands in both layouts: (int8 codes, packed int4 weights)
    and (FP6 activations, FP6 weights), plus scales."""
    rng = np.random.default_rng(seed)
    qa = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    n_a, n_w = (1, 1) if mode == "tensor" else (M, N)
    sa = (rng.random(n_a, dtype=np.float32) * 0.02 + 0.005).astype(np.float32)
    sw = (rng.random(n_w, dtype=np.float32) * 0.02 + 0.005).astype(np.float32)
    return qa, qw, sa, sw


@pytest.mark.parametrize("M,N,K", [(257, 400, 1024), (4059, 5104, 512)])
@pytest.mark.parametrize("mode", ["row", "tensor"])
def test_fp6_epilogues_equal_int4_path(Q, M, N, K, mode):
    import torch

    qa, qw, sa_h, sw_h = _same_codes_pair(M, N, K, M + N, mode)
    sa, sw = to_dev_scales(sa_h), to_dev_scales(sw_h)
    a8, w4 = to_dev(qa), to_dev(pair_w4(O.pack_int4(qw)))
    a6, w6 = to_dev(quad_fp6(O.pack_fp6(qa))), to_dev(quad_fp6(O.pack_fp6(qw)))
    bias = to_dev_bf16(_rand_bf16(M, (N,), 0.1))
    rows = np.unique(np.concatenate([np.arange(4), M - 1 - np.arange(4),
                                     np.random.default_rng(M).choice(M, 40, replace=False)]))
    qa_o = O.QuantResult(qa[rows], sa_h if mode == "tensor" else sa_h[rows], 4, mode, None)
    qw_o = O.QuantResult(qw, sw_h, 4, mode, None)
    for epi in ("bf16", "f32", "sigmoid"):
        for bb in (None, bias):
            ref = Q.qgemm_w4a4(a8, sa, w4, sw, K, a_scale_mode=mode, w_scale_mode=mode, bias=bb, epilogue=epi)
            got = Q.qgemm_w4a4_fp6(a6, sa, w6, sw, K, a_scale_mode=mode, w_scale_mode=mode, bias=bb,
                                   epilogue=epi)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16) if epi != "f32" else got.view(torch.int32),
                               ref.view(torch.int16) if epi != "f32" else ref.view(torch.int32)), (epi, bb is None)
            # and the oracle, on sampled rows
            y, dy = P.linear_bound(qa_o, qw_o, bias_bits=None if bb is None else bf16_bits(bb))
            want, dw = P.epilogue_with_bound(y, dy, "bf16" if epi == "f32" else epi)
            g = got[torch.as_tensor(rows, device="cuda")]
            gv = g.cpu().numpy().astype(np.float64) if epi == "f32" else O.bf16_bits_to_f64(bf16_bits(g))
            P.assert_outputs_close(gv, want, dw, bf16=epi != "f32", what=f"fp6 {mode} {epi}")


def test_fp6_strided_output_and_empty(Q):
    import torch

    M, N, K = 4059, 5104, 512
    qa, qw, sa_h, sw_h = _same_codes_pair(M, N, K, 77, "row")
    sa, sw = to_dev_scales(sa_h), to_dev_scales(sw_h)
    a6, w6 = to_dev(quad_fp6(O.pack_fp6(qa))), to_dev(quad_fp6(O.pack_fp6(qw)))
    big = torch.zeros((M, N + 16), dtype=torch.bfloat16, device="cuda")
    out = Q.qgemm_w4a4_fp6(a6, sa, w6, sw, K, out=big[:, :N])
    ref = Q.qgemm_w4a4(to_dev(qa), sa, to_dev(pair_w4(O.pack_int4(qw))), sw, K)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert not big[:, N:].any().item(), "store past the row end"
    # M = 0 is a no-op
    e = Q.qgemm_w4a4_fp6(a6[:0], sa[:0], w6, sw, K)
    torch.cuda.synchronize()
    assert e.shape == (0, N)


def test_fp6_attention_projection_full_size(Q):
    """4096 x 5120 x 5120 from bf16 through both prologues and weight packers:
    the FP6 output equals the INT4 path's bit for bit; sampled rows of the
    exact sum equal the oracle's integer product."""
    import torch

    M, N, K = 4096, 5120, 5120
    torch.manual_seed(3)
    x = (torch.randn(M, K, device="cuda") * 1.0).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
    a8, sa8, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row", layout="i8")
    a6, sa6, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row", layout="fp6")
    w4, sw4 = Q.pack_weight_int4(w, scale_mode="row")
    w6, sw6 = Q.pack_weight_fp6(w, scale_mode="row")
    ref = Q.qgemm_w4a4(a8, sa8, w4, sw4, K)
    got = Q.qgemm_w4a4_fp6(a6, sa6, w6, sw6, K)
    acc = Q.qgemm_w4a4_fp6(a6, sa6, w6, sw6, K, epilogue="i32")
    torch.cuda.synchronize()
    assert torch.equal(sa6, sa8) and torch.equal(sw6, sw4)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([np.arange(4), M - 1 - np.arange(4), rng.choice(M, 24, replace=False)]))
    qa = O.unpack_fp6(unquad_fp6(a6.cpu().numpy())[rows])
    assert np.array_equal(qa, a8[rows].cpu().numpy())
    qw = O.unpack_int4(unpair_w4(w4.cpu().numpy()))
    assert np.array_equal(acc[rows].cpu().numpy().astype(np.int64), O.int_gemm(qa, qw))
    assert bf16_bits(got).shape == (M, N)


@pytest.mark.parametrize("N,K", [(6144, 5120), (20480, 5120), (5120, 6144)])
def test_fp6_stack_shapes_full_size(Q, N, K):
    """The W4A4 shapes of the 224-linear stack at 16384 tokens (Q / gate,
    gate|up, wo) as the stack_fp6 workload runs them: the FP6 output equals
    the INT4 path's bit for bit on the same codes, and the exact sums of
    sampled rows and columns equal the oracle's integer product."""
    import torch

    M = 16384
    torch.manual_seed(N + K)
    x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
    a8, sa8, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row", layout="i8")
    a6, sa6, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="row", layout="fp6")
    w4, sw4 = Q.pack_weight_int4(w, scale_mode="row")
    w6, sw6 = Q.pack_weight_fp6(w, scale_mode="row")
    ref = Q.qgemm_w4a4(a8, sa8, w4, sw4, K)
    got = Q.qgemm_w4a4_fp6(a6, sa6, w6, sw6, K)
    acc = Q.qgemm_w4a4_fp6(a6, sa6, w6, sw6, K, epilogue="i32")
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    rng = np.random.default_rng(N + K)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 10, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 254, replace=False)]))
    qa = O.unpack_fp6(unquad_fp6(a6.cpu().numpy())[rows])
    assert np.array_equal(qa, a8[rows].cpu().numpy())
    qw = O.unpack_fp6(unquad_fp6(w6.cpu().numpy())[cols])
    assert np.array_equal(qw, O.unpack_int4(unpair_w4(w4.cpu().numpy()))[cols])
    want = O.int_gemm(qa, qw)
    assert np.array_equal(acc[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")]
                          .cpu().numpy().astype(np.int64), want)


# ------------------------------------------------------- group-64 GEMM ------

def _group_pair(M, N, K, seed):
    """Codes in both layouts and group-64 scales [M, K/64], [N, K/64]."""
    rng = np.random.default_rng(seed)
    qa = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sa = (rng.random((M, K // 64), dtype=np.float32) * 0.02 + 0.005).astype(np.float32)
    sw = (rng.random((N, K // 64), dtype=np.float32) * 0.02 + 0.005).astype(np.float32)
    return qa, qw, sa, sw


# 256 x 128 tiles: one ragged tile, several with ragged M and N, and a long K
@pytest.mark.parametrize("M,N,K", [(1, 16, 256), (257, 400, 1024), (300, 656, 768), (1000, 2080, 2048),
                                   (64, 48, 20480)])
def test_fp6_group64_equals_int4_path(Q, M, N, K):
    import torch

    qa, qw, sa_h, sw_h = _group_pair(M, N, K, M + 3 * N + K)
    sa, sw = to_dev_scales(sa_h), to_dev_scales(sw_h)
    a8, w4 = to_dev(qa), to_dev(pair_w4(O.pack_int4(qw)))
    a6, w6 = to_dev(quad_fp6(O.pack_fp6(qa))), to_dev(quad_fp6(O.pack_fp6(qw)))
    bias = to_dev_bf16(_rand_bf16(N, (N,), 0.1))
    for epi in ("bf16", "f32"):
        for bb in (None, bias):
            ref = Q.qgemm_w4a4(a8, sa, w4, sw, K, a_scale_mode="group64", w_scale_mode="group64", bias=bb,
                               epilogue=epi)
            got = Q.qgemm_w4a4_fp6(a6, sa, w6, sw, K, a_scale_mode="group64", w_scale_mode="group64", bias=bb,
                                   epilogue=epi)
            torch.cuda.synchronize()
            iv = torch.int32 if epi == "f32" else torch.int16
            assert torch.equal(got.view(iv), ref.view(iv)), (epi, bb is None)
    if M * N * K > 2e8:
        return
    # the float result itself against the oracle's rescaled group sums: G
    # fp32 multiply-adds of exact partials err by at most (G + 3) u times the
    # sum of the terms' magnitudes (u = 2^-24)
    y = O.linear_fp64(O.QuantResult(qa, sa_h, 4, "group64", None), O.QuantResult(qw, sw_h, 4, "group64", None))
    got = Q.qgemm_w4a4_fp6(a6, sa, w6, sw, K, a_scale_mode="group64", w_scale_mode="group64", epilogue="f32")
    torch.cuda.synchronize()
    G = K // 64
    mag = np.zeros((M, N))
    for g in range(G):
        sl = slice(64 * g, 64 * g + 64)
        part = np.abs(qa[:, sl]).astype(np.float64) @ np.abs(qw[:, sl]).astype(np.float64).T
        mag += part * (sa_h[:, g].astype(np.float64)[:, None] * sw_h[:, g].astype(np.float64)[None, :])
    err = np.abs(got.cpu().numpy().astype(np.float64) - y)
    assert np.all(err <= (G + 3) * 2.0 ** -24 * mag)


@pytest.mark.parametrize("rank", [0, 32])
@pytest.mark.parametrize("epi", ["swiglu", "bf16"])
def test_fp6_group64_lowrank_equals_int4_path(Q, rank, epi):
    import torch

    M, N, K = 300, 640, 1024
    qa, qw, sa_h, sw_h = _group_pair(M, N, K, 5 + rank)
    sa, sw = to_dev_scales(sa_h), to_dev_scales(sw_h)
    lr = to_dev_bf16(_rand_bf16(6, (M, rank), 0.5)) if rank else None
    l2 = to_dev_l2(_rand_bf16(7, (rank, N), 0.05)) if rank else None
    ref = Q.qgemm_w4a4_lowrank(to_dev(qa), sa, to_dev(pair_w4(O.pack_int4(qw))), sw, K, lr=lr, l2=l2, epilogue=epi)
    got = Q.qgemm_w4a4_fp6_lowrank(to_dev(quad_fp6(O.pack_fp6(qa))), sa, to_dev(quad_fp6(O.pack_fp6(qw))), sw, K, lr=lr, l2=l2,
                                   epilogue=epi)
    torch.cuda.synchronize()
    assert got.shape == ref.shape
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # the oracle: dequantized group sums plus lr L2 (lr as given), through the epilogue
    y, dy = P.linear_bound(O.QuantResult(qa, sa_h, 4, "group64", None), O.QuantResult(qw, sw_h, 4, "group64", None))
    if rank:
        lrf, l2f = O.bf16_bits_to_f64(bf16_bits(lr)), O.bf16_bits_to_f64(bf16_bits(l2).T)
        y = y + lrf @ l2f
        dy = dy + (rank + 4) * P.U * (np.abs(lrf) @ np.abs(l2f)) + 3 * P.U * np.abs(lrf @ l2f)
    want, dw = P.epilogue_with_bound(y, dy, epi)
    P.assert_outputs_close(O.bf16_bits_to_f64(bf16_bits(got)), want, dw, what=f"fp6 group64 r{rank} {epi}")


def test_fp6_group64_rejections(Q):
    import torch

    M, N, K = 32, 64, 256
    qa, qw, sa_h, sw_h = _group_pair(M, N, K, 1)
    a6, w6 = to_dev(quad_fp6(O.pack_fp6(qa))), to_dev(quad_fp6(O.pack_fp6(qw)))
    with pytest.raises(Q.QLinearError):   # group sums are rescaled: no exact I32 result
        Q.qgemm_w4a4_fp6(a6, to_dev_scales(sa_h), w6, to_dev_scales(sw_h), K, a_scale_mode="group64",
                         w_scale_mode="group64", epilogue="i32")
    row_a = torch.ones(M, dtype=torch.float32, device="cuda")
    row_w = torch.ones(N, dtype=torch.float32, device="cuda")
    with pytest.raises(Q.QLinearError):   # the INT4 low-rank GEMM takes no FP6 operands
        Q.qgemm_w4a4_lowrank(a6, to_dev_scales(sa_h), w6, to_dev_scales(sw_h), K, a_layout="fp6", epilogue="bf16")
    with pytest.raises(Q.QLinearError):   # the FP6 low-rank GEMM has no I32 or sigmoid epilogue
        Q.qgemm_w4a4_fp6_lowrank(a6, to_dev_scales(sa_h), w6, to_dev_scales(sw_h), K, epilogue="sigmoid")
    del row_a, row_w


def test_fp6_group64_svdq_gateup_full_size(Q):
    """The SVDQuant gate|up layer, 4096 x 40960 x 5120 with group-64 scales, a
    rank-32 branch and SwiGLU, from bf16 through both prologues and weight
    packers: the FP6 output equals the INT8 path's bit for bit."""
    import torch

    M, N, K, r = 4096, 40960, 5120, 32
    torch.manual_seed(11)
    x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
    l1 = (torch.randn(K, r, device="cuda") * 0.02).to(torch.bfloat16)
    l2 = (torch.randn(N, r, device="cuda") * 0.02).to(torch.bfloat16)  # L2 transposed
    a8, sa8, lr = Q.rotate_quantize_act(x, bits=4, scale_mode="group64", layout="i8", l1=l1)
    a6, sa6, _ = Q.rotate_quantize_act(x, bits=4, scale_mode="group64", layout="fp6")
    w4, sw4 = Q.pack_weight_int4(w, scale_mode="group64")
    w6, sw6 = Q.pack_weight_fp6(w, scale_mode="group64")
    ref = Q.qgemm_w4a4_lowrank(a8, sa8, w4, sw4, K, lr=lr, l2=l2, epilogue="swiglu")
    got = Q.qgemm_w4a4_fp6_lowrank(a6, sa6, w6, sw6, K, lr=lr, l2=l2, epilogue="swiglu")
    torch.cuda.synchronize()
    assert torch.equal(sa6, sa8) and torch.equal(sw6, sw4)
    assert got.shape == (M, N // 2)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # sampled rows and gate|up pairs against the oracle on the device's codes
    rng = np.random.default_rng(12)
    rows = np.sort(rng.choice(M, 12, replace=False))
    fs = np.sort(rng.choice(N // 2, 192, replace=False))
    ns = np.concatenate([fs, N // 2 + fs])
    ri = torch.as_tensor(rows, device="cuda")
    qa = O.QuantResult(O.unpack_fp6(unquad_fp6(a6.cpu().numpy())[rows]), sa6[ri].cpu().numpy(), 4, "group64", None)
    qw = O.QuantResult(O.unpack_fp6(unquad_fp6(w6.cpu().numpy())[ns]), sw6.cpu().numpy()[ns],
                       4, "group64", None)
    y, dy = P.linear_bound(qa, qw, bf16_bits(x[ri]), bf16_bits(l1), np.ascontiguousarray(bf16_bits(l2)[ns].T))
    want, dw = P.epilogue_with_bound(y, dy, "swiglu")
    P.assert_outputs_close(O.bf16_bits_to_f64(bf16_bits(got[ri][:, torch.as_tensor(fs, device="cuda")])),
                           want, dw, what="fp6 svdq gate|up")
