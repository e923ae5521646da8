"""GPU parity of the offline SVDQuant split (svdq_split) against the oracle.

The randomized SVD runs in fp32 on the device and in fp64 in the oracle, with
the same sketch.  Where the leading rank-r subspace is well separated the
branch itself is compared; otherwise singular vectors are not unique under
rounding, and the checks are what is unique: singular values, the objective
of every iteration, the selection of the best one, and that the returned
(L1, L2, codes, scales) achieve the reported objective and are the rotated
INT4 quantization of their own residual.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import parity_checks as P
from tests.helpers import bf16_bits, ensure_built, to_dev, to_dev_bf16, unpair_w4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import torch

    ensure_built()
    import rotated_bit_quantized_rotate_amd as Q

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert Q.device_supported(0), "device is not gfx950"
    return Q


def _run(Q, wb, omega, rank, over, pi, ri, mode, rms=None):
    import torch

    out = Q.svdq_split(to_dev_bf16(wb), to_dev(omega), rank, over, pi, ri, mode,
                       act_rms=None if rms is None else to_dev(rms))
    torch.cuda.synchronize()
    g = {k: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in out.items()}
    g["l2"] = np.ascontiguousarray(g["l2"].T)  # the library stores L2 transposed, [N, rank]
    g["packed"] = unpair_w4(g["packed"])  # and packed weights in paired-row order
    return g


def _check_split_quant(codes, scales, wb, l1_bits, l2_bits, mode, budget=P.FLIP_BUDGET):
    """The device's residual codes and scales against the oracle's definition
    applied to the residual of the device's own factors.  The device forms
    T = W - (L1 L2)^T in float32 (a rank-r sum, then the subtraction: at most
    (r + 2) u sum_r |L1 L2| + u |T| off) and rounds it to bf16; where T lies
    that close to a bf16 rounding tie the device's bf16 input may be the
    other neighbour, so those elements carry one bf16 step of input error
    into the rotation bound, the near-tie windows and the scale bound."""
    Wf = O.bf16_bits_to_f64(wb)
    l1 = O.bf16_bits_to_f64(l1_bits)
    l2 = O.bf16_bits_to_f64(l2_bits)
    T = Wf - (l1 @ l2).T
    errT = (l1.shape[1] + 2) * P.U * (np.abs(l1) @ np.abs(l2)).T + P.U * np.abs(T)
    lo, hi = O.bf16_round(T - errT), O.bf16_round(T + errT)
    pre = np.abs(hi - lo)                     # 0 unless T sits within errT of a tie
    Tb = O.bf16_round(T)
    return P.check_codes(codes, scales, O.rotate(Tb), P.rotation_error_bound(Tb, pre), 4, mode, budget)


def _objective(wb, g, mode, rms):
    """||(W - B - unrotate(deq(Q))) D||_F from the device's own outputs, and
    the oracle's quantization of the device's residual."""
    Wf = O.bf16_bits_to_f64(wb)
    d = np.ones(Wf.shape[1]) if rms is None else O.act_weights(rms)
    T = Wf - (O.bf16_bits_to_f64(g["l1"]) @ O.bf16_bits_to_f64(g["l2"])).T
    codes = O.unpack_int4(g["packed"])
    E = O.rotate(O.dequantize(codes, g["scales"], mode))
    return float(np.linalg.norm((T - E) * d[None, :])), O.quantize_weights(O.f64_to_bf16_bits(T), 4, mode, True), codes


@pytest.mark.parametrize("mode", ["group64", "row"])
@pytest.mark.parametrize("weighted", [False, True])
def test_split_gapped_weight_matches_oracle(Q, mode, weighted):
    N, K, r, over = 512, 1024, 32, 8
    wb = W.spectral_weight_bf16(N, K, 21, r, top=2.0, decay=0.95, noise=1e-4)
    omega = W.gaussian_sketch(K, r + over, 22)
    rms = W.act_rms(K, 23) if weighted else None
    ref = O.svdq_split(wb, omega, r, 2, 0, mode, rms)
    g = _run(Q, wb, omega, r, over, 2, 0, mode, rms)
    assert np.allclose(g["sigma"], ref.sigma, rtol=1e-3, atol=0)
    branch = (O.bf16_bits_to_f64(ref.l1_bits) @ O.bf16_bits_to_f64(ref.l2_bits)).T
    got = (O.bf16_bits_to_f64(g["l1"]) @ O.bf16_bits_to_f64(g["l2"])).T
    assert np.abs(got - branch).max() <= 2e-2 * np.abs(branch).max()
    # The residual of a nearly low-rank weight is tiny and dominated by the
    # bf16 rounding of L1 and L2, so one-ulp differences between the fp32 and
    # fp64 factors move its codes: the codes are checked against the oracle's
    # quantization of the device's own residual below, and the objective to 5 %.
    assert abs(g["errors"][0] - ref.errors[0]) <= 5e-2 * ref.errors[0]
    assert g["best_iter"][0] == 0
    obj, q, codes = _objective(wb, g, mode, rms)
    assert abs(obj - g["errors"][0]) <= 1e-4 * obj
    # this residual is almost pure rounding of the factors, so many of its
    # elements sit near bf16 ties: the near-tie flips may reach 1e-3 here
    _check_split_quant(codes, g["scales"], wb, g["l1"], g["l2"], mode, budget=1e-3)


@pytest.mark.parametrize("weighted", [False, True])
def test_split_refinement_flat_spectrum(Q, weighted):
    """A plain N(0, 0.02) weight (flat spectrum): the refinement's objectives
    track the oracle's, the best one is returned, and it is what the
    returned factors and codes achieve."""
    N, K, r, over, ri = 256, 512, 32, 8, 3
    wb = W.normal_bf16(np.random.default_rng(31), (N, K), 0.02)
    omega = W.gaussian_sketch(K, r + over, 32)
    rms = W.act_rms(K, 33) if weighted else None
    ref = O.svdq_split(wb, omega, r, 2, ri, "group64", rms)
    g = _run(Q, wb, omega, r, over, 2, ri, "group64", rms)
    e = g["errors"].astype(np.float64)
    # iteration one agrees closely; later iterations start from the previous
    # one's codes, whose +-1 flips compound on a flat spectrum
    assert abs(e[0] - ref.errors[0]) <= 2e-2 * ref.errors[0], (e, ref.errors)
    assert np.allclose(e, ref.errors, rtol=1e-1, atol=0), (e, ref.errors)
    best = int(g["best_iter"][0])
    assert best == int(np.argmin(e))
    assert e[best] <= e[0]
    obj, q, codes = _objective(wb, g, "group64", rms)
    assert abs(obj - e[best]) <= 1e-4 * obj
    _check_split_quant(codes, g["scales"], wb, g["l1"], g["l2"], "group64")
    # the returned sigma belongs to the returned fit: descending, non-negative
    s = g["sigma"]
    assert np.all(s[:-1] >= s[1:]) and s[-1] >= 0


def test_split_deterministic_and_tensor_scales(Q):
    N, K, r, over = 256, 512, 16, 8
    wb = W.normal_bf16(np.random.default_rng(41), (N, K), 0.02)
    omega = W.gaussian_sketch(K, r + over, 42)
    a = _run(Q, wb, omega, r, over, 1, 2, "tensor")
    b = _run(Q, wb, omega, r, over, 1, 2, "tensor")
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    ref = O.svdq_split(wb, omega, r, 1, 2, "tensor")
    assert np.allclose(a["errors"], ref.errors, rtol=2e-2)


def test_split_zero_weight(Q):
    N, K, r, over = 64, 256, 16, 8
    g = _run(Q, np.zeros((N, K), np.uint16), W.gaussian_sketch(K, r + over, 1), r, over, 2, 1, "row")
    assert not g["l1"].any() and not g["l2"].any() and not g["packed"].any()
    assert np.all(g["errors"] == 0) and np.all(g["sigma"] == 0)


def test_split_full_size_gateup(Q):
    """The svdq gate|up weight [40960 x 5120] at rank 32 with one refinement:
    objectives finite and best-kept, sigma descending, and sampled rows of the
    returned codes and scales equal the oracle's quantization of the returned
    residual."""
    import time

    import torch

    wl = W.svdq_gateup()
    wb = wl.w
    N, K = wb.shape
    r, over = 32, 8
    omega = W.gaussian_sketch(K, r + over, 0)
    w = to_dev_bf16(wb)
    om = to_dev(omega)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = Q.svdq_split(w, om, r, over, 2, 1, "group64")
    torch.cuda.synchronize()
    print(f"svdq_split 40960x5120 r32 (2 iterations): {time.perf_counter() - t0:.3f} s", flush=True)
    e = out["errors"].cpu().numpy()
    best = int(out["best_iter"].cpu().numpy()[0])
    assert np.all(np.isfinite(e)) and best == int(np.argmin(e))
    s = out["sigma"].cpu().numpy()
    assert np.all(s[:-1] >= s[1:]) and s[0] > 0
    rows = np.unique(np.concatenate([np.arange(4), N - 1 - np.arange(4),
                                     np.random.default_rng(5).choice(N, 24, replace=False)]))
    ri = torch.as_tensor(rows, device="cuda")
    codes = O.unpack_int4(unpair_w4(out["packed"].cpu().numpy())[rows])
    _check_split_quant(codes, out["scales"][ri].cpu().numpy(), np.ascontiguousarray(wb[rows]), bf16_bits(out["l1"]),
                       np.ascontiguousarray(bf16_bits(out["l2"])[rows].T), "group64")
    # the objective is a few percent of the weight
    assert 0.0 < e[best] < 0.2 * float(np.linalg.norm(O.bf16_bits_to_f64(wb[:2048]))) * np.sqrt(N / 2048)
