"""Pins of the offline low-rank split oracle (oracle/svdq_split_ref.py)
against what the mathematics and the page fix, independent of the oracle's
own code paths: closed-form weight normalization, exact recovery of
low-rank matrices, agreement with the full SVD under fast spectral decay,
the plain split rebuilt from a full SVD, best-kept refinement, and the zero
and scale-invariance cases."""

import numpy as np
import pytest

import oracle as O
import workloads as W


def _orth(rng, n, r):
    q, _ = np.linalg.qr(rng.standard_normal((n, r)))
    return q


def test_act_weights_closed_form():
    d = O.act_weights([1.0, 2.0, 3.0, 0.002])
    mean = (1.0 + 2.0 + 3.0 + 0.002) / 4
    assert np.allclose(d, [1.0 / mean, 2.0 / mean, 3.0 / mean, 0.05], rtol=0, atol=1e-15)
    # no channel below the floor: mean exactly 1
    d2 = O.act_weights([0.5, 1.5, 1.0, 1.0])
    assert abs(d2.mean() - 1.0) < 1e-15 and d2.min() == 0.5
    # scale invariance
    assert np.array_equal(O.act_weights(np.array([2.0, 6.0, 4.0])), O.act_weights(np.array([1.0, 3.0, 2.0])))


def test_randomized_svd_recovers_low_rank_exactly():
    rng = np.random.default_rng(1)
    n, k, r = 120, 200, 6
    s_true = np.array([5.0, 4.0, 3.0, 2.0, 1.0, 0.5])
    U, V = _orth(rng, n, r), _orth(rng, k, r)
    A = (U * s_true) @ V.T
    for q in (0, 2):
        Ur, s, Vt = O.randomized_svd(A, rng.standard_normal((k, 10)), r, q)
        assert np.allclose(s, s_true, rtol=0, atol=1e-12)
        assert np.allclose((Ur * s) @ Vt, A, rtol=0, atol=1e-12)
        assert np.allclose(Ur.T @ Ur, np.eye(r), atol=1e-12) and np.allclose(Vt @ Vt.T, np.eye(r), atol=1e-12)


def test_randomized_svd_matches_full_svd_under_fast_decay():
    # sigma_j = 2^-j: with l = 16 and two power iterations the subspace error
    # is of order (sigma_17 / sigma_8)^5 = 2^-45, far below the tolerance
    rng = np.random.default_rng(2)
    n, k, full = 200, 300, 60
    s_all = 2.0 ** -np.arange(full)
    A = (_orth(rng, n, full) * s_all) @ _orth(rng, k, full).T
    r = 8
    Ur, s, Vt = O.randomized_svd(A, rng.standard_normal((k, 16)), r, 2)
    assert np.allclose(s, s_all[:r], rtol=1e-10, atol=0)
    U0, s0, Vt0 = np.linalg.svd(A)
    assert np.allclose((Ur * s) @ Vt, (U0[:, :r] * s0[:r]) @ Vt0[:r], rtol=0, atol=1e-10)


def _gapped_weight(seed, N=256, K=512, r=16):
    """bf16 weight: a rank-r signal well above a small noise floor, so the
    leading rank-r subspace is well separated."""
    return W.spectral_weight_bf16(N, K, seed, r, top=2.0, decay=0.95, noise=1e-4)


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("mode", ["row", "group64"])
def test_plain_split_equals_full_svd_construction(weighted, mode):
    """Iteration one is the plain split: branch = SVD_r(W D) D^-1 in bf16,
    residual quantized.  Rebuilt here with the full SVD (not the randomized
    one) on a gapped weight, where both agree."""
    N, K, r = 256, 512, 16
    wb = _gapped_weight(3, N, K, r)
    rms = W.act_rms(K, 4) if weighted else None
    omega = W.gaussian_sketch(K, r + 8, 5)
    res = O.svdq_split(wb, omega, r, power_iters=2, refine_iters=0, scale_mode=mode, act_rms=rms)
    Wf = O.bf16_bits_to_f64(wb)
    d = np.ones(K) if rms is None else O.act_weights(rms)
    U, s, Vt = np.linalg.svd(Wf * d[None, :], full_matrices=False)
    L1 = O.bf16_round((Vt[:r].T * np.sqrt(s[:r])) / d[:, None])
    L2 = O.bf16_round((U[:, :r] * np.sqrt(s[:r])).T)
    branch = (L1 @ L2).T
    got_branch = (O.bf16_bits_to_f64(res.l1_bits) @ O.bf16_bits_to_f64(res.l2_bits)).T
    # singular vectors of a gapped matrix agree up to sign; the product is sign-free
    assert np.abs(got_branch - branch).max() <= 2e-2 * np.abs(branch).max()
    assert np.allclose(res.sigma, s[:r], rtol=1e-9)
    assert res.best == 0 and res.errors.shape == (1,)
    # the residual's quantization and the objective, rebuilt from the returned branch
    T = Wf - got_branch
    q = O.quantize_weights(O.f64_to_bf16_bits(T), 4, mode, True)
    assert np.array_equal(q.codes, res.quant.codes) and np.array_equal(q.scales, res.quant.scales)
    E = O.rotate(O.dequantize(q.codes, q.scales, mode))
    assert abs(np.linalg.norm((T - E) * d[None, :]) - res.errors[0]) <= 1e-12 * res.errors[0]
    # the error is the INT4 quantization error of the residual: a few percent of
    # the weight (a missing unrotation would make it as large as the weight)
    rel = res.errors[0] / np.linalg.norm(Wf * d[None, :])
    assert 1e-4 < rel < 0.15, rel


def test_refinement_keeps_the_best_and_never_does_worse():
    N, K, r = 256, 512, 32
    wb = W.normal_bf16(np.random.default_rng(6), (N, K), 0.02)
    omega = W.gaussian_sketch(K, r + 8, 7)
    plain = O.svdq_split(wb, omega, r, 2, 0, "group64")
    ref = O.svdq_split(wb, omega, r, 2, 4, "group64")
    assert ref.errors.shape == (5,)
    assert ref.errors[0] == plain.errors[0]                  # iteration one is the plain split
    assert ref.best == int(np.argmin(ref.errors))
    assert ref.errors[ref.best] <= plain.errors[0]
    assert ref.errors[ref.best] < plain.errors[0]            # on this weight refining helps
    if ref.best == 0:
        assert np.array_equal(ref.quant.codes, plain.quant.codes)


def test_refinement_refits_to_the_previous_iterate_not_the_best():
    """Iteration t > 1 fits the branch to W - unrotate(deq(Q_{t-1})), the
    iterate just before it, even when an earlier one was better.  On this
    weight (tensor scales) iteration 4 is worse than iteration 3, so the
    readings "from the previous iterate" and "from the best so far" part
    ways from iteration 5 on (index 4).  The sketch has as many columns as W
    has rows and no power steps are needed: its range is W's whole column
    space, so every fit is the exact truncated SVD, rebuilt here with
    numpy's full SVD."""
    N, K, r = 64, 256, 4
    wb = W.normal_bf16(np.random.default_rng(2), (N, K), 0.02)
    res = O.svdq_split(wb, W.gaussian_sketch(K, N, 102), r, 0, 6, "tensor")
    Wf = O.bf16_bits_to_f64(wb)

    def fit_to(t):
        q = res.history[t][2]
        U, s, Vt = np.linalg.svd(Wf - O.rotate(O.dequantize(q.codes, q.scales, "tensor")), full_matrices=False)
        return (U[:, :r] * s[:r]) @ Vt[:r]

    parted = 0
    for t in range(1, 7):
        l1, l2, _ = res.history[t]
        got = (O.bf16_bits_to_f64(l1) @ O.bf16_bits_to_f64(l2)).T
        want = fit_to(t - 1)
        scale = np.abs(want).max()
        assert np.abs(got - want).max() <= 1e-2 * scale, t          # bf16 factors: ~0.5 %
        best_before = int(np.argmin(res.errors[:t]))
        if best_before != t - 1:
            parted += 1
            assert np.abs(got - fit_to(best_before)).max() > 3e-2 * scale, t
    assert parted >= 2   # the case really separates the two readings
    assert res.best == int(np.argmin(res.errors))


def test_zero_weight_and_constant_act_stats():
    N, K, r = 32, 256, 16
    zero = np.zeros((N, K), dtype=np.uint16)
    res = O.svdq_split(zero, W.gaussian_sketch(K, r + 8, 1), r, 2, 1, "row")
    assert not res.l1_bits.any() and not res.l2_bits.any()
    assert not res.quant.codes.any() and np.all(res.errors == 0.0)
    # constant activation statistics normalize to d = 1: same as none
    wb = W.normal_bf16(np.random.default_rng(8), (N, K), 0.02)
    om = W.gaussian_sketch(K, r + 8, 2)
    a = O.svdq_split(wb, om, r, 2, 1, "row")
    b = O.svdq_split(wb, om, r, 2, 1, "row", act_rms=np.full(K, 3.5))
    assert np.array_equal(a.l1_bits, b.l1_bits) and np.array_equal(a.quant.codes, b.quant.codes)
    assert np.array_equal(a.errors, b.errors)


def test_act_aware_fit_lowers_the_weighted_branch_error():
    """Before quantization, the weighted fit is the best rank-r approximation
    in the weighted norm, so it beats the unweighted fit there."""
    N, K, r = 128, 512, 16
    wb = W.normal_bf16(np.random.default_rng(9), (N, K), 0.02)
    Wf = O.bf16_bits_to_f64(wb)
    d = O.act_weights(W.act_rms(K, 10))
    om = W.gaussian_sketch(K, r + 8, 11)
    l1w, l2w, _ = O.svdq_branch(Wf, d, om, r, 4)
    l1u, l2u, _ = O.svdq_branch(Wf, np.ones(K), om, r, 4)
    ew = np.linalg.norm((Wf - (l1w @ l2w).T) * d[None, :])
    eu = np.linalg.norm((Wf - (l1u @ l2u).T) * d[None, :])
    assert ew < eu
