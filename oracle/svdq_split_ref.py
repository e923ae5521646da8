"""Oracle of the offline SVDQuant low-rank split -- TEST INFRASTRUCTURE ONLY.

Source: README "Krea-2-SVDQuant-ComfyUI", sections on reproducible builds
(the split is a seeded randomized SVD), "Activation-aware branch" (the fit
is weighted by per-input-channel activation RMS d, normalized to mean 1 and
floored at 0.05) and "Low-rank refinement, and what the objective actually
is" (the branch is refit to the current quantization error and the residual
requantized, repeatedly, keeping the best; iteration one is the plain
single-shot split, so refining never does worse).

Readings taken where the page leaves a step open:
  * The split is W ~= Q + B with B = (L1 L2)^T the branch in the torch
    Linear layout [N, K] (the layer computes y += (x L1) L2), Q the rotated
    INT4 quantization of the residual W - B, reconstructed in the original
    basis as unrotate(deq(Q)).  L1 [K, r] and L2 [r, N] are stored as bf16
    and the residual is formed against those rounded factors, then rounded to
    bf16 before it is quantized (the quantizer's input format).
  * Objective (the reconstruction error each iteration reports):
    || (W - B - unrotate(deq(Q))) D ||_F with D = diag(d), d = 1 without
    activation statistics.
  * Iteration 1 fits B to W D; iteration t > 1 fits B to (W - unrotate(deq(Q)))
    D with the Q of iteration t - 1; each weighted fit of rank r is
    SVD_r(target D) D^-1.  The best iteration by the objective is returned.
  * The randomized SVD is randomized subspace iteration (Halko, Martinsson
    and Tropp, "Finding structure with randomness", 2011, Algorithm 4.4):
    Y = A Omega, Q = orth(Y); per power iteration Z = orth(A^T Q),
    Q = orth(A Z); then B = Q^T A, its SVD B = U~ S V^T, U = Q U~, truncated
    to the leading r triples.  Omega [K, r + p] is a Gaussian sketch passed
    in (drawn from a seeded generator by the caller).  The factors split S
    evenly: L1 = V_r S_r^1/2 / d (row k divided by d_k), L2 = (U_r S_r^1/2)^T.
    Singular values below 1e-5 of the largest are dropped (their component
    is set to zero).

Everything is float64 NumPy; numpy.linalg.qr and numpy.linalg.svd are the
library steps.
"""

from __future__ import annotations

import numpy as np

from .qlinear_ref import bf16_bits_to_f64, bf16_round, dequantize, f64_to_bf16_bits, quantize_weights, rotate

__all__ = ["act_weights", "randomized_svd", "svdq_branch", "svdq_split", "SplitResult"]

SIGMA_DROP = 1e-5   # singular values below this fraction of the largest are dropped
D_FLOOR = 0.05      # floor of the normalized activation weights


def act_weights(rms) -> np.ndarray:
    """Per-input-channel weights of the activation-aware objective: the
    channel RMS normalized to mean 1, then floor-clamped at 0.05."""
    rms = np.asarray(rms, dtype=np.float64)
    d = rms / rms.mean()
    return np.maximum(d, D_FLOOR)


def randomized_svd(A: np.ndarray, omega: np.ndarray, rank: int, power_iters: int):
    """Leading `rank` singular triples of A [n, k] by randomized subspace
    iteration with the sketch omega [k, l], l >= rank.  Returns (U [n, r],
    s [r], Vt [r, k])."""
    A = np.asarray(A, dtype=np.float64)
    Y = A @ np.asarray(omega, dtype=np.float64)
    Q, _ = np.linalg.qr(Y)
    for _ in range(power_iters):
        Z, _ = np.linalg.qr(A.T @ Q)
        Q, _ = np.linalg.qr(A @ Z)
    B = Q.T @ A
    Ub, s, Vt = np.linalg.svd(B, full_matrices=False)
    return (Q @ Ub)[:, :rank], s[:rank], Vt[:rank]


def svdq_branch(target: np.ndarray, d: np.ndarray, omega: np.ndarray, rank: int, power_iters: int):
    """Weighted rank-r fit of target [N, K]: SVD_r(target D) D^-1, returned as
    bf16-rounded float64 factors L1 [K, r], L2 [r, N] (branch = (L1 L2)^T),
    plus the kept singular values."""
    U, s, Vt = randomized_svd(target * d[None, :], omega, rank, power_iters)
    keep = s > SIGMA_DROP * s[0] if s.size and s[0] > 0 else np.zeros(s.shape, bool)
    root = np.where(keep, np.sqrt(np.where(keep, s, 0.0)), 0.0)
    L1 = (Vt.T * root[None, :]) / d[:, None]
    L2 = (U * root[None, :]).T
    return bf16_round(L1), bf16_round(L2), np.where(keep, s, 0.0)


class SplitResult:
    """Best split of svdq_split: branch factors as bf16 bits, the residual's
    quantization, the objective of every iteration and the best index."""

    def __init__(self, l1_bits, l2_bits, quant, errors, best, sigma, history):
        self.l1_bits = l1_bits      # uint16 [K, r]
        self.l2_bits = l2_bits      # uint16 [r, N]
        self.quant = quant          # QuantResult of the residual (codes, scales)
        self.errors = errors        # float64 [iterations]
        self.best = best            # index of the returned iteration
        self.sigma = sigma          # float64 [r] singular values of the best iteration's fit
        self.history = history      # per iteration: (l1_bits, l2_bits, QuantResult of its residual)


def svdq_split(w_bits, omega, rank: int, power_iters: int = 2, refine_iters: int = 0,
               scale_mode: str = "row", act_rms=None) -> SplitResult:
    """The offline split W ~= Q + (L1 L2)^T with INT4 rotated Q, keeping the
    best of 1 + refine_iters alternating iterations (see the module
    docstring)."""
    W = bf16_bits_to_f64(w_bits)
    N, K = W.shape
    d = np.ones(K) if act_rms is None else act_weights(act_rms)
    E = np.zeros_like(W)                      # unrotate(deq(Q)) of the previous iteration
    errors = []
    history = []
    best = None
    for t in range(refine_iters + 1):
        L1, L2, s = svdq_branch(W - E, d, omega, rank, power_iters)
        T = W - (L1 @ L2).T                   # W - B
        q = quantize_weights(f64_to_bf16_bits(T), 4, scale_mode, True)
        E = rotate(dequantize(q.codes, q.scales, scale_mode))   # Hn is its own inverse
        err = float(np.linalg.norm((T - E) * d[None, :]))
        errors.append(err)
        history.append((f64_to_bf16_bits(L1), f64_to_bf16_bits(L2), q))
        if best is None or err < errors[best[0]]:
            best = (t, L1, L2, q, s)
    t, L1, L2, q, s = best
    return SplitResult(f64_to_bf16_bits(L1), f64_to_bf16_bits(L2), q, np.array(errors), t, s, history)
