"""Seeded synthetic inputs for the rotated low-bit quantized linear.

This module only draws random tensors and rounds them to bfloat16 bit
patterns.  It holds none of the method's arithmetic (no rotation, no
quantization, no GEMM, no epilogue), so it can feed both the CPU oracle and
the HIP path without coupling them.

Every tensor is returned as a ``numpy.uint16`` array of bfloat16 bit patterns
(row-major), the form both sides consume.  Draws use
``numpy.random.default_rng(seed)`` in float32, in the order each recipe lists,
followed by one round-to-nearest-even cast to bfloat16 (done by torch's
float32 -> bfloat16 conversion).

Workload shapes follow the pages: a 28-block diffusion transformer with model
width 5120 and feed-forward width 20480 at 1024x1024 (4096 image tokens) and
2048x2048 (16384 tokens) (model cards "Krea 2 Turbo OrbitQuant W4A4",
section "Fused transformer", and "Krea-2-SVDQuant-ComfyUI", section
"--rank-alloc", which gives 48 query heads and 12 key/value heads of width
128).  The pages measure on prompts and trained checkpoints; these seeded
normal tensors stand in for both.
"""

from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "to_bf16_bits",
    "normal_bf16",
    "with_outlier_channels",
    "Workload",
    "tiny_w4a4",
    "attn_proj_w4a4",
    "ffdown_w8a8",
    "svdq_gateup",
    "stack_layers",
    "stack_layer",
    "gaussian_sketch",
    "spectral_weight_bf16",
    "act_rms",
]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draw in float32, returned as bfloat16 bits."""
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16_bits(a)


def with_outlier_channels(rng: np.random.Generator, a: np.ndarray, n_channels: int,
                          factor: float) -> tuple[np.ndarray, np.ndarray]:
    """Scale ``n_channels`` distinct input channels (columns) of float32 ``a``
    by ``factor`` in place.  Channels are drawn without replacement.
    Returns (a, channel_indices)."""
    ch = rng.choice(a.shape[1], size=n_channels, replace=False)
    a[:, ch] *= np.float32(factor)
    return a, np.sort(ch)


@dataclasses.dataclass
class Workload:
    """One linear-layer workload: bf16 bit tensors plus its quantization recipe."""

    name: str
    x: np.ndarray                 # [M, K] bf16 bits
    w: np.ndarray                 # [N, K] bf16 bits
    a_bits: int                   # 4 or 8
    w_bits: int                   # 4 or 8
    scale_mode: str               # "tensor" | "row" | "group64"
    epilogue: str                 # "bf16" | "gated_residual" | "swiglu"
    rotate: bool = True
    l1: np.ndarray | None = None  # [K, r] bf16 bits
    l2: np.ndarray | None = None  # [r, N] bf16 bits
    residual: np.ndarray | None = None  # [M, N] bf16 bits
    gate: np.ndarray | None = None      # [N] bf16 bits
    outlier_channels: np.ndarray | None = None

    @property
    def M(self) -> int:
        return self.x.shape[0]

    @property
    def K(self) -> int:
        return self.x.shape[1]

    @property
    def N(self) -> int:
        return self.w.shape[0]

    @property
    def int_ops(self) -> int:
        """Algorithmic integer operations of the contraction, 2*M*N*K."""
        return 2 * self.M * self.N * self.K


def tiny_w4a4(seed: int = 0, M: int = 64, K: int = 256, N: int = 256) -> Workload:
    """Tiny tensorwise W4A4 linear: X ~ N(0,1) with 4 outlier channels x20,
    W ~ N(0, 0.02); one rng, draws X, channel choice, W."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(M, K), dtype=np.float32)
    x, ch = with_outlier_channels(rng, x, 4, 20.0)
    w = rng.standard_normal(size=(N, K), dtype=np.float32) * np.float32(0.02)
    return Workload("tiny_w4a4", to_bf16_bits(x), to_bf16_bits(w), 4, 4, "tensor", "bf16",
                    outlier_channels=ch)


def attn_proj_w4a4(M: int = 4096, K: int = 5120, N: int = 5120, x_seed: int = 0,
                   w_seed: int = 1, outlier_frac: float = 0.01,
                   outlier_factor: float = 30.0) -> Workload:
    """DiT attention projection at 1024^2: X [4096 x 5120] ~ N(0,1) with
    floor(1% of K) outlier channels x30 (rng seed 0: X then channels),
    W [5120 x 5120] ~ N(0, 0.02) (seed 1); per-token / per-row int4."""
    rx = np.random.default_rng(x_seed)
    x = rx.standard_normal(size=(M, K), dtype=np.float32)
    x, ch = with_outlier_channels(rx, x, int(outlier_frac * K), outlier_factor)
    w = normal_bf16(np.random.default_rng(w_seed), (N, K), 0.02)
    return Workload("attn_proj_w4a4", to_bf16_bits(x), w, 4, 4, "row", "bf16",
                    outlier_channels=ch)


def ffdown_w8a8(M: int = 4096, K: int = 20480, N: int = 5120, seeds=(2, 3, 4, 5)) -> Workload:
    """Protected ff.down in W8A8 with a gated residual: X = silu(a)*b in float32
    with a, b ~ N(0,1) (seeds 2, 3), W ~ N(0, 0.01) (seed 4), residual
    [M x N] ~ N(0,1) then gate [N] ~ N(0,1) (seed 5).  The silu here only
    shapes the input distribution like a post-SwiGLU activation."""
    a = np.random.default_rng(seeds[0]).standard_normal(size=(M, K), dtype=np.float32)
    b = np.random.default_rng(seeds[1]).standard_normal(size=(M, K), dtype=np.float32)
    x = (a / (np.float32(1.0) + np.exp(-a))) * b
    del a, b
    w = normal_bf16(np.random.default_rng(seeds[2]), (N, K), 0.01)
    rr = np.random.default_rng(seeds[3])
    res = normal_bf16(rr, (M, N))
    gate = normal_bf16(rr, (N,))
    return Workload("ffdown_w8a8", to_bf16_bits(x), w, 8, 8, "row", "gated_residual",
                    residual=res, gate=gate)


def svdq_gateup(M: int = 4096, K: int = 5120, F: int = 20480, rank: int = 32,
                seeds=(6, 7, 8, 9)) -> Workload:
    """SVDQuant gate|up with SwiGLU: X [M x K] ~ N(0,1) (seed 6), W [2F x K]
    ~ N(0, 0.02) (seed 7; rows [0,F) gate, [F,2F) up), L1 [K x r] and
    L2 [r x 2F] ~ N(0, 0.02) (seeds 8, 9); group-64 int4 both sides."""
    x = normal_bf16(np.random.default_rng(seeds[0]), (M, K))
    w = normal_bf16(np.random.default_rng(seeds[1]), (2 * F, K), 0.02)
    l1 = normal_bf16(np.random.default_rng(seeds[2]), (K, rank), 0.02)
    l2 = normal_bf16(np.random.default_rng(seeds[3]), (rank, 2 * F), 0.02)
    return Workload("svdq_gateup", x, w, 4, 4, "group64", "swiglu", l1=l1, l2=l2)


# The 8 linears of one block of the 28-block stack at 2048^2 (16384 tokens):
# (name, N, K).  head_dim 128: 48 query heads -> 6144, 12 kv heads -> 1536.
STACK_BLOCK = (
    ("wq", 6144, 5120),
    ("wk", 1536, 5120),
    ("wv", 1536, 5120),
    ("attn_gate", 6144, 5120),
    ("wo", 5120, 6144),
    ("mlp_gate", 20480, 5120),
    ("mlp_up", 20480, 5120),
    ("mlp_down", 5120, 20480),
)
STACK_BLOCKS = 28


def stack_precision(block: int, name: str) -> int:
    """Weight/activation bit width of one stack linear (128 int4 + 96 int8):
    every wk and wv, every wo except block 0's, and mlp_down of blocks 15-27
    run W8A8; everything else W4A4."""
    if name in ("wk", "wv"):
        return 8
    if name == "wo":
        return 4 if block == 0 else 8
    if name == "mlp_down":
        return 8 if block >= 15 else 4
    return 4


def stack_layers():
    """All 224 (block, name, N, K, bits) entries of the mixed stack."""
    out = []
    for b in range(STACK_BLOCKS):
        for name, n, k in STACK_BLOCK:
            out.append((b, name, n, k, stack_precision(b, name)))
    return out


def stack_layer(index: int, M: int = 16384, rows: int | None = None) -> Workload:
    """Layer ``index`` (0..223) of the mixed stack: W ~ N(0, 0.02) seeded 2l,
    X ~ N(0, 1) seeded 2l+1, per-token / per-row scales, bf16 out.
    ``rows`` < M draws only the first rows of X (same values as the full draw)."""
    b, name, n, k, bits = stack_layers()[index]
    w = normal_bf16(np.random.default_rng(2 * index), (n, k), 0.02)
    m = M if rows is None else rows
    x = normal_bf16(np.random.default_rng(2 * index + 1), (m, k))
    return Workload(f"stack_b{b}_{name}", x, w, bits, bits, "row", "bf16")


# ---- inputs of the offline low-rank split ------------------------------------

def gaussian_sketch(K: int, cols: int, seed: int = 0) -> np.ndarray:
    """The randomized SVD's sketch: float32 [K, cols] ~ N(0, 1) (seed)."""
    return np.random.default_rng(seed).standard_normal(size=(K, cols), dtype=np.float32)


def spectral_weight_bf16(N: int, K: int, seed: int, rank: int, top: float = 0.5, decay: float = 0.93,
                         noise: float = 0.002) -> np.ndarray:
    """A weight with a decaying leading spectrum and a noise floor, as bf16
    bits [N, K]: W = U diag(s) V^T + noise * G with U [N, rank], V [K, rank]
    ~ N(0, 1/N), N(0, 1/K) (nearly orthonormal columns), s_j = top * decay^j,
    G ~ N(0, 1); drawn in the order U, V, G from one generator (seed)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(size=(N, rank), dtype=np.float32) / np.float32(np.sqrt(N))
    v = rng.standard_normal(size=(K, rank), dtype=np.float32) / np.float32(np.sqrt(K))
    g = rng.standard_normal(size=(N, K), dtype=np.float32)
    s = (top * decay ** np.arange(rank)).astype(np.float32)
    return to_bf16_bits((u * s[None, :]) @ v.T + np.float32(noise) * g)


def act_rms(K: int, seed: int, outlier_frac: float = 0.01, factor: float = 30.0) -> np.ndarray:
    """Synthetic per-input-channel activation RMS, float32 [K]: log-normal
    exp(N(0, 0.5^2)) with floor(outlier_frac * K) channels (drawn without
    replacement after the values) multiplied by `factor`."""
    rng = np.random.default_rng(seed)
    r = np.exp(0.5 * rng.standard_normal(size=K, dtype=np.float32)).astype(np.float32)
    n = int(outlier_frac * K)
    if n:
        r[rng.choice(K, n, replace=False)] *= np.float32(factor)
    return r
