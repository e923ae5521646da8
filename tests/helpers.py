"""Shared helpers for the test suite (marshalling between numpy and torch)."""

import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlinear.h")


def ensure_built():
    """Build libqlinear.so in-tree if it is not there yet; return its path."""
    from rotated_bit_quantized_rotate_amd import build as B

    if not os.path.exists(B.LIB_PATH):
        B.build()
    return B.LIB_PATH


def header_functions():
    """Names of the functions include/qlinear.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", txt, flags=re.M)))


def header_constants():
    txt = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"\b(QL_[A-Z0-9_]+)\s*=\s*(-?\d+)", txt)}


def to_dev_bf16(bits, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def pair_w4(packed):
    """Row-major packed int4 weights [N, K/2] -> the library's weight order:
    rows 2p and 2p + 1 interleaved per 128-channel slice (64 bytes each)."""
    p = np.asarray(packed)
    n, h = p.shape
    return np.ascontiguousarray(p.reshape(n // 2, 2, h // 64, 64).transpose(0, 2, 1, 3).reshape(n, h))


def unpair_w4(packed):
    """The library's packed weight order -> row-major [N, K/2]."""
    p = np.asarray(packed)
    n, h = p.shape
    return np.ascontiguousarray(p.reshape(n // 2, h // 64, 2, 64).transpose(0, 2, 1, 3).reshape(n, h))


def quad_fp6(codes):
    """Row-major FP6 codes [R, 3K/4] -> the library's FP6 row order: rows
    4q .. 4q + 3 interleaved per 128-channel block (96 bytes each) for every
    whole four of rows; the last R % 4 rows stay plain."""
    p = np.ascontiguousarray(np.asarray(codes))
    n, h = p.shape
    n4 = n // 4 * 4
    out = p.copy()
    out[:n4] = p[:n4].reshape(n4 // 4, 4, h // 96, 96).transpose(0, 2, 1, 3).reshape(n4, h)
    return out


def unquad_fp6(codes):
    """Inverse of quad_fp6."""
    p = np.ascontiguousarray(np.asarray(codes))
    n, h = p.shape
    n4 = n // 4 * 4
    out = p.copy()
    out[:n4] = p[:n4].reshape(n4 // 4, h // 96, 4, 96).transpose(0, 2, 1, 3).reshape(n4, h)
    return out


def to_dev_l2(l2_bits, device="cuda"):
    """The low-rank GEMMs take L2 transposed: bf16 [N, rank] from the
    oracle's [rank, N] bits."""
    return to_dev_bf16(np.ascontiguousarray(np.asarray(l2_bits).T), device)


def bf16_bits(t):
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev(a, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_dev_scales(s, device="cuda"):
    """Scales on the device in the library's layout: tensor / row scales as
    they are; group-64 scales [R, K/64] as the transposed view of group-major
    memory ([K/64, R] contiguous)."""
    s = np.asarray(s, np.float32)
    if s.ndim == 2:
        return to_dev(s.T, device).t()
    return to_dev(s, device)


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def f32_ulp_diff(a, b):
    """|ulp distance| between float32 arrays (same sign assumed for nonzeros)."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


def bf16_ulp_diff(a_bits, b_bits):
    def key(x):
        x = np.asarray(x, np.uint16).astype(np.int64)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(key(a_bits) - key(b_bits))


def code_flip_stats(got, want):
    """(fraction of differing codes, max |difference|)."""
    d = np.abs(got.astype(np.int32) - want.astype(np.int32))
    return float((d != 0).mean()) if d.size else 0.0, int(d.max()) if d.size else 0
