"""Properties of the seeded input generators (no method arithmetic here)."""

import numpy as np

import workloads as W


def test_tiny_is_deterministic_and_shaped():
    a = W.tiny_w4a4(0)
    b = W.tiny_w4a4(0)
    assert a.x.dtype == np.uint16 and a.x.shape == (64, 256) and a.w.shape == (256, 256)
    assert (a.x == b.x).all() and (a.w == b.w).all()
    assert not (W.tiny_w4a4(1).x == a.x).all()
    assert len(a.outlier_channels) == 4 and len(set(a.outlier_channels.tolist())) == 4


def test_outlier_channels_are_scaled():
    wl = W.tiny_w4a4(0)
    x = (wl.x.astype(np.uint32) << 16).view(np.float32)
    rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=0))
    out = set(wl.outlier_channels.tolist())
    assert all(rms[c] > 10 for c in out)
    assert all(rms[c] < 2 for c in range(256) if c not in out)


def test_row_prefix_draw_matches_full_draw():
    full = W.normal_bf16(np.random.default_rng(3), (64, 256))
    part = W.normal_bf16(np.random.default_rng(3), (16, 256))
    assert (full[:16] == part).all()


def test_stack_recipe_counts():
    layers = W.stack_layers()
    assert len(layers) == 224
    bits = [b for *_, b in layers]
    assert bits.count(4) == 128 and bits.count(8) == 96
    names8 = {(blk, n) for blk, n, _, _, b in layers if b == 8}
    assert all((blk, "wk") in names8 and (blk, "wv") in names8 for blk in range(28))
    assert sum(1 for blk, n in names8 if n == "wo") == 27
