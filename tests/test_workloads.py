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


def test_split_inputs_are_deterministic_and_shaped():
    om = W.gaussian_sketch(512, 40, 7)
    assert om.dtype == np.float32 and om.shape == (512, 40)
    assert np.array_equal(om, W.gaussian_sketch(512, 40, 7)) and not np.array_equal(om, W.gaussian_sketch(512, 40, 8))
    rms = W.act_rms(1000, 3)
    assert rms.dtype == np.float32 and rms.shape == (1000,) and (rms > 0).all()
    # 1 % of the channels (10) x30 on a log-normal base: they stand well above the median
    assert np.sort(rms)[-10:].min() > 5 * np.median(rms)
    w = W.spectral_weight_bf16(128, 256, 4, 8, top=1.0, decay=0.5, noise=1e-3)
    assert w.dtype == np.uint16 and w.shape == (128, 256)
    s = np.linalg.svd((w.astype(np.uint32) << 16).view(np.float32).astype(np.float64), compute_uv=False)
    assert s[0] > 0.5 and s[8] < 0.1 * s[0]          # a decaying leading spectrum above the noise floor
