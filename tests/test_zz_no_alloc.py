"""The allocation-free split entry point (svdq_split_noalloc) against the
entry point with a caller workspace (svdq_split), through the C ABI.

The split is deterministic on a device (no atomics, fixed-order reductions),
and both entry points run the same kernels, so every output must be equal
bit for bit.  Two calls in a row use the library's one array, the second on
a smaller weight: nothing from the first call may leak into it.  The call
itself must not allocate: with the outputs passed in, torch's allocator sees
no allocation across it."""

import numpy as np
import pytest

import workloads as W
from tests.helpers import ensure_built, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import torch

    ensure_built()
    import rotated_bit_quantized_rotate_amd as Q

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert Q.device_supported(0), "device is not gfx950"
    return Q


def _inputs(N, K, r, over, seed, weighted):
    rng = np.random.default_rng(seed)
    wb = W.normal_bf16(rng, (N, K), 0.02)
    om = W.gaussian_sketch(K, r + over, seed + 1)
    rms = W.act_rms(K, seed + 2) if weighted else None
    return to_dev_bf16(wb), to_dev(om), None if rms is None else to_dev(rms)


def _same(a, b):
    import torch

    assert a.keys() == b.keys()
    for k in a:
        x, y = a[k], b[k]
        assert x.shape == y.shape, k
        if x.dtype.is_floating_point:
            x = x.view(torch.int16 if x.element_size() == 2 else torch.int32)
            y = y.view(torch.int16 if y.element_size() == 2 else torch.int32)
        assert torch.equal(x, y), k


def test_noalloc_equals_workspace_entry_on_two_calls(Q):
    import torch

    # the larger problem first (2048 x 5120 fills most of the 128 MiB array),
    # then a smaller one with other modes on the same array
    cases = [(2048, 5120, 32, 8, 2, 1, "group64", True), (512, 1024, 16, 8, 1, 2, "row", False)]
    for i, (N, K, r, over, pi, ri, mode, weighted) in enumerate(cases):
        print(f"case {i}: N={N} K={K} rank={r} mode={mode}", flush=True)
        w, om, rms = _inputs(N, K, r, over, 50 + i, weighted)
        ref = Q.svdq_split(w, om, r, over, pi, ri, mode, act_rms=rms)
        torch.cuda.synchronize()
        out = {k: torch.full_like(v, 0x7F if v.dtype == torch.uint8 else 3) for k, v in ref.items()}
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        got = Q.svdq_split_noalloc(w, om, r, over, pi, ri, mode, act_rms=rms, out=out)
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == before
        assert got is out
        _same(got, ref)
        e = got["errors"].cpu().numpy()
        assert np.all(np.isfinite(e)) and int(got["best_iter"].cpu().numpy()[0]) == int(np.argmin(e))


def test_noalloc_rejects_a_problem_beyond_its_array(Q):
    import torch

    N, K, r, over = 2560, 5120, 32, 8
    assert Q.svdq_split_workspace_bytes(N, K, r, over, "group64") > Q.svdq_split_noalloc_max_bytes()
    w = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    om = torch.zeros((K, r + over), dtype=torch.float32, device="cuda")
    with pytest.raises(Q.QLinearError) as e:
        Q.svdq_split_noalloc(w, om, r, over, 1, 0, "group64")
    assert e.value.status == -7
