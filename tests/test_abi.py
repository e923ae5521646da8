"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, its constants match the binding, and argument
validation rejects bad calls before touching a device."""

import ctypes

import numpy as np
import pytest

from tests.helpers import ensure_built, header_constants, header_functions


@pytest.fixture(scope="module")
def L():
    ensure_built()
    from rotated_bit_quantized_rotate_amd import _lib

    return _lib.lib()


def test_header_declares_the_entry_points():
    fns = header_functions()
    for name in ["rotate_quantize_act", "rmsnorm_rotate_quantize_act", "pack_weight_int4", "pack_weight_fp6",
                 "qgemm_w4a4", "qgemm_w4a4_fp6", "qgemm_w8a8", "qgemm_w4a4_lowrank", "qgemm_w4a4_fp6_lowrank",
                 "qgemm_grouped",
                 "svdq_split", "svdq_split_workspace_bytes", "svdq_split_noalloc", "svdq_split_noalloc_max_bytes",
                 "rotate_quantize_mx", "qgemm_mx", "qgemm_mx_lowrank",
                 "ql_status_string", "ql_device_supported"]:
        assert name in fns


def test_library_exports_every_declared_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), name


def test_binding_constants_match_header():
    from rotated_bit_quantized_rotate_amd import _lib

    consts = header_constants()
    assert consts
    for k, v in consts.items():
        assert getattr(_lib, k) == v, k


def test_status_strings(L):
    from rotated_bit_quantized_rotate_amd import _lib

    for k, v in header_constants().items():
        if k.startswith("QL_ERR") or k == "QL_OK":
            s = _lib.status_string(v)
            assert s.startswith(k), (k, s)
    assert "unknown" in _lib.status_string(-99)


NULL = None
ALIGNED = ctypes.c_void_p(0x10000)     # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def rq(L, **kw):
    a = dict(x=ALIGNED, M=4, K=256, ldx=256, bits=4, mode=1, layout=0, rotate=1, codes=ALIGNED,
             scales=ALIGNED, l1=NULL, rank=0, lr=NULL)
    a.update(kw)
    return L.rotate_quantize_act(a["x"], a["M"], a["K"], a["ldx"], a["bits"], a["mode"], a["layout"],
                                 a["rotate"], a["codes"], a["scales"], a["l1"], a["rank"], a["lr"], None)


def test_rotate_quantize_validation(L):
    assert rq(L, bits=5) == -4
    assert rq(L, mode=7) == -4
    assert rq(L, layout=1, bits=8) == -4          # packed layout is int4-only
    assert rq(L, layout=2, bits=8) == -4          # so is the FP6 layout
    assert rq(L, layout=3) == -4
    assert rq(L, rotate=2) == -4
    assert rq(L, K=320, ldx=320) == -2            # K % 256
    assert rq(L, K=0, ldx=0) == -2
    assert rq(L, ldx=128) == -2                   # ldx < K
    assert rq(L, ldx=260) == -2                   # ldx % 8
    assert rq(L, M=-1) == -2
    assert rq(L, x=NULL) == -1
    assert rq(L, codes=NULL) == -1
    assert rq(L, scales=NULL) == -1
    assert rq(L, x=MISALIGNED) == -3
    assert rq(L, rank=32) == -2                   # rank without l1
    assert rq(L, l1=ALIGNED, rank=24, lr=ALIGNED) == -2
    assert rq(L, l1=ALIGNED, rank=32, lr=NULL) == -1



def rqn(L, **kw):
    a = dict(x=ALIGNED, M=4, K=256, ldx=256, g=NULL, s=NULL, t=NULL, eps=1e-6, bits=4, mode=1, layout=0,
             rotate=1, codes=ALIGNED, scales=ALIGNED)
    a.update(kw)
    return L.rmsnorm_rotate_quantize_act(a["x"], a["M"], a["K"], a["ldx"], a["g"], a["s"], a["t"], a["eps"],
                                         a["bits"], a["mode"], a["layout"], a["rotate"], a["codes"],
                                         a["scales"], None)


def test_rmsnorm_rotate_quantize_validation(L):
    # the checks of rotate_quantize_act ...
    assert rqn(L, bits=5) == -4
    assert rqn(L, layout=1, bits=8) == -4
    assert rqn(L, K=320, ldx=320) == -2
    assert rqn(L, ldx=260) == -2
    assert rqn(L, x=NULL) == -1
    assert rqn(L, x=MISALIGNED) == -3
    # ... plus its own: K fits the on-chip vectors, eps positive and finite, vectors 16-byte aligned
    assert rqn(L, K=8448, ldx=8448) == -2
    assert rqn(L, eps=0.0) == -2
    assert rqn(L, eps=-1.0) == -2
    assert rqn(L, eps=float("inf")) == -2
    assert rqn(L, eps=float("nan")) == -2
    assert rqn(L, g=MISALIGNED) == -3
    assert rqn(L, s=MISALIGNED) == -3
    assert rqn(L, t=MISALIGNED) == -3
    # a valid call gets past validation to the device check (no gfx950 here)
    assert rqn(L, g=ALIGNED, s=ALIGNED, t=ALIGNED, K=8192, ldx=8192) in (-4, -6)

def g44(L, **kw):
    a = dict(a=ALIGNED, sa=ALIGNED, am=1, al=0, w=ALIGNED, sw=ALIGNED, wm=1, M=4, N=32, K=256, bias=NULL,
             epi=0, out=ALIGNED, ldo=32)
    a.update(kw)
    return L.qgemm_w4a4(a["a"], a["sa"], a["am"], a["al"], a["w"], a["sw"], a["wm"], a["M"], a["N"], a["K"],
                        a["bias"], a["epi"], a["out"], a["ldo"], None)


def test_qgemm_w4a4_validation(L):
    assert g44(L, N=24) == -2                     # N % 16
    assert g44(L, K=128) == -2
    assert g44(L, ldo=16) == -2
    assert g44(L, ldo=36) == -3                   # bf16 row stride not 16-byte aligned
    assert g44(L, epi=1) == -4                    # SWIGLU goes through the low-rank entry
    assert g44(L, epi=2) == -4
    assert g44(L, am=2) == -4                     # group64 only on both sides
    assert g44(L, al=3) == -4
    assert g44(L, a=NULL) == -1
    assert g44(L, sw=NULL) == -1
    assert g44(L, w=MISALIGNED) == -3
    assert g44(L, am=2, wm=2, epi=4) == -4        # exact int32 output needs one scale per product
    # the layout and epilogue are checked before the group-64 scales forward
    # to the low-rank GEMM: FP6 operands never reach the int4 kernels here
    assert g44(L, am=2, wm=2, al=2) == -4
    assert g44(L, am=2, wm=2, epi=1) == -4        # no SwiGLU through this entry
    assert g44(L, am=2, wm=2, epi=5) == -4        # nor the sigmoid with group-64 scales
    assert g44(L, am=2, wm=2) in (-4, -6)
    # int32 accumulator overflow: K * max |product| must stay below 2^31
    assert g44(L, K=2738944) in (-4, -6)          # int8-container codes: 7 * 112 * K
    assert g44(L, K=2739200) == -2
    assert g44(L, al=1, K=171008) in (-4, -6)     # packed activations: 112 * 112 * K
    assert g44(L, al=1, K=171264) == -2
    # size limits of the 32-bit operand offsets
    assert g44(L, K=1 << 23, ldo=32) == -2
    assert g44(L, N=1 << 20, K=1 << 11, ldo=1 << 20) == -2   # N * K = 2^31
    assert g44(L, M=1 << 25, K=1 << 11) == -2                # M * K = 2^36


def g88(L, **kw):
    a = dict(a=ALIGNED, sa=ALIGNED, am=1, w=ALIGNED, sw=ALIGNED, wm=1, M=4, N=32, K=256, bias=NULL,
             res=NULL, gate=NULL, epi=0, out=ALIGNED, ldo=32)
    a.update(kw)
    return L.qgemm_w8a8(a["a"], a["sa"], a["am"], a["w"], a["sw"], a["wm"], a["M"], a["N"], a["K"],
                        a["bias"], a["res"], a["gate"], a["epi"], a["out"], a["ldo"], None)


def test_qgemm_w8a8_validation(L):
    assert g88(L, epi=2) == -1                    # gated residual needs residual and gate
    assert g88(L, epi=2, res=ALIGNED) == -1
    assert g88(L, am=2) == -4
    assert g88(L, epi=1) == -4
    assert g88(L, N=0) == -2
    assert g88(L, epi=2, res=MISALIGNED, gate=ALIGNED) == -3
    assert g88(L, K=133120) in (-4, -6)           # 127 * 127 * K < 2^31
    assert g88(L, K=133376) == -2


def glr(L, **kw):
    a = dict(a=ALIGNED, sa=ALIGNED, am=2, al=0, w=ALIGNED, sw=ALIGNED, wm=2, lr=ALIGNED, l2=ALIGNED, r=32,
             M=4, N=64, K=256, bias=NULL, epi=1, out=ALIGNED, ldo=32)
    a.update(kw)
    return L.qgemm_w4a4_lowrank(a["a"], a["sa"], a["am"], a["al"], a["w"], a["sw"], a["wm"], a["lr"],
                                a["l2"], a["r"], a["M"], a["N"], a["K"], a["bias"], a["epi"], a["out"],
                                a["ldo"], None)


def test_qgemm_lowrank_validation(L):
    assert glr(L, r=20) == -2
    assert glr(L, r=256) == -2
    assert glr(L, lr=NULL) == -1
    assert glr(L, N=48) == -2                     # SWIGLU needs N % 32
    assert glr(L, ldo=16) == -2                   # out needs N/2 columns
    assert glr(L, am=1) == -4                     # group64 on one side only
    assert glr(L, epi=4) == -4
    assert glr(L, epi=2) == -4
    assert glr(L, al=3) == -4                     # no such layout
    assert glr(L, al=2, am=1, wm=1) == -4         # no FP6 operands here ...
    assert glr(L, al=2) == -4                     # ... with any scales (qgemm_w4a4_fp6_lowrank has them)
    assert glr(L) in (-4, -6)
    # row scales keep one int32 accumulator: the overflow bound applies
    assert glr(L, am=1, wm=1, K=2738944, N=64) in (-4, -6)
    assert glr(L, am=1, wm=1, K=2739200) == -2
    assert glr(L, K=2739200) in (-4, -6)          # group-64 partials cannot overflow


def g6lr(L, **kw):
    a = dict(a=ALIGNED, sa=ALIGNED, w=ALIGNED, sw=ALIGNED, lr=ALIGNED, l2=ALIGNED, r=32, M=4, N=64, K=256,
             bias=NULL, epi=1, out=ALIGNED, ldo=32)
    a.update(kw)
    return L.qgemm_w4a4_fp6_lowrank(a["a"], a["sa"], a["w"], a["sw"], a["lr"], a["l2"], a["r"], a["M"], a["N"],
                                    a["K"], a["bias"], a["epi"], a["out"], a["ldo"], None)


def test_qgemm_fp6_lowrank_validation(L):
    assert g6lr(L, r=20) == -2
    assert g6lr(L, lr=NULL) == -1
    assert g6lr(L, N=48) == -2                    # SWIGLU needs N % 32
    assert g6lr(L, epi=4) == -4                   # group sums are rescaled: no I32
    assert g6lr(L, epi=5) == -4
    assert g6lr(L, epi=2) == -4
    assert g6lr(L, a=MISALIGNED) == -3
    for epi in (0, 1, 3):
        assert g6lr(L, epi=epi, ldo=64) in (-4, -6)
    assert g6lr(L, r=0, lr=NULL, l2=NULL) in (-4, -6)


def grp(L, segs, **kw):
    from rotated_bit_quantized_rotate_amd import _lib

    a = dict(a4=ALIGNED, sa4=ALIGNED, a8=ALIGNED, sa8=ALIGNED, M=4, K=256, nseg=None)
    a.update(kw)
    arr = (_lib.Segment * max(len(segs), 1))()
    for i, sg in enumerate(segs):
        d = dict(w=ALIGNED, sw=ALIGNED, n=32, w_bits=4, epilogue=0, out=ALIGNED, ldo=32)
        d.update(sg)
        arr[i] = _lib.Segment(*(d[k] if not isinstance(d[k], ctypes.c_void_p) else d[k].value
                                for k in ("w", "sw", "n", "w_bits", "epilogue", "out", "ldo")))
    nseg = len(segs) if a["nseg"] is None else a["nseg"]
    return L.qgemm_grouped(a["a4"], a["sa4"], a["a8"], a["sa8"], a["M"], a["K"], arr, nseg, None)


def test_qgemm_grouped_validation(L):
    assert L.qgemm_grouped(ALIGNED, ALIGNED, NULL, NULL, 4, 256, None, 1, None) == -1   # no segment array
    assert grp(L, [{}], nseg=0) == -2
    assert grp(L, [{}] * 9) == -2                                  # more than QL_MAX_SEGMENTS
    assert grp(L, [{}], K=320) == -2                               # K % 256
    assert grp(L, [{"n": 24, "ldo": 24}]) == -2                    # n % 16
    assert grp(L, [{"ldo": 16}]) == -2                             # ldo < n
    assert grp(L, [{"w_bits": 6}]) == -4
    assert grp(L, [{"epilogue": 2}]) == -4                         # only bf16 / sigmoid
    assert grp(L, [{"w": NULL}]) == -1
    assert grp(L, [{"out": NULL}]) == -1
    assert grp(L, [{"w": MISALIGNED}]) == -3
    assert grp(L, [{"ldo": 36, "n": 32}]) == -3                    # rows not 16-byte aligned
    assert grp(L, [{"w_bits": 8}], a8=NULL) == -1                  # int8 segment without int8 codes
    assert grp(L, [{"w_bits": 4}], a4=NULL, sa4=NULL) == -1
    assert grp(L, [{"w_bits": 4}], a8=NULL, sa8=NULL) in (-4, -6)  # unused operand may be NULL
    assert grp(L, [{}, {"w_bits": 8, "epilogue": 5}, {"n": 48, "ldo": 48}]) in (-4, -6)
    assert grp(L, [{}], M=0) in (0, -4, -6)
    assert grp(L, [{"w_bits": 8}], K=133376) == -2                 # int8 segment: 127 * 127 * K < 2^31
    assert grp(L, [{"w_bits": 8, "n": 16, "ldo": 16}], K=133120) in (-4, -6)

def g6(L, **kw):
    a = dict(a=ALIGNED, sa=ALIGNED, am=1, w=ALIGNED, sw=ALIGNED, wm=1, M=4, N=32, K=256, bias=NULL,
             epi=0, out=ALIGNED, ldo=32)
    a.update(kw)
    return L.qgemm_w4a4_fp6(a["a"], a["sa"], a["am"], a["w"], a["sw"], a["wm"], a["M"], a["N"], a["K"],
                            a["bias"], a["epi"], a["out"], a["ldo"], None)


def test_qgemm_w4a4_fp6_validation(L):
    assert g6(L, am=2) == -4                      # group-64 scales only on both sides
    assert g6(L, wm=2) == -4
    assert g6(L, am=2, wm=2, epi=4) == -4         # group sums are rescaled: no exact I32 result
    assert g6(L, am=2, wm=2, epi=5) == -4
    assert g6(L, am=2, wm=2, K=342528) in (-4, -6)  # group partials are exact at any K
    for epi in (0, 3):
        assert g6(L, am=2, wm=2, epi=epi) in (-4, -6)
    assert g6(L, epi=1) == -4                     # no SwiGLU / gated residual here
    assert g6(L, epi=2) == -4
    assert g6(L, N=24) == -2
    assert g6(L, K=384) == -2                     # K % 256
    assert g6(L, ldo=16) == -2
    assert g6(L, a=NULL) == -1
    assert g6(L, w=MISALIGNED) == -3
    assert g6(L, ldo=36) == -3
    # float32 sums of code products stay exact only while 49 K < 2^24
    assert g6(L, K=342528) == -2
    assert g6(L, K=342272) in (-4, -6)            # largest valid K reaches the device check
    assert g6(L, M=0) in (0, -4, -6)
    for epi in (0, 3, 4, 5):
        assert g6(L, epi=epi) in (-4, -6)


def test_pack_weight_int4_validation(L):
    """Packed INT4 weights are stored in row pairs (rows 2p, 2p + 1 per
    128-channel slice), so an odd row count is a shape error."""
    def pw(**kw):
        a = dict(w=ALIGNED, N=16, K=256, ldw=256, mode=1, rot=1, out=ALIGNED, sc=ALIGNED)
        a.update(kw)
        return L.pack_weight_int4(a["w"], a["N"], a["K"], a["ldw"], a["mode"], a["rot"], a["out"], a["sc"], None)

    assert pw(N=15) == -2
    assert pw(N=0) == -2
    assert pw(mode=3) == -4
    assert pw(K=320, ldw=320) == -2
    assert pw(out=NULL) == -1
    assert pw(w=MISALIGNED) == -3
    assert pw(N=2) in (-4, -6)                    # one row pair reaches the device check
    assert pw() in (-4, -6)


def test_pack_weight_fp6_validation(L):
    def pw(**kw):
        a = dict(w=ALIGNED, N=16, K=256, ldw=256, mode=1, rot=1, out=ALIGNED, sc=ALIGNED)
        a.update(kw)
        return L.pack_weight_fp6(a["w"], a["N"], a["K"], a["ldw"], a["mode"], a["rot"], a["out"], a["sc"], None)

    assert pw(mode=3) == -4                       # no such scale mode
    assert pw(mode=2) in (-4, -6)                 # group-64 passes validation (no device here)
    assert pw(N=0) == -2
    assert pw(N=18) in (-4, -6)                   # any row count: full fours interleaved, the rest plain
    assert pw(K=320, ldw=320) == -2
    assert pw(out=NULL) == -1
    assert pw(w=MISALIGNED) == -3
    assert pw() in (-4, -6)


@pytest.mark.parametrize("rows", [8, 11, 3, 0])
def test_fp6_row_order_round_trips(rows):
    from tests.helpers import quad_fp6, unquad_fp6

    rng = np.random.default_rng(3)
    p = rng.integers(0, 256, size=(rows, 3 * 96), dtype=np.uint8)
    q = quad_fp6(p)
    assert q.shape == p.shape
    # row 4q + j < 4 floor(rows / 4): block s at 4q * 288 + 384 s + 96 j of
    # the flat buffer; the last rows % 4 rows plain at r * 288 + 96 s
    flat = q.reshape(-1)
    for r in range(rows):
        for blk in range(3):
            if r < rows // 4 * 4:
                off = (r // 4) * 4 * 288 + 384 * blk + 96 * (r % 4)
            else:
                off = r * 288 + 96 * blk
            assert np.array_equal(flat[off:off + 96], p[r, 96 * blk:96 * blk + 96])
    assert np.array_equal(unquad_fp6(q), p)


def test_rotate_quantize_mx_validation(L):
    def mq(**kw):
        a = dict(x=ALIGNED, M=4, K=256, ldx=256, fmt=4, rot=1, codes=ALIGNED, sc=ALIGNED, l1=NULL, rank=0, lr=NULL)
        a.update(kw)
        return L.rotate_quantize_mx(a["x"], a["M"], a["K"], a["ldx"], a["fmt"], a["rot"], a["codes"], a["sc"],
                                    a["l1"], a["rank"], a["lr"], None)

    assert mq(fmt=6) == -4                        # FP4 or FP8 elements only
    assert mq(rot=2) == -4
    assert mq(K=384, ldx=384) == -2               # K % 256
    assert mq(K=0) == -2
    assert mq(M=-1) == -2
    assert mq(ldx=248) == -2                      # ldx >= K
    assert mq(ldx=260) == -2                      # ldx % 8
    assert mq(x=NULL) == -1
    assert mq(sc=NULL) == -1
    assert mq(codes=MISALIGNED) == -3
    assert mq(x=MISALIGNED) == -3
    assert mq(sc=ctypes.c_void_p(0x10001)) == -3  # a row's 4 slice scales leave as one dword
    assert mq(M=0, x=NULL, codes=NULL, sc=NULL) in (0, -4, -6)
    assert mq(rank=16) == -2                      # rank without l1
    assert mq(l1=ALIGNED, rank=8, lr=ALIGNED) == -2
    assert mq(l1=ALIGNED, rank=144, lr=ALIGNED) == -2
    assert mq(l1=ALIGNED, rank=32, lr=NULL) == -1
    assert mq(l1=MISALIGNED, rank=32, lr=ALIGNED) == -3
    assert mq(l1=ALIGNED, rank=32, lr=ALIGNED) in (-4, -6)
    for fmt in (4, 8):
        for rot in (0, 1):
            assert mq(fmt=fmt, rot=rot) in (-4, -6)


def test_qgemm_mx_validation(L):
    def gm(**kw):
        a = dict(a=ALIGNED, sa=ALIGNED, w=ALIGNED, sw=ALIGNED, fmt=4, M=16, N=32, K=256, bias=NULL, res=NULL,
                 gate=NULL, epi=0, out=ALIGNED, ldo=32)
        a.update(kw)
        return L.qgemm_mx(a["a"], a["sa"], a["w"], a["sw"], a["fmt"], a["M"], a["N"], a["K"], a["bias"], a["res"],
                          a["gate"], a["epi"], a["out"], a["ldo"], None)

    assert gm(fmt=0) == -4
    assert gm(epi=4) == -4                        # no exact integer result: the sums are float32
    assert gm(epi=9) == -4
    assert gm(N=24) == -2
    assert gm(K=384) == -2
    assert gm(epi=1, N=48) == -2                  # SwiGLU pairs 16-row gate / up fragments: N % 32
    assert gm(ldo=16) == -2
    assert gm(a=NULL) == -1
    assert gm(sw=NULL) == -1
    assert gm(sa=ctypes.c_void_p(0x10002)) == -3  # a row's 4 stage scales move as one dword
    assert gm(w=MISALIGNED) == -3
    assert gm(epi=2) == -1                        # gated residual needs residual and gate
    assert gm(epi=2, res=ALIGNED, gate=ALIGNED) in (-4, -6)
    assert gm(epi=2, res=MISALIGNED, gate=ALIGNED) == -3
    assert gm(K=1 << 23) == -2                    # 32-bit operand offsets
    assert gm(M=0) in (0, -4, -6)
    for fmt in (4, 8):
        for epi in (0, 1, 3, 5):
            assert gm(fmt=fmt, epi=epi) in (-4, -6)


def test_qgemm_mx_lowrank_validation(L):
    def gl(**kw):
        a = dict(a=ALIGNED, sa=ALIGNED, w=ALIGNED, sw=ALIGNED, fmt=4, lr=ALIGNED, l2=ALIGNED, rank=32, M=16, N=64,
                 K=256, bias=NULL, epi=1, out=ALIGNED, ldo=32)
        a.update(kw)
        return L.qgemm_mx_lowrank(a["a"], a["sa"], a["w"], a["sw"], a["fmt"], a["lr"], a["l2"], a["rank"], a["M"],
                                  a["N"], a["K"], a["bias"], a["epi"], a["out"], a["ldo"], None)

    assert gl(fmt=6) == -4
    assert gl(epi=2) == -4                        # bf16 | f32 | swiglu only
    assert gl(epi=5) == -4
    assert gl(epi=4) == -4
    assert gl(N=48) == -2                         # SwiGLU: N % 32
    assert gl(rank=8) == -2
    assert gl(rank=144) == -2
    assert gl(lr=NULL) == -1
    assert gl(l2=NULL) == -1
    assert gl(l2=MISALIGNED) == -3
    assert gl(rank=0, lr=NULL, l2=NULL) in (-4, -6)  # no branch: the pointers may be NULL
    assert gl(K=384) == -2
    assert gl(ldo=16) == -2                       # SwiGLU writes N/2 columns
    for fmt in (4, 8):
        for epi in (0, 1, 3):
            assert gl(fmt=fmt, epi=epi, ldo=64) in (-4, -6)


def test_svdq_split_workspace_bytes(L):
    n1 = L.svdq_split_workspace_bytes(512, 1024, 32, 8, 2)
    assert n1 >= int(10.5 * 512 * 1024)
    assert L.svdq_split_workspace_bytes(1024, 1024, 32, 8, 2) > n1
    assert L.svdq_split_workspace_bytes(512, 1000, 32, 8, 2) == -1      # K % 256
    assert L.svdq_split_workspace_bytes(512, 1024, 32, 8, 7) == -1      # scale mode


def sp(L, **kw):
    a = dict(w=ALIGNED, N=512, K=1024, ldw=1024, rms=NULL, om=ALIGNED, rank=32, over=8, pi=2, ri=1, mode=2,
             l1=ALIGNED, l2=ALIGNED, packed=ALIGNED, scales=ALIGNED, errors=ALIGNED, best=ALIGNED, sigma=NULL,
             ws=ALIGNED, wsb=1 << 40)
    a.update(kw)
    return L.svdq_split(a["w"], a["N"], a["K"], a["ldw"], a["rms"], a["om"], a["rank"], a["over"], a["pi"], a["ri"],
                        a["mode"], a["l1"], a["l2"], a["packed"], a["scales"], a["errors"], a["best"], a["sigma"],
                        a["ws"], a["wsb"], None)


def test_svdq_split_validation(L):
    assert sp(L, mode=5) == -4
    assert sp(L, N=500) == -2                     # N % 16
    assert sp(L, K=1000, ldw=1000) == -2
    assert sp(L, ldw=1020) == -2
    assert sp(L, rank=24) == -2
    assert sp(L, rank=144) == -2
    assert sp(L, over=33) == -2
    assert sp(L, N=32, rank=32, over=8) == -2     # rank + oversample > N
    assert sp(L, pi=9) == -2
    assert sp(L, ri=17) == -2
    assert sp(L, wsb=1024) == -2                  # workspace too small
    assert sp(L, w=NULL) == -1
    assert sp(L, om=NULL) == -1
    assert sp(L, ws=NULL) == -1
    assert sp(L, l1=MISALIGNED) == -3
    assert sp(L, sigma=MISALIGNED) == -3
    assert sp(L) in (-4, -6)                      # valid: reaches the device check
    assert sp(L, rms=ALIGNED, sigma=ALIGNED, mode=0, pi=0, ri=0, over=0) in (-4, -6)


def spn(L, **kw):
    a = dict(w=ALIGNED, N=512, K=1024, ldw=1024, rms=NULL, om=ALIGNED, rank=32, over=8, pi=2, ri=1, mode=2,
             l1=ALIGNED, l2=ALIGNED, packed=ALIGNED, scales=ALIGNED, errors=ALIGNED, best=ALIGNED, sigma=NULL)
    a.update(kw)
    return L.svdq_split_noalloc(a["w"], a["N"], a["K"], a["ldw"], a["rms"], a["om"], a["rank"], a["over"], a["pi"],
                                a["ri"], a["mode"], a["l1"], a["l2"], a["packed"], a["scales"], a["errors"], a["best"],
                                a["sigma"], None)


def test_svdq_split_noalloc_validation(L):
    cap = L.svdq_split_noalloc_max_bytes()
    assert cap == 128 << 20
    # the same argument checks as svdq_split
    assert spn(L, mode=5) == -4
    assert spn(L, N=500) == -2
    assert spn(L, rank=24) == -2
    assert spn(L, w=NULL) == -1
    assert spn(L, l1=MISALIGNED) == -3
    # problems whose workspace exceeds the fixed array are refused before any launch
    assert L.svdq_split_workspace_bytes(2048, 5120, 32, 8, 2) <= cap < L.svdq_split_workspace_bytes(2560, 5120, 32, 8, 2)
    assert spn(L, N=2560, K=5120, ldw=5120) == -7
    assert spn(L, N=40960, K=5120, ldw=5120) == -7
    assert spn(L, N=2048, K=5120, ldw=5120) in (-4, -6)   # fits: reaches the device check
    assert spn(L) in (-4, -6)


def test_device_supported_without_gpu_is_false(L):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.ql_device_supported(0) == 0


def test_group64_scales_are_group_major_views():
    """The binding hands out and accepts group-64 scales as [R, K/64] views of
    group-major memory ([K/64, R] contiguous: the layout the kernels read);
    other layouts are refused before any call."""
    import torch

    from rotated_bit_quantized_rotate_amd import _lib as B

    R, K = 6, 512
    s = B._new_scales(R, K, B.QL_SCALE_GROUP64, "cpu")
    assert tuple(s.shape) == (R, K // 64) and s.stride() == (1, R)
    assert B._sptr(s, R, K, "group64", "s").value == s.data_ptr()
    plain = torch.arange(R * (K // 64), dtype=torch.float32).reshape(R, K // 64)
    with pytest.raises(ValueError):
        B._sptr(plain, R, K, "group64", "s")          # row-major [R, K/64]
    with pytest.raises(ValueError):
        B._sptr(s[:, :4], R, K, "group64", "s")       # wrong shape
    g = B.group64_scales(plain)
    assert torch.equal(g, plain) and g.stride() == (1, R)
    # memory order: element (r, grp) at grp * R + r
    flat = g.t().contiguous().reshape(-1)
    assert float(flat[3 * R + 2]) == float(plain[2, 3])
    assert B.group64_scales(g) is g
    # tensor / row scales pass unchanged; empty group-64 scales are accepted
    assert B._sptr(torch.ones(R), R, K, "row", "s") is not None
    assert B._sptr(torch.empty((0, K // 64)), 0, K, "group64", "s") is not None
