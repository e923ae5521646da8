"""ctypes binding of libqlinear.so (the C ABI in include/qlinear.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI.  torch is used for device memory (output allocation) and to
name the current HIP stream.  There is no fallback: if the library is
missing or the device is not gfx950, calls raise.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so the library shares it

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libqlinear.so")

# ---- constants mirrored from include/qlinear.h ------------------------------
QL_OK = 0
QL_ERR_NULL = -1
QL_ERR_SHAPE = -2
QL_ERR_ALIGN = -3
QL_ERR_UNSUPPORTED = -4
QL_ERR_LAUNCH = -5
QL_ERR_DEVICE = -6
QL_ERR_SCRATCH = -7

QL_SCALE_TENSOR = 0
QL_SCALE_ROW = 1
QL_SCALE_GROUP64 = 2
QL_LAYOUT_I8 = 0
QL_LAYOUT_PACKED = 1
QL_LAYOUT_FP6 = 2
QL_MX_FP4 = 4
QL_MX_FP8 = 8
MX_FORMATS = {"fp4": QL_MX_FP4, "fp8": QL_MX_FP8}
QL_EPI_BF16 = 0
QL_EPI_SWIGLU = 1
QL_EPI_GATED_RESIDUAL = 2
QL_EPI_F32 = 3
QL_EPI_I32 = 4
QL_EPI_SIGMOID = 5
QL_MAX_SEGMENTS = 8

SCALE_MODES = {"tensor": QL_SCALE_TENSOR, "row": QL_SCALE_ROW, "group64": QL_SCALE_GROUP64}
LAYOUTS = {"i8": QL_LAYOUT_I8, "packed": QL_LAYOUT_PACKED, "fp6": QL_LAYOUT_FP6}
EPILOGUES = {"bf16": QL_EPI_BF16, "swiglu": QL_EPI_SWIGLU, "gated_residual": QL_EPI_GATED_RESIDUAL,
             "f32": QL_EPI_F32, "i32": QL_EPI_I32, "sigmoid": QL_EPI_SIGMOID}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int

class Segment(ctypes.Structure):
    """ql_segment of include/qlinear.h."""
    _fields_ = [("w", ctypes.c_void_p), ("sw", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("w_bits", ctypes.c_int), ("epilogue", ctypes.c_int), ("out", ctypes.c_void_p),
                ("ldo", ctypes.c_int64)]


_SIGNATURES = {
    "ql_status_string": (ctypes.c_char_p, [_i]),
    "ql_device_supported": (_i, [_i]),
    "rotate_quantize_act": (_i, [_p, _i64, _i64, _i64, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p]),
    "rmsnorm_rotate_quantize_act": (_i, [_p, _i64, _i64, _i64, _p, _p, _p, ctypes.c_float, _i, _i, _i, _i,
                                         _p, _p, _p]),
    "pack_weight_int4": (_i, [_p, _i64, _i64, _i64, _i, _i, _p, _p, _p]),
    "pack_weight_fp6": (_i, [_p, _i64, _i64, _i64, _i, _i, _p, _p, _p]),
    "qgemm_w4a4": (_i, [_p, _p, _i, _i, _p, _p, _i, _i64, _i64, _i64, _p, _i, _p, _i64, _p]),
    "qgemm_w4a4_fp6": (_i, [_p, _p, _i, _p, _p, _i, _i64, _i64, _i64, _p, _i, _p, _i64, _p]),
    "qgemm_w8a8": (_i, [_p, _p, _i, _p, _p, _i, _i64, _i64, _i64, _p, _p, _p, _i, _p, _i64, _p]),
    "qgemm_w4a4_lowrank": (_i, [_p, _p, _i, _i, _p, _p, _i, _p, _p, _i, _i64, _i64, _i64, _p, _i, _p,
                                _i64, _p]),
    "qgemm_w4a4_fp6_lowrank": (_i, [_p, _p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _p, _i, _p, _i64, _p]),
    "qgemm_grouped": (_i, [_p, _p, _p, _p, _i64, _i64, ctypes.POINTER(Segment), _i, _p]),
    "svdq_split": (_i, [_p, _i64, _i64, _i64, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _i64,
                        _p]),
    "svdq_split_workspace_bytes": (_i64, [_i64, _i64, _i, _i, _i]),
    "svdq_split_noalloc": (_i, [_p, _i64, _i64, _i64, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]),
    "svdq_split_noalloc_max_bytes": (_i64, []),
    "rotate_quantize_mx": (_i, [_p, _i64, _i64, _i64, _i, _i, _p, _p, _p, _i, _p, _p]),
    "qgemm_mx": (_i, [_p, _p, _p, _p, _i, _i64, _i64, _i64, _p, _p, _p, _i, _p, _i64, _p]),
    "qgemm_mx_lowrank": (_i, [_p, _p, _p, _p, _i, _p, _p, _i, _i64, _i64, _i64, _p, _i, _p, _i64, _p]),
}

_LIB = None


class QLinearError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if libqlinear.so has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m rotated_bit_quantized_rotate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().ql_status_string(status).decode()


def device_supported(device: int = 0) -> bool:
    return bool(lib().ql_device_supported(device))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, st):
    if st != QL_OK:
        raise QLinearError(fn, st)


def _mode(m):
    return SCALE_MODES[m] if isinstance(m, str) else int(m)


def _epi(e):
    return EPILOGUES[e] if isinstance(e, str) else int(e)


def _lay(l):
    return LAYOUTS[l] if isinstance(l, str) else int(l)


def _codes(R, K, lay, device):
    if lay == QL_LAYOUT_PACKED:
        return torch.empty((R, K // 2), dtype=torch.uint8, device=device)
    if lay == QL_LAYOUT_FP6:
        return torch.empty((R, K // 4 * 3), dtype=torch.uint8, device=device)
    return torch.empty((R, K), dtype=torch.int8, device=device)


def _scale_shape(R, K, mode):
    return {QL_SCALE_TENSOR: (1,), QL_SCALE_ROW: (R,), QL_SCALE_GROUP64: (R, K // 64)}[mode]


def _new_scales(R, K, mode, device):
    """Scales of R rows.  Group-64 scales live group-major ([K/64, R] in
    memory, the library's layout) and are handed out as the transposed
    [R, K/64] view, so element [r, g] is still row r's scale of group g."""
    if mode == QL_SCALE_GROUP64:
        return torch.empty((K // 64, R), dtype=torch.float32, device=device).t()
    return torch.empty(_scale_shape(R, K, mode), dtype=torch.float32, device=device)


def group64_scales(s):
    """A [R, K/64] scale tensor in the library's group-major memory layout
    (the transposed view of a contiguous [K/64, R] tensor); returns s itself
    when it already is one."""
    return s if _group_major(s) else s.t().contiguous().t()


def _group_major(s):
    return s.dim() == 2 and (s.numel() == 0 or s.t().is_contiguous())


def _sptr(s, R, K, mode, name):
    """Pointer to scales after checking that group-64 scales are the [R, K/64]
    view of group-major memory."""
    if s is not None and _mode(mode) == QL_SCALE_GROUP64:
        if tuple(s.shape) != (R, K // 64) or not _group_major(s):
            raise ValueError(f"{name}: group-64 scales must be a [{R}, {K // 64}] view of group-major memory "
                             "(see group64_scales)")
    return _ptr(s)


# ---- entry points (same names as the C ABI) ---------------------------------

def rotate_quantize_act(x, bits=4, scale_mode="row", layout="i8", rotate=True, codes=None, scales=None,
                        l1=None, lr=None, stream=None):
    """x: bf16 [M, K] (row stride x.stride(0)).  Returns (codes, scales, lr)."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    mode = _mode(scale_mode)
    lay = _lay(layout)
    if codes is None:
        codes = _codes(M, K, lay, x.device)
    if scales is None:
        scales = _new_scales(M, K, mode, x.device)
    rank = 0
    if l1 is not None:
        rank = l1.shape[1]
        if lr is None:
            lr = torch.empty((M, rank), dtype=torch.bfloat16, device=x.device)
    st = lib().rotate_quantize_act(_ptr(x), M, K, x.stride(0), bits, mode, lay, int(bool(rotate)),
                                   _ptr(codes), _sptr(scales, M, K, mode, "scales"), _ptr(l1), rank, _ptr(lr),
                                   _stream(stream))
    _check("rotate_quantize_act", st)
    return codes, scales, lr


def rmsnorm_rotate_quantize_act(x, gamma=None, mod_scale=None, mod_shift=None, eps=1e-6, bits=4,
                                scale_mode="row", layout="i8", rotate=True, codes=None, scales=None,
                                stream=None):
    """x: bf16 [M, K]; gamma, mod_scale, mod_shift: bf16 [K] or None.  The
    block's RMSNorm + modulation fused in front of rotate + quantize.
    Returns (codes, scales)."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    for v in (gamma, mod_scale, mod_shift):
        assert v is None or (v.dtype == torch.bfloat16 and v.numel() == K and v.is_contiguous())
    mode = _mode(scale_mode)
    lay = _lay(layout)
    if codes is None:
        codes = _codes(M, K, lay, x.device)
    if scales is None:
        scales = _new_scales(M, K, mode, x.device)
    st = lib().rmsnorm_rotate_quantize_act(_ptr(x), M, K, x.stride(0), _ptr(gamma), _ptr(mod_scale),
                                           _ptr(mod_shift), float(eps), bits, mode, lay, int(bool(rotate)),
                                           _ptr(codes), _sptr(scales, M, K, mode, "scales"), _stream(stream))
    _check("rmsnorm_rotate_quantize_act", st)
    return codes, scales


def pack_weight_int4(w, scale_mode="row", rotate=True, packed=None, scales=None, stream=None):
    """w: bf16 [N, K].  Returns (packed uint8 [N, K/2], scales)."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1
    N, K = w.shape
    mode = _mode(scale_mode)
    if packed is None:
        packed = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = _new_scales(N, K, mode, w.device)
    st = lib().pack_weight_int4(_ptr(w), N, K, w.stride(0), mode, int(bool(rotate)), _ptr(packed),
                                _sptr(scales, N, K, mode, "scales"), _stream(stream))
    _check("pack_weight_int4", st)
    return packed, scales


def pack_weight_fp6(w, scale_mode="row", rotate=True, packed=None, scales=None, stream=None):
    """w: bf16 [N, K].  Returns (uint8 [N, 3K/4] in the FP6 layout, scales)."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1
    N, K = w.shape
    mode = _mode(scale_mode)
    if packed is None:
        packed = _codes(N, K, QL_LAYOUT_FP6, w.device)
    if scales is None:
        scales = _new_scales(N, K, mode, w.device)
    st = lib().pack_weight_fp6(_ptr(w), N, K, w.stride(0), mode, int(bool(rotate)), _ptr(packed),
                               _sptr(scales, N, K, mode, "scales"), _stream(stream))
    _check("pack_weight_fp6", st)
    return packed, scales


def _mxfmt(f):
    return MX_FORMATS[f] if isinstance(f, str) else int(f)


def rotate_quantize_mx(x, fmt="fp4", rotate=True, codes=None, scales=None, l1=None, lr=None, stream=None):
    """x: bf16 [R, K] -> (element bytes [R, K/2] (fp4) | [R, K] (fp8) uint8,
    E8M0 scale bytes uint8 [K/128, R, 4], stage-major).  Serves activations
    and weights.  With l1 (bf16 [K, rank]) also returns lr = x @ l1 (bf16
    [R, rank], unrotated x) as a third value."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    R, K = x.shape
    f = _mxfmt(fmt)
    if codes is None:
        codes = torch.empty((R, K // 2 if f == QL_MX_FP4 else K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((K // 128, R, 4), dtype=torch.uint8, device=x.device)
    rank = 0 if l1 is None else l1.shape[1]
    if l1 is not None and lr is None:
        lr = torch.empty((R, rank), dtype=torch.bfloat16, device=x.device)
    st = lib().rotate_quantize_mx(_ptr(x), R, K, x.stride(0), f, int(bool(rotate)), _ptr(codes), _ptr(scales),
                                  _ptr(l1), rank, _ptr(lr), _stream(stream))
    _check("rotate_quantize_mx", st)
    return (codes, scales) if l1 is None else (codes, scales, lr)


def _out(out, M, cols, epi, device):
    if out is not None:
        return out
    dt = {QL_EPI_F32: torch.float32, QL_EPI_I32: torch.int32}.get(epi, torch.bfloat16)
    return torch.empty((M, cols), dtype=dt, device=device)


def qgemm_w4a4(a, sa, w, sw, K, a_scale_mode="row", w_scale_mode="row", a_layout="i8", bias=None,
               epilogue="bf16", out=None, stream=None):
    """a: codes [M, K] int8 or [M, K/2] packed; w: packed [N, K/2]."""
    M = a.shape[0]
    N = w.shape[0]
    epi = _epi(epilogue)
    out = _out(out, M, N // 2 if epi == QL_EPI_SWIGLU else N, epi, a.device)
    st = lib().qgemm_w4a4(_ptr(a), _sptr(sa, M, K, a_scale_mode, "sa"), _mode(a_scale_mode), _lay(a_layout),
                          _ptr(w), _sptr(sw, N, K, w_scale_mode, "sw"),
                          _mode(w_scale_mode), M, N, K, _ptr(bias), epi, _ptr(out), out.stride(0),
                          _stream(stream))
    _check("qgemm_w4a4", st)
    return out


def qgemm_w4a4_fp6(a, sa, w, sw, K, a_scale_mode="row", w_scale_mode="row", bias=None, epilogue="bf16",
                   out=None, stream=None):
    """a: codes [M, 3K/4], w: codes [N, 3K/4], both in the FP6 layout; tensor /
    row scales, or group-64 on both sides (BF16 / F32 epilogues)."""
    M = a.shape[0]
    N = w.shape[0]
    epi = _epi(epilogue)
    out = _out(out, M, N, epi, a.device)
    st = lib().qgemm_w4a4_fp6(_ptr(a), _sptr(sa, M, K, a_scale_mode, "sa"), _mode(a_scale_mode), _ptr(w),
                              _sptr(sw, N, K, w_scale_mode, "sw"), _mode(w_scale_mode),
                              M, N, K, _ptr(bias), epi, _ptr(out), out.stride(0), _stream(stream))
    _check("qgemm_w4a4_fp6", st)
    return out


def qgemm_mx(a, sa, w, sw, K, fmt="fp4", bias=None, residual=None, gate=None, epilogue="bf16", out=None,
             stream=None):
    """MX block-scaled GEMM: a, w element bytes and sa, sw E8M0 scale bytes
    from rotate_quantize_mx with the same fmt."""
    M = a.shape[0]
    N = w.shape[0]
    epi = _epi(epilogue)
    out = _out(out, M, N // 2 if epi == QL_EPI_SWIGLU else N, epi, a.device)
    st = lib().qgemm_mx(_ptr(a), _ptr(sa), _ptr(w), _ptr(sw), _mxfmt(fmt), M, N, K, _ptr(bias), _ptr(residual),
                        _ptr(gate), epi, _ptr(out), out.stride(0), _stream(stream))
    _check("qgemm_mx", st)
    return out


def qgemm_mx_lowrank(a, sa, w, sw, K, fmt="fp4", lr=None, l2=None, bias=None, epilogue="swiglu", out=None,
                     stream=None):
    """The MX GEMM plus the low-rank branch lr @ L2 (SVDQuant in MX form);
    l2 is L2 transposed, bf16 [N, rank]."""
    M = a.shape[0]
    N = w.shape[0]
    epi = _epi(epilogue)
    rank = 0 if lr is None else lr.shape[1]
    out = _out(out, M, N // 2 if epi == QL_EPI_SWIGLU else N, epi, a.device)
    st = lib().qgemm_mx_lowrank(_ptr(a), _ptr(sa), _ptr(w), _ptr(sw), _mxfmt(fmt), _ptr(lr), _ptr(l2), rank, M, N, K,
                                _ptr(bias), epi, _ptr(out), out.stride(0), _stream(stream))
    _check("qgemm_mx_lowrank", st)
    return out


def qgemm_w8a8(a, sa, w, sw, a_scale_mode="row", w_scale_mode="row", bias=None, residual=None, gate=None,
               epilogue="bf16", out=None, stream=None):
    """a: int8 [M, K]; w: int8 [N, K].  residual may be `out` itself."""
    M, K = a.shape
    N = w.shape[0]
    epi = _epi(epilogue)
    out = _out(out, M, N, epi, a.device)
    st = lib().qgemm_w8a8(_ptr(a), _sptr(sa, M, K, a_scale_mode, "sa"), _mode(a_scale_mode), _ptr(w),
                          _sptr(sw, N, K, w_scale_mode, "sw"), _mode(w_scale_mode),
                          M, N, K, _ptr(bias), _ptr(residual), _ptr(gate), epi, _ptr(out), out.stride(0),
                          _stream(stream))
    _check("qgemm_w8a8", st)
    return out


def qgemm_w4a4_lowrank(a, sa, w, sw, K, lr=None, l2=None, a_scale_mode="group64",
                       w_scale_mode="group64", a_layout="i8", bias=None, epilogue="swiglu", out=None,
                       stream=None):
    """Group-64 (or row / tensor) W4A4 GEMM + optional low-rank branch
    lr @ L2 + epilogue (l2: L2 transposed, bf16 [N, rank]); a_layout "i8" or
    "packed"."""
    M = a.shape[0]
    N = w.shape[0]
    epi = _epi(epilogue)
    rank = 0 if l2 is None else l2.shape[1]
    out = _out(out, M, N // 2 if epi == QL_EPI_SWIGLU else N, epi, a.device)
    st = lib().qgemm_w4a4_lowrank(_ptr(a), _sptr(sa, M, K, a_scale_mode, "sa"), _mode(a_scale_mode),
                                  _lay(a_layout), _ptr(w), _sptr(sw, N, K, w_scale_mode, "sw"), _mode(w_scale_mode), _ptr(lr), _ptr(l2), rank, M, N, K,
                                  _ptr(bias), epi, _ptr(out), out.stride(0), _stream(stream))
    _check("qgemm_w4a4_lowrank", st)
    return out


def qgemm_w4a4_fp6_lowrank(a, sa, w, sw, K, lr=None, l2=None, bias=None, epilogue="swiglu", out=None,
                           stream=None):
    """The group-64 low-rank GEMM on the FP6 matrix instruction: a [M, 3K/4]
    and w [N, 3K/4] in the FP6 layout, sa [M, K/64], sw [N, K/64] (group-
    major views, see group64_scales); same
    result as qgemm_w4a4_lowrank on the same codes."""
    M = a.shape[0]
    N = w.shape[0]
    epi = _epi(epilogue)
    rank = 0 if l2 is None else l2.shape[1]
    out = _out(out, M, N // 2 if epi == QL_EPI_SWIGLU else N, epi, a.device)
    st = lib().qgemm_w4a4_fp6_lowrank(_ptr(a), _sptr(sa, M, K, "group64", "sa"), _ptr(w),
                                      _sptr(sw, N, K, "group64", "sw"), _ptr(lr), _ptr(l2), rank, M, N, K,
                                      _ptr(bias), epi, _ptr(out), out.stride(0), _stream(stream))
    _check("qgemm_w4a4_fp6_lowrank", st)
    return out


def qgemm_grouped(a4, sa4, a8, sa8, K, segments, stream=None):
    """Several projections of the same activations in one launch.
    a4/sa4: int8-container int4 codes [M, K] + row scales (or None);
    a8/sa8: int8 codes [M, K] + row scales (or None).  segments: list of
    dicts with w (packed int4 [n, K/2] or int8 [n, K]), sw [n], bits (4 | 8),
    epilogue ("bf16" | "sigmoid") and optionally out (bf16 [M, n]).
    Returns the list of outputs."""
    ref = a4 if a4 is not None else a8
    M = ref.shape[0]
    arr = (Segment * len(segments))()
    outs = []
    for i, sg in enumerate(segments):
        n = sg["w"].shape[0]
        out = sg.get("out")
        if out is None:
            out = torch.empty((M, n), dtype=torch.bfloat16, device=ref.device)
        outs.append(out)
        arr[i] = Segment(_ptr(sg["w"]), _ptr(sg["sw"]), n, int(sg["bits"]), _epi(sg.get("epilogue", "bf16")),
                         _ptr(out), out.stride(0))
    st = lib().qgemm_grouped(_ptr(a4), _ptr(sa4), _ptr(a8), _ptr(sa8), M, K, arr, len(segments),
                             _stream(stream))
    _check("qgemm_grouped", st)
    return outs


def svdq_split_workspace_bytes(N, K, rank, oversample=8, scale_mode="group64"):
    return lib().svdq_split_workspace_bytes(N, K, rank, oversample, _mode(scale_mode))


def svdq_split(w, omega, rank, oversample=8, power_iters=2, refine_iters=0, scale_mode="group64",
               act_rms=None, workspace=None, stream=None):
    """Offline SVDQuant split of w (bf16 [N, K]) with the Gaussian sketch
    omega (float32 [K, rank + oversample]).  Returns a dict with l1 bf16
    [K, rank], l2 bf16 [N, rank] (L2 transposed), packed uint8 [N, K/2], scales, errors float32
    [refine_iters + 1], best_iter int32 [1] and sigma float32 [rank]."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1
    N, K = w.shape
    dev = w.device
    mode = _mode(scale_mode)
    assert omega.dtype == torch.float32 and tuple(omega.shape) == (K, rank + oversample) and omega.is_contiguous()
    if act_rms is not None:
        assert act_rms.dtype == torch.float32 and act_rms.numel() == K and act_rms.is_contiguous()
    need = lib().svdq_split_workspace_bytes(N, K, rank, oversample, mode)
    if need < 0:
        raise QLinearError("svdq_split_workspace_bytes", QL_ERR_SHAPE)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    out = {"l1": torch.empty((K, rank), dtype=torch.bfloat16, device=dev),
           "l2": torch.empty((N, rank), dtype=torch.bfloat16, device=dev),
           "packed": torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
           "scales": _new_scales(N, K, mode, dev),
           "errors": torch.empty(refine_iters + 1, dtype=torch.float32, device=dev),
           "best_iter": torch.empty(1, dtype=torch.int32, device=dev),
           "sigma": torch.empty(rank, dtype=torch.float32, device=dev)}
    st = lib().svdq_split(_ptr(w), N, K, w.stride(0), _ptr(act_rms), _ptr(omega), rank, oversample, power_iters,
                          refine_iters, mode, _ptr(out["l1"]), _ptr(out["l2"]), _ptr(out["packed"]),
                          _sptr(out["scales"], N, K, mode, "scales"), _ptr(out["errors"]), _ptr(out["best_iter"]),
                          _ptr(out["sigma"]),
                          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("svdq_split", st)
    return out


def svdq_split_noalloc_max_bytes():
    return lib().svdq_split_noalloc_max_bytes()


def svdq_split_noalloc(w, omega, rank, oversample=8, power_iters=2, refine_iters=0, scale_mode="group64",
                       act_rms=None, out=None, stream=None):
    """svdq_split without a workspace: the library's fixed per-GPU array holds
    it and the call allocates nothing.  `out` may pass the output dict of an
    earlier call (same shapes) to reuse its tensors; otherwise they are
    allocated here, before the call.  Returns the same dict as svdq_split."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1
    N, K = w.shape
    dev = w.device
    mode = _mode(scale_mode)
    assert omega.dtype == torch.float32 and tuple(omega.shape) == (K, rank + oversample) and omega.is_contiguous()
    if act_rms is not None:
        assert act_rms.dtype == torch.float32 and act_rms.numel() == K and act_rms.is_contiguous()
    if out is None:
        out = {"l1": torch.empty((K, rank), dtype=torch.bfloat16, device=dev),
               "l2": torch.empty((N, rank), dtype=torch.bfloat16, device=dev),
               "packed": torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
               "scales": _new_scales(N, K, mode, dev),
               "errors": torch.empty(refine_iters + 1, dtype=torch.float32, device=dev),
               "best_iter": torch.empty(1, dtype=torch.int32, device=dev),
               "sigma": torch.empty(rank, dtype=torch.float32, device=dev)}
    st = lib().svdq_split_noalloc(_ptr(w), N, K, w.stride(0), _ptr(act_rms), _ptr(omega), rank, oversample,
                                  power_iters, refine_iters, mode, _ptr(out["l1"]), _ptr(out["l2"]),
                                  _ptr(out["packed"]), _sptr(out["scales"], N, K, mode, "scales"), _ptr(out["errors"]),
                                  _ptr(out["best_iter"]), _ptr(out["sigma"]), _stream(stream))
    _check("svdq_split_noalloc", st)
    return out

