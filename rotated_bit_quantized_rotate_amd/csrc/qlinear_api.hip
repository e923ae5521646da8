// C ABI of libqlinear: argument validation, device check and dispatch to the
// HIP kernels.  Every precondition listed in include/qlinear.h is checked
// here before anything is enqueued; nothing is allocated, nothing is
// synchronized.

#include <string.h>

#include "../../include/qlinear.h"
#include "ql_internal.h"

static_assert(QL_MAX_SEGMENTS == ql::kMaxGroupSegments, "segment limit mismatch");

namespace {

constexpr int kMaxDevices = 64;
// Per-device cache of "is gfx950": 0 unknown, 1 yes, 2 no.  Written only with
// the value the runtime reports, so concurrent first calls agree.
int g_dev_ok[kMaxDevices];

int device_is_gfx950(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 0;
  const int c = __atomic_load_n(&g_dev_ok[dev], __ATOMIC_RELAXED);
  if (c) return c == 1;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  const int ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  __atomic_store_n(&g_dev_ok[dev], ok ? 1 : 2, __ATOMIC_RELAXED);
  return ok;
}

int check_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QL_ERR_DEVICE;
  return device_is_gfx950(dev) ? QL_OK : QL_ERR_UNSUPPORTED;
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool al2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

inline bool valid_mode(int m) { return m == QL_SCALE_TENSOR || m == QL_SCALE_ROW || m == QL_SCALE_GROUP64; }

// The int32 accumulator of a tensor / row-scale GEMM holds K products of
// codes; the largest product is qmax_a * qmax_w times 16 per packed INT4
// operand (its codes enter the int8 instruction as 16 * code).  The sum is
// exact only while K times that stays below 2^31.  Group-64 partials cover 64
// channels and never overflow.
inline bool acc_fits(int64_t K, int64_t max_product) { return K * max_product <= INT32_MAX; }
constexpr int64_t kProdW8A8 = 127 * 127;          // K <= 133144
constexpr int64_t kProdW4A4I8 = 7 * (16 * 7);     // int8-container codes x packed W: K <= 2739137
constexpr int64_t kProdW4A4P = (16 * 7) * (16 * 7);  // both packed: K <= 171196

}  // namespace

extern "C" {

const char* ql_status_string(int status) {
  switch (status) {
    case QL_OK: return "QL_OK: success";
    case QL_ERR_NULL: return "QL_ERR_NULL: a required pointer is NULL";
    case QL_ERR_SHAPE: return "QL_ERR_SHAPE: a size or stride violates a precondition";
    case QL_ERR_ALIGN: return "QL_ERR_ALIGN: a pointer or stride is misaligned";
    case QL_ERR_UNSUPPORTED: return "QL_ERR_UNSUPPORTED: mode combination or device not supported";
    case QL_ERR_LAUNCH: return "QL_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case QL_ERR_DEVICE: return "QL_ERR_DEVICE: the current device could not be queried";
    case QL_ERR_SCRATCH:
      return "QL_ERR_SCRATCH: the problem needs more workspace than the allocation-free entry point holds";
    default: return "unknown qlinear status";
  }
}

int ql_device_supported(int device) { return device_is_gfx950(device); }

static int validate_rq(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int bits, int scale_mode,
                       int layout, int rotate, const void* codes, const float* scales,
                       const uint16_t* l1, int rank, const uint16_t* lr) {
  if (bits != 4 && bits != 8) return QL_ERR_UNSUPPORTED;
  if (!valid_mode(scale_mode)) return QL_ERR_UNSUPPORTED;
  if (layout != QL_LAYOUT_I8 && layout != QL_LAYOUT_PACKED && layout != QL_LAYOUT_FP6) return QL_ERR_UNSUPPORTED;
  if (layout != QL_LAYOUT_I8 && bits != 4) return QL_ERR_UNSUPPORTED;
  if (rotate != 0 && rotate != 1) return QL_ERR_UNSUPPORTED;
  if (M < 0 || K <= 0 || K % 256 != 0 || K > 32768) return QL_ERR_SHAPE;
  if (ldx < K || ldx % 8 != 0) return QL_ERR_SHAPE;
  if (M > 0 && (!x || !codes || !scales)) return QL_ERR_NULL;
  if (!l1 && rank != 0) return QL_ERR_SHAPE;
  if (l1) {
    if (rank < 16 || rank > 128 || rank % 16 != 0) return QL_ERR_SHAPE;
    if (M > 0 && !lr) return QL_ERR_NULL;
    if (!al16(l1) || !al16(lr)) return QL_ERR_ALIGN;
  }
  if (!al16(x) || !al16(codes) || !al4(scales)) return QL_ERR_ALIGN;
  return QL_OK;
}

int rotate_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int bits, int scale_mode,
                        int layout, int rotate, void* codes, float* scales, const uint16_t* l1,
                        int rank, uint16_t* lr, void* stream) {
  int st = validate_rq(x, M, K, ldx, bits, scale_mode, layout, rotate, codes, scales, l1, rank, lr);
  if (st != QL_OK) return st;
  if ((st = check_current_device()) != QL_OK) return st;
  if (M == 0) return QL_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ql::RqArgs a{x, M, K, ldx, bits, scale_mode, layout, rotate, codes, scales};
  st = ql::launch_rotate_quantize(a, s);
  if (st != QL_OK) return QL_ERR_LAUNCH;
  if (l1) {
    st = ql::launch_lowrank_down(x, M, K, ldx, l1, rank, lr, s);
    if (st != QL_OK) return QL_ERR_LAUNCH;
  }
  return QL_OK;
}

int rmsnorm_rotate_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                const uint16_t* mod_scale, const uint16_t* mod_shift, float eps, int bits,
                                int scale_mode, int layout, int rotate, void* codes, float* scales,
                                void* stream) {
  int st = validate_rq(x, M, K, ldx, bits, scale_mode, layout, rotate, codes, scales, nullptr, 0, nullptr);
  if (st != QL_OK) return st;
  // the per-channel vectors are staged in LDS (8 bytes per channel)
  if (K > 8192) return QL_ERR_SHAPE;
  if (!(eps > 0.0f) || eps > 3.0e38f) return QL_ERR_SHAPE;  // positive and finite (NaN fails too)
  if (!al16(gamma) || !al16(mod_scale) || !al16(mod_shift)) return QL_ERR_ALIGN;
  if ((st = check_current_device()) != QL_OK) return st;
  if (M == 0) return QL_OK;
  ql::RqArgs a{x, M, K, ldx, bits, scale_mode, layout, rotate, codes, scales};
  a.norm = 1;
  a.gamma = gamma;
  a.mscale = mod_scale;
  a.mshift = mod_shift;
  a.eps = eps;
  return ql::launch_rotate_quantize(a, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

int pack_weight_int4(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, int scale_mode, int rotate,
                     uint8_t* packed, float* scales, void* stream) {
  if (N <= 0 || N % 2 != 0) return QL_ERR_SHAPE;  // rows are stored in pairs
  int st = validate_rq(w, N, K, ldw, 4, scale_mode, QL_LAYOUT_PACKED, rotate, packed, scales, nullptr, 0, nullptr);
  if (st != QL_OK) return st;
  if ((st = check_current_device()) != QL_OK) return st;
  ql::RqArgs a{w, N, K, ldw, 4, scale_mode, QL_LAYOUT_PACKED, rotate, packed, scales};
  a.paired = 1;
  return ql::launch_rotate_quantize(a, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

int pack_weight_fp6(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, int scale_mode, int rotate,
                    uint8_t* packed, float* scales, void* stream) {
  if (N <= 0) return QL_ERR_SHAPE;
  return rotate_quantize_act(w, N, K, ldw, 4, scale_mode, QL_LAYOUT_FP6, rotate, packed, scales, nullptr, 0,
                             nullptr, stream);
}

// Output element size per epilogue (SWIGLU / BF16 / GATED write bf16).
inline int64_t out_elem_size(int epilogue) {
  return (epilogue == QL_EPI_F32 || epilogue == QL_EPI_I32) ? 4 : 2;
}

static int validate_gemm_common(const void* a, const float* sa, const void* w, const float* sw,
                                int64_t M, int64_t N, int64_t K, const uint16_t* bias, void* out,
                                int64_t ldo, int epilogue) {
  if (M < 0 || N <= 0 || N % 16 != 0 || K <= 0 || K % 256 != 0) return QL_ERR_SHAPE;
  // the GEMM kernels address operands, scales included, with 32-bit offsets
  if (K >= (int64_t(1) << 23) || N * K >= (int64_t(1) << 31) || M >= (int64_t(1) << 36) / K)
    return QL_ERR_SHAPE;
  const int64_t out_cols = epilogue == QL_EPI_SWIGLU ? N / 2 : N;
  if (ldo < out_cols) return QL_ERR_SHAPE;
  if (M > 0 && (!a || !sa || !w || !sw || !out)) return QL_ERR_NULL;
  if (!al16(a) || !al16(w) || !al4(sa) || !al4(sw) || !al16(out)) return QL_ERR_ALIGN;
  if ((ldo * out_elem_size(epilogue)) % 16 != 0) return QL_ERR_ALIGN;
  if (bias && !al2(bias)) return QL_ERR_ALIGN;
  return QL_OK;
}

int qgemm_w4a4(const void* a, const float* sa, int a_scale_mode, int a_layout, const uint8_t* w,
               const float* sw, int w_scale_mode, int64_t M, int64_t N, int64_t K, const uint16_t* bias,
               int epilogue, void* out, int64_t ldo, void* stream) {
  if (!valid_mode(a_scale_mode) || !valid_mode(w_scale_mode)) return QL_ERR_UNSUPPORTED;
  if (a_layout != QL_LAYOUT_I8 && a_layout != QL_LAYOUT_PACKED) return QL_ERR_UNSUPPORTED;
  if (a_scale_mode == QL_SCALE_GROUP64 || w_scale_mode == QL_SCALE_GROUP64) {
    if (a_scale_mode != QL_SCALE_GROUP64 || w_scale_mode != QL_SCALE_GROUP64) return QL_ERR_UNSUPPORTED;
    // group partials are rescaled in fp32: no exact I32 result, and the
    // sigmoid gate / SwiGLU are not offered here
    if (epilogue != QL_EPI_BF16 && epilogue != QL_EPI_F32) return QL_ERR_UNSUPPORTED;
    return qgemm_w4a4_lowrank(a, sa, a_scale_mode, a_layout, w, sw, w_scale_mode, nullptr, nullptr, 0, M,
                              N, K, bias, epilogue, out, ldo, stream);
  }
  if (epilogue != QL_EPI_BF16 && epilogue != QL_EPI_F32 && epilogue != QL_EPI_I32 && epilogue != QL_EPI_SIGMOID)
    return QL_ERR_UNSUPPORTED;
  int st = validate_gemm_common(a, sa, w, sw, M, N, K, bias, out, ldo, epilogue);
  if (st != QL_OK) return st;
  if (!acc_fits(K, a_layout == QL_LAYOUT_PACKED ? kProdW4A4P : kProdW4A4I8)) return QL_ERR_SHAPE;
  if ((st = check_current_device()) != QL_OK) return st;
  if (M == 0) return QL_OK;
  ql::GemmArgs g{};
  g.a = a;
  g.w = w;
  g.sa = sa;
  g.sw = sw;
  g.M = M;
  g.N = N;
  g.K = K;
  g.a_packed = a_layout == QL_LAYOUT_PACKED;
  g.w_packed = 1;
  g.a_mode = a_scale_mode;
  g.w_mode = w_scale_mode;
  g.bias = bias;
  g.epilogue = epilogue;
  g.out = out;
  g.ldo = ldo;
  return ql::launch_qgemm(g, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

int qgemm_w4a4_fp6(const uint8_t* a, const float* sa, int a_scale_mode, const uint8_t* w, const float* sw,
                   int w_scale_mode, int64_t M, int64_t N, int64_t K, const uint16_t* bias, int epilogue,
                   void* out, int64_t ldo, void* stream) {
  const bool grp = a_scale_mode == QL_SCALE_GROUP64 && w_scale_mode == QL_SCALE_GROUP64;
  if (!grp && ((a_scale_mode != QL_SCALE_TENSOR && a_scale_mode != QL_SCALE_ROW) ||
               (w_scale_mode != QL_SCALE_TENSOR && w_scale_mode != QL_SCALE_ROW)))
    return QL_ERR_UNSUPPORTED;
  if (epilogue != QL_EPI_BF16 && epilogue != QL_EPI_F32 && epilogue != QL_EPI_I32 && epilogue != QL_EPI_SIGMOID)
    return QL_ERR_UNSUPPORTED;
  // group-64 partials are rescaled in fp32, so there is no exact sum to return
  if (grp && epilogue != QL_EPI_BF16 && epilogue != QL_EPI_F32) return QL_ERR_UNSUPPORTED;
  int st = validate_gemm_common(a, sa, w, sw, M, N, K, bias, out, ldo, epilogue);
  if (st != QL_OK) return st;
  // float32 sums of code products stay exact (a group-64 partial is at most 64 * 49)
  if (!grp && 49 * K >= (int64_t(1) << 24)) return QL_ERR_SHAPE;
  if ((st = check_current_device()) != QL_OK) return st;
  if (M == 0) return QL_OK;
  ql::GemmArgs g{};
  g.a = a;
  g.w = w;
  g.sa = sa;
  g.sw = sw;
  g.M = M;
  g.N = N;
  g.K = K;
  g.fp6 = 1;
  g.a_mode = a_scale_mode;
  g.w_mode = w_scale_mode;
  g.bias = bias;
  g.epilogue = epilogue;
  g.out = out;
  g.ldo = ldo;
  return ql::launch_qgemm(g, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

int rotate_quantize_mx(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int fmt, int rotate, void* codes,
                       uint8_t* scales, const uint16_t* l1, int rank, uint16_t* lr, void* stream) {
  if (fmt != QL_MX_FP4 && fmt != QL_MX_FP8) return QL_ERR_UNSUPPORTED;
  if (rotate != 0 && rotate != 1) return QL_ERR_UNSUPPORTED;
  if (M < 0 || K <= 0 || K % 256 != 0 || K >= (int64_t(1) << 23)) return QL_ERR_SHAPE;
  if (ldx < K || ldx % 8 != 0) return QL_ERR_SHAPE;
  if (M > 0 && (!x || !codes || !scales)) return QL_ERR_NULL;
  if (!l1 && rank != 0) return QL_ERR_SHAPE;
  if (l1) {
    if (rank < 16 || rank > 128 || rank % 16 != 0) return QL_ERR_SHAPE;
    if (M > 0 && !lr) return QL_ERR_NULL;
    if (!al16(l1) || !al16(lr)) return QL_ERR_ALIGN;
  }
  if (!al16(x) || !al16(codes) || !al4(scales)) return QL_ERR_ALIGN;
  int st = check_current_device();
  if (st != QL_OK) return st;
  if (M == 0) return QL_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ql::MxArgs a{x, M, K, ldx, fmt, rotate, codes, scales};
  if (ql::launch_mx_quantize(a, s) != QL_OK) return QL_ERR_LAUNCH;
  if (l1 && ql::launch_lowrank_down(x, M, K, ldx, l1, rank, lr, s) != QL_OK) return QL_ERR_LAUNCH;
  return QL_OK;
}

int qgemm_mx_lowrank(const void* a, const uint8_t* sa, const void* w, const uint8_t* sw, int fmt,
                     const uint16_t* lr, const uint16_t* l2, int rank, int64_t M, int64_t N, int64_t K,
                     const uint16_t* bias, int epilogue, void* out, int64_t ldo, void* stream) {
  if (fmt != QL_MX_FP4 && fmt != QL_MX_FP8) return QL_ERR_UNSUPPORTED;
  if (epilogue != QL_EPI_BF16 && epilogue != QL_EPI_SWIGLU && epilogue != QL_EPI_F32) return QL_ERR_UNSUPPORTED;
  if (epilogue == QL_EPI_SWIGLU && N % 32 != 0) return QL_ERR_SHAPE;
  int st = validate_gemm_common(a, reinterpret_cast<const float*>(sa), w, reinterpret_cast<const float*>(sw), M,
                                N, K, bias, out, ldo, epilogue);
  if (st != QL_OK) return st;
  if (rank < 0 || rank > 128 || rank % 16 != 0) return QL_ERR_SHAPE;
  if (rank > 0) {
    if (M > 0 && (!lr || !l2)) return QL_ERR_NULL;
    if (!al16(lr) || !al16(l2)) return QL_ERR_ALIGN;
  }
  if ((st = check_current_device()) != QL_OK) return st;
  if (M == 0) return QL_OK;
  ql::GemmArgs g{};
  g.a = a;
  g.w = w;
  g.M = M;
  g.N = N;
  g.K = K;
  g.mx = fmt;
  g.xa = sa;
  g.xw = sw;
  g.lr = lr;
  g.l2 = l2;
  g.rank = rank;
  g.bias = bias;
  g.epilogue = epilogue;
  g.out = out;
  g.ldo = ldo;
  return ql::launch_qgemm(g, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

int qgemm_mx(const void* a, const uint8_t* sa, const void* w, const uint8_t* sw, int fmt, int64_t M, int64_t N,
             int64_t K, const uint16_t* bias, const uint16_t* residual, const uint16_t* gate, int epilogue,
             void* out, int64_t ldo, void* stream) {
  if (fmt != QL_MX_FP4 && fmt != QL_MX_FP8) return QL_ERR_UNSUPPORTED;
  if (epilogue != QL_EPI_BF16 && epilogue != QL_EPI_F32 && epilogue != QL_EPI_SIGMOID &&
      epilogue != QL_EPI_GATED_RESIDUAL && epilogue != QL_EPI_SWIGLU)
    return QL_ERR_UNSUPPORTED;
  if (epilogue == QL_EPI_SWIGLU && N % 32 != 0) return QL_ERR_SHAPE;
  // scale bytes are checked like float scales: present and 4-byte aligned
  // (the kernel moves a row's 4 stage scales as one dword)
  int st = validate_gemm_common(a, reinterpret_cast<const float*>(sa), w, reinterpret_cast<const float*>(sw), M,
                                N, K, bias, out, ldo, epilogue);
  if (st != QL_OK) return st;
  if (epilogue == QL_EPI_GATED_RESIDUAL) {
    if (M > 0 && (!residual || !gate)) return QL_ERR_NULL;
    if (!al16(residual) || !al2(gate)) return QL_ERR_ALIGN;
  }
  if ((st = check_current_device()) != QL_OK) return st;
  if (M == 0) return QL_OK;
  ql::GemmArgs g{};
  g.a = a;
  g.w = w;
  g.M = M;
  g.N = N;
  g.K = K;
  g.mx = fmt;
  g.xa = sa;
  g.xw = sw;
  g.bias = bias;
  g.residual = residual;
  g.gate = gate;
  g.epilogue = epilogue;
  g.out = out;
  g.ldo = ldo;
  return ql::launch_qgemm(g, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

int qgemm_w8a8(const int8_t* a, const float* sa, int a_scale_mode, const int8_t* w, const float* sw,
               int w_scale_mode, int64_t M, int64_t N, int64_t K, const uint16_t* bias,
               const uint16_t* residual, const uint16_t* gate, int epilogue, void* out, int64_t ldo,
               void* stream) {
  if ((a_scale_mode != QL_SCALE_TENSOR && a_scale_mode != QL_SCALE_ROW) ||
      (w_scale_mode != QL_SCALE_TENSOR && w_scale_mode != QL_SCALE_ROW))
    return QL_ERR_UNSUPPORTED;
  if (epilogue != QL_EPI_BF16 && epilogue != QL_EPI_GATED_RESIDUAL && epilogue != QL_EPI_F32 &&
      epilogue != QL_EPI_I32 && epilogue != QL_EPI_SIGMOID)
    return QL_ERR_UNSUPPORTED;
  int st = validate_gemm_common(a, sa, w, sw, M, N, K, bias, out, ldo, epilogue);
  if (st != QL_OK) return st;
  if (!acc_fits(K, kProdW8A8)) return QL_ERR_SHAPE;
  if (epilogue == QL_EPI_GATED_RESIDUAL) {
    if (M > 0 && (!residual || !gate)) return QL_ERR_NULL;
    if (!al16(residual) || !al2(gate)) return QL_ERR_ALIGN;
  }
  if ((st = check_current_device()) != QL_OK) return st;
  if (M == 0) return QL_OK;
  ql::GemmArgs g{};
  g.a = a;
  g.w = w;
  g.sa = sa;
  g.sw = sw;
  g.M = M;
  g.N = N;
  g.K = K;
  g.a_packed = 0;
  g.w_packed = 0;
  g.a_mode = a_scale_mode;
  g.w_mode = w_scale_mode;
  g.bias = bias;
  g.residual = residual;
  g.gate = gate;
  g.epilogue = epilogue;
  g.out = out;
  g.ldo = ldo;
  return ql::launch_qgemm(g, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

// The low-rank GEMM on INT4 codes (fp6 == 0) or on FP6 codes with group-64
// scales (fp6 == 1); both entry points below validate their own layouts.
static int lowrank_gemm(const void* a, const float* sa, int a_scale_mode, int a_layout, const uint8_t* w,
                        const float* sw, int w_scale_mode, const uint16_t* lr, const uint16_t* l2, int rank,
                        int64_t M, int64_t N, int64_t K, const uint16_t* bias, int epilogue, void* out,
                        int64_t ldo, void* stream, int fp6) {
  if (epilogue != QL_EPI_BF16 && epilogue != QL_EPI_SWIGLU && epilogue != QL_EPI_F32) return QL_ERR_UNSUPPORTED;
  if (epilogue == QL_EPI_SWIGLU && N % 32 != 0) return QL_ERR_SHAPE;
  int st = validate_gemm_common(a, sa, w, sw, M, N, K, bias, out, ldo, epilogue);
  if (st != QL_OK) return st;
  // tensor / row scales keep one int32 accumulator over K
  if (a_scale_mode != QL_SCALE_GROUP64 && !acc_fits(K, a_layout == QL_LAYOUT_PACKED ? kProdW4A4P : kProdW4A4I8))
    return QL_ERR_SHAPE;
  if (rank < 0 || rank > 128 || rank % 16 != 0) return QL_ERR_SHAPE;
  if (rank > 0) {
    if (M > 0 && (!lr || !l2)) return QL_ERR_NULL;
    if (!al16(lr) || !al16(l2)) return QL_ERR_ALIGN;
  }
  if ((st = check_current_device()) != QL_OK) return st;
  if (M == 0) return QL_OK;
  ql::GemmArgs g{};
  g.a = a;
  g.w = w;
  g.sa = sa;
  g.sw = sw;
  g.M = M;
  g.N = N;
  g.K = K;
  g.a_packed = a_layout == QL_LAYOUT_PACKED;
  g.w_packed = 1;
  g.fp6 = fp6;
  g.a_mode = a_scale_mode;
  g.w_mode = w_scale_mode;
  g.bias = bias;
  g.lr = lr;
  g.l2 = l2;
  g.rank = rank;
  g.epilogue = epilogue;
  g.out = out;
  g.ldo = ldo;
  return ql::launch_qgemm(g, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

int qgemm_w4a4_lowrank(const void* a, const float* sa, int a_scale_mode, int a_layout, const uint8_t* w,
                       const float* sw, int w_scale_mode, const uint16_t* lr, const uint16_t* l2, int rank,
                       int64_t M, int64_t N, int64_t K, const uint16_t* bias, int epilogue, void* out,
                       int64_t ldo, void* stream) {
  if (!valid_mode(a_scale_mode) || !valid_mode(w_scale_mode)) return QL_ERR_UNSUPPORTED;
  if ((a_scale_mode == QL_SCALE_GROUP64) != (w_scale_mode == QL_SCALE_GROUP64)) return QL_ERR_UNSUPPORTED;
  if (a_layout != QL_LAYOUT_I8 && a_layout != QL_LAYOUT_PACKED) return QL_ERR_UNSUPPORTED;
  return lowrank_gemm(a, sa, a_scale_mode, a_layout, w, sw, w_scale_mode, lr, l2, rank, M, N, K, bias, epilogue,
                      out, ldo, stream, 0);
}

int qgemm_w4a4_fp6_lowrank(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                           const uint16_t* lr, const uint16_t* l2, int rank, int64_t M, int64_t N, int64_t K,
                           const uint16_t* bias, int epilogue, void* out, int64_t ldo, void* stream) {
  return lowrank_gemm(a, sa, QL_SCALE_GROUP64, QL_LAYOUT_FP6, w, sw, QL_SCALE_GROUP64, lr, l2, rank, M, N, K,
                      bias, epilogue, out, ldo, stream, 1);
}

int qgemm_grouped(const void* a4, const float* sa4, const void* a8, const float* sa8, int64_t M, int64_t K,
                  const ql_segment* segments, int nseg, void* stream) {
  if (!segments) return QL_ERR_NULL;
  if (nseg < 1 || nseg > QL_MAX_SEGMENTS) return QL_ERR_SHAPE;
  if (M < 0 || K <= 0 || K % 256 != 0) return QL_ERR_SHAPE;
  if (K >= (int64_t(1) << 23) || M >= (int64_t(1) << 36) / K) return QL_ERR_SHAPE;
  bool need4 = false, need8 = false;
  for (int i = 0; i < nseg; ++i) {
    const ql_segment& sg = segments[i];
    if (sg.w_bits != 4 && sg.w_bits != 8) return QL_ERR_UNSUPPORTED;
    if (sg.epilogue != QL_EPI_BF16 && sg.epilogue != QL_EPI_SIGMOID) return QL_ERR_UNSUPPORTED;
    if (sg.n <= 0 || sg.n % 16 != 0 || sg.n * K >= (int64_t(1) << 31)) return QL_ERR_SHAPE;
    if (!acc_fits(K, sg.w_bits == 8 ? kProdW8A8 : kProdW4A4I8)) return QL_ERR_SHAPE;
    if (sg.ldo < sg.n) return QL_ERR_SHAPE;
    if (M > 0 && (!sg.w || !sg.sw || !sg.out)) return QL_ERR_NULL;
    if (!al16(sg.w) || !al4(sg.sw) || !al16(sg.out) || (sg.ldo * 2) % 16 != 0) return QL_ERR_ALIGN;
    (sg.w_bits == 4 ? need4 : need8) = true;
  }
  if (M > 0 && ((need4 && (!a4 || !sa4)) || (need8 && (!a8 || !sa8)))) return QL_ERR_NULL;
  if (!al16(a4) || !al16(a8) || !al4(sa4) || !al4(sa8)) return QL_ERR_ALIGN;
  int st = check_current_device();
  if (st != QL_OK) return st;
  if (M == 0) return QL_OK;
  ql::GroupedArgs g{};
  g.a4 = a4;
  g.sa4 = sa4;
  g.a8 = a8;
  g.sa8 = sa8;
  g.M = M;
  g.K = K;
  g.nseg = nseg;
  for (int i = 0; i < nseg; ++i) {
    const ql_segment& src = segments[i];
    g.seg[i] = ql::GroupSegment{src.w, src.sw, src.n, src.w_bits, src.epilogue, src.out, src.ldo};
  }
  return ql::launch_qgemm_grouped(g, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

int64_t svdq_split_workspace_bytes(int64_t N, int64_t K, int rank, int oversample, int scale_mode) {
  if (N <= 0 || K <= 0 || K % 256 != 0 || rank <= 0 || oversample < 0 || !valid_mode(scale_mode)) return -1;
  return ql::svdq_split_workspace(N, K, rank, oversample, scale_mode);
}

static int validate_split(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, const float* act_rms,
                          const float* omega, int rank, int oversample, int power_iters, int refine_iters,
                          int scale_mode, uint16_t* l1, uint16_t* l2, uint8_t* packed, float* scales, float* errors,
                          int32_t* best_iter, float* sigma) {
  if (!valid_mode(scale_mode)) return QL_ERR_UNSUPPORTED;
  if (N <= 0 || N % 16 != 0 || K <= 0 || K % 256 != 0 || K > 32768) return QL_ERR_SHAPE;
  if (ldw < K || ldw % 8 != 0) return QL_ERR_SHAPE;
  if (rank < 16 || rank > 128 || rank % 16 != 0) return QL_ERR_SHAPE;
  if (oversample < 0 || oversample > 32) return QL_ERR_SHAPE;
  const int64_t l = rank + oversample;
  if (l > N || l > K) return QL_ERR_SHAPE;
  if (power_iters < 0 || power_iters > 8 || refine_iters < 0 || refine_iters > 16) return QL_ERR_SHAPE;
  // 32-bit-safe element counts for the one-thread-per-element kernels
  if (N * K >= (int64_t(1) << 31)) return QL_ERR_SHAPE;
  if (!w || !omega || !l1 || !l2 || !packed || !scales || !errors || !best_iter) return QL_ERR_NULL;
  if (!al16(w) || !al16(l1) || !al16(l2) || !al16(packed) || !al16(scales) || !al4(omega) || !al4(errors) ||
      !al4(best_iter) || (act_rms && !al4(act_rms)) || (sigma && !al16(sigma)))
    return QL_ERR_ALIGN;
  return QL_OK;
}

static int run_split(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, const float* act_rms, const float* omega,
                     int rank, int oversample, int power_iters, int refine_iters, int scale_mode, uint16_t* l1,
                     uint16_t* l2, uint8_t* packed, float* scales, float* errors, int32_t* best_iter, float* sigma,
                     void* workspace, void* stream) {
  ql::SplitArgs a{};
  a.w = w;
  a.N = N;
  a.K = K;
  a.ldw = ldw;
  a.act_rms = act_rms;
  a.omega = omega;
  a.rank = rank;
  a.oversample = oversample;
  a.power_iters = power_iters;
  a.refine_iters = refine_iters;
  a.scale_mode = scale_mode;
  a.l1 = l1;
  a.l2 = l2;
  a.packed = packed;
  a.scales = scales;
  a.errors = errors;
  a.best_iter = best_iter;
  a.sigma = sigma;
  a.workspace = workspace;
  return ql::launch_svdq_split(a, static_cast<hipStream_t>(stream)) == QL_OK ? QL_OK : QL_ERR_LAUNCH;
}

int svdq_split(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, const float* act_rms, const float* omega,
               int rank, int oversample, int power_iters, int refine_iters, int scale_mode, uint16_t* l1,
               uint16_t* l2, uint8_t* packed, float* scales, float* errors, int32_t* best_iter, float* sigma,
               void* workspace, int64_t workspace_bytes, void* stream) {
  int st = validate_split(w, N, K, ldw, act_rms, omega, rank, oversample, power_iters, refine_iters, scale_mode, l1,
                          l2, packed, scales, errors, best_iter, sigma);
  if (st != QL_OK) return st;
  if (!workspace) return QL_ERR_NULL;
  if (!al16(workspace)) return QL_ERR_ALIGN;
  if (workspace_bytes < ql::svdq_split_workspace(N, K, rank, oversample, scale_mode)) return QL_ERR_SHAPE;
  if ((st = check_current_device()) != QL_OK) return st;
  return run_split(w, N, K, ldw, act_rms, omega, rank, oversample, power_iters, refine_iters, scale_mode, l1, l2,
                   packed, scales, errors, best_iter, sigma, workspace, stream);
}

int svdq_split_noalloc(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, const float* act_rms,
                       const float* omega, int rank, int oversample, int power_iters, int refine_iters,
                       int scale_mode, uint16_t* l1, uint16_t* l2, uint8_t* packed, float* scales, float* errors,
                       int32_t* best_iter, float* sigma, void* stream) {
  int st = validate_split(w, N, K, ldw, act_rms, omega, rank, oversample, power_iters, refine_iters, scale_mode, l1,
                          l2, packed, scales, errors, best_iter, sigma);
  if (st != QL_OK) return st;
  if (ql::svdq_split_workspace(N, K, rank, oversample, scale_mode) > ql::kSplitScratchBytes) return QL_ERR_SCRATCH;
  if ((st = check_current_device()) != QL_OK) return st;
  void* ws = nullptr;
  if (ql::split_scratch(&ws) != QL_OK) return QL_ERR_DEVICE;
  return run_split(w, N, K, ldw, act_rms, omega, rank, oversample, power_iters, refine_iters, scale_mode, l1, l2,
                   packed, scales, errors, best_iter, sigma, ws, stream);
}

int64_t svdq_split_noalloc_max_bytes(void) { return ql::kSplitScratchBytes; }

}  // extern "C"
