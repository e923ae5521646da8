// Internal declarations shared by the HIP translation units of libqlinear.
// Not part of the public ABI (see include/qlinear.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

// ---------------------------------------------------------------- types ----
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// -------------------------------------------------------- bf16 helpers -----
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ------------------------------------------------------------ DPP -----------
// Cross-lane reads within 16-lane rows.  CTRL values follow the GFX9 DPP
// encoding: quad_perm = p0 | p1<<2 | p2<<4 | p3<<6, row_ror:n = 0x120 + n.
enum : int {
  DPP_QUAD_SWAP1 = 0xB1,  // quad_perm [1,0,3,2]
  DPP_QUAD_SWAP2 = 0x4E,  // quad_perm [2,3,0,1]
  DPP_ROR4 = 0x124,
  DPP_ROR8 = 0x128,
  DPP_ROR2 = 0x122,
  DPP_ROR1 = 0x121,
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// -------------------------------------------------- regular Hadamard -------
// H = H4 (x) H4 (x) H4 (x) H4 with H4 = J - 2I acts on the four base-4
// digits of the in-group channel index i = 64*d3 + 16*d2 + 4*d1 + d0.
// Applying H4 along one digit is the butterfly y = (sum of the 4 values
// that differ only in that digit) - 2*x.  A 16-lane DPP row owns one group;
// lane t holds the 16 consecutive channels i = 16*t + e.  Digits d0, d1
// come from e and are transformed in registers; digits d2 = t % 4 and
// d3 = t / 4 come from the lane and are transformed with DPP quad permutes
// and 16-lane row rotations.  Computes z = H x (no 1/16).  Every lane of the
// 16-lane row must be active.
__device__ __forceinline__ void hadamard256(float (&v)[16]) {
  // digit d0: e % 4
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float s = (v[4 * q] + v[4 * q + 1]) + (v[4 * q + 2] + v[4 * q + 3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[4 * q + i] = __builtin_fmaf(-2.0f, v[4 * q + i], s);
  }
  // digit d1: e / 4
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float s = (v[c] + v[c + 4]) + (v[c + 8] + v[c + 12]);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[c + 4 * i] = __builtin_fmaf(-2.0f, v[c + 4 * i], s);
  }
  // digit d2: lane bits 0-1 (the 4 lanes of a quad)
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float s1 = v[e] + dpp_f<DPP_QUAD_SWAP1>(v[e]);
    const float s = s1 + dpp_f<DPP_QUAD_SWAP2>(s1);
    v[e] = __builtin_fmaf(-2.0f, v[e], s);
  }
  // digit d3: lane bits 2-3 (lanes t, t+4, t+8, t+12 of the 16-lane row)
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float s1 = v[e] + dpp_f<DPP_ROR8>(v[e]);
    const float s = s1 + dpp_f<DPP_ROR4>(s1);
    v[e] = __builtin_fmaf(-2.0f, v[e], s);
  }
}

// ------------------------------------------------------- launch plumbing ---
// Status codes mirror include/qlinear.h.
enum { OK = 0, ERR_LAUNCH = -5 };

struct RqArgs {
  const uint16_t* x;
  int64_t M;
  int64_t K;
  int64_t ldx;
  int bits;        // 4 | 8
  int mode;        // 0 tensor, 1 row, 2 group64
  int packed;      // 0: int8 codes, 1: two int4 codes per byte, 2: FP6 e2m3 layout
  int rotate;      // 1: apply H per 256-group
  void* codes;
  float* scales;
  // RMSNorm + modulation in front (norm != 0): h = x * r * gamma * (1 + scale) + shift,
  // r = 1 / sqrt(mean(x^2) + eps); null vectors mean 1, 0, 0
  int norm;
  const uint16_t* gamma;
  const uint16_t* mscale;
  const uint16_t* mshift;
  float eps;
  // packed weights (packed == 1): rows 2p and 2p + 1 interleaved per
  // 128-channel slice (64 bytes each), the GEMM's weight order
  int paired;
};

int launch_rotate_quantize(const RqArgs& a, hipStream_t s);

// MX block quantization (mx_quant.hip): bf16 [M, K] -> optional group-256
// rotation -> E8M0 scale per 32 elements + FP4 / FP8 elements.
struct MxArgs {
  const uint16_t* x;
  int64_t M, K, ldx;
  int fmt;         // 4: FP4 E2M1, 8: FP8 E4M3
  int rotate;
  void* codes;     // [M, K/2] | [M, K] bytes, dense rows
  uint8_t* scales; // [K/128][M][4] (stage-major)
};
int launch_mx_quantize(const MxArgs& a, hipStream_t s);
int launch_lowrank_down(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        const uint16_t* l1, int rank, uint16_t* lr, hipStream_t s);

struct GemmArgs {
  const void* a;        // activation codes (int8 [M,K] or packed [M,K/2])
  const void* w;        // weight codes (int8 [N,K] or packed [N,K/2])
  const float* sa;
  const float* sw;
  int64_t M, N, K;
  int a_packed, w_packed;
  int fp6;              // 1: both operands in the FP6 e2m3 layout [rows, 3K/4]
  int mx;               // 4 / 8: both operands MX FP4 [rows, K/2] / FP8 [rows, K]
  const void* xa;       // MX: E8M0 scale bytes [K/128][M][4]
  const void* xw;       //     and [K/128][N][4]
  int a_mode, w_mode;   // 0 tensor, 1 row, 2 group64
  const uint16_t* bias;
  const uint16_t* residual;
  const uint16_t* gate;
  const uint16_t* lr;   // [M, rank]
  const uint16_t* l2;   // [N, rank] (L2 transposed)
  int rank;
  int epilogue;         // QL_EPI_*
  void* out;
  int64_t ldo;
};

// Every GEMM entry point: tensor / row / group-64 scales, all epilogues,
// optional low-rank branch.
int launch_qgemm(const GemmArgs& g, hipStream_t s);

// Grouped GEMM: up to kMaxGroupSegments projections of the same activations
// in one launch (packed int4 or int8 weights per segment, per-row scales,
// bf16 or sigmoid epilogue).
constexpr int kMaxGroupSegments = 8;
struct GroupSegment {
  const void* w;
  const float* sw;
  int64_t n;
  int w_bits;    // 4: packed int4 weights with the int4 activations; 8: int8 with int8
  int epilogue;  // 0 bf16, 5 sigmoid
  void* out;
  int64_t ldo;
};
struct GroupedArgs {
  const void* a4;
  const float* sa4;
  const void* a8;
  const float* sa8;
  int64_t M, K;
  int nseg;
  GroupSegment seg[kMaxGroupSegments];
};
int launch_qgemm_grouped(const GroupedArgs& g, hipStream_t s);

// Offline SVDQuant split (see svdq_split.hip).
struct SplitArgs {
  const uint16_t* w;      // bf16 [N, K], row stride ldw
  int64_t N, K, ldw;
  const float* act_rms;   // [K] or NULL
  const float* omega;     // [K, rank + oversample]
  int rank, oversample, power_iters, refine_iters, scale_mode;
  uint16_t* l1;           // [K, rank] bf16
  uint16_t* l2;           // [N, rank] bf16 (L2 transposed)
  uint8_t* packed;        // [N, K/2]
  float* scales;
  float* errors;          // [refine_iters + 1]
  int32_t* best_iter;     // [1]
  float* sigma;           // [rank] or NULL
  void* workspace;
};
int64_t svdq_split_workspace(int64_t N, int64_t K, int rank, int oversample, int scale_mode);
int launch_svdq_split(const SplitArgs& a, hipStream_t s);

// Allocation-free split: the workspace is a 128 MiB file-scope device array
// (one copy per GPU); split_scratch gives its address on the current device.
constexpr int64_t kSplitScratchBytes = int64_t(128) << 20;
int split_scratch(void** ptr);

}  // namespace ql
