// Internal declarations shared by the HIP translation units of libqlinear.
// Not part of the public ABI (see include/qlinear.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

// ---------------------------------------------------------------- types ----
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
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
};

int launch_rotate_quantize(const RqArgs& a, hipStream_t s);
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
  int a_mode, w_mode;   // 0 tensor, 1 row, 2 group64
  const uint16_t* bias;
  const uint16_t* residual;
  const uint16_t* gate;
  const uint16_t* lr;   // [M, rank]
  const uint16_t* l2;   // [rank, N]
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

}  // namespace ql
