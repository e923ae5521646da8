// MX block quantization of bf16 rows for gfx950: the activation prologue
// and the offline weight preparation of the block-scaled GEMM.
//
// The pages run the same model as an NVFP4 build on a GPU with native FP4
// matrix units (model card "Krea 2 Turbo Nunchaku Lite INT4 r32", section
// "Benchmark") and as an mxfp8 build (research log "lab", Study 1).  gfx950's
// block-scaled matrix instruction takes OCP MX operands -- 32-element blocks
// sharing one E8M0 scale -- so MXFP4 (E2M1 elements) is the MI355X
// counterpart of the FP4 build, MXFP8 (E4M3) of the mxfp8 one.
//
// Per block of 32 consecutive channels (OCP Microscaling Formats v1.0,
// conversion from wider formats):
//   e       = floor(log2 max|x|) - emax   (emax 2 for E2M1, 8 for E4M3),
//             clamped to [-127, 127]; -127 for an all-zero block
//   element = x / 2^e rounded to the nearest element value, ties to even,
//             saturating at the largest magnitude (6 | 448)
//   stored  : element bit patterns (every zero as +0) and the byte e + 127.
// Scale bytes are stored stage-major, [K/128][R][4]: for every 128-channel
// slice of K, the 4 block scales of row 0, then of row 1, ...  A GEMM tile
// then finds one slice's scales for consecutive rows in consecutive bytes.
//
// A 16-lane slot owns one 256-channel unit of a row; lane t holds channels
// 16 t .. 16 t + 15, so a block is the lane pair (2b, 2b + 1).  Units are
// visited row-fastest (unit u: row u % M, column group u / M), so the 16
// slots of a workgroup write the scales of 16 consecutive rows of a slice
// as 64 consecutive bytes; lanes 0 and 8 of a slot gather the 4 scales of
// their slice and store them as one dword.  With the
// rotation the slot first forms z = H x = 16 x' (hadamard256), so the block
// exponent of x' is that of max|z| minus 4 and x' / 2^e = z * 2^-(e + 4).
// The division by 2^e is an exact ldexp; the rounding is
// v_cvt_scalef32_pk_fp4_f32 / _pk_fp8_f32 with scale 1.  Measured on gfx950:
// both round to nearest even; the FP4 conversion saturates at 6, the FP8
// one turns magnitudes past 448 into NaN (so values are clamped to +-448
// first, which is the saturation); a negative value that rounds to zero
// keeps its sign bit, which is cleared here.

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int kMxThreads = 256;  // 16 slots of 16 lanes
constexpr int kMxMaxGrid = 8192;

typedef short v2s __attribute__((ext_vector_type(2)));

template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t old, float a, float b) {
  const v2s o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, old), a, b, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, o);
}

// Clear the sign of every zero element: an FP4 nibble 1000b / FP8 byte
// 0x80 becomes 0.  (low bits + all-ones-but-sign) carries into the sign
// position exactly when the low bits are nonzero, without crossing fields.
__device__ __forceinline__ uint32_t fp4_pos_zero(uint32_t w) {
  const uint32_t nz = (w & 0x77777777u) + 0x77777777u;
  return w ^ (w & ~nz & 0x88888888u);
}
__device__ __forceinline__ uint32_t fp8_pos_zero(uint32_t w) {
  const uint32_t nz = (w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
  return w ^ (w & ~nz & 0x80808080u);
}

template <int FMT, bool ROT>
__global__ __launch_bounds__(kMxThreads) void mx_quant_kernel(MxArgs a, int64_t units) {
  const int tid = threadIdx.x;
  const int slot = tid >> 4;
  const int t = tid & 15;
  constexpr int EMAX = FMT == 4 ? 2 : 8;
  for (int64_t base = (int64_t)blockIdx.x * 16; base < units; base += (int64_t)gridDim.x * 16) {
    // every lane of every slot runs the body (the butterflies read whole
    // 16-lane rows); lanes past the data hold zeros and store nothing
    const int64_t u = base + slot;
    const bool uok = u < units;
    const int64_t g = uok ? u / a.M : 0;
    const int64_t row = uok ? u - g * a.M : 0;
    const int64_t c0 = g * 256 + t * 16;  // the lane's first channel
    const bool ok = uok && c0 < a.K;
    uint4 r0 = make_uint4(0, 0, 0, 0), r1 = make_uint4(0, 0, 0, 0);
    if (ok) {
      const uint4* src = reinterpret_cast<const uint4*>(a.x + row * a.ldx + c0);
      r0 = src[0];
      r1 = src[1];
    }
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    float v[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
    if (ROT) hadamard256(v);

    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
    m = fmaxf(m, dpp_f<DPP_QUAD_SWAP1>(m));  // the block: lanes 2b, 2b + 1
    // floor(log2 m) = frexp exponent - 1
    int e = m > 0.0f ? __builtin_amdgcn_frexp_expf(m) - 1 - EMAX - (ROT ? 4 : 0) : -127;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    const int sh = -(e + (ROT ? 4 : 0));
    float s[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      s[k] = __builtin_amdgcn_ldexpf(v[k], sh);
      if (FMT == 8) s[k] = __builtin_amdgcn_fmed3f(s[k], -448.0f, 448.0f);
    }
    // scale bytes of blocks 4 (t / 8) .. + 3 gathered into lanes 0 and 8
    const int sb = e + 127;
    const int sb1 = __shfl_down(sb, 2, 16), sb2 = __shfl_down(sb, 4, 16), sb3 = __shfl_down(sb, 6, 16);
    if (!ok) continue;
    if ((t & 7) == 0)
      *reinterpret_cast<uint32_t*>(a.scales + (c0 / 128) * (a.M * 4) + row * 4) =
          (uint32_t)sb | ((uint32_t)sb1 << 8) | ((uint32_t)sb2 << 16) | ((uint32_t)sb3 << 24);
    if (FMT == 4) {
      uint32_t d0 = 0, d1 = 0;
      d0 = fp4_pair<0>(d0, s[0], s[1]);
      d0 = fp4_pair<1>(d0, s[2], s[3]);
      d0 = fp4_pair<2>(d0, s[4], s[5]);
      d0 = fp4_pair<3>(d0, s[6], s[7]);
      d1 = fp4_pair<0>(d1, s[8], s[9]);
      d1 = fp4_pair<1>(d1, s[10], s[11]);
      d1 = fp4_pair<2>(d1, s[12], s[13]);
      d1 = fp4_pair<3>(d1, s[14], s[15]);
      *reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.codes) + row * (a.K / 2) + c0 / 2) =
          make_uint2(fp4_pos_zero(d0), fp4_pos_zero(d1));
    } else {
      uint32_t d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t x = 0;
        x = fp8_pair<false>(x, s[4 * q], s[4 * q + 1]);
        x = fp8_pair<true>(x, s[4 * q + 2], s[4 * q + 3]);
        d[q] = fp8_pos_zero(x);
      }
      *reinterpret_cast<uint4*>(static_cast<uint8_t*>(a.codes) + row * a.K + c0) = make_uint4(d[0], d[1], d[2], d[3]);
    }
  }
}

template <int FMT, bool ROT>
int launch_fmt(const MxArgs& a, hipStream_t s) {
  const int64_t upr = a.K / 256;
  const int64_t units = a.M * upr;
  const int64_t blocks = (units + 15) / 16;
  const int grid = (int)(blocks < kMxMaxGrid ? blocks : kMxMaxGrid);
  hipLaunchKernelGGL((mx_quant_kernel<FMT, ROT>), dim3(grid), dim3(kMxThreads), 0, s, a, units);
  return hipGetLastError() == hipSuccess ? OK : ERR_LAUNCH;
}

}  // namespace

int launch_mx_quantize(const MxArgs& a, hipStream_t s) {
  if (a.M == 0) return OK;
  if (a.fmt == 4) return a.rotate ? launch_fmt<4, true>(a, s) : launch_fmt<4, false>(a, s);
  return a.rotate ? launch_fmt<8, true>(a, s) : launch_fmt<8, false>(a, s);
}

}  // namespace ql
