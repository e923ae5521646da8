// Online rotation + dynamic symmetric quantization (activations), offline
// weight packing, and the SVDQuant low-rank down-projection, for gfx950.
//
// Method (model card "Krea-2 Turbo -- INT4 tensorwise W4A4 (+ConvRot, mixed
// int8 fallback)", introduction): each aligned 256-channel group is rotated
// by a regular Hadamard matrix and the result is quantized to signed INT4 or
// INT8 with a scale computed at run time from the absolute maximum.
//
// Rotation.  H = H4 (x) H4 (x) H4 (x) H4 with H4 = J - 2I acts on the four
// base-4 digits of the in-group channel index i = 64*d3 + 16*d2 + 4*d1 + d0.
// Applying H4 along one digit is the butterfly y = (sum of the 4 values that
// differ only in that digit) - 2*x.  A 16-lane DPP row owns one group; lane
// t holds the 16 consecutive channels i = 16*t + e.  Digits d0, d1 come from
// e and are transformed in registers; digits d2 = t % 4 and d3 = t / 4 come
// from the lane and are transformed with DPP quad permutes and 16-lane row
// rotations.  The kernel forms z = H x (no 1/16): the codes do not depend on
// a power-of-two factor, and the 1/16 is folded into the stored scale
// exactly.
//
// Quantization (per tensor, per row, or per row x 64-channel group):
//   amax = max |z| over the unit,  inv = qmax / amax (correctly rounded fp32),
//   code = rint(z * inv) (already within [-qmax, qmax]),  scale = amax / qmax (/16 if rotated);
//   unrotated bf16 inputs take the correctly rounded quotient rint((x * qmax) / amax).
// A 64-channel group inside a 256-group is one value of d3, i.e. one quad of
// lanes.

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int kThreads = 256;  // 16 slots of 16 lanes

__device__ __forceinline__ float row16_max(float m) {
  m = fmaxf(m, dpp_f<DPP_ROR8>(m));
  m = fmaxf(m, dpp_f<DPP_ROR4>(m));
  m = fmaxf(m, dpp_f<DPP_ROR2>(m));
  m = fmaxf(m, dpp_f<DPP_ROR1>(m));
  return m;
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<DPP_ROR8>(v);
  v += dpp_f<DPP_ROR4>(v);
  v += dpp_f<DPP_ROR2>(v);
  v += dpp_f<DPP_ROR1>(v);
  return v;
}

// Position of channel c in the LDS copy of a per-channel vector: lane t of a
// 16-lane slot reads the 16 channels 16 t .. 16 t + 15 of a 256-group as four
// 16-byte pieces, piece q stored at q ^ (t / 4) so one ds_read_b128 by the
// 16 lanes touches every bank once.
__device__ __forceinline__ int nvec_pos(int c) {
  const int t = (c >> 4) & 15, q = (c >> 2) & 3;
  return (c & ~15) + ((q ^ (t >> 2)) << 2) + (c & 3);
}

__device__ __forceinline__ float quad_max(float m) {
  m = fmaxf(m, dpp_f<DPP_QUAD_SWAP1>(m));
  m = fmaxf(m, dpp_f<DPP_QUAD_SWAP2>(m));
  return m;
}

// Round to nearest integer, ties to even, for |x| < 2^22: adding 1.5 * 2^23
// leaves the rounded integer in the low mantissa bits, so the low byte of
// the sum's bit pattern is the code in two's complement.  The product and
// the sum are separate correctly rounded operations (no fusion).
__device__ __forceinline__ uint32_t code_bits(float x, float inv) {
#pragma clang fp contract(off)
  const float prod = x * inv;
  return __float_as_uint(prod + 12582912.0f);
}

// Bytes 0 of a, b, c, d -> one dword [a, b, c, d].
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // a.b0 | b.b0 << 8
  const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000c0cu);  // c.b0 << 16 | d.b0 << 24
  return lo | hi;
}

// Four int4 codes (bytes of x, two's complement, |c| <= 7) -> their FP6
// e2m3 bit patterns, one per byte.  |c| indexes the 8 magnitude patterns
// {0, 8, 16, 20, 24, 26, 28, 30} (1 = 1.0 * 2^0, 2..3 = 1.m * 2^1, 4..7 =
// 1.m * 2^2 with exponent bias 1) through one byte permute; bit 5 is the sign.
__device__ __forceinline__ uint32_t fp6_bytes(uint32_t x) {
  const uint32_t neg = (x >> 7) & 0x01010101u;          // 1 in each negative byte
  const uint32_t mag = (x ^ (neg * 0xFFu)) + neg;       // per-byte |c| (no carries: |c| <= 7)
  return __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, mag) | (neg << 5);
}

// Four 6-bit patterns (one per byte) -> 24 contiguous bits, byte i at bits 6i.
__device__ __forceinline__ uint32_t fp6_join4(uint32_t p) {
  return (p & 0x3Fu) | ((p >> 2) & 0xFC0u) | ((p >> 4) & 0x3F000u) | ((p >> 6) & 0xFC0000u);
}

// Encode 16 codes (channel order, as code_bits) and store them: fmt 0 int8,
// 1 packed int4, 2 FP6 e2m3 layout (every lane of the 16-lane slot active).
// int8-container codes leave with nontemporal stores: one instruction writes
// whole lines, the codes are read back only by the next kernel, and the
// prologue runs 11 % faster (the prologue + GEMM step ~1 %).  The packed and
// FP6 layouts keep plain stores: an FP6 block is written by two instructions
// (16- and 8-byte pieces), and as nontemporal partial lines those cost
// 8.5 us per 4096 x 5120 step.
// pair_k != 0 (packed weights): rows 2p and 2p + 1 interleaved per 128-channel
// slice -- channel c of row r at byte (r / 2) K + 128 (c / 128) + 64 (r % 2)
// + (c % 128) / 2 (K = pair_k); a lane's 16 channels never cross a slice.
// FP6 (pair_k = K, rows = R): rows in fours per 128-channel block, the last
// R % 4 rows plain (the QL_LAYOUT_FP6 row order).
__device__ __forceinline__ void store_codes(void* codes, int64_t off_elems, int fmt, const uint32_t (&u)[16],
                                            int64_t pair_k = 0, int64_t rows = 0) {
  if (fmt == 2) {
    // FP6 layout: a row is 96-byte blocks of 128 channels; in a block,
    // 32-channel sub-block g is the 192-bit value v_g (channel i at bits
    // 6i), its low 16 bytes at 16 g and its high 8 bytes at 64 + 8 g.  A
    // lane's 16 channels are bits 0..95 (even lane) or 96..191 (odd lane)
    // of one v_g, so the even lane stores the low 16 bytes with the first
    // dword of its odd neighbour and the odd lane the high 8 bytes.
    const uint32_t w0 = fp6_join4(fp6_bytes(pack4(u[0], u[1], u[2], u[3])));
    const uint32_t w1 = fp6_join4(fp6_bytes(pack4(u[4], u[5], u[6], u[7])));
    const uint32_t w2 = fp6_join4(fp6_bytes(pack4(u[8], u[9], u[10], u[11])));
    const uint32_t w3 = fp6_join4(fp6_bytes(pack4(u[12], u[13], u[14], u[15])));
    const uint32_t d0 = w0 | (w1 << 24), d1 = (w1 >> 8) | (w2 << 16), d2 = (w2 >> 16) | (w3 << 8);
    const uint32_t nd0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d0, DPP_QUAD_SWAP1, 0xF, 0xF, false);
    const int64_t c = off_elems & 127;                 // channel within the 128-channel block
    uint8_t* blk = static_cast<uint8_t*>(codes) + (off_elems >> 7) * 96;
    // rows 4q .. 4q + 3 interleaved per 128-channel slice (96 bytes each,
    // 384 bytes: three whole cache lines); the last rows % 4 rows stay plain
    // (pair_k: the row length K; rows: the matrix's row count)
    if (pair_k > 0) {
      const int64_t r = off_elems / pair_k, cc = off_elems - r * pair_k;
      if (r < (rows & ~int64_t(3)))
        blk = static_cast<uint8_t*>(codes) + (r >> 2) * (pair_k / 128 * 384) + (cc >> 7) * 384 + (r & 3) * 96;
    }
    const int g = (int)(c >> 5);
    if ((c & 16) == 0) *reinterpret_cast<uint4*>(blk + 16 * g) = make_uint4(d0, d1, d2, nd0);
    else *reinterpret_cast<uint2*>(blk + 64 + 8 * g) = make_uint2(d1, d2);
    return;
  }
  if (fmt == 0) {
    const v4u w{pack4(u[0], u[1], u[2], u[3]), pack4(u[4], u[5], u[6], u[7]), pack4(u[8], u[9], u[10], u[11]),
                pack4(u[12], u[13], u[14], u[15])};
    __builtin_nontemporal_store(w, reinterpret_cast<v4u*>(static_cast<int8_t*>(codes) + off_elems));
  } else {
    // byte 4c+j: low nibble channel 8c+j, high nibble channel 8c+j+4
    const uint32_t l0 = pack4(u[0], u[1], u[2], u[3]), h0 = pack4(u[4], u[5], u[6], u[7]);
    const uint32_t l1 = pack4(u[8], u[9], u[10], u[11]), h1 = pack4(u[12], u[13], u[14], u[15]);
    int64_t byte = off_elems / 2;
    if (pair_k) {
      const int64_t r = off_elems / pair_k, c = off_elems - r * pair_k;
      byte = (r >> 1) * pair_k + ((c >> 7) << 7) + ((r & 1) << 6) + ((c & 127) >> 1);
    }
    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(codes) + byte) =
        make_uint2((l0 & 0x0F0F0F0Fu) | ((h0 << 4) & 0xF0F0F0F0u), (l1 & 0x0F0F0F0Fu) | ((h1 << 4) & 0xF0F0F0F0u));
  }
}

// One workgroup handles blocks of rows_per_wg rows, slots_per_row 16-lane
// slots per row, GPL groups per slot; it loops over blocks blockIdx.x,
// blockIdx.x + gridDim.x, ... (one block each unless the grid is capped).
// phase 0: quantize (row / group64, or tensor mode reading the absmax cell)
// phase 1: tensor mode, absmax only (atomicMax into the cell)
// NORM: the RMSNorm + modulation of model card "Krea 2 Turbo OrbitQuant
// W4A4", section "Fused transformer (OrbitQuant 0.11)" (the block's norm and
// modulation run inside the activation quantization prologue), read as
//   h = x * r * gamma * (1 + scale) + shift,  r = 1 / sqrt(mean_k x^2 + eps)
// per row, with per-channel bf16 vectors; h stays in fp32 and is rotated and
// quantized in place of x.  The workgroup first stages g = gamma * (1 + scale)
// and shift as fp32 in dynamic LDS (8 K bytes).
template <int GPL, bool NORM>
__global__ __launch_bounds__(kThreads) void rq_kernel(RqArgs a, int slots_per_row, int rows_per_wg,
                                                      int phase, int64_t nblocks) {
  __shared__ float red[2][16];
  __shared__ float sred[NORM ? 2 : 1][16];
  extern __shared__ float nvec[];  // NORM: g at [0, K), shift at [K, 2K), nvec_pos order
  const int tid = threadIdx.x;
  const int slot = tid >> 4;
  const int t = tid & 15;
  const int row_in_wg = slot / slots_per_row;
  const int sir = slot - row_in_wg * slots_per_row;
  const int ngroups = (int)(a.K >> 8);
  const float qmax = a.bits == 4 ? 7.0f : 127.0f;
  const float post = a.rotate ? 0.0625f : 1.0f;  // z = 16 x' when rotated

  if (NORM) {
    const int K = (int)a.K;
    for (int c8 = tid; c8 < K / 8; c8 += kThreads) {
      const uint4 gw = a.gamma ? reinterpret_cast<const uint4*>(a.gamma)[c8] : make_uint4(0, 0, 0, 0);
      const uint4 sw = a.mscale ? reinterpret_cast<const uint4*>(a.mscale)[c8] : make_uint4(0, 0, 0, 0);
      const uint4 bw = a.mshift ? reinterpret_cast<const uint4*>(a.mshift)[c8] : make_uint4(0, 0, 0, 0);
      const uint32_t g2[4] = {gw.x, gw.y, gw.z, gw.w}, s2[4] = {sw.x, sw.y, sw.z, sw.w},
                     b2[4] = {bw.x, bw.y, bw.z, bw.w};
      float gv[8], bv[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float g0 = a.gamma ? __uint_as_float(g2[k] << 16) : 1.0f;
        const float g1 = a.gamma ? __uint_as_float(g2[k] & 0xffff0000u) : 1.0f;
        gv[2 * k] = g0 * (1.0f + __uint_as_float(s2[k] << 16));
        gv[2 * k + 1] = g1 * (1.0f + __uint_as_float(s2[k] & 0xffff0000u));
        bv[2 * k] = __uint_as_float(b2[k] << 16);
        bv[2 * k + 1] = __uint_as_float(b2[k] & 0xffff0000u);
      }
      // channels 8 c8 .. 8 c8 + 7: two 4-channel pieces
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = nvec_pos(8 * c8 + 4 * h);
        *reinterpret_cast<float4*>(nvec + p) = make_float4(gv[4 * h], gv[4 * h + 1], gv[4 * h + 2], gv[4 * h + 3]);
        *reinterpret_cast<float4*>(nvec + K + p) =
            make_float4(bv[4 * h], bv[4 * h + 1], bv[4 * h + 2], bv[4 * h + 3]);
      }
    }
    __syncthreads();
  }

  uint4 raw[GPL][2];
  auto load = [&](int64_t blk) {
    const int64_t row = blk * rows_per_wg + row_in_wg;
    const bool row_ok = (row_in_wg < rows_per_wg) && (row < a.M);
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int g = sir + j * slots_per_row;
      if (row_ok && g < ngroups) {
        const uint4* p = reinterpret_cast<const uint4*>(a.x + row * a.ldx + (int64_t)g * 256 + t * 16);
        raw[j][0] = p[0];
        raw[j][1] = p[1];
      } else {
        raw[j][0] = make_uint4(0, 0, 0, 0);
        raw[j][1] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  int it = 0;
  for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x, ++it) {
    const int64_t row = blk * rows_per_wg + row_in_wg;
    const bool row_ok = (row_in_wg < rows_per_wg) && (row < a.M);
    load(blk);
    float v[GPL][16];
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const uint32_t w[8] = {raw[j][0].x, raw[j][0].y, raw[j][0].z, raw[j][0].w,
                             raw[j][1].x, raw[j][1].y, raw[j][1].z, raw[j][1].w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[j][2 * k] = __uint_as_float(w[k] << 16);
        v[j][2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }

    if (NORM) {
      // mean square of the row: lane partials, the 16-lane slot, then the
      // row's slots through LDS (fixed order)
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < GPL; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) ss = __builtin_fmaf(v[j][e], v[j][e], ss);
      ss = row16_sum(ss);
      float* sb = sred[NORM ? (it & 1) : 0];
      if (t == 0) sb[slot] = ss;
      __syncthreads();
      float rs = 0.0f;
      const int s0 = row_in_wg * slots_per_row;
      for (int s2 = 0; s2 < slots_per_row; ++s2) rs += sb[(s0 + s2) & 15];
      const float r = __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(rs, (float)a.K) + a.eps));
#pragma unroll
      for (int j = 0; j < GPL; ++j) {
        const int g = sir + j * slots_per_row;
        if (g >= ngroups) continue;  // those lanes hold zeros and are never stored
        const float* gp = nvec + g * 256 + t * 16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int pq = (q ^ (t >> 2)) << 2;
          const float4 gq = *reinterpret_cast<const float4*>(gp + pq);
          const float4 bq = *reinterpret_cast<const float4*>(gp + a.K + pq);
          v[j][4 * q] = __builtin_fmaf(v[j][4 * q] * r, gq.x, bq.x);
          v[j][4 * q + 1] = __builtin_fmaf(v[j][4 * q + 1] * r, gq.y, bq.y);
          v[j][4 * q + 2] = __builtin_fmaf(v[j][4 * q + 2] * r, gq.z, bq.z);
          v[j][4 * q + 3] = __builtin_fmaf(v[j][4 * q + 3] * r, gq.w, bq.w);
        }
      }
    }

    if (a.rotate) {
#pragma unroll
      for (int j = 0; j < GPL; ++j) hadamard256(v[j]);
    }

    // per-unit absmax
    float amax[GPL];
    if (a.mode == 2) {  // group64: one quad of lanes per 64-channel group
#pragma unroll
      for (int j = 0; j < GPL; ++j) {
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[j][e]));
        amax[j] = quad_max(m);
      }
    } else {  // row or tensor: reduce over the row's slots
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < GPL; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[j][e]));
      m = row16_max(m);
      float* rb = red[it & 1];  // alternate buffers: one barrier per block
      if (t == 0) rb[slot] = m;
      __syncthreads();
      if (phase == 1) {
        if (tid == 0) {
          float wm = 0.0f;
          for (int s2 = 0; s2 < 16; ++s2) wm = fmaxf(wm, rb[s2]);
          atomicMax(reinterpret_cast<unsigned int*>(a.scales), __float_as_uint(wm));
        }
        continue;
      }
      float rm;
      if (a.mode == 0) {
        rm = __uint_as_float(*reinterpret_cast<const volatile unsigned int*>(a.scales));
      } else {
        rm = 0.0f;
        const int s0 = row_in_wg * slots_per_row;
        for (int s2 = 0; s2 < slots_per_row; ++s2) rm = fmaxf(rm, rb[(s0 + s2) & 15]);
      }
#pragma unroll
      for (int j = 0; j < GPL; ++j) amax[j] = rm;
    }

    if (!row_ok) continue;

    // |z * inv| <= qmax (1 + 2^-23) since |z| <= amax, so the rounded code
    // never leaves [-qmax, qmax] and needs no clamp.
    // Unrotated bf16 inputs: x * qmax is exact in fp32 (8 + 7 significant
    // bits) and amax is a bf16 value, so the correctly rounded quotient
    // (x * qmax) / amax rounds to the same code as the exact one: it is the
    // exact k + 1/2 at a tie (which then goes to even), and otherwise lies more
    // than 2^7 half-ulps from any tie.  A reciprocal product would break
    // exact ties (x = 3, amax = 6) either way.  Rotated or normalized values
    // carry the fp32 error of the butterflies anyway and keep the product.
    const bool exact_in = !NORM && !a.rotate;
    const int64_t code_row = row * a.K;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int g = sir + j * slots_per_row;
      if (g >= ngroups) continue;
      const float am = amax[j];
      const float inv = am > 0.0f ? __fdiv_rn(qmax, am) : 0.0f;
      uint32_t u[16];
      if (exact_in) {
#pragma unroll
        for (int e = 0; e < 16; ++e) u[e] = code_bits(am > 0.0f ? __fdiv_rn(v[j][e] * qmax, am) : 0.0f, 1.0f);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) u[e] = code_bits(v[j][e], inv);
      }
      store_codes(a.codes, code_row + (int64_t)g * 256 + t * 16, a.packed, u,
                  (a.paired || a.packed == 2) ? a.K : 0, a.M);
      if (a.mode == 2) {
        if ((t & 3) == 0)
          a.scales[(int64_t)(g * 4 + (t >> 2)) * a.M + row] = __fdiv_rn(am, qmax) * post;  // [K/64, M]
      } else if (a.mode == 1 && t == 0 && sir == 0 && j == 0) {
        a.scales[row] = __fdiv_rn(am, qmax) * post;
      }
    }
  }
}

__global__ void cell_clear_kernel(float* cell) { *reinterpret_cast<unsigned int*>(cell) = 0u; }

__global__ void cell_finalize_kernel(float* cell, float qmax, float post) {
  const float am = *cell;
  *cell = __fdiv_rn(am, qmax) * post;
}

struct Plan {
  int gpl, slots, rows;
};

Plan plan_rows(int ngroups) {
  static const int cand[] = {1, 2, 3, 4, 5, 6, 8};
  Plan best{0, 0, 0};
  double best_eff = -1.0;
  for (int g : cand) {
    const int s = (ngroups + g - 1) / g;
    if (s > 16) continue;
    const int rows = 16 / s;
    const double eff = (double)(rows * s) / 16.0 * (double)ngroups / (double)(s * g);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = Plan{g, s, rows};
    }
  }
  return best;
}

// Workgroups launched at most (16 per CU of MI355X); larger inputs loop.
constexpr int64_t kRqMaxGrid = 4096;

// With the norm fused in, every workgroup first stages the per-channel
// vectors, so fewer workgroups loop over more rows.
constexpr int64_t kRqNormMaxGrid = 512;

template <int GPL>
hipError_t launch_rq(const RqArgs& a, const Plan& p, int phase, hipStream_t s) {
  const int64_t nblocks = (a.M + p.rows - 1) / p.rows;
  const int64_t cap = a.norm ? kRqNormMaxGrid : kRqMaxGrid;
  const unsigned grid = (unsigned)(nblocks < cap ? nblocks : cap);
  if (a.norm) {
    hipLaunchKernelGGL((rq_kernel<GPL, true>), dim3(grid), dim3(kThreads), (size_t)(8 * a.K), s, a, p.slots,
                       p.rows, phase, nblocks);
  } else {
    hipLaunchKernelGGL((rq_kernel<GPL, false>), dim3(grid), dim3(kThreads), 0, s, a, p.slots, p.rows, phase,
                       nblocks);
  }
  return hipGetLastError();
}

hipError_t dispatch_rq(const RqArgs& a, const Plan& p, int phase, hipStream_t s) {
  switch (p.gpl) {
    case 1: return launch_rq<1>(a, p, phase, s);
    case 2: return launch_rq<2>(a, p, phase, s);
    case 3: return launch_rq<3>(a, p, phase, s);
    case 4: return launch_rq<4>(a, p, phase, s);
    case 5: return launch_rq<5>(a, p, phase, s);
    case 6: return launch_rq<6>(a, p, phase, s);
    case 8: return launch_rq<8>(a, p, phase, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// SVDQuant down-projection lr = bf16(X @ L1) with the unrotated bf16 X
// (README "Krea-2-SVDQuant-ComfyUI", section "Low-rank refinement": the
// branch is a small full-precision product next to the quantized weight).
//
// The product is skinny (rank <= 128) and bound by reading X once.  One
// workgroup per 16 rows; its 8 waves split K into eighths, so a 4096-row X
// gives 256 workgroups x 8 waves.  bf16 MFMA 16x16x32, fp32 accumulation:
// the first operand is a 16-rank block of L1^T (8 consecutive k of one L1
// column per lane), the second the 16 rows of X (one 16-byte load per lane
// per 32 channels).  A step's 32 L1 rows are one contiguous block of the
// [K, rank] matrix: the wave loads it with coalesced 16-byte loads into its
// own LDS slice and reads the columns back as 2-byte values (the four 8-row
// groups sit 32 bytes apart, so one read's 64 lanes hit 32 distinct banks).
// X is loaded four steps ahead and L1 two, so the loads of later steps are
// in flight while a step computes.  The eight partial sums meet in LDS.
// ---------------------------------------------------------------------------
constexpr int kLrWaves = 8;

// 16-byte L1 loads of step st (clamped to the last step): the step's
// 32 x rank block is contiguous; lane loads chunks lane + 64 i
template <int NB>
__device__ __forceinline__ void lr_load_l(v4u (&dst)[NB], const uint8_t* lb, int st, int nit, int lane) {
  const int ss = st < nit ? st : nit - 1;
  const uint8_t* b = lb + (int64_t)ss * 64 * (16 * NB);
#pragma unroll
  for (int i = 0; i < NB; ++i) dst[i] = *reinterpret_cast<const v4u*>(b + (lane + 64 * i) * 16);
}

__device__ __forceinline__ v4u lr_load_x(const uint16_t* xp, int st, int nit) {
  const int ss = st < nit ? st : nit - 1;
  return *reinterpret_cast<const v4u*>(xp + (int64_t)ss * 32);
}

// one 32-channel step: L1 chunks (lcur) through the wave's LDS slice into
// the MFMA's first operand, X fragment (xcur) as the second; lcur and xcur
// then take the loads of steps st + 2 and st + 4.  The wave's LDS
// operations run in order: the step's reads follow its writes, and the next
// step's writes follow these reads.
template <int NB>
__device__ __forceinline__ void lr_step(v4u (&lcur)[NB], v4u& xcur, v4f (&acc)[NB], const int (&woff)[NB],
                                        uint8_t* sl, int rbase, const uint8_t* lb, const uint16_t* xp, int st,
                                        int nit, int lane) {
  constexpr int rank = 16 * NB;
#pragma unroll
  for (int i = 0; i < NB; ++i) *reinterpret_cast<v4u*>(sl + woff[i]) = lcur[i];
  lr_load_l<NB>(lcur, lb, st + 2, nit, lane);
  const v8bf xf = __builtin_bit_cast(v8bf, xcur);
  xcur = lr_load_x(xp, st + 4, nit);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const uint16_t* rp = reinterpret_cast<const uint16_t*>(sl + rbase + j * 32);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)rp[(2 * e) * rank] | ((uint32_t)rp[(2 * e + 1) * rank] << 16);
    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3])),
                                                     xf, acc[j], 0, 0, 0);
  }
}

// NB = rank / 16
template <int NB>
__global__ __launch_bounds__(64 * kLrWaves) void lowrank_down_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, const uint16_t* __restrict__ l1,
    uint16_t* __restrict__ lr) {
  constexpr int rank = 16 * NB;
  constexpr int cpr = 2 * NB;                        // 16-byte chunks per L1 row
  constexpr int kSlice = 32 * rank * 2 + 4 * 32;     // bytes of a wave's L1 block in LDS
  __shared__ float part[kLrWaves][16 * rank];
  __shared__ __align__(16) uint8_t slice[kLrWaves][kSlice];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  int64_t arow = m0 + l16;
  if (arow > M - 1) arow = M - 1;
  const int64_t kw = K / kLrWaves;  // multiple of 32 (K is a multiple of 256)
  const int64_t kbeg = wave * kw;
  const int nit = (int)(kw >> 5);
  const uint16_t* xp = x + arow * ldx + kbeg + lg * 8;
  const uint8_t* lb = reinterpret_cast<const uint8_t*>(l1 + kbeg * rank);
  uint8_t* sl = slice[wave];
  // chunk q = lane + 64 i of a step's block: row q / cpr, chunk q % cpr
  int woff[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int q = lane + 64 * i;
    const int k = q / cpr;
    woff[i] = k * 2 * rank + (k >> 3) * 32 + (q - k * cpr) * 16;
  }
  // lane reads rows 8 lg + t (t < 8) at rank 16 j + l16
  const int rbase = lg * 8 * 2 * rank + lg * 32 + l16 * 2;

  v4f acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  v4u x0 = lr_load_x(xp, 0, nit), x1 = lr_load_x(xp, 1, nit), x2 = lr_load_x(xp, 2, nit),
        x3 = lr_load_x(xp, 3, nit);
  v4u la[NB], lc[NB];
  lr_load_l<NB>(la, lb, 0, nit, lane);
  lr_load_l<NB>(lc, lb, 1, nit, lane);
  int s0 = 0;
  for (; s0 + 4 <= nit; s0 += 4) {
    lr_step<NB>(la, x0, acc, woff, sl, rbase, lb, xp, s0, nit, lane);
    lr_step<NB>(lc, x1, acc, woff, sl, rbase, lb, xp, s0 + 1, nit, lane);
    lr_step<NB>(la, x2, acc, woff, sl, rbase, lb, xp, s0 + 2, nit, lane);
    lr_step<NB>(lc, x3, acc, woff, sl, rbase, lb, xp, s0 + 3, nit, lane);
  }
  // last nit % 4 steps: operands loaded in place (the ring's registers would
  // need a step-dependent choice, which the compiler turns into scratch)
  for (; s0 < nit; ++s0) {
    v4u lt[NB];
    lr_load_l<NB>(lt, lb, s0, nit, lane);
    v4u xt = lr_load_x(xp, s0, nit);
    lr_step<NB>(lt, xt, acc, woff, sl, rbase, lb, xp, s0, nit, lane);
  }
  // lane holds ranks 16 j + 4 lg + r of row m0 + l16
#pragma unroll
  for (int j = 0; j < NB; ++j) *reinterpret_cast<v4f*>(&part[wave][l16 * rank + j * 16 + lg * 4]) = acc[j];
  __syncthreads();
  for (int o = tid; o < 16 * rank; o += 64 * kLrWaves) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kLrWaves; ++w) sum += part[w][o];
    const int64_t m = m0 + o / rank;
    if (m < M) lr[m * rank + o % rank] = (uint16_t)f32_to_bf16(sum);
  }
}

}  // namespace

int launch_rotate_quantize(const RqArgs& a, hipStream_t s) {
  if (a.M == 0) return OK;
  const Plan p = plan_rows((int)(a.K >> 8));
  if (p.gpl == 0) return ERR_LAUNCH;
  const float qmax = a.bits == 4 ? 7.0f : 127.0f;
  hipError_t e;
  if (a.mode == 0) {
    hipLaunchKernelGGL(cell_clear_kernel, dim3(1), dim3(1), 0, s, a.scales);
    if ((e = hipGetLastError()) != hipSuccess) return ERR_LAUNCH;
    if ((e = dispatch_rq(a, p, 1, s)) != hipSuccess) return ERR_LAUNCH;
    if ((e = dispatch_rq(a, p, 0, s)) != hipSuccess) return ERR_LAUNCH;
    hipLaunchKernelGGL(cell_finalize_kernel, dim3(1), dim3(1), 0, s, a.scales, qmax,
                       a.rotate ? 0.0625f : 1.0f);
    if ((e = hipGetLastError()) != hipSuccess) return ERR_LAUNCH;
    return OK;
  }
  return dispatch_rq(a, p, 0, s) == hipSuccess ? OK : ERR_LAUNCH;
}

int launch_lowrank_down(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* l1,
                        int rank, uint16_t* lr, hipStream_t s) {
  if (M == 0) return OK;
  const unsigned blocks = (unsigned)((M + 15) / 16);
  switch (rank >> 4) {
#define QL_LR_CASE(nb)                                                                                      \
  case nb:                                                                                                  \
    hipLaunchKernelGGL(lowrank_down_kernel<nb>, dim3(blocks), dim3(64 * kLrWaves), 0, s, x, M, K, ldx, l1, lr); \
    break;
    QL_LR_CASE(1) QL_LR_CASE(2) QL_LR_CASE(3) QL_LR_CASE(4) QL_LR_CASE(5) QL_LR_CASE(6) QL_LR_CASE(7) QL_LR_CASE(8)
#undef QL_LR_CASE
    default: return ERR_LAUNCH;  // the API admits ranks 16..128 in steps of 16 only
  }
  return hipGetLastError() == hipSuccess ? OK : ERR_LAUNCH;
}

}  // namespace ql
