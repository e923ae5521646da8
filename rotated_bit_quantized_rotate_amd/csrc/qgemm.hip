// Integer GEMM with exact int32 accumulation on gfx950 int8 MFMA, plus the
// dequantize epilogues of the rotated low-bit linear.
//
//   acc[m, n] = sum_k qa[m, k] * qw[n, k]                 (exact, int32)
//   y[m, n]   = acc * s_a * s_w            (tensor / row scales)
//             = sum_g acc_g * s_a[m,g] * s_w[n,g]   (group-64 scales, fp32 sum)
//   (+ bias[n]) (+ sum_r lr[m,r] * L2[r,n])  -> epilogue -> out
//
// (model card "Krea 2 Turbo OrbitQuant W4A4", section "Fused transformer
// (OrbitQuant 0.11)": W4A4 GEMMs with SwiGLU and gated-residual epilogues,
// W8A8 for ff.down; README "Krea-2-SVDQuant-ComfyUI", section "Why this
// exists": the speed comes from integer units on quantized activations, with
// a low-rank correction branch on top of the W4A4 kernel.)
//
// INT4 operands reach the int8 MFMA through a nibble trick: for a packed
// dword p, (p << 4) & 0xF0F0F0F0 and p & 0xF0F0F0F0 are four int8 lanes each
// holding 16 * (low nibble) and 16 * (high nibble).  With the library's
// packed order (byte 4c+j = channels 8c+j | 8c+j+4 << 4) the two words come
// out in channel order, so no shuffle is needed; the exact factor 16 per
// packed operand is removed in the epilogue (shift for int32 output, power
// of two folded into the scale otherwise).
//
// Tiling: 128x128 output tile per 256-thread workgroup (2x2 waves of 64x64),
// K staged through LDS 128 channels at a time, double-buffered with a
// register prefetch of the next stage.  v_mfma_i32_16x16x64_i8: lane l holds
// row (l % 16) of each operand and one 16-channel slice (l / 16) of K; the
// same slice map is used for both operands, so their channel pairing is
// exact whatever the hardware's internal K order.  Output lane l holds
// column l % 16, rows 4*(l/16) + r.

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 128;  // channels per LDS stage
constexpr int kThreads = 256;

enum { EPI_BF16 = 0, EPI_SWIGLU = 1, EPI_GATED = 2, EPI_F32 = 3, EPI_I32 = 4 };

template <bool PACKED>
struct Op {
  static constexpr int RB = PACKED ? BK / 2 : BK;  // bytes per row per stage
  static constexpr int BYTES = 128 * RB;            // bytes per stage (128 rows)
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int NLOAD = 128 * CPR / kThreads;  // chunks per thread
};

// LDS placement.  Unpacked rows (128 B): 16-byte chunk c of row r goes to
// chunk c ^ (r & 7).  Packed rows (64 B): 8-byte unit u of row r goes to
// unit u ^ ((r >> 1) & 7).  Both make the 16 rows read by one MFMA fragment
// load hit distinct banks.
template <bool PACKED>
__device__ __forceinline__ void lds_store_chunk(uint8_t* base, int r, int c, const uint4& v) {
  if (!PACKED) {
    *reinterpret_cast<uint4*>(base + r * 128 + ((c ^ (r & 7)) << 4)) = v;
  } else {
    const int f = (r >> 1) & 7;
    uint8_t* rb = base + r * 64;
    *reinterpret_cast<uint2*>(rb + (((2 * c) ^ f) << 3)) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2*>(rb + (((2 * c + 1) ^ f) << 3)) = make_uint2(v.z, v.w);
  }
}

// Fragment of 16 channels (slice = kk*4 + l/16 of the 128-channel stage) of row r.
template <bool PACKED>
__device__ __forceinline__ v4i lds_frag(const uint8_t* base, int r, int slice) {
  if (!PACKED) {
    return *reinterpret_cast<const v4i*>(base + r * 128 + ((slice ^ (r & 7)) << 4));
  } else {
    const uint2 p = *reinterpret_cast<const uint2*>(base + r * 64 + ((slice ^ ((r >> 1) & 7)) << 3));
    v4i o;
    o[0] = (int)((p.x << 4) & 0xF0F0F0F0u);
    o[1] = (int)(p.x & 0xF0F0F0F0u);
    o[2] = (int)((p.y << 4) & 0xF0F0F0F0u);
    o[3] = (int)(p.y & 0xF0F0F0F0u);
    return o;
  }
}

struct KArgs {
  const uint8_t* a;
  const uint8_t* w;
  const float* sa;
  const float* sw;
  int64_t M, N, K;
  int sa_stride, sw_stride;  // 0 tensor, 1 row (group64: K/64 per row)
  const uint16_t* bias;
  const uint16_t* residual;
  const uint16_t* gate;
  const uint16_t* lr;
  const uint16_t* l2;
  int rank;
  void* out;
  int64_t ldo;
  float post;     // 1/16 per packed operand
  int shift;      // 4 per packed operand (I32 output)
  int tiles_m;
  int64_t half_n; // SWIGLU: N/2
};

// Row of the W tile that wave column wn, fragment j, lane-row lr16 maps to.
template <int EPI>
__device__ __forceinline__ int w_tile_row(int wn, int j) {
  if (EPI == EPI_SWIGLU) return (j >> 1) * 64 + wn * 32 + (j & 1) * 16;
  return wn * 64 + j * 16;
}

template <bool AP, bool WP, bool GROUP, int EPI, bool LOWRANK>
__global__ __launch_bounds__(kThreads, 2) void qgemm_kernel(KArgs p) {
  using OA = Op<AP>;
  using OW = Op<WP>;
  constexpr int STAGE = OA::BYTES + OW::BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ float s_sa[GROUP ? 2 * BM * 2 : 1];  // [buf][2 groups][128 rows]
  __shared__ float s_sw[GROUP ? 2 * BN * 2 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const int tile_m = blockIdx.x % p.tiles_m;
  const int tile_n = blockIdx.x / p.tiles_m;
  const int64_t m0 = (int64_t)tile_m * BM;
  // SWIGLU: the tile covers gate rows [f0, f0+64) and up rows [F+f0, F+f0+64)
  const int64_t n0 = EPI == EPI_SWIGLU ? (int64_t)tile_n * (BN / 2) : (int64_t)tile_n * BN;

  const int64_t lda = AP ? p.K / 2 : p.K;
  const int64_t ldw = WP ? p.K / 2 : p.K;

  // global -> register prefetch addressing (rows clamped into range)
  const uint8_t* ga[OA::NLOAD];
  int ra[OA::NLOAD], ca[OA::NLOAD];
#pragma unroll
  for (int i = 0; i < OA::NLOAD; ++i) {
    const int c = tid + i * kThreads;
    ra[i] = c / OA::CPR;
    ca[i] = c % OA::CPR;
    int64_t gm = m0 + ra[i];
    if (gm > p.M - 1) gm = p.M - 1;
    ga[i] = p.a + gm * lda + ca[i] * 16;
  }
  const uint8_t* gw[OW::NLOAD];
  int rw[OW::NLOAD], cw[OW::NLOAD];
#pragma unroll
  for (int i = 0; i < OW::NLOAD; ++i) {
    const int c = tid + i * kThreads;
    rw[i] = c / OW::CPR;
    cw[i] = c % OW::CPR;
    int64_t gn;
    if (EPI == EPI_SWIGLU)
      gn = (rw[i] < 64) ? n0 + rw[i] : p.half_n + n0 + (rw[i] - 64);
    else
      gn = n0 + rw[i];
    if (gn > p.N - 1) gn = p.N - 1;
    gw[i] = p.w + gn * ldw + cw[i] * 16;
  }

  uint4 pa[OA::NLOAD], pw[OW::NLOAD];
  float psa = 0.f, psw = 0.f;
  const int KT = (int)(p.K / BK);
  const int64_t kgroups = p.K >> 6;

  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < OA::NLOAD; ++i)
      pa[i] = *reinterpret_cast<const uint4*>(ga[i] + (int64_t)kt * OA::RB);
#pragma unroll
    for (int i = 0; i < OW::NLOAD; ++i)
      pw[i] = *reinterpret_cast<const uint4*>(gw[i] + (int64_t)kt * OW::RB);
    if (GROUP) {
      // thread t < 256: scale of (row t/2, group kt*2 + t%2) for A and W
      const int r = tid >> 1, gsel = tid & 1;
      int64_t gm = m0 + r;
      if (gm > p.M - 1) gm = p.M - 1;
      psa = p.sa[gm * kgroups + kt * 2 + gsel];
      int64_t gn;
      if (EPI == EPI_SWIGLU)
        gn = (r < 64) ? n0 + r : p.half_n + n0 + (r - 64);
      else
        gn = n0 + r;
      if (gn > p.N - 1) gn = p.N - 1;
      psw = p.sw[gn * kgroups + kt * 2 + gsel];
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* sa_ = smem + buf * STAGE;
    uint8_t* sw_ = sa_ + OA::BYTES;
#pragma unroll
    for (int i = 0; i < OA::NLOAD; ++i) lds_store_chunk<AP>(sa_, ra[i], ca[i], pa[i]);
#pragma unroll
    for (int i = 0; i < OW::NLOAD; ++i) lds_store_chunk<WP>(sw_, rw[i], cw[i], pw[i]);
    if (GROUP) {
      const int r = tid >> 1, gsel = tid & 1;
      s_sa[buf * 2 * BM + gsel * BM + r] = psa;
      s_sw[buf * 2 * BN + gsel * BN + r] = psw;
    }
  };

  v4i acc[4][4];
  v4f yf[GROUP ? 4 : 1][GROUP ? 4 : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  if (GROUP) {
#pragma unroll
    for (int i = 0; i < (GROUP ? 4 : 1); ++i)
#pragma unroll
      for (int j = 0; j < (GROUP ? 4 : 1); ++j) yf[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint8_t* sa_ = smem + buf * STAGE;
    const uint8_t* sw_ = sa_ + OA::BYTES;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int slice = kk * 4 + lg;
      v4i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = lds_frag<AP>(sa_, wm * 64 + i * 16 + l16, slice);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = lds_frag<WP>(sw_, w_tile_row<EPI>(wn, j) + l16, slice);
      if (!GROUP) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
      } else {
        // one 64-channel group: exact int32 partial, then fp32 rescale
        float swv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          swv[j] = s_sw[buf * 2 * BN + kk * BN + w_tile_row<EPI>(wn, j) + l16] * p.post;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sav[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) sav[r] = s_sa[buf * 2 * BM + kk * BM + wm * 64 + i * 16 + lg * 4 + r];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v4i part = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              yf[i][j][r] = __builtin_fmaf((float)part[r], sav[r] * swv[j], yf[i][j][r]);
          }
        }
      }
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue --
  // Low-rank up-projection: y += lr[m, :] @ L2[:, n] (bf16 MFMA, fp32 acc).
  v4f lrv[4][4];
  if (LOWRANK) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) lrv[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < p.rank; k0 += 32) {
      const int kc = k0 + lg * 8;  // this lane's 8 rank indices
      const bool kin = kc < p.rank;
      v8bf la[4], lb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t m = m0 + wm * 64 + i * 16 + l16;
        if (m > p.M - 1) m = p.M - 1;
        const uint4 u = kin ? *reinterpret_cast<const uint4*>(p.lr + m * p.rank + kc)
                            : make_uint4(0, 0, 0, 0);
        la[i] = __builtin_bit_cast(v8bf, u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tr = w_tile_row<EPI>(wn, j) + l16;
        int64_t n;
        if (EPI == EPI_SWIGLU)
          n = (tr < 64) ? n0 + tr : p.half_n + n0 + (tr - 64);
        else
          n = n0 + tr;
        if (n > p.N - 1) n = p.N - 1;
        uint32_t wv[4] = {0u, 0u, 0u, 0u};
        if (kin) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            wv[e] = (uint32_t)p.l2[(int64_t)(kc + 2 * e) * p.N + n] |
                    ((uint32_t)p.l2[(int64_t)(kc + 2 * e + 1) * p.N + n] << 16);
        }
        lb[j] = __builtin_bit_cast(v8bf, make_uint4(wv[0], wv[1], wv[2], wv[3]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          lrv[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(la[i], lb[j], lrv[i][j], 0, 0, 0);
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wm * 64 + i * 16 + lg * 4 + r;
      if (m >= p.M) continue;
      const float sa_m = GROUP ? 1.0f : p.sa[m * p.sa_stride];
      if (EPI == EPI_SWIGLU) {
        // fragments j = 0,1 are gate columns, j = 2,3 the matching up columns
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t f = n0 + wn * 32 + j * 16 + l16;
          if (f >= p.half_n) continue;
          float g, u;
          if (GROUP) {
            g = yf[i][j][r];
            u = yf[i][j + 2][r];
          } else {
            g = (float)acc[i][j][r] * p.post * sa_m * p.sw[f * p.sw_stride];
            u = (float)acc[i][j + 2][r] * p.post * sa_m * p.sw[(p.half_n + f) * p.sw_stride];
          }
          if (p.bias) {
            g += bf16_to_f32(p.bias[f]);
            u += bf16_to_f32(p.bias[p.half_n + f]);
          }
          if (LOWRANK) {
            g += lrv[i][j][r];
            u += lrv[i][j + 2][r];
          }
          const float o = g / (1.0f + __expf(-g)) * u;
          static_cast<uint16_t*>(p.out)[m * p.ldo + f] = (uint16_t)f32_to_bf16(o);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t n = n0 + wn * 64 + j * 16 + l16;
          if (n >= p.N) continue;
          if (EPI == EPI_I32) {
            static_cast<int32_t*>(p.out)[m * p.ldo + n] = acc[i][j][r] >> p.shift;
            continue;
          }
          float y;
          if (GROUP)
            y = yf[i][j][r];
          else
            y = (float)acc[i][j][r] * p.post * sa_m * p.sw[n * p.sw_stride];
          if (p.bias) y += bf16_to_f32(p.bias[n]);
          if (LOWRANK) y += lrv[i][j][r];
          if (EPI == EPI_F32) {
            static_cast<float*>(p.out)[m * p.ldo + n] = y;
          } else if (EPI == EPI_GATED) {
            const float res = bf16_to_f32(p.residual[m * p.ldo + n]);
            const float o = __builtin_fmaf(bf16_to_f32(p.gate[n]), y, res);
            static_cast<uint16_t*>(p.out)[m * p.ldo + n] = (uint16_t)f32_to_bf16(o);
          } else {
            static_cast<uint16_t*>(p.out)[m * p.ldo + n] = (uint16_t)f32_to_bf16(y);
          }
        }
      }
    }
  }
}

template <bool AP, bool WP, bool GROUP, int EPI, bool LOWRANK>
hipError_t launch_t(const KArgs& k, int64_t tiles_n, hipStream_t s) {
  const int64_t blocks = (int64_t)k.tiles_m * tiles_n;
  hipLaunchKernelGGL((qgemm_kernel<AP, WP, GROUP, EPI, LOWRANK>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, s, k);
  return hipGetLastError();
}

template <bool AP, bool WP, bool GROUP, int EPI>
hipError_t launch_lr(const KArgs& k, int64_t tiles_n, hipStream_t s) {
  if (k.rank > 0) return launch_t<AP, WP, GROUP, EPI, true>(k, tiles_n, s);
  return launch_t<AP, WP, GROUP, EPI, false>(k, tiles_n, s);
}

}  // namespace

int launch_qgemm(const GemmArgs& g, hipStream_t s) {
  if (g.M == 0) return OK;
  if (g.a_mode != 2 && g.rank == 0 && g.epilogue != EPI_SWIGLU) return launch_qgemm_pipe(g, s);
  KArgs k;
  k.a = static_cast<const uint8_t*>(g.a);
  k.w = static_cast<const uint8_t*>(g.w);
  k.sa = g.sa;
  k.sw = g.sw;
  k.M = g.M;
  k.N = g.N;
  k.K = g.K;
  const bool group = g.a_mode == 2;
  k.sa_stride = group ? (int)(g.K >> 6) : (g.a_mode == 1 ? 1 : 0);
  k.sw_stride = group ? (int)(g.K >> 6) : (g.w_mode == 1 ? 1 : 0);
  k.bias = g.bias;
  k.residual = g.residual;
  k.gate = g.gate;
  k.lr = g.lr;
  k.l2 = g.l2;
  k.rank = g.rank;
  k.out = g.out;
  k.ldo = g.ldo;
  const int npacked = (g.a_packed ? 1 : 0) + (g.w_packed ? 1 : 0);
  k.post = npacked == 2 ? 1.0f / 256.0f : (npacked == 1 ? 1.0f / 16.0f : 1.0f);
  k.shift = 4 * npacked;
  k.tiles_m = (int)((g.M + BM - 1) / BM);
  k.half_n = g.N / 2;
  const int64_t tiles_n =
      g.epilogue == EPI_SWIGLU ? (k.half_n + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
  hipError_t e = hipErrorInvalidValue;
  const bool ap = g.a_packed != 0;
  const bool wp = g.w_packed != 0;
#define QL_DISPATCH_GROUP(AP_, WP_, GR_)                                          \
  switch (g.epilogue) {                                                           \
    case EPI_BF16: e = launch_lr<AP_, WP_, GR_, EPI_BF16>(k, tiles_n, s); break;  \
    case EPI_SWIGLU: e = launch_lr<AP_, WP_, GR_, EPI_SWIGLU>(k, tiles_n, s); break; \
    case EPI_F32: e = launch_lr<AP_, WP_, GR_, EPI_F32>(k, tiles_n, s); break;    \
    default: break;                                                               \
  }
  if (!wp) {
    // W8A8: int8 x int8, tensor/row scales
    switch (g.epilogue) {
      case EPI_BF16: e = launch_t<false, false, false, EPI_BF16, false>(k, tiles_n, s); break;
      case EPI_GATED: e = launch_t<false, false, false, EPI_GATED, false>(k, tiles_n, s); break;
      case EPI_F32: e = launch_t<false, false, false, EPI_F32, false>(k, tiles_n, s); break;
      case EPI_I32: e = launch_t<false, false, false, EPI_I32, false>(k, tiles_n, s); break;
      default: break;
    }
  } else if (g.epilogue == EPI_I32) {
    if (ap) e = launch_t<true, true, false, EPI_I32, false>(k, tiles_n, s);
    else e = launch_t<false, true, false, EPI_I32, false>(k, tiles_n, s);
  } else if (group) {
    if (ap) { QL_DISPATCH_GROUP(true, true, true) }
    else { QL_DISPATCH_GROUP(false, true, true) }
  } else {
    if (ap) { QL_DISPATCH_GROUP(true, true, false) }
    else { QL_DISPATCH_GROUP(false, true, false) }
  }
#undef QL_DISPATCH_GROUP
  return e == hipSuccess ? OK : ERR_LAUNCH;
}

}  // namespace ql
