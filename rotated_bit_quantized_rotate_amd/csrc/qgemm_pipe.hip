// Large-tile integer GEMM for the rotated low-bit linear on gfx950:
// exact int32 accumulation on int8 MFMA with tensor / row scales and the
// plain, f32, int32 and gated-residual epilogues (model card "Krea 2 Turbo
// OrbitQuant W4A4", section "Fused transformer (OrbitQuant 0.11)": W4A4
// GEMMs, and W8A8 for ff.down with the gated residual in the epilogue).
//
// Design (MI355X: 256 CUs in 8 XCDs, 160 KB LDS per CU):
//  * one 512-thread workgroup (8 waves, 2 x 4) per BM x BN output tile; with
//    256 x 320 tiles a 4096 x 5120 output is exactly 256 tiles, one per CU;
//  * K is staged through LDS 128 channels at a time in a 3-deep ring filled
//    by direct global->LDS loads (global_load_lds_dwordx4): no staging
//    registers, and the loads of stage s+2 overlap the MFMAs of stage s;
//    one barrier per stage;
//  * 16-byte chunks are XOR-swizzled by row so every fragment read
//    (ds_read_b128) hits distinct banks;
//  * the MFMA is v_mfma_i32_16x16x64_i8 with the weight fragment as the
//    first operand, so the accumulator lane layout holds 4 consecutive
//    output columns of one row (8-byte bf16 stores in the epilogue);
//  * INT4 weights are unpacked in registers: for a packed dword p,
//    (p << 4) & 0xF0F0F0F0 and p & 0xF0F0F0F0 are four int8 lanes holding
//    16 * (low nibble) and 16 * (high nibble); with the library's packed
//    order they come out in channel order.  The factor 16 is removed exactly
//    in the epilogue.
//  * K-slice map: lane group g = lane / 16 owns channels [32g, 32g + 32) of
//    each 128-channel stage, split over two MFMAs (kk = 0, 1) of 16 channels.
//    In the packed layout those 32 channels are the 16 contiguous bytes
//    [16g, 16g + 16), so one b128 read feeds both MFMAs.  Both operands use
//    the same map, so the channel pairing is exact.
//  * workgroup ids are remapped so the tiles one XCD runs form a compact
//    block of the tile grid (shared A / W panels hit that XCD's L2).

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int BK = 128;      // channels per stage
constexpr int kLdsBytes = 160 * 1024;

enum { EPI_BF16 = 0, EPI_SWIGLU = 1, EPI_GATED = 2, EPI_F32 = 3, EPI_I32 = 4 };

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

#define LDS_AS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt with only vmcnt constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ v4i unpack_lo(uint32_t x, uint32_t y) {
  v4i o;
  o[0] = (int)((x << 4) & 0xF0F0F0F0u);
  o[1] = (int)(x & 0xF0F0F0F0u);
  o[2] = (int)((y << 4) & 0xF0F0F0F0u);
  o[3] = (int)(y & 0xF0F0F0F0u);
  return o;
}

struct PArgs {
  const uint8_t* a;
  const uint8_t* w;
  const float* sa;
  const float* sw;
  int64_t M, N, K;
  int sa_stride, sw_stride;
  const uint16_t* bias;
  const uint16_t* residual;
  const uint16_t* gate;
  void* out;
  int64_t ldo;
  float post;
  int shift;
  int tiles_m, tiles_n;
  int group_m;     // tile rows per L2 group
};

template <int BM_, int BN_, int WGM_, int WGN_, bool AP_, bool WP_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WGM = WGM_, WGN = WGN_;   // wave grid
  static constexpr int NW = WGM * WGN;           // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr bool AP = AP_, WP = WP_;
  static constexpr int WM = BM / WGM;       // wave tile rows
  static constexpr int WN = BN / WGN;       // wave tile cols
  static constexpr int FI = WM / 16;
  static constexpr int FJ = WN / 16;
  static constexpr int ARB = AP ? BK / 2 : BK;  // bytes per A row per stage
  static constexpr int WRB = WP ? BK / 2 : BK;
  static constexpr int SA = BM * ARB;
  static constexpr int SW = BN * WRB;
  static constexpr int STAGE = SA + SW;
  static constexpr int A_INSTR = SA / 1024;  // 1 KB per DMA instruction
  static constexpr int W_INSTR = SW / 1024;
  static_assert(SA % 1024 == 0 && SW % 1024 == 0, "stage must be whole KB");
  static_assert(A_INSTR % NW == 0, "A DMA must split evenly over the waves");
  static constexpr int A_PER_WAVE = A_INSTR / NW;
  static constexpr int W_HI = (W_INSTR + NW - 1) / NW;  // waves < W_SPLIT issue W_HI
  static constexpr int W_SPLIT = W_INSTR - (W_HI - 1) * NW;
  static constexpr int NSTAGE = (3 * STAGE <= kLdsBytes) ? 3 : 2;  // LDS ring depth
  static_assert(NSTAGE * STAGE <= kLdsBytes, "LDS ring too large");
  static_assert((NSTAGE - 2) * (A_PER_WAVE + W_HI) < 64, "vmcnt range");
};

// Chunk position inside an LDS row of RB bytes: chunk c of row r lives at
// c ^ f(r).  A fragment read (ds_read_b128) has 16 lanes on 16 consecutive
// rows at one chunk index per lane group; these XOR patterns were measured
// on gfx950 (bank-conflict counter) to serve every such read, for 128-byte
// rows with chunk 2g + kk and 64-byte rows with chunk g, without bank
// conflicts.  f depends only on r & 15.
template <int RB>
__device__ __forceinline__ int swz(int r, int c) {
  if (RB == 128) return c ^ (((r & 3) << 1) | ((r >> 2) & 1));
  return c ^ ((r >> 1) & 3);
}

// One DMA instruction q (1 KB) of an operand: lane i fills LDS chunk i of
// that KB; rows are RB bytes.  Returns the global source for this lane.
template <int RB>
__device__ __forceinline__ const uint8_t* dma_src(const uint8_t* base, int64_t ld, int64_t row0,
                                                  int64_t rows_valid, int q, int lane, int64_t kbyte) {
  constexpr int CPR = RB / 16;
  const int rl = q * (1024 / RB) + lane / CPR;  // row inside the tile
  const int pos = lane % CPR;
  const int c = swz<RB>(rl, pos);               // inverse of the XOR is itself
  int64_t gr = row0 + rl;
  if (gr > rows_valid - 1) gr = rows_valid - 1;
  return base + gr * ld + kbyte + c * 16;
}

template <class C, int EPI>
__global__ __launch_bounds__(C::NT, 1) void qgemm_pipe_kernel(PArgs p) {
  constexpr int NS = C::NSTAGE;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * C::STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WGN;
  const int wn = wave % C::WGN;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  // ---- XCD-aware tile order -------------------------------------------
  const int nb = p.tiles_m * p.tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, q8 = nb >> 3, r8 = nb & 7;
  const int bl = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + (b >> 3);
  const int gsz = p.group_m * p.tiles_n;
  const int grp = bl / gsz;
  const int first_m = grp * p.group_m;
  const int gm = min(p.tiles_m - first_m, p.group_m);
  const int inb = bl - grp * gsz;
  const int tile_m = first_m + inb % gm;
  const int tile_n = inb / gm;
  const int64_t m0 = (int64_t)tile_m * C::BM;
  const int64_t n0 = (int64_t)tile_n * C::BN;

  const int64_t lda = C::AP ? p.K / 2 : p.K;
  const int64_t ldw = C::WP ? p.K / 2 : p.K;
  const int KT = (int)(p.K / BK);

  // ---- DMA issue -----------------------------------------------------------
  // Instruction t (0 .. NDMA-1) of this wave's share of stage kt: the first
  // A_PER_WAVE move A, the rest W.  A burst of these right after a barrier
  // stalls the wave on VMEM issue while its MFMA pipe idles, so the main
  // loop spreads them through the MFMA stream.
  const bool w_hi = wave < C::W_SPLIT;
  constexpr int NDMA = C::A_PER_WAVE + C::W_HI;
  auto issue_one = [&](int kt, int t) {
    uint8_t* st = smem + (kt % NS) * C::STAGE;
    if (t < C::A_PER_WAVE) {
      const int q = wave + C::NW * t;
      const uint8_t* src = dma_src<C::ARB>(p.a, lda, m0, p.M, q, lane, (int64_t)kt * C::ARB);
      __builtin_amdgcn_global_load_lds(src, LDS_AS(st + q * 1024), 16, 0, 0);
    } else {
      const int tw = t - C::A_PER_WAVE;
      if (tw < C::W_HI - 1 || w_hi) {
        const int q = wave + C::NW * tw;
        const uint8_t* src = dma_src<C::WRB>(p.w, ldw, n0, p.N, q, lane, (int64_t)kt * C::WRB);
        __builtin_amdgcn_global_load_lds(src, LDS_AS(st + C::SA + q * 1024), 16, 0, 0);
      }
    }
  };

  v4i acc[C::FJ][C::FI];
#pragma unroll
  for (int j = 0; j < C::FJ; ++j)
#pragma unroll
    for (int i = 0; i < C::FI; ++i) acc[j][i] = v4i{0, 0, 0, 0};

  // lane-constant LDS offsets: fragment rows differ by multiples of 16, so
  // the swizzle term depends on l16 only.
  static_assert(C::WM % 16 == 0 && C::WN % 16 == 0, "wave tile must be 16-aligned");
  const int a_row = wm * C::WM + l16;
  const int w_row = wn * C::WN + l16;
  int a_off[2];
  int w_off;
  if (C::AP) {
    a_off[0] = a_row * 64 + (swz<64>(a_row, lg) << 4);
    a_off[1] = a_off[0];
  } else {
    a_off[0] = a_row * 128 + (swz<128>(a_row, 2 * lg) << 4);
    a_off[1] = a_row * 128 + (swz<128>(a_row, 2 * lg + 1) << 4);
  }
  if (C::WP) w_off = w_row * 64 + (swz<64>(w_row, lg) << 4);
  else w_off = w_row * 128 + (swz<128>(w_row, 2 * lg) << 4);
  const int w_off1 = C::WP ? w_off : w_row * 128 + (swz<128>(w_row, 2 * lg + 1) << 4);

  // prologue: stages 0 .. NS-2 in flight
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0)
    if (s0 < KT) {
#pragma unroll
      for (int t = 0; t < NDMA; ++t) issue_one(s0, t);
    }

  for (int kt = 0; kt < KT; ++kt) {
    // Stage kt has landed once only the later stages (at most NS-2 of them)
    // are still in flight; the barrier then publishes every wave's part and
    // guarantees all waves finished reading the buffer the next DMA reuses.
    if (NS == 3 && kt + 1 < KT) {
      if (w_hi) wait_vmcnt<(NS - 2) * NDMA>();
      else wait_vmcnt<(NS - 2) * (NDMA - 1)>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    const bool dma = kt + NS - 1 < KT;

    const uint8_t* As = smem + (kt % NS) * C::STAGE;
    const uint8_t* Ws = As + C::SA;
    // W fragments: packed -> one b128 per fragment carries both halves (kk);
    // int8 -> one b128 per fragment and half.
    uint4 wraw[C::FJ];
    uint4 wraw1[C::WP ? 1 : C::FJ];
#pragma unroll
    for (int j = 0; j < C::FJ; ++j) {
      wraw[j] = *reinterpret_cast<const uint4*>(Ws + w_off + j * 16 * C::WRB);
      if (!C::WP) wraw1[j] = *reinterpret_cast<const uint4*>(Ws + w_off1 + j * 16 * C::WRB);
    }
    // A fragments: int8 -> streamed through a small window read PF ahead;
    // packed -> one b128 per fragment carries both halves.
    constexpr int PF = 3;
    constexpr int NQ = 2 * C::FI;
    v4i abuf[PF + 1];
    uint4 araw[C::AP ? C::FI : 1];
    if (C::AP) {
#pragma unroll
      for (int i = 0; i < C::FI; ++i) araw[i] = *reinterpret_cast<const uint4*>(As + a_off[0] + i * 16 * C::ARB);
    } else {
#pragma unroll
      for (int q = 0; q < PF; ++q)
        abuf[q] = *reinterpret_cast<const v4i*>(As + a_off[q / C::FI] + (q % C::FI) * 16 * C::ARB);
    }
    v4i bw0[C::FJ], bw1[C::FJ];
#pragma unroll
    for (int j = 0; j < C::FJ; ++j)
      bw0[j] = C::WP ? unpack_lo(wraw[j].x, wraw[j].y)
                     : v4i{(int)wraw[j].x, (int)wraw[j].y, (int)wraw[j].z, (int)wraw[j].w};
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int kk = q / C::FI, i = q % C::FI;
      v4i af;
      if (C::AP) {
        af = kk == 0 ? unpack_lo(araw[i].x, araw[i].y) : unpack_lo(araw[i].z, araw[i].w);
      } else {
        if (q + PF < NQ)
          abuf[(q + PF) % (PF + 1)] = *reinterpret_cast<const v4i*>(
              As + a_off[(q + PF) / C::FI] + ((q + PF) % C::FI) * 16 * C::ARB);
        af = abuf[q % (PF + 1)];
      }
      if (dma && (q % 2) == 0 && q / 2 < NDMA) issue_one(kt + NS - 1, q / 2);
      // second-half W fragments, spread over the first half's MFMA groups
      if (kk == 0 && i < C::FJ)
        bw1[i] = C::WP ? unpack_lo(wraw[i].z, wraw[i].w)
                       : v4i{(int)wraw1[i].x, (int)wraw1[i].y, (int)wraw1[i].z, (int)wraw1[i].w};
      if (kk == 0 && i == C::FI - 1) {
#pragma unroll
        for (int j = C::FI; j < C::FJ; ++j)
          bw1[j] = C::WP ? unpack_lo(wraw[j].z, wraw[j].w)
                         : v4i{(int)wraw1[j].x, (int)wraw1[j].y, (int)wraw1[j].z, (int)wraw1[j].w};
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < C::FJ; ++j)
        acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kk == 0 ? bw0[j] : bw1[j], af, acc[j][i], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // any DMA instructions not yet issued (only if NDMA > NQ / 2)
    if (dma) {
#pragma unroll
      for (int t = NQ / 2; t < NDMA; ++t) issue_one(kt + NS - 1, t);
    }
  }

  // ---- epilogue: lane holds out[m][n .. n+3] for each (i, j) --------------
#pragma unroll
  for (int j = 0; j < C::FJ; ++j) {
    const int64_t n = n0 + wn * C::WN + j * 16 + lg * 4;
    if (n >= p.N) continue;
    float swv[4], addv[4], gatev[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      swv[r] = EPI == EPI_I32 ? 0.f : p.sw[(n + r) * p.sw_stride];
      addv[r] = p.bias ? bf16_to_f32(p.bias[n + r]) : 0.f;
      gatev[r] = EPI == EPI_GATED ? bf16_to_f32(p.gate[n + r]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < C::FI; ++i) {
      const int64_t m = m0 + wm * C::WM + i * 16 + l16;
      if (m >= p.M) continue;
      const v4i a4 = acc[j][i];
      if (EPI == EPI_I32) {
        int4 o;
        o.x = a4[0] >> p.shift;
        o.y = a4[1] >> p.shift;
        o.z = a4[2] >> p.shift;
        o.w = a4[3] >> p.shift;
        *reinterpret_cast<int4*>(static_cast<int32_t*>(p.out) + m * p.ldo + n) = o;
        continue;
      }
      const float sam = p.sa[m * p.sa_stride] * p.post;
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = (float)a4[r] * sam * swv[r] + addv[r];
      if (EPI == EPI_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + m * p.ldo + n) =
            make_float4(y[0], y[1], y[2], y[3]);
        continue;
      }
      if (EPI == EPI_GATED) {
        const uint2 rr = *reinterpret_cast<const uint2*>(p.residual + m * p.ldo + n);
        y[0] = __builtin_fmaf(gatev[0], y[0], bf16_to_f32(rr.x & 0xffff));
        y[1] = __builtin_fmaf(gatev[1], y[1], bf16_to_f32(rr.x >> 16));
        y[2] = __builtin_fmaf(gatev[2], y[2], bf16_to_f32(rr.y & 0xffff));
        y[3] = __builtin_fmaf(gatev[3], y[3], bf16_to_f32(rr.y >> 16));
      }
      const bf2 h0 = __builtin_convertvector(f2{y[0], y[1]}, bf2);
      const bf2 h1 = __builtin_convertvector(f2{y[2], y[3]}, bf2);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + m * p.ldo + n) =
          make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
    }
  }
}

template <class C, int EPI>
hipError_t launch_pipe(PArgs p, hipStream_t s) {
  p.tiles_m = (int)((p.M + C::BM - 1) / C::BM);
  p.tiles_n = (int)((p.N + C::BN - 1) / C::BN);
  p.group_m = 4;
  const int nb = p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL((qgemm_pipe_kernel<C, EPI>), dim3(nb), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

template <class C>
hipError_t launch_epi(const PArgs& p, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_BF16: return launch_pipe<C, EPI_BF16>(p, s);
    case EPI_F32: return launch_pipe<C, EPI_F32>(p, s);
    case EPI_I32: return launch_pipe<C, EPI_I32>(p, s);
    case EPI_GATED: return launch_pipe<C, EPI_GATED>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Tensor / row scales, epilogues BF16 | F32 | I32 | GATED.
int launch_qgemm_pipe(const GemmArgs& g, hipStream_t s) {
  PArgs p{};
  p.a = static_cast<const uint8_t*>(g.a);
  p.w = static_cast<const uint8_t*>(g.w);
  p.sa = g.sa;
  p.sw = g.sw;
  p.M = g.M;
  p.N = g.N;
  p.K = g.K;
  p.sa_stride = g.a_mode == 1 ? 1 : 0;
  p.sw_stride = g.w_mode == 1 ? 1 : 0;
  p.bias = g.bias;
  p.residual = g.residual;
  p.gate = g.gate;
  p.out = g.out;
  p.ldo = g.ldo;
  const int npacked = (g.a_packed ? 1 : 0) + (g.w_packed ? 1 : 0);
  p.post = npacked == 2 ? 1.0f / 256.0f : (npacked == 1 ? 1.0f / 16.0f : 1.0f);
  p.shift = 4 * npacked;
  hipError_t e;
  if (g.w_packed) {
    if (g.a_packed) e = launch_epi<Cfg<256, 320, 2, 4, true, true>>(p, g.epilogue, s);
    else e = launch_epi<Cfg<256, 320, 2, 4, false, true>>(p, g.epilogue, s);
  } else {
    e = launch_epi<Cfg<256, 256, 2, 4, false, false>>(p, g.epilogue, s);
  }
  return e == hipSuccess ? OK : ERR_LAUNCH;
}

}  // namespace ql
