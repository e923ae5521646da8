// Integer GEMM of the rotated low-bit linear on gfx950: exact int32
// accumulation on int8 MFMA, then the dequantize epilogue.
//
//   acc[m, n] = sum_k qa[m, k] * qw[n, k]                 (exact, int32)
//   y[m, n]   = acc * s_a * s_w                   (tensor / row scales)
//             = sum_g acc_g * s_a[m,g] * s_w[n,g]   (group-64 scales: exact
//                                     int32 partial per group, fp32 sum)
//   (+ bias[n]) (+ sum_r lr[m,r] * L2[r,n])  -> epilogue -> out
//
// Epilogues: bf16, f32, int32 (debug), gated residual res + gate[n] * y,
// SwiGLU silu(y_gate) * y_up over a gate|up weight.  (Model card "Krea 2
// Turbo OrbitQuant W4A4", section "Fused transformer (OrbitQuant 0.11)":
// W4A4 GEMMs with SwiGLU and gated residuals in their epilogues, W8A8 for
// ff.down; README "Krea-2-SVDQuant-ComfyUI", sections "Why this exists" and
// "Low-rank refinement": a low-rank branch on top of the W4A4 kernel; model
// card "Krea 2 Turbo Nunchaku Lite INT4 r32": group size 64, rank 32.)
//
// Design (MI355X: 256 CUs in 8 XCDs, 160 KB LDS per CU):
//  * one 512-thread workgroup (8 waves, 2 x 4) per BM x BN output tile; with
//    256 x 320 tiles a 4096 x 5120 output is exactly 256 tiles, one per CU;
//  * K is staged through LDS 128 channels at a time in a ring of 2-3 stages
//    filled by direct global->LDS loads (global_load_lds): no staging
//    registers, and the loads of later stages overlap the MFMAs of the
//    current one; one barrier per stage.  Group-64 scales of the stage's two
//    groups ride in the same ring (4-byte loads, gathered into the order
//    the lanes read them);
//  * 16-byte chunks are XOR-swizzled by row so every fragment read
//    (ds_read_b128) hits distinct banks;
//  * the MFMA is v_mfma_i32_16x16x64_i8 with the weight fragment as the
//    first operand, so the accumulator lane layout holds 4 consecutive
//    output columns of one row (8-byte bf16 stores in the epilogue);
//  * INT4 codes are unpacked in registers: for a packed dword p,
//    (p << 4) & 0xF0F0F0F0 and p & 0xF0F0F0F0 are four int8 lanes holding
//    16 * (low nibble) and 16 * (high nibble); with the library's packed
//    order they come out in channel order.  The factor 16 per packed operand
//    is removed exactly in the epilogue;
//  * K-slice map (tensor / row scales): lane group g = lane / 16 owns
//    channels [32g, 32g + 32) of each 128-channel stage, split over two
//    MFMAs (kk = 0, 1) of 16 channels each.  In the packed layout those 32
//    channels are the 16 contiguous bytes [16g, 16g + 16), so one b128 read
//    feeds both MFMAs.  Both operands use the same map, so the channel
//    pairing is exact;
//  * K-slice map (group-64 scales): MFMA kk must cover exactly the stage's
//    64-channel group kk, so lane group g takes channels 64 kk + 16 g +
//    [0, 16) (packed: 8 bytes, one b64 read per MFMA).  Every MFMA starts
//    from zero, its int32 result is that group's exact partial, and it is
//    converted and added into an fp32 accumulator with s_a[m,g] * s_w[n,g];
//    the scales are stored group-major ([K/64][rows]), so a stage's loads of
//    one group's scales read consecutive rows (whole cache lines);
//  * the same codes in the FP6 layout with group-64 scales run the
//    32x32x64 FP6 instruction (64 channels: exactly one group), whose fp32
//    result is the group's exact partial, rescaled without a conversion;
//  * SwiGLU: the W tile of a workgroup holds, per wave column, 32 gate rows
//    f and the 32 matching up rows F + f, so a lane holds gate and up of the
//    same outputs;
//  * workgroup ids are remapped so the tiles one XCD runs form a compact
//    block of the tile grid (shared A / W panels hit that XCD's L2);
//  * int8 activations with tensor / row scales (plain epilogues: the
//    attention projections, the W8A8 ff.down) run a ping-pong K loop:
//    the two waves of each SIMD alternate, one phase apart, between reading
//    fragments from LDS (and issuing global -> LDS loads) and a cluster of
//    MFMAs from registers (40 on a 256 x 320 tile), so one of them always
//    feeds the matrix pipe
//    (measured on gfx950: -3 to -5 % at 4096 x 5120 x 5120, -8 % at K =
//    20480; the same loop with packed activations gains nothing).

#include <type_traits>

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int BK = 128;      // channels per stage
constexpr int kLdsBytes = 160 * 1024;

enum { EPI_BF16 = 0, EPI_SWIGLU = 1, EPI_GATED = 2, EPI_F32 = 3, EPI_I32 = 4, EPI_SIGMOID = 5 };

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

#define LDS_AS(p) ((__attribute__((address_space(3))) void*)(p))

// Wave priority for quarter `level` (0..3) of a stage's MFMA groups: it
// falls from 3 to 0 as the wave works through the stage, so when both waves
// of a SIMD contend for the matrix pipe, the one further behind issues
// first.  With equal priorities the older wave takes every contested slot,
// runs ahead and then idles at the stage barrier while its partner finishes
// alone with its read and load latencies exposed (measured on gfx950:
// waves reached the barrier up to a third of a stage apart).
__device__ __forceinline__ void stage_prio(int level) {
  if (level <= 0) __builtin_amdgcn_s_setprio(3);
  else if (level == 1) __builtin_amdgcn_s_setprio(2);
  else if (level == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Stage barrier.  The wave's own LDS reads are complete first, so no read
// of a ring stage can still be in flight when another wave, past the
// barrier, starts loading into that stage.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct global -> LDS load (global_load_lds, saddr form): lane l moves 16
// (dma_b128) or 4 (dma_b32) bytes from base + voff[l] to LDS address
// lds + l * size; base is wave-uniform, lds goes through M0.  Written as asm
// so the compiler does not track these loads: its wait-count pass cannot
// tell which ring stage a load fills and would drain every load in flight
// (the prefetch of later stages included) before a stage's first fragment
// read.  The kernel orders them itself with wait_vmcnt + barrier.  No VGPR
// is written, so nothing the compiler allocates is overwritten later.  The
// compiler's hazard pass does not look into the asm either: s_nop 4 gives
// the five wait states a VMEM read of an SGPR (the base, M0) needs after a
// VALU write of it (the base may come from v_readfirstlane).
// (The base is passed through readfirstlane: it is uniform, but the compiler
// does not always keep it in SGPRs, which the saddr operand requires.)
__device__ __forceinline__ uint64_t sgpr_u64(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void dma_b128(const void* base, uint32_t voff, const void* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)LDS_AS(lds);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sgpr_u64(base)), "{m0}"(la));
}
__device__ __forceinline__ void dma_b32(const void* base, uint32_t voff, const void* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)LDS_AS(lds);
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(sgpr_u64(base)), "{m0}"(la));
}

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
  const uint8_t* xa;         // MX: E8M0 block scales [K/128][M][4], [K/128][N][4]
  const uint8_t* xw;
  int64_t M, N, K;
  int sa_stride, sw_stride;  // tensor / row scales: 0 or 1
  int kg;                    // group-64 scales: K / 64 per row
  uint32_t sa_gs, sw_gs;     // group-64 scales ([K/64, M], [K/64, N]): bytes per stage (two groups)
  const uint16_t* bias;
  const uint16_t* residual;
  const uint16_t* gate;
  const uint16_t* lr;        // [M, rank]
  const uint16_t* l2;        // [N, rank] (L2 transposed)
  int rank;
  void* out;
  int64_t ldo;
  float post;      // 1/16 per packed operand
  int shift;       // 4 per packed operand (int32 output)
  int tiles_m, tiles_n;
  int group_m;     // tile rows per L2 group
  int64_t half_n;  // SwiGLU: F = N / 2
};

// F6: both operands in the FP6 e2m3 layout (96 bytes per row per stage),
// multiplied on the FP6 matrix instruction with fp32 accumulation.
// MX = 4 / 8: both operands MX block-scaled (OCP Microscaling v1.0): FP4
// E2M1 (64 bytes per row per stage) or FP8 E4M3 (128 bytes) elements, one
// E8M0 scale per 32 elements along K, applied by the block-scaled matrix
// instruction itself; fp32 accumulation.
// SUB = 2: each LDS stage holds 256 channels (two 128-channel sub-stages),
// so 4-bit operand rows are 128 contiguous bytes a stage -- whole cache
// lines, half the line requests per channel of 64-byte rows (the loads'
// cost follows the number of lines they touch) and half the barriers.
// M32 (FP6 with group-64 scales): the 32x32x64 FP6 instruction, whose 64
// channels are exactly one scale group, so each instruction's fp32 result is
// one group's exact partial for a 32 x 32 block (16 per lane).
template <int BM_, int BN_, int WGM_, int WGN_, bool AP_, bool WP_, bool GROUP_ = false, bool F6_ = false,
          int MX_ = 0, int MAXS_ = 3, int SUB_ = 1, bool PP_ = false, bool M32_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WGM = WGM_, WGN = WGN_;   // wave grid
  static constexpr int NW = WGM * WGN;           // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr bool AP = AP_, WP = WP_, GROUP = GROUP_, F6 = F6_;
  static constexpr int MX = MX_;
  static constexpr int SUB = SUB_;         // 128-channel sub-stages per LDS stage
  static constexpr bool PP = PP_;          // ping-pong K loop (see pipe_tile)
  static constexpr bool M32 = M32_;        // 32x32x64 FP6 instruction per scale group
  static constexpr int BKS = BK * SUB;     // channels per LDS stage
  static constexpr bool FMMA = F6 || MX != 0;   // float matrix instruction, fp32 accumulators
  static constexpr bool NOSC = GROUP || MX != 0;  // accumulators already carry both scales
  static constexpr bool SCL = GROUP || MX != 0;   // scales ride in the LDS ring
  static constexpr int WM = BM / WGM;       // wave tile rows
  static constexpr int WN = BN / WGN;       // wave tile cols
  static constexpr int FI = WM / 16;
  static constexpr int FJ = WN / 16;
  static constexpr int FI32 = WM / 32;      // M32: 32-row fragments of the wave tile
  static constexpr int FJ32 = WN / 32;
  static_assert(!M32_ || (F6_ && GROUP_ && WM % 32 == 0 && WN % 32 == 0 && WM / 32 == 4),
                "M32: FP6 operands with group-64 scales, four 32-row fragments per wave");
  static constexpr int ARB = F6 ? BKS * 3 / 4 : (MX ? BKS * MX / 8 : (AP ? BKS / 2 : BKS));  // bytes per A row per stage
  static constexpr int WRB = F6 ? BKS * 3 / 4 : (MX ? BKS * MX / 8 : (WP ? BKS / 2 : BKS));
  static_assert(!F6 || (AP && WP), "FP6 operands: both sides");
  static_assert(MX == 0 || MX == 4 || MX == 8, "MX element width");
  static_assert(!MX || (!AP && !WP && !GROUP && !F6), "MX operands have their own layout");
  static_assert(SUB == 1 || (SUB == 2 && !GROUP && !F6 && ((AP && WP) || MX == 4)),
                "256-channel stages: packed INT4 on both sides or MXFP4");
  static constexpr int SA = BM * ARB;
  static constexpr int SW = BN * WRB;
  // group-64: two groups of fp32 scales per row; MX: the 4 E8M0 bytes of
  // the stage's 4 blocks per row.  Padded so every wave issues the same
  // number of 256-byte loads.
  static constexpr int SCB = GROUP ? 8 * (BM + BN) : (MX ? 4 * SUB * (BM + BN) : 0);
  static constexpr int SC = (SCB + 256 * NW - 1) / (256 * NW) * (256 * NW);
  static constexpr int STAGE = SA + SW + SC;
  static constexpr int A_INSTR = SA / 1024;  // 1 KB per 16-byte-per-lane load
  static constexpr int W_INSTR = SW / 1024;
  static constexpr int S_INSTR = SC / 256;   // 256 B per 4-byte-per-lane load
  static_assert(SA % 1024 == 0 && SW % 1024 == 0, "stage must be whole KB");
  static_assert(A_INSTR % NW == 0, "A loads must split evenly over the waves");
  static_assert(S_INSTR % NW == 0, "scale loads must split evenly over the waves");
  static constexpr int A_PER_WAVE = A_INSTR / NW;
  static constexpr int S_PER_WAVE = S_INSTR / NW;
  static constexpr int W_HI = (W_INSTR + NW - 1) / NW;  // waves < W_SPLIT issue W_HI
  static constexpr int W_SPLIT = W_INSTR - (W_HI - 1) * NW;
  static constexpr int NDMA = A_PER_WAVE + W_HI + S_PER_WAVE;
  // LDS ring depth: the deepest of MAXS_, 3, 2 stages that fits
  static constexpr int NSTAGE = (MAXS_ >= 4 && 4 * STAGE <= kLdsBytes) ? 4 : ((3 * STAGE <= kLdsBytes) ? 3 : 2);
  static_assert(NSTAGE * STAGE <= kLdsBytes, "LDS ring too large");
  static_assert((NSTAGE - 2) * NDMA < 64, "vmcnt range");
  static_assert(!GROUP || FI % 4 == 0, "group scales are read 4 rows at a time");
  static_assert(!PP || (!AP && !GROUP && !F6 && MX == 0 && SUB == 1 && WGM == 2 && WGN == 4 && NSTAGE <= 3),
                "ping-pong loop: int8 A, tensor / row scales, 2 x 4 waves, 2 or 3 stages");
};

template <bool F>
struct AccOf { typedef v4i type; };
template <>
struct AccOf<true> { typedef v4f type; };

// FP6 stage rows: 6 chunks of 16 bytes (96 bytes: 24 of the 32 4-byte
// banks).  A b128 fragment read is served 8 lanes at a time, 8 consecutive
// rows at one chunk index; rows r and r + 4 start on the same bank, so the
// four low-part chunks 0..3 are XOR-ed with row bits 2..3, which gives the 8
// rows 8 different 16-byte bank groups.  The high parts (chunks 4, 5, read
// as b64 by 16 lanes) can only swap whole chunks, by row bit 3; their rows r
// and r + 4 still share banks (a 2-way conflict the 16-byte loads cannot
// split).  f depends on r & 15 only, so fragment rows 16 apart agree.
// The group-64 kernel (M32) keeps the plain row-bit-3 swap of every chunk,
// which measured 1.5 % faster there (its reads overlap the VALU-heavy
// rescale); the 16x16x128 kernel gains 3 % from the bits-2..3 form.
template <bool M32>
__device__ __forceinline__ int swz6(int r, int c) {
  if (M32) return c ^ ((r >> 3) & 1);
  return c < 4 ? c ^ ((r >> 2) & 3) : c ^ ((r >> 3) & 1);
}

// Chunk position inside an LDS row of RB bytes: chunk c of row r lives at
// c ^ f(r).  A fragment read (ds_read_b128) has 16 lanes on 16 consecutive
// rows at one chunk index per lane group; these XOR patterns were measured
// on gfx950 (bank-conflict counter) to serve every such read without bank
// conflicts: 128-byte rows read at chunk 2g + kk (GK = false) or 4 kk + g
// (GK = true, the group-64 map), 64-byte rows at chunk g, and MXFP8's
// 128-byte rows read at chunks g and 4 + g (F8: 15 % of the kernel's cycles
// in conflict with the int8 pattern, 0.8 % with this one).  f depends only
// on r & 15.
template <int RB, bool GK, bool F8 = false>
__device__ __forceinline__ int swz(int r, int c) {
  if (F8) return c ^ ((r >> 1) & 7);
  if (RB == 128) return GK ? c ^ (r & 7) : c ^ (((r & 3) << 1) | ((r >> 2) & 1));
  return c ^ ((r >> 1) & 3);
}

// Weight row (row of W, of its scales and of L2's columns) held by W-tile
// row t.  Plain: n0 + t.  SwiGLU (n0 = first output column f0 of the tile):
// each wave column's WN rows are WN/2 gate rows f then the WN/2 up rows
// F + f of the same outputs.  Rows past the end are clamped to the last row
// (their results are never stored).
template <class C, bool SWIG>
__device__ __forceinline__ int64_t w_row_of(const PArgs& p, int64_t n0, int t) {
  if (!SWIG) {
    const int64_t r = n0 + t;
    return r > p.N - 1 ? p.N - 1 : r;
  }
  constexpr int HW = C::WN / 2;
  const int wv = t / C::WN, u = t % C::WN;
  int64_t f = n0 + wv * HW + (u % HW);
  if (f > p.half_n - 1) f = p.half_n - 1;
  return (u >= HW ? p.half_n : 0) + f;
}

// Linear position of workgroup b in an XCD-aware order: the hardware hands
// workgroups to the 8 XCDs round-robin, so consecutive positions go to the
// same XCD and the tiles one XCD runs form a compact block.
__device__ __forceinline__ int xcd_linear(int b, int nb) {
  const int xcd = b & 7, q8 = nb >> 3, r8 = nb & 7;
  return (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + (b >> 3);
}

// Tile (tile_m, tile_n) of linear position bl: groups of group_m tile rows,
// column-major inside a group, so neighbouring positions share A and W panels.
__device__ __forceinline__ void grouped_tile(int bl, int tiles_m, int tiles_n, int group_m, int& tile_m,
                                             int& tile_n) {
  const int gsz = group_m * tiles_n;
  const int grp = bl / gsz;
  const int first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int inb = bl - grp * gsz;
  tile_m = first_m + inb % gm;
  tile_n = inb / gm;
}

// One output tile of the GEMM on the workgroup's LDS ring (sm0 .. sm3:
// C::STAGE bytes each; the first C::NSTAGE of them are used).
template <class C, int EPI, bool LOWRANK>
__device__ __forceinline__ void pipe_tile(const PArgs& p, int tile_m, int tile_n, uint8_t* const sm0,
                                          uint8_t* const sm1, uint8_t* const sm2, uint8_t* const sm3) {
  constexpr int NS = C::NSTAGE;
  auto ring = [&](int i) -> uint8_t* { return i == 0 ? sm0 : (i == 1 ? sm1 : (i == 2 ? sm2 : sm3)); };
  constexpr bool SWIG = EPI == EPI_SWIGLU;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform; readfirstlane keeps everything derived from it in SGPRs
  // (load bases, LDS destinations, branch conditions)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WGN;
  const int wn = wave % C::WGN;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int64_t m0 = (int64_t)tile_m * C::BM;
  const int64_t n0 = (int64_t)tile_n * (SWIG ? C::BN / 2 : C::BN);

  // row strides in bytes: a stage holds BKS channels of a row in ARB / WRB bytes
  const int64_t lda = p.K / C::BKS * C::ARB;
  const int64_t ldw = p.K / C::BKS * C::WRB;
  const int KT = (int)(p.K / C::BKS);

  // ---- global -> LDS loads -------------------------------------------------
  // Load t (0 .. NDMA-1) of this wave's share of stage kt: the first
  // A_PER_WAVE move A, the next W_HI move W, the rest move group scales.  A
  // burst of these right after a barrier stalls the wave on VMEM issue
  // while its MFMA pipe idles, so the main loop spreads them through the
  // MFMA stream.
  const bool w_hi = wave < C::W_SPLIT;
  constexpr int NDMA = C::NDMA;
  constexpr bool WPAIR = C::WP && !C::F6;  // packed INT4 weights: paired rows
  static_assert(!WPAIR || C::WRB == 64, "paired weight rows need 64-byte stage rows");
  // Per-lane byte offsets of every load slot, fixed for the whole K loop:
  // a load is a wave-uniform base (advanced by the stage) plus a 32-bit lane
  // offset, the global_load_lds saddr form, so issuing one costs no vector
  // address arithmetic.  (The host checks that the offsets fit in 32 bits.)
  // A slot t: 1 KB chunk q = wave + NW t of the A stage; W slot likewise;
  // scale slot: 64 floats at LDS position si * 64 (2*BM A-scale positions,
  // then 2*BN W-scale positions, then padding).  A-scale positions put the
  // FI rows a lane reads (i*16 + l16 of its wave row) next to each other;
  // W-scale positions are in tile-row order.
  const int64_t a_row0 = m0 * lda;
  uint32_t a_vo[C::A_PER_WAVE];
  // FP6 rows come in fours (rows 4q .. 4q + 3 interleaved per stage, 384
  // bytes) below M & ~3 and plain after, so a lane's stage advance is 384
  // or 96 bytes (m0 is a multiple of 4)
  uint32_t a_adv[C::F6 ? C::A_PER_WAVE : 1];
#pragma unroll
  for (int t = 0; t < C::A_PER_WAVE; ++t) {
    constexpr int CPR = C::ARB / 16;
    // FP6 rows (6 chunks) straddle the 1 KB loads: lane chunk -> row, chunk
    const int ci = (wave + C::NW * t) * 64 + lane;
    const int rl = C::F6 ? ci / CPR : (wave + C::NW * t) * (1024 / C::ARB) + lane / CPR;
    const int64_t gr = m0 + rl > p.M - 1 ? p.M - 1 : m0 + rl;
    const int ch = C::F6 ? swz6<C::M32>(rl, ci % CPR) : swz<C::ARB, C::GROUP, C::MX == 8>(rl, lane % CPR);
    a_vo[t] = (uint32_t)((gr - m0) * lda + (ch << 4));
    if constexpr (C::F6) {
      const bool quad = gr < (p.M & ~int64_t(3));
      if (quad) a_vo[t] = (uint32_t)(((gr - m0) >> 2) * 4 * lda + ((gr - m0) & 3) * 96 + (ch << 4));
      a_adv[t] = quad ? 4 * C::ARB : C::ARB;
    }
  }
  uint32_t w_vo[C::W_HI];
#pragma unroll
  for (int tw = 0; tw < C::W_HI; ++tw) {
    constexpr int CPR = C::WRB / 16;
    const int ci = (wave + C::NW * tw) * 64 + lane;
    const int rl = C::F6 ? ci / CPR : (wave + C::NW * tw) * (1024 / C::WRB) + lane / CPR;
    const int ch = C::F6 ? swz6<C::M32>(rl, ci % CPR) : swz<C::WRB, C::GROUP, C::MX == 8>(rl, lane % CPR);
    // packed INT4 weights: rows 2p, 2p + 1 interleaved per 128-channel stage
    // (64 bytes each), so a stage of two rows is one cache line
    const int64_t wr = w_row_of<C, SWIG>(p, n0, rl);
    // FP6 weights: rows 4q .. 4q + 3 interleaved per 128-channel stage (96
    // bytes each), so a stage of four rows is three whole cache lines (the
    // GEMM's N is a multiple of 16: whole fours only)
    w_vo[tw] = WPAIR  ? (uint32_t)((wr >> 1) * 2 * ldw + ((wr & 1) << 6) + (ch << 4))
               : C::F6 ? (uint32_t)((wr >> 2) * 4 * ldw + (wr & 3) * 96 + (ch << 4))
                       : (uint32_t)(wr * ldw + (ch << 4));
  }
  uint32_t s_vo[C::SCL ? C::S_PER_WAVE : 1];
#pragma unroll
  for (int ts = 0; ts < (C::SCL ? C::S_PER_WAVE : 0); ++ts) {
    const int pos = (wave + C::NW * ts) * 64 + lane;
    int64_t e = 0;  // float index relative to p.sa (A part) or p.sw (W part)
    if (C::MX) {
      // MX: position h (BM + BN) + pos holds the 4 scale bytes of tile row
      // pos (A rows, then W rows in tile-row order) for sub-stage h; e is
      // the byte offset of that row in slice h of the stage's first slice
      // of p.xa / p.xw (stage-major [K/128][rows][4]: the 64 rows of one
      // load are 256 consecutive bytes)
      const int h = pos / (C::BM + C::BN), pr = pos % (C::BM + C::BN);
      if (h < C::SUB && pr < C::BM) {
        const int64_t gr = m0 + pr > p.M - 1 ? p.M - 1 : m0 + pr;
        e = h * p.M * 4 + gr * 4;
      } else if (h < C::SUB) {
        e = h * p.N * 4 + w_row_of<C, SWIG>(p, n0, pr - C::BM) * 4;
      }
      s_vo[ts] = (uint32_t)e;
      continue;
    }
    if (pos < 2 * C::BM) {
      const int kk = pos / C::BM, rem = pos % C::BM;
      const int wv = rem / C::WM, u = rem % C::WM;
      // u = 64 f + 4 l16 + q holds the scale of fragment 4 f + q, lane row l16;
      // M32: u = 4 l32 + i holds the scale of 32-row fragment i, lane row l32
      const int row = C::M32 ? wv * C::WM + 32 * (u % 4) + u / 4
                             : wv * C::WM + (4 * (u / 64) + u % 4) * 16 + (u % 64) / 4;
      const int64_t gr = m0 + row > p.M - 1 ? p.M - 1 : m0 + row;
      e = kk * p.M + gr;  // scales are group-major: a stage's are contiguous per group
    } else if (pos < 2 * (C::BM + C::BN)) {
      const int pw = pos - 2 * C::BM;
      const int kk = pw / C::BN, trow = pw % C::BN;
      e = kk * p.N + w_row_of<C, SWIG>(p, n0, trow);
    }  // padding slots load the first W scale, never read back
    s_vo[ts] = (uint32_t)(e * 4);
  }
  // MX scale slices: bytes per stage (SUB 128-channel slices) of xa / xw
  const uint32_t xsa = (uint32_t)(p.M * 4 * C::SUB), xsw = (uint32_t)(p.N * 4 * C::SUB);
  // The stage advance goes into the 32-bit lane offset (one VALU add), so
  // the SGPR bases stay loop-invariant.
  const uint8_t* const a_base = p.a + a_row0;
  auto issue_one = [&](uint8_t* st, int kt, int t) {
    if (t < C::A_PER_WAVE) {
      const int q = wave + C::NW * t;
      if constexpr (C::F6) dma_b128(a_base, a_vo[t] + (uint32_t)kt * a_adv[t], st + q * 1024);
      else dma_b128(a_base, a_vo[t] + (uint32_t)(kt * C::ARB), st + q * 1024);
    } else if (t < C::A_PER_WAVE + C::W_HI) {
      const int tw = t - C::A_PER_WAVE;
      if (tw < C::W_HI - 1 || w_hi) {
        const int q = wave + C::NW * tw;
        dma_b128(p.w, w_vo[tw] + (uint32_t)(kt * (WPAIR ? 2 * C::WRB : (C::F6 ? 4 * C::WRB : C::WRB))),
                 st + C::SA + q * 1024);
      }
    } else if (C::MX) {
      const int ts = t - C::A_PER_WAVE - C::W_HI;
      const int si = wave + C::NW * ts;
      const int h0 = si * 64 / (C::BM + C::BN);
      const bool sa_side = h0 < C::SUB && si * 64 % (C::BM + C::BN) < C::BM;
      dma_b32(sa_side ? p.xa : p.xw, s_vo[C::SCL ? ts : 0] + (uint32_t)kt * (sa_side ? xsa : xsw),
              st + C::SA + C::SW + si * 256);
    } else if (C::GROUP) {
      const int ts = t - C::A_PER_WAVE - C::W_HI;
      const int si = wave + C::NW * ts;
      const bool sa_side = si * 64 < 2 * C::BM;
      dma_b32(sa_side ? p.sa : p.sw, s_vo[C::SCL ? ts : 0] + (uint32_t)kt * (sa_side ? p.sa_gs : p.sw_gs),
              st + C::SA + C::SW + si * 256);
    }
  };

  // int32 accumulators (tensor / row scales), fp32 sums of rescaled group
  // partials (group-64 scales), or fp32 sums of FP6 code products (exact
  // integers below 2^24).
  typedef typename AccOf<C::FMMA>::type acc_t;
  acc_t acc[C::GROUP ? 1 : C::FJ][C::GROUP ? 1 : C::FI];
  v4f yf[C::GROUP ? C::FJ : 1][C::GROUP ? C::FI : 1];
  // M32: the sums in the 32x32 instruction's layout (lane: one activation
  // row l32, weight rows 8 b + 4 (lane / 32) + t for register 4 b + t),
  // moved into yf's 16x16 layout after the K loop
  v16f y32[C::M32 ? C::FI32 : 1][C::M32 ? C::FJ32 : 1];
#pragma unroll
  for (int j = 0; j < C::FJ; ++j)
#pragma unroll
    for (int i = 0; i < C::FI; ++i) {
      if (C::GROUP && !C::M32) yf[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
      else if (!C::GROUP) acc[j][i] = acc_t{0, 0, 0, 0};
    }
  if constexpr (C::M32) {
#pragma unroll
    for (int i = 0; i < C::FI32; ++i)
#pragma unroll
      for (int j = 0; j < C::FJ32; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) y32[i][j][r] = 0.f;
  }

  // lane-constant LDS offsets: fragment rows differ by multiples of 16, so
  // the swizzle term depends on l16 only.
  static_assert(C::WM % 16 == 0 && C::WN % 16 == 0, "wave tile must be 16-aligned");
  const int a_row = wm * C::WM + l16;
  const int w_row = wn * C::WN + l16;
  // a_off[kk] / w_off, w_off1: fragment reads of half kk (b128); in the
  // group-64 map packed operands are read per half as b64 at a_off[kk] /
  // w_off (kk = 0) and w_off1 (kk = 1).
  static_assert(!C::GROUP || C::WP, "group-64 scales come with INT4 weights");
  constexpr bool GK = C::GROUP;
  int a_off[2];
  int w_off, w_off1;
  if (C::AP) {
    if (GK) {
      a_off[0] = a_row * 64 + (swz<64, GK>(a_row, lg >> 1) << 4) + 8 * (lg & 1);
      a_off[1] = a_row * 64 + (swz<64, GK>(a_row, 2 + (lg >> 1)) << 4) + 8 * (lg & 1);
    } else {
      a_off[0] = a_row * 64 + (swz<64, GK>(a_row, lg) << 4);
      a_off[1] = a_off[0];
    }
  } else {
    a_off[0] = a_row * 128 + (swz<128, GK>(a_row, GK ? lg : 2 * lg) << 4);
    a_off[1] = a_row * 128 + (swz<128, GK>(a_row, GK ? 4 + lg : 2 * lg + 1) << 4);
  }
  if (C::WP) {
    if (GK) {
      w_off = w_row * 64 + (swz<64, GK>(w_row, lg >> 1) << 4) + 8 * (lg & 1);
      w_off1 = w_row * 64 + (swz<64, GK>(w_row, 2 + (lg >> 1)) << 4) + 8 * (lg & 1);
    } else {
      w_off = w_row * 64 + (swz<64, GK>(w_row, lg) << 4);
      w_off1 = w_off;
    }
  } else {
    w_off = w_row * 128 + (swz<128, GK>(w_row, 2 * lg) << 4);
    w_off1 = w_row * 128 + (swz<128, GK>(w_row, 2 * lg + 1) << 4);
  }
  // FP6: sub-block lg of a 96-byte row, low 16 bytes at chunk lg, high 8
  // bytes in chunk 4 + lg / 2 (half lg % 2); fragment rows differ by
  // multiples of 16, which leaves the swizzle (row bits 2..3) unchanged.
  const int a6_hi = a_row * 96 + (swz6<C::M32>(a_row, lg) << 4);
  const int a6_lo = a_row * 96 + (swz6<C::M32>(a_row, 4 + (lg >> 1)) << 4) + 8 * (lg & 1);
  const int w6_hi = w_row * 96 + (swz6<C::M32>(w_row, lg) << 4);
  const int w6_lo = w_row * 96 + (swz6<C::M32>(w_row, 4 + (lg >> 1)) << 4) + 8 * (lg & 1);
  // M32: lane supplies row l32 (+ 32 per fragment) and the 32-channel
  // sub-block 2 kk + lane / 32 of group kk: 16 bytes at that chunk, 8 bytes
  // in chunk 4 + kk (half lane / 32).  Rows + 32 keep the swizzle.
  const int l32 = lane & 31, h32 = lane >> 5;
  const int a32_row = wm * C::WM + l32, w32_row = wn * C::WN + l32;
  int a32_hi[2], a32_lo[2], w32_hi[2], w32_lo[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    a32_hi[kk] = a32_row * 96 + (swz6<C::M32>(a32_row, 2 * kk + h32) << 4);
    a32_lo[kk] = a32_row * 96 + (swz6<C::M32>(a32_row, 4 + kk) << 4) + 8 * h32;
    w32_hi[kk] = w32_row * 96 + (swz6<C::M32>(w32_row, 2 * kk + h32) << 4);
    w32_lo[kk] = w32_row * 96 + (swz6<C::M32>(w32_row, 4 + kk) << 4) + 8 * h32;
  }
  // M32 scales: the lane's four 32-row fragments' s_a as one b128 at
  // position wm WM + 4 l32; its 16 weight rows' s_w as four b128 at tile
  // rows wn WN + 32 j + 8 b + 4 (lane / 32)
  const int sa32_off = (wm * C::WM + 4 * l32) * 4;
  const int sw32_off = (2 * C::BM + wn * C::WN + 4 * h32) * 4;
  // MX: lane group lg supplies K-block lg of the sub-stage (32 elements)
  // and its scale.  FP4: the block is the 16 bytes of chunk 4 h + lg.  FP8:
  // the instruction takes 16 elements of each of two blocks per lane -- K
  // [16 lg, 16 lg + 16) in its first four dwords and [64 + 16 lg, ...) in
  // the last four (measured on gfx950; the scale of lane group b still
  // covers K [32 b, 32 b + 32)), so the lane reads chunks lg and 4 + lg.
  // Packed INT4 (tensor / row scales): chunk 4 h + lg, both halves (kk).
  // Two sub-stages (MXFP4, packed INT4): sub-stage h, lane group lg takes
  // the 32 channels of chunk 2 lg + h of the 256-channel stage -- the chunk
  // pattern of the int8 reads (kk, 2 + kk, ...) that the swizzle serves
  // without bank conflicts; an MX lane's scale is byte (2 lg + h) % 4 of
  // slice lg / 2.
  constexpr bool MXI = (C::MX == 4 || (C::AP && C::WP && !C::GROUP)) && C::SUB == 2;
  int axp[C::SUB], wxp[C::SUB];
#pragma unroll
  for (int h = 0; h < C::SUB; ++h) {
    const int ch = MXI ? 2 * lg + h : 4 * h + lg;
    axp[h] = a_row * C::ARB + (swz<C::ARB, false, C::MX == 8>(a_row, ch) << 4);
    wxp[h] = w_row * C::WRB + (swz<C::WRB, false, C::MX == 8>(w_row, ch) << 4);
  }
  const int ax1 = a_row * C::ARB + (swz<C::ARB, false, C::MX == 8>(a_row, 4 + lg) << 4);
  const int wx1 = w_row * C::WRB + (swz<C::WRB, false, C::MX == 8>(w_row, 4 + lg) << 4);
  // group scales: byte offsets inside the stage's scale block.  A lane reads
  // the scales of its fragments 4f .. 4f+3 as one b128 at 64 f + 4 l16, so
  // the 16 lanes of a read sit at a 16-byte stride (no bank conflicts).
  const int sa_off = (wm * C::WM + l16 * 4) * 4;
  const int sw_off = (2 * C::BM + wn * C::WN + 4 * lg) * 4;

  // Staged epilogue: the tile's row factors (s_a * post) and column factors
  // (s_w, bias, gate) as one vector of NV floats, fetched cooperatively (NVT
  // per thread) before the K loop, so their latency hides under it; they
  // reach the other lanes through LDS.  Row factors are kept
  // in the order the lanes read them: tile row wm * WM + 16 i + l16 at
  // wm * WM + FI * l16 + i, so a lane's FI rows are contiguous.
  constexpr bool STAGED =
      (EPI == EPI_BF16 || EPI == EPI_GATED || EPI == EPI_SIGMOID) && !SWIG && !LOWRANK && C::WGM == 2;
  constexpr int NV = C::BM + (EPI == EPI_GATED ? 3 : 2) * C::BN;
  constexpr int NVT = STAGED ? (NV + C::NT - 1) / C::NT : 1;
  float vec[NVT];
  if constexpr (STAGED) {
#pragma unroll
    for (int u = 0; u < NVT; ++u) {
      const int e = tid + u * C::NT;
      float v = 0.f;
      if (e < C::BM) {
        const int64_t m = m0 + e > p.M - 1 ? p.M - 1 : m0 + e;
        v = C::NOSC ? p.post : p.sa[m * p.sa_stride] * p.post;
      } else if (e < NV) {
        const int f = (e - C::BM) / C::BN;
        const int64_t n = n0 + (e - C::BM) % C::BN > p.N - 1 ? p.N - 1 : n0 + (e - C::BM) % C::BN;
        if (f == 0) v = C::NOSC ? 1.f : p.sw[n * p.sw_stride];
        else if (f == 1) v = p.bias ? bf16_to_f32(p.bias[n]) : 0.f;
        else v = bf16_to_f32(p.gate[n]);
      }
      vec[u] = v;
    }
  }
  // prologue: stages 0 .. NS-2 in flight
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0)
    if (s0 < KT) {
#pragma unroll
      for (int t = 0; t < NDMA; ++t) issue_one(ring(s0), s0, t);
    }

  // Tensor / row scales: the MFMA group of a stage's last A fragment is
  // deferred into the next stage, right after its barrier and first
  // fragment reads, so the MFMA pipe has work while those reads are in
  // flight (both waves of a SIMD leave the barrier together and would
  // otherwise wait on them at the same time).  Its operands (the stage's
  // second-half W fragments and last A fragment) stay in registers.
  constexpr bool DEFER = !C::GROUP && C::WP && !C::F6 && !C::PP;  // int8 W: not enough registers
  v4i bw1[C::FJ];
  v4i af_def = v4i{0, 0, 0, 0};
  if constexpr (C::PP) {
    // Ping-pong K loop.  Waves w and w + 4 share a SIMD (measured: pairing
    // waves 2i and 2i + 1 instead runs 40 % slower); they form groups
    // gp = 0 (waves 0-3) and gp = 1 (waves 4-7) that run the same sequence
    // of phases per stage -- L0 C0 L1 C1, where L(kk) reads the fragments of
    // half kk from LDS (and issues some of the wave's global -> LDS loads of
    // stage kt + 2) and C(kk) runs its 40 MFMAs from registers -- one phase
    // apart: every phase ends at a workgroup barrier, and group 1 passes one
    // extra barrier before its first phase, group 0 one after its last.  So
    // while one wave of a SIMD issues MFMAs back to back, the other waits on
    // LDS and memory, and the MFMA stream does not stall on its own
    // fragment reads.
    // Slot 4 kt + p (p = 0..3) is group 0's phase p of stage kt and group
    // 1's phase p - 1.  Stage kt is read in slots 4 kt .. 4 kt + 4, the
    // loads of stage kt + 2 (into stage kt - 1's buffer, last read in slot
    // 4 kt - 1) are issued in slots 4 kt .. 4 kt + 3, and every wave waits
    // for its own loads of stage kt + 1 before the barrier that opens slot
    // 4 kt + 4 (group 0 after C1, group 1 after L1).
    // With a 2-stage ring (int8 W) the loads of stage kt + 1 go into stage
    // kt - 1's buffer during stage kt; all of them are issued in L0, so they
    // have two slots to land before the waits.
    const int gp = wave >> 2;
    if (NS == 3 && KT > 1) {
      if (w_hi) wait_vmcnt<NDMA>();
      else wait_vmcnt<NDMA - 1>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (gp == 1) __builtin_amdgcn_s_barrier();
    auto wait_next = [&](int kt) {
      if (NS == 3 && kt + 2 < KT) {
        if (w_hi) wait_vmcnt<NDMA>();
        else wait_vmcnt<NDMA - 1>();
      } else {
        wait_vmcnt<0>();
      }
    };
    v4i af[C::FI];
    v4i bw[C::FJ];
    uint2 whi[C::FJ];
    constexpr int H0 = NS == 3 ? (NDMA + 1) / 2 : NDMA;  // loads issued in L0; the rest in L1
    for (int kb = 0; kb < KT; kb += NS) {
#pragma unroll
      for (int sc = 0; sc < NS; ++sc) {
        const int kt = kb + sc;
        if (kt >= KT) break;
        const uint8_t* As = ring(sc);
        const uint8_t* Ws = As + C::SA;
        uint8_t* const nxt = ring((sc + NS - 1) % NS);
        const bool dma = kt + NS - 1 < KT;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          // L(kk)
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < C::FI; ++i) af[i] = *reinterpret_cast<const v4i*>(As + a_off[kk] + i * 16 * C::ARB);
          if (!C::WP) {
            // int8 W: one 16-byte read per fragment and half
#pragma unroll
            for (int j = 0; j < C::FJ; ++j)
              bw[j] = *reinterpret_cast<const v4i*>(Ws + (kk == 0 ? w_off : w_off1) + j * 16 * C::WRB);
          } else if (kk == 0) {
#pragma unroll
            for (int j = 0; j < C::FJ; ++j) {
              const uint4 r = *reinterpret_cast<const uint4*>(Ws + wxp[0] + j * 16 * C::WRB);
              bw[j] = unpack_lo(r.x, r.y);
              whi[j] = make_uint2(r.z, r.w);
            }
          } else {
#pragma unroll
            for (int j = 0; j < C::FJ; ++j) bw[j] = unpack_lo(whi[j].x, whi[j].y);
          }
          if (dma) {
#pragma unroll
            for (int t = kk == 0 ? 0 : H0; t < (kk == 0 ? H0 : NDMA); ++t) issue_one(nxt, kt + NS - 1, t);
          }
#pragma unroll
          for (int j = 0; j < C::FJ; ++j) asm volatile("" : "+v"(bw[j]));
#pragma unroll
          for (int i = 0; i < C::FI; ++i) asm volatile("" : "+v"(af[i]));
          if (kk == 1 && gp == 1 && kt + 1 < KT) wait_next(kt);
          lds_barrier();
          // C(kk)
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < C::FI; ++i)
#pragma unroll
            for (int j = 0; j < C::FJ; ++j) {
              acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bw[j], af[i], acc[j][i], 0, 0, 0);
              asm volatile("" : "+v"(acc[j][i]));
            }
          __builtin_amdgcn_sched_barrier(0);
          if (kk == 1 && gp == 0 && kt + 1 < KT) wait_next(kt);
          __builtin_amdgcn_s_barrier();
        }
      }
    }
    if (gp == 0) __builtin_amdgcn_s_barrier();
  } else {
  // M32 state carried across stages: the last step's partial is rescaled at
  // the next stage's first step, beside its first instruction, with group
  // 1's scales, which that stage reads only at its middle step.
  v4f sa4[C::M32 ? 2 : 1];
  v4f sw4[C::M32 ? 2 : 1][C::M32 ? C::FJ32 : 1][4];
  v16f part[C::M32 ? 2 : 1][C::M32 ? C::FJ32 : 1];
  if constexpr (C::M32) {
#pragma unroll
    for (int j = 0; j < C::FJ32; ++j) part[1][j] = v16f{};  // passes the first step's pin unused
  }
  auto rescale32 = [&](int st) {
    if constexpr (C::M32) {
      const int kk = st / C::FI32, i = st % C::FI32;
      const float s_i = sa4[kk][i];
#pragma unroll
      for (int j = 0; j < C::FJ32; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          y32[i][j][r] = __builtin_fmaf(part[st & 1][j][r], s_i * sw4[kk][j][r / 4][r % 4], y32[i][j][r]);
        asm volatile("" : "+v"(y32[i][j]));
      }
    }
  };
  for (int kb = 0; kb < KT; kb += NS) {
#pragma unroll
  for (int sc = 0; sc < NS; ++sc) {
    const int kt = kb + sc;
    if (kt >= KT) break;
    uint8_t* const cur = ring(sc);
    const int sn = (sc + NS - 1) % NS;  // stage that kt + NS - 1 lands in
    uint8_t* const nxt = ring(sn);
    // Stage kt has landed once only the later stages (at most NS-2 of them,
    // fewer at the end of K) are still in flight; the barrier then
    // publishes every wave's part and guarantees all waves finished reading
    // the buffer the next load reuses.
    if (NS >= 3 && kt + NS - 2 < KT) {
      if (w_hi) wait_vmcnt<(NS - 2) * NDMA>();
      else wait_vmcnt<(NS - 2) * (NDMA - 1)>();
    } else if (NS == 4 && kt + 1 < KT) {
      if (w_hi) wait_vmcnt<NDMA>();
      else wait_vmcnt<NDMA - 1>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    stage_prio(0);
    const bool dma = kt + NS - 1 < KT;

    if constexpr (C::MX) {
      // MX stage: one block-scaled 16x16x128 instruction per fragment pair
      // covers the stage's 128 channels; each lane passes the E8M0 scale of
      // its own row and block (byte lg of the row's 4 stage scales).
      const uint8_t* As = cur;
      const uint8_t* Ws = As + C::SA;
      const uint8_t* Ss = Ws + C::SW;
      constexpr int FMT = C::MX == 4 ? 4 : 0;  // instruction format: FP4 E2M1 | FP8 E4M3
      auto frag = [&](const uint8_t* base, int o0, int o1) -> v8i {
        const uint4 h = *reinterpret_cast<const uint4*>(base + o0);
        if (C::MX == 4) return v8i{(int)h.x, (int)h.y, (int)h.z, (int)h.w, 0, 0, 0, 0};
        const uint4 g = *reinterpret_cast<const uint4*>(base + o1);
        return v8i{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)g.x, (int)g.y, (int)g.z, (int)g.w};
      };
#pragma unroll
      for (int h = 0; h < C::SUB; ++h) {
        // the lane's scale byte: slice and byte of its block in this sub-stage
        const int sb = MXI ? (lg >> 1) * (C::BM + C::BN) * 4 + ((2 * lg + h) & 3)
                           : h * (C::BM + C::BN) * 4 + lg;
        v8i wf[C::FJ];
        int wsc[C::FJ];
#pragma unroll
        for (int j = 0; j < C::FJ; ++j) {
          wf[j] = frag(Ws + j * 16 * C::WRB, wxp[h], wx1);
          wsc[j] = Ss[sb + (C::BM + w_row + 16 * j) * 4];
        }
        // FP8 fragments are 8 dwords: a one-fragment read-ahead window keeps
        // the 256 x 320 tile's registers under the 256 a wave may hold
        constexpr int PF = C::MX == 8 ? 1 : 2;
        v8i abuf[PF + 1];
#pragma unroll
        for (int q = 0; q < PF; ++q) abuf[q] = frag(As + q * 16 * C::ARB, axp[h], ax1);
#pragma unroll
        for (int i = 0; i < C::FI; ++i) {
          const int step = h * C::FI + i;  // position in the stage's MFMA groups
          if (step > 0 && (4 * step) % (C::SUB * C::FI) < 4) stage_prio((4 * step) / (C::SUB * C::FI));
          if (i + PF < C::FI) abuf[(i + PF) % (PF + 1)] = frag(As + (i + PF) * 16 * C::ARB, axp[h], ax1);
          const int asc_i = Ss[sb + (a_row + 16 * i) * 4];
          if (dma && step < NDMA) issue_one(nxt, kt + NS - 1, step);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < C::FJ; ++j) {
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], abuf[i % (PF + 1)], acc[j][i],
                                                                        FMT, FMT, 0, wsc[j], 0, asc_i);
            asm volatile("" : "+v"(acc[j][i]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (dma) {
#pragma unroll
        for (int t = C::SUB * C::FI; t < NDMA; ++t) issue_one(nxt, kt + NS - 1, t);
      }
    } else if constexpr (C::M32) {
      // FP6 stage with group-64 scales on the 32x32x64 instruction: step
      // s = FI32 kk + i multiplies 32-row A fragment i with the wave's
      // 32-row W fragments over group kk (sub-blocks 2 kk and 2 kk + 1, one
      // per lane half), giving that group's exact partial of a 32 x 32 block
      // in fp32.  Its rescale y += part * (s_a * s_w) runs one step later,
      // beside the next step's instruction, so it does not wait on it.
      // Operands are read from LDS one step before their use (group kk's
      // W fragments and scales in the step before its first instruction):
      // the empty asm statements with a memory clobber keep each step's
      // reads in that step, and those on the partials and sums keep each
      // instruction and its rescale in their steps (otherwise the compiler hoists every
      // read of the stage above the first instruction, which then waits for
      // all of them, and sinks every rescale below the last instruction).
      const uint8_t* As = cur;
      const uint8_t* Ws = As + C::SA;
      const uint8_t* Ss = Ws + C::SW;
      auto frag6 = [&](const uint8_t* base, int hi, int lo) -> v8i {
        const uint4 h = *reinterpret_cast<const uint4*>(base + hi);
        const uint2 l = *reinterpret_cast<const uint2*>(base + lo);
        return v8i{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)l.x, (int)l.y, 0, 0};  // FP6 reads 6 dwords
      };
      v8i wf[2][C::FJ32];
      auto read_w = [&](int kk) {
#pragma unroll
        for (int j = 0; j < C::FJ32; ++j) wf[kk][j] = frag6(Ws + j * 32 * C::WRB, w32_hi[kk], w32_lo[kk]);
      };
      auto read_s = [&](int kk) {
        sa4[kk] = *reinterpret_cast<const v4f*>(Ss + sa32_off + kk * C::BM * 4);
#pragma unroll
        for (int j = 0; j < C::FJ32; ++j)
#pragma unroll
          for (int b = 0; b < 4; ++b)
            sw4[kk][j][b] = *reinterpret_cast<const v4f*>(Ss + sw32_off + (kk * C::BN + 32 * j + 8 * b) * 4);
      };
      constexpr int NSTEP = 2 * C::FI32;
      v8i abuf[2];
      read_w(0);
      abuf[0] = frag6(As, a32_hi[0], a32_lo[0]);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        const int kk = st / C::FI32;
        asm volatile("" ::: "memory");
        if (st > 0 && (4 * st) % NSTEP < 4) stage_prio((4 * st) / NSTEP);
        if (st + 1 < NSTEP)
          abuf[(st + 1) & 1] = frag6(As + ((st + 1) % C::FI32) * 32 * C::ARB, a32_hi[(st + 1) / C::FI32],
                                     a32_lo[(st + 1) / C::FI32]);
        if (st == 0) read_s(0);
        if (st == C::FI32 - 1) read_w(1);
        if (st == C::FI32) read_s(1);
        if (dma && st < NDMA) issue_one(nxt, kt + NS - 1, st);
#pragma unroll
        for (int j = 0; j < C::FJ32; ++j) {
          part[st & 1][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wf[kk][j], abuf[st & 1], v16f{}, 2, 2, 0, 127, 0, 127);
          // the previous step's partial passes through here too, so its
          // rescale comes after this instruction and overlaps it
          asm volatile("" : "+v"(part[st & 1][j]), "+v"(part[(st + 1) & 1][j]));
        }
        if (st > 0) rescale32(st - 1);
        else if (kt > 0) rescale32(NSTEP - 1);  // the previous stage's last step
      }
      if (dma) {
#pragma unroll
        for (int t = NSTEP; t < NDMA; ++t) issue_one(nxt, kt + NS - 1, t);
      }
    } else if constexpr (C::F6) {
      // FP6 stage: one 16x16x128 instruction per fragment pair covers the
      // stage's 128 channels.  W fragments are read whole; A fragments
      // stream through a window read PF ahead; the next stage's loads go
      // one per A fragment.
      const uint8_t* As = cur;
      const uint8_t* Ws = As + C::SA;
      v8i wf[C::FJ];
#pragma unroll
      for (int j = 0; j < C::FJ; ++j) {
        const uint4 h = *reinterpret_cast<const uint4*>(Ws + w6_hi + j * 16 * C::WRB);
        const uint2 l = *reinterpret_cast<const uint2*>(Ws + w6_lo + j * 16 * C::WRB);
        wf[j] = v8i{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)l.x, (int)l.y, 0, 0};  // FP6 reads 6 dwords
      }
      static_assert(!C::GROUP, "FP6 with group-64 scales runs the 32x32x64 (M32) form");
      constexpr int PF = 2;
      auto read_a = [&](int i) {
        const uint4 h = *reinterpret_cast<const uint4*>(As + a6_hi + i * 16 * C::ARB);
        const uint2 l = *reinterpret_cast<const uint2*>(As + a6_lo + i * 16 * C::ARB);
        return v8i{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)l.x, (int)l.y, 0, 0};
      };
      v8i abuf[PF + 1];
#pragma unroll
      for (int q = 0; q < PF; ++q) abuf[q] = read_a(q);
#pragma unroll
      for (int i = 0; i < C::FI; ++i) {
        if (i > 0 && (4 * i) % C::FI < 4) stage_prio((4 * i) / C::FI);
        if (i + PF < C::FI) abuf[(i + PF) % (PF + 1)] = read_a(i + PF);
        if (dma && i < NDMA) issue_one(nxt, kt + NS - 1, i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < C::FJ; ++j) {
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], abuf[i % (PF + 1)], acc[j][i],
                                                                      2, 2, 0, 127, 0, 127);
          // pin the group here: otherwise the compiler sinks every MFMA
          // below the loads' branches and must hold all A fragments at once
          asm volatile("" : "+v"(acc[j][i]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (dma) {
#pragma unroll
        for (int t = C::FI; t < NDMA; ++t) issue_one(nxt, kt + NS - 1, t);
      }
    } else {
      const uint8_t* As = cur;
      const uint8_t* Ws = As + C::SA;
      const uint8_t* Ss = Ws + C::SW;
      constexpr int PF = 2;
      constexpr int NQ = 2 * C::FI;
#pragma unroll
      for (int h = 0; h < C::SUB; ++h) {
      // W fragments: packed -> one b128 per fragment carries both halves (kk);
      // int8 -> one b128 per fragment and half.
      uint4 wraw[GK ? 1 : C::FJ];
      uint4 wraw1[(C::WP || GK) ? 1 : C::FJ];
      v4i bw0[C::FJ];
      if (GK) {
#pragma unroll
        for (int j = 0; j < C::FJ; ++j) {
          const uint2 h0 = *reinterpret_cast<const uint2*>(Ws + w_off + j * 16 * C::WRB);
          const uint2 h1 = *reinterpret_cast<const uint2*>(Ws + w_off1 + j * 16 * C::WRB);
          bw0[j] = unpack_lo(h0.x, h0.y);
          bw1[j] = unpack_lo(h1.x, h1.y);
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::FJ; ++j) {
          wraw[j] = *reinterpret_cast<const uint4*>(Ws + (C::WP ? wxp[h] : w_off) + j * 16 * C::WRB);
          if (!C::WP) wraw1[j] = *reinterpret_cast<const uint4*>(Ws + w_off1 + j * 16 * C::WRB);
        }
      }
      // A fragments: int8 -> streamed through a small window read PF ahead;
      // packed -> one b128 per fragment carries both halves.
      v4i abuf[PF + 1];
      // packed A (tensor / row scales): the 8-byte half kk of fragment i's
      // chunk, streamed through a window read PF ahead like int8 A
      uint2 pbuf[PF + 1];
      auto read_pa = [&](int qq) {
        return *reinterpret_cast<const uint2*>(As + axp[h] + 8 * (qq / C::FI) + (qq % C::FI) * 16 * C::ARB);
      };
      if (C::AP) {
        if (!GK) {
#pragma unroll
          for (int q = 0; q < PF; ++q) pbuf[q] = read_pa(q);
        }
      } else {
#pragma unroll
        for (int q = 0; q < PF; ++q)
          abuf[q] = *reinterpret_cast<const v4i*>(As + a_off[q / C::FI] + (q % C::FI) * 16 * C::ARB);
      }
      if (DEFER && kt > 0 && h == 0) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < C::FJ; ++j)
          acc[j][C::FI - 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bw1[j], af_def, acc[j][C::FI - 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Two sub-stages: both halves are unpacked at once (after the deferred
      // group, which still reads the previous high half), so the packed
      // words die here -- three copies of the W fragments do not fit.
      constexpr bool EARLY_W = C::SUB == 2 && C::WP && !GK;
      if (!GK) {
#pragma unroll
        for (int j = 0; j < C::FJ; ++j) {
          bw0[j] = C::WP ? unpack_lo(wraw[j].x, wraw[j].y)
                         : v4i{(int)wraw[j].x, (int)wraw[j].y, (int)wraw[j].z, (int)wraw[j].w};
          if (EARLY_W) bw1[j] = unpack_lo(wraw[j].z, wraw[j].w);
        }
      }
      v4f sav[C::GROUP ? C::FI / 4 : 1];
      v4f swv[C::GROUP ? C::FJ : 1];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int kk = q / C::FI, i = q % C::FI;
        const int step = h * NQ + q;  // position in the stage's MFMA groups
        if (step > 0 && (4 * step) % (C::SUB * NQ) < 4) stage_prio((4 * step) / (C::SUB * NQ));
        v4i af;
        if (C::AP && GK) {
          const uint2 h = *reinterpret_cast<const uint2*>(As + a_off[kk] + i * 16 * C::ARB);
          af = unpack_lo(h.x, h.y);
        } else if (C::AP) {
          if (q + PF < NQ) pbuf[(q + PF) % (PF + 1)] = read_pa(q + PF);
          af = unpack_lo(pbuf[q % (PF + 1)].x, pbuf[q % (PF + 1)].y);
        } else {
          if (q + PF < NQ)
            abuf[(q + PF) % (PF + 1)] = *reinterpret_cast<const v4i*>(
                As + a_off[(q + PF) / C::FI] + ((q + PF) % C::FI) * 16 * C::ARB);
          af = abuf[q % (PF + 1)];
        }
        if (dma && (step % 2) == 0 && step / 2 < NDMA) issue_one(nxt, kt + NS - 1, step / 2);
        // second-half W fragments, spread over the first half's MFMA groups
        if (!GK && !EARLY_W && kk == 0 && i < C::FJ)
          bw1[i] = C::WP ? unpack_lo(wraw[i].z, wraw[i].w)
                         : v4i{(int)wraw1[i].x, (int)wraw1[i].y, (int)wraw1[i].z, (int)wraw1[i].w};
        if (!GK && !EARLY_W && kk == 0 && i == C::FI - 1) {
#pragma unroll
          for (int j = C::FI; j < C::FJ; ++j)
            bw1[j] = C::WP ? unpack_lo(wraw[j].z, wraw[j].w)
                           : v4i{(int)wraw1[j].x, (int)wraw1[j].y, (int)wraw1[j].z, (int)wraw1[j].w};
        }
        if (!C::GROUP) {
          if (DEFER && q == NQ - 1 && h == C::SUB - 1) {
            af_def = af;  // issued after the next barrier (or after the loop)
          } else {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < C::FJ; ++j)
              acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kk == 0 ? bw0[j] : bw1[j], af, acc[j][i], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          if (i == 0) {
            // scales of group kk: s_a of the lane's FI rows, s_w of its 4
            // columns in each fragment
#pragma unroll
            for (int f = 0; f < C::FI / 4; ++f)
              sav[f] = *reinterpret_cast<const v4f*>(Ss + sa_off + (kk * C::BM + 64 * f) * 4);
#pragma unroll
            for (int j = 0; j < C::FJ; ++j)
              swv[j] = *reinterpret_cast<const v4f*>(Ss + sw_off + (kk * C::BN + j * 16) * 4);
          }
          const float s_i = sav[i / 4][i % 4];
          v4i part[C::FJ];
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < C::FJ; ++j)
            part[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kk == 0 ? bw0[j] : bw1[j], af, v4i{0, 0, 0, 0},
                                                            0, 0, 0);
#pragma unroll
          for (int j = 0; j < C::FJ; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              yf[j][i][r] = __builtin_fmaf((float)part[j][r], s_i * swv[j][r], yf[j][i][r]);
            // keep the rescale next to its MFMAs: without this the compiler
            // sinks every rescale below all of the stage's MFMAs and must hold
            // all their partials at once
            asm volatile("" : "+v"(yf[j][i]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      }  // sub-stages
      // any loads not yet issued (only if NDMA > SUB * NQ / 2)
      if (dma) {
#pragma unroll
        for (int t = C::SUB * NQ / 2; t < NDMA; ++t) issue_one(nxt, kt + NS - 1, t);
      }
    }
  }
  }
  if constexpr (C::M32) {
    if (KT > 0) rescale32(2 * C::FI32 - 1);  // the last stage's last step
  }
  }  // ping-pong / pipelined K loop
  stage_prio(3);  // back to the lowest priority for the epilogue

  // M32: move the sums from the 32x32 instruction's layout into yf's 16x16
  // layout through LDS (the ring is free once every wave is past the
  // barrier): each wave owns a 64 x 32 fp32 block (pitch 36 floats) in sm0
  // (waves 0-3) or sm1 (waves 4-7) and converts its 128 rows in two passes.
  if constexpr (C::M32) {
    constexpr int P = 36;
    static_assert(C::NW == 8 && C::FJ32 == 1 && C::FJ == 2 && C::FI == 8, "M32 epilogue: 8 waves of 128 x 32");
    static_assert(4 * 64 * P * 4 <= C::STAGE, "M32 blocks must fit one ring stage");
    lds_barrier();
    float* const blk = reinterpret_cast<float*>((wave < 4 ? sm0 : sm1) + (wave & 3) * (64 * P * 4));
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const v16f& y = y32[2 * pass + ii][0];
          *reinterpret_cast<v4f*>(blk + (32 * ii + l32) * P + 8 * b + 4 * h32) =
              v4f{y[4 * b], y[4 * b + 1], y[4 * b + 2], y[4 * b + 3]};
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i16 = 0; i16 < 4; ++i16)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          yf[j][4 * pass + i16] = *reinterpret_cast<const v4f*>(blk + (16 * i16 + l16) * P + 16 * j + 4 * lg);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }

  if constexpr (DEFER) {
    if (KT > 0) {
#pragma unroll
      for (int j = 0; j < C::FJ; ++j)
        acc[j][C::FI - 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bw1[j], af_def, acc[j][C::FI - 1], 0, 0, 0);
    }
  }

  // ---- staged epilogue (plain bf16, sigmoid gate, gated residual) ----------
  // A lane holds 4 consecutive columns of one row per fragment, so direct
  // stores write 32-byte row pieces, and the 128-byte lines that two wave
  // columns share reach memory in parts.  Instead the tile goes through LDS
  // (the ring is free now) two bands of rows at a time, one per wave row,
  // and leaves as whole rows with 16-byte stores.  bf16 output (plain or
  // through the sigmoid of the attention gate): the bands hold finished bf16
  // values (four bands of BM/4 rows).  Gated residual: the bands hold y in
  // fp32 (eight bands of BM/8 rows), and the copy-out reads the residual with the same
  // coalesced 16-byte accesses, so out = res + gate * y is still rounded
  // once.
  if constexpr (STAGED) {
    constexpr bool F32 = EPI == EPI_GATED;
    constexpr int EB = F32 ? 4 : 2;          // staged bytes per value
    constexpr int NB = F32 ? 8 : 4;          // bands; round p stages bands p and NB / 2 + p
    constexpr int HR = C::BM / NB;           // rows per band
    constexpr int FPB = C::FI * 2 / NB;      // fragments of a wave per band (FI * 16 = BM / 2)
    constexpr int RB = C::BN * EB;           // staged bytes of one tile row
    constexpr int PITCH = RB + 16;           // LDS row pitch
    constexpr int RPA = (2 * HR + NS - 1) / NS;  // staging rows per ring array (two bands per round)
    static_assert(C::FI * 16 * 2 == C::BM && (C::FI * 2) % NB == 0, "bands cover whole fragments");
    static_assert(RPA * PITCH <= C::STAGE, "staging rows must fit the ring");
    // the factor vector sits behind the staging rows of the last ring array
    constexpr int SVOFF = (RPA * PITCH + 15) / 16 * 16;
    static_assert(SVOFF + 4 * NV <= C::STAGE, "factor vector must fit the ring");
    float* const sv = reinterpret_cast<float*>(ring(NS - 1) + SVOFF);
    auto row_ptr = [&](int r) -> uint8_t* {
      const int a = r / RPA, o = (r % RPA) * PITCH;
      return ring(a) + o;
    };
    // The band barriers below order LDS only (lds_barrier: the wave's LDS
    // accesses complete, then s_barrier).  __syncthreads would also wait for
    // every global store issued so far, stalling each band on the previous
    // band's writes to memory.
    lds_barrier();  // every wave is done with the ring (its loads all landed)
#pragma unroll
    for (int u = 0; u < NVT; ++u) {
      const int e = tid + u * C::NT;
      if (e < C::BM) {
        const int w = e / C::WM, r = e % C::WM;
        sv[w * C::WM + (r % 16) * C::FI + r / 16] = vec[u];
      } else if (e < NV) {
        sv[e] = vec[u];
      }
    }
    lds_barrier();
    constexpr int CH = C::BN / 8;  // 8-column chunks per row (16 bf16 bytes out)
    constexpr int NIT = (2 * HR * CH + C::NT - 1) / C::NT;  // copy-out chunks per thread and round
#pragma unroll
    for (int band = 0; band < NB / 2; ++band) {
      // gated residual: the round's residual chunks are loaded before its
      // bands are staged, so their memory latency passes during the staging
      // (loaded inside the copy-out, each wave waited for them one at a time)
      uint4 rres[F32 ? NIT : 1];
      if constexpr (F32) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int c = tid + it * C::NT;
          const int r = c / CH, ch = c % CH;
          const int64_t m = m0 + (r < HR ? band * HR + r : C::BM / 2 + band * HR + (r - HR));
          const int64_t n = n0 + ch * 8;
          rres[it] = (c < 2 * HR * CH && m < p.M && n < p.N)
                         ? *reinterpret_cast<const uint4*>(p.residual + m * p.ldo + n)
                         : make_uint4(0, 0, 0, 0);
        }
      }
      // both wave rows stage at once: wave row wm its band wm * NB / 2 + band
      // (fragments i0 .. i0 + FPB - 1) into staging rows wm * HR + ...
      {
        const int i0 = band * FPB;
        float samv[FPB];
#pragma unroll
        for (int f = 0; f < FPB; ++f) samv[f] = sv[wm * C::WM + l16 * C::FI + i0 + f];
#pragma unroll
        for (int j = 0; j < C::FJ; ++j) {
          const int col = wn * C::WN + j * 16 + lg * 4;   // tile column
          const float4 sw4 = *reinterpret_cast<const float4*>(sv + C::BM + col);
          const float4 ad4 = *reinterpret_cast<const float4*>(sv + C::BM + C::BN + col);
          const float swv[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
          const float addv[4] = {ad4.x, ad4.y, ad4.z, ad4.w};
#pragma unroll
          for (int ii = 0; ii < FPB; ++ii) {
            const int i = i0 + ii;
            const float sam = samv[ii];
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = C::GROUP ? yf[C::GROUP ? j : 0][C::GROUP ? i : 0][r]
                                       : (float)acc[C::GROUP ? 0 : j][C::GROUP ? 0 : i][r];
              y[r] = v * sam * swv[r] + addv[r];
              if (EPI == EPI_SIGMOID) y[r] = 1.0f / (1.0f + __expf(-y[r]));  // the attention gate
            }
            uint8_t* dst = row_ptr(wm * HR + ii * 16 + l16) + col * EB;
            if (F32) {
              *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
            } else {
              const bf2 h0 = __builtin_convertvector(f2{y[0], y[1]}, bf2);
              const bf2 h1 = __builtin_convertvector(f2{y[2], y[3]}, bf2);
              *reinterpret_cast<uint2*>(dst) =
                  make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
            }
          }
        }
      }
      lds_barrier();
      // Output rows leave with nontemporal stores: nothing reads them in this
      // kernel, and streaming them past L2 allocation measured 3-4 % faster.
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int c = tid + it * C::NT;
        if (c >= 2 * HR * CH) break;
        const int r = c / CH, ch = c % CH;
        const int64_t m = m0 + (r < HR ? band * HR + r : C::BM / 2 + band * HR + (r - HR));
        const int64_t n = n0 + ch * 8;  // 16 | N: a chunk is wholly in or out
        if (m >= p.M || n >= p.N) continue;
        uint16_t* o = static_cast<uint16_t*>(p.out) + m * p.ldo + n;
        if (F32) {
          const float4 y0 = *reinterpret_cast<const float4*>(row_ptr(r) + ch * 32);
          const float4 y1 = *reinterpret_cast<const float4*>(row_ptr(r) + ch * 32 + 16);
          const uint4 rr = rres[F32 ? it : 0];
          const float4 g0 = *reinterpret_cast<const float4*>(sv + C::BM + 2 * C::BN + ch * 8);
          const float4 g1 = *reinterpret_cast<const float4*>(sv + C::BM + 2 * C::BN + ch * 8 + 4);
          const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
          const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
          const uint32_t rw[4] = {rr.x, rr.y, rr.z, rr.w};
          uint32_t ow[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a0 = __builtin_fmaf(gv[2 * e], yv[2 * e], bf16_to_f32(rw[e] & 0xffff));
            const float a1 = __builtin_fmaf(gv[2 * e + 1], yv[2 * e + 1], bf16_to_f32(rw[e] >> 16));
            ow[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a0, a1}, bf2));
          }
          __builtin_nontemporal_store(v4u{ow[0], ow[1], ow[2], ow[3]}, reinterpret_cast<v4u*>(o));
        } else {
          __builtin_nontemporal_store(*reinterpret_cast<const v4u*>(row_ptr(r) + ch * 16), reinterpret_cast<v4u*>(o));
        }
      }
      lds_barrier();
    }
    return;
  }

  // ---- epilogue: lane holds out[m][n .. n+3] for each (i, j) --------------
  // Low-rank branch: L2 is stored [N, rank] (row n: the rank vector of
  // weight row / output column n), so a lane's 8 consecutive ranks of one
  // weight row are one 16-byte load -- the first MFMA operand as it is.
  // MX and group-64 tiles: the lr fragments of ranks 0 .. 31 for all FI
  // rows are loaded here, ahead of the column loop (they do not depend on
  // the output columns); later 32-rank chunks, and every chunk of the other
  // tiles (whose epilogues have no registers to spare), are loaded per half
  // of the rows.
  constexpr bool PRE_LR = LOWRANK && (C::MX != 0 || C::GROUP);
  uint4 ua0[PRE_LR ? C::FI : 1];
  if constexpr (PRE_LR) {
    const int kc = lg * 8;
#pragma unroll
    for (int i = 0; i < C::FI; ++i) {
      int64_t mc = m0 + wm * C::WM + i * 16 + l16;
      if (mc > p.M - 1) mc = p.M - 1;
      ua0[i] = kc < p.rank ? *reinterpret_cast<const uint4*>(p.lr + mc * p.rank + kc) : make_uint4(0, 0, 0, 0);
    }
  }
  // SwiGLU pairs fragment j (gate) with j + FJ/2 (up) of the same outputs.
  constexpr int NJ = SWIG ? C::FJ / 2 : C::FJ;
  static_assert(!SWIG || C::FJ % 2 == 0, "SwiGLU needs gate/up fragment pairs");
  // Loads are issued ahead of their use (rows past M read row M-1) so a
  // wave keeps many in flight instead of waiting on one per output.
  float sam[C::FI];
#pragma unroll
  for (int i = 0; i < C::FI; ++i) {
    int64_t m = m0 + wm * C::WM + i * 16 + l16;
    if (m > p.M - 1) m = p.M - 1;
    sam[i] = (C::NOSC || EPI == EPI_I32) ? p.post : p.sa[m * p.sa_stride] * p.post;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int t0 = wn * C::WN + j * 16;          // first W-tile row of fragment j
    const int64_t n = SWIG ? n0 + wn * (C::WN / 2) + j * 16 + lg * 4 : n0 + t0 + lg * 4;
    if (n >= (SWIG ? p.half_n : p.N)) continue;  // 4 | 16 | N: all four columns valid
    // weight-side values of the lane's 4 columns (gate side, and up side)
    float swv[2][4], addv[2][4], gatev[4];
#pragma unroll
    for (int h = 0; h < (SWIG ? 2 : 1); ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t wr = SWIG ? (h ? p.half_n : 0) + n + r : n + r;
        swv[h][r] = (C::NOSC || EPI == EPI_I32) ? 1.f : p.sw[wr * p.sw_stride];
        addv[h][r] = p.bias ? bf16_to_f32(p.bias[wr]) : 0.f;
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) gatev[r] = EPI == EPI_GATED ? bf16_to_f32(p.gate[n + r]) : 0.f;
    // L2 fragments (first MFMA operand): the lane supplies ranks k0 + 8 lg ..
    // + 7 of the L2 row of W-tile row t0 + l16 (and of its up partner
    // t0 + WN/2 + l16); ranks 0 .. 31 are loaded here.  The skip above is
    // uniform over the wave (16 | N, 16 | F), so every lane reaches the MFMAs
    // below.
    const uint16_t* l2row[2];
    l2row[0] = p.l2 + w_row_of<C, SWIG>(p, n0, t0 + l16) * p.rank;
    l2row[1] = p.l2 + w_row_of<C, SWIG>(p, n0, SWIG ? t0 + C::WN / 2 + l16 : t0 + l16) * p.rank;
    uint4 wv0[LOWRANK ? (SWIG ? 2 : 1) : 1];
    if constexpr (LOWRANK) {
#pragma unroll
      for (int h = 0; h < (SWIG ? 2 : 1); ++h)
        wv0[h] = lg * 8 < p.rank ? *reinterpret_cast<const uint4*>(l2row[h] + lg * 8) : make_uint4(0, 0, 0, 0);
    }
    uint2 res[EPI == EPI_GATED ? C::FI : 1];
    if (EPI == EPI_GATED) {
#pragma unroll
      for (int i = 0; i < C::FI; ++i) {
        int64_t m = m0 + wm * C::WM + i * 16 + l16;
        if (m > p.M - 1) m = p.M - 1;
        res[i] = *reinterpret_cast<const uint2*>(p.residual + m * p.ldo + n);
      }
    }

    // The rows in two halves (IB fragments each).  Low-rank branch first,
    // with every lane active: an MFMA mixes all 64 lanes' operands, so rows
    // past M load row M-1 instead of skipping.  lr[m, :] . L2[:, cols] with
    // bf16 MFMA 16x16x32 over the rank; per 32-rank chunk the lr fragments
    // of the half's rows are loaded together, so one memory latency covers
    // them (loaded next to the output stores of the row loop below, each
    // would wait for its own).
    constexpr int IB = C::FI >= 2 ? C::FI / 2 : 1;
#pragma unroll
    for (int ib = 0; ib < C::FI; ib += IB) {
    v4f lrv[LOWRANK ? IB : 1][SWIG ? 2 : 1];
#pragma unroll
    for (int i = 0; i < (LOWRANK ? IB : 1); ++i)
#pragma unroll
      for (int h = 0; h < (SWIG ? 2 : 1); ++h) lrv[i][h] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (LOWRANK) {
      for (int k0 = 0; k0 < p.rank; k0 += 32) {
        const int kc = k0 + lg * 8;
        const bool kin = kc < p.rank;
        uint4 ua[IB];
#pragma unroll
        for (int i = 0; i < IB; ++i) {
          if (PRE_LR && k0 == 0) {
            ua[i] = ua0[PRE_LR ? ib + i : 0];
          } else {
            int64_t mc = m0 + wm * C::WM + (ib + i) * 16 + l16;
            if (mc > p.M - 1) mc = p.M - 1;
            ua[i] = kin ? *reinterpret_cast<const uint4*>(p.lr + mc * p.rank + kc) : make_uint4(0, 0, 0, 0);
          }
        }
        uint4 wv[SWIG ? 2 : 1];
#pragma unroll
        for (int h = 0; h < (SWIG ? 2 : 1); ++h)
          wv[h] = k0 == 0 ? wv0[h] : (kin ? *reinterpret_cast<const uint4*>(l2row[h] + kc) : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int i = 0; i < IB; ++i)
#pragma unroll
          for (int h = 0; h < (SWIG ? 2 : 1); ++h)
            lrv[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, wv[h]),
                                                                __builtin_bit_cast(v8bf, ua[i]), lrv[i][h], 0, 0, 0);
      }
    }

#pragma unroll
    for (int i = ib; i < ib + IB; ++i) {
      const int64_t m = m0 + wm * C::WM + i * 16 + l16;
      if (m >= p.M) continue;
      if (EPI == EPI_I32) {
        const acc_t a4 = acc[C::GROUP ? 0 : j][C::GROUP ? 0 : i];  // FP6: exact integers in fp32
        int4 o;
        o.x = (int)a4[0] >> p.shift;
        o.y = (int)a4[1] >> p.shift;
        o.z = (int)a4[2] >> p.shift;
        o.w = (int)a4[3] >> p.shift;
        *reinterpret_cast<int4*>(static_cast<int32_t*>(p.out) + m * p.ldo + n) = o;
        continue;
      }
      float y[2][4];
#pragma unroll
      for (int h = 0; h < (SWIG ? 2 : 1); ++h) {
        const int jj = j + h * (C::FJ / 2);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = C::GROUP ? yf[C::GROUP ? jj : 0][C::GROUP ? i : 0][r]
                                   : (float)acc[C::GROUP ? 0 : jj][C::GROUP ? 0 : i][r];
          y[h][r] = v * sam[i] * swv[h][r] + addv[h][r] + (LOWRANK ? lrv[LOWRANK ? i - ib : 0][SWIG ? h : 0][r] : 0.f);
        }
      }
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = y[0][r];
      if (EPI == EPI_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + m * p.ldo + n) =
            make_float4(o[0], o[1], o[2], o[3]);
        continue;
      }
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[r] = y[0][r] * __builtin_amdgcn_rcpf(1.0f + __expf(-y[0][r])) * y[1][r];  // silu(gate) * up
      }
      if (EPI == EPI_GATED) {
        const uint2 rr = res[EPI == EPI_GATED ? i : 0];
        o[0] = __builtin_fmaf(gatev[0], o[0], bf16_to_f32(rr.x & 0xffff));
        o[1] = __builtin_fmaf(gatev[1], o[1], bf16_to_f32(rr.x >> 16));
        o[2] = __builtin_fmaf(gatev[2], o[2], bf16_to_f32(rr.y & 0xffff));
        o[3] = __builtin_fmaf(gatev[3], o[3], bf16_to_f32(rr.y >> 16));
      }
      const bf2 h0 = __builtin_convertvector(f2{o[0], o[1]}, bf2);
      const bf2 h1 = __builtin_convertvector(f2{o[2], o[3]}, bf2);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + m * p.ldo + n) =
          make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
    }
    }  // row halves
  }
}

template <class C, int EPI, bool LOWRANK>
__global__ __launch_bounds__(C::NT, 1) void qgemm_pipe_kernel(PArgs p) {
  // the LDS ring: one array per stage
  __shared__ __attribute__((aligned(16))) uint8_t sm0[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm2[C::NSTAGE >= 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sm3[C::NSTAGE == 4 ? C::STAGE : 16];
  int tile_m, tile_n;
  grouped_tile(xcd_linear(blockIdx.x, p.tiles_m * p.tiles_n), p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
  pipe_tile<C, EPI, LOWRANK>(p, tile_m, tile_n, sm0, sm1, sm2, sm3);
}

template <class C, int EPI, bool LOWRANK>
hipError_t launch_pipe(PArgs p, hipStream_t s) {
  p.tiles_m = (int)((p.M + C::BM - 1) / C::BM);
  p.tiles_n = EPI == EPI_SWIGLU ? (int)((p.half_n + C::BN / 2 - 1) / (C::BN / 2))
                                : (int)((p.N + C::BN - 1) / C::BN);
  p.group_m = 4;
  const int nb = p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL((qgemm_pipe_kernel<C, EPI, LOWRANK>), dim3(nb), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

// Tensor / row scales without low-rank branch: BF16 | F32 | I32 | GATED.
template <class C>
hipError_t launch_plain(const PArgs& p, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_BF16: return launch_pipe<C, EPI_BF16, false>(p, s);
    case EPI_F32: return launch_pipe<C, EPI_F32, false>(p, s);
    case EPI_I32: return launch_pipe<C, EPI_I32, false>(p, s);
    case EPI_GATED: return launch_pipe<C, EPI_GATED, false>(p, s);
    case EPI_SIGMOID: return launch_pipe<C, EPI_SIGMOID, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// INT4 weights with group-64 scales, SwiGLU and/or the low-rank branch:
// BF16 | F32 | SWIGLU, each with or without the branch.
template <class C>
hipError_t launch_lowrank(const PArgs& p, int epi, hipStream_t s) {
  const bool lr = p.rank > 0;
  switch (epi) {
    case EPI_BF16: return lr ? launch_pipe<C, EPI_BF16, true>(p, s) : launch_pipe<C, EPI_BF16, false>(p, s);
    case EPI_F32: return lr ? launch_pipe<C, EPI_F32, true>(p, s) : launch_pipe<C, EPI_F32, false>(p, s);
    case EPI_SWIGLU:
      return lr ? launch_pipe<C, EPI_SWIGLU, true>(p, s) : launch_pipe<C, EPI_SWIGLU, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// MX operands: BF16 | F32 | GATED | SIGMOID on the given tile, SwiGLU on
// 256 x 256 tiles (gate/up fragment pairs); with the low-rank branch
// (rank > 0) BF16 | F32 on the given tile and SwiGLU on 256 x 256.
template <class C, class CS>
hipError_t launch_mx(const PArgs& p, int epi, hipStream_t s) {
  if (p.rank > 0) {
    switch (epi) {
      case EPI_BF16: return launch_pipe<C, EPI_BF16, true>(p, s);
      case EPI_F32: return launch_pipe<C, EPI_F32, true>(p, s);
      case EPI_SWIGLU: return launch_pipe<CS, EPI_SWIGLU, true>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case EPI_BF16: return launch_pipe<C, EPI_BF16, false>(p, s);
    case EPI_F32: return launch_pipe<C, EPI_F32, false>(p, s);
    case EPI_GATED: return launch_pipe<C, EPI_GATED, false>(p, s);
    case EPI_SIGMOID: return launch_pipe<C, EPI_SIGMOID, false>(p, s);
    case EPI_SWIGLU: return launch_pipe<CS, EPI_SWIGLU, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// ---- grouped GEMM: several projections of one input in one launch --------
// (model card "Krea 2 Turbo OrbitQuant W4A4", section "Fused transformer
// (OrbitQuant 0.11)": one grouped Q|K|V|gate W4A4 GEMM per block with the
// sigmoid gate in its epilogue, the INT8 projections kept inside the group.)
// Each segment is a [M x n] product with its own weights, per-row scales,
// precision (packed INT4 or INT8 weights; int8-container INT4 or INT8
// activation codes, per-token scales) and epilogue (bf16 or sigmoid).  The
// tiles of all segments form one grid, so the small projections fill the
// large ones' last wave instead of leaving their own tail.  Each segment
// uses 256 x 320 or 256 x 256 tiles, whichever pads its columns less (320 on
// a tie), like a single launch; a workgroup runs the tile body of its
// segment's format and width on one LDS buffer sized for the largest ring.
// The four bodies run the ping-pong K loop; together they need 256 VGPRs
// and spill a few values outside the K loops (measured on gfx950: level with
// separate launches, where the pipelined bodies ran 3-7 % slower).
using CfgG4W = Cfg<256, 320, 2, 4, false, true, false, false, 0, 3, 1, true>;
using CfgG4N = Cfg<256, 256, 2, 4, false, true, false, false, 0, 3, 1, true>;
using CfgG8W = Cfg<256, 320, 2, 4, false, false, false, false, 0, 3, 1, true>;
using CfgG8N = Cfg<256, 256, 2, 4, false, false, false, false, 0, 3, 1, true>;
template <class C>
constexpr int ring_bytes() { return C::NSTAGE * C::STAGE; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kGroupedLds = cmax(cmax(ring_bytes<CfgG4W>(), ring_bytes<CfgG4N>()),
                                 cmax(ring_bytes<CfgG8W>(), ring_bytes<CfgG8N>()));
static_assert(kGroupedLds <= kLdsBytes, "grouped LDS ring too large");

// the segment's tile body on the shared ring
template <class C>
__device__ __forceinline__ void grouped_body(const PArgs& p, int tile_m, int tile_n, bool sigmoid,
                                             uint8_t* const r) {
  uint8_t* const r2 = C::NSTAGE >= 3 ? r + 2 * C::STAGE : r;
  uint8_t* const r3 = C::NSTAGE == 4 ? r + 3 * C::STAGE : r;
  if (sigmoid) pipe_tile<C, EPI_SIGMOID, false>(p, tile_m, tile_n, r, r + C::STAGE, r2, r3);
  else pipe_tile<C, EPI_BF16, false>(p, tile_m, tile_n, r, r + C::STAGE, r2, r3);
}

struct GSeg {
  const uint8_t* w;
  const float* sw;
  void* out;
  int64_t ldo;
  int64_t n;
  int w8;        // 1: int8 weights and int8 activation codes
  int sigmoid;   // 1: sigmoid epilogue
  int wide;      // 1: 256 x 320 tiles, 0: 256 x 256
  int tiles_n;
  int tile0;     // first linear tile of the segment
};

struct GArgs {
  PArgs base;    // M, K, the activation operands of segment 0, group_m, tiles_m
  const uint8_t* a4;
  const float* sa4;
  const uint8_t* a8;
  const float* sa8;
  int nseg;
  int ntiles;
  GSeg seg[kMaxGroupSegments];
};

__global__ __launch_bounds__(512, 1) void qgemm_grouped_kernel(GArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kGroupedLds];
  const int bl = xcd_linear(blockIdx.x, g.ntiles);
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroupSegments; ++i)
    if (i < g.nseg && bl >= g.seg[i].tile0) si = i;
  const GSeg& sg = g.seg[si];
  PArgs p = g.base;
  p.a = sg.w8 ? g.a8 : g.a4;
  p.sa = sg.w8 ? g.sa8 : g.sa4;
  p.w = sg.w;
  p.sw = sg.sw;
  p.N = sg.n;
  p.half_n = sg.n / 2;
  p.out = sg.out;
  p.ldo = sg.ldo;
  p.tiles_n = sg.tiles_n;
  p.post = sg.w8 ? 1.0f : 1.0f / 16.0f;
  p.shift = sg.w8 ? 0 : 4;
  int tile_m, tile_n;
  grouped_tile(bl - sg.tile0, p.tiles_m, sg.tiles_n, p.group_m, tile_m, tile_n);
  const bool sig = sg.sigmoid != 0;
  if (sg.w8) {
    if (sg.wide) grouped_body<CfgG8W>(p, tile_m, tile_n, sig, lds);
    else grouped_body<CfgG8N>(p, tile_m, tile_n, sig, lds);
  } else {
    if (sg.wide) grouped_body<CfgG4W>(p, tile_m, tile_n, sig, lds);
    else grouped_body<CfgG4N>(p, tile_m, tile_n, sig, lds);
  }
}

}  // namespace

int launch_qgemm_grouped(const GroupedArgs& ga, hipStream_t s) {
  if (ga.M == 0) return OK;
  GArgs g{};
  g.base.M = ga.M;
  g.base.K = ga.K;
  g.base.sa_stride = 1;
  g.base.sw_stride = 1;
  g.base.kg = (int)(ga.K >> 6);
  g.base.tiles_m = (int)((ga.M + 255) / 256);
  g.base.group_m = 4;
  g.a4 = static_cast<const uint8_t*>(ga.a4);
  g.sa4 = ga.sa4;
  g.a8 = static_cast<const uint8_t*>(ga.a8);
  g.sa8 = ga.sa8;
  g.nseg = ga.nseg;
  int t = 0;
  for (int i = 0; i < ga.nseg; ++i) {
    GSeg& d = g.seg[i];
    const GroupSegment& src = ga.seg[i];
    d.w = static_cast<const uint8_t*>(src.w);
    d.sw = src.sw;
    d.out = src.out;
    d.ldo = src.ldo;
    d.n = src.n;
    d.w8 = src.w_bits == 8 ? 1 : 0;
    d.sigmoid = src.epilogue == EPI_SIGMOID ? 1 : 0;
    const int64_t pad320 = (src.n + 319) / 320 * 320 - src.n, pad256 = (src.n + 255) / 256 * 256 - src.n;
    d.wide = pad320 <= pad256 ? 1 : 0;
    d.tiles_n = (int)(d.wide ? (src.n + 319) / 320 : (src.n + 255) / 256);
    d.tile0 = t;
    t += g.base.tiles_m * d.tiles_n;
  }
  g.ntiles = t;
  hipLaunchKernelGGL(qgemm_grouped_kernel, dim3(t), dim3(512), 0, s, g);
  return hipGetLastError() == hipSuccess ? OK : ERR_LAUNCH;
}

int launch_qgemm(const GemmArgs& g, hipStream_t s) {
  if (g.M == 0) return OK;
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
  p.kg = (int)(g.K >> 6);
  p.sa_gs = (uint32_t)(8 * g.M);
  p.sw_gs = (uint32_t)(8 * g.N);
  p.bias = g.bias;
  p.residual = g.residual;
  p.gate = g.gate;
  p.lr = g.lr;
  p.l2 = g.l2;
  p.rank = g.rank;
  p.out = g.out;
  p.ldo = g.ldo;
  p.half_n = g.N / 2;
  const int npacked = (g.a_packed ? 1 : 0) + (g.w_packed ? 1 : 0);
  p.post = npacked == 2 ? 1.0f / 256.0f : (npacked == 1 ? 1.0f / 16.0f : 1.0f);
  p.shift = 4 * npacked;
  const bool group = g.a_mode == 2;
  hipError_t e;
  // 256 x 320 tiles unless 256 x 256 needs fewer tile-area waves on the
  // 256 CUs (one workgroup per CU): time ~ waves * tile area.
  auto cost = [&](int64_t bn) {
    const int64_t tiles = ((g.M + 255) / 256) * ((g.N + bn - 1) / bn);
    return ((tiles + 255) / 256) * 256 * bn;
  };
  const bool wide = cost(320) <= cost(256);
  if (g.mx) {
    // the block-scaled instruction applies both scales itself
    p.xa = static_cast<const uint8_t*>(g.xa);
    p.xw = static_cast<const uint8_t*>(g.xw);
    p.post = 1.0f;
    p.shift = 0;
    // SwiGLU pairs gate and up fragments, which a 320-wide tile (5 per
    // wave) cannot: it takes 256 x 256.
    using M4W = Cfg<256, 320, 2, 4, false, false, false, false, 4, 3, 2>;
    using M4N = Cfg<256, 256, 2, 4, false, false, false, false, 4, 3, 2>;
    using M8W = Cfg<256, 320, 2, 4, false, false, false, false, 8>;
    using M8N = Cfg<256, 256, 2, 4, false, false, false, false, 8>;
    if (g.mx == 4) e = wide ? launch_mx<M4W, M4N>(p, g.epilogue, s) : launch_mx<M4N, M4N>(p, g.epilogue, s);
    else e = wide ? launch_mx<M8W, M8N>(p, g.epilogue, s) : launch_mx<M8N, M8N>(p, g.epilogue, s);
    return e == hipSuccess ? OK : ERR_LAUNCH;
  }
  if (g.fp6) {
    // the FP6 instruction sums the code products themselves (no nibble shift)
    p.post = 1.0f;
    p.shift = 0;
  }
  if (group || g.rank > 0 || g.epilogue == EPI_SWIGLU) {
    // INT4 weights only (the ABI routes nothing else here); 256 x 256
    // tiles keep the gate/up fragment pairs and the scale block in LDS.
    // Group-64 FP6: 256 x 128 tiles, whose 24 KB A stage splits evenly over
    // the 8 waves' 1 KB loads (a 128-row FP6 stage would not).
    if (group && g.fp6) {
      e = launch_lowrank<Cfg<256, 128, 2, 4, true, true, true, true, 0, 3, 1, false, true>>(p, g.epilogue, s);
    } else if (group) {
      // 256 x 128 tiles with 16 waves (64 x 32 wave tiles, under 128 VGPRs):
      // four waves per SIMD interleave the MFMA -> rescale chains
      e = g.a_packed ? launch_lowrank<Cfg<256, 128, 4, 4, true, true, true>>(p, g.epilogue, s)
                     : launch_lowrank<Cfg<256, 128, 4, 4, false, true, true>>(p, g.epilogue, s);
    } else {
      e = g.a_packed ? launch_lowrank<Cfg<256, 256, 2, 4, true, true>>(p, g.epilogue, s)
                     : launch_lowrank<Cfg<256, 256, 2, 4, false, true>>(p, g.epilogue, s);
    }
    return e == hipSuccess ? OK : ERR_LAUNCH;
  }
  if (g.fp6) {
    e = wide ? launch_plain<Cfg<256, 320, 2, 4, true, true, false, true>>(p, g.epilogue, s)
             : launch_plain<Cfg<256, 256, 2, 4, true, true, false, true>>(p, g.epilogue, s);
  } else if (g.w_packed) {
    if (g.a_packed)
      e = wide ? launch_plain<Cfg<256, 320, 2, 4, true, true>>(p, g.epilogue, s)
               : launch_plain<Cfg<256, 256, 2, 4, true, true>>(p, g.epilogue, s);
    else
      e = wide ? launch_plain<Cfg<256, 320, 2, 4, false, true, false, false, 0, 3, 1, true>>(p, g.epilogue, s)
               : launch_plain<Cfg<256, 256, 2, 4, false, true, false, false, 0, 3, 1, true>>(p, g.epilogue, s);
  } else if (cost(192) < (wide ? cost(320) : cost(256))) {
    // int8 W, N = 1536 at M = 16384: 512 tiles of 256 x 192 fill two waves
    // exactly where 384 tiles of 256 x 256 leave half the second one idle
    e = launch_plain<Cfg<256, 192, 2, 4, false, false, false, false, 0, 3, 1, true>>(p, g.epilogue, s);
  } else {
    e = wide ? launch_plain<Cfg<256, 320, 2, 4, false, false, false, false, 0, 3, 1, true>>(p, g.epilogue, s)
             : launch_plain<Cfg<256, 256, 2, 4, false, false, false, false, 0, 3, 1, true>>(p, g.epilogue, s);
  }
  return e == hipSuccess ? OK : ERR_LAUNCH;
}

}  // namespace ql
