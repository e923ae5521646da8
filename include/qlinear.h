/*
 * qlinear.h -- C ABI of the rotated low-bit quantized linear for AMD MI355X
 * (gfx950).
 *
 * The layer (model card "Krea-2 Turbo -- INT4 tensorwise W4A4 (+ConvRot,
 * mixed int8 fallback)", introduction; model card "Krea 2 Turbo OrbitQuant
 * W4A4", sections "Fused transformer (OrbitQuant 0.11)" and "What is
 * quantized"; README "Krea-2-SVDQuant-ComfyUI", section "Why this exists"):
 *
 *   1. rotate every aligned 256-channel group of the bf16 activations by the
 *      orthonormal regular Hadamard matrix H/16 (H = H4 (x) H4 (x) H4 (x) H4,
 *      H4 = J - 2I), online;
 *   2. quantize them dynamically to symmetric INT4 or INT8 codes
 *      (scale = absmax / qmax per tensor, per token or per token x 64
 *      channels; code = round-half-even(x * qmax / absmax), |code| <= qmax);
 *   3. multiply the codes with weights that were rotated the same way and
 *      quantized offline (packed signed INT4, or INT8), accumulating exactly
 *      in int32;
 *   4. dequantize (acc * s_a * s_w) and apply an epilogue: plain bf16, SwiGLU
 *      over a gate|up product, or a gated residual update; optionally add a
 *      bf16 low-rank branch (X L1) L2 (README "Krea-2-SVDQuant-ComfyUI",
 *      sections "Low-rank refinement" and "LoRA"; model card "Krea 2 Turbo
 *      Nunchaku Lite INT4 r32": INT4 with group size 64 and rank 32).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and frees nothing.  Its only global state is a
 *    per-device cache of the device-architecture check.
 *  - bf16 values travel as uint16_t bit patterns.  Matrices are row-major
 *    with the row stride given in elements.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on that stream and returns; it never synchronizes.
 *    Calls are reentrant; two calls that write the same buffers race unless
 *    the caller orders them.
 *  - Arguments are validated before anything is enqueued.  On any error the
 *    call returns a negative status and has enqueued nothing.  A launch
 *    failure reported by the runtime right after enqueueing maps to
 *    QL_ERR_LAUNCH (work already enqueued for that call may then be partial).
 *    Faults inside kernels surface at the caller's next synchronization.
 *  - There is no fallback path: on a device other than gfx950 every compute
 *    entry point returns QL_ERR_UNSUPPORTED.
 *  - Pointers to code / packed / bf16 matrices must be 16-byte aligned and
 *    their row strides must keep every row 16-byte aligned.  Scale, bias and
 *    gate pointers must be 4-byte (float) or 2-byte (bf16) aligned.
 *  - K must be a positive multiple of 256 (one rotation group) for every
 *    call; M may be any value >= 0 (M == 0 enqueues nothing); N must be a
 *    positive multiple of 16.
 *  - GEMM size limits (the kernels address operands with 32-bit offsets):
 *    K < 2^23, N * K < 2^31 and M * K < 2^36.  Violations return
 *    QL_ERR_SHAPE.
 *  - Exactness of the int32 accumulator (tensor / row scales): it sums K
 *    products of codes, each at most qmax_a * qmax_w and 16 times larger per
 *    packed INT4 operand (packed codes enter the int8 instruction as
 *    16 * code).  Every call whose sum could reach 2^31 returns QL_ERR_SHAPE
 *    before launching: W8A8 K > 133144 (127 * 127 * K), W4A4 with int8-
 *    container activations K > 2739137 (7 * 112 * K), W4A4 with packed
 *    activations K > 171196 (112 * 112 * K).  Group-64 partials span 64
 *    channels and are never at risk.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  QL_OK = 0,
  QL_ERR_NULL = -1,        /* a required pointer is NULL                  */
  QL_ERR_SHAPE = -2,       /* a size or stride violates a precondition    */
  QL_ERR_ALIGN = -3,       /* a pointer or stride is misaligned           */
  QL_ERR_UNSUPPORTED = -4, /* mode combination or device not supported    */
  QL_ERR_LAUNCH = -5,      /* the HIP runtime rejected a launch           */
  QL_ERR_DEVICE = -6,      /* the current device could not be queried     */
  QL_ERR_SCRATCH = -7      /* larger than the allocation-free entry's fixed workspace */
};

/* ---- quantization scale granularity ------------------------------------ */
enum {
  QL_SCALE_TENSOR = 0,  /* one scale for the whole matrix            -> [1]      */
  QL_SCALE_ROW = 1,     /* one per row (token / output channel)      -> [R]      */
  QL_SCALE_GROUP64 = 2  /* one per row x aligned 64-channel group    -> [K/64, R] */
};
/* GROUP64 scales are stored group-major: float g * R + r is the scale of row
 * r over channels 64 g .. 64 g + 63, so the R scales of one group are
 * contiguous and the GEMM fetches a K step's scales as whole cache lines. */

/* ---- INT4 code layouts --------------------------------------------------
 * QL_LAYOUT_I8     : one code per int8 byte, [R, K] (int4 codes -7..7 kept in
 *                    int8 containers; int8 codes always use this layout).
 * QL_LAYOUT_PACKED : two signed 4-bit codes per byte, [R, K/2].  Within every
 *                    run of 8 consecutive channels 8c..8c+7, byte 4c+j
 *                    (j = 0..3) holds channel 8c+j in its low nibble and
 *                    channel 8c+j+4 in its high nibble (two's complement).
 *                    Packed INT4 WEIGHTS (pack_weight_int4, svdq_split, the
 *                    w operand of the INT4 GEMMs) also pair their rows: for
 *                    every 128-channel slice s of K, the 64 bytes of row 2p
 *                    and then those of row 2p + 1 are adjacent, at byte
 *                    p * K + 128 s (+ 64 for row 2p + 1), so one cache line
 *                    holds a slice of two rows.  Packed activations keep
 *                    plain rows.
 * QL_LAYOUT_FP6    : each int4 code as its exact FP6 e2m3 value (sign bit, 2
 *                    exponent bits with bias 1, 3 mantissa bits), [R, 3K/4]
 *                    bytes; for the FP6 GEMM only.  A row is K/128 blocks of
 *                    96 bytes.  In a block, 32-channel sub-block g (0..3) is
 *                    the 192-bit little-endian value v_g holding its channel
 *                    i in bits 6i..6i+5; block bytes 16g..16g+15 hold the
 *                    low 16 bytes of v_g and bytes 64+8g..64+8g+7 its high
 *                    8 bytes.  Rows are interleaved in fours: for every
 *                    128-channel block s, the 96-byte blocks of rows 4q,
 *                    4q+1, 4q+2, 4q+3 are adjacent, row 4q+j's at byte
 *                    4q * 3K/4 + 384 s + 96 j (three whole cache lines per
 *                    block of four rows); the last R % 4 rows of an R-row
 *                    matrix keep plain rows (row r's block s at
 *                    r * 3K/4 + 96 s).  The size stays R * 3K/4 bytes.      */
enum { QL_LAYOUT_I8 = 0, QL_LAYOUT_PACKED = 1, QL_LAYOUT_FP6 = 2 };

/* ---- MX block formats (OCP Microscaling Formats v1.0) -------------------
 * Every 32 consecutive elements of a row along K share one E8M0 scale byte
 * (the power of two 2^(byte - 127)); elements are
 * QL_MX_FP4 : FP4 E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; sign in bit
 *             3), two per byte, element 2i in the low nibble of byte i:
 *             [R, K/2] bytes;
 * QL_MX_FP8 : FP8 E4M3 (bias 7, largest magnitude 448, no infinities), one
 *             per byte: [R, K] bytes.
 * Scales: stage-major [K/128][R][4] bytes -- for each 128-channel slice s
 * of K, the 4 scale bytes of row 0 (blocks 4s .. 4s+3), then of row 1, ...
 * (a GEMM tile reads one slice's scales for consecutive rows as consecutive
 * bytes).  Zero elements are stored as +0. */
enum { QL_MX_FP4 = 4, QL_MX_FP8 = 8 };

/* ---- GEMM epilogues ---------------------------------------------------- */
enum {
  QL_EPI_BF16 = 0,           /* out[m,n] = bf16(y)                               */
  QL_EPI_SWIGLU = 1,         /* out[m,j] = bf16(silu(y[m,j]) * y[m,j+N/2]), j<N/2 */
  QL_EPI_GATED_RESIDUAL = 2, /* out[m,n] = bf16(res[m,n] + gate[n] * y[m,n])     */
  QL_EPI_F32 = 3,            /* out[m,n] = y as float32                          */
  QL_EPI_I32 = 4,            /* out[m,n] = exact int32 accumulator (no scales)   */
  QL_EPI_SIGMOID = 5         /* out[m,n] = bf16(1 / (1 + exp(-y[m,n])))          */
};
/* y[m,n] = sum_k deq(a)[m,k] * deq(w)[n,k] (+ bias[n]) (+ (lr L2)[m,n]; the
 * entry points take L2 stored transposed, l2[n, j] = L2[j, n]),
 * i.e. acc * s_a * s_w for tensor / row scales, and the sum over 64-channel
 * groups of acc_g * s_a[m,g] * s_w[n,g] for group-64 scales.  bf16 outputs
 * are rounded to nearest even. */

/* ---- entry points ------------------------------------------------------ */

/* Human-readable name of a status code (static string, never NULL). */
const char* ql_status_string(int status);

/* 1 if `device` is a gfx950 GPU this library was built for, 0 otherwise
 * (also 0 if the device cannot be queried).  Needs no model or data
 * (README "Krea-2-SVDQuant-ComfyUI", section "The nodes": an availability
 * check that needs no model). */
int ql_device_supported(int device);

/* Online activation prologue (model card "Krea-2 Turbo -- INT4 tensorwise
 * W4A4 (+ConvRot, mixed int8 fallback)", introduction: activations are
 * rotated online and quantized dynamically inside the kernel).
 *
 *   x      [M, K] bf16, row stride ldx (elements, >= K, multiple of 8)
 *   bits   4 or 8
 *   scale_mode  QL_SCALE_TENSOR | QL_SCALE_ROW | QL_SCALE_GROUP64
 *   layout QL_LAYOUT_I8, QL_LAYOUT_PACKED or QL_LAYOUT_FP6 (the last two
 *          only with bits == 4)
 *   rotate 1: rotate each 256-group by H/16 first; 0: quantize x as is
 *   codes  out: [M, K] int8, [M, K/2] packed or [M, 3K/4] FP6 bytes (QL_LAYOUT_FP6 row order), dense
 *   scales out: float32 [1] | [M] | [K/64, M] (scale = absmax / qmax)
 *   l1, rank, lr  optional SVDQuant down-projection: if l1 != NULL,
 *          lr[M, rank] (bf16, dense rows) = bf16(x[M,K] @ l1[K, rank]) with the
 *          UNROTATED x, l1 bf16 row-major; rank a multiple of 16, 16..128.
 *          l1 == NULL requires rank == 0.
 * QL_SCALE_TENSOR uses scales[0] as its grid-wide reduction cell; the library
 * initializes it on the stream. */
int rotate_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        int bits, int scale_mode, int layout, int rotate,
                        void* codes, float* scales,
                        const uint16_t* l1, int rank, uint16_t* lr,
                        void* stream);

/* Activation prologue with the block's RMSNorm and adaLN modulation fused in
 * front (model card "Krea 2 Turbo OrbitQuant W4A4", section "Fused
 * transformer (OrbitQuant 0.11)": the norm and the modulation run inside the
 * activation quantization prologue, so the normalized activation is never
 * written).  The page names the steps; the formula is the usual batch-1
 * reading:
 *
 *   h[m,k] = x[m,k] * r[m] * gamma[k] * (1 + mod_scale[k]) + mod_shift[k],
 *   r[m]   = 1 / sqrt(mean_k x[m,k]^2 + eps),
 *
 * in fp32 (h is not rounded to bf16); h is then rotated and quantized exactly
 * as rotate_quantize_act does with x.  One prepared activation serves every
 * projection that reads the same normalized input (Q|K|V|gate, gate|up): the
 * caller passes the same codes and scales to each GEMM.
 *
 *   x, M, K, ldx, bits, scale_mode, layout, rotate, codes, scales
 *          as rotate_quantize_act; K <= 8192 (the vectors are staged on chip)
 *   gamma, mod_scale, mod_shift   bf16 [K] each, 16-byte aligned, or NULL
 *          (meaning all ones, all zeros, all zeros)
 *   eps    > 0 and finite, else QL_ERR_SHAPE
 * There is no low-rank output here (the SVDQuant branch reads the unrotated
 * layer input; use rotate_quantize_act for that layer). */
int rmsnorm_rotate_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                const uint16_t* gamma, const uint16_t* mod_scale,
                                const uint16_t* mod_shift, float eps, int bits, int scale_mode,
                                int layout, int rotate, void* codes, float* scales, void* stream);

/* Offline weight preparation for INT4 (model card "Krea-2 Turbo -- INT4
 * tensorwise W4A4 (+ConvRot, mixed int8 fallback)", introduction: packed
 * signed INT4 weights carrying the same group-256 rotation).  Same
 * arithmetic as rotate_quantize_act(w, N, K, ldw, 4, scale_mode,
 * QL_LAYOUT_PACKED, rotate, ...).  INT8 per-row weights (model card "Krea 2
 * Turbo OrbitQuant W4A4", section "What is quantized") are produced by
 * rotate_quantize_act with bits = 8 and QL_SCALE_ROW.
 *   w      [N, K] bf16 (torch Linear layout: out x in), row stride ldw
 *   packed out: [N, K/2] bytes in the QL_LAYOUT_PACKED weight order (row
 *            pairs interleaved per 128-channel slice)
 *   scales out: float32 [1] | [N] | [K/64, N]                              */
int pack_weight_int4(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                     int scale_mode, int rotate, uint8_t* packed, float* scales,
                     void* stream);

/* Offline INT4 weight preparation for the FP6 GEMMs (qgemm_w4a4_fp6,
 * qgemm_w4a4_fp6_lowrank): the same codes and scales as pack_weight_int4,
 * stored in QL_LAYOUT_FP6; equal to rotate_quantize_act(w, N, K, ldw, 4,
 * scale_mode, QL_LAYOUT_FP6, rotate, ...).  scale_mode TENSOR | ROW |
 * GROUP64.
 *   packed out: [N, 3K/4] bytes in the QL_LAYOUT_FP6 order                 */
int pack_weight_fp6(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                    int scale_mode, int rotate, uint8_t* packed, float* scales,
                    void* stream);

/* W4A4 GEMM + dequant epilogue (model card "Krea 2 Turbo OrbitQuant W4A4",
 * section "Fused transformer (OrbitQuant 0.11)": W4A4 GEMMs for attention
 * and gate/up projections).
 *   a        [M, K] activation codes in `a_layout`, dense rows
 *   sa       activation scales per a_scale_mode (TENSOR | ROW)
 *   w        [N, K/2] packed int4 weight codes in the weight order of
 *            QL_LAYOUT_PACKED (row pairs interleaved per 128-channel slice)
 *   sw       weight scales per w_scale_mode (TENSOR | ROW)
 *   bias     NULL or bf16 [N]
 *   epilogue QL_EPI_BF16 | QL_EPI_F32 | QL_EPI_I32 (I32 ignores scales and bias) |
 *            QL_EPI_SIGMOID (tensor / row scales; the attention gate)
 *   out      [M, N] bf16 / float32 / int32, row stride ldo (elements)
 *   a_layout QL_LAYOUT_I8 | QL_LAYOUT_PACKED (else QL_ERR_UNSUPPORTED)
 * Group-64 scales (both sides, BF16 | F32 only) run qgemm_w4a4_lowrank with
 * rank 0. */
int qgemm_w4a4(const void* a, const float* sa, int a_scale_mode, int a_layout,
               const uint8_t* w, const float* sw, int w_scale_mode,
               int64_t M, int64_t N, int64_t K,
               const uint16_t* bias, int epilogue, void* out, int64_t ldo,
               void* stream);

/* Experimental W4A4 GEMM on gfx950's FP6 matrix instructions.  The pages
 * run the same checkpoint faster as an FP4 build on a GPU whose matrix units
 * take that format natively (model card "Krea 2 Turbo Nunchaku Lite INT4
 * r32", section "Benchmark"); the MI355X counterpart for INT4 codes is FP6
 * e2m3, which holds every code -7..7 exactly and runs at twice the INT8
 * matrix rate.  Products of two codes are integers of magnitude <= 49 and
 * their float32 sums are exact while 49 K < 2^24, so for K < 342392 the
 * result equals qgemm_w4a4's bit for bit.
 *   a   [M, 3K/4] activation codes in QL_LAYOUT_FP6 (rotate_quantize_act or
 *       rmsnorm_rotate_quantize_act with layout QL_LAYOUT_FP6), dense rows
 *   w   [N, 3K/4] weight codes in QL_LAYOUT_FP6 (pack_weight_fp6)
 *   sa, a_scale_mode, sw, w_scale_mode   TENSOR | ROW scales, as qgemm_w4a4,
 *       or GROUP64 on both sides (README "Krea-2-SVDQuant-ComfyUI": INT4 with
 *       group size 64); the 32x32x64 FP6 instruction then covers exactly one
 *       64-channel group, and its fp32 result, the group's exact partial, is
 *       rescaled as qgemm_w4a4_lowrank does, so the output again equals the
 *       INT8 path's bit for bit
 *   bias, epilogue, out, ldo             as qgemm_w4a4 (BF16 | F32 | I32 |
 *       SIGMOID; GROUP64: BF16 | F32); QL_EPI_I32 returns the exact sum of
 *       code products
 * With tensor / row scales K must also be < 342392 (else QL_ERR_SHAPE). */
int qgemm_w4a4_fp6(const uint8_t* a, const float* sa, int a_scale_mode,
                   const uint8_t* w, const float* sw, int w_scale_mode,
                   int64_t M, int64_t N, int64_t K,
                   const uint16_t* bias, int epilogue, void* out, int64_t ldo,
                   void* stream);

/* MX block quantization: the activation prologue and the offline weight
 * preparation of qgemm_mx (both operands use the same quantizer).  The pages
 * run the model as an NVFP4 build on a GPU with native FP4 matrix units
 * (model card "Krea 2 Turbo Nunchaku Lite INT4 r32", section "Benchmark")
 * and as an mxfp8 build (research log "lab", Study 1); gfx950's
 * block-scaled matrix instruction takes OCP MX operands (32-element blocks,
 * E8M0 scales), so MXFP4 stands in for NVFP4 and MXFP8 for mxfp8.  Per
 * block, after the optional rotation (as rotate_quantize_act):
 *   e = floor(log2 max|x|) - emax (emax 2 for FP4, 8 for FP8), clamped to
 *       [-127, 127]; -127 for an all-zero block;
 *   element = x / 2^e rounded to nearest, ties to even, saturating at the
 *       largest magnitude (OCP MX v1.0, conversion from wider formats).
 *   x      [M, K] bf16 (finite), row stride ldx (elements, >= K, multiple of 8)
 *   fmt    QL_MX_FP4 | QL_MX_FP8 (else QL_ERR_UNSUPPORTED)
 *   rotate 1: rotate each 256-group by H/16 first; 0: quantize x as is
 *   codes  out: element bytes per fmt, dense rows (16-byte aligned)
 *   scales out: [K/128][M][4] E8M0 bytes (stage-major, see QL_MX_FP4),
 *          4-byte aligned
 *   l1, rank, lr  optional SVDQuant down-projection, exactly as
 *          rotate_quantize_act: lr[M, rank] = bf16(x @ l1) with the
 *          UNROTATED x (l1 == NULL requires rank == 0)                      */
int rotate_quantize_mx(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                       int fmt, int rotate, void* codes, uint8_t* scales,
                       const uint16_t* l1, int rank, uint16_t* lr,
                       void* stream);

/* MX block-scaled GEMM + epilogue on gfx950's block-scaled matrix
 * instruction (pages and formats as rotate_quantize_mx):
 *   y[m,n] = sum_b 2^(ea[m,b] + ew[n,b]) * sum_{k in block b} a[m,k] w[n,k]
 *            (+ bias[n]),
 * accumulated in float32 over the K/32 blocks (block scale products below
 * 2^-126 underflow).  FP4 block products are exact.  FP8 products are
 * summed by the matrix instruction on a fixed-point grid (measured on
 * gfx950): inside a small group of adjacent elements each product is
 * truncated toward zero to a multiple of 2^-13 times the binade of the
 * group's largest product, so an FP8 block product can differ from the
 * exact one by up to about 2^-13 of that product per element.
 *   a, sa    activation elements [M, K/2 | K] and scales [K/128][M][4]
 *   w, sw    weight elements [N, K/2 | K] and scales [K/128][N][4]
 *            (rotate_quantize_mx with the same fmt; scale pointers 4-byte
 *            aligned)
 *   fmt      QL_MX_FP4 | QL_MX_FP8
 *   bias     NULL or bf16 [N]
 *   residual, gate   as qgemm_w8a8, for QL_EPI_GATED_RESIDUAL
 *   epilogue QL_EPI_BF16 | QL_EPI_F32 | QL_EPI_SIGMOID |
 *            QL_EPI_GATED_RESIDUAL | QL_EPI_SWIGLU (N a multiple of 32;
 *            gate rows first, as qgemm_w4a4_lowrank); not QL_EPI_I32
 *   out      [M, N] (SWIGLU: [M, N/2]) bf16 / float32, row stride ldo    */
int qgemm_mx(const void* a, const uint8_t* sa, const void* w, const uint8_t* sw,
             int fmt, int64_t M, int64_t N, int64_t K,
             const uint16_t* bias, const uint16_t* residual, const uint16_t* gate,
             int epilogue, void* out, int64_t ldo, void* stream);

/* The SVDQuant layer in MX form: qgemm_mx's product plus the bf16 low-rank
 * branch, y = mx(a) mx(w)^T (+ bias) + lr @ l2, then the epilogue -- the
 * pages' "NVFP4 r32" build, an FP4 SVDQuant checkpoint with a rank-32 branch
 * (model card "Krea 2 Turbo Nunchaku Lite INT4 r32", section "Benchmark";
 * README "Krea-2-SVDQuant-ComfyUI", sections "Low-rank refinement" and
 * "LoRA").  On gfx950 its FP4 runs as MXFP4 (see rotate_quantize_mx).
 *   a, sa, w, sw, fmt   as qgemm_mx
 *   lr       bf16 [M, rank] (rotate_quantize_mx's down-projection), dense rows
 *   l2       bf16 [N, rank]: row n is the rank vector of output column n
 *            (the branch's L2 factor stored transposed), 16-byte aligned
 *   rank     0..128, a multiple of 16 (0: no branch)
 *   bias     NULL or bf16 [N]
 *   epilogue QL_EPI_BF16 | QL_EPI_F32 | QL_EPI_SWIGLU (N a multiple of 32;
 *            gate rows first)
 *   out      [M, N] (SWIGLU: [M, N/2]), row stride ldo                      */
int qgemm_mx_lowrank(const void* a, const uint8_t* sa, const void* w, const uint8_t* sw,
                     int fmt, const uint16_t* lr, const uint16_t* l2, int rank,
                     int64_t M, int64_t N, int64_t K, const uint16_t* bias,
                     int epilogue, void* out, int64_t ldo, void* stream);

/* W8A8 GEMM + dequant epilogue for the protected ff.down projections (model
 * card "Krea 2 Turbo OrbitQuant W4A4", sections "Fused transformer" and
 * "What is quantized": per-row INT8 weights with INT8 activations, gated
 * residual update in the GEMM epilogue).
 *   a [M, K] int8, w [N, K] int8 (dense rows); sa, sw per their scale modes
 *   (TENSOR | ROW)
 *   residual  bf16 [M, N] with row stride ldo; may alias out (in-place
 *             h += gate * y).  Required for QL_EPI_GATED_RESIDUAL.
 *   gate      bf16 [N]; required for QL_EPI_GATED_RESIDUAL.
 *   epilogue  QL_EPI_BF16 | QL_EPI_GATED_RESIDUAL | QL_EPI_F32 | QL_EPI_I32 |
 *             QL_EPI_SIGMOID */
int qgemm_w8a8(const int8_t* a, const float* sa, int a_scale_mode,
               const int8_t* w, const float* sw, int w_scale_mode,
               int64_t M, int64_t N, int64_t K,
               const uint16_t* bias, const uint16_t* residual, const uint16_t* gate,
               int epilogue, void* out, int64_t ldo, void* stream);

/* W4A4 GEMM with group-64 (or row / tensor) scales, optional SVDQuant
 * low-rank branch and SwiGLU epilogue (model card "Krea 2 Turbo Nunchaku
 * Lite INT4 r32": INT4, group size 64, rank 32; README
 * "Krea-2-SVDQuant-ComfyUI", section "Why this exists": a low-rank
 * correction branch on top of the W4A4 kernel; model card "Krea 2 Turbo
 * OrbitQuant W4A4", section "Fused transformer": SwiGLU gate|up GEMM).
 *   a, sa, a_scale_mode, a_layout, w, sw, w_scale_mode   as qgemm_w4a4, and
 *             GROUP64 is allowed only on both sides at once; a_layout
 *             QL_LAYOUT_I8 | QL_LAYOUT_PACKED (the FP6 experiment has its
 *             own entry point, qgemm_w4a4_fp6_lowrank)
 *   lr        bf16 [M, rank] (from rotate_quantize_act), dense rows
 *   l2        bf16 [N, rank]: row n is the rank vector of output column n
 *             (the branch's L2 factor stored transposed, so the epilogue
 *             reads 8 consecutive ranks with one 16-byte load), 16-byte aligned
 *   rank      0 (no branch; lr, l2 may be NULL) or a multiple of 16, <= 128
 *   epilogue  QL_EPI_BF16 | QL_EPI_SWIGLU | QL_EPI_F32; SWIGLU pairs output
 *             column j (gate) with column j + N/2 (up), needs N % 32 == 0
 *             and writes out[M, N/2]
 *   out       row stride ldo (elements) */
int qgemm_w4a4_lowrank(const void* a, const float* sa, int a_scale_mode, int a_layout,
                       const uint8_t* w, const float* sw, int w_scale_mode,
                       const uint16_t* lr, const uint16_t* l2, int rank,
                       int64_t M, int64_t N, int64_t K,
                       const uint16_t* bias, int epilogue, void* out, int64_t ldo,
                       void* stream);

/* The group-64 low-rank GEMM of qgemm_w4a4_lowrank on the FP6 matrix
 * instructions -- the experiment beside the int8 path (model card "Krea 2
 * Turbo Nunchaku Lite INT4 r32", section "Benchmark": the same checkpoint as
 * an FP4 build on a GPU whose matrix units take it natively).  Both operands
 * hold the int4 codes in QL_LAYOUT_FP6 (a [M, 3K/4] from the prologues with
 * layout QL_LAYOUT_FP6, w [N, 3K/4] from pack_weight_fp6), with group-64
 * scales on both sides (sa [K/64, M], sw [K/64, N]).  Each 32x32x64 FP6
 * instruction covers exactly one 64-channel group; its fp32 result is the
 * group's exact partial and is rescaled exactly as
 * the INT8 path does, so the output equals qgemm_w4a4_lowrank's with group-64
 * scales bit for bit.
 *   lr, l2, rank, bias, out, ldo   as qgemm_w4a4_lowrank
 *   epilogue  QL_EPI_BF16 | QL_EPI_SWIGLU | QL_EPI_F32 */
int qgemm_w4a4_fp6_lowrank(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                           const uint16_t* lr, const uint16_t* l2, int rank,
                           int64_t M, int64_t N, int64_t K,
                           const uint16_t* bias, int epilogue, void* out, int64_t ldo,
                           void* stream);

/* One projection of a grouped GEMM. */
typedef struct {
  const void* w;    /* packed int4 [n, K/2] (w_bits 4) or int8 [n, K] (w_bits 8), dense rows */
  const float* sw;  /* per-row weight scales [n] */
  int64_t n;        /* output columns: a positive multiple of 16, n * K < 2^31 */
  int w_bits;       /* 4: int4 weights with the INT4 activation codes a4;
                       8: int8 weights with the INT8 activation codes a8 */
  int epilogue;     /* QL_EPI_BF16 or QL_EPI_SIGMOID */
  void* out;        /* bf16 [M, n], row stride ldo (elements, >= n, 16-byte rows) */
  int64_t ldo;
} ql_segment;

enum { QL_MAX_SEGMENTS = 8 };

/* Grouped GEMM: up to QL_MAX_SEGMENTS projections of the same activations
 * in one launch (model card "Krea 2 Turbo OrbitQuant W4A4", section "Fused
 * transformer (OrbitQuant 0.11)": one grouped Q|K|V|gate W4A4 GEMM per block
 * with the sigmoid gate in its epilogue, while the K and V projections stay
 * INT8).  Segment s computes out_s = epilogue_s(deq(a) deq(w_s)^T) with
 * per-token activation and per-row weight scales, exactly as qgemm_w4a4 /
 * qgemm_w8a8 would; the tiles of every segment share one grid.
 *   a4, sa4   int8-container INT4 codes [M, K] (dense rows) and their per-row
 *             scales [M]; required if any segment has w_bits 4, else may be NULL
 *   a8, sa8   INT8 codes [M, K] and per-row scales [M]; required if any
 *             segment has w_bits 8, else may be NULL
 *   segments  HOST array of nseg descriptors, 1 <= nseg <= QL_MAX_SEGMENTS;
 *             read during the call only
 * Outputs must not overlap each other or the inputs. */
int qgemm_grouped(const void* a4, const float* sa4, const void* a8, const float* sa8,
                  int64_t M, int64_t K, const ql_segment* segments, int nseg, void* stream);

/* Offline SVDQuant split of a weight into a low-rank branch and an INT4
 * residual, on the device (README "Krea-2-SVDQuant-ComfyUI": the split is a
 * seeded randomized SVD, reproducible per device; "Activation-aware branch":
 * the fit is weighted by per-input-channel activation RMS d, normalized to
 * mean 1 and floored at 0.05; "Low-rank refinement, and what the objective
 * actually is": the branch is refit to the current quantization error and
 * the residual requantized, repeatedly, keeping the best, iteration 1 being
 * the plain split).  With D = diag(d) (identity without statistics):
 *   iteration t: fit target A = (W - E_{t-1}) D (E_0 = 0); randomized SVD of A
 *     (subspace iteration with the sketch omega and power_iters power steps);
 *     L1 = bf16(V_r S_r^1/2 / d), L2 = bf16((U_r S_r^1/2)^T) (singular values
 *     below 1e-5 of the largest dropped); residual T = W - (L1 L2)^T,
 *     quantized from bf16(T) exactly as pack_weight_int4 does (rotated INT4,
 *     scale_mode); E_t = the residual's dequantized codes rotated back;
 *     objective err_t = ||(T - E_t) D||_F.
 *   The outputs hold the iteration with the smallest objective (ties: the
 *   earlier one).  Deterministic: the same inputs give the same result on
 *   the same device (no atomics; fixed-order reductions).
 *   w        [N, K] bf16, row stride ldw (>= K, multiple of 8), 16-byte aligned;
 *            N % 16 == 0, K % 256 == 0, K <= 32768, N * K < 2^31
 *   act_rms  NULL or float32 [K] per-input-channel activation RMS
 *   omega    float32 [K, rank + oversample], row-major: the Gaussian sketch
 *            (draw it from a seeded generator for reproducible builds)
 *   rank     16..128, multiple of 16; oversample 0..32; rank + oversample <= min(N, K)
 *   power_iters 0..8; refine_iters 0..16 (iterations = refine_iters + 1)
 *   scale_mode QL_SCALE_TENSOR | QL_SCALE_ROW | QL_SCALE_GROUP64 (the residual's scales)
 *   l1 out: bf16 [K, rank]; l2 out: bf16 [N, rank], L2 transposed (the layout of the low-rank
 *            GEMM entry points); packed out: [N, K/2] (QL_LAYOUT_PACKED);
 *            scales out: float32 [1] | [N] | [K/64, N]; all 16-byte aligned
 *   errors out: float32 [refine_iters + 1], err_t of every iteration
 *   best_iter out: int32 [1], the iteration returned
 *   sigma   NULL or out float32 [rank] (16-byte aligned): singular values of
 *            the returned iteration's fit (0 where dropped)
 *   workspace, workspace_bytes  device scratch of at least
 *            svdq_split_workspace_bytes(N, K, rank, oversample, scale_mode)
 *            bytes, 16-byte aligned, owned by the caller, not in use by
 *            another call; about 10.5 N K bytes.
 * All pointers are device pointers.  The call only enqueues work on `stream`. */
int svdq_split(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, const float* act_rms,
               const float* omega, int rank, int oversample, int power_iters, int refine_iters,
               int scale_mode, uint16_t* l1, uint16_t* l2, uint8_t* packed, float* scales,
               float* errors, int32_t* best_iter, float* sigma, void* workspace,
               int64_t workspace_bytes, void* stream);

/* Workspace bytes svdq_split needs for these sizes; -1 for invalid sizes. */
int64_t svdq_split_workspace_bytes(int64_t N, int64_t K, int rank, int oversample, int scale_mode);

/* svdq_split for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments and results as svdq_split without the workspace, which
 * lives in a fixed 128 MiB array inside the library (one copy per GPU, held
 * until the process ends; its device address is looked up once per device).
 * The call allocates nothing.  It returns QL_ERR_SCRATCH before enqueueing
 * anything when svdq_split_workspace_bytes(N, K, rank, oversample,
 * scale_mode) exceeds svdq_split_noalloc_max_bytes() (at rank 32: up to about
 * 11.7 M weight elements, e.g. 1536 x 5120 or 2048 x 5120, not 5120 x 5120).
 * Every call on a GPU uses that GPU's one array: calls that overlap on the
 * same GPU (other streams, other threads) race and must be ordered by the
 * caller.  No part of the array has to start at zero. */
int svdq_split_noalloc(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, const float* act_rms,
                       const float* omega, int rank, int oversample, int power_iters, int refine_iters,
                       int scale_mode, uint16_t* l1, uint16_t* l2, uint8_t* packed, float* scales,
                       float* errors, int32_t* best_iter, float* sigma, void* stream);

/* Size in bytes of svdq_split_noalloc's fixed workspace. */
int64_t svdq_split_noalloc_max_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
