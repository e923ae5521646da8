// Offline SVDQuant low-rank split on the device, for gfx950.
//
// Method (README "Krea-2-SVDQuant-ComfyUI"): the weight is split into a
// low-rank branch L1 L2 and an INT4 residual Q, W ~= Q + (L1 L2)^T.  The
// branch comes from a seeded randomized SVD (section on reproducible builds);
// the fit can be weighted by per-input-channel activation RMS d, normalized
// to mean 1 and floored at 0.05 ("Activation-aware branch"); the branch is
// then refit to the current quantization error and the residual
// requantized, repeatedly, keeping the best ("Low-rank refinement, and what
// the objective actually is").  Objective: ||(W - B - unrotate(deq(Q))) D||_F.
//
// The randomized SVD is randomized subspace iteration (Halko, Martinsson and
// Tropp, 2011): Y = A Omega, Q = orth(Y), per power iteration Z = orth(A^T Q),
// Q = orth(A Z); then B^T = A^T Q, the eigen-decomposition of B B^T gives
// B = U~ S V^T, and the branch factors are L1 = (B^T U~_r S_r^-1/2) / d and
// L2^T = Q U~_r S_r^1/2.  orth() is CholeskyQR2 (a Gram matrix, its Cholesky
// factor and triangular inverse in fp64 on one workgroup, then X R^-1), the
// eigen-decomposition a parallel cyclic Jacobi in fp64.
//
// Everything is stream-ordered and deterministic: reductions run in a fixed
// order (split-K partials summed in sequence), so the same inputs give the
// same split on the same device.  Nothing is allocated; the caller passes a
// workspace.

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int kSplitThreads = 256;
constexpr int64_t kSmallLds = 65536;  // dynamic LDS for the one-workgroup fp64 kernels (64 KB)
constexpr float kDFloor = 0.05f;      // floor of the normalized activation weights
constexpr double kSigmaDrop = 1e-5;   // singular values below this fraction of the largest are dropped

// ---- fp32 tile GEMM with generic strides and split-K -----------------------
// C[M x Nc] (+ z * M * Nc) = sum over k in split z of A(i, k) * B(k, j), with
// A(i, k) = a[i * a_rs + k * a_cs] and B(k, j) = b[k * b_rs + j * b_cs].
// 64 x 64 tiles, 32-deep k steps.  Each wave computes a 32 x 32 quadrant as
// 2 x 2 fp32 MFMA 16x16x4 blocks (lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds C[4 (l / 16) + r][l % 16]).  Tile loads run
// along whichever index is contiguous, so transposed operands stay
// coalesced, and the next step's tiles are loaded into registers while the
// current step computes from LDS.
struct GemmDesc {
  const float* a;
  int64_t a_rs, a_cs;
  const float* b;
  int64_t b_rs, b_cs;
  float* c;
  int64_t M, Nc, Kd, kchunk;
};

constexpr int kGemmBK = 32;

__global__ __launch_bounds__(kSplitThreads) void sgemm_kernel(GemmDesc g) {
  __shared__ float As[kGemmBK][64 + 4];
  __shared__ float Bs[kGemmBK][64 + 4];
  const int tid = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  const int64_t kbeg = (int64_t)blockIdx.z * g.kchunk;
  const int64_t kend = kbeg + g.kchunk < g.Kd ? kbeg + g.kchunk : g.Kd;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;  // the wave's quadrant
  const bool a_along_i = g.a_rs == 1 && g.a_cs != 1;
  const bool b_along_j = g.b_cs == 1;
  constexpr int PER = 64 * kGemmBK / kSplitThreads;  // tile elements per thread and operand
  float ra[PER], rb[PER];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + kSplitThreads * u;
      const int ii = a_along_i ? (e & 63) : (e / kGemmBK);
      const int ka = a_along_i ? (e >> 6) : (e % kGemmBK);
      const int64_t gi = i0 + ii, gk = k0 + ka;
      ra[u] = (gi < g.M && gk < kend) ? g.a[gi * g.a_rs + gk * g.a_cs] : 0.f;
      const int jj = b_along_j ? (e & 63) : (e / kGemmBK);
      const int kb = b_along_j ? (e >> 6) : (e % kGemmBK);
      const int64_t gj = j0 + jj, gk2 = k0 + kb;
      rb[u] = (gj < g.Nc && gk2 < kend) ? g.b[gk2 * g.b_rs + gj * g.b_cs] : 0.f;
    }
  };
  v4f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
  if (kbeg < kend) fetch(kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += kGemmBK) {
    __syncthreads();  // the previous step's reads of As / Bs are done
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + kSplitThreads * u;
      As[a_along_i ? (e >> 6) : (e % kGemmBK)][a_along_i ? (e & 63) : (e / kGemmBK)] = ra[u];
      Bs[b_along_j ? (e >> 6) : (e % kGemmBK)][b_along_j ? (e & 63) : (e / kGemmBK)] = rb[u];
    }
    __syncthreads();
    if (k0 + kGemmBK < kend) fetch(k0 + kGemmBK);  // in flight during the step below
#pragma unroll
    for (int kq = 0; kq < kGemmBK; kq += 4) {
      const float a0 = As[kq + lg][wr + l16], a1 = As[kq + lg][wr + 16 + l16];
      const float b0 = Bs[kq + lg][wc + l16], b1 = Bs[kq + lg][wc + 16 + l16];
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
    }
  }
  float* const cz = g.c + (int64_t)blockIdx.z * g.M * g.Nc;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = i0 + wr + 16 * a + 4 * lg + r;
        const int64_t j = j0 + wc + 16 * b + l16;
        if (i < g.M && j < g.Nc) cz[i * g.Nc + j] = acc[a][b][r];
      }
}

// out[e] = sum over s of parts[s * n + e], in order s = 0, 1, ... (fp64 sum);
// written as fp32 and / or fp64.
__global__ void reduce_parts_kernel(const float* __restrict__ parts, int S, int64_t n, float* out32,
                                    double* out64) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  double s = 0.0;
  for (int z = 0; z < S; ++z) s += (double)parts[(int64_t)z * n + e];
  if (out32) out32[e] = (float)s;
  if (out64) out64[e] = s;
}

// ---- activation weights ------------------------------------------------------
// d[k] = max(rms[k] / mean(rms), 0.05), or 1 without statistics.  One
// workgroup; the mean is a fixed-order fp64 reduction.
__global__ __launch_bounds__(kSplitThreads) void act_weights_kernel(const float* rms, int64_t K, float* d) {
  __shared__ double red[kSplitThreads];
  const int tid = threadIdx.x;
  if (!rms) {
    for (int64_t k = tid; k < K; k += kSplitThreads) d[k] = 1.0f;
    return;
  }
  double s = 0.0;
  for (int64_t k = tid; k < K; k += kSplitThreads) s += (double)rms[k];
  red[tid] = s;
  __syncthreads();
  for (int w = kSplitThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const double mean = red[0] / (double)K;
  for (int64_t k = tid; k < K; k += kSplitThreads) {
    const float v = mean > 0.0 ? (float)((double)rms[k] / mean) : 1.0f;
    d[k] = v > kDFloor ? v : kDFloor;
  }
}

// ---- CholeskyQR step: Cholesky of a Gram matrix and its inverse factor -----
// G (fp64 [l x l]) + delta I = R^T R with R upper triangular, delta = 1e-7 of
// the mean diagonal (a tiny shift that keeps a rank-deficient Gram matrix
// positive definite); rinv = R^-1 (fp32, row-major), so X R^-1 has
// orthonormal columns when G = X^T X.  A zero Gram matrix (trace <= 1e-60)
// gives rinv = 0.  One workgroup; its two l x l fp64 scratch matrices live in
// dynamic LDS when the launch provides 2 l^2 doubles of it, else in Wg / Rg
// (global memory).
__global__ __launch_bounds__(kSplitThreads) void chol_inv_kernel(const double* __restrict__ G, int l, double* Wg,
                                                                 double* Rg, float* __restrict__ rinv, int in_lds) {
  extern __shared__ double dyn[];
  __shared__ double tr;
  double* const W = in_lds ? dyn : Wg;
  double* const R = in_lds ? dyn + l * l : Rg;
  const int tid = threadIdx.x;
  if (tid == 0) {
    double t = 0.0;
    for (int i = 0; i < l; ++i) t += G[i * l + i];
    tr = t;
  }
  __syncthreads();
  if (!(tr > 1e-60)) {
    // X is zero (or negligible): any orthonormal completion would be noise;
    // R^-1 = 0 makes X R^-1 = 0, which the eigen step then drops
    for (int e = tid; e < l * l; e += kSplitThreads) rinv[e] = 0.0f;
    return;
  }
  const double delta = 1e-7 * tr / l;
  for (int e = tid; e < l * l; e += kSplitThreads) {
    const int i = e / l, j = e % l;
    W[e] = G[e] + (i == j ? delta : 0.0);
    R[e] = 0.0;
  }
  __syncthreads();
  for (int j = 0; j < l; ++j) {
    const double piv = sqrt(W[j * l + j] > delta ? W[j * l + j] : delta);
    for (int k = j + tid; k < l; k += kSplitThreads) R[j * l + k] = k == j ? piv : W[j * l + k] / piv;
    __syncthreads();
    const int m = l - j - 1;  // trailing block (j+1 .. l-1)^2, upper part
    for (int e = tid; e < m * m; e += kSplitThreads) {
      const int a = j + 1 + e / m, b = j + 1 + e % m;
      if (b >= a) W[a * l + b] -= R[j * l + a] * R[j * l + b];
    }
    __syncthreads();
  }
  // R^-1 (upper triangular), one column per thread: R X = I by back
  // substitution, X kept in fp64 in W (the Cholesky scratch is free now)
  for (int c = tid; c < l; c += kSplitThreads) {
    for (int i = l - 1; i >= 0; --i) {
      double v = 0.0;
      if (i <= c) {
        double s = i == c ? 1.0 : 0.0;
        for (int k = i + 1; k <= c; ++k) s -= R[i * l + k] * W[k * l + c];
        v = s / R[i * l + i];
      }
      W[i * l + c] = v;
      rinv[i * l + c] = (float)v;
    }
  }
}

// ---- symmetric eigen-decomposition (parallel cyclic Jacobi, fp64) ----------
// S (fp64 [l x l], symmetric) is diagonalized in place by rounds of disjoint
// Givens rotations (round-robin pairing, n - 1 rounds per sweep for n = l
// rounded up to even); V accumulates the rotations (both in LDS when they fit).  Sweeps stop once the
// off-diagonal mass is below 1e-30 of the diagonal's (at most 40).  Then
// the eigenvalues are sorted in decreasing order and the leading r give
//   sigma_j = sqrt(lambda_j)  (0 when below 1e-5 sigma_0: dropped),
//   M1[:, j] = v_j sigma_j^-1/2,  M2[:, j] = v_j sigma_j^1/2   (fp32 [l x r]).
__global__ __launch_bounds__(kSplitThreads) void jacobi_eig_kernel(const double* __restrict__ S0, int l, int r,
                                                                   double* Sg, double* Vg, float* __restrict__ M1,
                                                                   float* __restrict__ M2, float* __restrict__ sigma,
                                                                   int in_lds) {
  extern __shared__ double dyn[];
  __shared__ int pp[96], pq[96];
  __shared__ double pc[96], ps[96];
  __shared__ double red[2][kSplitThreads];
  __shared__ int order[192];
  __shared__ int stop;
  const int tid = threadIdx.x;
  const int n = l + (l & 1);
  const int npair = n / 2;
  // S and V in dynamic LDS when the launch provides 2 n^2 doubles, else global
  double* const S = in_lds ? dyn : Sg;
  double* const V = in_lds ? dyn + n * n : Vg;
  for (int e = tid; e < n * n; e += kSplitThreads) {
    const int i = e / n, j = e % n;
    S[e] = (i < l && j < l) ? S0[i * l + j] : 0.0;
    V[e] = i == j ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 40; ++sweep) {
    for (int round = 0; round < n - 1; ++round) {
      if (tid < npair) {
        // circle method: position 0 fixed, positions 1 .. n-1 rotate
        auto at = [&](int pos) { return pos == 0 ? 0 : 1 + (pos - 1 + round) % (n - 1); };
        int p = at(tid), q = at(n - 1 - tid);
        if (p > q) {
          const int t = p;
          p = q;
          q = t;
        }
        const double apq = S[p * n + q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double tau = (S[q * n + q] - S[p * n + p]) / (2.0 * apq);
          const double t = tau >= 0.0 ? 1.0 / (tau + sqrt(1.0 + tau * tau)) : -1.0 / (-tau + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        pp[tid] = p;
        pq[tid] = q;
        pc[tid] = c;
        ps[tid] = s;
      }
      __syncthreads();
      // rows p, q:  S <- J^T S
      for (int e = tid; e < npair * n; e += kSplitThreads) {
        const int k = e / npair, i = e % npair;
        const int p = pp[i], q = pq[i];
        const double c = pc[i], s = ps[i];
        const double a = S[p * n + k], b = S[q * n + k];
        S[p * n + k] = c * a - s * b;
        S[q * n + k] = s * a + c * b;
      }
      __syncthreads();
      // columns p, q:  S <- S J,  V <- V J
      for (int e = tid; e < npair * n; e += kSplitThreads) {
        const int k = e / npair, i = e % npair;
        const int p = pp[i], q = pq[i];
        const double c = pc[i], s = ps[i];
        const double a = S[k * n + p], b = S[k * n + q];
        S[k * n + p] = c * a - s * b;
        S[k * n + q] = s * a + c * b;
        const double va = V[k * n + p], vb = V[k * n + q];
        V[k * n + p] = c * va - s * vb;
        V[k * n + q] = s * va + c * vb;
      }
      __syncthreads();
    }
    double off = 0.0, dia = 0.0;
    for (int e = tid; e < n * n; e += kSplitThreads) {
      const double v = S[e];
      if (e / n == e % n) dia += v * v;
      else off += v * v;
    }
    red[0][tid] = off;
    red[1][tid] = dia;
    __syncthreads();
    for (int w = kSplitThreads / 2; w > 0; w >>= 1) {
      if (tid < w) {
        red[0][tid] += red[0][tid + w];
        red[1][tid] += red[1][tid + w];
      }
      __syncthreads();
    }
    if (tid == 0) stop = (red[0][0] <= 1e-30 * red[1][0]) ? 1 : 0;
    __syncthreads();
    if (stop) break;
  }
  if (tid == 0) {
    // selection sort of the real indices by eigenvalue, decreasing (ties: lower index first)
    for (int i = 0; i < l; ++i) order[i] = i;
    for (int i = 0; i < l; ++i) {
      int best = i;
      for (int j = i + 1; j < l; ++j)
        if (S[order[j] * n + order[j]] > S[order[best] * n + order[best]]) best = j;
      const int t = order[i];
      order[i] = order[best];
      order[best] = t;
    }
  }
  __syncthreads();
  const double lam0 = S[order[0] * n + order[0]];
  const double s0 = lam0 > 0.0 ? sqrt(lam0) : 0.0;
  for (int e = tid; e < l * r; e += kSplitThreads) {
    const int a = e / r, j = e % r;
    const int idx = order[j];
    const double lam = S[idx * n + idx];
    const double sg = lam > 0.0 ? sqrt(lam) : 0.0;
    const bool keep = s0 > 0.0 && sg > kSigmaDrop * s0;
    const double v = V[a * n + idx];
    M1[e] = keep ? (float)(v / sqrt(sg)) : 0.0f;
    M2[e] = keep ? (float)(v * sqrt(sg)) : 0.0f;
    if (a == 0) sigma[j] = keep ? (float)sg : 0.0f;
  }
}

// ---- branch factors ------------------------------------------------------
// L1[k, j] = bf16(F[k, j] / d[k]) (F = B^T M1, [K x r]); l1r keeps the rounded
// value as fp32 for the residual product.
__global__ void finish_l1_kernel(const float* __restrict__ F, const float* __restrict__ d, int64_t K, int r,
                                 uint16_t* __restrict__ l1, float* __restrict__ l1r) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= K * r) return;
  const uint32_t b = f32_to_bf16(F[e] / d[e / r]);
  l1[e] = (uint16_t)b;
  l1r[e] = bf16_to_f32(b);
}

// L2 = bf16(F) with F = Q M2 = L2^T, [N x r]: the factor is stored in the
// [N, rank] layout the low-rank GEMM reads (row n: the rank vector of output
// column n); l2r keeps the rounded values as fp32 in the same layout.
__global__ void finish_l2_kernel(const float* __restrict__ F, int64_t N, int r, uint16_t* __restrict__ l2,
                                 float* __restrict__ l2r) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= N * r) return;
  const uint32_t b = f32_to_bf16(F[e]);
  l2[e] = (uint16_t)b;
  l2r[e] = bf16_to_f32(b);
}

// T = W - C (in place over C = the branch in Linear layout), Rb = bf16(T).
__global__ void residual_kernel(const uint16_t* __restrict__ w, int64_t ldw, int64_t N, int64_t K,
                                float* __restrict__ T, uint16_t* __restrict__ Rb) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= N * K) return;
  const int64_t n = e / K, k = e % K;
  const float t = bf16_to_f32(w[n * ldw + k]) - T[e];
  T[e] = t;
  Rb[e] = (uint16_t)f32_to_bf16(t);
}

// ---- dequantize + unrotate: error partials and the next fit target ---------
// One 16-lane slot per 256-channel group (lane t: channels 16 t .. 16 t + 15).
// E = H (codes * scale) / 16 reconstructs the residual in the original basis
// (H / 16 is its own inverse).  has_q = 0: E = 0 (the first target A = W D).
// partial[block] = sum over the block of ((T - E) d)^2 (fixed order, fp64);
// A = (W - E) d when A != NULL.
__global__ __launch_bounds__(kSplitThreads) void deq_target_kernel(
    const uint16_t* __restrict__ w, int64_t ldw, int64_t N, int64_t K, const float* __restrict__ d,
    const uint8_t* __restrict__ codes, const float* __restrict__ scales, int mode, const float* __restrict__ T,
    float* __restrict__ A, double* __restrict__ partial) {
  __shared__ double red[kSplitThreads];
  const int tid = threadIdx.x;
  const int slot = tid >> 4, t = tid & 15;
  const int64_t ngroups = K >> 8;
  const int64_t gidx = (int64_t)blockIdx.x * 16 + slot;
  const bool ok = gidx < N * ngroups;  // uniform over the 16-lane slot
  double err = 0.0;
  if (ok) {
    const int64_t row = gidx / ngroups, g = gidx % ngroups;
    const int64_t c0 = g * 256 + t * 16;
    float e[16];
    if (codes) {
      // packed weight order: rows 2p, 2p + 1 interleaved per 128-channel slice
      const uint2 pk = *reinterpret_cast<const uint2*>(codes + (row >> 1) * K + ((c0 >> 7) << 7) + ((row & 1) << 6) +
                                                       ((c0 & 127) >> 1));
      const float sc = mode == 0 ? scales[0] : (mode == 1 ? scales[row] : scales[(c0 >> 6) * N + row]);
      const uint32_t wds[2] = {pk.x, pk.y};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // byte j of a run: low nibble channel 8h + j, high nibble 8h + j + 4
          const int byte = (int)((wds[h] >> (8 * j)) & 0xFFu);
          e[8 * h + j] = (float)(((byte & 0xF) ^ 8) - 8) * sc;
          e[8 * h + j + 4] = (float)((((byte >> 4) & 0xF) ^ 8) - 8) * sc;
        }
      hadamard256(e);
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] *= 0.0625f;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = 0.0f;
    }
    const uint4* wp = reinterpret_cast<const uint4*>(w + row * ldw + c0);
    const uint4 w0 = wp[0], w1 = wp[1];
    const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float wv[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      wv[2 * k] = __uint_as_float(ww[k] << 16);
      wv[2 * k + 1] = __uint_as_float(ww[k] & 0xffff0000u);
    }
    const float4* dp = reinterpret_cast<const float4*>(d + c0);
    float dv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = dp[q];
      dv[4 * q] = v.x;
      dv[4 * q + 1] = v.y;
      dv[4 * q + 2] = v.z;
      dv[4 * q + 3] = v.w;
    }
    if (codes && T) {
      const float4* tp = reinterpret_cast<const float4*>(T + row * K + c0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 tv = tp[q];
        const float tt[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const double x = (double)((tt[i] - e[4 * q + i]) * dv[4 * q + i]);
          err += x * x;
        }
      }
    }
    if (A) {
      float4* ap = reinterpret_cast<float4*>(A + row * K + c0);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ap[q] = make_float4((wv[4 * q] - e[4 * q]) * dv[4 * q], (wv[4 * q + 1] - e[4 * q + 1]) * dv[4 * q + 1],
                            (wv[4 * q + 2] - e[4 * q + 2]) * dv[4 * q + 2],
                            (wv[4 * q + 3] - e[4 * q + 3]) * dv[4 * q + 3]);
    }
  }
  if (!partial) return;
  red[tid] = err;
  __syncthreads();
  for (int wdt = kSplitThreads / 2; wdt > 0; wdt >>= 1) {
    if (tid < wdt) red[tid] += red[tid + wdt];
    __syncthreads();
  }
  if (tid == 0) partial[blockIdx.x] = red[0];
}

// Objective of iteration `it`: sqrt of the partials' sum (fixed order), into
// errors[it]; keeps the best (strictly smaller wins, ties keep the earlier).
__global__ __launch_bounds__(kSplitThreads) void select_best_kernel(const double* __restrict__ partial,
                                                                    int64_t nparts, int it, float* errors,
                                                                    double* best_err, int32_t* best_iter,
                                                                    int32_t* flag) {
  __shared__ double red[kSplitThreads];
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int64_t i = tid; i < nparts; i += kSplitThreads) s += partial[i];
  red[tid] = s;
  __syncthreads();
  for (int w = kSplitThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    const double err = sqrt(red[0]);
    errors[it] = (float)err;
    const bool better = it == 0 || err < *best_err;
    if (better) {
      *best_err = err;
      *best_iter = it;
    }
    *flag = better ? 1 : 0;
  }
}

// dst = src (bytes, 16-byte aligned, multiple of 4) when *flag is set.
__global__ void copy_if_kernel(const int32_t* __restrict__ flag, const uint8_t* __restrict__ src,
                               uint8_t* __restrict__ dst, int64_t bytes) {
  if (!*flag) return;
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16;
  if (i + 16 <= bytes) {
    *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(src + i);
  } else {
    for (int64_t j = i; j < bytes; j += 4)
      *reinterpret_cast<uint32_t*>(dst + j) = *reinterpret_cast<const uint32_t*>(src + j);
  }
}

// ---- workspace -----------------------------------------------------------
constexpr int64_t kAlign = 256;
int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t split_parts(int64_t Kd) {  // split-K factor of the long reductions
  const int64_t s = (Kd + 2047) / 2048;
  return s < 1 ? 1 : (s > 64 ? 64 : s);
}

struct Ws {
  float *A, *T, *Y, *Y2, *Z, *Z2, *parts, *rinv, *M1, *M2, *F1, *F2, *l1r, *l2r, *d, *sigma_c, *scales_c;
  double *G, *W, *R, *S, *V, *partial, *best_err;
  uint16_t *Rb, *l1_c, *l2_c;
  uint8_t* codes_c;
  int32_t* flag;
  int64_t bytes;
};

int64_t scale_count(int64_t N, int64_t K, int mode) { return mode == 0 ? 1 : (mode == 1 ? N : N * (K / 64)); }

Ws carve(uint8_t* base, int64_t N, int64_t K, int rank, int oversample, int mode) {
  const int64_t l = rank + oversample, n = l + (l & 1);
  const int64_t parts = split_parts(N > K ? N : K) * (K > N ? K : N) * l;
  Ws w{};
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  w.A = reinterpret_cast<float*>(take(N * K * 4));
  w.T = reinterpret_cast<float*>(take(N * K * 4));
  w.Rb = reinterpret_cast<uint16_t*>(take(N * K * 2));
  w.codes_c = take(N * K / 2);
  w.scales_c = reinterpret_cast<float*>(take(scale_count(N, K, mode) * 4));
  w.Y = reinterpret_cast<float*>(take(N * l * 4));
  w.Y2 = reinterpret_cast<float*>(take(N * l * 4));
  w.Z = reinterpret_cast<float*>(take(K * l * 4));
  w.Z2 = reinterpret_cast<float*>(take(K * l * 4));
  w.parts = reinterpret_cast<float*>(take(parts * 4));
  w.rinv = reinterpret_cast<float*>(take(l * l * 4));
  w.M1 = reinterpret_cast<float*>(take(l * rank * 4));
  w.M2 = reinterpret_cast<float*>(take(l * rank * 4));
  w.F1 = reinterpret_cast<float*>(take(K * rank * 4));
  w.F2 = reinterpret_cast<float*>(take(N * rank * 4));
  w.l1r = reinterpret_cast<float*>(take(K * rank * 4));
  w.l2r = reinterpret_cast<float*>(take(N * rank * 4));
  w.d = reinterpret_cast<float*>(take(K * 4));
  w.sigma_c = reinterpret_cast<float*>(take(rank * 4));
  w.l1_c = reinterpret_cast<uint16_t*>(take(K * rank * 2));
  w.l2_c = reinterpret_cast<uint16_t*>(take(N * rank * 2));
  w.G = reinterpret_cast<double*>(take(l * l * 8));
  w.W = reinterpret_cast<double*>(take(l * l * 8));
  w.R = reinterpret_cast<double*>(take(l * l * 8));
  w.S = reinterpret_cast<double*>(take(n * n * 8));
  w.V = reinterpret_cast<double*>(take(n * n * 8));
  w.partial = reinterpret_cast<double*>(take((N * (K >> 8) + 15) / 16 * 8));
  w.best_err = reinterpret_cast<double*>(take(8));
  w.flag = reinterpret_cast<int32_t*>(take(4));
  w.bytes = off;
  return w;
}

// ---- host-side sequencing ----------------------------------------------------
struct Runner {
  hipStream_t s;
  bool ok = true;
  void check() {
    if (hipGetLastError() != hipSuccess) ok = false;
  }
  // C = A * B (descriptor strides), split-K over S parts reduced into c32 / c64
  void gemm(const float* a, int64_t a_rs, int64_t a_cs, const float* b, int64_t b_rs, int64_t b_cs, float* c32,
            double* c64, int64_t M, int64_t Nc, int64_t Kd, int64_t S, float* parts) {
    GemmDesc g{a, a_rs, a_cs, b, b_rs, b_cs, nullptr, M, Nc, Kd, 0};
    if (S < 1) S = 1;
    g.kchunk = ((Kd + S - 1) / S + kGemmBK - 1) / kGemmBK * kGemmBK;
    S = (Kd + g.kchunk - 1) / g.kchunk;
    const bool direct = S == 1 && c32 && !c64;
    g.c = direct ? c32 : parts;
    const dim3 grid((unsigned)((Nc + 63) / 64), (unsigned)((M + 63) / 64), (unsigned)S);
    hipLaunchKernelGGL(sgemm_kernel, grid, dim3(kSplitThreads), 0, s, g);
    check();
    if (!direct) {
      const int64_t n = M * Nc;
      hipLaunchKernelGGL(reduce_parts_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, parts, (int)S, n,
                         c32, c64);
      check();
    }
  }
};

}  // namespace

int64_t svdq_split_workspace(int64_t N, int64_t K, int rank, int oversample, int mode) {
  return carve(nullptr, N, K, rank, oversample, mode).bytes;
}

int launch_svdq_split(const SplitArgs& a, hipStream_t s) {
  const int64_t N = a.N, K = a.K;
  const int r = a.rank;
  const int64_t l = a.rank + a.oversample;
  Ws w = carve(static_cast<uint8_t*>(a.workspace), N, K, a.rank, a.oversample, a.scale_mode);
  Runner run{s};
  const int64_t groups = N * (K >> 8);
  // the small fp64 matrices go to LDS when they fit (l <= 64), else they stay in the workspace
  const int64_t npad = l + (l & 1);
  const size_t chol_lds = 2 * l * l * 8 <= kSmallLds ? (size_t)(2 * l * l * 8) : 0;
  const size_t eig_lds = 2 * npad * npad * 8 <= kSmallLds ? (size_t)(2 * npad * npad * 8) : 0;
  const unsigned deq_blocks = (unsigned)((groups + 15) / 16);

  // CholeskyQR2: X [R x l] (row-major) -> orthonormal columns, back in X
  auto orth = [&](float* X, float* X2, int64_t R) {
    for (int pass = 0; pass < 2; ++pass) {
      float* src = pass == 0 ? X : X2;
      float* dst = pass == 0 ? X2 : X;
      run.gemm(src, 1, l, src, l, 1, nullptr, w.G, l, l, R, split_parts(R), w.parts);
      hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(kSplitThreads), chol_lds, s, w.G, (int)l, w.W, w.R, w.rinv,
                         chol_lds ? 1 : 0);
      run.check();
      run.gemm(src, l, 1, w.rinv, l, 1, dst, nullptr, R, l, l, 1, w.parts);
    }
  };

  hipLaunchKernelGGL(act_weights_kernel, dim3(1), dim3(kSplitThreads), 0, s, a.act_rms, K, w.d);
  run.check();
  // first target: A = W D
  hipLaunchKernelGGL(deq_target_kernel, dim3(deq_blocks), dim3(kSplitThreads), 0, s, a.w, a.ldw, N, K, w.d,
                     static_cast<const uint8_t*>(nullptr), static_cast<const float*>(nullptr), a.scale_mode,
                     static_cast<const float*>(nullptr), w.A, static_cast<double*>(nullptr));
  run.check();
  for (int it = 0; it <= a.refine_iters && run.ok; ++it) {
    // randomized subspace iteration on A [N x K]
    run.gemm(w.A, K, 1, a.omega, l, 1, w.Y, nullptr, N, l, K, 1, w.parts);
    orth(w.Y, w.Y2, N);
    for (int q = 0; q < a.power_iters; ++q) {
      run.gemm(w.A, 1, K, w.Y, l, 1, w.Z, nullptr, K, l, N, split_parts(N), w.parts);
      orth(w.Z, w.Z2, K);
      run.gemm(w.A, K, 1, w.Z, l, 1, w.Y, nullptr, N, l, K, 1, w.parts);
      orth(w.Y, w.Y2, N);
    }
    run.gemm(w.A, 1, K, w.Y, l, 1, w.Z, nullptr, K, l, N, split_parts(N), w.parts);  // Z = B^T
    run.gemm(w.Z, 1, l, w.Z, l, 1, nullptr, w.G, l, l, K, split_parts(K), w.parts);  // B B^T
    hipLaunchKernelGGL(jacobi_eig_kernel, dim3(1), dim3(kSplitThreads), eig_lds, s, w.G, (int)l, r, w.S, w.V, w.M1,
                       w.M2, w.sigma_c, eig_lds ? 1 : 0);
    run.check();
    // branch factors
    run.gemm(w.Z, l, 1, w.M1, r, 1, w.F1, nullptr, K, r, l, 1, w.parts);
    run.gemm(w.Y, l, 1, w.M2, r, 1, w.F2, nullptr, N, r, l, 1, w.parts);
    hipLaunchKernelGGL(finish_l1_kernel, dim3((unsigned)((K * r + 255) / 256)), dim3(256), 0, s, w.F1, w.d, K, r,
                       w.l1_c, w.l1r);
    run.check();
    hipLaunchKernelGGL(finish_l2_kernel, dim3((unsigned)((N * r + 255) / 256)), dim3(256), 0, s, w.F2, N, r, w.l2_c,
                       w.l2r);
    run.check();
    // residual T = W - (L1 L2)^T, quantized from its bf16 rounding
    run.gemm(w.l2r, r, 1, w.l1r, 1, r, w.T, nullptr, N, K, r, 1, w.parts);
    hipLaunchKernelGGL(residual_kernel, dim3((unsigned)((N * K + 255) / 256)), dim3(256), 0, s, a.w, a.ldw, N, K,
                       w.T, w.Rb);
    run.check();
    RqArgs q{w.Rb, N, K, K, 4, a.scale_mode, 1, 1, w.codes_c, w.scales_c};
    q.paired = 1;  // the GEMM's packed weight order
    if (launch_rotate_quantize(q, s) != OK) return ERR_LAUNCH;
    // objective, and the next iteration's target from this iteration's Q
    hipLaunchKernelGGL(deq_target_kernel, dim3(deq_blocks), dim3(kSplitThreads), 0, s, a.w, a.ldw, N, K, w.d,
                       static_cast<const uint8_t*>(w.codes_c), static_cast<const float*>(w.scales_c), a.scale_mode,
                       static_cast<const float*>(w.T), it < a.refine_iters ? w.A : static_cast<float*>(nullptr),
                       w.partial);
    run.check();
    hipLaunchKernelGGL(select_best_kernel, dim3(1), dim3(kSplitThreads), 0, s, w.partial, (int64_t)deq_blocks, it,
                       a.errors, w.best_err, a.best_iter, w.flag);
    run.check();
    auto copy = [&](const void* src, void* dst, int64_t bytes) {
      if (!dst) return;
      const int64_t chunks = (bytes + 15) / 16;
      hipLaunchKernelGGL(copy_if_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, w.flag,
                         static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), bytes);
      run.check();
    };
    copy(w.codes_c, a.packed, N * K / 2);
    copy(w.scales_c, a.scales, scale_count(N, K, a.scale_mode) * 4);
    copy(w.l1_c, a.l1, K * r * 2);
    copy(w.l2_c, a.l2, N * r * 2);
    copy(w.sigma_c, a.sigma, (int64_t)r * 4);
  }
  return run.ok ? OK : ERR_LAUNCH;
}

}  // namespace ql

// ---- allocation-free variant: the workspace in a library-owned array -------
// For callers that cannot allocate (graph capture, serving loops): the
// split's workspace lives in this file-scope device array instead of the
// caller's buffer.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address on the current device comes from
// hipGetSymbolAddress, looked up once per device and kept.  Every region of
// the workspace is written before it is read, so nothing needs clearing
// between calls; calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint8_t scratch[ql::kSplitScratchBytes];

namespace ql {
namespace {
constexpr int kMaxScratchDevices = 64;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch` per device; null until looked up
}  // namespace

int split_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return ERR_LAUNCH;
  void* p = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
  if (!p) {
    // with `dev` current: that device's copy of the array
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return ERR_LAUNCH;
    __atomic_store_n(&g_scratch_ptr[dev], q, __ATOMIC_RELEASE);  // concurrent first calls store the same value
    p = q;
  }
  *ptr = p;
  return OK;
}

}  // namespace ql
