// Closed-form absorb on gfx950: dW = (G + lambda I)^-1 (C W) by a blocked
// float32 Cholesky factorisation and blocked triangular solves, batched over
// layers; and the Gram-form reconstruction error used to rank layers.
//
// Source: "Technical Summary: Instance-Specific Parametric Absorption (ISPA)
// for Memory-Efficient Video Generation", section 2 "Methodology", step 2
// "Layer Absorb" (ridge objective, closed-form minimiser, non-iterative),
// step 3 "Memory-Efficient Inference" (W_new = W + dW) and "Dynamic Layer
// Selection" (rank layers by reconstruction error).
//
// Structure (nb = 64 column panels, right-looking):
//   M = G + lambda I (lambda scalar or per layer)      (init kernel)
//   R = C W at float32 accuracy                        (bf16 matrix cores, three-part splits; on the caller's
//                                                       side stream, if given, beside the factorisation)
//   factor M_00 = L_00 L_00^T and invert L_00        (one workgroup per layer)
//   for each panel k:
//     L_ik = M_ik L_kk^-T                             (GEMM, in place)
//     M_ij -= L_ik L_jk^T  (lower tiles only)         (GEMM; the workgroup of the next diagonal
//                                                      block then factors and inverts it)
//   explicit inverse of L by recursive doubling over block ranges (the levels inside the leading
//                                                      range of the last one on the side stream, beside
//                                                      the factorisation's last steps)
//   X = L^-T (L^-1 R)                                  (two triangular GEMMs)
//   one refinement step: r = R - G X - lambda X to ~2^-35 of the scales (exact int8
//   digit-slice products, else float64 accumulation), dW = X + L^-T (L^-1 r).
// The float32 factorisation alone loses about kappa * 2^-24 (about 1e-3 at the
// conditioning warmup statistics have, 1e5); the refinement step with a
// residual far more accurate than float32 brings dW to the accuracy of its
// float32 inputs.  Forming L^-1 once turns each triangular solve into one GEMM
// launch instead of one per panel.  The factor and inverse GEMMs run on
// v_mfma_f32_32x32x2_f32 with 64x64 tiles (triangular operands skip their zero
// blocks); the float64-accumulated products on v_mfma_f64_16x16x4_f64.  A layer whose pivot
// fails records info = column + 1 and is skipped by later kernels; its dW is
// set to NaN at the end and its W_new is left alone.
#include <algorithm>
#include <utility>
#include <vector>

#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int NB = 64;  // panel width

// Cholesky of the NB x NB diagonal block at (k0, k0) of each layer (lower L written in place, zeros
// above its diagonal) and its inverse L^-1 into the same block of Linvf
// (zeros above the diagonal).  info[b] = k0 + j + 1 if the leading minor of order k0 + j + 1 of
// G + lambda I is not positive definite (LAPACK potrf convention); then nothing is written.
//
// One workgroup of 4 waves; wave w holds block column w (16 columns) with lane i = row i.  The
// 16 pivot steps of a block column run inside its wave (cross-lane reads, no barrier); the wave
// publishes the finished columns in LDS, the later block columns subtract their rank-16 update
// in parallel, and meanwhile the wave inverts its 16 x 16 diagonal block.  The off-diagonal blocks
// of L^-1 follow by two doubling levels, inv([A 0; B C]) = [A^-1 0; -C^-1 B A^-1  C^-1].
// Workgroups (over the batch) that R = C W may hold while it runs beside the factorisation: one
// per compute unit, so every unit keeps room for the factorisation's launches.
#ifndef ISPA_CW_WORKGROUPS
#define ISPA_CW_WORKGROUPS 256
#endif
// Workgroups the bf16 R = C W may hold beside the factorisation (one per compute unit at most).  On
// 256 x 256 tiles (8 waves each) at d = 5120, per refined solve on one box: 67 -> 11.13 ms,
// 80 -> 10.51, 90 -> 10.49, 100 -> 10.57 (its 400 tiles in four whole rounds), 110 -> 10.60;
// 128 -> 11.2 on another.
#ifndef ISPA_RESID_I8
#define ISPA_RESID_I8 1  // the refinement residual from int8 digit slices (else float64 accumulation)
#endif
#ifndef ISPA_CW6_WORKGROUPS
#define ISPA_CW6_WORKGROUPS 100
#endif
// Columns per panel of the blocked trailing update (a multiple of NB).
#ifndef ISPA_CHOL_PANEL
#define ISPA_CHOL_PANEL 512
#endif
#ifndef ISPA_CHOL_DEFER
#define ISPA_CHOL_DEFER 1  // defer the panel updates right of the next panel into its steps' launches
#endif
#ifndef ISPA_PAIR_WORKGROUPS
#define ISPA_PAIR_WORKGROUPS 0  // workgroups the inverse's last-pair product may hold beside the chain (0: all)
#endif
#ifndef ISPA_DEFER_SKIP_XCD
#define ISPA_DEFER_SKIP_XCD 1  // deferred tiles leave the XCD of the factoring workgroup alone
#endif
#ifndef ISPA_CHOL_DEFER_MIN
#define ISPA_CHOL_DEFER_MIN 1024  // fewest columns right of the next panel for which that pays
#endif
constexpr int CP = ISPA_CHOL_PANEL;
static_assert(CP % 64 == 0, "panel of whole blocks");
constexpr int SB = NB / 4;     // block column width
constexpr int LSTR = NB + 4;   // LDS row stride (floats): rows stay 16-byte aligned for vector reads
static_assert(NB == 64 && SB == 16, "the diagonal kernel maps 64 rows onto the 64 lanes of a wave");

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// LDS of one diagonal-block factorisation: L (zeros above the diagonal), L^-1, and the product
// scratch of the doubling steps with the failure flag after it.
constexpr int DIAG_LS_FLOATS = NB * LSTR, DIAG_TS_FLOATS = 32 * 36 + 4;

// Body of the factorisation for layer b; called by all 256 threads of a workgroup, which must not
// be inside a branch that differs between its waves.  Ls and Xs hold NB * LSTR floats each, Ts
// DIAG_TS_FLOATS, all 16-byte aligned.  With from_ls the block is read from Ls (written there by
// the caller before a barrier) instead of from M.
__device__ __forceinline__ void potrf_diag_block(float* M, int d, int k0, float* Linvf, int32_t* info, int b,
                                                 float (*Ls)[LSTR], float (*Xs)[LSTR], float (*Ts)[36],
                                                 bool from_ls = false) {
  int& fail_s = *(int*)&Ts[32][0];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* Mb = M + (size_t)b * d * d + (size_t)k0 * d + k0;

  float a[SB];  // row `lane`, columns SB*wave .. SB*wave+15
  if (from_ls) {
#pragma unroll
    for (int q = 0; q < SB / 4; ++q) {
      const f32x4 v = *(const f32x4*)(&Ls[lane][SB * wave + 4 * q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[4 * q + e] = v[e];
    }  // (Ls is next written after the barrier below)
  } else {
    const float* src = Mb + (size_t)lane * d + SB * wave;
#pragma unroll
    for (int q = 0; q < SB / 4; ++q) {
      const f32x4 v = *(const f32x4*)(src + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[4 * q + e] = v[e];
    }
  }
  // zero X outside the diagonal 16-blocks (the lower blocks are filled by the doubling steps)
  for (int e = tid; e < NB * NB; e += 256) {
    const int rr = e / NB, cc = e % NB;
    if (rr / SB != cc / SB) Xs[rr][cc] = 0.f;
  }
  if (tid == 0) fail_s = 0;
  __syncthreads();

  for (int kb = 0; kb < NB / SB; ++kb) {
    const int c0 = SB * kb;
    if (wave == kb) {
      // right-looking steps inside the block column; rows above c0 + j carry values that are
      // never used (only lanes >= c0 + j feed pivots and multipliers) and are masked on publication.
      // A failed pivot is recorded and the steps run on; nothing is published then.
      int failed = 0;
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const float piv = readlane_f(a[j], c0 + j);
        if (!(piv > 0.f) && failed == 0) failed = c0 + j + 1;
        const float lij = a[j] * __builtin_amdgcn_rsqf(piv);  // v_rsq_f32 (pivots are normal positives)
#pragma unroll
        for (int k = j + 1; k < SB; ++k) a[k] = fmaf(-lij, readlane_f(lij, c0 + k), a[k]);
        a[j] = lij;
        // one pivot step at a time: its cross-lane reads issue before the next pivot's (17.0 -> 16.0 us
        // per 64 x 64 block)
        __builtin_amdgcn_sched_barrier(0);
      }
      if (failed) {
        if (lane == 0) fail_s = k0 + failed;
      } else {
#pragma unroll
        for (int m = 0; m < SB; m += 4)
          *(f32x4*)(&Ls[lane][c0 + m]) = f32x4{lane >= c0 + m ? a[m] : 0.f, lane >= c0 + m + 1 ? a[m + 1] : 0.f,
                                              lane >= c0 + m + 2 ? a[m + 2] : 0.f, lane >= c0 + m + 3 ? a[m + 3] : 0.f};
      }
    }
    __syncthreads();
    if (fail_s != 0) {
      if (tid == 0) info[b] = fail_s;
      return;
    }
    if (wave > kb) {
      // a[:, m] -= L[:, block kb] L[SB*wave + m, block kb]^T
      // (16 independent accumulation chains: the FMAs are not latency-bound)
#pragma unroll
      for (int q = 0; q < SB / 4; ++q) {
        const f32x4 li = *(const f32x4*)(&Ls[lane][c0 + 4 * q]);
#pragma unroll
        for (int m = 0; m < SB; ++m) {
          const f32x4 lc = *(const f32x4*)(&Ls[SB * wave + m][c0 + 4 * q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) a[m] = fmaf(-li[e], lc[e], a[m]);
        }
      }
    } else if (wave == kb) {
      // inverse of the diagonal block (rows c0 .. c0+15 = lanes): lane c0+i keeps row i of
      // X = L_kk^-1 unnormalised, x = e_i - sum_{p<i} L[i][p] X[p]; row k is final once divided
      // by L[k][k].  Lanes outside the block compute values that are never stored.
      float x[SB];
#pragma unroll
      for (int c = 0; c < SB; ++c) x[c] = (lane == c0 + c) ? 1.f : 0.f;
#pragma unroll
      for (int k = 0; k < SB - 1; ++k) {
        const float inv_kk = __builtin_amdgcn_rcpf(readlane_f(a[k], c0 + k));
        const float t = lane > c0 + k ? a[k] * inv_kk : 0.f;  // L[i][k] / L[k][k] for the rows below k
#pragma unroll
        for (int c = 0; c <= k; ++c) x[c] = fmaf(-t, readlane_f(x[c], c0 + k), x[c]);
      }
      // lane c0+i: X[i] = x / L[i][i]; a[i] of lane c0+i is L[i][i]: read it from LDS
      const float inv_ii = lane >= c0 && lane < c0 + SB ? __builtin_amdgcn_rcpf(Ls[lane][lane]) : 0.f;
      if (lane >= c0 && lane < c0 + SB) {
#pragma unroll
        for (int c = 0; c < SB; c += 4)
          *(f32x4*)(&Xs[lane][c0 + c]) = f32x4{x[c] * inv_ii, x[c + 1] * inv_ii, x[c + 2] * inv_ii, x[c + 3] * inv_ii};
      }
    }
  }
  __syncthreads();

  // ---- level 1: X[hi][lo] = -X[hi][hi] L[hi][lo] X[lo][lo] for 16-block pairs (0,1) and (2,3),
  // waves 1 and 3 (lane (i, g): row i, columns 4g .. 4g+3 of the 16 x 16 result)
  if (wave & 1) {
    const int lo = SB * (wave - 1), hi = SB * wave;
    const int i = lane & 15, g = lane >> 4;
    const int tr = (wave >> 1) * SB;
    // (four partial sums per product keep the FMA chains short)
    f32x4 t[4] = {};  // (L[hi][lo] X[lo][lo])[i][4g .. 4g+3]
#pragma unroll
    for (int p = 0; p < SB; ++p) t[p & 3] += Ls[hi + i][lo + p] * *(const f32x4*)(&Xs[lo + p][lo + 4 * g]);
    *(f32x4*)(&Ts[tr + i][4 * g]) = (t[0] + t[1]) + (t[2] + t[3]);
    __builtin_amdgcn_wave_barrier();  // the same wave reads Ts back (LDS is in order within a wave)
    f32x4 o[4] = {};
#pragma unroll
    for (int p = 0; p < SB; ++p) o[p & 3] += Xs[hi + i][hi + p] * *(const f32x4*)(&Ts[tr + p][4 * g]);
    *(f32x4*)(&Xs[hi + i][lo + 4 * g]) = -((o[0] + o[1]) + (o[2] + o[3]));
  }
  __syncthreads();

  // ---- level 2: X[32:64][0:32] = -X[32:64][32:64] L[32:64][0:32] X[0:32][0:32]; thread: row tid / 8,
  // columns 4 (tid % 8) .. +3 of the 32 x 32 result
  {
    const int i = tid >> 3, c = 4 * (tid & 7);
    f32x4 t[4] = {};
#pragma unroll
    for (int p = 0; p < 32; ++p) t[p & 3] += Ls[32 + i][p] * *(const f32x4*)(&Xs[p][c]);
    *(f32x4*)(&Ts[i][c]) = (t[0] + t[1]) + (t[2] + t[3]);
    __syncthreads();
    f32x4 o[4] = {};
#pragma unroll
    for (int p = 0; p < 32; ++p) o[p & 3] += Xs[32 + i][32 + p] * *(const f32x4*)(&Ts[p][c]);
    *(f32x4*)(&Xs[32 + i][c]) = -((o[0] + o[1]) + (o[2] + o[3]));
  }
  __syncthreads();

  float* Xb = Linvf + (size_t)b * d * d + (size_t)k0 * d + k0;
  for (int e = tid; e < NB * NB / 4; e += 256) {
    const int rr = e / (NB / 4), cc = 4 * (e % (NB / 4));
    *(f32x4*)(Xb + (size_t)rr * d + cc) = *(const f32x4*)(&Xs[rr][cc]);
    // whole rows of L, with the zeros above its diagonal: the strict upper part of a diagonal
    // block of M is never read
    *(f32x4*)(Mb + (size_t)rr * d + cc) = *(const f32x4*)(&Ls[rr][cc]);
  }
}

__global__ __launch_bounds__(256) void potrf_diag_kernel(float* M, int d, int k0, float* Linvf, int32_t* info) {
  const int b = blockIdx.x;
  if (info[b] != 0) return;
  __shared__ __attribute__((aligned(16))) float Ls[NB][LSTR];
  __shared__ __attribute__((aligned(16))) float Xs[NB][LSTR];
  __shared__ __attribute__((aligned(16))) float Ts[DIAG_TS_FLOATS / 36 + 1][36];
  potrf_diag_block(M, d, k0, Linvf, info, b, Ls, Xs, Ts);
}

struct GemmParams {
  const float* A;
  const float* B;
  const float* Cin;
  float* D;
  int M, N, K;
  int lda, ldb, ldc, ldd;
  size_t sA, sB, sC, sD;  // batch strides (elements)
  float alpha, beta;
  int lower_only;         // skip 64x64 tiles strictly above the diagonal
  int kmode;              // 0 all k; 1 op(A) lower: k < m0+T; 2 op(A) upper: k >= m0; 3 op(B) lower: k >= n0
  const int32_t* info;    // skip batch entries with info != 0 (nullable)
  int npairs;             // grid.z = batch * npairs; pair q adds q * pA, pB, pC, pD
  size_t pA, pB, pC, pD;
  // fused look-ahead (trailing update only): the workgroup of output tile (0, 0), the next
  // diagonal block, factors it afterwards (potrf_diag_block on block diag_k0 of diag_M)
  float* diag_M;
  float* diag_Linv;
  int32_t* diag_info;
  int diag_d, diag_k0;
  // deferred trailing-update tiles carried by a fused look-ahead launch (one layer only): the
  // workgroups in grid rows past M / T take lower tiles ex_t0 .. ex_t0 + ex_n - 1 (row-major over
  // the lower triangle of an ex_nt x ex_nt grid of T x T tiles) of ex_D -= ex_A ex_A^T with depth
  // ex_K, row stride ex_ld for both.  Slots whose dispatch index is a multiple of 8 (the XCD of
  // tile (0, 0), whose workgroup then runs the latency-bound factorisation) stay empty.
  const float* ex_A;
  float* ex_D;
  int ex_ld, ex_K, ex_t0, ex_n;
};

// D = alpha * op(A) op(B) + beta * Cin; op(A) is MxK, op(B) is KxN.
// TA: A stored KxM (op(A) = A^T); TB: B stored NxK (op(B) = B^T).
// T x T output tile (T = 64 or 128), 4 waves in 2x2, each (T/2)x(T/2) as blocks of
// v_mfma_f32_32x32x2_f32.  K advances in slabs of GKS: the next slab's operands are loaded into
// registers while the current one is multiplied from LDS (two LDS buffers, one barrier per slab),
// so few resident workgroups still hide the load latency.  M, N multiples of T; K multiple of GKS.
// Cin may equal D.
constexpr int GKS = 32;

// PERSIST: grid.x workgroups per batch entry loop over the output tiles (row-major, each XCD's
// workgroups on consecutive tiles), so a long product holds at most grid.x slots of the GPU while
// a latency-bound chain of small launches runs beside it on another stream.
template <bool TA, bool TB, int T, bool DIAG = false, bool PERSIST = false>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  constexpr int WB = T / 64;               // 32x32 blocks per wave per dimension
  constexpr int NLD = T * GKS / 1024;      // float4 loads per thread per operand per slab
  const int b = blockIdx.z / p.npairs, q = blockIdx.z % p.npairs;
  if (p.info && p.info[b] != 0) return;
  __shared__ __attribute__((aligned(16))) float As[2][GKS][T + 4];  // [buffer][k][m]
  __shared__ __attribute__((aligned(16))) float Bs[2][GKS][T + 4];  // [buffer][k][n]
  static_assert(2 * GKS * (T + 4) >= DIAG_LS_FLOATS, "the diagonal factorisation reuses As and Bs");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = (wave >> 1) * (T / 2), wn = (wave & 1) * (T / 2);
  // one output tile: D = alpha * op(A) op(B) + beta * Cin over k in [kb, ke)
  // With ldsd the tile's leading NB x NB block goes to ldsd (row stride LSTR) instead of D.
  auto run_tile = [&](const float* A, const float* B, int lda, int ldb, const float* Cin, int ldc, float* D, int ldd,
                      const int tm, const int tn, const int kb, const int ke, float* ldsd) {
  const int m0 = tm * T, n0 = tn * T;
  f32x16 acc[WB][WB];
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j) acc[i][j] = f32x16{0};
  f32x4 ra[NLD], rb[NLD];
  auto load = [&](int k0) {
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
      const int t = tid + 256 * r;
      if (!TA) {
        const int m = t / (GKS / 4), kq = t % (GKS / 4);
        ra[r] = *(const f32x4*)(A + (size_t)(m0 + m) * lda + k0 + 4 * kq);
      } else {
        const int k = t / (T / 4), mq = t % (T / 4);
        ra[r] = *(const f32x4*)(A + (size_t)(k0 + k) * lda + m0 + 4 * mq);
      }
      if (TB) {
        const int n = t / (GKS / 4), kq = t % (GKS / 4);
        rb[r] = *(const f32x4*)(B + (size_t)(n0 + n) * ldb + k0 + 4 * kq);
      } else {
        const int k = t / (T / 4), nq = t % (T / 4);
        rb[r] = *(const f32x4*)(B + (size_t)(k0 + k) * ldb + n0 + 4 * nq);
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
      const int t = tid + 256 * r;
      if (!TA) {
        const int m = t / (GKS / 4), kq = t % (GKS / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) As[buf][4 * kq + e][m] = ra[r][e];
      } else {
        const int k = t / (T / 4), mq = t % (T / 4);
        *(f32x4*)(&As[buf][k][4 * mq]) = ra[r];
      }
      if (TB) {
        const int n = t / (GKS / 4), kq = t % (GKS / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[buf][4 * kq + e][n] = rb[r][e];
      } else {
        const int k = t / (T / 4), nq = t % (T / 4);
        *(f32x4*)(&Bs[buf][k][4 * nq]) = rb[r];
      }
    }
  };
  if (kb < ke) {
    load(kb);
    store(0);
    __syncthreads();
  }
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += GKS) {
    const bool more = k0 + GKS < ke;
    if (more) load(k0 + GKS);  // in flight during the multiplies below
    // operands of step kk + 1 are read from LDS before the multiplies of step kk are issued, so the
    // LDS latency hides behind them (sched_barrier keeps the compiler from sinking the reads)
    float a[2][WB], bv[2][WB];
#pragma unroll
    for (int i = 0; i < WB; ++i) {
      a[0][i] = As[buf][hh][wm + 32 * i + l32];
      bv[0][i] = Bs[buf][hh][wn + 32 * i + l32];
    }
#pragma unroll
    for (int kk = 0; kk < GKS / 2; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < GKS / 2) {
#pragma unroll
        for (int i = 0; i < WB; ++i) {
          a[c ^ 1][i] = As[buf][2 * (kk + 1) + hh][wm + 32 * i + l32];
          bv[c ^ 1][i] = Bs[buf][2 * (kk + 1) + hh][wn + 32 * i + l32];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[c][i], bv[c][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) store(buf ^ 1);  // the other buffer: its last readers finished before the previous barrier
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
        const int c = n0 + wn + 32 * j + l32;
        float x = p.alpha * acc[i][j][v];
        if (Cin && p.beta != 0.f) x = fmaf(p.beta, Cin[(size_t)r * ldc + c], x);
        if (ldsd != nullptr && wm + 32 * i < NB && wn + 32 * j < NB)
          ldsd[(r - m0) * LSTR + (c - n0)] = x;
        else
          D[(size_t)r * ldd + c] = x;
      }
  };
  const float* A = p.A + b * p.sA + q * p.pA;
  const float* B = p.B + b * p.sB + q * p.pB;
  const float* Cin = p.Cin ? p.Cin + b * p.sC + q * p.pC : nullptr;
  float* D = p.D + b * p.sD + q * p.pD;
  auto kbeg = [&](int tm, int tn) { return p.kmode == 2 ? tm * T : (p.kmode == 3 ? tn * T : 0); };
  auto kend = [&](int tm) { return p.kmode == 1 ? min(p.K, tm * T + T) : p.K; };
  if constexpr (PERSIST) {
    // (every slab ends with a barrier, so the LDS is free when the next tile starts)
    const int tiles_n = p.N / T, tiles = (p.M / T) * tiles_n;
    for (int t = (int)xcd_remap(blockIdx.x, gridDim.x); t < tiles; t += gridDim.x) {
      const int tm = t / tiles_n, tn = t % tiles_n;
      run_tile(A, B, p.lda, p.ldb, Cin, p.ldc, D, p.ldd, tm, tn, kbeg(tm, tn), kend(tm), nullptr);
    }
    return;
  }
  if constexpr (DIAG) {
    if (p.ex_n > 0 && (int)blockIdx.y >= p.M / T) {
      // a deferred tile (kmode 0, one layer): skip the slots on the XCD of tile (0, 0)
      const int lin = (int)(blockIdx.y * gridDim.x + blockIdx.x), prim = (p.M / T) * (int)gridDim.x;
      if (ISPA_DEFER_SKIP_XCD && lin % 8 == 0) return;
      const int ti = (lin - prim) - (ISPA_DEFER_SKIP_XCD ? (lin + 7) / 8 - (prim + 7) / 8 : 0);
      if (ti >= p.ex_n) return;
      const int t = p.ex_t0 + ti;
      int r = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);  // row of the lower-triangle tile t
      while (r > 0 && r * (r + 1) / 2 > t) --r;
      while ((r + 1) * (r + 2) / 2 <= t) ++r;
      const int c = t - r * (r + 1) / 2;
      run_tile(p.ex_A, p.ex_A, p.ex_ld, p.ex_ld, p.ex_D, p.ex_ld, p.ex_D, p.ex_ld, r, c, 0, p.ex_K, nullptr);
      return;
    }
  }
  // with op(A) lower the last row tiles carry the most K work: dispatch them first
  const int tm = p.kmode == 1 ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y, tn = blockIdx.x;
  if (p.lower_only && tm < tn) return;
  // the workgroup of tile (0, 0) of a fused look-ahead launch keeps the next diagonal block (the
  // tile's leading 64 x 64) in the LDS the multiply no longer needs and factors it from there; its
  // updated values never go to M, whose block the factorisation overwrites with L
  const bool diag_tile = DIAG && tm == 0 && tn == 0 && q == 0;
  run_tile(A, B, p.lda, p.ldb, Cin, p.ldc, D, p.ldd, tm, tn, kbeg(tm, tn), kend(tm),
           diag_tile ? &As[0][0][0] : nullptr);
  if constexpr (DIAG) {
    if (diag_tile) {
      __shared__ __attribute__((aligned(16))) float Tx[DIAG_TS_FLOATS / 36 + 1][36];
      __syncthreads();
      potrf_diag_block(p.diag_M, p.diag_d, p.diag_k0, p.diag_Linv, p.diag_info, b, (float(*)[LSTR]) & As[0][0][0],
                       (float(*)[LSTR]) & Bs[0][0][0], Tx, true);
    }
  }
}

struct GemmDParams {
  const float* A;      // M x K, row-major (lda)
  const float* B;      // K x N, row-major (ldb)
  const float* Cin;    // M x N float32 (ldc), nullable; widened to float64 in the epilogue
  const float* X;      // M x N float32 (ldx), nullable
  double* D64;         // nullable
  float* D32;          // nullable
  int M, N, K;
  int lda, ldb, ldc, ldx, ldd;
  size_t sA, sB, sC, sX, sD;
  double alpha, beta, gamma;
  const float* gamma_b;  // nullable: gamma * gamma_b[b] for batch entry b (per-layer lambda)
  const int32_t* info;
};

typedef double f64x4 __attribute__((ext_vector_type(4)));

// D = alpha * A B + beta * Cin + gamma * X with float64 accumulation of the
// (exact) products of float32 operands, on v_mfma_f64_16x16x4_f64.  64x64 tile,
// 4 waves of 32x32 (2x2 blocks of 16x16).  Operand layout of the f64 MFMA:
// lane l holds A[l%16][l/16] and B[l/16][l%16]; output element v of lane l is
// row 4v + l/16, column l%16 of its block.  M, N multiples of 64, K of 16.
__global__ __launch_bounds__(256) void gemm_f64acc_kernel(GemmDParams p) {
  const int b = blockIdx.z;
  if (p.info && p.info[b] != 0) return;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  __shared__ float As[16][64 + 4];  // [k][m]
  __shared__ float Bs[16][64 + 4];  // [k][n]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const float* A = p.A + b * p.sA;
  const float* B = p.B + b * p.sB;
  const double gb = p.gamma_b ? p.gamma * (double)p.gamma_b[b] : p.gamma;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0, 0, 0, 0};
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    {
      const int m = tid >> 2, kq = tid & 3;
      const f32x4 v = *(const f32x4*)(A + (size_t)(m0 + m) * p.lda + k0 + 4 * kq);
#pragma unroll
      for (int e = 0; e < 4; ++e) As[4 * kq + e][m] = v[e];
      const int k = tid >> 4, nq = tid & 15;
      *(f32x4*)(&Bs[k][4 * nq]) = *(const f32x4*)(B + (size_t)(k0 + k) * p.ldb + n0 + 4 * nq);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      double a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = (double)As[4 * kk + g][wm + 16 * i + l16];
        bb[i] = (double)Bs[4 * kk + g][wn + 16 * i + l16];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = m0 + wm + 16 * i + 4 * v + g;
        const int c = n0 + wn + 16 * j + l16;
        double x = p.alpha * acc[i][j][v];
        if (p.Cin) x += p.beta * (double)p.Cin[b * p.sC + (size_t)r * p.ldc + c];
        if (p.X) x += gb * (double)p.X[b * p.sX + (size_t)r * p.ldx + c];
        if (p.D64) p.D64[b * p.sD + (size_t)r * p.ldd + c] = x;
        if (p.D32) p.D32[b * p.sD + (size_t)r * p.ldd + c] = (float)x;
      }
}

// The same product with 32-deep K slabs: the next slab's operands are loaded into registers while
// the current one is multiplied from LDS (two LDS buffers, one barrier per slab).
constexpr int DKS = 32;
#ifndef ISPA_F64_WAVES
#define ISPA_F64_WAVES 5  // waves per SIMD the register budget allows (five workgroups per compute unit)
#endif
__global__ __launch_bounds__(256, ISPA_F64_WAVES) void gemm_f64acc2_kernel(GemmDParams p) {
  const int b = blockIdx.z;
  if (p.info && p.info[b] != 0) return;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  // rows of 64 floats with column c of row k stored at c ^ 16 (k % 4): the four k rows a fragment
  // read touches (lanes 16 apart) fall on different 16-bank groups.  32 KB: five workgroups per
  // compute unit, so 64 x 64 tiles of a 5120 x 5120 output fill the chip in five whole rounds.
  __shared__ float As[2][DKS][64];  // [buffer][k][m ^ 16 (k % 4)]
  __shared__ float Bs[2][DKS][64];  // [buffer][k][n ^ 16 (k % 4)]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const float* A = p.A + b * p.sA;
  const float* B = p.B + b * p.sB;
  const double gb = p.gamma_b ? p.gamma * (double)p.gamma_b[b] : p.gamma;
  f32x4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t = tid + 256 * r;
      const int m = t >> 3, kq = t & 7;  // A: 64 rows x 8 float4 along k
      ra[r] = *(const f32x4*)(A + (size_t)(m0 + m) * p.lda + k0 + 4 * kq);
      const int k = t >> 4, nq = t & 15;  // B: 32 rows (k) x 16 float4 along n
      rb[r] = *(const f32x4*)(B + (size_t)(k0 + k) * p.ldb + n0 + 4 * nq);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t = tid + 256 * r;
      const int m = t >> 3, kq = t & 7;
#pragma unroll
      for (int e = 0; e < 4; ++e) As[buf][4 * kq + e][m ^ (16 * e)] = ra[r][e];
      const int k = t >> 4, nq = t & 15;
      *(f32x4*)(&Bs[buf][k][(4 * nq) ^ (16 * (k & 3))]) = rb[r];
    }
  };
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0, 0, 0, 0};
  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < p.K; k0 += DKS) {
    const bool more = k0 + DKS < p.K;
    if (more) load(k0 + DKS);
#pragma unroll
    for (int kk = 0; kk < DKS / 4; ++kk) {
      double a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = (double)As[buf][4 * kk + g][(wm + 16 * i + l16) ^ (16 * g)];
        bb[i] = (double)Bs[buf][4 * kk + g][(wn + 16 * i + l16) ^ (16 * g)];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
    if (more) store(buf ^ 1);  // the other buffer: its last readers finished before the previous barrier
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = m0 + wm + 16 * i + 4 * v + g;
        const int c = n0 + wn + 16 * j + l16;
        double x = p.alpha * acc[i][j][v];
        if (p.Cin) x += p.beta * (double)p.Cin[b * p.sC + (size_t)r * p.ldc + c];
        if (p.X) x += gb * (double)p.X[b * p.sX + (size_t)r * p.ldx + c];
        if (p.D64) p.D64[b * p.sD + (size_t)r * p.ldd + c] = x;
        if (p.D32) p.D32[b * p.sD + (size_t)r * p.ldd + c] = (float)x;
      }
}


// M = G + lambda I (full matrix); L^-1 = 0; info = 0.
__global__ __launch_bounds__(256) void init_shift_kernel(const float* __restrict__ G, float* M, float* Linvf, int d,
                                                         float lambda, const float* __restrict__ lam_b,
                                                         int32_t* info) {
  const int b = blockIdx.y;
  if (lam_b) lambda = lam_b[b];
  const size_t dd = (size_t)d * d;
  const size_t i4 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (blockIdx.x == 0 && threadIdx.x == 0) info[b] = 0;
  if (i4 >= dd) return;
  f32x4 v = *(const f32x4*)(G + b * dd + i4);
  const int row = (int)(i4 / d), col = (int)(i4 % d);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (col + e == row) v[e] += lambda;
  *(f32x4*)(M + b * dd + i4) = v;
  // L^-1 is only ever written on and below its diagonal blocks, while the triangular products read
  // whole 128 x 128 tiles of it: the part above must be zero, whatever the workspace held before
  *(f32x4*)(Linvf + b * dd + i4) = f32x4{0.f, 0.f, 0.f, 0.f};
}


// dW = X + correction, or NaN for failed layers; W_new = W + dW for the others (W_new may be W).
__global__ __launch_bounds__(256) void finalize_kernel(const float* W, float* dW, const float* corr, float* Wn,
                                                       size_t n, const int32_t* info) {
  const int b = blockIdx.y;
  const size_t i4 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= n) return;
  float* dw = dW + b * n + i4;
  if (info[b] != 0) {
    *(f32x4*)dw = f32x4{NAN, NAN, NAN, NAN};
    return;
  }
  const f32x4 x = corr ? *(const f32x4*)dw + *(const f32x4*)(corr + b * n + i4) : *(const f32x4*)dw;
  *(f32x4*)dw = x;
  if (Wn) *(f32x4*)(Wn + b * n + i4) = *(const f32x4*)(W + b * n + i4) + x;
}

// Inner products for the reconstruction error of the fitted dW, reduced in float64 in a fixed
// order.  With D = A_full - A_loc and the statistics G = A_loc^T A_loc, C = A_loc^T D, E = D^T D:
//   eps = ||D W - A_loc dW||^2 = <E W, W> - 2 <C W, dW> + <G dW, dW>, and the normal equation
//   (G + lambda I) dW = C W turns the last two terms into -<dW, C W> - lambda ||dW||^2;
//   ||A_full W||^2 = <(G + C + C^T + E) W, W> = <E W, W> + 2 <C W, W> + <G W, W>.
// Forming E from D (not from A_full^T A_full) keeps eps accurate when D is small.
__global__ __launch_bounds__(256) void eps_reduce_kernel(const float* W, const float* dW, const float* EW,
                                                         const float* CW, const float* GW, size_t n, float lambda,
                                                         double* eps_abs, double* eps_rel) {
  const int b = blockIdx.x;
  const size_t off = (size_t)b * n;
  double s[5] = {0, 0, 0, 0, 0};
  for (size_t i = threadIdx.x; i < n; i += 256) {
    const double w = W[off + i], dw = dW[off + i], cw = CW[off + i];
    s[0] += (double)EW[off + i] * w;
    s[1] += cw * w;
    s[2] += (double)GW[off + i] * w;
    s[3] += dw * cw;
    s[4] += dw * dw;
  }
  __shared__ double red[5][256];
  for (int k = 0; k < 5; ++k) red[k][threadIdx.x] = s[k];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w)
      for (int k = 0; k < 5; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double e = red[0][0] - red[3][0] - (double)lambda * red[4][0];
    eps_abs[b] = e;
    eps_rel[b] = e / (red[0][0] + 2.0 * red[1][0] + red[2][0]);
  }
}

// Reconstruction error for any dW (held-out rows, or dW = 0 before the fit), from the statistics:
// eps = <E W, W> + <G dW, dW> - 2 <dW, C W>; float64 reductions.
__global__ __launch_bounds__(256) void fit_error_reduce_kernel(const float* W, const float* dW, const float* EW,
                                                               const float* CW, const float* GW, const float* GdW,
                                                               size_t n, double* eps_abs, double* eps_rel) {
  const int b = blockIdx.x;
  const size_t off = (size_t)b * n;
  double s[5] = {0, 0, 0, 0, 0};
  for (size_t i = threadIdx.x; i < n; i += 256) {
    const double w = W[off + i], cw = CW[off + i];
    s[0] += (double)EW[off + i] * w;
    s[1] += cw * w;
    s[2] += (double)GW[off + i] * w;
    if (dW) {
      const double dw = dW[off + i];
      s[3] += (double)GdW[off + i] * dw;
      s[4] += dw * cw;
    }
  }
  __shared__ double red[5][256];
  for (int k = 0; k < 5; ++k) red[k][threadIdx.x] = s[k];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w)
      for (int k = 0; k < 5; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double e = red[0][0] + red[3][0] - 2.0 * red[4][0];
    eps_abs[b] = e;
    eps_rel[b] = e / (red[0][0] + 2.0 * red[1][0] + red[2][0]);
  }
}

// lambda_b = scale * tr(G_b) / d (trace summed in float64, fixed order).
__global__ __launch_bounds__(256) void trace_lambda_kernel(int d, const float* G, float scale, float* lam) {
  const int b = blockIdx.x;
  const float* g = G + (size_t)b * d * d;
  double t = 0;
  for (int i = threadIdx.x; i < d; i += 256) t += g[(size_t)i * d + i];
  __shared__ double red[256];
  red[threadIdx.x] = t;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) lam[b] = (float)((double)scale * red[0] / d);
}

// Lower 64 x 64 tiles t0 .. t0 + n - 1 of D -= A A^T (A: rows of the tiles, depth K, row stride ld for
// A and D; tiles row-major over the lower triangle), handed to a fused look-ahead launch.
struct DeferredTiles {
  const float* A;
  float* D;
  int ld, K, t0, n;
};

template <bool TA, bool TB>
ispa_status_t gemm(hipStream_t s, int batch, int M, int N, int K, const float* A, int lda, size_t sA, const float* B,
                   int ldb, size_t sB, const float* Cin, int ldc, size_t sC, float* D, int ldd, size_t sD, float alpha,
                   float beta, bool lower_only, const int32_t* info, int kmode = 0, int npairs = 1,
                   size_t pA = 0, size_t pB = 0, size_t pC = 0, size_t pD = 0, float* diag_M = nullptr,
                   float* diag_Linv = nullptr, int32_t* diag_info = nullptr, int diag_d = 0, int diag_k0 = 0,
                   int max_wg = 0, const DeferredTiles* ex = nullptr) {
  if (M <= 0 || N <= 0 || K <= 0) return ISPA_OK;
  if (K % GKS != 0) {
    set_error("internal: GEMM depth not a multiple of 32");
    return ISPA_E_INVALID_ARG;
  }
  GemmParams p;
  p.A = A; p.B = B; p.Cin = Cin; p.D = D;
  p.M = M; p.N = N; p.K = K;
  p.lda = lda; p.ldb = ldb; p.ldc = ldc; p.ldd = ldd;
  p.sA = sA; p.sB = sB; p.sC = sC; p.sD = sD;
  p.alpha = alpha; p.beta = beta;
  p.lower_only = lower_only ? 1 : 0;
  p.kmode = kmode;
  p.info = info;
  p.npairs = npairs;
  p.pA = pA; p.pB = pB; p.pC = pC; p.pD = pD;
  p.diag_M = diag_M; p.diag_Linv = diag_Linv; p.diag_info = diag_info;
  p.diag_d = diag_d; p.diag_k0 = diag_k0;
  p.ex_A = nullptr; p.ex_D = nullptr;
  p.ex_ld = 0; p.ex_K = 0; p.ex_t0 = 0; p.ex_n = 0;
  // large products use 128x128 tiles (half the operand traffic per FLOP) when they still fill the GPU
  const int z = batch * npairs;
  const bool big = M % 128 == 0 && N % 128 == 0 && (size_t)(M / 128) * (N / 128) * z >= 192;
  if constexpr (!TA && TB) {
    if (diag_M) {
      if (npairs != 1) {
        set_error("internal: fused diagonal factorisation with paired products");
        return ISPA_E_INVALID_ARG;
      }
      if (ex != nullptr && ex->n > 0) {
        if (batch != 1 || kmode != 0 || ex->K % GKS != 0 || M % 64 != 0 || N % 64 != 0) {
          set_error("internal: deferred tiles on an unsupported launch");
          return ISPA_E_INVALID_ARG;
        }
        p.ex_A = ex->A; p.ex_D = ex->D;
        p.ex_ld = ex->ld; p.ex_K = ex->K; p.ex_t0 = ex->t0; p.ex_n = ex->n;
        // slots after the primary grid, the multiples of 8 left empty, until n remain
        const int nx = N / 64, prim = (M / 64) * nx;
        int slots = 0;
        for (int got = 0; got < ex->n; ++slots)
          if (!ISPA_DEFER_SKIP_XCD || (prim + slots) % 8 != 0) ++got;
        const int ey = (slots + nx - 1) / nx;
        hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, 64, true>), dim3(nx, M / 64 + ey, 1), dim3(256), 0, s, p);
        return hip_check(hipGetLastError(), "gemm_f32_kernel launch");
      }
      if (big)
        hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, 128, true>), dim3(N / 128, M / 128, z), dim3(256), 0, s, p);
      else
        hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, 64, true>), dim3(N / 64, M / 64, z), dim3(256), 0, s, p);
      return hip_check(hipGetLastError(), "gemm_f32_kernel launch");
    }
  }
  if (big && max_wg > 0 && !lower_only && (M / 128) * (N / 128) > max_wg) {
    hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, 128, false, true>), dim3(max_wg, 1, z), dim3(256), 0, s, p);
    return hip_check(hipGetLastError(), "gemm_f32_kernel launch");
  }
  if (big)
    hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, 128>), dim3(N / 128, M / 128, z), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, 64>), dim3(N / 64, M / 64, z), dim3(256), 0, s, p);
  return hip_check(hipGetLastError(), "gemm_f32_kernel launch");
}

ispa_status_t gemm_d(hipStream_t s, int batch, int M, int N, int K, const float* A, int lda, size_t sA,
                     const float* B, int ldb, size_t sB, const float* Cin, int ldc, size_t sC, const float* X,
                     int ldx, size_t sX, double* D64, float* D32, int ldd, size_t sD, double alpha, double beta,
                     double gamma, const int32_t* info, const float* gamma_b = nullptr) {
  GemmDParams p;
  p.A = A; p.B = B; p.Cin = Cin; p.X = X; p.D64 = D64; p.D32 = D32;
  p.M = M; p.N = N; p.K = K;
  p.lda = lda; p.ldb = ldb; p.ldc = ldc; p.ldx = ldx; p.ldd = ldd;
  p.sA = sA; p.sB = sB; p.sC = sC; p.sX = sX; p.sD = sD;
  p.alpha = alpha; p.beta = beta; p.gamma = gamma;
  p.gamma_b = gamma_b;
  p.info = info;
#ifndef ISPA_F64_V2
#define ISPA_F64_V2 1
#endif
  if (ISPA_F64_V2 && K % DKS == 0) {
    hipLaunchKernelGGL(gemm_f64acc2_kernel, dim3(N / 64, M / 64, batch), dim3(256), 0, s, p);
    return hip_check(hipGetLastError(), "gemm_f64acc2_kernel launch");
  }
  hipLaunchKernelGGL(gemm_f64acc_kernel, dim3(N / 64, M / 64, batch), dim3(256), 0, s, p);
  return hip_check(hipGetLastError(), "gemm_f64acc_kernel launch");
}

#define ISPA_TRY(x)                       \
  do {                                    \
    ispa_status_t st_ = (x);              \
    if (st_ != ISPA_OK) return st_;       \
  } while (0)

}  // namespace

size_t absorb_workspace_size(int32_t d, int32_t d_out, int32_t batch) {
  const size_t b = (size_t)batch;
  return b * d * d * sizeof(float)          // factor L (lower triangle of M)
         + b * d * d * sizeof(float)        // L^-1
         + b * d * d * sizeof(float)        // intermediate products of the inverse
         + 3 * b * d * d_out * sizeof(float)   // R = C W, the residual / correction, an intermediate
         + b * (size_t)d * (d + d_out) * 2       // third bf16 parts of R = C W's split operands
         + residual_i8_scale_bytes(d, d_out, batch) + 256;  // the residual's row and column scales
}

namespace {

constexpr int KM_LOWER_A = 1, KM_UPPER_A = 2, KM_LOWER_B = 3;

// Y_out <- L^-T (L^-1 Y_in) with the explicit inverse; Z is scratch (d x d_out).
ispa_status_t chol_apply(hipStream_t s, int batch, int d, int d_out, const float* Linvf, const float* Yin, float* Z,
                         float* Yout, const int32_t* info) {
  const size_t dd = (size_t)d * d, dn = (size_t)d * d_out;
  ISPA_TRY((gemm<false, false>(s, batch, d, d_out, d, Linvf, d, dd, Yin, d_out, dn, nullptr, 0, 0, Z, d_out, dn, 1.f,
                               0.f, false, info, KM_LOWER_A)));
  ISPA_TRY((gemm<true, false>(s, batch, d, d_out, d, Linvf, d, dd, Z, d_out, dn, nullptr, 0, 0, Yout, d_out, dn, 1.f,
                              0.f, false, info, KM_UPPER_A)));
  return ISPA_OK;
}

}  // namespace

// Fill the blocks of L^-1 below its 64x64 diagonal inverses (already in Linvf) by recursive
// doubling.  Ranges are [start, start+len) in 64-row blocks; each level merges adjacent ranges.
// One level of the explicit inverse's recursive doubling for np adjacent pairs of block ranges (A of
// sa blocks, then C of sc blocks), the first A starting at block a: inv([A 0; B C]) has off-diagonal
// block -C^-1 (B A^-1).  T (one pair's nC x nA after another, layer stride sT) holds B A^-1.
// part: 0 both products, 1 only T = B A^-1, 2 only the second product (T already formed); at most
// max_wg workgroups per layer take the first product's tiles (0: no bound).
ispa_status_t invert_pairs(hipStream_t s, int batch, int d, const float* L, float* Linvf, float* T, size_t sT,
                           const int32_t* info, int a, int sa, int sc, int np, int part = 0, int max_wg = 0) {
  const size_t dd = (size_t)d * d;
  const int nA = sa * NB, nC = sc * NB;
  const size_t a0 = (size_t)a * NB;
  const size_t pstep = (size_t)(nA + nC) * (d + 1);  // from one pair's corner to the next
  // T = B A^-1, with B = L[a0+nA : a0+nA+nC, a0 : a0+nA] and A^-1 lower triangular
  if (part != 2)
    ISPA_TRY((gemm<false, false>(s, batch, nC, nA, nA, L + (a0 + nA) * d + a0, d, dd, Linvf + a0 * d + a0, d, dd,
                                 nullptr, 0, 0, T, nA, sT, 1.f, 0.f, false, info, KM_LOWER_B, np, pstep, pstep, 0,
                                 (size_t)nC * nA, nullptr, nullptr, nullptr, 0, 0, np == 1 ? max_wg : 0)));
  if (part == 1) return ISPA_OK;
  // off-diagonal block of the inverse: -C^-1 T, with C^-1 lower triangular
  return gemm<false, false>(s, batch, nC, nA, nC, Linvf + (a0 + nA) * (d + 1), d, dd, T, nA, sT, nullptr, 0, 0,
                            Linvf + (a0 + nA) * d + a0, d, dd, -1.f, 0.f, false, info, KM_LOWER_A, np, pstep,
                            (size_t)nC * nA, 0, pstep);
}

// The doubling's levels over blocks [b0, b0 + nb): ranges merge pairwise, left to right, an odd last
// range passing a level unchanged; pairs of equal sizes run as one launch.  With emit false nothing
// is launched and the result is the scratch T needs per layer (floats).
size_t invert_range(hipStream_t s, int batch, int d, const float* L, float* Linvf, float* T, size_t sT,
                    const int32_t* info, int b0, int nb, bool emit, ispa_status_t* st) {
  std::vector<std::pair<int, int>> rng;
  for (int k = b0; k < b0 + nb; ++k) rng.push_back({k, 1});
  size_t need = 0;
  while (rng.size() > 1) {
    std::vector<std::pair<int, int>> next;
    size_t i = 0;
    while (i + 1 < rng.size()) {
      const int sa = rng[i].second, sc = rng[i + 1].second;
      int np = 0;
      size_t j = i;
      while (j + 1 < rng.size() && rng[j].second == sa && rng[j + 1].second == sc) {
        ++np;
        j += 2;
      }
      need = std::max(need, (size_t)np * sa * sc * NB * NB);
      if (emit && *st == ISPA_OK) *st = invert_pairs(s, batch, d, L, Linvf, T, sT, info, rng[i].first, sa, sc, np);
      for (int k = 0; k < np; ++k) next.push_back({rng[i + 2 * k].first, sa + sc});
      i = j;
    }
    if (i < rng.size()) next.push_back(rng[i]);
    rng.swap(next);
  }
  return need;
}

// Blocks in the leading range of the doubling's last level (nblk >= 2): the inverse is the leading
// range's levels, the trailing range's, and one last pair.
int inverse_split(int nblk) {
  std::vector<int> sz(nblk, 1);
  while (sz.size() > 2) {
    std::vector<int> next;
    size_t i = 0;
    for (; i + 1 < sz.size(); i += 2) next.push_back(sz[i] + sz[i + 1]);
    if (i < sz.size()) next.push_back(sz[i]);
    sz.swap(next);
  }
  return sz.size() == 2 ? sz[0] : nblk;
}

namespace {
// After R = C W has been forked onto the caller's side stream, every return joins the side stream
// back to the main one, error returns included: the call then leaves nothing unordered against the
// caller's stream and never breaks a graph capture in progress.
struct SideJoin {
  hipStream_t s = nullptr, s2 = nullptr;
  hipEvent_t ev = nullptr;
  bool armed = false;
  ispa_status_t join() {
    if (!armed) return ISPA_OK;
    armed = false;
    ispa_status_t st = hip_check(hipEventRecord(ev, s2), "hipEventRecord (join)");
    const ispa_status_t st2 = hip_check(hipStreamWaitEvent(s, ev, 0), "hipStreamWaitEvent (join)");
    return st != ISPA_OK ? st : st2;
  }
  ~SideJoin() { join(); }
};
}  // namespace

ispa_status_t launch_absorb(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C, const float* W,
                            float lambda, const float* lam_b, float* dW, float* W_new, int32_t* info, void* ws,
                            size_t ws_bytes, hipStream_t s, bool refine, const SideStream* side) {
  const size_t need = absorb_workspace_size(d, d_out, batch);
  if (ws == nullptr || ws_bytes < need) {
    set_error("ispa_absorb_solve: workspace too small");
    return ISPA_E_WORKSPACE;
  }
  const size_t dd = (size_t)d * d, dn = (size_t)d * d_out;
  float* M = (float*)ws;
  float* Linvf = M + (size_t)batch * dd;
  float* Tb = Linvf + (size_t)batch * dd;
  float* Rb = Tb + (size_t)batch * dd;
  float* Rr = Rb + (size_t)batch * dn;
  float* Zb = Rr + (size_t)batch * dn;
  const int nblk = d / NB;

  hipLaunchKernelGGL(init_shift_kernel, dim3((unsigned)((dd / 4 + 255) / 256), batch), dim3(256), 0, s, G, M, Linvf,
                     d, lambda, lam_b, info);
  ISPA_TRY(hip_check(hipGetLastError(), "init_shift_kernel launch"));
  // R = C W (at float32 accuracy; R's rounding perturbs the solution like the float32 statistics
  // themselves do).
  // With a caller-owned side stream it runs there, beside the latency-bound factorisation; for small
  // d it is forked after the first panel steps, since sharing the GPU with it would slow the first
  // diagonal factorisations, which sit on the chain (d = 1536: 1.36 -> 1.33 ms per solve); at
  // d = 5120 it goes first.  Without a side stream it runs on `s` before the factorisation.
  // Where the factorisation's workspace allows (d, d_out multiples of 128), R = C W runs on the bf16
  // matrix cores as six-term products of three-part splits (float32 accuracy; its splits go to the
  // inverse's scratch, R's neighbours and the workspace tail, none of which the factorisation
  // touches); otherwise as a float32 GEMM.
  const bool cw6 = apply3_supported(d, d_out);
  SideJoin joiner;
  // bounded: hold only some workgroups, leaving compute units to the factorisation beside it
  auto cw = [&](hipStream_t cs, bool bounded) -> ispa_status_t {
    if (cw6) {
      __bf16* tail = (__bf16*)(Zb + (size_t)batch * dn);
      void* const cs3[3] = {Tb, (__bf16*)Tb + (size_t)batch * dd, tail};
      void* const ws3[3] = {Rr, (__bf16*)Rr + (size_t)batch * dn, tail + (size_t)batch * dd};
      return launch_prod6(d, d_out, d, batch, C, W, Rb, cs3, ws3, info, cs, bounded ? ISPA_CW6_WORKGROUPS : 0);
    }
    return gemm<false, false>(cs, batch, d, d_out, d, C, d, dd, W, d_out, dn, nullptr, 0, 0, Rb, d_out, dn, 1.f, 0.f,
                              false, nullptr, 0, 1, 0, 0, 0, 0, nullptr, nullptr, nullptr, 0, 0,
                              bounded ? ISPA_CW_WORKGROUPS / batch : 0);
  };
  auto fork_cw = [&]() -> ispa_status_t {
    if (side == nullptr) return cw(s, false);
    ISPA_TRY(hip_check(hipEventRecord(side->ev_fork, s), "hipEventRecord (fork)"));
    ISPA_TRY(hip_check(hipStreamWaitEvent(side->stream, side->ev_fork, 0), "hipStreamWaitEvent (fork)"));
    joiner.s = s;
    joiner.s2 = side->stream;
    joiner.ev = side->ev_join;
    joiner.armed = true;
    return cw(side->stream, d > 2048);
  };
  const int fork_k = (side != nullptr && d <= 2048) ? 4 : -1;  // panel step before which it is forked (-1: first)
  bool forked = false;
  // The explicit L^-1 by recursive doubling over block ranges (for adjacent ranges A, then C,
  // inv([A 0; B C]) has off-diagonal block -C^-1 (B A^-1)) in three parts: the levels inside the
  // leading range of the last level (its P blocks of L are final once the factorisation has factored
  // block P - 1), those inside the trailing range, and the last pair.  With a side stream the first
  // part runs there, after R = C W, beside the factorisation's last steps; the trailing part runs on
  // `s` after the factorisation, in the intermediate buffer Zb (free until the solves) when it is
  // large enough, and the last pair after both.  Without one, the same launches run in order on `s`.
  const int inv_p = inverse_split(nblk), inv_q = nblk - inv_p;
  ispa_status_t inv_st = ISPA_OK;
  auto inv_lead = [&](hipStream_t st) {
    invert_range(st, batch, d, M, Linvf, Tb, dd, info, 0, inv_p, true, &inv_st);
    return inv_st;
  };
  const bool inv_q_in_zb =
      invert_range(s, batch, d, M, Linvf, Zb, dn, info, inv_p, inv_q, false, &inv_st) <= dn;
  bool inv_lead_forked = false, pair_left_forked = false;
  if (fork_k < 0) {
    ISPA_TRY(fork_cw());
    forked = true;
  }
  // Cholesky, right-looking by 64-column panels, with a one-panel look-ahead inside the trailing
  // update: the workgroup that updates the next diagonal block factors it right away, while the
  // other workgroups finish the update, so the factorisation (a latency-bound chain of 64 pivot
  // steps) overlaps the update instead of following it.  (One stream: a wait on an event recorded
  // on another stream costs ~15 us of latency here.)
  hipLaunchKernelGGL(potrf_diag_kernel, dim3(batch), dim3(256), 0, s, M, d, 0, Linvf, info);
  ISPA_TRY(hip_check(hipGetLastError(), "potrf_diag_kernel launch"));
  // Deferred panel updates (one layer, wide trailing matrices): the last step of a CP-column panel
  // updates only the next panel's columns with all CP columns (K = CP) on the chain; the lower
  // tiles right of the next panel go to the fused launches of the next panel's steps, in equal
  // shares, where they fill compute units that otherwise idle while one workgroup factors the next
  // diagonal block.  They touch only columns the next panel's steps neither read nor write, and
  // the next panel's own last step (which updates some of the same entries) follows them in
  // stream order.
  DeferredTiles pend{};
  int pend_left = 0;
  for (int k = 0; k + 1 < nblk; ++k) {
    if (k == fork_k) {
      ISPA_TRY(fork_cw());
      forked = true;
    }
    const int k0 = k * NB;
    const int rest = d - k0 - NB;
    float* panel = M + (size_t)(k0 + NB) * d + k0;
    const float* Lkk_inv = Linvf + (size_t)k0 * d + k0;
    // L_ik = M_ik L_kk^-T (in place)
    ISPA_TRY((gemm<false, true>(s, batch, rest, NB, NB, panel, d, dd, Lkk_inv, d, dd, nullptr, 0, 0, panel, d, dd,
                                1.f, 0.f, false, info)));
    // the leading block columns of L are final: with the leading range of L^-1 on the side stream, the
    // last pair's first product T = B A^-1 follows it there (into Tb; the trailing range is in Zb)
    if (k + 1 == inv_p && inv_lead_forked && inv_q_in_zb) {
      ISPA_TRY(hip_check(hipEventRecord(side->ev_fork, s), "hipEventRecord (fork, last pair)"));
      ISPA_TRY(hip_check(hipStreamWaitEvent(side->stream, side->ev_fork, 0), "hipStreamWaitEvent (fork, last pair)"));
      ISPA_TRY(invert_pairs(side->stream, batch, d, M, Linvf, Tb, dd, info, 0, inv_p, inv_q, 1, 1,
                            ISPA_PAIR_WORKGROUPS));
      pair_left_forked = true;
    }
    // trailing update, lower tiles; tile (0, 0) is diagonal block k + 1, factored in the same launch.
    // Blocks are grouped in panels of CP columns: inside a panel a step updates only the panel's
    // remaining columns (a narrow launch on the chain); the panel's last step updates everything to
    // its right with all CP columns at once (K = CP), so the trailing matrix is read and written once
    // per panel instead of once per block.
    float* trail = M + (size_t)(k0 + NB) * d + k0 + NB;
    const int p0 = k0 / CP * CP, pe = std::min(d, p0 + CP);
    if (k0 + NB < pe) {
      DeferredTiles part{};
      if (pend_left > 0) {  // this step's share of the deferred tiles (the panel's last narrow step takes the rest)
        const int steps = (pe - k0 - NB) / NB;
        part = pend;
        part.t0 = pend.n - pend_left;
        part.n = (pend_left + steps - 1) / steps;
        pend_left -= part.n;
      }
      ISPA_TRY((gemm<false, true>(s, batch, rest, pe - k0 - NB, NB, panel, d, dd, panel, d, dd, trail, d, dd, trail, d,
                                  dd, -1.f, 1.f, true, info, 0, 1, 0, 0, 0, 0, M, Linvf, info, d, k0 + NB, 0, &part)));
    } else {
      if (pend_left != 0) {
        set_error("internal: deferred trailing update not consumed");
        return ISPA_E_INVALID_ARG;
      }
      const float* pan = M + (size_t)pe * d + p0;  // rows pe.., columns p0 .. pe of L
      const int far = d - pe - CP;                 // columns right of the next panel
      if (ISPA_CHOL_DEFER && batch == 1 && far >= ISPA_CHOL_DEFER_MIN) {
        ISPA_TRY((gemm<false, true>(s, batch, rest, CP, pe - p0, pan, d, dd, pan, d, dd, trail, d, dd, trail, d, dd,
                                    -1.f, 1.f, true, info, 0, 1, 0, 0, 0, 0, M, Linvf, info, d, k0 + NB)));
        const int nt = far / 64;
        pend.A = pan + (size_t)CP * d;
        pend.D = M + (size_t)(pe + CP) * d + pe + CP;
        pend.ld = d;
        pend.K = pe - p0;
        pend.t0 = 0;
        pend.n = nt * (nt + 1) / 2;
        pend_left = pend.n;
      } else {
        ISPA_TRY((gemm<false, true>(s, batch, rest, rest, pe - p0, pan, d, dd, pan, d, dd, trail, d, dd, trail, d, dd,
                                    -1.f, 1.f, true, info, 0, 1, 0, 0, 0, 0, M, Linvf, info, d, k0 + NB)));
      }
    }
    // block k + 1 is factored: once it is block inv_p - 1, the leading range of L^-1 can be formed
    // beside the rest of the factorisation (on the side stream, after R = C W, which uses Tb)
    if (k + 2 == inv_p && forked && side != nullptr && inv_q > 0) {
      ISPA_TRY(hip_check(hipEventRecord(side->ev_fork, s), "hipEventRecord (fork, inverse)"));
      ISPA_TRY(hip_check(hipStreamWaitEvent(side->stream, side->ev_fork, 0), "hipStreamWaitEvent (fork, inverse)"));
      ISPA_TRY(inv_lead(side->stream));
      inv_lead_forked = true;
    }
  }
  if (!forked) ISPA_TRY(fork_cw());
  if (inv_q > 0 && inv_q_in_zb)
    ISPA_TRY((invert_range(s, batch, d, M, Linvf, Zb, dn, info, inv_p, inv_q, true, &inv_st), inv_st));
  // join: R = C W (and the leading range of L^-1) are done before Tb is reused and the solve reads R
  ISPA_TRY(joiner.join());
  if (!inv_lead_forked) ISPA_TRY(inv_lead(s));
  if (inv_q > 0 && !inv_q_in_zb)
    ISPA_TRY((invert_range(s, batch, d, M, Linvf, Tb, dd, info, inv_p, inv_q, true, &inv_st), inv_st));
  if (inv_q > 0) ISPA_TRY(invert_pairs(s, batch, d, M, Linvf, Tb, dd, info, 0, inv_p, inv_q, 1, pair_left_forked ? 2 : 0));
  // X = (L L^T)^-1 R.  With the refinement, both solves run on the bf16 matrix cores as three-term
  // products (about 2^-16 relative per product); the accurate residual then corrects
  // the first solve's error and the correction's error is that much smaller again.  L (M) and the
  // doubling scratch (Tb) are free once L^-1 is built and take its splits; Rr (not yet written)
  // takes the split R, Zb the split intermediate.
  const bool use3 = refine && apply3_supported(d, d_out);
  if (use3) {
    ISPA_TRY(launch_split_lower(d, batch, Linvf, Tb, M, info, s));
    ISPA_TRY(launch_chol_apply3(d, d_out, batch, Tb, M, Rb, Rr, Zb, dW, info, s));
  } else {
    ISPA_TRY(chol_apply(s, batch, d, d_out, Linvf, Rb, Zb, dW, info));
  }
  if (!refine) {
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((dn / 4 + 255) / 256), batch), dim3(256), 0, s, W, dW,
                       (const float*)nullptr, W_new, dn, (const int32_t*)info);
    return hip_check(hipGetLastError(), "finalize_kernel launch");
  }
  // refinement: r = R - G X - lambda X far more accurate than float32 (the cancellation needs it),
  // correction = (L L^T)^-1 r.  Where supported G X is an exact product of int8 digit slices on the
  // int8 matrix cores (its planes in the free L^-1, intermediate and tail buffers), else it is
  // accumulated in float64 on the float64 matrix cores.
  if (use3 && ISPA_RESID_I8 && residual_i8_supported(d, d_out)) {
    int8_t* g8 = (int8_t*)Linvf;                    // 4 planes of batch * d * d bytes
    int8_t* x8 = (int8_t*)Zb;                       // 4 planes of batch * d * d_out bytes
    int8_t* t8 = (int8_t*)(Zb + (size_t)batch * dn);  // tail: 2 more of each
    const size_t bdd = (size_t)batch * dd, bdn = (size_t)batch * dn;
    void* const gp[6] = {g8, g8 + bdd, g8 + 2 * bdd, g8 + 3 * bdd, t8, t8 + bdd};
    void* const xp[6] = {x8, x8 + bdn, x8 + 2 * bdn, x8 + 3 * bdn, t8 + 2 * bdd, t8 + 2 * bdd + bdn};
    void* scales = (void*)((((uintptr_t)(t8 + 2 * bdd + 2 * bdn)) + 255) & ~(uintptr_t)255);
    ISPA_TRY(launch_residual_i8(d, d_out, batch, G, dW, Rb, lam_b ? -1.0 : -(double)lambda, lam_b, Rr, gp, xp,
                                scales, info, s));
  } else {
    ISPA_TRY(gemm_d(s, batch, d, d_out, d, G, d, dd, dW, d_out, dn, Rb, d_out, dn, dW, d_out, dn, nullptr, Rr, d_out,
                    dn, -1.0, 1.0, lam_b ? -1.0 : -(double)lambda, info, lam_b));
  }
  if (use3)  // R is no longer needed: its buffer takes the split residual
    ISPA_TRY(launch_chol_apply3(d, d_out, batch, Tb, M, Rr, Rb, Zb, Rr, info, s));
  else
    ISPA_TRY(chol_apply(s, batch, d, d_out, Linvf, Rr, Zb, Rr, info));
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((dn / 4 + 255) / 256), batch), dim3(256), 0, s, W, dW,
                     (const float*)Rr, W_new, dn, (const int32_t*)info);
  return hip_check(hipGetLastError(), "finalize_kernel launch");
}

size_t fit_error_workspace_size(int32_t d, int32_t d_out, int32_t batch) {
  return 4 * (size_t)batch * d * d_out * sizeof(float);
}

ispa_status_t launch_fit_error(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                               const float* E, const float* W, const float* dW, double* eps_abs, double* eps_rel,
                               void* ws, size_t ws_bytes, hipStream_t s) {
  if (ws == nullptr || ws_bytes < fit_error_workspace_size(d, d_out, batch)) {
    set_error("ispa_fit_error: workspace too small");
    return ISPA_E_WORKSPACE;
  }
  const size_t dd = (size_t)d * d, dn = (size_t)d * d_out;
  float* EW = (float*)ws;
  float* CW = EW + (size_t)batch * dn;
  float* GW = CW + (size_t)batch * dn;
  float* GdW = GW + (size_t)batch * dn;
  ISPA_TRY((gemm<false, false>(s, batch, d, d_out, d, E, d, dd, W, d_out, dn, nullptr, 0, 0, EW, d_out, dn, 1.f, 0.f,
                               false, nullptr)));
  ISPA_TRY((gemm<false, false>(s, batch, d, d_out, d, C, d, dd, W, d_out, dn, nullptr, 0, 0, CW, d_out, dn, 1.f, 0.f,
                               false, nullptr)));
  ISPA_TRY((gemm<false, false>(s, batch, d, d_out, d, G, d, dd, W, d_out, dn, nullptr, 0, 0, GW, d_out, dn, 1.f, 0.f,
                               false, nullptr)));
  if (dW)
    ISPA_TRY((gemm<false, false>(s, batch, d, d_out, d, G, d, dd, dW, d_out, dn, nullptr, 0, 0, GdW, d_out, dn, 1.f,
                                 0.f, false, nullptr)));
  hipLaunchKernelGGL(fit_error_reduce_kernel, dim3(batch), dim3(256), 0, s, W, dW, EW, CW, GW, GdW, dn, eps_abs,
                     eps_rel);
  return hip_check(hipGetLastError(), "fit_error_reduce_kernel launch");
}

ispa_status_t launch_trace_lambda(int32_t d, int32_t batch, const float* G, float scale, float* lam, hipStream_t s) {
  hipLaunchKernelGGL(trace_lambda_kernel, dim3(batch), dim3(256), 0, s, d, G, scale, lam);
  return hip_check(hipGetLastError(), "trace_lambda_kernel launch");
}

size_t eps_workspace_size(int32_t d, int32_t d_out, int32_t batch) {
  return 3 * (size_t)batch * d * d_out * sizeof(float);
}

ispa_status_t launch_eps(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C, const float* E,
                         const float* W, const float* dW, float lambda, double* eps_abs, double* eps_rel, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  if (ws == nullptr || ws_bytes < eps_workspace_size(d, d_out, batch)) {
    set_error("ispa_layer_eps: workspace too small");
    return ISPA_E_WORKSPACE;
  }
  const size_t dd = (size_t)d * d, dn = (size_t)d * d_out;
  float* EW = (float*)ws;
  float* CW = EW + (size_t)batch * dn;
  float* GW = CW + (size_t)batch * dn;
  ISPA_TRY((gemm<false, false>(s, batch, d, d_out, d, E, d, dd, W, d_out, dn, nullptr, 0, 0, EW, d_out, dn, 1.f, 0.f,
                               false, nullptr)));
  ISPA_TRY((gemm<false, false>(s, batch, d, d_out, d, C, d, dd, W, d_out, dn, nullptr, 0, 0, CW, d_out, dn, 1.f, 0.f,
                               false, nullptr)));
  ISPA_TRY((gemm<false, false>(s, batch, d, d_out, d, G, d, dd, W, d_out, dn, nullptr, 0, 0, GW, d_out, dn, 1.f, 0.f,
                               false, nullptr)));
  hipLaunchKernelGGL(eps_reduce_kernel, dim3(batch), dim3(256), 0, s, W, dW, EW, CW, GW, dn, lambda, eps_abs, eps_rel);
  return hip_check(hipGetLastError(), "eps_reduce_kernel launch");
}

}  // namespace ispa
