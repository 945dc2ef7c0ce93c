// The refinement residual of the absorb solve on the int8 matrix cores (gfx950).
//
// The closed-form layer absorb (ISPA technical summary, section 2, "Layer Absorb") solves
// (G + lambda I) dW = C W; its one refinement step needs r = R - (G + lambda I) X for the float32
// solution X.  r is small next to R, so G X must be formed far more accurately than a float32
// product gives: about 2^-34 relative to |G| |X| at the conditioning warmup statistics have (the
// float32 rounding of G X, amplified by that conditioning, is the error the step removes).
//
// G X is formed as an exact integer product of digit slices (the splitting scheme of Ozaki et al.
// for accurate matrix products, here on int8 digits with int32 accumulation):
//  * every row i of G gets a power-of-two scale 2^e_i with |G_ik| < 2^e_i, every column j of X a
//    scale 2^f_j; the scaled values lie in (-1, 1) and are cut into S = 5 signed 7-bit digits
//    (v -> 128 v, digit = its integer part, v -> the remainder; all exact in float32), so
//    G_ik = 2^e_i (sum_s a_s,ik 2^(-7(s+1)) + rest) with |rest| < 2^-35;
//  * G X = 2^(e_i + f_j) sum_{s,t} 2^(-7(s+t+2)) (A_s B_t)_ij; the int8 products A_s B_t are exact
//    in int32 (|digit| <= 127, at most five products of d terms share one accumulator), and the pairs
//    with s + t <= S - 1 are kept (15 products; each term then within ~2^-35 of the scales' product);
//  * the S diagonal sums s + t = c are combined in float64, scaled, and r = R - G X - lambda X is
//    formed in float64 and rounded once to float32.
// 15 int8 products at 5 POP/s against one float64 product at 78.6 TFLOP/s.  Five digits take the
// refined dW to within 2e-7 to 1e-6 of the float64 solve at cond ~4e4 to 2e5 (six: 4e-8 to 7e-7,
// 0.42 ms more at d = 5120), far below the float32 statistics' own rounding.
#include "ispa_internal.h"

namespace ispa {
namespace {

#ifndef ISPA_OZ_DIGITS
#define ISPA_OZ_DIGITS 5
#endif
constexpr int OZ_S = ISPA_OZ_DIGITS;  // 7-bit digits per value
constexpr int OZ_T = 128;   // output tile: 8 waves of 32 x 64 (two per SIMD)
constexpr int OZ_K = 32;    // K per stage: one v_mfma_i32_32x32x32_i8 step
constexpr int OZ_NSTG = 3;  // stages in the LDS ring (40 KB each)
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v16i_t __attribute__((ext_vector_type(16)));

// e with max|x| < 2^e over the reduced values (0 when all are zero)
__device__ __forceinline__ int scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  frexpf(amax, &e);
  return e;
}

// the S digits of v in (-1, 1), as bytes: digits 0-3 in lo, the rest in hi
__device__ __forceinline__ void digits(float v, uint32_t& lo, uint32_t& hi) {
  lo = hi = 0;
#pragma unroll
  for (int s = 0; s < OZ_S; ++s) {
    v *= 128.f;
    const float a = truncf(v);
    v -= a;
    const uint32_t byte = (uint32_t)(int)a & 0xFFu;
    if (s < 4) lo |= byte << (8 * s);
    else hi |= byte << (8 * (s - 4));
  }
}

// eG[b][i] for every row of G[b] (one workgroup per row); also clears X's column maxima
__global__ __launch_bounds__(256) void oz_rowexp_kernel(const float* __restrict__ G, int d, int n, int* eG,
                                                        uint32_t* xmax, const int32_t* __restrict__ info) {
  const int i = blockIdx.x, b = blockIdx.y;
  for (int c = i * 256 + (int)threadIdx.x; c < n && i * 256 < n; c += 256 * d) xmax[(size_t)b * n + c] = 0u;
  if (info[b] != 0) return;
  const float* row = G + (size_t)b * d * d + (size_t)i * d;
  float m = 0.f;
  for (int k = threadIdx.x * 4; k < d; k += 1024) {
    const f32x4 v = *(const f32x4*)(row + k);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
  __shared__ float red[256];
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) eG[(size_t)b * d + i] = scale_exp(red[0]);
}

// xmax[b][j] = bits of max_k |X[b][k][j]| (non-negative floats order as their bits), per 64 columns
// x 128 rows per workgroup with an integer atomic maximum (the order of the atomics cannot change it)
__global__ __launch_bounds__(256) void oz_colmax_kernel(const float* __restrict__ X, int d, int n, uint32_t* xmax,
                                                        const int32_t* __restrict__ info) {
  const int b = blockIdx.z;
  if (info[b] != 0) return;
  const int c = blockIdx.x * 64 + (threadIdx.x & 63), g = threadIdx.x >> 6;
  const float* x = X + (size_t)b * d * n + (size_t)blockIdx.y * 128 * n + c;
  float m = 0.f;
#pragma unroll 4
  for (int r = g; r < 128; r += 4) m = fmaxf(m, fabsf(x[(size_t)r * n]));
  __shared__ float red[4][64];
  red[g][threadIdx.x & 63] = m;
  __syncthreads();
  if (g == 0) {
    const float mm = fmaxf(fmaxf(red[0][threadIdx.x], red[1][threadIdx.x]), fmaxf(red[2][threadIdx.x], red[3][threadIdx.x]));
    atomicMax(xmax + (size_t)b * n + c, __float_as_uint(mm));
  }
}

// GS[s][b][i][k] = digit s of G[b][i][k] 2^-eG[b][i]; 8 elements per thread
struct Planes {
  int8_t* p[OZ_S];  // digit planes, each batch x rows x K bytes
};
__global__ __launch_bounds__(256) void oz_slice_rows_kernel(const float* __restrict__ G, const int* __restrict__ eG,
                                                            int d, Planes GS, const int32_t* __restrict__ info) {
  const int b = blockIdx.y;
  if (info[b] != 0) return;
  const size_t dd = (size_t)d * d;
  const size_t e8 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e8 >= dd) return;
  const int ex = eG[(size_t)b * d + (int)(e8 / d)];
  const f32x4 v0 = *(const f32x4*)(G + b * dd + e8);
  const f32x4 v1 = *(const f32x4*)(G + b * dd + e8 + 4);
  uint32_t lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    digits(ldexpf(v0[e], -ex), lo[e], hi[e]);
    digits(ldexpf(v1[e], -ex), lo[4 + e], hi[4 + e]);
  }
#pragma unroll
  for (int s = 0; s < OZ_S; ++s) {
    const int sh = 8 * (s & 3);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w0 |= (((s < 4 ? lo[e] : hi[e]) >> sh) & 0xFFu) << (8 * e);
      w1 |= (((s < 4 ? lo[4 + e] : hi[4 + e]) >> sh) & 0xFFu) << (8 * e);
    }
    *(u32x2*)(GS.p[s] + b * dd + e8) = u32x2{w0, w1};
  }
}

// XS[s][b][j][k] = digit s of X[b][k][j] 2^-f_j (transposed: k contiguous), f_j from the column
// maximum; 64 x 64 blocks through LDS
__global__ __launch_bounds__(256) void oz_slice_cols_kernel(const float* __restrict__ X,
                                                            const uint32_t* __restrict__ xmax, int d, int n,
                                                            Planes XS, const int32_t* __restrict__ info) {
  const int bk = blockIdx.y, bj = blockIdx.x, b = blockIdx.z;
  if (info[b] != 0) return;
  __shared__ float T[64][65];
  const size_t dn = (size_t)d * n;
  const float* src = X + b * dn + (size_t)bk * 64 * n + bj * 64;
  const int tid = threadIdx.x, r0 = tid / 16, c4 = 4 * (tid % 16);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + 16 * q;
    const f32x4 v = *(const f32x4*)(src + (size_t)r * n + c4);
#pragma unroll
    for (int e = 0; e < 4; ++e) T[r][c4 + e] = v[e];
  }
  __syncthreads();
  // thread: output row j = tid / 4 (a column of X), k = 16 (tid % 4) .. + 15 of this block
  const int j = tid >> 2, k0 = 16 * (tid & 3);
  const int ex = scale_exp(__uint_as_float(xmax[(size_t)b * n + bj * 64 + j]));
  uint32_t w[OZ_S][4];
#pragma unroll
  for (int s = 0; s < OZ_S; ++s)
#pragma unroll
    for (int q = 0; q < 4; ++q) w[s][q] = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    uint32_t lo, hi;
    digits(ldexpf(T[k0 + e][j], -ex), lo, hi);
#pragma unroll
    for (int s = 0; s < OZ_S; ++s) w[s][e >> 2] |= (((s < 4 ? lo : hi) >> (8 * (s & 3))) & 0xFFu) << (8 * (e & 3));
  }
  const size_t o = b * dn + ((size_t)(bj * 64 + j)) * d + bk * 64 + k0;
#pragma unroll
  for (int s = 0; s < OZ_S; ++s) *(u32x4*)(XS.p[s] + o) = u32x4{w[s][0], w[s][1], w[s][2], w[s][3]};
}

struct OzParams {
  Planes GS;                // [s][batch][d][d]
  Planes XS;                // [s][batch][n][d]
  const int* eG;            // [batch][d]
  const uint32_t* xmax;     // [batch][n]
  const float* R;           // [batch][d][n]
  const float* X;           // [batch][d][n]
  float* r;                 // [batch][d][n]
  double gamma;             // r = R - G X + gamma X (gamma * gamma_b[b] per layer if gamma_b)
  const float* gamma_b;
  const int32_t* info;
  int d, n;
};

// Slot of 16-byte chunk c (0 or 1) of staged row `row` (32-byte rows): the 16 rows of a fragment read
// pass then cover all 64 banks.
__device__ __forceinline__ int oz_slot(int row, int c) { return c ^ ((row >> 3) & 1); }

// r = R - (G X) + gamma X for one 128 x 128 output tile (rows of G: m0.., columns of X: n0..).
// Per 32-deep K stage the S digit slices of both operands (2 S x 128 rows x 32 bytes) go into
// a ring of LDS buffers by buffer loads into LDS; each of the 8 waves owns 32 x 64 outputs with S
// int32 accumulator sets (one per diagonal s + t), two waves per SIMD.
__global__ __launch_bounds__(512) void oz_gemm_kernel(OzParams p) {
  const int b = blockIdx.z;
  if (p.info[b] != 0) return;
  const int m0 = blockIdx.y * OZ_T, n0 = blockIdx.x * OZ_T;
  constexpr int OPB = OZ_T * OZ_K;    // bytes of one slice tile per stage
  constexpr int SB = 2 * OZ_S * OPB;  // bytes per stage
  constexpr int WLW = SB / 1024 / 8;  // wave loads (1 KB) per wave per stage
  static_assert(WLW * 8 * 1024 == SB, "stage loads must split over the waves");
  __shared__ __attribute__((aligned(1024))) int8_t B0[SB];
  __shared__ __attribute__((aligned(1024))) int8_t B1[SB];
  __shared__ __attribute__((aligned(1024))) int8_t B2[SB];
  int8_t* const buf[OZ_NSTG] = {B0, B1, B2};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 64;  // 32 rows x 64 columns per wave
  const uint32_t d = (uint32_t)p.d, n = (uint32_t)p.n;
  const size_t dd = (size_t)d * d, dn = (size_t)d * n;
  // wave load g = wave + 8 j: operand slice o = g / 4 (0..S-1: digits of G, S..2S-1: of X), rows
  // 32 (g % 4) .. + 31 of the tile; lane: row 32 (g % 4) + lane / 2, slot lane % 2
  rsrc_t rs[WLW];
  uint32_t gofs[WLW];
  int ldst[WLW];
#pragma unroll
  for (int j = 0; j < WLW; ++j) {
    const int g = wave + 8 * j;
    const int o = g >> 2, q = g & 3;
    const bool isa = o < OZ_S;
    const int s = isa ? o : o - OZ_S;
    const int8_t* plane = isa ? p.GS.p[s] + b * dd + (size_t)m0 * d : p.XS.p[s] + b * dn + (size_t)n0 * d;
    rs[j] = make_rsrc(plane, (uint32_t)OZ_T * d);
    const int row = 32 * q + (lane >> 1);
    gofs[j] = (uint32_t)row * d + 16u * (uint32_t)oz_slot(row, lane & 1);
    ldst[j] = o * OPB + q * 1024;
  }
  auto load_stage = [&](int st, int8_t* bb) {
    const uint32_t kofs = (uint32_t)(st * OZ_K);
#pragma unroll
    for (int j = 0; j < WLW; ++j) load_to_lds(rs[j], (uint16_t*)(bb + ldst[j]), gofs[j] + kofs);
  };
  auto frag = [&](const int8_t* bb, int o, int r0) {
    const int row = r0 + l32;
    return *(const v4i_t*)(bb + o * OPB + row * OZ_K + 16 * oz_slot(row, hh));
  };
  v16i_t acc[OZ_S][2];
#pragma unroll
  for (int c = 0; c < OZ_S; ++c)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[c][i] = v16i_t{0};
  // the row block's digit fragments are read once and kept; each column block's are streamed (15
  // fragment reads per stage and wave)
  auto compute = [&](const int8_t* bb) {
    v4i_t a[OZ_S];
#pragma unroll
    for (int s = 0; s < OZ_S; ++s) a[s] = frag(bb, s, wi);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < OZ_S; ++t) {
        const v4i_t x = frag(bb, OZ_S + t, wj + 32 * i);
#pragma unroll
        for (int s = 0; s + t < OZ_S; ++s)
          acc[s + t][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[s], x, acc[s + t][i], 0, 0, 0);
      }
  };
  // Ring of three stages, stage st in buffer st % 3: step st loads stage st + 2 and multiplies
  // stage st, two stages in flight.  At the top of step st each wave waits for its own loads of
  // stage st (all but stage st + 1's: vmcnt counts this wave's loads, which complete in order); the
  // barrier then makes every wave's loads visible and frees the buffer stage st - 1 was read from.
  // A plain barrier, not __syncthreads(), whose fence would wait for stage st + 1's loads as well.
  // Every step issues its loads, also the (at most four) past the last stage: they read bytes of
  // the tile's own rows (or zeros past its end) into buffers that are not multiplied, and the wait
  // after the loop drains them.
  static_assert(OZ_NSTG == 3, "three-stage ring");
  constexpr int WAIT_CUR = 0xF70 | (WLW & 15) | ((WLW >> 4) << 14);  // vmcnt(WLW)
  const int nst = p.d / OZ_K;
  const int nstR = (nst + 2) / 3 * 3;
#pragma unroll
  for (int k = 0; k < 2; ++k) load_stage(k, buf[k]);
  for (int st = 0; st < nstR; st += 3) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_CUR);
      __builtin_amdgcn_s_barrier();
      load_stage(st + u + 2, buf[(u + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
      if (st + u < nst) compute(buf[u]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  // acc[c][i][v]: row m0 + wi + 8 (v / 4) + 4 hh + v % 4, column n0 + wj + 32 i + l32
  const double gb = p.gamma_b ? p.gamma * (double)p.gamma_b[b] : p.gamma;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = n0 + wj + 32 * i + l32;
    const int fj = scale_exp(__uint_as_float(p.xmax[(size_t)b * n + j]));
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = m0 + wi + 8 * (v >> 2) + 4 * hh + (v & 3);
      double sum = 0.0;
#pragma unroll
      for (int c = OZ_S - 1; c >= 0; --c) sum += ldexp((double)acc[c][i][v], -7 * (c + 2));
      const double gx = ldexp(sum, p.eG[(size_t)b * d + r] + fj);
      const size_t o = (size_t)b * dn + (size_t)r * n + j;
      double x = -gx;
      x += (double)p.R[o];
      x += gb * (double)p.X[o];
      p.r[o] = (float)x;
    }
  }
}

}  // namespace

bool residual_i8_supported(int32_t d, int32_t d_out) {
  // int32 accumulators: at most S products of d digit pairs (|digit| <= 127) share one
  return d % OZ_T == 0 && d_out % OZ_T == 0 && (int64_t)d * OZ_S * 127 * 127 < ((int64_t)1 << 31);
}

size_t residual_i8_scale_bytes(int32_t d, int32_t d_out, int32_t batch) {
  return (size_t)batch * 4 * ((size_t)d + d_out);
}

ispa_status_t launch_residual_i8(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* X,
                                 const float* R, double gamma, const float* gamma_b, float* r,
                                 void* const gplanes[6], void* const xplanes[6], void* scales, const int32_t* info,
                                 hipStream_t s) {
  if (!residual_i8_supported(d, d_out)) {
    set_error("internal: int8 residual needs d, d_out multiples of 128 and d * 5 * 127^2 below 2^31");
    return ISPA_E_INVALID_ARG;
  }
  Planes GS, XS;
  for (int k = 0; k < OZ_S; ++k) {
    GS.p[k] = (int8_t*)gplanes[k];
    XS.p[k] = (int8_t*)xplanes[k];
  }
  int* eG = (int*)scales;
  uint32_t* xmax = (uint32_t*)(eG + (size_t)batch * d);
  hipLaunchKernelGGL(oz_rowexp_kernel, dim3(d, batch), dim3(256), 0, s, G, d, d_out, eG, xmax, info);
  ispa_status_t st = hip_check(hipGetLastError(), "oz_rowexp_kernel launch");
  if (st != ISPA_OK) return st;
  hipLaunchKernelGGL(oz_colmax_kernel, dim3(d_out / 64, d / 128, batch), dim3(256), 0, s, X, d, d_out, xmax, info);
  st = hip_check(hipGetLastError(), "oz_colmax_kernel launch");
  if (st != ISPA_OK) return st;
  const size_t dd8 = (size_t)d * d / 8;
  hipLaunchKernelGGL(oz_slice_rows_kernel, dim3((unsigned)((dd8 + 255) / 256), batch), dim3(256), 0, s, G, eG, d,
                     GS, info);
  st = hip_check(hipGetLastError(), "oz_slice_rows_kernel launch");
  if (st != ISPA_OK) return st;
  hipLaunchKernelGGL(oz_slice_cols_kernel, dim3(d_out / 64, d / 64, batch), dim3(256), 0, s, X, xmax, d, d_out, XS,
                     info);
  st = hip_check(hipGetLastError(), "oz_slice_cols_kernel launch");
  if (st != ISPA_OK) return st;
  OzParams p{GS, XS, eG, xmax, R, X, r, gamma, gamma_b, info, d, d_out};
  hipLaunchKernelGGL(oz_gemm_kernel, dim3(d_out / OZ_T, d / OZ_T, batch), dim3(512), 0, s, p);
  return hip_check(hipGetLastError(), "oz_gemm_kernel launch");
}

}  // namespace ispa
