// Gram accumulation for the closed-form absorb on gfx950.
//
// Source: "Technical Summary: Instance-Specific Parametric Absorption (ISPA)
// for Memory-Efficient Video Generation", section 2 "Methodology", step 2
// "Layer Absorb": dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W
// needs only G = A_loc^T A_loc and C = A_loc^T (A_full - A_loc) summed over
// the warmup rows.  C is formed as A_loc^T A_full - A_loc^T A_loc from the
// exact stored operands (same value; no rounding of A_full - A_loc).
//
// bf16 design: a workgroup owns a 128x128 output tile (I, J) and a range of
// rows.  Per 32-row stage it stages A_loc[:, I], A_loc[:, J], A_full[:, J]
// (and A_full[:, I] when Q_ff is wanted) in LDS transposed (column-major, the
// row index contiguous), so every MFMA operand is one 16-byte LDS read; the
// A_loc[:, I] operand feeds both products.  4 waves in a 2x2 grid each own a
// 64x64 sub-tile (2x2 blocks of v_mfma_f32_32x32x16_bf16).  Rows are split
// over workgroups when there are too few tiles to fill the GPU; the split
// partials go to a workspace and a second kernel sums them in a fixed order
// (deterministic, no atomics).
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int GT = 128;      // output tile edge
constexpr int GBK = 32;      // rows per stage
constexpr int GTS = GBK + 8; // transposed-tile row stride (elements)

struct GramParams {
  const uint16_t* Al;
  const uint16_t* Af;
  float* G;  // direct outputs (splits == 1) or partial slabs (splits > 1)
  float* C;
  float* Q;
  int64_t n_rows;
  int d;
  int tiles_per_dim;
  int64_t rows_per_split;
  int accumulate;
  int direct;
  size_t slab;  // elements per partial matrix (d*d) when !direct
};

template <bool QFF>
__global__ __launch_bounds__(256, 2) void gram_bf16_kernel(GramParams p) {
  constexpr int NM = QFF ? 4 : 3;  // staged matrices: locI, locJ, fullJ, [fullI]
  __shared__ __attribute__((aligned(16))) uint16_t sT[2][NM][GT * GTS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int ti = tile / p.tiles_per_dim, tj = tile % p.tiles_per_dim;
  const int I0 = ti * GT, J0 = tj * GT;
  const int64_t r_begin = (int64_t)split * p.rows_per_split;
  const int64_t r_end = min(p.n_rows, r_begin + p.rows_per_split);
  const int nst = r_end > r_begin ? (int)((r_end - r_begin + GBK - 1) / GBK) : 0;
  const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;  // wave sub-tile origin

  // staging: item = 8 rows x 4 columns of one matrix; 128 items per matrix
  constexpr int ITEMS = NM * (GBK / 8) * (GT / 4);
  constexpr int PER = (ITEMS + 255) / 256;
  u32x2 reg[PER][8];

  auto load = [&](int st) {
    const int64_t r0 = r_begin + (int64_t)st * GBK;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = tid + i * 256;
      if (it >= ITEMS) break;
      const int mtx = it / 128, w = it % 128;
      const int rg = w % (GBK / 8), cq = w / (GBK / 8);
      const uint16_t* src = (mtx == 1 || mtx == 0) ? p.Al : p.Af;
      const int col0 = (mtx == 0 || mtx == 3) ? I0 : J0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t r = r0 + rg * 8 + e;
        reg[i][e] = r < r_end ? *(const u32x2*)(src + r * p.d + col0 + cq * 4) : u32x2{0, 0};
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = tid + i * 256;
      if (it >= ITEMS) break;
      const int mtx = it / 128, w = it % 128;
      const int rg = w % (GBK / 8), cq = w / (GBK / 8);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        uint32_t o[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const uint32_t a = cc < 2 ? reg[i][2 * x].x : reg[i][2 * x].y;
          const uint32_t b = cc < 2 ? reg[i][2 * x + 1].x : reg[i][2 * x + 1].y;
          o[x] = (cc & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
        }
        *(u32x4*)(&sT[buf][mtx][(cq * 4 + cc) * GTS + rg * 8]) = u32x4{o[0], o[1], o[2], o[3]};
      }
    }
  };

  f32x16 accG[2][2], accX[2][2], accQ[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      accG[a][b] = f32x16{0};
      accX[a][b] = f32x16{0};
      accQ[a][b] = f32x16{0};
    }

  if (nst > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load(st + 1);
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 aI[2], bJ[2], fJ[2], fI[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        aI[b] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&sT[buf][0][(wi + 32 * b + l32) * GTS + 16 * ks + 8 * hh]));
        bJ[b] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&sT[buf][1][(wj + 32 * b + l32) * GTS + 16 * ks + 8 * hh]));
        fJ[b] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&sT[buf][2][(wj + 32 * b + l32) * GTS + 16 * ks + 8 * hh]));
        if (QFF)
          fI[b] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&sT[buf][NM - 1][(wi + 32 * b + l32) * GTS + 16 * ks + 8 * hh]));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          accG[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aI[a], bJ[b], accG[a][b], 0, 0, 0);
          accX[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aI[a], fJ[b], accX[a][b], 0, 0, 0);
          if (QFF) accQ[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fI[a], fJ[b], accQ[a][b], 0, 0, 0);
        }
    }
    if (st + 1 < nst) store((st + 1) & 1);
    __syncthreads();
  }

  // epilogue: accumulator element v of lane (col, hh) is row 8(v/4) + 4hh + v%4.
  const size_t d = p.d;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = I0 + wi + 32 * a + 8 * (v >> 2) + 4 * hh + (v & 3);
        const int j = J0 + wj + 32 * b + l32;
        const size_t o = (size_t)i * d + j;
        const float g = accG[a][b][v];
        const float x = accX[a][b][v];
        if (p.direct) {
          if (p.accumulate) {
            p.G[o] += g;
            p.C[o] += x - g;
            if (QFF) p.Q[o] += accQ[a][b][v];
          } else {
            p.G[o] = g;
            p.C[o] = x - g;
            if (QFF) p.Q[o] = accQ[a][b][v];
          }
        } else {
          const size_t base = (size_t)split * (QFF ? 3 : 2) * p.slab;
          p.G[base + o] = g;
          p.G[base + p.slab + o] = x;
          if (QFF) p.G[base + 2 * p.slab + o] = accQ[a][b][v];
        }
      }
}

// Sum split partials in split order into G, C (and Q_ff).
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ part, int splits, int nmat,
                                                          size_t slab, float* G, float* C, float* Q,
                                                          int accumulate) {
  const size_t i4 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= slab) return;
  f32x4 g = {0, 0, 0, 0}, x = {0, 0, 0, 0}, q = {0, 0, 0, 0};
  for (int s = 0; s < splits; ++s) {
    const float* b = part + (size_t)s * nmat * slab;
    g += *(const f32x4*)(b + i4);
    x += *(const f32x4*)(b + slab + i4);
    if (nmat == 3) q += *(const f32x4*)(b + 2 * slab + i4);
  }
  f32x4 c = x - g;
  if (accumulate) {
    g += *(const f32x4*)(G + i4);
    c += *(const f32x4*)(C + i4);
    if (nmat == 3) q += *(const f32x4*)(Q + i4);
  }
  *(f32x4*)(G + i4) = g;
  *(f32x4*)(C + i4) = c;
  if (nmat == 3) *(f32x4*)(Q + i4) = q;
}

// float32 path: 64x64 tile per workgroup, each thread a 4x4 block; rows staged in LDS.
constexpr int FT = 64;
constexpr int FBK = 32;

__global__ __launch_bounds__(256) void gram_f32_kernel(const float* __restrict__ Al, const float* __restrict__ Af,
                                                       float* G, float* C, float* Q, int64_t n_rows, int d,
                                                       int accumulate) {
  __shared__ float sLI[FBK][FT], sLJ[FBK][FT], sFJ[FBK][FT], sFI[FBK][FT];
  const int tpd = d / FT;
  const int ti = blockIdx.x / tpd, tj = blockIdx.x % tpd;
  const int I0 = ti * FT, J0 = tj * FT;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;  // thread block: rows I0+4ty.., cols J0+4tx..
  float g[4][4] = {}, x[4][4] = {}, q[4][4] = {};
  const bool qff = Q != nullptr;
  for (int64_t r0 = 0; r0 < n_rows; r0 += FBK) {
    __syncthreads();
    for (int e = tid; e < FBK * FT; e += 256) {
      const int rr = e / FT, cc = e % FT;
      const int64_t r = r0 + rr;
      const bool ok = r < n_rows;
      sLI[rr][cc] = ok ? Al[r * d + I0 + cc] : 0.f;
      sLJ[rr][cc] = ok ? Al[r * d + J0 + cc] : 0.f;
      sFJ[rr][cc] = ok ? Af[r * d + J0 + cc] : 0.f;
      sFI[rr][cc] = (ok && qff) ? Af[r * d + I0 + cc] : 0.f;
    }
    __syncthreads();
    for (int rr = 0; rr < FBK; ++rr) {
      float li[4], lj[4], fj[4], fi[4];
      for (int u = 0; u < 4; ++u) {
        li[u] = sLI[rr][4 * ty + u];
        fi[u] = sFI[rr][4 * ty + u];
        lj[u] = sLJ[rr][4 * tx + u];
        fj[u] = sFJ[rr][4 * tx + u];
      }
      for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b) {
          g[a][b] = fmaf(li[a], lj[b], g[a][b]);
          x[a][b] = fmaf(li[a], fj[b], x[a][b]);
          q[a][b] = fmaf(fi[a], fj[b], q[a][b]);
        }
    }
  }
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b) {
      const size_t o = (size_t)(I0 + 4 * ty + a) * d + J0 + 4 * tx + b;
      const float cv = x[a][b] - g[a][b];
      if (accumulate) {
        G[o] += g[a][b];
        C[o] += cv;
        if (qff) Q[o] += q[a][b];
      } else {
        G[o] = g[a][b];
        C[o] = cv;
        if (qff) Q[o] = q[a][b];
      }
    }
}

int gram_splits(int64_t n_rows, int d) {
  const int tiles = (d / GT) * (d / GT);
  // aim for about two resident workgroups per CU (256 CUs), at least 256 rows per split
  int s = (512 + tiles - 1) / tiles;
  const int64_t max_s = std::max<int64_t>(1, n_rows / 256);
  if (s > max_s) s = (int)max_s;
  if (s > 8) s = 8;
  if (s < 1) s = 1;
  return s;
}

}  // namespace

size_t gram_workspace_size(int64_t n_rows, int32_t d, int32_t dtype) {
  if (dtype != ISPA_BF16 || d % GT != 0) return 0;
  const int s = gram_splits(n_rows, d);
  if (s <= 1) return 0;
  return (size_t)s * 3 * (size_t)d * d * sizeof(float);
}

ispa_status_t launch_gram(int64_t n_rows, int32_t d, int32_t dtype, const void* A_loc, const void* A_full,
                          float* G, float* C, float* Qff, int32_t accumulate, void* ws, size_t ws_bytes,
                          hipStream_t s) {
  if (dtype == ISPA_F32 || d % GT != 0) {
    if (dtype != ISPA_F32) {
      set_error("bf16 Gram needs d to be a multiple of 128");
      return ISPA_E_INVALID_ARG;
    }
    const int tpd = d / FT;
    hipLaunchKernelGGL(gram_f32_kernel, dim3(tpd * tpd), dim3(256), 0, s, (const float*)A_loc,
                       (const float*)A_full, G, C, Qff, n_rows, d, accumulate);
    return hip_check(hipGetLastError(), "gram_f32_kernel launch");
  }
  const int splits = gram_splits(n_rows, d);
  const size_t need = gram_workspace_size(n_rows, d, dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) {
    set_error("ispa_gram_accum: workspace too small");
    return ISPA_E_WORKSPACE;
  }
  GramParams p;
  p.Al = (const uint16_t*)A_loc;
  p.Af = (const uint16_t*)A_full;
  p.n_rows = n_rows;
  p.d = d;
  p.tiles_per_dim = d / GT;
  p.accumulate = accumulate;
  p.slab = (size_t)d * d;
  const int64_t per = (n_rows + splits - 1) / splits;
  p.rows_per_split = ((per + GBK - 1) / GBK) * GBK;
  if (p.rows_per_split == 0) p.rows_per_split = GBK;
  p.direct = splits == 1;
  if (p.direct) {
    p.G = G;
    p.C = C;
    p.Q = Qff;
  } else {
    p.G = (float*)ws;
    p.C = nullptr;
    p.Q = nullptr;
  }
  const dim3 grid(p.tiles_per_dim * p.tiles_per_dim, splits), block(256);
  if (Qff)
    hipLaunchKernelGGL((gram_bf16_kernel<true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gram_bf16_kernel<false>), grid, block, 0, s, p);
  ispa_status_t st = hip_check(hipGetLastError(), "gram_bf16_kernel launch");
  if (st != ISPA_OK || p.direct) return st;
  const size_t n4 = p.slab / 4;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, (const float*)ws,
                     splits, Qff ? 3 : 2, p.slab, G, C, Qff, accumulate);
  return hip_check(hipGetLastError(), "gram_reduce_kernel launch");
}

}  // namespace ispa
