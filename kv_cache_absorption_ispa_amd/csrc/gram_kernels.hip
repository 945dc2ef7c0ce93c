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
// rows.  Per 32-row stage (three stages in flight) it stages A_loc[:, I],
// A_loc[:, J], A_full[:, J] (and A_full[:, I] when Q_ff is wanted) row-major
// in LDS, straight from
// global memory (buffer loads into LDS, 16-byte chunks XOR-swizzled by row);
// MFMA operands need 8 consecutive rows at one column and come from two
// transposing LDS reads (ds_read_b64_tr_b16).  The A_loc[:, I] operand feeds
// both products.  4 waves in a 2x2 grid each own a
// 64x64 sub-tile (2x2 blocks of v_mfma_f32_32x32x16_bf16).  Rows are split
// over workgroups when there are too few tiles to fill the GPU; the split
// partials go to a workspace and a second kernel sums them in a fixed order
// (deterministic, no atomics).
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int GT = 128;      // output tile J extent (and the I extent of the small tile)
constexpr int GBK = 32;      // rows per stage

// Slot of 16-byte chunk c of staged row r: c ^ gram_swizzle(r).  Each 32-lane
// pass of a transposing operand read takes 4 consecutive chunks from each of 4
// consecutive rows; giving those rows different groups of 4 slots keeps the
// read free of bank conflicts (64 four-byte banks, 256-byte rows).
__device__ __forceinline__ int gram_swizzle(int r) { return (r & 3) << 2; }

struct GramParams {
  const uint16_t* Al;
  const uint16_t* Af;
  float* G;  // direct outputs (splits == 1) or partial slabs (splits > 1)
  float* C;
  float* Q;
  int64_t n_rows;
  int d;
  int tiles_j;  // output tiles along J (d / 128); tile t is (t / tiles_j, t % tiles_j)
  int64_t rows_per_split;
  int accumulate;
  int direct;
  size_t slab;  // elements per partial matrix (d*d) when !direct
};

// Staged matrix m of a stage: 0 A_loc[:, I] and 3 A_full[:, I] (TI columns), 1 A_loc[:, J] and
// 2 A_full[:, J] (GT columns); each GBK rows, row-major, stored one after the other.
template <int TI>
__host__ __device__ constexpr int gram_width(int m) { return (m == 0 || m == 3) ? TI : GT; }
template <int TI>
__host__ __device__ constexpr int gram_moff(int m) {  // element offset of matrix m in a stage
  return m == 0 ? 0 : gram_moff<TI>(m - 1) + GBK * gram_width<TI>(m - 1);
}
template <int TI>
__host__ __device__ constexpr int gram_mloads(int m) { return GBK * gram_width<TI>(m) / 512; }  // 1 KB loads

// TI = I extent of the output tile (128: 4 waves, two workgroups per CU; 256: 8 waves, one per CU,
// a third less operand traffic per product).  Waves sit in a (TI / 64) x 2 grid of 64 x 64 tiles.
template <bool QFF, int TI>
__global__ __launch_bounds__(TI * 2, (TI == 128 && !QFF) ? 2 : 1) void gram_bf16_kernel(GramParams p) {
  constexpr int NWV = TI / 32;      // waves
  constexpr int NM = QFF ? 4 : 3;   // staged matrices: A_loc[:,I], A_loc[:,J], A_full[:,J], [A_full[:,I]]
  constexpr int SS = gram_moff<TI>(NM);  // elements per stage
  constexpr int NLD = gram_moff<TI>(NM) / 512;  // 1 KB wave loads per stage
  constexpr int WLW = NLD / NWV;    // wave loads per wave per stage
  static_assert(WLW * NWV == NLD, "stage loads must split over the waves");
  // three stage buffers as distinct arrays (see the attention kernel: lets the
  // compiler overlap the next stages' loads with this stage's reads)
  __shared__ __attribute__((aligned(1024))) uint16_t s0[SS];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[SS];
  __shared__ __attribute__((aligned(1024))) uint16_t s2[SS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: buffer choice stays scalar
  const int l32 = lane & 31, hh = lane >> 5;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int ti = tile / p.tiles_j, tj = tile % p.tiles_j;
  const int I0 = ti * TI, J0 = tj * GT;
  const int64_t r_begin = (int64_t)split * p.rows_per_split;
  const int64_t r_end = min(p.n_rows, r_begin + p.rows_per_split);
  const int nst = r_end > r_begin ? (int)((r_end - r_begin + GBK - 1) / GBK) : 0;
  const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;  // wave sub-tile origin
  const uint32_t row_bytes = (uint32_t)p.d * 2u;
  // Buffers start at this split's first row; rows at or past r_end read as 0 (range-checked
  // buffer loads).  The host keeps (rows per launch + 64) * row_bytes <= 2^31, so the byte offsets
  // of the padding stages (at most 95 rows past the last row) stay far below 2^32.
  const uint32_t span = r_end > r_begin ? (uint32_t)(r_end - r_begin) * row_bytes : 0u;
  const rsrc_t rl = make_rsrc(p.Al + r_begin * p.d, span);
  const rsrc_t rf = make_rsrc(p.Af + r_begin * p.d, span);

  // this wave's stage loads: wave load g = wave + NWV*j covers load (g - first load of its matrix)
  // of matrix m: 512 / width rows of it
  uint32_t gofs[WLW];
  int lmat[WLW], ldst[WLW];
#pragma unroll
  for (int j = 0; j < WLW; ++j) {
    const int g = wave + NWV * j;
    int mtx = 0;
#pragma unroll
    for (int m = 1; m < NM; ++m)
      if (g >= gram_moff<TI>(m) / 512) mtx = m;
    const int w = gram_width<TI>(mtx), cpr = w / 8, rpw = 64 / cpr;
    const int li = g - gram_moff<TI>(mtx) / 512;
    const int rr = li * rpw + lane / cpr;
    const int chunk = (lane % cpr) ^ gram_swizzle(rr);
    const int col0 = (mtx == 0 || mtx == 3) ? I0 : J0;
    gofs[j] = (uint32_t)rr * row_bytes + (uint32_t)(col0 + chunk * 8) * 2u;
    lmat[j] = mtx;
    ldst[j] = gram_moff<TI>(mtx) + li * 512;
  }
  auto load_stage = [&](int st, uint16_t* buf) {
    const uint32_t sb = (uint32_t)(st * GBK) * row_bytes;
#pragma unroll
    for (int j = 0; j < WLW; ++j) load_to_lds(lmat[j] <= 1 ? rl : rf, buf + ldst[j], gofs[j] + sb);
  };

  // Operand for columns xb .. xb+31 of a staged [32 rows][128 cols] tile and rows 16ks .. 16ks+15:
  // lane (column xb + lane%32, hh) gets rows 16ks + 8*(j/4) + 4*hh + j%4, j = 0..7, through two
  // transposing reads (the same row order serves both operands of a product).
  const int q16 = lane >> 4, i16 = lane & 15;
  const int trow = 4 * (q16 >> 1) + (i16 >> 2);  // row within each 8-row half of a 16-row step
  const int tcol = 16 * (q16 & 1) + 4 * (i16 & 3);
  // The swizzle depends on row & 3 == trow & 3, a lane constant, so each operand block has one
  // per-lane base offset; the row step is a compile-time offset.
  int offI[2], offJ[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int ci = wi + 32 * x + tcol, cj = wj + 32 * x + tcol;
    offI[x] = trow * TI + (((ci >> 3) ^ gram_swizzle(trow)) << 3) + (ci & 7);
    offJ[x] = trow * GT + (((cj >> 3) ^ gram_swizzle(trow)) << 3) + (cj & 7);
  }
  // rows 16ks + 8*(j/4) + 4hh + j%4 of the matrix at t, w columns wide
  auto frag = [&](const uint16_t* t, int off, int ks, int w) {
    const uint16_t* q = t + off + 16 * ks * w;
    const u32x2 a = lds_read_tr(q), b = lds_read_tr(q + 8 * w);
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
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

  auto compute = [&](const uint16_t* buf) {
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 aI[2], bJ[2], fJ[2], fI[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        aI[b] = frag(buf + gram_moff<TI>(0), offI[b], ks, TI);
        bJ[b] = frag(buf + gram_moff<TI>(1), offJ[b], ks, GT);
        fJ[b] = frag(buf + gram_moff<TI>(2), offJ[b], ks, GT);
        if (QFF) fI[b] = frag(buf + gram_moff<TI>(3), offI[b], ks, TI);
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
  };

  // Stages past r_end read as zeros, so the stage count is rounded up to a multiple of three and
  // the loop body (three stages, one per buffer) has no early exit.  Stage st + 2 is in flight
  // while stage st is multiplied; each wait leaves the newest stage's loads outstanding (vmcnt
  // counts this wave's loads, which complete in order).
  constexpr int WAIT_OLDER = 0xF70 | (WLW & 15) | ((WLW >> 4) << 14);  // vmcnt(WLW); expcnt, lgkmcnt free
  const int nst3 = (nst + 2) / 3 * 3;
  if (nst3 > 0) {
    load_stage(0, s0);
    load_stage(1, s1);
  }
  __builtin_amdgcn_s_waitcnt(WAIT_OLDER);
  __syncthreads();
  for (int st = 0; st < nst3; st += 3) {
    load_stage(st + 2, s2);
    compute(s0);
    __builtin_amdgcn_s_waitcnt(WAIT_OLDER);
    __syncthreads();
    const bool more = st + 3 < nst3;
    if (more) load_stage(st + 3, s0);
    compute(s1);
    if (more) __builtin_amdgcn_s_waitcnt(WAIT_OLDER);
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (more) load_stage(st + 4, s1);
    compute(s2);
    if (more) __builtin_amdgcn_s_waitcnt(WAIT_OLDER);
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // epilogue: accumulator element v of lane (col, hh) is row 8(v/4) + 4hh + v%4 of its block.
  // Offsets fit in 32 bits (d <= 2^15 and at most 8 splits of 3 d x d slabs).
  const uint32_t d = (uint32_t)p.d;
  float* G = p.G;
  float* C = p.C;
  float* Q = p.Q;
  if (!p.direct) {
    G = p.G + (size_t)split * (QFF ? 3 : 2) * p.slab;
    C = G + p.slab;  // holds A_loc^T A_full here; the reduction forms C
    Q = G + 2 * p.slab;
  }
  const int mode = !p.direct ? 0 : (p.accumulate ? 2 : 1);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint32_t o0 = (uint32_t)(I0 + wi + 32 * a + 4 * hh) * d + (uint32_t)(J0 + wj + 32 * b + l32);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t o = o0 + (uint32_t)(8 * (v >> 2) + (v & 3)) * d;
        const float g = accG[a][b][v], x = accX[a][b][v];
        if (mode == 0) {
          G[o] = g;
          C[o] = x;
          if (QFF) Q[o] = accQ[a][b][v];
        } else if (mode == 1) {
          G[o] = g;
          C[o] = x - g;
          if (QFF) Q[o] = accQ[a][b][v];
        } else {
          G[o] += g;
          C[o] += x - g;
          if (QFF) Q[o] += accQ[a][b][v];
        }
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

// Rows per launch: (rows + 64) * 2d bytes stays within 2^31 (buffer offsets are 32-bit).
int64_t gram_block_rows(int d) {
  const int64_t r = ((int64_t)1 << 31) / (2 * (int64_t)d) - 2 * GBK;
  return (r / GBK) * GBK;
}

// I extent of the output tile: 256 where d allows it and its tiles fit one round of the 256 CUs
// (with split rows); for larger d the 4-wave 128 tiles pack the rounds better (measured at d = 5120:
// 0.47 ms against 0.49)
int gram_ti(int d) { return (d % 256 == 0 && (d / 256) * (d / GT) <= 256) ? 256 : 128; }

int gram_splits(int64_t n_rows, int d) {
  const int ti = gram_ti(d);
  const int tiles = (d / ti) * (d / GT);
  // 4-wave tiles: about two resident workgroups per CU (256 CUs); 8-wave tiles (one per CU): the
  // most splits that still fit one round.  At least 256 rows per split.
  int s = ti == 128 ? (512 + tiles - 1) / tiles : (tiles >= 256 ? 1 : 256 / tiles);
  const int64_t max_s = std::max<int64_t>(1, n_rows / 256);
  if (s > max_s) s = (int)max_s;
  if (s > 8) s = 8;
  if (s < 1) s = 1;
  return s;
}

}  // namespace

size_t gram_workspace_size(int64_t n_rows, int32_t d, int32_t dtype) {
  if (dtype != ISPA_BF16 || d % GT != 0) return 0;
  const int s = gram_splits(std::min(n_rows, gram_block_rows(d)), d);
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
  const size_t need = gram_workspace_size(n_rows, d, dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) {
    set_error("ispa_gram_accum: workspace too small");
    return ISPA_E_WORKSPACE;
  }
  // Rows go in blocks small enough for 32-bit buffer offsets; later blocks accumulate.
  const int64_t block_rows = gram_block_rows(d);
  int64_t r0 = 0;
  do {
    const int64_t nr = std::min(block_rows, n_rows - r0);
    const int acc = (r0 > 0) ? 1 : accumulate;
    const int splits = gram_splits(nr, d);
    GramParams p;
    p.Al = (const uint16_t*)A_loc + r0 * d;
    p.Af = (const uint16_t*)A_full + r0 * d;
    p.n_rows = nr;
    p.d = d;
    const int ti = gram_ti(d);
    p.tiles_j = d / GT;
    p.accumulate = acc;
    p.slab = (size_t)d * d;
    const int64_t per = (nr + splits - 1) / splits;
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
    const dim3 grid((d / ti) * p.tiles_j, splits), block(2 * ti);
    if (ti == 256) {
      if (Qff)
        hipLaunchKernelGGL((gram_bf16_kernel<true, 256>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((gram_bf16_kernel<false, 256>), grid, block, 0, s, p);
    } else {
      if (Qff)
        hipLaunchKernelGGL((gram_bf16_kernel<true, 128>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((gram_bf16_kernel<false, 128>), grid, block, 0, s, p);
    }
    ispa_status_t st = hip_check(hipGetLastError(), "gram_bf16_kernel launch");
    if (st != ISPA_OK) return st;
    if (!p.direct) {
      const size_t n4 = p.slab / 4;
      hipLaunchKernelGGL(gram_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                         (const float*)ws, splits, Qff ? 3 : 2, p.slab, G, C, Qff, acc);
      st = hip_check(hipGetLastError(), "gram_reduce_kernel launch");
      if (st != ISPA_OK) return st;
    }
    r0 += nr;
  } while (r0 < n_rows);
  return ISPA_OK;
}

}  // namespace ispa
