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
// (and A_full[:, I] when Q_ff is wanted) row-major in LDS, straight from
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

constexpr int GT = 128;      // output tile edge
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
  int tiles_per_dim;
  int64_t rows_per_split;
  int accumulate;
  int direct;
  size_t slab;  // elements per partial matrix (d*d) when !direct
};

template <bool QFF>
__global__ __launch_bounds__(256, 2) void gram_bf16_kernel(GramParams p) {
  constexpr int NM = QFF ? 4 : 3;   // staged matrices: A_loc[:,I], A_loc[:,J], A_full[:,J], [A_full[:,I]]
  constexpr int CPR = GT / 8;       // 16-byte chunks per staged row
  constexpr int RPW = 64 / CPR;     // rows per wave load (1 KB)
  constexpr int WLM = GBK / RPW;    // wave loads per matrix per stage
  constexpr int WLW = NM * WLM / 4; // wave loads per wave per stage
  static_assert(WLW * 4 == NM * WLM, "stage loads must split over 4 waves");
  // two stage buffers as distinct arrays (see the attention kernel: lets the
  // compiler overlap the next stage's loads with this stage's reads)
  __shared__ __attribute__((aligned(1024))) uint16_t s0[NM][GBK * GT];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[NM][GBK * GT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: buffer choice stays scalar
  const int l32 = lane & 31, hh = lane >> 5;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int ti = tile / p.tiles_per_dim, tj = tile % p.tiles_per_dim;
  const int I0 = ti * GT, J0 = tj * GT;
  const int64_t r_begin = (int64_t)split * p.rows_per_split;
  const int64_t r_end = min(p.n_rows, r_begin + p.rows_per_split);
  const int nst = r_end > r_begin ? (int)((r_end - r_begin + GBK - 1) / GBK) : 0;
  const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;  // wave sub-tile origin
  const uint32_t row_bytes = (uint32_t)p.d * 2u;
  // Buffers start at this split's first row; rows at or past r_end read as 0 (range-checked
  // buffer loads).  The host keeps (rows per launch + 64) * row_bytes below 2^31.
  const uint32_t span = r_end > r_begin ? (uint32_t)(r_end - r_begin) * row_bytes : 0u;
  const rsrc_t rl = make_rsrc(p.Al + r_begin * p.d, span);
  const rsrc_t rf = make_rsrc(p.Af + r_begin * p.d, span);

  // this wave's stage loads: wave load g = wave + 4j covers matrix g / WLM, rows (g % WLM) * RPW ..
  uint32_t gofs[WLW];
#pragma unroll
  for (int j = 0; j < WLW; ++j) {
    const int g = wave + 4 * j, mtx = g / WLM;
    const int rr = (g % WLM) * RPW + lane / CPR;
    const int chunk = (lane % CPR) ^ gram_swizzle(rr);
    const int col0 = (mtx == 0 || mtx == 3) ? I0 : J0;
    gofs[j] = (uint32_t)rr * row_bytes + (uint32_t)(col0 + chunk * 8) * 2u;
  }
  auto load_stage = [&](int st, uint16_t (*buf)[GBK * GT]) {
    const uint32_t sb = (uint32_t)(st * GBK) * row_bytes;
#pragma unroll
    for (int j = 0; j < WLW; ++j) {
      const int g = wave + 4 * j, mtx = g / WLM;
      load_to_lds(mtx <= 1 ? rl : rf, buf[mtx] + (g % WLM) * RPW * GT, gofs[j] + sb);
    }
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
    offI[x] = trow * GT + (((ci >> 3) ^ gram_swizzle(trow)) << 3) + (ci & 7);
    offJ[x] = trow * GT + (((cj >> 3) ^ gram_swizzle(trow)) << 3) + (cj & 7);
  }
  auto frag = [&](const uint16_t* t, int off, int ks) {
    const uint16_t* q = t + off + 16 * ks * GT;
    const u32x2 a = lds_read_tr(q), b = lds_read_tr(q + 8 * GT);
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

  auto compute = [&](uint16_t (*buf)[GBK * GT]) {
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 aI[2], bJ[2], fJ[2], fI[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        aI[b] = frag(buf[0], offI[b], ks);
        bJ[b] = frag(buf[1], offJ[b], ks);
        fJ[b] = frag(buf[2], offJ[b], ks);
        if (QFF) fI[b] = frag(buf[NM - 1], offI[b], ks);
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

  // Stages past r_end read as zeros, so the stage count is rounded up to even and the loop
  // body (two stages, one per buffer) has no early exit.
  const int nst2 = (nst + 1) & ~1;
  if (nst2 > 0) load_stage(0, s0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int st = 0; st < nst2; st += 2) {
    load_stage(st + 1, s1);
    compute(s0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (st + 2 < nst2) load_stage(st + 2, s0);
    compute(s1);
    __builtin_amdgcn_s_waitcnt(0);
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

// Rows per launch: (rows + 64) * 2d bytes stays below 2^31 (buffer offsets are 32-bit).
int64_t gram_block_rows(int d) {
  const int64_t r = ((int64_t)1 << 31) / (2 * (int64_t)d) - 2 * GBK;
  return (r / GBK) * GBK;
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
    p.tiles_per_dim = d / GT;
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
    const dim3 grid(p.tiles_per_dim * p.tiles_per_dim, splits), block(256);
    if (Qff)
      hipLaunchKernelGGL((gram_bf16_kernel<true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((gram_bf16_kernel<false>), grid, block, 0, s, p);
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
