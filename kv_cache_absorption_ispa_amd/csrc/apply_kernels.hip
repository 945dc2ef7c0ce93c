// Triangular applies of the absorb solve on the bf16 matrix cores (gfx950).
//
// The closed-form layer absorb (ISPA technical summary, section 2, "Layer Absorb") solves
// (G + lambda I) dW = C W.  With the Cholesky factor's explicit inverse L^-1 the solve is two
// products, Z = L^-1 Y and X = L^-T Z.  On the refined path the float64-accumulated residual
// corrects whatever error the first solve leaves (the refined result converges to the float64 solve
// of the float32 statistics as long as each solve is accurate to well below 1), so both solves
// there may run at reduced precision.  Each float32 operand x is carried as hi = bf16(x) and
// lo = bf16(x - hi) (|x - hi - lo| <= 2^-17 |x|), and a product takes the three bf16 products
// hi*hi + hi*lo + lo*hi with float32 accumulation (the dropped lo*lo term is below 2^-16 of it):
// about 2^-16 relative per product, at three bf16 matrix-core passes instead of one float32 pass
// (float32: 157 TFLOP/s dense; bf16: 2.5 PFLOP/s).
//
// Layout: both operands K-contiguous (A as M x K, B as N x K, row-major), so every 16-byte LDS read
// is one lane's MFMA fragment (v_mfma_f32_32x32x16_bf16: lane l holds row l % 32, k = 8 (l / 32)
// .. + 7).  The first product forms Z^T = Y^T L^-T (A = split(Y^T), B = split(L^-1), lower in k)
// and writes it split, row-major: the second product's B operand; the second, X = L^-T Z
// (A = split(L^-T)), writes float32.  L^-1 is split once per solve, row-major and transposed.
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int PT = 128;        // output tile (PT x PT), 4 waves of 64 x 64
constexpr int SPB = 64;        // split / transpose block
#ifndef APPLY3_RK
#define APPLY3_RK 32    // K columns per stage of the bf16x3 products
#endif
#ifndef APPLY3_NSTG
#define APPLY3_NSTG 3   // stages in the LDS ring
#endif
#ifndef APPLY3W_RK
#define APPLY3W_RK 32   // K columns per stage of the 256-tile products
#endif
#ifndef APPLY3W_NSTG
#define APPLY3W_NSTG 2  // stages in their ring (64 KB each)
#endif
#ifndef APPLY3W_MIN_TILES
#define APPLY3W_MIN_TILES 256
#endif

__device__ __forceinline__ void split2(float x, __bf16& h, __bf16& l) {
  h = (__bf16)x;
  l = (__bf16)(x - (float)h);
}

// Lh, Ll = split(L^-1) and LTh, LTl = split(L^-T) over the 64 x 64 blocks (bi, bj) of L^-1 with
// bj <= 4 (bi / 4) + 3: those the 128- and 256-row tiles of the two products read (lower:
// k < n0 + tile; upper, transposed: k >= m0).  Everything they read outside the triangle is zero in
// L^-1.
__global__ __launch_bounds__(256) void split_lower_kernel(const float* __restrict__ Linv, int d, __bf16* Lh,
                                                          __bf16* Ll, __bf16* LTh, __bf16* LTl,
                                                          const int32_t* __restrict__ info) {
  const int bi = blockIdx.y, bj = blockIdx.x, b = blockIdx.z;
  if (bj > 4 * (bi / 4) + 3 || info[b] != 0) return;
  __shared__ float T[SPB][SPB + 1];
  const size_t dd = (size_t)d * d;
  const float* src = Linv + b * dd + (size_t)bi * SPB * d + bj * SPB;
  const int tid = threadIdx.x, r0 = tid / 16, c = 4 * (tid % 16);
  const size_t o = b * dd + (size_t)bi * SPB * d + bj * SPB;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + 16 * q;
    const f32x4 v = *(const f32x4*)(src + (size_t)r * d + c);
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      T[r][c + e] = v[e];
      __bf16 he, le;
      split2(v[e], he, le);
      h[e] = he;
      l[e] = le;
    }
    *(bf16x4*)(Lh + o + (size_t)r * d + c) = h;
    *(bf16x4*)(Ll + o + (size_t)r * d + c) = l;
  }
  __syncthreads();
  const size_t ot = b * dd + (size_t)bj * SPB * d + bi * SPB;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + 16 * q;  // row of L^-T = column of L^-1
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 he, le;
      split2(T[c + e][r], he, le);
      h[e] = he;
      l[e] = le;
    }
    *(bf16x4*)(LTh + ot + (size_t)r * d + c) = h;
    *(bf16x4*)(LTl + ot + (size_t)r * d + c) = l;
  }
}

// YTh, YTl = split(Y^T): Y is K x N float32 row-major, the outputs N x K.
__global__ __launch_bounds__(256) void split_t_kernel(const float* __restrict__ Y, int K, int N, __bf16* YTh,
                                                      __bf16* YTl, const int32_t* __restrict__ info) {
  const int bk = blockIdx.y, bn = blockIdx.x, b = blockIdx.z;
  if (info[b] != 0) return;
  __shared__ float T[SPB][SPB + 1];
  const size_t kn = (size_t)K * N;
  const float* src = Y + b * kn + (size_t)bk * SPB * N + bn * SPB;
  const int tid = threadIdx.x, r0 = tid / 16, c = 4 * (tid % 16);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + 16 * q;
    const f32x4 v = *(const f32x4*)(src + (size_t)r * N + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) T[r][c + e] = v[e];
  }
  __syncthreads();
  const size_t ot = b * kn + (size_t)bn * SPB * K + bk * SPB;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + 16 * q;  // row of Y^T
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 he, le;
      split2(T[c + e][r], he, le);
      h[e] = he;
      l[e] = le;
    }
    *(bf16x4*)(YTh + ot + (size_t)r * K + c) = h;
    *(bf16x4*)(YTl + ot + (size_t)r * K + c) = l;
  }
}

struct Apply3Params {
  const __bf16 *Ah, *Al;  // M x K (row stride K)
  const __bf16 *Bh, *Bl;  // N x K (row stride K)
  __bf16 *Dh, *Dl;        // OUT_SPLIT: D split, M x N (row stride N)
  float* D;               // else: D float32, M x N (row stride N)
  int M, N, K;
  size_t sA, sB, sD;      // batch strides (elements)
  const int32_t* info;
};

// D = A B^T with one operand triangular (KM_LA: A lower, k < m0 + PT; KM_UA: A upper, k >= m0;
// KM_LB: B lower, k < n0 + PT), as hi*hi + hi*lo + lo*hi.
// K advances in stages of RK columns held in a ring of NSTG LDS buffers, filled straight from global
// memory by buffer loads into LDS (a wave moves 1 KB per load: 32 rows x 16 columns, or 16 rows x 32
// columns); while stage st is multiplied, stages st + 1 .. st + NSTG - 1 are in flight.  A row's
// 16-byte chunks are permuted by row (apply3_slot) so that the 16 rows of a fragment read pass cover
// all 64 banks.  Measured at d = 5120 (refined solve): 32 columns x 3 stages 12.81 ms, x 2 stages
// 13.06, 16 x 4 13.55, 16 x 3 13.83, and 12.96 for register-staged 32-column slabs in two LDS
// buffers.  M, N multiples of PT, K of RK.
template <int RK>
__device__ __forceinline__ int apply3_slot(int row, int chunk) {
  if constexpr (RK == 16) return chunk ^ ((row >> 3) & 1);
  else return chunk ^ ((row >> 2) & 3);
}

constexpr int KM_LA = 0, KM_UA = 1, KM_LB = 2;
template <int KM, bool OUT_SPLIT, int RK, int NSTG>
__global__ __launch_bounds__(256, (NSTG * 4 * PT * RK * 2 <= 80 * 1024) ? 2 : 1) void apply3_kernel(Apply3Params p) {
  const int b = blockIdx.z;
  if (p.info[b] != 0) return;
  // tiles with the most K work first (the dispatch order): for a lower operand the last tiles of
  // its triangle; KM_LB's grid is (M tiles, N tiles) so that its N tile is the slow index
  const int m0 = (KM == KM_LB ? blockIdx.x : (KM == KM_LA ? gridDim.y - 1 - blockIdx.y : blockIdx.y)) * PT;
  const int n0 = (KM == KM_LB ? gridDim.y - 1 - blockIdx.y : blockIdx.x) * PT;
  constexpr int CPR = RK / 8;              // 16-byte chunks per staged row
  constexpr int RPL = 64 / CPR;            // rows per wave load
  constexpr int OPS = PT * RK;             // elements of one operand per stage
  constexpr int SS = 4 * OPS;              // elements per stage: Ah, Al, Bh, Bl
  constexpr int NLD = SS / 512;            // wave loads per stage
  constexpr int WLW = NLD / 4;             // per wave
  static_assert(NLD % 4 == 0, "stage loads must split over the waves");
  __shared__ __attribute__((aligned(1024))) __bf16 S0[SS];
  __shared__ __attribute__((aligned(1024))) __bf16 S1[SS];
  __shared__ __attribute__((aligned(1024))) __bf16 S2[NSTG >= 3 ? SS : 8];
  __shared__ __attribute__((aligned(1024))) __bf16 S3[NSTG >= 4 ? SS : 8];
  __bf16* const buf[4] = {S0, S1, S2, S3};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const uint32_t K = (uint32_t)p.K;
  const uint32_t rows_bytes = (uint32_t)PT * K * 2u;
  const int kb = KM == KM_UA ? m0 : 0;
  const int ke = KM == KM_LA ? min(p.K, m0 + PT) : (KM == KM_LB ? min(p.K, n0 + PT) : p.K);
  const int nst = (ke - kb) / RK;

  const rsrc_t rs[4] = {make_rsrc(p.Ah + b * p.sA + (size_t)m0 * K, rows_bytes),
                        make_rsrc(p.Al + b * p.sA + (size_t)m0 * K, rows_bytes),
                        make_rsrc(p.Bh + b * p.sB + (size_t)n0 * K, rows_bytes),
                        make_rsrc(p.Bl + b * p.sB + (size_t)n0 * K, rows_bytes)};
  // this wave's loads: wave load g = wave + 4 j is rows RPL * (g % BPO) .. of operand g / BPO =
  // 4 j / BPO, known at compile time (a resource indexed at run time costs a waterfall loop per load)
  constexpr int BPO = PT / RPL;  // wave loads per operand and stage
  static_assert(BPO % 4 == 0, "a wave's loads of one j share an operand");
  uint32_t gofs[WLW];
  int ldst[WLW];
#pragma unroll
  for (int j = 0; j < WLW; ++j) {
    const int g = wave + 4 * j;
    const int o = 4 * j / BPO, blk = g % BPO;
    const int row = blk * RPL + lane / CPR;
    const int chunk = apply3_slot<RK>(row, lane % CPR);  // the data chunk that lands in slot lane % CPR
    gofs[j] = (uint32_t)row * K * 2u + (uint32_t)chunk * 16u;
    ldst[j] = o * OPS + blk * 512;
  }
  auto load_stage = [&](int st, __bf16* bb) {
    const uint32_t kofs = (uint32_t)(kb + st * RK) * 2u;
#pragma unroll
    for (int j = 0; j < WLW; ++j) load_to_lds(rs[4 * j / BPO], (uint16_t*)(bb + ldst[j]), gofs[j] + kofs);
  };
  // fragment of rows r0 + l32, columns 16 ks + 8 hh .. + 7 of operand o in a stage
  auto frag = [&](const __bf16* bb, int o, int r0, int ks) {
    const int row = r0 + l32;
    return *(const bf16x8*)(bb + o * OPS + row * RK + 8 * apply3_slot<RK>(row, 2 * ks + hh));
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};
  auto compute = [&](const __bf16* bb) {
#pragma unroll
    for (int ks = 0; ks < RK / 16; ++ks) {
      bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = frag(bb, 0, wm + 32 * i, ks);
        al[i] = frag(bb, 1, wm + 32 * i, ks);
        bh[i] = frag(bb, 2, wn + 32 * i, ks);
        bl[i] = frag(bb, 3, wn + 32 * i, ks);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        }
    }
  };
  // Ring: stage st in buffer st % NSTG (buffers chosen at compile time).  Step st loads stage
  // st + NSTG - 1 and multiplies stage st, NSTG - 1 stages in flight.  At the top of step st each wave
  // waits for its own loads of stage st (all but the NSTG - 2 newer stages': vmcnt counts this wave's
  // loads, which complete in order); the barrier then makes every wave's loads visible and frees the
  // buffer stage st - 1 was read from.  A plain barrier, not __syncthreads(), whose fence would wait
  // for the newer stages too.  Every step issues its loads, also past the last stage: they read
  // columns past ke of the tile's own rows (or zeros past its end) into buffers that are not
  // multiplied, and the wait after the loop drains them.
  constexpr int KEEP = (NSTG - 2) * WLW;
  constexpr int WAIT_CUR = 0xF70 | (KEEP & 15) | ((KEEP >> 4) << 14);  // vmcnt(KEEP)
  const int nstR = (nst + NSTG - 1) / NSTG * NSTG;
#pragma unroll
  for (int k = 0; k + 1 < NSTG; ++k) load_stage(k, buf[k]);
  for (int st = 0; st < nstR; st += NSTG) {
#pragma unroll
    for (int u = 0; u < NSTG; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_CUR);
      __builtin_amdgcn_s_barrier();
      load_stage(st + u + NSTG - 1, buf[(u + NSTG - 1) % NSTG]);
      __builtin_amdgcn_sched_barrier(0);
      if (st + u < nst) compute(buf[u]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave's products are done before the epilogue reuses the ring
  // acc[i][j][v]: row m0 + wm + 32 i + 8 (v / 4) + 4 hh + v % 4, column n0 + wn + 32 j + l32
  if constexpr (OUT_SPLIT) {
    // through LDS (the ring is free after the last barrier): each wave parks half of its 64 x 64
    // float32 tile at a time (32 rows, 8.5 KB; waves 0-2 in the first buffer, wave 3 in the second),
    // then every lane splits 8 consecutive elements of a row and stores 16 bytes of hi and of lo, 8
    // lanes covering a 128-byte row segment
    constexpr int TS = 64 + 4;  // row stride (floats) of a parked half tile
    static_assert(3 * 32 * TS * 4 <= SS * 2 && 32 * TS * 4 <= SS * 2, "parked halves fit the buffers");
    float* T = wave < 3 ? (float*)&S0[0] + wave * 32 * TS : (float*)&S1[0];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) T[(8 * (v >> 2) + 4 * hh + (v & 3)) * TS + 32 * j + l32] = acc[i][j][v];
      __builtin_amdgcn_wave_barrier();  // the same wave reads its half back (LDS is in order within a wave)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = (lane >> 3) + 8 * q, c8 = 8 * (lane & 7);
        const f32x4 x0 = *(const f32x4*)(T + row * TS + c8);
        const f32x4 x1 = *(const f32x4*)(T + row * TS + c8 + 4);
        bf16x8 h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          __bf16 he, le;
          split2(x0[e], he, le);
          h[e] = he;
          l[e] = le;
          split2(x1[e], he, le);
          h[4 + e] = he;
          l[4 + e] = le;
        }
        const size_t o = b * p.sD + (size_t)(m0 + wm + 32 * i + row) * p.N + n0 + wn + c8;
        *(bf16x8*)(p.Dh + o) = h;
        *(bf16x8*)(p.Dl + o) = l;
      }
      __builtin_amdgcn_wave_barrier();  // all reads of this half are issued before the next overwrites it
    }
  } else {
    float* D = p.D + b * p.sD;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
          const int c = n0 + wn + 32 * j + l32;
          D[(size_t)r * p.N + c] = acc[i][j][v];
        }
  }
}

// The same products on 256 x 256 tiles with 8 waves (two per SIMD) of 128 x 64 each: every operand
// byte staged serves twice the multiplies of a 128 x 128 tile, which halves the operand traffic
// from the caches that bounds the 128-tile products (about 4 GB per product at d = 5120: 7.7 TB/s).
// A stage holds RK columns of the four operands (64 KB at RK = 32); M, N multiples of 256.  Each
// output element sums the same products in the same order as on 128 x 128 tiles, so the two give
// the same bits.  d = 5120: 515 -> 390 us per product (refined solve 11.56 -> 11.07 ms).
constexpr int PTW = 256;
template <int KM, bool OUT_SPLIT, int RK, int NSTG>
__global__ __launch_bounds__(512) void apply3w_kernel(Apply3Params p) {
  const int b = blockIdx.z;
  if (p.info[b] != 0) return;
  const int m0 = (KM == KM_LB ? blockIdx.x : (KM == KM_LA ? gridDim.y - 1 - blockIdx.y : blockIdx.y)) * PTW;
  const int n0 = (KM == KM_LB ? gridDim.y - 1 - blockIdx.y : blockIdx.x) * PTW;
  constexpr int CPR = RK / 8;
  constexpr int RPL = 64 / CPR;
  constexpr int OPS = PTW * RK;
  constexpr int SS = 4 * OPS;
  constexpr int NLD = SS / 512;
  constexpr int WLW = NLD / 8;
  static_assert(NLD % 8 == 0, "stage loads must split over the waves");
  static_assert(NSTG >= 2 && NSTG <= 4, "ring of two to four stages");
  __shared__ __attribute__((aligned(1024))) __bf16 S0[SS];
  __shared__ __attribute__((aligned(1024))) __bf16 S1[SS];
  __shared__ __attribute__((aligned(1024))) __bf16 S2[NSTG >= 3 ? SS : 8];
  __shared__ __attribute__((aligned(1024))) __bf16 S3[NSTG >= 4 ? SS : 8];
  __bf16* const buf[4] = {S0, S1, S2, S3};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = (wave >> 2) * 128, wn = (wave & 3) * 64;
  const uint32_t K = (uint32_t)p.K;
  const uint32_t rows_bytes = (uint32_t)PTW * K * 2u;
  const int kb = KM == KM_UA ? m0 : 0;
  const int ke = KM == KM_LA ? min(p.K, m0 + PTW) : (KM == KM_LB ? min(p.K, n0 + PTW) : p.K);
  const int nst = (ke - kb) / RK;

  const rsrc_t rs[4] = {make_rsrc(p.Ah + b * p.sA + (size_t)m0 * K, rows_bytes),
                        make_rsrc(p.Al + b * p.sA + (size_t)m0 * K, rows_bytes),
                        make_rsrc(p.Bh + b * p.sB + (size_t)n0 * K, rows_bytes),
                        make_rsrc(p.Bl + b * p.sB + (size_t)n0 * K, rows_bytes)};
  // wave load g = wave + 8 j: operand g / BPO = 8 j / BPO, known at compile time (a resource indexed
  // at run time costs a waterfall loop per load)
  constexpr int BPO = PTW / RPL;  // wave loads per operand and stage
  static_assert(BPO % 8 == 0, "a wave's loads of one j share an operand");
  uint32_t gofs[WLW];
  int ldst[WLW];
#pragma unroll
  for (int j = 0; j < WLW; ++j) {
    const int g = wave + 8 * j;
    const int o = 8 * j / BPO, blk = g % BPO;
    const int row = blk * RPL + lane / CPR;
    const int chunk = apply3_slot<RK>(row, lane % CPR);
    gofs[j] = (uint32_t)row * K * 2u + (uint32_t)chunk * 16u;
    ldst[j] = o * OPS + blk * 512;
  }
  auto load_stage = [&](int st, __bf16* bb) {
    const uint32_t kofs = (uint32_t)(kb + st * RK) * 2u;
#pragma unroll
    for (int j = 0; j < WLW; ++j) load_to_lds(rs[8 * j / BPO], (uint16_t*)(bb + ldst[j]), gofs[j] + kofs);
  };
  auto frag = [&](const __bf16* bb, int o, int r0, int ks) {
    const int row = r0 + l32;
    return *(const bf16x8*)(bb + o * OPS + row * RK + 8 * apply3_slot<RK>(row, 2 * ks + hh));
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};
  auto compute = [&](const __bf16* bb) {
#pragma unroll
    for (int ks = 0; ks < RK / 16; ++ks) {
      bf16x8 ah[4], al[4], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ah[i] = frag(bb, 0, wm + 32 * i, ks);
        al[i] = frag(bb, 1, wm + 32 * i, ks);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bh[j] = frag(bb, 2, wn + 32 * j, ks);
        bl[j] = frag(bb, 3, wn + 32 * j, ks);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
    }
  };
  // Ring: stage st in buffer st % NSTG.  Step st loads stage st + NSTG - 1 and multiplies stage st,
  // NSTG - 1 stages in flight.  At the top of step st each wave waits for its own loads of stage st
  // (all but the NSTG - 2 newer stages': vmcnt counts this wave's loads, which complete in order);
  // the barrier then makes every wave's loads visible and frees the buffer stage st - 1 was read
  // from.  A plain barrier, not __syncthreads(), whose fence would wait for the newer stages too.
  // Every step issues its loads, also past the last stage: they read columns past ke of the tile's
  // own rows (or zeros past its end) into buffers that are not multiplied, and the wait after the
  // loop drains them.
  constexpr int KEEP = (NSTG - 2) * WLW;
  constexpr int WAIT_CUR = 0xF70 | (KEEP & 15) | ((KEEP >> 4) << 14);  // vmcnt(KEEP)
  const int nstR = (nst + NSTG - 1) / NSTG * NSTG;
#pragma unroll
  for (int k = 0; k + 1 < NSTG; ++k) load_stage(k, buf[k]);
  for (int st = 0; st < nstR; st += NSTG) {
#pragma unroll
    for (int u = 0; u < NSTG; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_CUR);
      __builtin_amdgcn_s_barrier();
      load_stage(st + u + NSTG - 1, buf[(u + NSTG - 1) % NSTG]);
      __builtin_amdgcn_sched_barrier(0);
      if (st + u < nst) compute(buf[u]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave's products are done before the epilogue reuses the ring
  // acc[i][j][v]: row m0 + wm + 32 i + 8 (v / 4) + 4 hh + v % 4, column n0 + wn + 32 j + l32
  if constexpr (OUT_SPLIT) {
    // through LDS: each wave parks one 32 x 64 float32 row of tiles at a time (8.5 KB; WPB waves per
    // ring buffer), then every lane splits 8 consecutive elements of a row and stores 16 bytes of hi
    // and of lo
    constexpr int TS = 64 + 4;
    constexpr int WPB = SS * 2 / (32 * TS * 4);
    static_assert(WPB * (NSTG < 3 ? NSTG : 3) >= 8, "parked rows fit the first three buffers");
    float* T = (float*)(wave < WPB ? S0 : (wave < 2 * WPB ? S1 : S2)) + (wave % WPB) * 32 * TS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) T[(8 * (v >> 2) + 4 * hh + (v & 3)) * TS + 32 * j + l32] = acc[i][j][v];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = (lane >> 3) + 8 * q, c8 = 8 * (lane & 7);
        const f32x4 x0 = *(const f32x4*)(T + row * TS + c8);
        const f32x4 x1 = *(const f32x4*)(T + row * TS + c8 + 4);
        bf16x8 h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          __bf16 he, le;
          split2(x0[e], he, le);
          h[e] = he;
          l[e] = le;
          split2(x1[e], he, le);
          h[4 + e] = he;
          l[4 + e] = le;
        }
        const size_t o = b * p.sD + (size_t)(m0 + wm + 32 * i + row) * p.N + n0 + wn + c8;
        *(bf16x8*)(p.Dh + o) = h;
        *(bf16x8*)(p.Dl + o) = l;
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    float* D = p.D + b * p.sD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
          const int c = n0 + wn + 32 * j + l32;
          D[(size_t)r * p.N + c] = acc[i][j][v];
        }
  }
}

// R = C W of the absorb on the bf16 matrix cores, at float32 accuracy.  Each float32 operand is
// carried as three bf16 parts, x = h + m + l exactly (h = bf16(x); the remainder x - h is exact in
// float32 and has at most 16 significant bits, so m = bf16(x - h) leaves at most 8, which l holds
// exactly; only values within 2^16 of float32's smallest normal lose low bits).  A product keeps the
// six terms of order <= 2 (hh, hm, mh, hl, mm, lh); the three it drops (ml, lm, ll) are below 2^-23
// of it, so the result is as accurate as a float32 GEMM's, at six bf16 passes (2.5 PFLOP/s) instead
// of one float32 pass (157.3 TFLOP/s).  On 256 x 256 tiles (prod6w_kernel, two waves per SIMD) the
// sum over K accumulates in float32 as in a float32 GEMM; the 128 x 128 kernel (prod6_kernel, one
// wave per SIMD) adds each 256-column slab into float64 registers instead.  (The refinement's
// residual needs far more than float32 accuracy, about 2^-34 relative to |G| |X| at the conditioning
// the statistics have, which float32 accumulators cannot hold; it stays on the float64 matrix
// cores.)
__device__ __forceinline__ void split3(float x, __bf16& h, __bf16& m, __bf16& l) {
  h = (__bf16)x;
  const float r = x - (float)h;
  m = (__bf16)r;
  l = (__bf16)(r - (float)m);
}

// P0, P1, P2 = split3(S), elementwise: S is `count` float32 per batch entry (count % 4 == 0).
__global__ __launch_bounds__(256) void split3_kernel(const float* __restrict__ S, size_t count, __bf16* P0,
                                                     __bf16* P1, __bf16* P2, const int32_t* __restrict__ info) {
  const int b = blockIdx.y;
  if (info[b] != 0) return;
  const size_t i = 4 * ((size_t)blockIdx.x * 256 + threadIdx.x);
  if (i >= count) return;
  const size_t o = b * count + i;
  const f32x4 v = *(const f32x4*)(S + o);
  bf16x4 h, m, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    __bf16 he, me, le;
    split3(v[e], he, me, le);
    h[e] = he;
    m[e] = me;
    l[e] = le;
  }
  *(bf16x4*)(P0 + o) = h;
  *(bf16x4*)(P1 + o) = m;
  *(bf16x4*)(P2 + o) = l;
}

// P0, P1, P2 = split3(Y^T): Y is K x N float32 row-major, the planes N x K.
__global__ __launch_bounds__(256) void split3_t_kernel(const float* __restrict__ Y, int K, int N, __bf16* P0,
                                                       __bf16* P1, __bf16* P2, const int32_t* __restrict__ info) {
  const int bk = blockIdx.y, bn = blockIdx.x, b = blockIdx.z;
  if (info[b] != 0) return;
  __shared__ float T[SPB][SPB + 1];
  const size_t kn = (size_t)K * N;
  const float* src = Y + b * kn + (size_t)bk * SPB * N + bn * SPB;
  const int tid = threadIdx.x, r0 = tid / 16, c = 4 * (tid % 16);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + 16 * q;
    const f32x4 v = *(const f32x4*)(src + (size_t)r * N + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) T[r][c + e] = v[e];
  }
  __syncthreads();
  const size_t ot = b * kn + (size_t)bn * SPB * K + bk * SPB;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + 16 * q;  // row of Y^T
    bf16x4 h, m, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 he, me, le;
      split3(T[c + e][r], he, me, le);
      h[e] = he;
      m[e] = me;
      l[e] = le;
    }
    const size_t o = ot + (size_t)r * K + c;
    *(bf16x4*)(P0 + o) = h;
    *(bf16x4*)(P1 + o) = m;
    *(bf16x4*)(P2 + o) = l;
  }
}

struct Prod6Params {
  const __bf16* A[3];    // M x K planes (row stride K)
  const __bf16* B[3];    // N x K planes (row stride K)
  float* D;              // M x N float32: A B^T
  int M, N, K, batch;
  size_t sA, sB, sD;     // batch strides (elements)
  const int32_t* info;
};

#ifndef PROD6_NSTG
#define PROD6_NSTG 2   // stages in the LDS ring (48 KB each)
#endif
#ifndef PROD6_FLS
#define PROD6_FLS 8    // 32-column stages per float64 flush (each flush moves the float32 accumulators
                       // out of the accumulation registers: 2 -> 8 stages, 3.87 -> 3.74 ms at d = 5120)
#endif

// Same ring as apply3_kernel with six operand planes per stage (RK = 32 columns of K); PT x PT
// output tile, 4 waves of 64 x 64.  M, N multiples of PT, K of RK.
// Tiles in row-major order over (batch, M tiles, N tiles); with fewer workgroups than tiles each
// workgroup takes tiles gridDim.x apart (a bounded launch leaves compute units to other streams).
template <int NSTG, int FLS>
__global__ __launch_bounds__(256, 1) void prod6_kernel(Prod6Params p) {
  constexpr int RK = 32;
  constexpr int CPR = RK / 8;
  constexpr int RPL = 64 / CPR;
  constexpr int OPS = PT * RK;
  constexpr int SS = 6 * OPS;   // A0 A1 A2 B0 B1 B2
  constexpr int NLD = SS / 512;
  constexpr int WLW = NLD / 4;
  static_assert(NLD % 4 == 0, "stage loads must split over the waves");
  __shared__ __attribute__((aligned(1024))) __bf16 S0[SS];
  __shared__ __attribute__((aligned(1024))) __bf16 S1[SS];
  __shared__ __attribute__((aligned(1024))) __bf16 S2[NSTG >= 3 ? SS : 8];
  __bf16* const buf[3] = {S0, S1, S2};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const uint32_t K = (uint32_t)p.K;
  const uint32_t rows_bytes = (uint32_t)PT * K * 2u;
  const int nst = p.K / RK;
  const int tn = p.N / PT, tmn = (p.M / PT) * tn;
  const int ntiles = tmn * p.batch;

  // wave load g = wave + 4 j: plane g / BPO = 4 j / BPO, known at compile time (a resource indexed
  // at run time costs a waterfall loop per load)
  constexpr int NW = 4, BPO = PT / RPL;
  static_assert(BPO % NW == 0, "a wave's loads of one j share a plane");
  uint32_t gofs[WLW];
  int ldst[WLW];
#pragma unroll
  for (int j = 0; j < WLW; ++j) {
    const int g = wave + NW * j;
    const int o = NW * j / BPO, blk = g % BPO;
    const int row = blk * RPL + lane / CPR;
    const int chunk = apply3_slot<RK>(row, lane % CPR);
    gofs[j] = (uint32_t)row * K * 2u + (uint32_t)chunk * 16u;
    ldst[j] = o * OPS + blk * 512;
  }
  auto frag = [&](const __bf16* bb, int o, int r0, int ks) {
    const int row = r0 + l32;
    return *(const bf16x8*)(bb + o * OPS + row * RK + 8 * apply3_slot<RK>(row, 2 * ks + hh));
  };

  for (int t = blockIdx.y * gridDim.x + blockIdx.x + (int)blockIdx.z * tmn; t < ntiles;
       t += gridDim.x * gridDim.y * gridDim.z) {
    const int b = t / tmn;
    const int m0 = (t % tmn) / tn * PT, n0 = (t % tn) * PT;
    if (p.info[b] != 0) continue;
    rsrc_t rs[6];
#pragma unroll
    for (int o = 0; o < 3; ++o) {
      rs[o] = make_rsrc(p.A[o] + b * p.sA + (size_t)m0 * K, rows_bytes);
      rs[3 + o] = make_rsrc(p.B[o] + b * p.sB + (size_t)n0 * K, rows_bytes);
    }
    auto load_stage = [&](int st, __bf16* bb) {
      const uint32_t kofs = (uint32_t)(st * RK) * 2u;
#pragma unroll
      for (int j = 0; j < WLW; ++j) load_to_lds(rs[NW * j / BPO], (uint16_t*)(bb + ldst[j]), gofs[j] + kofs);
    };
    f32x16 acc[2][2];
    double acc64[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = f32x16{0};
#pragma unroll
        for (int v = 0; v < 16; ++v) acc64[i][j][v] = 0.0;
      }
    auto compute = [&](const __bf16* bb) {
#pragma unroll
      for (int ks = 0; ks < RK / 16; ++ks) {
        bf16x8 a[3][2], bq[3][2];
#pragma unroll
        for (int o = 0; o < 3; ++o)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            a[o][i] = frag(bb, o, wm + 32 * i, ks);
            bq[o][i] = frag(bb, 3 + o, wn + 32 * i, ks);
          }
        // smallest terms first; the four tiles' chains interleave
        constexpr int TA[6] = {2, 0, 1, 1, 0, 0}, TB[6] = {0, 2, 1, 0, 1, 0};
#pragma unroll
        for (int q = 0; q < 6; ++q)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[TA[q]][i], bq[TB[q]][j], acc[i][j], 0, 0, 0);
      }
    };
    auto flush = [&]() {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int v = 0; v < 16; ++v) acc64[i][j][v] += (double)acc[i][j][v];
          acc[i][j] = f32x16{0};
        }
    };
    constexpr int KEEP = (NSTG - 2) * WLW;
    constexpr int WAIT_KEEP = 0xF70 | (KEEP & 15) | ((KEEP >> 4) << 14);  // vmcnt(KEEP)
    const int nstR = (nst + NSTG - 1) / NSTG * NSTG;
    // the previous tile's last barrier ended every read of the ring
#pragma unroll
    for (int k = 0; k + 1 < NSTG; ++k)
      if (k < nst) load_stage(k, buf[k]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int st = 0; st < nstR; st += NSTG) {
#pragma unroll
      for (int k = 0; k < NSTG; ++k) {
        const int cur = st + k, nxt = cur + NSTG - 1;
        if (nxt < nst) load_stage(nxt, buf[(k + NSTG - 1) % NSTG]);
        if (cur < nst) {
          compute(buf[k]);
          if ((cur + 1) % FLS == 0 || cur + 1 == nst) flush();
        }
        if (nxt < nst) __builtin_amdgcn_s_waitcnt(WAIT_KEEP);
        else __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
    // acc64[i][j][v]: row m0 + wm + 32 i + 8 (v / 4) + 4 hh + v % 4, column n0 + wn + 32 j + l32
    float* D = p.D + b * p.sD;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
          const int c = n0 + wn + 32 * j + l32;
          D[(size_t)r * p.N + c] = (float)acc64[i][j][v];
        }
  }
}

// The same product on 256 x 256 tiles with 8 waves (two per SIMD) of 128 x 64 each, accumulating in
// float32 over all of K like a float32 GEMM (its K-long sum rounds in float32; the product terms are
// still exact to 2^-23).  Without the float64 registers two waves fit each SIMD, and a staged byte
// serves twice the multiplies of a 128 x 128 tile: at d = 5120 on 128 workgroups beside the
// factorisation 3.74 -> 2.84 ms (the 128-tile kernel's one wave per SIMD left it at 34 % MFMA-busy
// on its compute units).  A stage holds RK columns of the six planes (48 KB at RK = 16).  Tiles in
// row-major order; with fewer workgroups than tiles each takes tiles gridDim.x apart.  M, N
// multiples of 256, K of RK.
template <int RK, int NSTG>
__global__ __launch_bounds__(512) void prod6w_kernel(Prod6Params p) {
  constexpr int CPR = RK / 8;
  constexpr int RPL = 64 / CPR;
  constexpr int OPS = PTW * RK;
  constexpr int SS = 6 * OPS;   // A0 A1 A2 B0 B1 B2
  constexpr int NLD = SS / 512;
  constexpr int WLW = NLD / 8;
  static_assert(NLD % 8 == 0, "stage loads must split over the waves");
  static_assert(NSTG >= 2 && NSTG <= 3, "ring of two or three stages");
  __shared__ __attribute__((aligned(1024))) __bf16 S0[SS];
  __shared__ __attribute__((aligned(1024))) __bf16 S1[SS];
  __shared__ __attribute__((aligned(1024))) __bf16 S2[NSTG >= 3 ? SS : 8];
  __bf16* const buf[3] = {S0, S1, S2};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = (wave >> 2) * 128, wn = (wave & 3) * 64;
  const uint32_t K = (uint32_t)p.K;
  const uint32_t rows_bytes = (uint32_t)PTW * K * 2u;
  const int nst = p.K / RK;
  const int tn = p.N / PTW, tmn = (p.M / PTW) * tn;
  const int ntiles = tmn * p.batch;

  // wave load g = wave + 8 j: plane g / BPO = 8 j / BPO, known at compile time (a resource indexed
  // at run time costs a waterfall loop per load)
  constexpr int NW = 8, BPO = PTW / RPL;
  static_assert(BPO % NW == 0, "a wave's loads of one j share a plane");
  uint32_t gofs[WLW];
  int ldst[WLW];
#pragma unroll
  for (int j = 0; j < WLW; ++j) {
    const int g = wave + NW * j;
    const int o = NW * j / BPO, blk = g % BPO;
    const int row = blk * RPL + lane / CPR;
    const int chunk = apply3_slot<RK>(row, lane % CPR);
    gofs[j] = (uint32_t)row * K * 2u + (uint32_t)chunk * 16u;
    ldst[j] = o * OPS + blk * 512;
  }
  auto frag = [&](const __bf16* bb, int o, int r0, int ks) {
    const int row = r0 + l32;
    return *(const bf16x8*)(bb + o * OPS + row * RK + 8 * apply3_slot<RK>(row, 2 * ks + hh));
  };

  for (int t = blockIdx.y * gridDim.x + blockIdx.x + (int)blockIdx.z * tmn; t < ntiles;
       t += gridDim.x * gridDim.y * gridDim.z) {
    const int b = t / tmn;
    const int m0 = (t % tmn) / tn * PTW, n0 = (t % tn) * PTW;
    if (p.info[b] != 0) continue;
    rsrc_t rs[6];
#pragma unroll
    for (int o = 0; o < 3; ++o) {
      rs[o] = make_rsrc(p.A[o] + b * p.sA + (size_t)m0 * K, rows_bytes);
      rs[3 + o] = make_rsrc(p.B[o] + b * p.sB + (size_t)n0 * K, rows_bytes);
    }
    auto load_stage = [&](int st, __bf16* bb) {
      const uint32_t kofs = (uint32_t)(st * RK) * 2u;
#pragma unroll
      for (int j = 0; j < WLW; ++j) load_to_lds(rs[NW * j / BPO], (uint16_t*)(bb + ldst[j]), gofs[j] + kofs);
    };
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};
    auto compute = [&](const __bf16* bb) {
#pragma unroll
      for (int ks = 0; ks < RK / 16; ++ks) {
        bf16x8 a[3][4], bq[3][2];
#pragma unroll
        for (int o = 0; o < 3; ++o) {
#pragma unroll
          for (int i = 0; i < 4; ++i) a[o][i] = frag(bb, o, wm + 32 * i, ks);
#pragma unroll
          for (int j = 0; j < 2; ++j) bq[o][j] = frag(bb, 3 + o, wn + 32 * j, ks);
        }
        // smallest terms first; the eight tiles' chains interleave
        constexpr int TA[6] = {2, 0, 1, 1, 0, 0}, TB[6] = {0, 2, 1, 0, 1, 0};
#pragma unroll
        for (int q = 0; q < 6; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[TA[q]][i], bq[TB[q]][j], acc[i][j], 0, 0, 0);
      }
    };
    // Ring as in apply3w_kernel: step st loads stage st + NSTG - 1 and multiplies stage st; each wave
    // waits for its own loads of stage st only, then a plain barrier (a __syncthreads() fence would
    // wait for the newer stages too).  Loads past the last stage read columns of the tile's own rows
    // (or zeros past its end) into buffers that are not multiplied.  The previous tile's closing
    // barrier ended every read of the ring.
    constexpr int KEEP = (NSTG - 2) * WLW;
    constexpr int WAIT_CUR = 0xF70 | (KEEP & 15) | ((KEEP >> 4) << 14);  // vmcnt(KEEP)
    const int nstR = (nst + NSTG - 1) / NSTG * NSTG;
#pragma unroll
    for (int k = 0; k + 1 < NSTG; ++k) load_stage(k, buf[k]);
    for (int st = 0; st < nstR; st += NSTG) {
#pragma unroll
      for (int u = 0; u < NSTG; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WAIT_CUR);
        __builtin_amdgcn_s_barrier();
        load_stage(st + u + NSTG - 1, buf[(u + NSTG - 1) % NSTG]);
        __builtin_amdgcn_sched_barrier(0);
        if (st + u < nst) compute(buf[u]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every wave is done with the ring before the next tile's loads
    // acc[i][j][v]: row m0 + wm + 32 i + 8 (v / 4) + 4 hh + v % 4, column n0 + wn + 32 j + l32
    float* D = p.D + b * p.sD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
          const int c = n0 + wn + 32 * j + l32;
          D[(size_t)r * p.N + c] = acc[i][j][v];
        }
  }
}

#ifndef PROD6W_RK
#define PROD6W_RK 16
#endif
#ifndef PROD6W_NSTG
#define PROD6W_NSTG 3
#endif
#ifndef PROD6_WIDE
#define PROD6_WIDE 1
#endif

}  // namespace

bool apply3_supported(int32_t d, int32_t d_out) { return d % PT == 0 && d_out % PT == 0; }

ispa_status_t launch_split_lower(int32_t d, int32_t batch, const float* Linv, void* Lsplit, void* LTsplit,
                                 const int32_t* info, hipStream_t s) {
  const size_t bdd = (size_t)batch * d * d;
  __bf16* L = (__bf16*)Lsplit;
  __bf16* LT = (__bf16*)LTsplit;
  hipLaunchKernelGGL(split_lower_kernel, dim3(d / SPB, d / SPB, batch), dim3(256), 0, s, Linv, d, L, L + bdd, LT,
                     LT + bdd, info);
  return hip_check(hipGetLastError(), "split_lower_kernel launch");
}

ispa_status_t launch_chol_apply3(int32_t d, int32_t d_out, int32_t batch, const void* Lsplit, const void* LTsplit,
                                 const float* Y, void* YTsplit, void* ZTsplit, float* X, const int32_t* info,
                                 hipStream_t s) {
  if (!apply3_supported(d, d_out)) {
    set_error("internal: bf16x3 apply needs d and d_out multiples of 128");
    return ISPA_E_INVALID_ARG;
  }
  const size_t dd = (size_t)d * d, dn = (size_t)d * d_out;
  const size_t bdd = (size_t)batch * dd, bdn = (size_t)batch * dn;
  const __bf16* L = (const __bf16*)Lsplit;
  const __bf16* LT = (const __bf16*)LTsplit;
  __bf16* YT = (__bf16*)YTsplit;
  __bf16* ZT = (__bf16*)ZTsplit;
  hipLaunchKernelGGL(split_t_kernel, dim3(d_out / SPB, d / SPB, batch), dim3(256), 0, s, Y, d, d_out, YT, YT + bdn,
                     info);
  ispa_status_t st = hip_check(hipGetLastError(), "split_t_kernel launch");
  if (st != ISPA_OK) return st;
  // Z^T = Y^T L^-T (A = Y^T, d_out x d; B = L^-1 as rows of k, lower: k <= n), split, row-major:
  // exactly the second product's B operand
  // 256 x 256 tiles where they still give every compute unit a tile
  const bool wide = d % PTW == 0 && d_out % PTW == 0 && (size_t)(d / PTW) * (d_out / PTW) * batch >= APPLY3W_MIN_TILES;
  Apply3Params p{};
  p.Ah = YT; p.Al = YT + bdn; p.Bh = L; p.Bl = L + bdd; p.Dh = ZT; p.Dl = ZT + bdn;
  p.M = d_out; p.N = d; p.K = d;
  p.sA = dn; p.sB = dd; p.sD = dn;
  p.info = info;
  if (wide)
    hipLaunchKernelGGL((apply3w_kernel<KM_LB, true, APPLY3W_RK, APPLY3W_NSTG>), dim3(d_out / PTW, d / PTW, batch),
                       dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((apply3_kernel<KM_LB, true, APPLY3_RK, APPLY3_NSTG>), dim3(d_out / PT, d / PT, batch),
                       dim3(256), 0, s, p);
  st = hip_check(hipGetLastError(), "apply3_kernel launch");
  if (st != ISPA_OK) return st;
  // X = L^-T Z
  Apply3Params q{};
  q.Ah = LT; q.Al = LT + bdd; q.Bh = ZT; q.Bl = ZT + bdn; q.D = X;
  q.M = d; q.N = d_out; q.K = d;
  q.sA = dd; q.sB = dn; q.sD = dn;
  q.info = info;
  if (wide)
    hipLaunchKernelGGL((apply3w_kernel<KM_UA, false, APPLY3W_RK, APPLY3W_NSTG>), dim3(d_out / PTW, d / PTW, batch),
                       dim3(512), 0, s, q);
  else
    hipLaunchKernelGGL((apply3_kernel<KM_UA, false, APPLY3_RK, APPLY3_NSTG>), dim3(d_out / PT, d / PT, batch),
                       dim3(256), 0, s, q);
  return hip_check(hipGetLastError(), "apply3_kernel launch");
}

ispa_status_t launch_prod6(int32_t M, int32_t N, int32_t K, int32_t batch, const float* A, const float* B, float* D,
                           void* const asplit[3], void* const bsplit[3], const int32_t* info, hipStream_t s,
                           int max_wg) {
  if (M % PT != 0 || N % PT != 0 || K % PT != 0) {
    set_error("internal: bf16x6 product needs M, N and K multiples of 128");
    return ISPA_E_INVALID_ARG;
  }
  const size_t mk = (size_t)M * K, kn = (size_t)K * N, mn = (size_t)M * N;
  __bf16* Ap[3] = {(__bf16*)asplit[0], (__bf16*)asplit[1], (__bf16*)asplit[2]};
  __bf16* Bp[3] = {(__bf16*)bsplit[0], (__bf16*)bsplit[1], (__bf16*)bsplit[2]};
  hipLaunchKernelGGL(split3_kernel, dim3((unsigned)((mk / 4 + 255) / 256), batch), dim3(256), 0, s, A, mk, Ap[0],
                     Ap[1], Ap[2], info);
  ispa_status_t st = hip_check(hipGetLastError(), "split3_kernel launch");
  if (st != ISPA_OK) return st;
  hipLaunchKernelGGL(split3_t_kernel, dim3(N / SPB, K / SPB, batch), dim3(256), 0, s, B, K, N, Bp[0], Bp[1], Bp[2],
                     info);
  st = hip_check(hipGetLastError(), "split3_t_kernel launch");
  if (st != ISPA_OK) return st;
  Prod6Params p{};
  for (int o = 0; o < 3; ++o) {
    p.A[o] = Ap[o];
    p.B[o] = Bp[o];
  }
  p.D = D;
  p.M = M; p.N = N; p.K = K; p.batch = batch;
  p.sA = mk; p.sB = kn; p.sD = mn;
  p.info = info;
  // 256 x 256 tiles where there are enough of them to spread over the chip
  if (PROD6_WIDE && M % PTW == 0 && N % PTW == 0 && (M / PTW) * (N / PTW) * batch >= 128) {
    const int tiles = (M / PTW) * (N / PTW) * batch;
    if (max_wg > 0 && max_wg < tiles)
      hipLaunchKernelGGL((prod6w_kernel<PROD6W_RK, PROD6W_NSTG>), dim3(max_wg, 1, 1), dim3(512), 0, s, p);
    else
      hipLaunchKernelGGL((prod6w_kernel<PROD6W_RK, PROD6W_NSTG>), dim3(N / PTW, M / PTW, batch), dim3(512), 0, s, p);
    return hip_check(hipGetLastError(), "prod6w_kernel launch");
  }
  const int tiles = (M / PT) * (N / PT) * batch;
  if (max_wg > 0 && max_wg < tiles)
    hipLaunchKernelGGL((prod6_kernel<PROD6_NSTG, PROD6_FLS>), dim3(max_wg, 1, 1), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((prod6_kernel<PROD6_NSTG, PROD6_FLS>), dim3(N / PT, M / PT, batch), dim3(256), 0, s, p);
  return hip_check(hipGetLastError(), "prod6_kernel launch");
}

}  // namespace ispa
