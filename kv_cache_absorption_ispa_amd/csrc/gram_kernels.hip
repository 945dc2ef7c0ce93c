// Gram accumulation for the closed-form absorb on gfx950.
//
// Source: "Technical Summary: Instance-Specific Parametric Absorption (ISPA)
// for Memory-Efficient Video Generation", section 2 "Methodology", step 2
// "Layer Absorb": dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W
// needs only G = A_loc^T A_loc and C = A_loc^T (A_full - A_loc) summed over
// the warmup rows; "Dynamic Layer Selection" ranks layers by the fit's error,
// which also needs E = (A_full - A_loc)^T (A_full - A_loc).
//
// C and E are formed from the difference D = A_full - A_loc itself, as the
// page writes them, not as A_loc^T A_full - A_loc^T A_loc: that form cancels
// when the two streams nearly agree, which is exactly the layers the selection
// converts.  D is exact in float32 (a difference of two bf16 values) and is
// carried to the bf16 matrix cores as D = D_hi + D_lo, both bf16 (D_hi the
// nearest bf16 to D, D_lo the nearest to the remainder): D_hi + D_lo is within
// 2^-17 of D, and C = A_loc^T D_hi + A_loc^T D_lo accumulates in one float32
// accumulator.  E = D_hi^T D_hi + D_hi^T D_lo + D_lo^T D_hi (the D_lo^T D_lo
// term is below 2^-17 of E).
//
// bf16 design (two or three launches per block of rows):
//  * split pass (HBM-bound): D_hi, D_lo [rows, d] into the workspace;
//  * Gram kernel, two passes over the rows.  The C pass owns output tiles of TI x 128 (TI = 256
//    where d allows) and forms C from A_loc[:, I], D_hi[:, J], D_lo[:, J]; the G pass owns the
//    TI x 128 tiles that reach the upper triangle and forms G (and, in a launch of its own, E) from
//    A_loc[:, I], A_loc[:, J] (and D_hi, D_lo of both).  Without E both passes run in one launch.
//    Through a ring of 16-row stages (two or three in flight) the staged matrices go row-major into
//    LDS straight from global memory (buffer loads into LDS, 16-byte chunks XOR-swizzled by row); MFMA operands need
//    8 consecutive rows at one column and come from two transposing LDS reads (ds_read_b64_tr_b16).
//    Four waves own (TI / 2) x 64 sub-tiles (blocks of v_mfma_f32_32x32x16_bf16): each operand
//    fragment read from LDS feeds TI / 32 or 4 MFMAs, and one accumulator set per pass keeps two
//    waves per SIMD.  G and E are stored at and above the diagonal and, from the same registers,
//    at the mirrored positions below it, so both triangles hold the same bits.  Rows are split
//    over workgroups when the tiles alone cannot fill the GPU; every split then stores its
//    partial tile in the workspace, and
//  * a finish kernel adds the partials in split order (bitwise deterministic, no atomics) and
//    mirrors G and E through LDS transposes.
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int GT = 128;  // output tile J extent (and the I extent of the small tile)
constexpr int GBK = 32;  // rows per stage

// Slot of 16-byte chunk c of staged row r: c ^ gram_swizzle(r).  Each 32-lane
// pass of a transposing operand read takes 4 consecutive chunks from each of 4
// consecutive rows; giving those rows different groups of 4 slots keeps the
// read free of bank conflicts (64 four-byte banks, 256-byte rows).
__device__ __forceinline__ int gram_swizzle(int r) { return (r & 3) << 2; }

struct GramParams {
  const uint16_t* A;   // A_loc rows of this block
  const uint16_t* Dh;  // D_hi rows of this block (workspace)
  const uint16_t* Dl;  // D_lo rows of this block (workspace)
  float* G;
  float* C;
  float* E;            // nullable
  float* part;         // split partials: [split][matrix (C, G, E)][d][d] (splits > 1), else NULL
  int64_t n_rows;
  int d;
  int tiles_j;  // output tiles along J (d / 128); C pass tile t is (t / tiles_j, t % tiles_j)
  int tiles_c, tiles_ge;  // tiles of the C pass and of the G (and E) pass
  int64_t rows_per_split;
  int splits;  // row splits (the same for both passes)
  int accumulate;
};

// The kernel runs as two passes over the same rows.
//  * PASS_C: C = A_loc^T D_hi + A_loc^T D_lo on every output tile.  Tiles are TI (256 where d allows,
//    else 128) x 128; a wave owns (TI / 2) x 64, so each operand fragment read from LDS feeds
//    TI / 32 (A side) or 4 (D side) MFMAs, and one accumulator set keeps two waves per SIMD.
//  * PASS_GE: G = A_loc^T A_loc, and E = D_hi^T D_hi + D_hi^T D_lo + D_lo^T D_hi when EV, on the
//    TI x 128 tiles that reach the upper triangle only (listed compactly, row by row), each
//    element above the diagonal also stored at its mirror position.
// Staged matrices of a stage, one after the other, each GBK rows, row-major:
//   PASS_C:  0 A_loc[:, I] (TI)   1 D_hi[:, J]   2 D_lo[:, J]
//   PASS_GE: 0 A_loc[:, I]   1 A_loc[:, J]   (EV: 2 D_hi[:, I]   3 D_lo[:, I]   4 D_hi[:, J]   5 D_lo[:, J])
constexpr int PASS_C = 0, PASS_GE = 1;

template <int PASS, bool EV, int TI_, int SR = GBK>
struct GramShape {
  static constexpr int TI = TI_;
  static constexpr int TJ = GT;
  static constexpr int NM = PASS == PASS_C ? 3 : (EV ? 6 : 2);
  static constexpr int WBI = TI / 64;  // 32-row blocks per wave along I (2 x 2 waves)
  static constexpr int WBJ = TJ / 64;
  __host__ __device__ static constexpr int side(int m) {  // 0: columns I, 1: columns J
    return PASS == PASS_C ? (m == 0 ? 0 : 1) : ((m == 0 || m == 2 || m == 3) ? 0 : 1);
  }
  __host__ __device__ static constexpr int src(int m) {  // 0: A_loc, 1: D_hi, 2: D_lo
    return PASS == PASS_C ? m : (m < 2 ? 0 : ((m == 2 || m == 4) ? 1 : 2));
  }
  __host__ __device__ static constexpr int width(int m) { return side(m) == 0 ? TI : TJ; }
  __host__ __device__ static constexpr int moff(int m) { return m == 0 ? 0 : moff(m - 1) + SR * width(m - 1); }
  static constexpr int SS = moff(NM);  // elements per stage
};

// Tile (ti, tj) of PASS_GE's compact list of TI x 128 tiles that reach the upper triangle: u runs
// row by row; row ti holds the n - r*ti tiles tj >= r*ti (n = d / 128, r = TI / 128).
__device__ __forceinline__ void upper_tile(int u, int n, int r, int& ti, int& tj) {
  int t = 0;
  while (u >= n - r * t) {
    u -= n - r * t;
    ++t;
  }
  ti = t;
  tj = r * t + u;
}

// All 256 threads of a workgroup; NSTG stage buffers of SR rows each in LDS (SR = 32: two buffers;
// SR = 16: a ring of four).
template <int PASS, bool EV, int TI_, int NSTG, int SR = GBK>
__device__ __forceinline__ void gram_pass(const GramParams& p, const int tile, const int split, uint16_t* s0,
                                          uint16_t* s1, uint16_t* s2, uint16_t* s3 = nullptr) {
  static_assert((SR == GBK && NSTG == 2) || (SR == 16 && (NSTG == 3 || NSTG == 4)), "stage shapes");
  using S = GramShape<PASS, EV, TI_, SR>;
  constexpr int TI = S::TI, TJ = S::TJ, NM = S::NM, WBI = S::WBI, WBJ = S::WBJ;
  constexpr int NWV = 4;
  constexpr int NLD = S::SS / 512;  // 1 KB wave loads per stage
  constexpr int WLW = NLD / NWV;    // wave loads per wave per stage
  static_assert(WLW * NWV == NLD, "stage loads must split over the waves");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: buffer choice stays scalar
  const int l32 = lane & 31, hh = lane >> 5;
  int ti, tj;
  if (PASS == PASS_C) {
    ti = tile / p.tiles_j;
    tj = tile % p.tiles_j;
  } else {
    upper_tile(tile, p.d / GT, TI / GT, ti, tj);
  }
  const int I0 = ti * TI, J0 = tj * TJ;
  const int64_t r_begin = (int64_t)split * p.rows_per_split;
  const int64_t r_end = min(p.n_rows, r_begin + p.rows_per_split);
  const int nst = r_end > r_begin ? (int)((r_end - r_begin + SR - 1) / SR) : 0;
  const int wi = (wave >> 1) * (TI / 2), wj = (wave & 1) * (TJ / 2);  // wave sub-tile origin
  const uint32_t row_bytes = (uint32_t)p.d * 2u;
  // Buffers start at this split's first row; rows at or past r_end read as 0 (range-checked
  // buffer loads).  The host keeps (rows per launch + 64) * row_bytes <= 2^31, so the byte offsets
  // of the padding stages (at most 111 rows past the last row) stay far below 2^32.
  const uint32_t span = r_end > r_begin ? (uint32_t)(r_end - r_begin) * row_bytes : 0u;
  const rsrc_t rsc[3] = {make_rsrc(p.A + r_begin * p.d, span), make_rsrc(p.Dh + r_begin * p.d, span),
                         make_rsrc(p.Dl + r_begin * p.d, span)};

  // this wave's stage loads: wave load g = wave + NWV*j is load (g - first load of its matrix) of
  // matrix m: 512 / width rows of it
  uint32_t gofs[WLW];
  int lsrc[WLW], ldst[WLW];
#pragma unroll
  for (int j = 0; j < WLW; ++j) {
    const int g = wave + NWV * j;
    int mtx = 0;
#pragma unroll
    for (int m = 1; m < NM; ++m)
      if (g >= S::moff(m) / 512) mtx = m;
    const int w = S::width(mtx), cpr = w / 8, rpw = 64 / cpr;
    const int li = g - S::moff(mtx) / 512;
    const int rr = li * rpw + lane / cpr;
    const int chunk = (lane % cpr) ^ gram_swizzle(rr);
    const int col0 = S::side(mtx) == 0 ? I0 : J0;
    gofs[j] = (uint32_t)rr * row_bytes + (uint32_t)(col0 + chunk * 8) * 2u;
    lsrc[j] = S::src(mtx);
    ldst[j] = S::moff(mtx) + li * 512;
  }
  auto load_stage = [&](int st, uint16_t* buf) {
    const uint32_t sb = (uint32_t)(st * SR) * row_bytes;
#pragma unroll
    for (int j = 0; j < WLW; ++j) load_to_lds(rsc[lsrc[j]], buf + ldst[j], gofs[j] + sb);
  };

  // Operand for columns xb .. xb+31 of a staged [32 rows][w cols] matrix and rows 16ks .. 16ks+15:
  // lane (column xb + lane%32, hh) gets rows 16ks + 8*(j/4) + 4*hh + j%4, j = 0..7, through two
  // transposing reads (the same row order serves both operands of a product).
  const int q16 = lane >> 4, i16 = lane & 15;
  const int trow = 4 * (q16 >> 1) + (i16 >> 2);  // row within each 8-row half of a 16-row step
  const int tcol = 16 * (q16 & 1) + 4 * (i16 & 3);
  // The swizzle depends on row & 3 == trow & 3, a lane constant, so each operand block has one
  // per-lane base offset; the row step is a compile-time offset.
  int offI[WBI], offJ[WBJ];
#pragma unroll
  for (int x = 0; x < WBI; ++x) {
    const int ci = wi + 32 * x + tcol;
    offI[x] = trow * TI + (((ci >> 3) ^ gram_swizzle(trow)) << 3) + (ci & 7);
  }
#pragma unroll
  for (int x = 0; x < WBJ; ++x) {
    const int cj = wj + 32 * x + tcol;
    offJ[x] = trow * TJ + (((cj >> 3) ^ gram_swizzle(trow)) << 3) + (cj & 7);
  }
  auto frag = [&](const uint16_t* t, int off, int ks, int w) {
    const uint16_t* q = t + off + 16 * ks * w;
    const u32x2 a = lds_read_tr(q), b = lds_read_tr(q + 8 * w);
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
  };

  // PASS_C: acc0 = C; PASS_GE: acc0 = G, acc1 = E
  f32x16 acc0[WBI][WBJ], acc1[WBI][WBJ];
#pragma unroll
  for (int a = 0; a < WBI; ++a)
#pragma unroll
    for (int b = 0; b < WBJ; ++b) {
      acc0[a][b] = f32x16{0};
      acc1[a][b] = f32x16{0};
    }

  // Operand fragments of one 16-row step: PASS_C: A_I (WBI), D_hi,J (WBJ), D_lo,J (WBJ); PASS_GE: A_I,
  // A_J, and with EV D_hi,I, D_lo,I, D_hi,J, D_lo,J.
  constexpr int NF = PASS == PASS_C ? WBI + 2 * WBJ : (EV ? 3 : 1) * (WBI + WBJ);
  using Frags = bf16x8[NF];
  auto read = [&](const uint16_t* buf, int ks, Frags& f) {
#pragma unroll
    for (int a = 0; a < WBI; ++a) f[a] = frag(buf + S::moff(0), offI[a], ks, TI);
    if constexpr (PASS == PASS_C) {
#pragma unroll
      for (int b = 0; b < WBJ; ++b) {
        f[WBI + b] = frag(buf + S::moff(1), offJ[b], ks, TJ);
        f[WBI + WBJ + b] = frag(buf + S::moff(2), offJ[b], ks, TJ);
      }
    } else {
#pragma unroll
      for (int b = 0; b < WBJ; ++b) f[WBI + b] = frag(buf + S::moff(1), offJ[b], ks, TJ);
      if constexpr (EV) {
        constexpr int E0 = WBI + WBJ;
#pragma unroll
        for (int a = 0; a < WBI; ++a) {
          f[E0 + a] = frag(buf + S::moff(2), offI[a], ks, TI);
          f[E0 + WBI + a] = frag(buf + S::moff(3), offI[a], ks, TI);
        }
#pragma unroll
        for (int b = 0; b < WBJ; ++b) {
          f[E0 + 2 * WBI + b] = frag(buf + S::moff(4), offJ[b], ks, TJ);
          f[E0 + 2 * WBI + WBJ + b] = frag(buf + S::moff(5), offJ[b], ks, TJ);
        }
      }
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int a = 0; a < WBI; ++a)
#pragma unroll
      for (int b = 0; b < WBJ; ++b) {
        if constexpr (PASS == PASS_C) {
          acc0[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[a], f[WBI + b], acc0[a][b], 0, 0, 0);
          acc0[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[a], f[WBI + WBJ + b], acc0[a][b], 0, 0, 0);
        } else {
          acc0[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[a], f[WBI + b], acc0[a][b], 0, 0, 0);
        }
      }
    if constexpr (PASS == PASS_GE && EV) {
      constexpr int E0 = WBI + WBJ;
#pragma unroll
      for (int a = 0; a < WBI; ++a)
#pragma unroll
        for (int b = 0; b < WBJ; ++b) {
          const bf16x8 &hI = f[E0 + a], &lI = f[E0 + WBI + a];
          const bf16x8 &hJ = f[E0 + 2 * WBI + b], &lJ = f[E0 + 2 * WBI + WBJ + b];
          acc1[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hI, hJ, acc1[a][b], 0, 0, 0);
          acc1[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hI, lJ, acc1[a][b], 0, 0, 0);
          acc1[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lI, hJ, acc1[a][b], 0, 0, 0);
        }
    }
  };
  auto compute = [&](const uint16_t* buf) {
#pragma unroll
    for (int ks = 0; ks < SR / 16; ++ks) {
      Frags f;
      read(buf, ks, f);
      mma(f);
    }
  };

  // Stages past r_end read as zeros, so the stage count is rounded up to a multiple of NSTG and the
  // loop body (one stage per buffer) has no early exit.  vmcnt counts this wave's loads, which
  // complete in order.
  if constexpr (NSTG == 3) {
    // Ring of three 16-row buffers without the register double buffer (the E pass: its twelve
    // fragments twice over would not fit two waves per SIMD): step st loads stage st + 2 and
    // multiplies stage st, two stages in flight.  At the top of step st each wave waits for its own
    // loads of stage st (all but stage st + 1's); the barrier makes every wave's loads visible and
    // frees the buffer stage st - 1 was read from.
    constexpr int WAIT_CUR = 0xF70 | (WLW & 15) | ((WLW >> 4) << 14);  // vmcnt(WLW)
    uint16_t* const buf[3] = {s0, s1, s2};
    const int nstr = (nst + 2) / 3 * 3;
#pragma unroll
    for (int j = 0; j < 2; ++j) load_stage(j, buf[j]);
    // loads run up to two stages past the last one (rows past r_end read as zeros)
    for (int st = 0; st < nstr; st += 3) {
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WAIT_CUR);
        __builtin_amdgcn_s_barrier();
        load_stage(st + u + 2, buf[(u + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        compute(buf[u]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  } else if constexpr (NSTG == 4) {
    // Ring of four 16-row buffers with the operand fragments double-buffered in registers: step st
    // loads stage st + 3 (three stages in flight), reads stage st + 1's fragments from LDS and
    // multiplies stage st's, read one step earlier, so the products never wait for LDS.  At the top
    // of step st each wave waits for its own loads of stage st + 1 (all but stage st + 2's, which
    // complete after them); the barrier then makes every wave's loads visible, and every wave has
    // multiplied stage st - 1, so the buffer it came from takes the next load.
    constexpr int WAIT_NEXT = 0xF70 | (WLW & 15) | ((WLW >> 4) << 14);      // vmcnt(WLW)
    constexpr int WAIT_FIRST = 0xF70 | ((2 * WLW) & 15) | (((2 * WLW) >> 4) << 14);  // vmcnt(2 WLW)
    uint16_t* const buf[4] = {s0, s1, s2, s3};
    const int nstr = (nst + 3) / 4 * 4;
    // The loads run up to three stages past the last one and the reads one (rows past r_end read as
    // zeros), so every wait has the same count; the last wait drains the loads before the workgroup
    // ends.
#pragma unroll
    for (int j = 0; j < 3; ++j) load_stage(j, buf[j]);
    __builtin_amdgcn_s_waitcnt(WAIT_FIRST);
    __builtin_amdgcn_s_barrier();
    Frags f0, f1;
    read(buf[0], 0, f0);
    for (int st = 0; st < nstr; st += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
        __builtin_amdgcn_s_barrier();
        load_stage(st + u + 3, buf[(u + 3) & 3]);
        __builtin_amdgcn_sched_barrier(0);
        if (u % 2 == 0) {
          read(buf[(u + 1) & 3], 0, f1);
          mma(f0);
        } else {
          read(buf[(u + 1) & 3], 0, f0);
          mma(f1);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    const int nst2 = (nst + 1) / 2 * 2;
    if (nst2 > 0) load_stage(0, s0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int st = 0; st < nst2; st += 2) {
      load_stage(st + 1, s1);
      // keep the next stage's loads ahead of this stage's reads and products: left to itself the
      // scheduler sinks them to just before the wait below, which then waits out their latency
      __builtin_amdgcn_sched_barrier(0);
      compute(s0);
      __builtin_amdgcn_sched_barrier(0);  // and the wait after all of them
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const bool more = st + 2 < nst2;
      if (more) load_stage(st + 2, s0);
      __builtin_amdgcn_sched_barrier(0);
      compute(s1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- epilogue, straight from the accumulators: element v of lane (col, hh) is row
  // 8(v/4) + 4hh + v%4 of its 32 x 32 block, so for each v the 32 lanes of a half-wave cover 32
  // consecutive columns of one row (128-byte stores).  With split rows every split stores its
  // partial tile, and gram_finish_kernel adds the partials in split order and mirrors G and E.
  // Otherwise C is stored everywhere, and G and E at and above the diagonal, each element strictly
  // above it also at its mirror position: lane (col, hh) holds rows 8q + 4hh .. 8q + 4hh + 3 of its
  // column, which are 16 consecutive bytes of row `col` of the lower triangle (the 64 lanes of one
  // store fill 32 bytes of each of 32 rows; the four q fill those rows' 128-byte lines), so both
  // triangles hold the same bits.  Offsets within a d x d matrix fit in 32 bits (d <= 2^15).
  const uint32_t d = (uint32_t)p.d;
  constexpr int NOUT = PASS == PASS_C ? 1 : (EV ? 2 : 1);
#pragma unroll
  for (int o = 0; o < NOUT; ++o) {
    const int m = PASS == PASS_C ? 0 : 1 + o;  // matrix: 0 C, 1 G, 2 E
    float* X;
    if (p.part != nullptr)
      X = p.part + ((size_t)split * 3 + m) * (size_t)d * d;
    else
      X = m == 0 ? p.C : (m == 1 ? p.G : p.E);
    const bool mirror = p.part == nullptr && m > 0;
#pragma unroll
    for (int a = 0; a < WBI; ++a)
#pragma unroll
      for (int b = 0; b < WBJ; ++b) {
        const f32x16& acc = o == 0 ? acc0[a][b] : acc1[a][b];
        const uint32_t c = (uint32_t)(J0 + wj + 32 * b + l32);
        const uint32_t r0 = (uint32_t)(I0 + wi + 32 * a + 4 * hh);
        if (!mirror) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t r = r0 + (uint32_t)(8 * (v >> 2) + (v & 3));
            float* x = X + r * d + c;
            *x = (p.part == nullptr && p.accumulate) ? *x + acc[v] : acc[v];
          }
        } else {
          f32x16 val = acc;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t r = r0 + (uint32_t)(8 * (v >> 2) + (v & 3));
            if (r > c) continue;
            float* x = X + r * d + c;
            if (p.accumulate) val[v] += *x;
            *x = val[v];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t rq = r0 + 8 * q;
            float* y = X + c * d + rq;
            if (rq + 3 < c) {
              *(f32x4*)y = f32x4{val[4 * q], val[4 * q + 1], val[4 * q + 2], val[4 * q + 3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (rq + e < c) y[e] = val[4 * q + e];
            }
          }
        }
        // one block at a time: keeps the loads of the accumulate from being hoisted (and held in
        // registers) across the whole tile
        __builtin_amdgcn_sched_barrier(0);
      }
  }
}

// Completes a Gram call with split rows, per 64 x 64 block (bi, bj) of the output: C = the splits'
// partials added in split order (plus the old C when accumulating), and for bi <= bj the same for
// the elements of G (and E, NMAT = 3) at and above the diagonal, which are then mirrored: element
// (r, c) with r < c is copied to (c, r) through an LDS transpose, so both triangles hold the same
// bits.  A split's loads for all matrices and rows of the thread are issued together, so a block
// waits out one load latency per split rather than one per row and matrix.
template <int NMAT>
__global__ __launch_bounds__(256) void gram_finish_kernel(const float* __restrict__ part, int splits,
                                                          float* __restrict__ C, float* __restrict__ G,
                                                          float* __restrict__ E, int d, int accumulate) {
  __shared__ float T[NMAT - 1][64][65];
  const int bi = blockIdx.y, bj = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t dd = (size_t)d * d;
  const int r_in = tid >> 4, c4 = (tid & 15) * 4;  // thread: rows r_in + 16 k, columns c4 .. c4 + 3
  const bool up = bi <= bj;                        // G and E: the upper blocks carry them
  size_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = (size_t)(bi * 64 + r_in + 16 * k) * d + bj * 64 + c4;
  f32x4 v[NMAT][4];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int k = 0; k < 4; ++k) v[m][k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const float* ps = part + (size_t)s * 3 * dd;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[0][k] += *(const f32x4*)(ps + o[k]);
    if (up) {
#pragma unroll
      for (int m = 1; m < NMAT; ++m)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[m][k] += *(const f32x4*)(ps + m * dd + o[k]);
    }
  }
  if (accumulate) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[0][k] += *(const f32x4*)(C + o[k]);
    if (up) {
#pragma unroll
      for (int m = 1; m < NMAT; ++m)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[m][k] += *(const f32x4*)((m == 1 ? G : E) + o[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) *(f32x4*)(C + o[k]) = v[0][k];
  if (!up) return;
#pragma unroll
  for (int m = 1; m < NMAT; ++m) {
    float* X = m == 1 ? G : E;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = bi * 64 + r_in + 16 * k, c = bj * 64 + c4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (r <= c + e) X[o[k] + e] = v[m][k][e];
        T[m - 1][r_in + 16 * k][c4 + e] = v[m][k][e];
      }
    }
  }
  __syncthreads();
  // transposed: X[bj*64 + rr][bi*64 + cc] = T[cc][rr] for the strictly upper source elements
#pragma unroll
  for (int m = 1; m < NMAT; ++m) {
    float* X = m == 1 ? G : E;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = r_in + 16 * k;  // row of the mirrored block = column of the source
      const int r = bj * 64 + rr;
      const int c = bi * 64 + c4;
      float* x = X + (size_t)r * d + c;
      const f32x4 w = {T[m - 1][c4][rr], T[m - 1][c4 + 1][rr], T[m - 1][c4 + 2][rr], T[m - 1][c4 + 3][rr]};
      if (c + 3 < r) {
        *(f32x4*)x = w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < r) x[e] = w[e];
      }
    }
  }
}

// Stage shape of the Gram passes: a ring of four 16-row stages, else two 32-row stages (the same
// LDS either way).
#ifndef ISPA_GRAM_RING
#define ISPA_GRAM_RING 1
#endif
constexpr int GNS = ISPA_GRAM_RING ? 4 : 2;       // stage buffers
constexpr int GSR = ISPA_GRAM_RING ? 16 : GBK;    // rows per stage
// The E pass (six staged matrices, two accumulator sets): three 16-row stages, two workgroups per CU.
constexpr int GNS_E = ISPA_GRAM_RING ? 3 : 2;

// One Gram pass per launch (grid: tiles x splits): 256 threads (4 waves, 2 x 2), NSTG stage buffers of
// SR rows.
template <int PASS, bool EV, int TI, int NSTG, int SR>
__global__ __launch_bounds__(256, (PASS == PASS_GE && EV && NSTG != 3) ? 1 : 2) void gram_bf16_kernel(GramParams p) {
  constexpr int SS = GramShape<PASS, EV, TI, SR>::SS;
  // the stage buffers as distinct arrays (see the attention kernel: lets the compiler overlap the
  // next stages' loads with this stage's reads)
  __shared__ __attribute__((aligned(1024))) uint16_t s0[SS];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[SS];
  __shared__ __attribute__((aligned(1024))) uint16_t s2[NSTG >= 3 ? SS : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t s3[NSTG >= 4 ? SS : 8];
  gram_pass<PASS, EV, TI, NSTG, SR>(p, blockIdx.x, blockIdx.y, s0, s1, s2, s3);
}

// C and G in one launch (without E): workgroups [0, tiles_c * splits) run the C pass, the rest the G
// pass, so the two fill the GPU together (the G tiles, shorter, come last).
template <int TIC, int TIG>
__global__ __launch_bounds__(256, 2) void gram_cg_kernel(GramParams p) {
  constexpr int SC = GramShape<PASS_C, false, TIC, GSR>::SS, SG = GramShape<PASS_GE, false, TIG, GSR>::SS;
  constexpr int SS = SC > SG ? SC : SG;
  __shared__ __attribute__((aligned(1024))) uint16_t s0[SS];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[SS];
  __shared__ __attribute__((aligned(1024))) uint16_t s2[GNS >= 3 ? SS : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t s3[GNS >= 4 ? SS : 8];
  const int bid = blockIdx.x, nc = p.tiles_c * p.splits;
  if (bid < nc)
    gram_pass<PASS_C, false, TIC, GNS, GSR>(p, bid % p.tiles_c, bid / p.tiles_c, s0, s1, s2, s3);
  else
    gram_pass<PASS_GE, false, TIG, GNS, GSR>(p, (bid - nc) % p.tiles_ge, (bid - nc) / p.tiles_ge, s0, s1, s2, s3);
}

// D = A_full - A_loc (exact in float32) as D_hi = bf16(D), D_lo = bf16(D - D_hi); 8 elements per
// thread (16-byte loads and stores).
__global__ __launch_bounds__(256) void gram_split_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ F,
                                                         uint16_t* Dh, uint16_t* Dl, size_t n8) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const u32x4 a = *(const u32x4*)(A + 8 * i);
  const u32x4 f = *(const u32x4*)(F + 8 * i);
  u32x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float d0 = __builtin_bit_cast(float, f[e] << 16) - __builtin_bit_cast(float, a[e] << 16);
    const float d1 = __builtin_bit_cast(float, f[e] & 0xFFFF0000u) - __builtin_bit_cast(float, a[e] & 0xFFFF0000u);
    const bf16x2 hi = {(__bf16)d0, (__bf16)d1};
    const uint32_t hu = __builtin_bit_cast(uint32_t, hi);
    const float r0 = d0 - __builtin_bit_cast(float, hu << 16);
    const float r1 = d1 - __builtin_bit_cast(float, hu & 0xFFFF0000u);
    const bf16x2 lo = {(__bf16)r0, (__bf16)r1};
    h[e] = hu;
    l[e] = __builtin_bit_cast(uint32_t, lo);
  }
  *(u32x4*)(Dh + 8 * i) = h;
  *(u32x4*)(Dl + 8 * i) = l;
}

// float32 path: 64x64 tile per workgroup, each thread a 4x4 block; rows staged in LDS with the
// difference D = A_full - A_loc formed there (float32).
constexpr int FT = 64;
constexpr int FBK = 32;

__global__ __launch_bounds__(256) void gram_f32_kernel(const float* __restrict__ Al, const float* __restrict__ Af,
                                                       float* G, float* C, float* E, int64_t n_rows, int d,
                                                       int accumulate) {
  __shared__ float sLI[FBK][FT], sLJ[FBK][FT], sDJ[FBK][FT], sDI[FBK][FT];
  const int tpd = d / FT;
  const int ti = blockIdx.x / tpd, tj = blockIdx.x % tpd;
  const int I0 = ti * FT, J0 = tj * FT;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;  // thread block: rows I0+4ty.., cols J0+4tx..
  float g[4][4] = {}, x[4][4] = {}, q[4][4] = {};
  const bool ev = E != nullptr;
  for (int64_t r0 = 0; r0 < n_rows; r0 += FBK) {
    __syncthreads();
    for (int e = tid; e < FBK * FT; e += 256) {
      const int rr = e / FT, cc = e % FT;
      const int64_t r = r0 + rr;
      const bool ok = r < n_rows;
      const float li = ok ? Al[r * d + I0 + cc] : 0.f, lj = ok ? Al[r * d + J0 + cc] : 0.f;
      sLI[rr][cc] = li;
      sLJ[rr][cc] = lj;
      sDJ[rr][cc] = ok ? Af[r * d + J0 + cc] - lj : 0.f;
      sDI[rr][cc] = (ok && ev) ? Af[r * d + I0 + cc] - li : 0.f;
    }
    __syncthreads();
    for (int rr = 0; rr < FBK; ++rr) {
      float li[4], lj[4], dj[4], di[4];
      for (int u = 0; u < 4; ++u) {
        li[u] = sLI[rr][4 * ty + u];
        di[u] = sDI[rr][4 * ty + u];
        lj[u] = sLJ[rr][4 * tx + u];
        dj[u] = sDJ[rr][4 * tx + u];
      }
      for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b) {
          g[a][b] = fmaf(li[a], lj[b], g[a][b]);
          x[a][b] = fmaf(li[a], dj[b], x[a][b]);
          q[a][b] = fmaf(di[a], dj[b], q[a][b]);
        }
    }
  }
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b) {
      const size_t o = (size_t)(I0 + 4 * ty + a) * d + J0 + 4 * tx + b;
      if (accumulate) {
        G[o] += g[a][b];
        C[o] += x[a][b];
        if (ev) E[o] += q[a][b];
      } else {
        G[o] = g[a][b];
        C[o] = x[a][b];
        if (ev) E[o] = q[a][b];
      }
    }
}

// Rows per launch block: the D_hi / D_lo workspace holds one block, and the buffer offsets of a
// launch are 32-bit ((rows + 64) * 2d bytes < 2^31).
int64_t gram_block_rows(int d) {
  int64_t r = ((int64_t)1 << 31) / (2 * (int64_t)d) - 2 * GBK;
  r = std::min<int64_t>(r, 32768);
  return (r / GBK) * GBK;
}

// I extent of the C pass's output tile: 256 where d allows it (a wave then owns 128 x 64), else 128.
// Without E at d <= 2048 the 128 tiles are twice as many, so fewer row splits fill the GPU and the
// finish adds fewer partials (d = 1536: 222 tiles in 3 splits at three workgroups per CU, 79 us per
// 4680-row chunk, against 84 in 2 splits and 90 with 256 tiles; with E the 256 tiles stay ahead,
// 139 against 159 us).
int gram_ti(int d, bool ev) { return (d % 256 == 0 && (ev || d > 2048)) ? 256 : 128; }

int gram_tiles_c(int d, bool ev) { return (d / gram_ti(d, ev)) * (d / GT); }
// TI x 128 tiles that reach the upper triangle (G and E pass): sum over I rows of n - r * ti
int gram_tiles_ge(int d, int ti) {
  const int n = d / GT, r = ti / GT;
  int t = 0;
  for (int i = 0; i < d / ti; ++i) t += n - r * i;
  return t;
}
int gram_ti_ge(int d, bool ev) { return (!ev && d % 256 == 0 && d > 2048) ? 256 : 128; }

#ifndef ISPA_GRAM_SLOTS128
#define ISPA_GRAM_SLOTS128 768
#endif
// Workgroups of one launch resident at once: two per CU, three for the 128-tile kernel without E
// (136 VGPRs, 48 KB of LDS).
int gram_slots(int d, bool ev) { return (!ev && gram_ti(d, ev) == 128 && gram_ti_ge(d, ev) == 128) ? ISPA_GRAM_SLOTS128 : 512; }

int gram_splits(int64_t n_rows, int tiles, int slots) {
  // the most splits that still fit one round of resident workgroups, at least 256 rows per split,
  // at most 8
  int s = tiles >= slots ? 1 : slots / tiles;
  const int64_t max_s = std::max<int64_t>(1, n_rows / 256);
  if (s > max_s) s = (int)max_s;
  if (s > 8) s = 8;
  if (s < 1) s = 1;
  return s;
}

struct GramWs {
  size_t dsplit, dbytes, parts, total;  // byte offsets / sizes
};

// Workspace: D_hi and D_lo of one block of rows and the split partials ([split][C, G, E][d][d]) of
// the pass with the most splits.
GramWs gram_ws_layout(int64_t n_rows, int d) {
  GramWs w;
  const int64_t rows = std::max<int64_t>(std::min(n_rows, gram_block_rows(d)), 0);
  w.dbytes = ((size_t)rows * d * 2 + 255) & ~(size_t)255;
  w.dsplit = 0;
  const int64_t r1 = std::max<int64_t>(rows, 1);
  const int s = std::max(gram_splits(r1, gram_tiles_c(d, false) + gram_tiles_ge(d, gram_ti_ge(d, false)), gram_slots(d, false)),
                         gram_splits(r1, gram_tiles_c(d, true) + gram_tiles_ge(d, gram_ti_ge(d, true)), gram_slots(d, true)));
  const size_t part_bytes = s > 1 ? (size_t)s * 3 * (size_t)d * d * sizeof(float) : 0;
  w.parts = 2 * w.dbytes;
  w.total = w.parts + part_bytes;
  return w;
}

}  // namespace

size_t gram_workspace_size(int64_t n_rows, int32_t d, int32_t dtype) {
  if (dtype != ISPA_BF16 || d % GT != 0 || n_rows <= 0) return 0;
  return gram_ws_layout(n_rows, d).total;
}

ispa_status_t launch_gram(int64_t n_rows, int32_t d, int32_t dtype, const void* A_loc, const void* A_full,
                          float* G, float* C, float* E, int32_t accumulate, void* ws, size_t ws_bytes,
                          hipStream_t s) {
  if (dtype == ISPA_F32 || d % GT != 0) {
    if (dtype != ISPA_F32) {
      set_error("bf16 Gram needs d to be a multiple of 128");
      return ISPA_E_INVALID_ARG;
    }
    const int tpd = d / FT;
    hipLaunchKernelGGL(gram_f32_kernel, dim3(tpd * tpd), dim3(256), 0, s, (const float*)A_loc,
                       (const float*)A_full, G, C, E, n_rows, d, accumulate);
    return hip_check(hipGetLastError(), "gram_f32_kernel launch");
  }
  if (n_rows == 0 && accumulate) return ISPA_OK;  // nothing to add
  const size_t need = gram_workspace_size(n_rows, d, dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) {
    set_error("ispa_gram_accum: workspace too small");
    return ISPA_E_WORKSPACE;
  }
  const GramWs lay = gram_ws_layout(n_rows, d);
  const int ti = gram_ti(d, E != nullptr);
  const int ti_ge = gram_ti_ge(d, E != nullptr);
  const int tiles_c = gram_tiles_c(d, E != nullptr), tiles_ge = gram_tiles_ge(d, ti_ge);
  // Rows go in blocks (the D_hi / D_lo workspace holds one); later blocks accumulate.
  const int64_t block_rows = gram_block_rows(d);
  int64_t r0 = 0;
  do {
    const int64_t nr = std::min(block_rows, n_rows - r0);
    const int acc = (r0 > 0) ? 1 : accumulate;
    const int64_t nr1 = std::max<int64_t>(nr, 1);
    const int splits = gram_splits(nr1, tiles_c + tiles_ge, gram_slots(d, E != nullptr));
    GramParams p;
    p.A = (const uint16_t*)A_loc + r0 * d;
    p.Dh = (const uint16_t*)((char*)ws + lay.dsplit);
    p.Dl = (const uint16_t*)((char*)ws + lay.dsplit + lay.dbytes);
    p.G = G;
    p.C = C;
    p.E = E;
    p.n_rows = nr;
    p.d = d;
    p.tiles_j = d / GT;
    p.tiles_c = tiles_c;
    p.tiles_ge = tiles_ge;
    p.accumulate = acc;
    p.splits = splits;
    p.part = splits > 1 ? (float*)((char*)ws + lay.parts) : nullptr;
    const int64_t per = (nr + splits - 1) / splits;
    p.rows_per_split = std::max<int64_t>(((per + GBK - 1) / GBK) * GBK, GBK);
    const size_t n8 = (size_t)nr * d / 8;
    if (nr > 0) {  // (no rows: no workspace; one split writes zeros)
      hipLaunchKernelGGL(gram_split_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                         (const uint16_t*)A_loc + r0 * d, (const uint16_t*)A_full + r0 * d, (uint16_t*)p.Dh,
                         (uint16_t*)p.Dl, n8);
      ispa_status_t st = hip_check(hipGetLastError(), "gram_split_kernel launch");
      if (st != ISPA_OK) return st;
    }
    if (E) {
      // E needs six staged matrices: its pass runs on its own (one workgroup per CU), after C's
      if (ti == 256)
        hipLaunchKernelGGL((gram_bf16_kernel<PASS_C, false, 256, GNS, GSR>), dim3(tiles_c, splits), dim3(256), 0, s, p);
      else
        hipLaunchKernelGGL((gram_bf16_kernel<PASS_C, false, 128, GNS, GSR>), dim3(tiles_c, splits), dim3(256), 0, s, p);
      ispa_status_t st = hip_check(hipGetLastError(), "gram_bf16_kernel launch (C)");
      if (st != ISPA_OK) return st;
      hipLaunchKernelGGL((gram_bf16_kernel<PASS_GE, true, GT, GNS_E, GSR>), dim3(tiles_ge, splits), dim3(256), 0, s, p);
    } else {
      const dim3 grid((unsigned)((tiles_c + tiles_ge) * splits));
      if (ti == 256 && ti_ge == 256)
        hipLaunchKernelGGL((gram_cg_kernel<256, 256>), grid, dim3(256), 0, s, p);
      else
        hipLaunchKernelGGL((gram_cg_kernel<128, 128>), grid, dim3(256), 0, s, p);
    }
    ispa_status_t st = hip_check(hipGetLastError(), "gram_bf16_kernel launch");
    if (st != ISPA_OK) return st;
    if (splits > 1) {  // (one split: the passes stored the final C, G and E, both triangles)
      const float* part = (const float*)((char*)ws + lay.parts);
      if (E)
        hipLaunchKernelGGL(gram_finish_kernel<3>, dim3(d / 64, d / 64), dim3(256), 0, s, part, splits, C, G, E, d, acc);
      else
        hipLaunchKernelGGL(gram_finish_kernel<2>, dim3(d / 64, d / 64), dim3(256), 0, s, part, splits, C, G, E, d, acc);
      st = hip_check(hipGetLastError(), "gram_finish_kernel launch");
      if (st != ISPA_OK) return st;
    }
    r0 += nr;
  } while (r0 < n_rows);
  return ISPA_OK;
}

}  // namespace ispa
