// Decomposable attention on gfx950: local branch, history branch and their
// log-sum-exp merge in one launch; plus the single-pass comparison attention
// and a standalone N-way merge.
//
// Source: "Technical Summary: Instance-Specific Parametric Absorption (ISPA)
// for Memory-Efficient Video Generation", section 2 "Methodology", step 1
// "Dual-Stream Warmup" (local stream = sink + current chunk, full stream =
// entire context, decomposed into local and historical branches that keep
// log-sum-exp states and are fused afterwards) and section 3 (online softmax).
//
// bf16 kernel design (one workgroup = NW waves, one head, NW*32 queries, BN-key tiles):
//  * Each wave owns 32 queries and computes S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16, so a lane holds scores of ONE query (column
//    lane%32) for 16 keys: the softmax row max and row sum are in-lane, plus
//    one exchange between the two 32-lane halves.
//  * O^T = V^T P^T accumulates on the same MFMA; P goes from the score
//    accumulator straight into the B operand (no LDS round trip).  The V^T
//    operand comes from the row-major V tile through transposing LDS reads
//    (ds_read_b64_tr_b16).
//  * K and V tiles of BN keys are double-buffered in LDS and filled straight
//    from global memory by buffer loads into LDS, issued before the current
//    tile's MFMAs; 16-byte chunks are permuted per row so that the K reads and
//    the transposing V reads are free of bank conflicts.
//  * Local tiles then history tiles form one tile sequence (the pipeline does
//    not drain at the branch switch).  At the switch the local branch is
//    normalised and written (O_loc, LSE_loc); its float32 values go to the
//    caller's workspace (each lane later reads back exactly what it wrote, so
//    no synchronisation is needed).  After the last history tile the merge
//    runs in registers from the float32 O_loc and O_full is rounded once.
//  * Scores are scaled by scale*log2(e) and exponentiated with v_exp_f32
//    (2^x); LSE is exported in natural log.
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct AttnKParams {
  const uint16_t* Q;
  // key segments: tiles st0[s] .. st0[s+1]-1 of the tile sequence come from segment s (n[s] rows);
  // segments [0, n_loc_seg) are the local branch
  const uint16_t* Ks[MAX_KV_SEGS];
  const uint16_t* Vs[MAX_KV_SEGS];
  int sn[MAX_KV_SEGS];
  int st0[MAX_KV_SEGS + 1];
  int n_seg, n_loc_seg;
  uint16_t* O_loc;
  float* LSE_loc;
  uint16_t* O_hist;
  float* LSE_hist;
  uint16_t* O_full;
  float* LSE_full;
  float* stash;  // float32 O_loc kept for the merge ([n_q, H, D]); used when O_full and history exist
  int n_q, heads;
  float c2;  // scale * log2(e)
  int n_qtiles, nblocks;
  // split mode: unit u's key tiles are cut into sk_p equal pieces, piece i on its own workgroup,
  // which leaves its branch states in partial slot u * sk_p + i
  int sk_p;
  float* part;
  // fp8 keys (KF8 kernels): Q and the K segments hold E4M3 codes, score scale per head and segment
  // c2 * q_scale[head] * k_scale[segment][head]
  const float* q_scale;
  const float* k_scale[MAX_KV_SEGS];
};

// Split-mode schedule.  Workgroup b runs on XCD b % 8 (round-robin dispatch).  The units are
// dealt to the XCDs in contiguous blocks; on an XCD with n units, workgroup slot j takes piece
// j / n of unit j % n, so the workgroups reading the same key range of a head sit on one XCD and
// march through it together (shared L2), as the unsplit launch does.  Pure function of (b,
// number of workgroups, units, pieces), shared with the host.
__host__ __device__ inline void sk_xcd_counts(int x, int n_wg, int n_units, int& wx, int& nx, int& bx) {
  wx = n_wg / 8 + (x < n_wg % 8 ? 1 : 0);
  nx = n_units / 8 + (x < n_units % 8 ? 1 : 0);
  bx = x * (n_units / 8) + (x < n_units % 8 ? x : n_units % 8);
}
// Pieces per unit: the most every XCD can give each of its units (1 = no split), at most T.
__host__ __device__ inline int sk_pieces(int n_wg, int n_units, int T) {
  int pc = T;
  for (int x = 0; x < 8; ++x) {
    int wx, nx, bx;
    sk_xcd_counts(x, n_wg, n_units, wx, nx, bx);
    if (nx > 0) pc = wx / nx < pc ? wx / nx : pc;
  }
  return pc < 1 ? 1 : pc;
}
// Key tiles [t0, t1) of piece i of P.
__host__ __device__ inline void sk_piece_range(int i, int P, int T, int& t0, int& t1) {
  t0 = (int)((int64_t)i * T / P);
  t1 = (int)((int64_t)(i + 1) * T / P);
}

// Partial slot: float32 O for the local and the history branch ([2][BM][D]), then their
// log2-domain LSEs ([2][BM]).
__host__ __device__ constexpr size_t part_slot_floats(int bm, int d) { return (size_t)2 * bm * d + 2 * bm; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by the lane 32 away (the other half of the wave), via v_permlane32_swap.
__device__ __forceinline__ float other_half(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Slot of 16-byte chunk c of tile row r in LDS: c ^ kv_swizzle<D>(r).  The LDS has
// 64 four-byte banks (256 bytes per cycle).  The K operand reads take one
// chunk from each of 16 consecutive rows per 16-lane pass, and the
// transposing V reads take 4 consecutive chunks from each of 4 consecutive
// rows per 32-lane pass; a plain XOR with (r & 7) would leave both 2-way and
// 4-way bank conflicts.  XOR-ing with a bit rotation of the row's low bits
// puts the 16 rows of a K pass on 16 different slots, and the 4 rows of a V
// pass on 4 different groups of 4 slots, so both read patterns are
// conflict-free.  (D = 64: rows are 128 bytes, two rows per bank cycle.)
// fp8 K rows (D bytes): slot of 16-byte chunk c of row r is c ^ kf8_swizzle<D>(r); the 16 rows of a
// read pass (one chunk each) then cover all 64 banks.
template <int D>
__device__ __forceinline__ int kf8_swizzle(int r) {
  if constexpr (D == 128) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

template <int D>
__device__ __forceinline__ int kv_swizzle(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// QB = 32-query blocks per wave (1: 32 queries per wave; 2: 64 queries, one wave per SIMD).
//
// K and V tiles (BN keys x D) are kept row-major in LDS, each row's 16-byte
// chunks permuted by kv_swizzle so that both the K operand reads and the
// transposing V reads are free of bank conflicts.  They are filled straight from global memory by buffer loads into LDS
// (a wave moves 1 KB per load), so tile staging costs no VGPRs and no LDS
// store instructions; rows past the branch's end read as 0 (range-checked).
//
// SK = split mode: the grid is a fixed set of workgroups (one per CU) that
// share the units' tiles evenly, so no CU idles when the units do not fill the
// last wave of workgroups; pieces of split units are merged afterwards (sk_fixup_kernel).
//
// KF8 = fp8 keys: Q and K are E4M3 codes and S^T = K Q^T runs on
// v_mfma_f32_32x32x64_f8f6f4 (twice the bf16 rate, half the K bytes); the
// softmax, P and V stay as in the bf16 kernel.
template <int D, int NW, int QB, int BN, bool SK, bool KF8 = false>
__global__ __launch_bounds__(NW * 64, (QB == 1 && NW <= 4) ? 2 : 1) void attn_bf16_kernel(AttnKParams p) {
  constexpr int KK = KF8 ? D / 64 : D / 16;  // MFMA k-steps of S^T
  constexpr int DB = D / 32;                  // 32-row blocks of O^T
  constexpr int NKB = BN / 32;
  constexpr int CPR = D / 8;                  // 16-byte chunks per V row
  constexpr int RPW = 64 / CPR;               // V rows per wave load (1 KB)
  constexpr int WLT = BN / RPW;               // wave loads per V tile
  constexpr int KRB = KF8 ? D : 2 * D;        // bytes per K row in LDS
  constexpr int CPRK = KRB / 16;              // 16-byte chunks per K row
  constexpr int RPWK = 64 / CPRK;             // K rows per wave load
  constexpr int WLTK = BN / RPWK;             // wave loads per K tile
  constexpr int WLW = (WLTK + WLT) / NW;      // wave loads per wave per tile (K and V)
  static_assert(WLW * NW == WLTK + WLT, "tile loads must split evenly over the waves");
  using QFrag = typename std::conditional<KF8, v8i_t, bf16x8>::type;
  constexpr int BM = NW * 32 * QB;
  // The running max used as the exponent reference is raised only when a new
  // score exceeds it by more than 2^8: p then stays below 2^8, and the
  // accumulator rescale (D multiplies per query) is skipped on most tiles.
  constexpr float RESCALE_T = 8.0f;

  // Two buffers as four distinct arrays, addressed only with compile-time
  // buffer choices, so the compiler can tell the loads landing in one buffer
  // from the reads of the other and does not wait for the prefetch early.
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: load targets stay scalar
  const int l32 = lane & 31, hh = lane >> 5;
  const int n_q = p.n_q;
  const uint32_t HD = (uint32_t)p.heads * D;
  const uint32_t row_bytes = HD * 2u;            // V (and bf16 K) row in memory
  const uint32_t krow_bytes = KF8 ? HD : HD * 2u;  // K row in memory
  const int Tl = p.st0[p.n_loc_seg];  // local tiles, then history tiles
  const int T = p.st0[p.n_seg];
  const int Th = T - Tl;

  // One piece: tiles [t0, t1) of unit `unit` (all of them outside split mode).
  auto piece = [&](const int unit, const int t0, const int t1, float* slot) {
  const bool whole = !SK || (t0 == 0 && t1 == T);
  const int head = unit / p.n_qtiles, qt = unit % p.n_qtiles;
  // Tiles are visited in order, so the loads and the compute each keep a cursor
  // (segment, tile within it) in scalar registers; the segment table is read
  // only when a cursor crosses into the next segment (a scalar-memory read
  // per tile would make every tile wait on it together with its LDS reads).
  struct Cur {
    int sg, tt, nt, n;
    const uint16_t* kb;
    const uint16_t* vb;
    float c2;  // score scale of the segment (log2 domain)
  };
  const float c2h = KF8 ? p.c2 * p.q_scale[head] : p.c2;
  auto cur_at = [&](int sg) {
    Cur c;
    c.sg = sg;
    c.tt = 0;
    c.n = p.sn[sg];
    c.nt = (c.n + BN - 1) / BN;
    c.kb = p.Ks[sg];
    c.vb = p.Vs[sg];
    c.c2 = KF8 ? c2h * p.k_scale[sg][head] : c2h;
    return c;
  };
  auto cur_next = [&](Cur& c) {
    if (++c.tt == c.nt && c.sg + 1 < p.n_seg) c = cur_at(c.sg + 1);
  };
  int sg0 = 0;
  if (t0 > 0)
    while (sg0 + 1 < p.n_seg && p.st0[sg0 + 1] <= t0) ++sg0;
  Cur lcur = cur_at(sg0);
  lcur.tt = t0 - p.st0[sg0];
  Cur ccur = lcur;

  int myq[QB];
  bool qvalid[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    myq[qb] = qt * BM + wave * 32 * QB + qb * 32 + l32;
    qvalid[qb] = myq[qb] < n_q;
  }

  // Q^T fragments (B operand of S^T = K Q^T).  bf16: lane holds q[myq][16kk + 8hh .. +7];
  // fp8: codes q[myq][64kk + 32hh .. +31] (K fragments use the same dims, so the k order matches).
  QFrag qf[QB][KK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if constexpr (KF8) {
      const uint8_t* qp = (const uint8_t*)p.Q + (size_t)(qvalid[qb] ? myq[qb] : 0) * HD + head * D + 32 * hh;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 a = qvalid[qb] ? *(const u32x4*)(qp + 64 * kk) : u32x4{0, 0, 0, 0};
        const u32x4 b = qvalid[qb] ? *(const u32x4*)(qp + 64 * kk + 16) : u32x4{0, 0, 0, 0};
        qf[qb][kk] = v8i_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
      }
    } else {
      const uint16_t* qp = p.Q + (size_t)(qvalid[qb] ? myq[qb] : 0) * HD + head * D + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 v = qvalid[qb] ? *(const u32x4*)(qp + 16 * kk) : u32x4{0, 0, 0, 0};
        qf[qb][kk] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  // This wave's tile loads: load j is wave load g = wave + j*NW of the tile (K loads first, then V).
  // Lane i fills row r0 + i/CPR(K), slot i%CPR(K), with the row's chunk slot ^ swizzle(row).
  // When NW divides the K loads, load j is a K load exactly when j < WLTK/NW (wave < NW): a
  // compile-time choice, so no per-load condition is kept in scalar registers.
  auto is_kload = [&](int j) { return WLTK % NW == 0 ? j < WLTK / NW : wave + j * NW < WLTK; };
  uint32_t gofs[WLW];
#pragma unroll
  for (int j = 0; j < WLW; ++j) {
    const int g = wave + j * NW;
    if (is_kload(j)) {
      const int row = g * RPWK + lane / CPRK;
      const int chunk = (lane % CPRK) ^ (KF8 ? kf8_swizzle<D>(row) : kv_swizzle<D>(row));
      gofs[j] = (uint32_t)row * krow_bytes + (uint32_t)(head * D) * (KF8 ? 1u : 2u) + chunk * 16u;
    } else {
      const int row = (g - WLTK) * RPW + lane / CPR;
      const int chunk = (lane % CPR) ^ kv_swizzle<D>(row);
      gofs[j] = (uint32_t)row * row_bytes + (uint32_t)(head * D + chunk * 8) * 2u;
    }
  }

  auto load_tile = [&](uint16_t* sKb, uint16_t* sVb) {
    const uint32_t tbk = (uint32_t)(lcur.tt * BN) * krow_bytes;
    const uint32_t tb = (uint32_t)(lcur.tt * BN) * row_bytes;
    const rsrc_t rk = make_rsrc(lcur.kb, (uint32_t)lcur.n * krow_bytes);
    const rsrc_t rv = make_rsrc(lcur.vb, (uint32_t)lcur.n * row_bytes);
    cur_next(lcur);
#pragma unroll
    for (int j = 0; j < WLW; ++j) {
      const int g = wave + j * NW;
      if (is_kload(j))
        load_to_lds(rk, (uint16_t*)((uint8_t*)sKb + g * RPWK * KRB), gofs[j] + tbk);
      else
        load_to_lds(rv, sVb + (g - WLTK) * RPW * D, gofs[j] + tb);
    }
  };

  // Online-softmax state per query block (log2 domain): reference max m, sum l, accumulator.
  f32x16 acc[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{0};
  }

  // LDS fragment reads run two ahead of the MFMAs that consume them
  // (sched_barrier keeps the compiler from sinking them next to their use).
  constexpr int NS = NKB * KK;      // K fragments per tile: (kb, kk), chains of the NKB accumulators interleaved
  constexpr int NV = DB * NKB * 2;  // V fragments per tile: (db, kb, mm), DB accumulators interleaved
  // K operand: row kb*32 + l32; bf16: chunk 2kk + hh; fp8: chunks 4kk + 2hh and 4kk + 2hh + 1
  // (the swizzles depend on row & 15 == l32 & 15).
  const int ksw = KF8 ? kf8_swizzle<D>(l32) : kv_swizzle<D>(l32);
  auto kfrag = [&](const uint16_t* sKb, int i) {
    const int kb = i % NKB, kk = i / NKB;
    const int row = kb * 32 + l32;
    if constexpr (KF8) {
      const uint8_t* rp = (const uint8_t*)sKb + row * KRB;
      const u32x4 a = *(const u32x4*)(rp + (((4 * kk + 2 * hh) ^ ksw) << 4));
      const u32x4 b = *(const u32x4*)(rp + (((4 * kk + 2 * hh + 1) ^ ksw) << 4));
      return v8i_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    } else {
      return __builtin_bit_cast(bf16x8, *(const u32x4*)(&sKb[row * D + (((2 * kk + hh) ^ ksw) << 3)]));
    }
  };
  // V^T operand of O^T = V^T P^T for lane (dim 32db + lane%32, hh): keys 32kb + 16mm + 4hh + {0..3}
  // and + 8 + {0..3} (the key order of the P accumulator), read with two transposing loads.
  // As a source lane, lane i of its 16-lane group points at key (4hh + i/4) and dims dbase + 4*(i%4).
  const int q16 = lane >> 4, i16 = lane & 15;
  const int vdim = 16 * (q16 & 1) + 4 * (i16 & 3);  // dim offset within the 32-dim block
  const int vkey = 4 * (q16 >> 1) + (i16 >> 2);     // key offset within the 16-key step
  const int vsw_a = kv_swizzle<D>(vkey), vsw_b = kv_swizzle<D>(vkey + 8);  // keys are vkey (+8) mod 16
  auto vfrag = [&](const uint16_t* sVb, int i) {
    const int db = i % DB, j = i / DB, kb = j / 2, mm = j % 2;
    const int d0 = 32 * db + vdim;
    const int key_a = 32 * kb + 16 * mm + vkey, key_b = key_a + 8;
    const uint16_t* pa = &sVb[key_a * D + (((d0 >> 3) ^ vsw_a) << 3) + (d0 & 7)];
    const uint16_t* pb = &sVb[key_b * D + (((d0 >> 3) ^ vsw_b) << 3) + (d0 & 7)];
    const u32x2 a = lds_read_tr(pa), b = lds_read_tr(pb);
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
  };

  auto compute_tile = [&](const uint16_t* sKb, const uint16_t* sVb) {
    const int key0 = ccur.tt * BN;
    const int nvalid = ccur.n;
    const float c2 = ccur.c2;
    cur_next(ccur);
    f32x16 s[QB][NKB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = f32x16{0};
    QFrag kf[3];
    kf[0] = kfrag(sKb, 0);
    kf[1] = kfrag(sKb, 1);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + 2 < NS) kf[(i + 2) % 3] = kfrag(sKb, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int kb = i % NKB, kk = i / NKB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (KF8)
          s[qb][kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[i % 3], qf[qb][kk], s[qb][kb], 0, 0, 0, 0,
                                                                      0, 0);
        else
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % 3], qf[qb][kk], s[qb][kb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first V fragments do not depend on P: start reading them before the softmax
    bf16x8 vf[3];
    vf[0] = vfrag(sVb, 0);
    vf[1] = vfrag(sVb, 1);
    // Accumulator element v of lane (query, hh) in key block kb is key
    // kb*32 + 8*(v/4) + 4*hh + v%4.  Mask keys past the branch's end.
    if (key0 + BN > nvalid) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key0 + kb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (key >= nvalid) s[qb][kb][v] = -INFINITY;
        }
    }
    u32x4 pk[QB][NKB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // row max as a tree (the halves' partial maxima are exchanged once)
      float mt[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) mt[r] = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mt[v & 3] = fmaxf(mt[v & 3], s[qb][kb][v]);
      float mx = fmaxf(fmaxf(mt[0], mt[1]), fmaxf(mt[2], mt[3]));
      mx = fmaxf(mx, other_half(mx)) * c2;
      if (__builtin_amdgcn_ballot_w64(mx > m[qb] + RESCALE_T) != 0) {
        const float mnew = fmaxf(m[qb], mx);
        const float alpha = fast_exp2(m[qb] - mnew);
        m[qb] = mnew;
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
      }
      const float mref = m[qb];
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const float p0 = fast_exp2(fmaf(s[qb][kb][8 * mm + j], c2, -mref));
            const float p1 = fast_exp2(fmaf(s[qb][kb][8 * mm + j + 1], c2, -mref));
            ls[j >> 1] += p0 + p1;
            const bf16x2 b = {(__bf16)p0, (__bf16)p1};
            w[j >> 1] = __builtin_bit_cast(uint32_t, b);
          }
          pk[qb][kb][mm] = u32x4{w[0], w[1], w[2], w[3]};
        }
      l[qb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i + 2 < NV) vf[(i + 2) % 3] = vfrag(sVb, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int db = i % DB, j = i / DB, kb = j / 2, mm = j % 2;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % 3], __builtin_bit_cast(bf16x8, pk[qb][kb][mm]),
                                                              acc[qb][db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // O^T accumulator element v of lane (query, hh) in block db is dim 32db + 8(v/4) + 4hh + v%4.
  auto write_o = [&](uint16_t* O, int qb, const u32x2 (&vals)[DB][4]) {
    if (O == nullptr || !qvalid[qb]) return;
    uint16_t* op = O + (size_t)myq[qb] * HD + head * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) *(u32x2*)(op + 32 * db + 8 * g) = vals[db][g];
  };
  auto pack_acc = [&](u32x2 (&out)[DB][4], int qb, float scale_by) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2 a = {(__bf16)(acc[qb][db][4 * g] * scale_by), (__bf16)(acc[qb][db][4 * g + 1] * scale_by)};
        const bf16x2 b = {(__bf16)(acc[qb][db][4 * g + 2] * scale_by), (__bf16)(acc[qb][db][4 * g + 3] * scale_by)};
        out[db][g] = u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
      }
  };
  auto lse_store = [&](float* L, int qb, float v2) {
    if (L && hh == 0 && qvalid[qb]) L[(size_t)head * n_q + myq[qb]] = v2 * LN2;
  };

  // a branch's part of a split unit: normalised float32 O and log2 LSE into the partial slot
  auto write_part = [&](int br, int qb, float inv, float lse2) {
    const int row = wave * 32 * QB + qb * 32 + l32;
    float* op = slot + ((size_t)br * BM + row) * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(op + 32 * db + 8 * g) = f32x4{acc[qb][db][4 * g] * inv, acc[qb][db][4 * g + 1] * inv,
                                                 acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv};
    if (hh == 0) slot[(size_t)2 * BM * D + br * BM + row] = lse2;
  };

  float lse2_loc[QB];
  // local branch done: normalise, write O_loc / LSE_loc, keep float32 O_loc for the merge
  auto end_of_local = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = l[qb] + other_half(l[qb]);
      const float inv = 1.0f / lt;
      lse2_loc[qb] = m[qb] + __log2f(lt);
      if (!whole) {
        write_part(0, qb, inv, lse2_loc[qb]);
        m[qb] = -INFINITY;
        l[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{0};
        continue;
      }
      u32x2 oloc[DB][4];
      pack_acc(oloc, qb, inv);
      write_o(p.O_loc, qb, oloc);
      lse_store(p.LSE_loc, qb, lse2_loc[qb]);
      if (Th == 0) {
        // local-attention mode: the full output is the local one, bit for bit
        write_o(p.O_full, qb, oloc);
        lse_store(p.LSE_full, qb, lse2_loc[qb]);
      } else if (p.O_full && qvalid[qb]) {
        float* stash = p.stash + (size_t)myq[qb] * HD + head * D + 4 * hh;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(f32x4*)(stash + 32 * db + 8 * g) = f32x4{acc[qb][db][4 * g] * inv, acc[qb][db][4 * g + 1] * inv,
                                                       acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv};
      }
      m[qb] = -INFINITY;
      l[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{0};
    }
  };

  load_tile(sK0, sV0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = t0; t < t1; t += 2) {
    // even tile in buffer 0, odd tile in buffer 1; the next tile's loads are in flight meanwhile
    if (t + 1 < t1) load_tile(sK1, sV1);
    compute_tile(sK0, sV0);
    if (t == Tl - 1) end_of_local();
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile t+1 have landed in LDS
    __syncthreads();
    if (t + 1 >= t1) break;
    if (t + 2 < t1) load_tile(sK0, sV0);
    compute_tile(sK1, sV1);
    if (t + 1 == Tl - 1) end_of_local();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (!whole) {
    // the branch this piece of a split unit ends in: the history, or the local branch when the
    // piece stops before the local tiles end (t1 == Tl: end_of_local already wrote it)
    if (t1 != Tl) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float lt = l[qb] + other_half(l[qb]);
        write_part(t1 > Tl ? 1 : 0, qb, 1.0f / lt, m[qb] + __log2f(lt));
      }
    }
    return;
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (Th > 0) {
      const float lt = l[qb] + other_half(l[qb]);
      const float inv = 1.0f / lt;
      const float lse2_hist = m[qb] + __log2f(lt);
      if (p.O_hist) {
        u32x2 oh[DB][4];
        pack_acc(oh, qb, inv);
        write_o(p.O_hist, qb, oh);
      }
      lse_store(p.LSE_hist, qb, lse2_hist);
      // merge: LSE = logaddexp(LSE_loc, LSE_hist); O = w_loc O_loc + w_hist O_hist
      const float mx = fmaxf(lse2_loc[qb], lse2_hist);
      const float lse2 = mx + __log2f(fast_exp2(lse2_loc[qb] - mx) + fast_exp2(lse2_hist - mx));
      const float wl = fast_exp2(lse2_loc[qb] - lse2);
      const float wh = fast_exp2(lse2_hist - lse2) * inv;
      if (p.O_full && qvalid[qb]) {
        const float* stash = p.stash + (size_t)myq[qb] * HD + head * D + 4 * hh;
        u32x2 of[DB][4];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 ol = *(const f32x4*)(stash + 32 * db + 8 * g);
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = fmaf(wl, ol[e], wh * acc[qb][db][4 * g + e]);
            const bf16x2 a = {(__bf16)x[0], (__bf16)x[1]};
            const bf16x2 b = {(__bf16)x[2], (__bf16)x[3]};
            of[db][g] = u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
          }
        write_o(p.O_full, qb, of);
      }
      lse_store(p.LSE_full, qb, lse2);
    } else {
      if (p.O_hist) {
        u32x2 z[DB][4];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) z[db][g] = u32x2{0, 0};
        write_o(p.O_hist, qb, z);
      }
      if (p.LSE_hist && hh == 0 && qvalid[qb]) p.LSE_hist[(size_t)head * n_q + myq[qb]] = -INFINITY;
    }
  }
  };  // piece

  if constexpr (SK) {
    int wx, nx, bx;
    sk_xcd_counts(blockIdx.x % 8, gridDim.x, p.nblocks, wx, nx, bx);
    const int j = blockIdx.x / 8;
    if (nx > 0 && j < nx * p.sk_p) {
      const int unit = bx + j % nx, i = j / nx;
      int t0, t1;
      sk_piece_range(i, p.sk_p, T, t0, t1);
      piece(unit, t0, t1, p.part + (size_t)(unit * p.sk_p + i) * part_slot_floats(BM, D));
    }
  } else {
    piece((int)xcd_remap(blockIdx.x, p.nblocks), 0, T, nullptr);
  }
}

// Merge of the pieces of split units (split mode): per (query, head) the
// pieces' local states merge into O_loc / LSE_loc, their history states into
// O_hist / LSE_hist, and the two into O_full / LSE_full (log-sum-exp weights;
// float32 inputs, outputs rounded once).  Thread: one query row, 4 dims.
struct FixupParams {
  const float* part;
  uint16_t* O_loc;
  float* LSE_loc;
  uint16_t* O_hist;
  float* LSE_hist;
  uint16_t* O_full;
  float* LSE_full;
  int n_q, heads, n_qtiles, bm, T, Tl, sk_p;
};

template <int D>
__global__ __launch_bounds__(256) void sk_fixup_kernel(FixupParams p) {
  constexpr int TPR = D / 4;      // threads per query row (4 dims each)
  constexpr int RPB = 256 / TPR;  // rows per workgroup
  const int unit = blockIdx.x;
  const int r = blockIdx.y * RPB + threadIdx.x / TPR;
  const int head = unit / p.n_qtiles, qt = unit % p.n_qtiles;
  const int q = qt * p.bm + r;
  if (r >= p.bm || q >= p.n_q) return;
  const int T = p.T, Tl = p.Tl, P = p.sk_p;
  const size_t slot_f = part_slot_floats(p.bm, D);
  const float* base = p.part + (size_t)unit * P * slot_f;
  const int c4 = (threadIdx.x % TPR) * 4;
  float ml = -INFINITY, mh = -INFINITY;
  for (int i = 0; i < P; ++i) {
    int t0, t1;
    sk_piece_range(i, P, T, t0, t1);
    const float* sl = base + i * slot_f + (size_t)2 * p.bm * D;
    if (t0 < Tl) ml = fmaxf(ml, sl[r]);
    if (t1 > Tl) mh = fmaxf(mh, sl[p.bm + r]);
  }
  float sl_sum = 0.f, sh_sum = 0.f;
  f32x4 ol = {0.f, 0.f, 0.f, 0.f}, oh = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < P; ++i) {
    int t0, t1;
    sk_piece_range(i, P, T, t0, t1);
    const float* sb = base + i * slot_f;
    const float* sl = sb + (size_t)2 * p.bm * D;
    if (t0 < Tl) {
      const float e = exp2f(sl[r] - ml);
      sl_sum += e;
      ol += e * *(const f32x4*)(sb + (size_t)r * D + c4);
    }
    if (t1 > Tl) {
      const float e = exp2f(sl[p.bm + r] - mh);
      sh_sum += e;
      oh += e * *(const f32x4*)(sb + ((size_t)p.bm + r) * D + c4);
    }
  }
  const float lse_l = ml + log2f(sl_sum);
  ol *= 1.0f / sl_sum;
  const size_t o = (size_t)q * p.heads * D + head * D + c4;
  auto store_bf16 = [&](uint16_t* O, f32x4 v) {
    if (O == nullptr) return;
    const bf16x2 a = {(__bf16)v[0], (__bf16)v[1]};
    const bf16x2 b = {(__bf16)v[2], (__bf16)v[3]};
    *(u32x2*)(O + o) = u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
  };
  const bool lead = threadIdx.x % TPR == 0;
  const size_t li = (size_t)head * p.n_q + q;
  store_bf16(p.O_loc, ol);
  if (lead && p.LSE_loc) p.LSE_loc[li] = lse_l * LN2;
  if (T == Tl) {
    store_bf16(p.O_hist, f32x4{0.f, 0.f, 0.f, 0.f});
    if (lead && p.LSE_hist) p.LSE_hist[li] = -INFINITY;
    store_bf16(p.O_full, ol);
    if (lead && p.LSE_full) p.LSE_full[li] = lse_l * LN2;
    return;
  }
  const float lse_h = mh + log2f(sh_sum);
  oh *= 1.0f / sh_sum;
  store_bf16(p.O_hist, oh);
  if (lead && p.LSE_hist) p.LSE_hist[li] = lse_h * LN2;
  const float mx = fmaxf(lse_l, lse_h);
  const float lse = mx + log2f(exp2f(lse_l - mx) + exp2f(lse_h - mx));
  const float wl = exp2f(lse_l - lse), wh = exp2f(lse_h - lse);
  store_bf16(p.O_full, wl * ol + wh * oh);
  if (lead && p.LSE_full) p.LSE_full[li] = lse * LN2;
}

// ----------------------------------------------------------------------------
// float32 path: one thread per (query, head); K/V tiles of 32 keys in LDS.
// Used for the float32 configuration (parity-grade, not a performance path).
// ----------------------------------------------------------------------------
struct AttnF32Params {
  const float* Q;
  const float* Ks[MAX_KV_SEGS];  // key segments; [0, n_loc_seg) local, the rest history
  const float* Vs[MAX_KV_SEGS];
  int sn[MAX_KV_SEGS];
  int n_seg, n_loc_seg;
  float* O_loc;
  float* LSE_loc;
  float* O_hist;
  float* LSE_hist;
  float* O_full;
  float* LSE_full;
  int n_q, n_hist, heads;
  float c2;
  int n_qtiles;
};

constexpr int F32_NT = 128;
constexpr int F32_BN = 32;

template <int D>
__global__ __launch_bounds__(F32_NT) void attn_f32_kernel(AttnF32Params p) {
  __shared__ float sK[F32_BN][D];
  __shared__ float sV[F32_BN][D];
  __shared__ float stash[D][F32_NT];  // normalised O_loc of each thread's query
  const int tid = threadIdx.x;
  const int head = blockIdx.x / p.n_qtiles, qt = blockIdx.x % p.n_qtiles;
  const size_t HD = (size_t)p.heads * D;
  const int myq = qt * F32_NT + tid;
  const bool qvalid = myq < p.n_q;
  float q[D];
  for (int e = 0; e < D; ++e) q[e] = qvalid ? p.Q[(size_t)myq * HD + head * D + e] : 0.f;

  float lse2_loc = -INFINITY, lse2_hist = -INFINITY, inv_hist = 0.f;
  float acc[D];
  for (int br = 0; br < 2; ++br) {
    float m = -INFINITY, l = 0.f;
    for (int e = 0; e < D; ++e) acc[e] = 0.f;
    const int s_end = br == 0 ? p.n_loc_seg : p.n_seg;
    int n = 0;  // keys of this branch
    for (int sg = br == 0 ? 0 : p.n_loc_seg; sg < s_end; ++sg) {
    const float* Kp = p.Ks[sg];
    const float* Vp = p.Vs[sg];
    const int ns = p.sn[sg];
    n += ns;
    for (int k0 = 0; k0 < ns; k0 += F32_BN) {
      __syncthreads();
      for (int i = tid; i < F32_BN * D; i += F32_NT) {
        const int r = i / D, c = i % D;
        const int key = k0 + r;
        sK[r][c] = key < ns ? Kp[(size_t)key * HD + head * D + c] : 0.f;
        sV[r][c] = key < ns ? Vp[(size_t)key * HD + head * D + c] : 0.f;
      }
      __syncthreads();
      const int nk = min(F32_BN, ns - k0);
      float s[F32_BN];
      float mx = -INFINITY;
      for (int j = 0; j < F32_BN; ++j) {
        float a = 0.f;
        for (int e = 0; e < D; ++e) a = fmaf(q[e], sK[j][e], a);
        s[j] = j < nk ? a * p.c2 : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float mnew = fmaxf(m, mx);
      const float alpha = exp2f(m - mnew);
      m = mnew;
      l *= alpha;
      for (int e = 0; e < D; ++e) acc[e] *= alpha;
      for (int j = 0; j < F32_BN; ++j) {
        const float pj = exp2f(s[j] - mnew);
        l += pj;
        for (int e = 0; e < D; ++e) acc[e] = fmaf(pj, sV[j][e], acc[e]);
      }
    }
    }
    if (br == 0) {
      const float inv = 1.0f / l;
      lse2_loc = m + log2f(l);
      for (int e = 0; e < D; ++e) stash[e][tid] = acc[e] * inv;
      if (qvalid) {
        if (p.O_loc)
          for (int e = 0; e < D; ++e) p.O_loc[(size_t)myq * HD + head * D + e] = stash[e][tid];
        if (p.LSE_loc) p.LSE_loc[(size_t)head * p.n_q + myq] = lse2_loc * LN2;
      }
    } else if (n > 0) {
      inv_hist = 1.0f / l;
      lse2_hist = m + log2f(l);
    }
  }
  if (!qvalid) return;
  float* ob = nullptr;
  if (p.O_hist) {
    ob = p.O_hist + (size_t)myq * HD + head * D;
    for (int e = 0; e < D; ++e) ob[e] = p.n_hist > 0 ? acc[e] * inv_hist : 0.f;
  }
  if (p.LSE_hist) p.LSE_hist[(size_t)head * p.n_q + myq] = lse2_hist * LN2;
  float lse2 = lse2_loc, wl = 1.f, wh = 0.f;
  if (p.n_hist > 0) {
    const float mx = fmaxf(lse2_loc, lse2_hist);
    lse2 = mx + log2f(exp2f(lse2_loc - mx) + exp2f(lse2_hist - mx));
    wl = exp2f(lse2_loc - lse2);
    wh = exp2f(lse2_hist - lse2) * inv_hist;
  }
  if (p.O_full) {
    float* of = p.O_full + (size_t)myq * HD + head * D;
    for (int e = 0; e < D; ++e) of[e] = p.n_hist > 0 ? fmaf(wl, stash[e][tid], wh * acc[e]) : stash[e][tid];
  }
  if (p.LSE_full) p.LSE_full[(size_t)head * p.n_q + myq] = lse2 * LN2;
}

// ----------------------------------------------------------------------------
// N-way LSE merge (memory bound): one thread per (query, head, 8 dims).
// ----------------------------------------------------------------------------
constexpr int MAX_PARTS = 16;
struct MergeParams {
  const void* O[MAX_PARTS];
  const float* LSE[MAX_PARTS];
  int n_parts;
  int64_t n_q;
  int heads, head_dim;
  void* O_out;
  float* LSE_out;
};

template <bool BF16>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeParams p) {
  const int chunks = p.head_dim / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = p.n_q * p.heads * chunks;
  if (idx >= total) return;
  const int c = idx % chunks;
  const int64_t qh = idx / chunks;
  const int h = qh % p.heads;
  const int64_t q = qh / p.heads;
  float lse[MAX_PARTS];
  float mx = -INFINITY;
  for (int i = 0; i < p.n_parts; ++i) {
    lse[i] = p.LSE[i][(size_t)h * p.n_q + q];
    mx = fmaxf(mx, lse[i]);
  }
  float sum = 0.f;
  for (int i = 0; i < p.n_parts; ++i) sum += (lse[i] == -INFINITY) ? 0.f : __expf(lse[i] - mx);
  const float lse_out = (mx == -INFINITY) ? -INFINITY : mx + __logf(sum);
  float out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const size_t off = (size_t)qh * p.head_dim + c * 8;
  for (int i = 0; i < p.n_parts; ++i) {
    if (lse[i] == -INFINITY) continue;
    const float w = __expf(lse[i] - lse_out);
    if (BF16) {
      const u32x4 v = *(const u32x4*)((const uint16_t*)p.O[i] + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[2 * e] = fmaf(w, __builtin_bit_cast(float, v[e] << 16), out[2 * e]);
        out[2 * e + 1] = fmaf(w, __builtin_bit_cast(float, v[e] & 0xFFFF0000u), out[2 * e + 1]);
      }
    } else {
      const f32x4 a = *(const f32x4*)((const float*)p.O[i] + off);
      const f32x4 b = *(const f32x4*)((const float*)p.O[i] + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[e] = fmaf(w, a[e], out[e]);
        out[4 + e] = fmaf(w, b[e], out[4 + e]);
      }
    }
  }
  if (BF16) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2 b = {(__bf16)out[2 * e], (__bf16)out[2 * e + 1]};
      v[e] = __builtin_bit_cast(uint32_t, b);
    }
    *(u32x4*)((uint16_t*)p.O_out + off) = v;
  } else {
    *(f32x4*)((float*)p.O_out + off) = f32x4{out[0], out[1], out[2], out[3]};
    *(f32x4*)((float*)p.O_out + off + 4) = f32x4{out[4], out[5], out[6], out[7]};
  }
  if (p.LSE_out && c == 0) p.LSE_out[(size_t)h * p.n_q + q] = lse_out;
}

}  // namespace

// One shape: 8 waves x 32 queries with 128-key tiles (256 queries share each staged tile; two waves
// per SIMD; 128 KB of LDS for the double-buffered K and V tiles).  Measured against 64-key tiles
// (2 % slower: twice the per-tile barrier, load issue and row-max finishing) and 4 waves x 32 queries.
constexpr int ATTN_NW = 8, ATTN_BN = 128, ATTN_BM = ATTN_NW * 32;

template <int D, bool SK>
void launch_bf16(dim3 grid, hipStream_t s, const AttnKParams& p) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, ATTN_NW, 1, ATTN_BN, SK>), grid, dim3(ATTN_NW * 64), 0, s, p);
}

size_t stash_bytes(int64_t n_q, int32_t heads, int32_t head_dim, int64_t n_hist) {
  return n_hist == 0 ? 0 : ((size_t)n_q * heads * head_dim * sizeof(float) + 255) & ~(size_t)255;
}

ispa_status_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n_q == 0) return ISPA_OK;
  if (a.dtype == ISPA_BF16) {
    AttnKParams p;
    p.Q = (const uint16_t*)a.Q;
    p.O_loc = (uint16_t*)a.O_loc;
    p.LSE_loc = a.LSE_loc;
    p.O_hist = (uint16_t*)a.O_hist;
    p.LSE_hist = a.LSE_hist;
    p.O_full = (uint16_t*)a.O_full;
    p.LSE_full = a.LSE_full;
    p.stash = (float*)a.ws;
    p.n_q = (int)a.n_q;
    p.heads = a.heads;
    p.c2 = a.scale * LOG2E;
    const size_t ws_need = attention_workspace_size(a.n_q, a.heads, a.head_dim, a.n_hist, a.dtype);
    if (a.O_full && ws_need > 0 && (a.ws == nullptr || a.ws_bytes < ws_need)) {
      set_error("ispa_decomp_attn: workspace too small for the merge (query ispa_decomp_attn_workspace_size)");
      return ISPA_E_WORKSPACE;
    }
    p.q_scale = a.q_scale;
    p.n_seg = a.kv.n_seg;
    p.n_loc_seg = a.kv.n_loc_seg;
    p.st0[0] = 0;
    for (int i = 0; i < MAX_KV_SEGS; ++i) {
      const bool used = i < a.kv.n_seg;
      p.Ks[i] = used ? (const uint16_t*)a.kv.K[i] : nullptr;
      p.Vs[i] = used ? (const uint16_t*)a.kv.V[i] : nullptr;
      p.sn[i] = used ? (int)a.kv.n[i] : 0;
      p.k_scale[i] = used ? a.k_scale[i] : nullptr;
      p.st0[i + 1] = p.st0[i] + (int)((p.sn[i] + ATTN_BN - 1) / ATTN_BN);
    }
    const int bm = ATTN_BM;
    p.n_qtiles = (int)((a.n_q + bm - 1) / bm);
    p.nblocks = p.n_qtiles * a.heads;
    p.sk_p = 1;
    p.part = nullptr;
    if (a.k_fp8) {
      const dim3 grid(p.nblocks);
      if (a.head_dim == 128)
        hipLaunchKernelGGL((attn_bf16_kernel<128, ATTN_NW, 1, ATTN_BN, false, true>), grid, dim3(ATTN_NW * 64), 0, s, p);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<64, ATTN_NW, 1, ATTN_BN, false, true>), grid, dim3(ATTN_NW * 64), 0, s, p);
      return hip_check(hipGetLastError(), "attn_bf16_kernel (fp8 keys) launch");
    }
    if (a.sk_workers <= 0) {
      const dim3 grid(p.nblocks);
      if (a.head_dim == 128)
        launch_bf16<128, false>(grid, s, p);
      else
        launch_bf16<64, false>(grid, s, p);
      return hip_check(hipGetLastError(), "attn_bf16_kernel launch");
    }
    // split mode: each unit's key tiles cut into P pieces on P workgroups of its XCD
    const int T = p.st0[p.n_seg];
    const size_t need = splitkv_workspace_size(a.n_q, a.heads, a.head_dim, a.n_hist, a.sk_workers);
    if (a.ws == nullptr || a.ws_bytes < need) {
      set_error("split-KV attention: workspace smaller than ispa_decomp_attn_splitkv_workspace_size()");
      return ISPA_E_WORKSPACE;
    }
    p.sk_p = sk_pieces(a.sk_workers, p.nblocks, T);
    p.part = (float*)((char*)a.ws + stash_bytes(a.n_q, a.heads, a.head_dim, a.n_hist));
    if (p.sk_p <= 1) {  // nothing to split: the unsplit launch
      const dim3 grid(p.nblocks);
      if (a.head_dim == 128)
        launch_bf16<128, false>(grid, s, p);
      else
        launch_bf16<64, false>(grid, s, p);
      return hip_check(hipGetLastError(), "attn_bf16_kernel launch");
    }
    const dim3 grid(a.sk_workers);
    if (a.head_dim == 128)
      launch_bf16<128, true>(grid, s, p);
    else
      launch_bf16<64, true>(grid, s, p);
    ispa_status_t st = hip_check(hipGetLastError(), "attn_bf16_kernel (split) launch");
    if (st != ISPA_OK) return st;
    FixupParams f;
    f.part = p.part;
    f.O_loc = p.O_loc;
    f.LSE_loc = p.LSE_loc;
    f.O_hist = p.O_hist;
    f.LSE_hist = p.LSE_hist;
    f.O_full = p.O_full;
    f.LSE_full = p.LSE_full;
    f.n_q = p.n_q;
    f.heads = p.heads;
    f.n_qtiles = p.n_qtiles;
    f.bm = bm;
    f.T = T;
    f.Tl = p.st0[p.n_loc_seg];
    f.sk_p = p.sk_p;
    const int rpb = 256 / (a.head_dim / 4);
    const dim3 fgrid(p.nblocks, (bm + rpb - 1) / rpb);
    if (a.head_dim == 128)
      hipLaunchKernelGGL(sk_fixup_kernel<128>, fgrid, dim3(256), 0, s, f);
    else
      hipLaunchKernelGGL(sk_fixup_kernel<64>, fgrid, dim3(256), 0, s, f);
    return hip_check(hipGetLastError(), "sk_fixup_kernel launch");
  }
  AttnF32Params p;
  p.Q = (const float*)a.Q;
  p.n_seg = a.kv.n_seg;
  p.n_loc_seg = a.kv.n_loc_seg;
  for (int i = 0; i < MAX_KV_SEGS; ++i) {
    const bool used = i < a.kv.n_seg;
    p.Ks[i] = used ? (const float*)a.kv.K[i] : nullptr;
    p.Vs[i] = used ? (const float*)a.kv.V[i] : nullptr;
    p.sn[i] = used ? (int)a.kv.n[i] : 0;
  }
  p.O_loc = (float*)a.O_loc;
  p.LSE_loc = a.LSE_loc;
  p.O_hist = (float*)a.O_hist;
  p.LSE_hist = a.LSE_hist;
  p.O_full = (float*)a.O_full;
  p.LSE_full = a.LSE_full;
  p.n_q = (int)a.n_q;
  p.n_hist = (int)a.n_hist;
  p.heads = a.heads;
  p.c2 = a.scale * LOG2E;
  p.n_qtiles = (int)((a.n_q + F32_NT - 1) / F32_NT);
  const dim3 grid(p.n_qtiles * a.heads), block(F32_NT);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((attn_f32_kernel<128>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_f32_kernel<64>), grid, block, 0, s, p);
  return hip_check(hipGetLastError(), "attn_f32_kernel launch");
}

size_t attention_workspace_size(int64_t n_q, int32_t heads, int32_t head_dim, int64_t n_hist, int32_t dtype) {
  if (dtype != ISPA_BF16 || n_hist == 0) return 0;
  return (size_t)n_q * heads * head_dim * sizeof(float);
}

size_t splitkv_workspace_size(int64_t n_q, int32_t heads, int32_t head_dim, int64_t n_hist, int32_t n_workers) {
  if (n_q <= 0 || n_workers <= 0) return 0;
  const int bm = ATTN_BM;
  return stash_bytes(n_q, heads, head_dim, n_hist) + (size_t)n_workers * part_slot_floats(bm, head_dim) * 4;
}

ispa_status_t launch_lse_merge(int32_t n_parts, const void* const* O, const float* const* LSE, int64_t n_q,
                               int32_t heads, int32_t head_dim, int32_t dtype, void* O_out, float* LSE_out,
                               hipStream_t s) {
  if (n_q == 0) return ISPA_OK;
  MergeParams p;
  for (int i = 0; i < n_parts; ++i) {
    p.O[i] = O[i];
    p.LSE[i] = LSE[i];
  }
  p.n_parts = n_parts;
  p.n_q = n_q;
  p.heads = heads;
  p.head_dim = head_dim;
  p.O_out = O_out;
  p.LSE_out = LSE_out;
  const int64_t total = n_q * heads * (head_dim / 8);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (dtype == ISPA_BF16)
    hipLaunchKernelGGL((lse_merge_kernel<true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((lse_merge_kernel<false>), grid, block, 0, s, p);
  return hip_check(hipGetLastError(), "lse_merge_kernel launch");
}

}  // namespace ispa
