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
// .. + 7).  The first product writes its result transposed and split (the second product's B), the
// second one float32.  L^-1 is split once per solve, row-major (A of Z = L^-1 Y) and transposed
// (A of X = L^-T Z).
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int PT = 128;        // output tile (PT x PT), 4 waves of 64 x 64
constexpr int PKS = 32;        // K slab
constexpr int PLS = PKS + 8;   // LDS row stride (bf16): 80-byte rows, conflict-free 16-byte reads
constexpr int SPB = 64;        // split / transpose block

__device__ __forceinline__ void split2(float x, __bf16& h, __bf16& l) {
  h = (__bf16)x;
  l = (__bf16)(x - (float)h);
}

// Lh, Ll = split(L^-1) and LTh, LTl = split(L^-T) over the 64 x 64 blocks (bi, bj) of L^-1 with
// bj <= 2 (bi / 2) + 1: those the 128-row tiles of the two products read (lower: k < m0 + 128;
// upper, transposed: k >= m0).  Everything they read outside the triangle is zero in L^-1.
__global__ __launch_bounds__(256) void split_lower_kernel(const float* __restrict__ Linv, int d, __bf16* Lh,
                                                          __bf16* Ll, __bf16* LTh, __bf16* LTl,
                                                          const int32_t* __restrict__ info) {
  const int bi = blockIdx.y, bj = blockIdx.x, b = blockIdx.z;
  if (bj > 2 * (bi / 2) + 1 || info[b] != 0) return;
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
  __bf16 *Dh, *Dl;        // OUT_T: D^T split, N x M (row stride M)
  float* D;               // else: D float32, M x N (row stride N)
  int M, N, K;
  size_t sA, sB, sD;      // batch strides (elements)
  const int32_t* info;
};

// D = A B^T with A triangular (LOWER: k < m0 + PT; else k >= m0), as hi*hi + hi*lo + lo*hi.
// The next slab's operands are loaded into registers while the current one is multiplied from LDS
// (two LDS buffers, one barrier per slab).  M, N multiples of PT, K of PKS.
template <bool LOWER, bool OUT_T>
__global__ __launch_bounds__(256, 2) void apply3_kernel(Apply3Params p) {
  const int b = blockIdx.z;
  if (p.info[b] != 0) return;
  const int m0 = blockIdx.y * PT, n0 = blockIdx.x * PT;
  __shared__ __attribute__((aligned(16))) __bf16 S[2][4][PT][PLS];  // [buffer][Ah, Al, Bh, Bl][row][k]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const size_t K = (size_t)p.K;
  const __bf16* src[4] = {p.Ah + b * p.sA + (size_t)m0 * K, p.Al + b * p.sA + (size_t)m0 * K,
                          p.Bh + b * p.sB + (size_t)n0 * K, p.Bl + b * p.sB + (size_t)n0 * K};
  const int kb = LOWER ? 0 : m0;
  const int ke = LOWER ? min(p.K, m0 + PT) : p.K;
  // thread t moves rows t / 4 and 64 + t / 4, 16-byte chunk t % 4, of each operand
  const int lr = tid >> 2, lc = 8 * (tid & 3);
  u32x4 reg[4][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
      for (int h = 0; h < 2; ++h) reg[o][h] = *(const u32x4*)(src[o] + (size_t)(lr + 64 * h) * K + k0 + lc);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
      for (int h = 0; h < 2; ++h) *(u32x4*)(&S[buf][o][lr + 64 * h][lc]) = reg[o][h];
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};
  load(kb);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += PKS) {
    const bool more = k0 + PKS < ke;
    if (more) load(k0 + PKS);
#pragma unroll
    for (int ks = 0; ks < PKS / 16; ++ks) {
      bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = *(const bf16x8*)(&S[buf][0][wm + 32 * i + l32][16 * ks + 8 * hh]);
        al[i] = *(const bf16x8*)(&S[buf][1][wm + 32 * i + l32][16 * ks + 8 * hh]);
        bh[i] = *(const bf16x8*)(&S[buf][2][wn + 32 * i + l32][16 * ks + 8 * hh]);
        bl[i] = *(const bf16x8*)(&S[buf][3][wn + 32 * i + l32][16 * ks + 8 * hh]);
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
    if (more) store(buf ^ 1);  // the other buffer: its last readers finished before the previous barrier
    __syncthreads();
    buf ^= 1;
  }
  // acc[i][j][v]: row m0 + wm + 32 i + 8 (v / 4) + 4 hh + v % 4, column n0 + wn + 32 j + l32
  if constexpr (OUT_T) {
    const size_t M = (size_t)p.M;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const size_t col = (size_t)(n0 + wn + 32 * j + l32);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = m0 + wm + 32 * i + 8 * g + 4 * hh;
          bf16x4 h, l;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            __bf16 he, le;
            split2(acc[i][j][4 * g + e], he, le);
            h[e] = he;
            l[e] = le;
          }
          *(bf16x4*)(p.Dh + b * p.sD + col * M + row) = h;
          *(bf16x4*)(p.Dl + b * p.sD + col * M + row) = l;
        }
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
  // Z^T = (L^-1 Y)^T, split
  Apply3Params p{};
  p.Ah = L; p.Al = L + bdd; p.Bh = YT; p.Bl = YT + bdn; p.Dh = ZT; p.Dl = ZT + bdn;
  p.M = d; p.N = d_out; p.K = d;
  p.sA = dd; p.sB = dn; p.sD = dn;
  p.info = info;
  hipLaunchKernelGGL((apply3_kernel<true, true>), dim3(d_out / PT, d / PT, batch), dim3(256), 0, s, p);
  st = hip_check(hipGetLastError(), "apply3_kernel launch");
  if (st != ISPA_OK) return st;
  // X = L^-T Z
  Apply3Params q{};
  q.Ah = LT; q.Al = LT + bdd; q.Bh = ZT; q.Bl = ZT + bdn; q.D = X;
  q.M = d; q.N = d_out; q.K = d;
  q.sA = dd; q.sB = dn; q.sD = dn;
  q.info = info;
  hipLaunchKernelGGL((apply3_kernel<false, false>), dim3(d_out / PT, d / PT, batch), dim3(256), 0, s, q);
  return hip_check(hipGetLastError(), "apply3_kernel launch");
}

}  // namespace ispa
