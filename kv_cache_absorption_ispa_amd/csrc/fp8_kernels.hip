// fp8 (E4M3, OCP "FN" encoding) quantisation and the W8A8 product on gfx950.
//
// Source: "Technical Summary: Instance-Specific Parametric Absorption (ISPA)
// for Memory-Efficient Video Generation", section 4 "Results" (ISPA combined
// with W8A8 post-training quantisation).  The pages fix no format or scaling;
// the reading: E4M3, one absmax scale per block (scale = amax / 448 in
// float32, 1 if amax = 0), codes = round-to-nearest-even of x / scale (float32
// division, clamped to +-448) by v_cvt_pk_fp8_f32.
//
// Blocks: per head over all rows and dims (Q and K of the attention), per row
// (activations of the W8A8 product), per output column (its weights).
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr float E4M3_MAX = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

__device__ __forceinline__ float load_elem(const void* X, size_t i, int dtype) {
  return dtype == ISPA_BF16 ? bf16_to_f32(((const uint16_t*)X)[i]) : ((const float*)X)[i];
}

// Eight consecutive elements (16 bytes of bf16 or 32 of float32; i a multiple of 8) as float32.
__device__ __forceinline__ void load8(const void* X, size_t i, int dtype, float (&v)[8]) {
  if (dtype == ISPA_BF16) {
    const u32x4 w = *(const u32x4*)((const uint16_t*)X + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __builtin_bit_cast(float, w[e] << 16);
      v[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *(const f32x4*)((const float*)X + i), b = *(const f32x4*)((const float*)X + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
}

// Four codes of x[0..3] / scale, packed little-endian (x[0] in the low byte).
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float scale) {
  const float qa = fminf(fmaxf(a / scale, -E4M3_MAX), E4M3_MAX);
  const float qb = fminf(fmaxf(b / scale, -E4M3_MAX), E4M3_MAX);
  const float qc = fminf(fmaxf(c / scale, -E4M3_MAX), E4M3_MAX);
  const float qd = fminf(fmaxf(d / scale, -E4M3_MAX), E4M3_MAX);
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(qa, qb, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(qc, qd, w, true);
}

__device__ __forceinline__ float scale_of(float amax) { return amax > 0.f ? amax / E4M3_MAX : 1.0f; }

// Block max of v over 256 threads (LDS tree).
__device__ __forceinline__ float block_max256(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

constexpr int QH_ROWS = 16;          // rows per workgroup of the per-head quantiser
constexpr int QH_MAX_CHUNKS = 2048;  // 8-element chunks per row it supports (H * D <= 16384)

// Pass 1: partial |x| maxima per head over rows [b * QH_ROWS, ...): part[h * nblk + b].  Thread t
// owns the 8-element chunks t, t + 256, ... of every row (one head each), so rows are read whole
// and contiguously.
__global__ __launch_bounds__(256) void head_amax_kernel(const void* X, int dtype, int64_t n, int H, int D,
                                                        float* part) {
  __shared__ float cmax[QH_MAX_CHUNKS];
  const int b = blockIdx.x;
  const int cpr = H * D / 8;
  const int64_t r0 = (int64_t)b * QH_ROWS, r1 = min(r0 + QH_ROWS, n);
  for (int c = threadIdx.x; c < cpr; c += 256) {
    float m = 0.f;
    for (int64_t r = r0; r < r1; ++r) {
      float v[8];
      load8(X, (size_t)r * H * D + (size_t)c * 8, dtype, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    }
    cmax[c] = m;
  }
  __syncthreads();
  const int cph = D / 8;  // chunks per head
  for (int h = threadIdx.x; h < H; h += 256) {
    float m = 0.f;
    for (int c = 0; c < cph; ++c) m = fmaxf(m, cmax[h * cph + c]);
    part[(size_t)h * gridDim.x + b] = m;
  }
}

// Pass 2: one workgroup per head reduces its partials to scale[h].
__global__ __launch_bounds__(256) void head_scale_kernel(const float* part, int nblk, float* scale) {
  __shared__ float red[256];
  const int h = blockIdx.x;
  float m = 0.f;
  for (int i = threadIdx.x; i < nblk; i += 256) m = fmaxf(m, part[(size_t)h * nblk + i]);
  m = block_max256(m, red);
  if (threadIdx.x == 0) scale[h] = scale_of(m);
}

// Pass 3: the codes, 8 elements per thread per step, rows read whole.
__global__ __launch_bounds__(256) void head_quant_kernel(const void* X, int dtype, int64_t n, int H, int D,
                                                         const float* scale, uint8_t* X8) {
  const int cpr = H * D / 8, cph = D / 8;
  const int64_t r0 = (int64_t)blockIdx.x * QH_ROWS, r1 = min(r0 + QH_ROWS, n);
  for (int64_t r = r0; r < r1; ++r)
    for (int c = threadIdx.x; c < cpr; c += 256) {
      const float s = scale[c / cph];
      const size_t i = (size_t)r * H * D + (size_t)c * 8;
      float v[8];
      load8(X, i, dtype, v);
      *(u32x2*)(X8 + i) = u32x2{quant4(v[0], v[1], v[2], v[3], s), quant4(v[4], v[5], v[6], v[7], s)};
    }
}

// One wave per row of X [n, d]: scale[r] = amax(row) / 448 and the row's codes.
__global__ __launch_bounds__(256) void row_quant_kernel(const void* X, int dtype, int64_t n, int d, uint8_t* X8,
                                                        float* scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const size_t base = (size_t)r * d;
  float m = 0.f;
  for (int c = lane * 4; c < d; c += 256)
    for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(load_elem(X, base + c + e, dtype)));
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float s = scale_of(m);
  if (lane == 0) scale[r] = s;
  for (int c = lane * 4; c < d; c += 256)
    *(uint32_t*)(X8 + base + c) = quant4(load_elem(X, base + c, dtype), load_elem(X, base + c + 1, dtype),
                                         load_elem(X, base + c + 2, dtype), load_elem(X, base + c + 3, dtype), s);
}

// One thread per column j of W [d, d_out] (float32): scale[j] and the column's codes written as row j of
// W8T [d_out, d] (the K-contiguous operand layout of the product).  Runs once per converted layer.
__global__ __launch_bounds__(256) void col_quant_kernel(const float* W, int d, int d_out, uint8_t* W8T,
                                                        float* scale) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d_out) return;
  float m = 0.f;
  for (int k = 0; k < d; ++k) m = fmaxf(m, fabsf(W[(size_t)k * d_out + j]));
  const float s = scale_of(m);
  scale[j] = s;
  for (int k = 0; k < d; k += 4)
    *(uint32_t*)(W8T + (size_t)j * d + k) = quant4(W[(size_t)k * d_out + j], W[(size_t)(k + 1) * d_out + j],
                                                   W[(size_t)(k + 2) * d_out + j], W[(size_t)(k + 3) * d_out + j],
                                                   s);
}

// ---------------------------------------------------------------- W8A8 product
// Y [n, N] (bf16) = (A8 [n, K] . W8T [N, K]^T) * sa[row] * sw[col]: E4M3 codes, float32 accumulation
// on v_mfma_f32_32x32x64_f8f6f4 (products of codes are exact in float32).
//
// 128 x 128 output tile per workgroup of 4 waves (2 x 2, each 64 x 64 = 2 x 2 blocks of 32 x 32).
// K advances 64 codes per stage; both 128 x 64-byte operand tiles go global -> LDS by buffer loads
// into LDS (double-buffered), rows of 64 bytes with their 16-byte chunks permuted by
// c ^ ((r >> 2) & 3), which spreads the 16 rows of a read pass over all 64 banks.  Lane l reads
// row l % 32 of its block, bytes 32 (l / 32) .. +31 of the stage (the same k order for A and B).
constexpr int GB = 128;   // tile rows and columns
constexpr int GK = 64;    // codes per stage

__device__ __forceinline__ int g8_swz(int r) { return (r >> 2) & 3; }

__global__ __launch_bounds__(256) void w8a8_gemm_kernel(const uint8_t* __restrict__ A8, const float* __restrict__ sa,
                                                        const uint8_t* __restrict__ W8T,
                                                        const float* __restrict__ sw, uint16_t* __restrict__ Y,
                                                        int n, int N, int K, int ntn) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA[2][GB * GK];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[2][GB * GK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (int)(tile / ntn) * GB, n0 = (int)(tile % ntn) * GB;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const rsrc_t ra = make_rsrc(A8 + (size_t)m0 * K, (uint32_t)(min(GB, n - m0) * K));
  const rsrc_t rb = make_rsrc(W8T + (size_t)n0 * K, (uint32_t)(GB * K));
  // this wave's 4 loads per stage: loads 0..7 fill A rows 16 j .. 16 j + 15, 8..15 the B rows
  uint32_t goff[4];
  int ldst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = wave + 4 * i;
    const int row = (g % 8) * 16 + lane / 4;
    const int chunk = (lane % 4) ^ g8_swz(row);
    goff[i] = (uint32_t)row * K + chunk * 16;
    ldst[i] = (g % 8) * 16 * GK;
  }
  auto load_stage = [&](int buf, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = wave + 4 * i;
      if (g < 8)
        load_to_lds(ra, (uint16_t*)(sA[buf] + ldst[i]), goff[i] + k0);
      else
        load_to_lds(rb, (uint16_t*)(sB[buf] + ldst[i]), goff[i] + k0);
    }
  };
  const int l32 = lane & 31, hh = lane >> 5;
  auto frag = [&](const uint8_t* t, int r0) {
    const int r = r0 + l32;
    const u32x4 a = *(const u32x4*)(t + r * GK + (((2 * hh) ^ g8_swz(r)) << 4));
    const u32x4 b = *(const u32x4*)(t + r * GK + (((2 * hh + 1) ^ g8_swz(r)) << 4));
    return v8i_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};
  const int nst = K / GK;
  load_stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load_stage(buf ^ 1, (st + 1) * GK);
    const v8i_t a0 = frag(sA[buf], wm), a1 = frag(sA[buf], wm + 32);
    const v8i_t b0 = frag(sB[buf], wn), b1 = frag(sB[buf], wn + 32);
    acc[0][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, acc[0][0], 0, 0, 0, 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b1, acc[0][1], 0, 0, 0, 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b0, acc[1][0], 0, 0, 0, 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, acc[1][1], 0, 0, 0, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // element v of lane l in a 32 x 32 block: row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + 32 * j + l32;
      const float swc = sw[col];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (row < n) {
          const __bf16 y = (__bf16)(acc[i][j][v] * sa[row] * swc);
          Y[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, y);
        }
      }
    }
}

}  // namespace

size_t quant_head_workspace_size(int64_t n, int32_t heads) {
  const int64_t nb = (n + QH_ROWS - 1) / QH_ROWS;
  return (size_t)(nb > 0 ? nb : 1) * heads * sizeof(float);
}

int32_t quant_head_max_width() { return QH_MAX_CHUNKS * 8; }

ispa_status_t launch_quant_head(int64_t n, int32_t H, int32_t D, int32_t dtype, const void* X, uint8_t* X8,
                                float* scale, void* ws, hipStream_t s) {
  const unsigned nb = (unsigned)std::max<int64_t>((n + QH_ROWS - 1) / QH_ROWS, 1);
  hipLaunchKernelGGL(head_amax_kernel, dim3(nb), dim3(256), 0, s, X, dtype, n, H, D, (float*)ws);
  ispa_status_t st = hip_check(hipGetLastError(), "head_amax_kernel launch");
  if (st != ISPA_OK) return st;
  hipLaunchKernelGGL(head_scale_kernel, dim3(H), dim3(256), 0, s, (const float*)ws, (int)nb, scale);
  st = hip_check(hipGetLastError(), "head_scale_kernel launch");
  if (st != ISPA_OK || n == 0) return st;
  hipLaunchKernelGGL(head_quant_kernel, dim3(nb), dim3(256), 0, s, X, dtype, n, H, D, (const float*)scale, X8);
  return hip_check(hipGetLastError(), "head_quant_kernel launch");
}

ispa_status_t launch_quant_rows(int64_t n, int32_t d, int32_t dtype, const void* X, uint8_t* X8, float* scale,
                                hipStream_t s) {
  if (n == 0) return ISPA_OK;
  hipLaunchKernelGGL(row_quant_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, X, dtype, n, d, X8, scale);
  return hip_check(hipGetLastError(), "row_quant_kernel launch");
}

ispa_status_t launch_quant_cols(int32_t d, int32_t d_out, const float* W, uint8_t* W8T, float* scale,
                                hipStream_t s) {
  hipLaunchKernelGGL(col_quant_kernel, dim3((unsigned)((d_out + 255) / 256)), dim3(256), 0, s, W, d, d_out, W8T,
                     scale);
  return hip_check(hipGetLastError(), "col_quant_kernel launch");
}

ispa_status_t launch_w8a8_gemm(int64_t n, int32_t N, int32_t K, const uint8_t* A8, const float* sa,
                               const uint8_t* W8T, const float* sw, uint16_t* Y, hipStream_t s) {
  if (n == 0) return ISPA_OK;
  const int ntm = (int)((n + GB - 1) / GB), ntn = N / GB;
  hipLaunchKernelGGL(w8a8_gemm_kernel, dim3((unsigned)(ntm * ntn)), dim3(256), 0, s, A8, sa, W8T, sw, Y, (int)n, N,
                     K, ntn);
  return hip_check(hipGetLastError(), "w8a8_gemm_kernel launch");
}

}  // namespace ispa
