// Stack transition of the warmup: rank layers by reconstruction error and
// absorb dW into the chosen ones.
//
// Source: "Technical Summary: Instance-Specific Parametric Absorption (ISPA)
// for Memory-Efficient Video Generation", section 2 "Methodology":
// "Dynamic Layer Selection" ranks every layer by its reconstruction error
// after warmup and converts the lowest-error ones to local-attention layers;
// step 3 "Memory-Efficient Inference" gives those layers W_new = W + dW.
//
// The ranking is a strict total order (eps ascending, NaN last, ties to the
// lower layer index), so the chosen set is unique; a workgroup computes every
// layer's rank by counting the layers ordered before it (n <= 4096 layers, the
// O(n^2) comparisons are a few microseconds).
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int SEL_THREADS = 1024;

// true if layer j (eps ej) ranks before layer i (eps ei)
__device__ __forceinline__ bool ranks_before(double ej, int j, double ei, int i) {
  const bool nj = ej != ej, ni = ei != ei;
  if (nj != ni) return ni;  // finite values rank before NaN
  if (!nj && ej != ei) return ej < ei;
  return j < i;
}

__global__ __launch_bounds__(SEL_THREADS) void select_layers_kernel(int n, const double* __restrict__ eps, int k,
                                                                    int* __restrict__ selected,
                                                                    int* __restrict__ rank) {
  __shared__ double se[MAX_STACK_LAYERS];
  for (int i = threadIdx.x; i < n; i += SEL_THREADS) se[i] = eps[i];
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += SEL_THREADS) {
    const double ei = se[i];
    int r = 0;
    for (int j = 0; j < n; ++j) r += ranks_before(se[j], j, ei, i) ? 1 : 0;
    if (rank) rank[i] = r;
    if (r < k) selected[r] = i;
  }
}

// Threshold selection: the layers with eps <= tau, lowest first (same total order), at most k_max.
// Those are exactly the first c ranks, c = #{eps <= tau} (a NaN is never <= tau).
__global__ __launch_bounds__(SEL_THREADS) void select_below_kernel(int n, const double* __restrict__ eps, double tau,
                                                                   int k_max, int* __restrict__ selected,
                                                                   int* __restrict__ count, int* __restrict__ rank) {
  __shared__ double se[MAX_STACK_LAYERS];
  __shared__ int cnt[SEL_THREADS];
  int c = 0;
  for (int i = threadIdx.x; i < n; i += SEL_THREADS) {
    se[i] = eps[i];
    c += eps[i] <= tau ? 1 : 0;
  }
  cnt[threadIdx.x] = c;
  __syncthreads();
  for (int w = SEL_THREADS / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) cnt[threadIdx.x] += cnt[threadIdx.x + w];
    __syncthreads();
  }
  const int k = min(cnt[0], k_max);
  if (threadIdx.x == 0) count[0] = k;
  for (int i = threadIdx.x; i < n; i += SEL_THREADS) {
    const double ei = se[i];
    int r = 0;
    for (int j = 0; j < n; ++j) r += ranks_before(se[j], j, ei, i) ? 1 : 0;
    if (rank) rank[i] = r;
    if (r < k) selected[r] = i;
  }
}

// dst[s] = src[sel[s]] (per_layer floats each), s < k; ids outside [0, n_layers) give NaN.
__global__ __launch_bounds__(256) void gather_layers_kernel(size_t per_layer, const float* __restrict__ src,
                                                            const int* __restrict__ selected, int n_layers,
                                                            float* __restrict__ dst) {
  const int l = selected[blockIdx.y];
  float* o = dst + (size_t)blockIdx.y * per_layer;
  const bool ok = l >= 0 && l < n_layers;
  const float* in = src + (size_t)(ok ? l : 0) * per_layer;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < per_layer; e += (size_t)gridDim.x * 256)
    o[e] = ok ? in[e] : __builtin_nanf("");
}

// W[sel[s]] += dW[s] (dW holds the chosen layers only, in selection order).
__global__ __launch_bounds__(256) void absorb_apply_compact_kernel(size_t per_layer4, int n_layers,
                                                                   const int* __restrict__ selected,
                                                                   const float* __restrict__ dW,
                                                                   float* __restrict__ W) {
  const int l = selected[blockIdx.y];
  if (l < 0 || l >= n_layers) return;
  const f32x4* src = (const f32x4*)(dW + (size_t)blockIdx.y * per_layer4 * 4);
  f32x4* dst = (f32x4*)(W + (size_t)l * per_layer4 * 4);
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < per_layer4; e += (size_t)gridDim.x * 256)
    dst[e] = dst[e] + src[e];
}

// W[sel[s]] += dW[sel[s]] for s < k; grid.y walks the selected layers, grid.x the elements (4 per thread).
__global__ __launch_bounds__(256) void absorb_apply_kernel(size_t per_layer4, int n_layers,
                                                           const int* __restrict__ selected,
                                                           const float* __restrict__ dW, float* __restrict__ W) {
  const int l = selected[blockIdx.y];
  if (l < 0 || l >= n_layers) return;
  const f32x4* src = (const f32x4*)(dW + (size_t)l * per_layer4 * 4);
  f32x4* dst = (f32x4*)(W + (size_t)l * per_layer4 * 4);
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < per_layer4; e += (size_t)gridDim.x * 256)
    dst[e] = dst[e] + src[e];
}

}  // namespace

ispa_status_t launch_select_layers(int32_t n_layers, const double* eps, int32_t k, int32_t* selected,
                                   int32_t* rank, hipStream_t s) {
  hipLaunchKernelGGL(select_layers_kernel, dim3(1), dim3(SEL_THREADS), 0, s, n_layers, eps, k, selected, rank);
  return hip_check(hipGetLastError(), "select_layers_kernel launch");
}

ispa_status_t launch_absorb_apply(int32_t d, int32_t d_out, int32_t n_layers, const int32_t* selected, int32_t k,
                                  const float* dW, float* W, hipStream_t s) {
  if (k == 0) return ISPA_OK;
  const size_t per4 = (size_t)d * d_out / 4;
  const unsigned bx = (unsigned)std::min<size_t>((per4 + 255) / 256, 1024);
  hipLaunchKernelGGL(absorb_apply_kernel, dim3(bx, k), dim3(256), 0, s, per4, n_layers, selected, dW, W);
  return hip_check(hipGetLastError(), "absorb_apply_kernel launch");
}

ispa_status_t launch_select_below(int32_t n_layers, const double* eps, double tau, int32_t k_max, int32_t* selected,
                                  int32_t* count, int32_t* rank, hipStream_t s) {
  hipLaunchKernelGGL(select_below_kernel, dim3(1), dim3(SEL_THREADS), 0, s, n_layers, eps, tau, k_max, selected,
                     count, rank);
  return hip_check(hipGetLastError(), "select_below_kernel launch");
}

ispa_status_t launch_gather_layers(int32_t k, size_t per_layer, const float* src, const int32_t* selected,
                                   int32_t n_layers, float* dst, hipStream_t s) {
  if (k == 0) return ISPA_OK;
  const unsigned bx = (unsigned)std::min<size_t>((per_layer + 255) / 256, 1024);
  hipLaunchKernelGGL(gather_layers_kernel, dim3(bx, k), dim3(256), 0, s, per_layer, src, selected, n_layers, dst);
  return hip_check(hipGetLastError(), "gather_layers_kernel launch");
}

ispa_status_t launch_absorb_apply_compact(int32_t d, int32_t d_out, int32_t n_layers, const int32_t* selected,
                                          int32_t k, const float* dW, float* W, hipStream_t s) {
  if (k == 0) return ISPA_OK;
  const size_t per4 = (size_t)d * d_out / 4;
  const unsigned bx = (unsigned)std::min<size_t>((per4 + 255) / 256, 1024);
  hipLaunchKernelGGL(absorb_apply_compact_kernel, dim3(bx, k), dim3(256), 0, s, per4, n_layers, selected, dW, W);
  return hip_check(hipGetLastError(), "absorb_apply_compact_kernel launch");
}

}  // namespace ispa
