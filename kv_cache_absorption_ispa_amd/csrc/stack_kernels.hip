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

}  // namespace ispa
