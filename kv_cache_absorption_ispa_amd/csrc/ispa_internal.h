// Internal declarations shared by the ISPA HIP translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>
#include <type_traits>

#include "../../include/ispa.h"

namespace ispa {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int v8i_t __attribute__((ext_vector_type(8)));  // 32 fp8 codes: an operand of the f8f6f4 MFMA

// ---------------------------------------------------------------- error state
void set_error(const std::string& msg);
ispa_status_t hip_check(hipError_t e, const char* what);

// ---------------------------------------------------------------- launchers
// Keys of one attention call as segments: segments [0, n_loc_seg) form the local branch, the rest
// the history branch; each segment is a [n, H, D] K buffer and V buffer.
constexpr int MAX_KV_SEGS = ISPA_MAX_KV_SEGMENTS;
struct KvSegments {
  const void* K[MAX_KV_SEGS];
  const void* V[MAX_KV_SEGS];
  int64_t n[MAX_KV_SEGS];
  int32_t n_seg, n_loc_seg;
};

struct AttnArgs {
  const void* Q;
  KvSegments kv;
  void* O_loc;
  float* LSE_loc;
  void* O_hist;
  float* LSE_hist;
  void* O_full;
  float* LSE_full;
  int64_t n_q, n_loc, n_hist;
  int32_t heads, head_dim;
  float scale;
  int32_t dtype;
  void* ws;
  size_t ws_bytes;
  int32_t sk_workers;  // > 0: split mode with this many workgroups (bf16 only); 0: one workgroup per unit
  int32_t k_fp8;       // 1: Q and K are E4M3 codes with the scales below (V and outputs bf16)
  const float* q_scale;                 // [heads] device
  const float* k_scale[MAX_KV_SEGS];    // per segment: [heads] device
};
size_t attention_workspace_size(int64_t n_q, int32_t heads, int32_t head_dim, int64_t n_hist, int32_t dtype);
// Workspace of split mode: the merge's float32 O_loc (as above) and one partial slot per workgroup.
size_t splitkv_workspace_size(int64_t n_q, int32_t heads, int32_t head_dim, int64_t n_hist, int32_t n_workers);
ispa_status_t launch_attention(const AttnArgs& a, hipStream_t s);

ispa_status_t launch_lse_merge(int32_t n_parts, const void* const* O, const float* const* LSE, int64_t n_q,
                               int32_t heads, int32_t head_dim, int32_t dtype, void* O_out, float* LSE_out,
                               hipStream_t s);

size_t quant_head_workspace_size(int64_t n, int32_t heads);
int32_t quant_head_max_width();  // largest heads * head_dim the per-head quantiser takes
ispa_status_t launch_quant_head(int64_t n, int32_t H, int32_t D, int32_t dtype, const void* X, uint8_t* X8,
                                float* scale, void* ws, hipStream_t s);
ispa_status_t launch_quant_rows(int64_t n, int32_t d, int32_t dtype, const void* X, uint8_t* X8, float* scale,
                                hipStream_t s);
ispa_status_t launch_quant_cols(int32_t d, int32_t d_out, const float* W, uint8_t* W8T, float* scale,
                                hipStream_t s);
ispa_status_t launch_w8a8_gemm(int64_t n, int32_t N, int32_t K, const uint8_t* A8, const float* sa,
                               const uint8_t* W8T, const float* sw, uint16_t* Y, hipStream_t s);

size_t gram_workspace_size(int64_t n_rows, int32_t d, int32_t dtype);
ispa_status_t launch_gram(int64_t n_rows, int32_t d, int32_t dtype, const void* A_loc, const void* A_full,
                          float* G, float* C, float* E, int32_t accumulate, void* ws, size_t ws_bytes,
                          hipStream_t s);

size_t absorb_workspace_size(int32_t d, int32_t d_out, int32_t batch);
// A caller-owned second stream and its fork / join events (see ispa_side_stream_t).
struct SideStream {
  hipStream_t stream;
  hipEvent_t ev_fork, ev_join;
};
ispa_status_t launch_absorb(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                            const float* W, float lambda, const float* lam_b, float* dW, float* W_new,
                            int32_t* info, void* ws, size_t ws_bytes, hipStream_t s, bool refine = true,
                            const SideStream* side = nullptr);
// bf16x3 triangular applies (hi*hi + hi*lo + lo*hi): Lsplit / LTsplit hold split(L^-1) and
// split(L^-T) (2 * batch * d * d bf16 each), YTsplit and ZTsplit 2 * batch * d * d_out bf16 each.
bool apply3_supported(int32_t d, int32_t d_out);
ispa_status_t launch_split_lower(int32_t d, int32_t batch, const float* Linv, void* Lsplit, void* LTsplit,
                                 const int32_t* info, hipStream_t s);
ispa_status_t launch_chol_apply3(int32_t d, int32_t d_out, int32_t batch, const void* Lsplit, const void* LTsplit,
                                 const float* Y, void* YTsplit, void* ZTsplit, float* X, const int32_t* info,
                                 hipStream_t s);
// D = A B (A M x K, B K x N, D M x N; float32, row-major, batched) from three-part bf16 splits of A and
// B^T, float64-accumulated slabs; M, N, K multiples of 128.  asplit / bsplit: three planes of
// batch * M * K and batch * K * N bf16 each, scratch.  max_wg > 0 bounds the product's workgroups.
ispa_status_t launch_prod6(int32_t M, int32_t N, int32_t K, int32_t batch, const float* A, const float* B, float* D,
                           void* const asplit[3], void* const bsplit[3], const int32_t* info, hipStream_t s,
                           int max_wg = 0);
// r = R - G X + gamma X (gamma * gamma_b[b] per layer if gamma_b) from exact int8 digit-slice
// products of G and X (Ozaki's splitting, five digits, 15 int8 products, ~2^-35 relative to the row
// and column scales); d, d_out multiples of 128.  gplanes / xplanes: digit planes (the first five
// used) of batch * d * d and batch * d_out * d bytes; scales: residual_i8_scale_bytes bytes.  All
// scratch.
bool residual_i8_supported(int32_t d, int32_t d_out);
size_t residual_i8_scale_bytes(int32_t d, int32_t d_out, int32_t batch);
ispa_status_t launch_residual_i8(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* X,
                                 const float* R, double gamma, const float* gamma_b, float* r,
                                 void* const gplanes[6], void* const xplanes[6], void* scales, const int32_t* info,
                                 hipStream_t s);
size_t fit_error_workspace_size(int32_t d, int32_t d_out, int32_t batch);
ispa_status_t launch_fit_error(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                               const float* E, const float* W, const float* dW, double* eps_abs, double* eps_rel,
                               void* ws, size_t ws_bytes, hipStream_t s);
ispa_status_t launch_trace_lambda(int32_t d, int32_t batch, const float* G, float scale, float* lam, hipStream_t s);
ispa_status_t launch_select_below(int32_t n_layers, const double* eps, double tau, int32_t k_max, int32_t* selected,
                                  int32_t* count, int32_t* rank, hipStream_t s);
ispa_status_t launch_gather_layers(int32_t k, size_t per_layer, const float* src, const int32_t* selected,
                                   int32_t n_layers, float* dst, hipStream_t s);
ispa_status_t launch_absorb_apply_compact(int32_t d, int32_t d_out, int32_t n_layers, const int32_t* selected,
                                          int32_t k, const float* dW, float* W, hipStream_t s);

size_t eps_workspace_size(int32_t d, int32_t d_out, int32_t batch);
ispa_status_t launch_eps(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                         const float* E, const float* W, const float* dW, float lambda, double* eps_abs,
                         double* eps_rel, void* ws, size_t ws_bytes, hipStream_t s);

constexpr int MAX_STACK_LAYERS = 4096;
ispa_status_t launch_select_layers(int32_t n_layers, const double* eps, int32_t k, int32_t* selected,
                                   int32_t* rank, hipStream_t s);
ispa_status_t launch_absorb_apply(int32_t d, int32_t d_out, int32_t n_layers, const int32_t* selected, int32_t k,
                                  const float* dW, float* W, hipStream_t s);

// ---------------------------------------------------------------- device helpers
// Map a linear workgroup id so that ids dispatched to the same XCD (the
// hardware deals workgroups round-robin over the 8 XCDs) get consecutive
// logical ids: tiles that share operands then share one XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblocks) {
  constexpr uint32_t NXCD = 8;
  const uint32_t xcd = bid % NXCD;
  const uint32_t slot = bid / NXCD;
  const uint32_t q = nblocks / NXCD, r = nblocks % NXCD;
  // XCDs < r hold q+1 blocks, the rest hold q.
  const uint32_t base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  return base + slot;
}

// ---------------------------------------------------------------- buffer / LDS helpers (gfx950)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_DW3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// Buffer resource over `bytes` bytes: loads at offsets >= bytes return 0 (hardware range check),
// which masks the ragged last tile of each branch without branches.
__device__ __forceinline__ rsrc_t make_rsrc(const void* ptr, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ptr), (short)0, (int)bytes, RSRC_DW3);
}

typedef short bf16x4_raw __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) void lds_void;

// Transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane i
// receives element (i % 4) of the 8-byte words addressed by lanes i/4, 4 + i/4,
// 8 + i/4 and 12 + i/4 of its group.
// (The gfx950-only builtins below are hidden from the host compilation pass,
// which otherwise drops the kernel's launch stub.)
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  const bf16x4_raw r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bf16x4_raw*)(p));
  return __builtin_bit_cast(u32x2, r);
#else
  return u32x2{0, 0};
#endif
}

// One wave moves 64 x 16 bytes from the buffer (at per-lane byte offset `voffset`) to LDS,
// lane i's 16 bytes landing at lds_base + 16 i.  Offsets past the buffer's size read 0.
__device__ __forceinline__ void load_to_lds(rsrc_t r, uint16_t* lds_base, uint32_t voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voffset, 0, 0, 0);
#endif
}

}  // namespace ispa
