// C ABI of the ISPA library: argument validation, device check, error state.
// The declarations and their documentation are in include/ispa.h.
#include <mutex>
#include <string>

#include "ispa_internal.h"

namespace ispa {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

ispa_status_t hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return ISPA_OK;
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return ISPA_E_HIP;
}

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];  // 1 = gfx950, 0 = other, -1 = query failed

ispa_status_t check_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device index out of range");
    return ISPA_E_UNSUPPORTED;
  }
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      g_dev_ok[dev] = -1;
      return;
    }
    g_dev_ok[dev] = std::string(prop.gcnArchName).rfind("gfx950", 0) == 0 ? 1 : 0;
  });
  if (g_dev_ok[dev] == 1) return ISPA_OK;
  if (g_dev_ok[dev] == -1) {
    set_error("hipGetDeviceProperties failed");
    return ISPA_E_HIP;
  }
  set_error("device is not gfx950 (MI355X)");
  return ISPA_E_UNSUPPORTED;
}

ispa_status_t check_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_error("hipGetDevice failed");
    return ISPA_E_HIP;
  }
  return check_device(dev);
}

ispa_status_t invalid(const std::string& msg) {
  set_error(msg);
  return ISPA_E_INVALID_ARG;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Required pointer: non-null and 16-byte aligned.  Optional: null or aligned.
bool req(const void* p) { return p != nullptr && aligned16(p); }
bool opt(const void* p) { return p == nullptr || aligned16(p); }

ispa_status_t check_attn_desc(const ispa_attn_desc_t* d, bool allow_hist) {
  if (d == nullptr) return invalid("desc is NULL");
  if (d->heads < 1) return invalid("heads must be >= 1");
  if (d->head_dim != 64 && d->head_dim != 128) return invalid("head_dim must be 64 or 128");
  if (d->n_q < 0 || d->n_loc < 1 || d->n_hist < 0) return invalid("need n_q >= 0, n_loc >= 1, n_hist >= 0");
  if (!allow_hist && d->n_hist != 0) return invalid("n_hist must be 0 here");
  if (!(d->scale > 0.f) || d->scale == INFINITY) return invalid("scale must be finite and > 0");
  if (d->dtype != ISPA_F32 && d->dtype != ISPA_BF16) return invalid("dtype must be ISPA_F32 or ISPA_BF16");
  const int64_t hd = (int64_t)d->heads * d->head_dim;
  const int64_t lim = (int64_t)1 << 31;
  if (d->n_q * hd >= lim || (d->n_loc + d->n_hist) * hd >= lim || (int64_t)d->heads * d->n_q >= lim)
    return invalid("tensor too large (2^31 elements per tensor)");
  return ISPA_OK;
}

// One local segment and, with history keys, one history segment.
KvSegments two_segments(const ispa_attn_desc_t* d, const void* Kl, const void* Vl, const void* Kh, const void* Vh) {
  KvSegments kv = {};
  kv.K[0] = Kl;
  kv.V[0] = Vl;
  kv.n[0] = d->n_loc;
  kv.n_loc_seg = 1;
  kv.n_seg = 1;
  if (d->n_hist > 0) {
    kv.K[1] = Kh;
    kv.V[1] = Vh;
    kv.n[1] = d->n_hist;
    kv.n_seg = 2;
  }
  return kv;
}

ispa_status_t check_decomp_outputs(const ispa_attn_desc_t* desc, void* O_loc, float* LSE_loc, void* O_hist,
                                   float* LSE_hist, void* O_full, float* LSE_full, void* workspace,
                                   size_t workspace_bytes) {
  if (!opt(O_loc) || !opt(LSE_loc) || !opt(O_hist) || !opt(LSE_hist) || !opt(O_full) || !opt(LSE_full) ||
      !opt(workspace))
    return invalid("output and workspace pointers must be 16-byte aligned");
  const size_t ws_need = desc->n_q < 0 || desc->n_hist < 0
                             ? 0
                             : attention_workspace_size(desc->n_q, desc->heads, desc->head_dim, desc->n_hist,
                                                        desc->dtype);
  if (O_full != nullptr && ws_need > 0 && (workspace == nullptr || workspace_bytes < ws_need)) {
    set_error("workspace smaller than ispa_decomp_attn_workspace_size()");
    return ISPA_E_WORKSPACE;
  }
  return ISPA_OK;
}

// Compute units of the current device (0 if there is none).
int32_t current_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

// Validate a segment list against desc; fill kv.
ispa_status_t check_segments(const ispa_attn_desc_t* desc, const ispa_kv_segment_t* segs, int32_t n_segs,
                             int32_t n_loc_segs, KvSegments& kv) {
  if (segs == nullptr) return invalid("segs is NULL");
  if (n_segs < 1 || n_segs > ISPA_MAX_KV_SEGMENTS) return invalid("n_segs must be in [1, ISPA_MAX_KV_SEGMENTS]");
  if (n_loc_segs < 1 || n_loc_segs > n_segs) return invalid("n_loc_segs must be in [1, n_segs]");
  int64_t sum_loc = 0, sum_hist = 0;
  kv = KvSegments{};
  for (int i = 0; i < n_segs; ++i) {
    if (segs[i].n_rows < 1) return invalid("every segment needs n_rows >= 1");
    if (!req(segs[i].K) || !req(segs[i].V)) return invalid("segment K, V must be non-NULL and 16-byte aligned");
    (i < n_loc_segs ? sum_loc : sum_hist) += segs[i].n_rows;
    kv.K[i] = segs[i].K;
    kv.V[i] = segs[i].V;
    kv.n[i] = segs[i].n_rows;
  }
  if (sum_loc != desc->n_loc || sum_hist != desc->n_hist)
    return invalid("segment rows must add up to desc->n_loc (local) and desc->n_hist (history)");
  kv.n_seg = n_segs;
  kv.n_loc_seg = n_loc_segs;
  return ISPA_OK;
}

ispa_status_t run_decomp(const ispa_attn_desc_t* desc, const void* Q, const KvSegments& kv, void* O_loc,
                         float* LSE_loc, void* O_hist, float* LSE_hist, void* O_full, float* LSE_full,
                         void* workspace, size_t workspace_bytes, void* stream, int32_t sk_workers = 0) {
  const ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  AttnArgs a = {};
  a.Q = Q;
  a.kv = kv;
  a.O_loc = O_loc;
  a.LSE_loc = LSE_loc;
  a.O_hist = O_hist;
  a.LSE_hist = LSE_hist;
  a.O_full = O_full;
  a.LSE_full = LSE_full;
  a.n_q = desc->n_q;
  a.n_loc = desc->n_loc;
  a.n_hist = desc->n_hist;
  a.heads = desc->heads;
  a.head_dim = desc->head_dim;
  a.scale = desc->scale;
  a.dtype = desc->dtype;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  a.sk_workers = sk_workers;
  return launch_attention(a, (hipStream_t)stream);
}

}  // namespace
}  // namespace ispa

using namespace ispa;

extern "C" {

size_t ispa_decomp_attn_workspace_size(const ispa_attn_desc_t* desc) {
  if (desc == nullptr || desc->n_q < 0 || desc->heads < 1 || desc->n_hist < 0) return 0;
  return attention_workspace_size(desc->n_q, desc->heads, desc->head_dim, desc->n_hist, desc->dtype);
}

ispa_status_t ispa_decomp_attn(const ispa_attn_desc_t* desc, const void* Q, const void* K_loc, const void* V_loc,
                               const void* K_hist, const void* V_hist, void* O_loc, float* LSE_loc, void* O_hist,
                               float* LSE_hist, void* O_full, float* LSE_full, void* workspace,
                               size_t workspace_bytes, void* stream) {
  ispa_status_t st = check_attn_desc(desc, true);
  if (st != ISPA_OK) return st;
  if ((desc->n_q > 0 && !req(Q)) || !req(K_loc) || !req(V_loc))
    return invalid("Q, K_loc, V_loc must be non-NULL and 16-byte aligned");
  if (desc->n_hist > 0 && (!req(K_hist) || !req(V_hist)))
    return invalid("K_hist, V_hist must be non-NULL and 16-byte aligned when n_hist > 0");
  st = check_decomp_outputs(desc, O_loc, LSE_loc, O_hist, LSE_hist, O_full, LSE_full, workspace, workspace_bytes);
  if (st != ISPA_OK) return st;
  return run_decomp(desc, Q, two_segments(desc, K_loc, V_loc, K_hist, V_hist), O_loc, LSE_loc, O_hist, LSE_hist,
                    O_full, LSE_full, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// ispa_decomp_attn_noalloc: the merge's float32 O_loc (the only scratch the decomposable attention
// needs) lives in this file-scope device array instead of a caller workspace.  Every GPU the library
// runs on holds its own copy until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in): the device address is looked up once per device with
// hipGetSymbolAddress, on the first call with that device current, and only that address is used.
namespace ispa {
namespace {
static __device__ __align__(256) unsigned char scratch[ISPA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

// Device address of `scratch` on the current device (looked up once per device).
ispa_status_t scratch_address(void** out) {
  int dev = 0;
  ispa_status_t st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st != ISPA_OK) return st;
  if (dev < 0 || dev >= kMaxScratchDevices) {
    set_error("device index above 63");
    return ISPA_E_UNSUPPORTED;
  }
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  st = hip_check(g_scratch_err[dev], "hipGetSymbolAddress(scratch)");
  if (st != ISPA_OK) return st;
  *out = g_scratch_ptr[dev];
  return ISPA_OK;
}
}  // namespace
}  // namespace ispa

extern "C" {

ispa_status_t ispa_decomp_attn_noalloc(const ispa_attn_desc_t* desc, const void* Q, const void* K_loc,
                                       const void* V_loc, const void* K_hist, const void* V_hist, void* O_loc,
                                       float* LSE_loc, void* O_hist, float* LSE_hist, void* O_full,
                                       float* LSE_full, void* stream) {
  ispa_status_t st = check_attn_desc(desc, true);
  if (st != ISPA_OK) return st;
  if ((desc->n_q > 0 && !req(Q)) || !req(K_loc) || !req(V_loc))
    return invalid("Q, K_loc, V_loc must be non-NULL and 16-byte aligned");
  if (desc->n_hist > 0 && (!req(K_hist) || !req(V_hist)))
    return invalid("K_hist, V_hist must be non-NULL and 16-byte aligned when n_hist > 0");
  if (!opt(O_loc) || !opt(LSE_loc) || !opt(O_hist) || !opt(LSE_hist) || !opt(O_full) || !opt(LSE_full))
    return invalid("output pointers must be 16-byte aligned");
  const size_t need = attention_workspace_size(desc->n_q, desc->heads, desc->head_dim, desc->n_hist, desc->dtype);
  if (need > ISPA_NOALLOC_SCRATCH_BYTES)
    return invalid("ispa_decomp_attn_noalloc: the merge needs " + std::to_string(need) +
                   " bytes of scratch (n_q * heads * head_dim * 4), above ISPA_NOALLOC_SCRATCH_BYTES = " +
                   std::to_string((size_t)ISPA_NOALLOC_SCRATCH_BYTES) + "; use ispa_decomp_attn with a workspace");
  st = check_current_device();
  if (st != ISPA_OK) return st;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != ISPA_OK) return st;
  }
  return run_decomp(desc, Q, two_segments(desc, K_loc, V_loc, K_hist, V_hist), O_loc, LSE_loc, O_hist, LSE_hist,
                    O_full, LSE_full, ws, need, stream);
}

ispa_status_t ispa_decomp_attn_segments(const ispa_attn_desc_t* desc, const void* Q, const ispa_kv_segment_t* segs,
                                        int32_t n_segs, int32_t n_loc_segs, void* O_loc, float* LSE_loc,
                                        void* O_hist, float* LSE_hist, void* O_full, float* LSE_full,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  ispa_status_t st = check_attn_desc(desc, true);
  if (st != ISPA_OK) return st;
  KvSegments kv;
  st = check_segments(desc, segs, n_segs, n_loc_segs, kv);
  if (st != ISPA_OK) return st;
  if (desc->n_q > 0 && !req(Q)) return invalid("Q must be non-NULL and 16-byte aligned");
  st = check_decomp_outputs(desc, O_loc, LSE_loc, O_hist, LSE_hist, O_full, LSE_full, workspace, workspace_bytes);
  if (st != ISPA_OK) return st;
  return run_decomp(desc, Q, kv, O_loc, LSE_loc, O_hist, LSE_hist, O_full, LSE_full, workspace, workspace_bytes,
                    stream);
}

ispa_status_t ispa_decomp_attn_fp8k(const ispa_attn_desc_t* desc, const void* Q8, const float* q_scale,
                                    const ispa_kv_segment_fp8k_t* segs, int32_t n_segs, int32_t n_loc_segs,
                                    void* O_loc, float* LSE_loc, void* O_hist, float* LSE_hist, void* O_full,
                                    float* LSE_full, void* workspace, size_t workspace_bytes, void* stream) {
  ispa_status_t st = check_attn_desc(desc, true);
  if (st != ISPA_OK) return st;
  if (desc->dtype != ISPA_BF16) return invalid("fp8-key attention: desc->dtype (V and outputs) must be ISPA_BF16");
  if (segs == nullptr) return invalid("segs is NULL");
  if (n_segs < 1 || n_segs > ISPA_MAX_KV_SEGMENTS) return invalid("n_segs must be in [1, ISPA_MAX_KV_SEGMENTS]");
  if (n_loc_segs < 1 || n_loc_segs > n_segs) return invalid("n_loc_segs must be in [1, n_segs]");
  if ((desc->n_q > 0 && !req(Q8)) || !req(q_scale)) return invalid("Q8, q_scale must be non-NULL and 16-byte aligned");
  KvSegments kv = {};
  const float* ks[MAX_KV_SEGS] = {};
  int64_t sum_loc = 0, sum_hist = 0;
  for (int i = 0; i < n_segs; ++i) {
    if (segs[i].n_rows < 1) return invalid("every segment needs n_rows >= 1");
    if (!req(segs[i].K8) || !req(segs[i].V) || !req(segs[i].k_scale))
      return invalid("segment K8, V, k_scale must be non-NULL and 16-byte aligned");
    (i < n_loc_segs ? sum_loc : sum_hist) += segs[i].n_rows;
    kv.K[i] = segs[i].K8;
    kv.V[i] = segs[i].V;
    kv.n[i] = segs[i].n_rows;
    ks[i] = segs[i].k_scale;
  }
  if (sum_loc != desc->n_loc || sum_hist != desc->n_hist)
    return invalid("segment rows must add up to desc->n_loc (local) and desc->n_hist (history)");
  kv.n_seg = n_segs;
  kv.n_loc_seg = n_loc_segs;
  st = check_decomp_outputs(desc, O_loc, LSE_loc, O_hist, LSE_hist, O_full, LSE_full, workspace, workspace_bytes);
  if (st != ISPA_OK) return st;
  st = check_current_device();
  if (st != ISPA_OK) return st;
  AttnArgs a = {};
  a.Q = Q8;
  a.kv = kv;
  a.O_loc = O_loc;
  a.LSE_loc = LSE_loc;
  a.O_hist = O_hist;
  a.LSE_hist = LSE_hist;
  a.O_full = O_full;
  a.LSE_full = LSE_full;
  a.n_q = desc->n_q;
  a.n_loc = desc->n_loc;
  a.n_hist = desc->n_hist;
  a.heads = desc->heads;
  a.head_dim = desc->head_dim;
  a.scale = desc->scale;
  a.dtype = ISPA_BF16;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  a.k_fp8 = 1;
  a.q_scale = q_scale;
  for (int i = 0; i < n_segs; ++i) a.k_scale[i] = ks[i];
  return launch_attention(a, (hipStream_t)stream);
}

size_t ispa_quantize_fp8_heads_workspace_size(int64_t n_rows, int32_t heads) {
  if (n_rows < 0 || heads < 1) return 0;
  return quant_head_workspace_size(n_rows, heads);
}

ispa_status_t ispa_quantize_fp8_heads(int64_t n_rows, int32_t heads, int32_t head_dim, int32_t dtype, const void* X,
                                      uint8_t* X8, float* scale, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (n_rows < 0 || heads < 1 || (head_dim != 64 && head_dim != 128) || heads * head_dim > quant_head_max_width())
    return invalid("need n_rows >= 0, head_dim 64 or 128, heads * head_dim <= 16384");
  if (dtype != ISPA_F32 && dtype != ISPA_BF16) return invalid("dtype must be ISPA_F32 or ISPA_BF16");
  if ((n_rows > 0 && (!req(X) || !req(X8))) || !req(scale)) return invalid("X, X8, scale must be non-NULL and 16-byte aligned");
  if (!req(workspace) || workspace_bytes < quant_head_workspace_size(n_rows, heads)) {
    set_error("ispa_quantize_fp8_heads: workspace smaller than ispa_quantize_fp8_heads_workspace_size()");
    return ISPA_E_WORKSPACE;
  }
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_quant_head(n_rows, heads, head_dim, dtype, X, X8, scale, workspace, (hipStream_t)stream);
}

ispa_status_t ispa_quantize_fp8_rows(int64_t n_rows, int32_t d, int32_t dtype, const void* X, uint8_t* X8, float* scale,
                                     void* stream) {
  if (n_rows < 0 || d < 4 || d % 4 != 0) return invalid("need n_rows >= 0 and d a positive multiple of 4");
  if (dtype != ISPA_F32 && dtype != ISPA_BF16) return invalid("dtype must be ISPA_F32 or ISPA_BF16");
  if (n_rows > 0 && (!req(X) || !req(X8) || !req(scale))) return invalid("X, X8, scale must be non-NULL and 16-byte aligned");
  if (n_rows == 0) return ISPA_OK;
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_quant_rows(n_rows, d, dtype, X, X8, scale, (hipStream_t)stream);
}

ispa_status_t ispa_quantize_fp8_cols(int32_t d, int32_t d_out, const float* W, uint8_t* W8T, float* scale,
                                     void* stream) {
  if (d < 4 || d % 4 != 0 || d_out < 1) return invalid("need d a positive multiple of 4 and d_out >= 1");
  if (!req(W) || !req(W8T) || !req(scale)) return invalid("W, W8T, scale must be non-NULL and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_quant_cols(d, d_out, W, W8T, scale, (hipStream_t)stream);
}

ispa_status_t ispa_w8a8_gemm(int64_t n, int32_t d, int32_t d_out, const uint8_t* A8, const float* a_scale,
                             const uint8_t* W8T, const float* w_scale, void* Y, void* stream) {
  if (n < 0 || d < 64 || d % 64 != 0 || d_out < 128 || d_out % 128 != 0)
    return invalid("need n >= 0, d a multiple of 64, d_out a multiple of 128");
  if (n * (int64_t)d >= ((int64_t)1 << 32) || (int64_t)d_out * d >= ((int64_t)1 << 32) || n >= ((int64_t)1 << 31))
    return invalid("operands too large (2^32 bytes each)");
  if (n > 0 && (!req(A8) || !req(a_scale) || !req(W8T) || !req(w_scale) || !req(Y)))
    return invalid("A8, a_scale, W8T, w_scale, Y must be non-NULL and 16-byte aligned");
  if (n == 0) return ISPA_OK;
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_w8a8_gemm(n, d_out, d, A8, a_scale, W8T, w_scale, (uint16_t*)Y, (hipStream_t)stream);
}

size_t ispa_decomp_attn_splitkv_workspace_size(const ispa_attn_desc_t* desc, int32_t n_workers) {
  if (desc == nullptr || desc->n_q < 0 || desc->heads < 1 || desc->n_hist < 0 || n_workers < 0 ||
      n_workers > ISPA_MAX_SPLITKV_WORKERS || (desc->head_dim != 64 && desc->head_dim != 128))
    return 0;
  const int32_t w = n_workers > 0 ? n_workers : current_cu_count();
  return splitkv_workspace_size(desc->n_q, desc->heads, desc->head_dim, desc->n_hist, w);
}

ispa_status_t ispa_decomp_attn_splitkv(const ispa_attn_desc_t* desc, const void* Q, const ispa_kv_segment_t* segs,
                                       int32_t n_segs, int32_t n_loc_segs, int32_t n_workers, void* O_loc,
                                       float* LSE_loc, void* O_hist, float* LSE_hist, void* O_full,
                                       float* LSE_full, void* workspace, size_t workspace_bytes, void* stream) {
  ispa_status_t st = check_attn_desc(desc, true);
  if (st != ISPA_OK) return st;
  if (desc->dtype != ISPA_BF16) return invalid("split-KV attention is bf16 only");
  if (n_workers < 0 || n_workers > ISPA_MAX_SPLITKV_WORKERS)
    return invalid("n_workers must be in [0, ISPA_MAX_SPLITKV_WORKERS]");
  KvSegments kv;
  st = check_segments(desc, segs, n_segs, n_loc_segs, kv);
  if (st != ISPA_OK) return st;
  if (desc->n_q > 0 && !req(Q)) return invalid("Q must be non-NULL and 16-byte aligned");
  if (!opt(O_loc) || !opt(LSE_loc) || !opt(O_hist) || !opt(LSE_hist) || !opt(O_full) || !opt(LSE_full) ||
      !opt(workspace))
    return invalid("output and workspace pointers must be 16-byte aligned");
  st = check_current_device();
  if (st != ISPA_OK) return st;
  const int32_t w = n_workers > 0 ? n_workers : current_cu_count();
  if (w < 1) return invalid("no compute units on the current device");
  const size_t need = splitkv_workspace_size(desc->n_q, desc->heads, desc->head_dim, desc->n_hist, w);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
    set_error("workspace smaller than ispa_decomp_attn_splitkv_workspace_size()");
    return ISPA_E_WORKSPACE;
  }
  return run_decomp(desc, Q, kv, O_loc, LSE_loc, O_hist, LSE_hist, O_full, LSE_full, workspace, workspace_bytes,
                    stream, w);
}

ispa_status_t ispa_full_attn(const ispa_attn_desc_t* desc, const void* Q, const void* K, const void* V, void* O,
                             float* LSE, void* stream) {
  ispa_status_t st = check_attn_desc(desc, true);
  if (st != ISPA_OK) return st;
  if ((desc->n_q > 0 && !req(Q)) || !req(K) || !req(V)) return invalid("Q, K, V must be non-NULL and 16-byte aligned");
  if (!opt(O) || !opt(LSE)) return invalid("output pointers must be 16-byte aligned");
  st = check_current_device();
  if (st != ISPA_OK) return st;
  AttnArgs a = {};
  a.Q = Q;
  a.kv.K[0] = K;
  a.kv.V[0] = V;
  a.kv.n[0] = desc->n_loc + desc->n_hist;
  a.kv.n_seg = 1;
  a.kv.n_loc_seg = 1;
  a.O_loc = O;
  a.LSE_loc = LSE;
  a.n_q = desc->n_q;
  a.n_loc = desc->n_loc + desc->n_hist;
  a.n_hist = 0;
  a.heads = desc->heads;
  a.head_dim = desc->head_dim;
  a.scale = desc->scale;
  a.dtype = desc->dtype;
  return launch_attention(a, (hipStream_t)stream);
}

ispa_status_t ispa_lse_merge(int32_t n_parts, const void* const* O_parts, const float* const* LSE_parts, int64_t n_q,
                             int32_t heads, int32_t head_dim, int32_t dtype, void* O_out, float* LSE_out,
                             void* stream) {
  if (n_parts < 1 || n_parts > 16) return invalid("n_parts must be in [1, 16]");
  if (O_parts == nullptr || LSE_parts == nullptr) return invalid("O_parts / LSE_parts is NULL");
  if (n_q < 0 || heads < 1 || (head_dim != 64 && head_dim != 128)) return invalid("bad shape");
  if (dtype != ISPA_F32 && dtype != ISPA_BF16) return invalid("bad dtype");
  for (int i = 0; i < n_parts && n_q > 0; ++i)
    if (!req(O_parts[i]) || !req(LSE_parts[i])) return invalid("part pointers must be non-NULL and 16-byte aligned");
  if ((n_q > 0 && !req(O_out)) || !opt(LSE_out)) return invalid("O_out must be non-NULL; outputs 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_lse_merge(n_parts, O_parts, LSE_parts, n_q, heads, head_dim, dtype, O_out, LSE_out,
                          (hipStream_t)stream);
}

size_t ispa_gram_workspace_size(int64_t n_rows, int32_t d, int32_t dtype) {
  if (n_rows < 0 || d <= 0) return 0;
  return gram_workspace_size(n_rows, d, dtype);
}

ispa_status_t ispa_gram_accum(int64_t n_rows, int32_t d, int32_t dtype, const void* A_loc, const void* A_full, float* G,
                              float* C, float* E, int32_t accumulate, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (n_rows < 0) return invalid("n_rows must be >= 0");
  if (dtype != ISPA_F32 && dtype != ISPA_BF16) return invalid("bad dtype");
  if (d <= 0 || (dtype == ISPA_BF16 && d % 128 != 0) || (dtype == ISPA_F32 && d % 64 != 0))
    return invalid("d must be a multiple of 128 (bf16) or 64 (f32)");
  if (accumulate != 0 && accumulate != 1) return invalid("accumulate must be 0 or 1");
  if ((n_rows > 0 && (!req(A_loc) || !req(A_full))) || !req(G) || !req(C) || !opt(E))
    return invalid("A_loc, A_full, G, C must be non-NULL and 16-byte aligned");
  if (n_rows * (int64_t)d >= ((int64_t)1 << 40)) return invalid("too many rows");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_gram(n_rows, d, dtype, A_loc, A_full, G, C, E, accumulate, workspace, workspace_bytes,
                     (hipStream_t)stream);
}

size_t ispa_absorb_workspace_size(int32_t d, int32_t d_out, int32_t batch) {
  if (d <= 0 || d_out <= 0 || batch <= 0) return 0;
  return absorb_workspace_size(d, d_out, batch);
}

ispa_status_t ispa_absorb_solve(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                                const float* W, float lambda, float* dW, float* W_new, int32_t* info, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (d <= 0 || d % 64 != 0 || d_out <= 0 || d_out % 64 != 0) return invalid("d and d_out must be multiples of 64");
  if (batch < 1 || batch > 65535) return invalid("batch must be in [1, 65535]");
  if (!(lambda >= 0.f) || lambda == INFINITY) return invalid("lambda must be finite and >= 0");
  if (!req(G) || !req(C) || !req(W) || !req(dW) || !req(info) || !opt(W_new))
    return invalid("G, C, W, dW, info must be non-NULL and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_absorb(d, d_out, batch, G, C, W, lambda, nullptr, dW, W_new, info, workspace, workspace_bytes,
                       (hipStream_t)stream);
}

ispa_status_t ispa_absorb_solve_lambdas(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                                        const float* W, const float* lambdas, float* dW, float* W_new,
                                        int32_t* info, void* workspace, size_t workspace_bytes, void* stream) {
  if (d <= 0 || d % 64 != 0 || d_out <= 0 || d_out % 64 != 0) return invalid("d and d_out must be multiples of 64");
  if (batch < 1 || batch > 65535) return invalid("batch must be in [1, 65535]");
  if (!req(G) || !req(C) || !req(W) || !req(lambdas) || !req(dW) || !req(info) || !opt(W_new))
    return invalid("G, C, W, lambdas, dW, info must be non-NULL and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_absorb(d, d_out, batch, G, C, W, 0.f, lambdas, dW, W_new, info, workspace, workspace_bytes,
                       (hipStream_t)stream);
}

ispa_status_t ispa_absorb_solve_ex(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                                   const float* W, float lambda, const float* lambdas, int32_t flags, float* dW,
                                   float* W_new, int32_t* info, void* workspace, size_t workspace_bytes,
                                   const ispa_side_stream_t* side, void* stream) {
  if (d <= 0 || d % 64 != 0 || d_out <= 0 || d_out % 64 != 0) return invalid("d and d_out must be multiples of 64");
  if (batch < 1 || batch > 65535) return invalid("batch must be in [1, 65535]");
  if ((flags & ~ISPA_ABSORB_NO_REFINE) != 0) return invalid("unknown flags");
  if (lambdas == nullptr && (!(lambda >= 0.f) || lambda == INFINITY)) return invalid("lambda must be finite and >= 0");
  if (!req(G) || !req(C) || !req(W) || !opt(lambdas) || !req(dW) || !req(info) || !opt(W_new))
    return invalid("G, C, W, dW, info must be non-NULL and 16-byte aligned");
  SideStream ss = {};
  if (side != nullptr) {
    if (side->stream == nullptr || side->ev_fork == nullptr || side->ev_join == nullptr)
      return invalid("side stream: stream, ev_fork and ev_join must all be given");
    if (side->stream == stream) return invalid("side stream must differ from the main stream");
    ss.stream = (hipStream_t)side->stream;
    ss.ev_fork = (hipEvent_t)side->ev_fork;
    ss.ev_join = (hipEvent_t)side->ev_join;
  }
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_absorb(d, d_out, batch, G, C, W, lambda, lambdas, dW, W_new, info, workspace, workspace_bytes,
                       (hipStream_t)stream, (flags & ISPA_ABSORB_NO_REFINE) == 0, side ? &ss : nullptr);
}

ispa_status_t ispa_lambda_from_trace(int32_t d, int32_t batch, const float* G, float lam_scale, float* lambdas,
                                     void* stream) {
  if (d <= 0 || batch < 1 || batch > 65535) return invalid("need d > 0 and batch in [1, 65535]");
  if (!(lam_scale >= 0.f) || lam_scale == INFINITY) return invalid("lam_scale must be finite and >= 0");
  if (!req(G) || !req(lambdas)) return invalid("G, lambdas must be non-NULL and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_trace_lambda(d, batch, G, lam_scale, lambdas, (hipStream_t)stream);
}

size_t ispa_fit_error_workspace_size(int32_t d, int32_t d_out, int32_t batch) {
  if (d <= 0 || d_out <= 0 || batch <= 0) return 0;
  return fit_error_workspace_size(d, d_out, batch);
}

ispa_status_t ispa_fit_error(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                             const float* E, const float* W, const float* dW, double* eps_abs, double* eps_rel,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (d <= 0 || d % 64 != 0 || d_out <= 0 || d_out % 64 != 0) return invalid("d and d_out must be multiples of 64");
  if (batch < 1 || batch > 65535) return invalid("batch must be in [1, 65535]");
  if (!req(G) || !req(C) || !req(E) || !req(W) || !opt(dW) || !req(eps_abs) || !req(eps_rel))
    return invalid("G, C, E, W, eps_abs, eps_rel must be non-NULL (dW may be NULL) and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_fit_error(d, d_out, batch, G, C, E, W, dW, eps_abs, eps_rel, workspace, workspace_bytes,
                          (hipStream_t)stream);
}

size_t ispa_eps_workspace_size(int32_t d, int32_t d_out, int32_t batch) {
  if (d <= 0 || d_out <= 0 || batch <= 0) return 0;
  return eps_workspace_size(d, d_out, batch);
}

ispa_status_t ispa_layer_eps(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C, const float* E,
                             const float* W, const float* dW, float lambda, double* eps_abs, double* eps_rel,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (d <= 0 || d % 64 != 0 || d_out <= 0 || d_out % 64 != 0) return invalid("d and d_out must be multiples of 64");
  if (batch < 1 || batch > 65535) return invalid("batch must be in [1, 65535]");
  if (!(lambda >= 0.f) || lambda == INFINITY) return invalid("lambda must be finite and >= 0");
  if (!req(G) || !req(C) || !req(E) || !req(W) || !req(dW) || !req(eps_abs) || !req(eps_rel))
    return invalid("all pointers must be non-NULL and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_eps(d, d_out, batch, G, C, E, W, dW, lambda, eps_abs, eps_rel, workspace, workspace_bytes,
                    (hipStream_t)stream);
}

ispa_status_t ispa_select_layers(int32_t n_layers, const double* eps, int32_t k, int32_t* selected, int32_t* rank,
                                 void* stream) {
  if (n_layers < 1 || n_layers > MAX_STACK_LAYERS) return invalid("n_layers must be in [1, 4096]");
  if (k < 0 || k > n_layers) return invalid("k must be in [0, n_layers]");
  if (!req(eps) || (k > 0 && !req(selected)) || !opt(selected) || !opt(rank))
    return invalid("eps (and selected when k > 0) must be non-NULL and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_select_layers(n_layers, eps, k, selected, rank, (hipStream_t)stream);
}

ispa_status_t ispa_select_layers_below(int32_t n_layers, const double* eps, double tau, int32_t k_max,
                                       int32_t* selected, int32_t* count, int32_t* rank, void* stream) {
  if (n_layers < 1 || n_layers > MAX_STACK_LAYERS) return invalid("n_layers must be in [1, 4096]");
  if (k_max < 0 || k_max > n_layers) return invalid("k_max must be in [0, n_layers]");
  if (tau != tau) return invalid("tau is NaN");
  if (!req(eps) || !req(count) || (k_max > 0 && !req(selected)) || !opt(selected) || !opt(rank))
    return invalid("eps, count (and selected when k_max > 0) must be non-NULL and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_select_below(n_layers, eps, tau, k_max, selected, count, rank, (hipStream_t)stream);
}

ispa_status_t ispa_gather_layers(int32_t n_layers, int64_t per_layer, const float* src, const int32_t* selected,
                                 int32_t k, float* dst, void* stream) {
  if (n_layers < 1 || n_layers > 65535 || per_layer < 1) return invalid("need n_layers in [1, 65535], per_layer >= 1");
  if (k < 0 || k > 65535) return invalid("k must be in [0, 65535]");
  if (k == 0) return ISPA_OK;
  if (!req(src) || !req(selected) || !req(dst)) return invalid("src, selected, dst must be non-NULL and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_gather_layers(k, (size_t)per_layer, src, selected, n_layers, dst, (hipStream_t)stream);
}

ispa_status_t ispa_absorb_apply_compact(int32_t d, int32_t d_out, int32_t n_layers, const int32_t* selected,
                                        int32_t k, const float* dW, float* W, void* stream) {
  if (d <= 0 || d_out <= 0 || ((int64_t)d * d_out) % 4 != 0) return invalid("d * d_out must be a positive multiple of 4");
  if (n_layers < 1 || n_layers > 65535) return invalid("n_layers must be in [1, 65535]");
  if (k < 0 || k > n_layers) return invalid("k must be in [0, n_layers]");
  if (k == 0) return ISPA_OK;
  if (!req(selected) || !req(dW) || !req(W)) return invalid("selected, dW, W must be non-NULL and 16-byte aligned");
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_absorb_apply_compact(d, d_out, n_layers, selected, k, dW, W, (hipStream_t)stream);
}

ispa_status_t ispa_absorb_apply(int32_t d, int32_t d_out, int32_t n_layers, const int32_t* selected, int32_t k,
                                const float* dW, float* W, void* stream) {
  if (d <= 0 || d_out <= 0 || ((int64_t)d * d_out) % 4 != 0) return invalid("d * d_out must be a positive multiple of 4");
  if (n_layers < 1 || n_layers > 65535) return invalid("n_layers must be in [1, 65535]");
  if (k < 0 || k > n_layers) return invalid("k must be in [0, n_layers]");
  if (k > 0 && (!req(selected) || !req(dW) || !req(W)))
    return invalid("selected, dW, W must be non-NULL and 16-byte aligned");
  if (k == 0) return ISPA_OK;
  ispa_status_t st = check_current_device();
  if (st != ISPA_OK) return st;
  return launch_absorb_apply(d, d_out, n_layers, selected, k, dW, W, (hipStream_t)stream);
}

const char* ispa_status_string(ispa_status_t s) {
  switch (s) {
    case ISPA_OK: return "ISPA_OK";
    case ISPA_E_INVALID_ARG: return "ISPA_E_INVALID_ARG";
    case ISPA_E_UNSUPPORTED: return "ISPA_E_UNSUPPORTED";
    case ISPA_E_WORKSPACE: return "ISPA_E_WORKSPACE";
    case ISPA_E_HIP: return "ISPA_E_HIP";
  }
  return "ISPA_E_UNKNOWN";
}

const char* ispa_last_error(void) { return g_last_error.c_str(); }

int32_t ispa_version(void) { return 100; }

ispa_status_t ispa_device_check(int32_t device) { return check_device(device); }

}  // extern "C"
