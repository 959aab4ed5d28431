// C ABI of libfa.so (declared in include/fa.h): argument validation and kernel dispatch.
// Nothing here allocates, and no error leaves as a C++ exception.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

// Per-head buffers are addressed with 32-bit byte offsets: N * d * 2 < 2^31 for d <= 128.
constexpr int64_t kMaxN = int64_t(1) << 22;
constexpr int64_t kMaxBH = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxGroups = (int64_t(1) << 24) - 1;

bool supported_d(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by both entry points; on success fills *s. Pointer checks come later,
// once the caller knows which tensors a call will touch.
fa_status check_common(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                       float scale, int is_causal, fa::Shape* s) {
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERROR_NOT_SUPPORTED;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d <= 0) return FA_ERROR_INVALID_VALUE;
  if (!supported_d(d)) return FA_ERROR_NOT_SUPPORTED;
  if (!isfinite(scale)) return FA_ERROR_INVALID_VALUE;
  if (Nq > kMaxN || Nk > kMaxN) return FA_ERROR_NOT_SUPPORTED;
  if (H != 0 && B > kMaxBH / H) return FA_ERROR_NOT_SUPPORTED;
  const int64_t BH = B * H;
  // Launch grids count work-items in 32 bits: with 256-thread workgroups every grid here
  // stays below BH * (ceil(Nq/32) + ceil(Nk/32)) < 2^24 workgroups.
  if (BH > 0 && ((Nq + 31) / 32 + (Nk + 31) / 32) > (kMaxGroups / BH))
    return FA_ERROR_NOT_SUPPORTED;
  s->BH = static_cast<int>(BH);
  s->Nq = static_cast<int>(Nq);
  s->Nk = static_cast<int>(Nk);
  s->d = static_cast<int>(d);
  s->causal = is_causal != 0;
  s->scale = scale;
  return FA_SUCCESS;
}

bool bad_ptr(const void* p) { return p == nullptr || !aligned16(p); }

}  // namespace

// fa_backward_noalloc's workspace: one array per GPU, part of the library's device code object,
// so it exists on a device once the library's code is loaded there and lives until the
// process ends. Host code never uses this name as an address (on the host it is only a
// stand-in for the symbol): scratch_address() gives each device's address.
static __device__ __align__(256) unsigned char scratch[FA_BACKWARD_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the stream's device, looked up once per device with that
// device current and kept.
hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status status) {
  switch (status) {
    case FA_SUCCESS:
      return "FA_SUCCESS";
    case FA_ERROR_INVALID_VALUE:
      return "FA_ERROR_INVALID_VALUE";
    case FA_ERROR_NOT_SUPPORTED:
      return "FA_ERROR_NOT_SUPPORTED";
    case FA_ERROR_LAUNCH_FAILED:
      return "FA_ERROR_LAUNCH_FAILED";
    case FA_ERROR_SCRATCH_TOO_SMALL:
      return "FA_ERROR_SCRATCH_TOO_SMALL";
  }
  return "FA_UNKNOWN_STATUS";
}

// The part of the backward workspace every bf16 call needs: L log2(e) and -D per query row
// (two floats); the fp32 path needs nothing.
static size_t backward_rows_bytes(fa_dtype dtype, const fa::Shape& s) {
  return dtype == FA_DTYPE_BF16 ? (size_t)s.BH * (size_t)s.Nq * 2 * sizeof(float) : 0;
}

size_t fa_backward_workspace_bytes(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                   int64_t d) {
  fa::Shape s;
  if (check_common(dtype, B, H, Nq, Nk, d, 1.f, 0, &s) != FA_SUCCESS) return 0;
  const size_t rows = backward_rows_bytes(dtype, s);
  // Room for the partial sums of small grids (the larger of the causal and the non-causal
  // call's), after the per-row terms (bf16 only).
  if (dtype == FA_DTYPE_F32) return fa::bwd_split_workspace_bytes_f32(s);
  return rows > 0 ? rows + fa::bwd_split_workspace_bytes_bf16(s) : 0;
}

size_t fa_forward_workspace_bytes(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                  int64_t d, int is_causal) {
  fa::Shape s;
  if (check_common(dtype, B, H, Nq, Nk, d, 1.f, is_causal, &s) != FA_SUCCESS) return 0;
  return dtype == FA_DTYPE_BF16 ? fa::fwd_workspace_bytes_bf16(s)
                                : fa::fwd_workspace_bytes_f32(s);
}

fa_status fa_forward_with_workspace(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                    int64_t d, const void* Q, const void* K, const void* V,
                                    int is_causal, float scale, void* O, float* L,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa::Shape s;
  const fa_status st = check_common(dtype, B, H, Nq, Nk, d, scale, is_causal, &s);
  if (st != FA_SUCCESS) return st;
  if (workspace_bytes > 0 &&
      (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0))
    return FA_ERROR_INVALID_VALUE;
  if ((int64_t)s.BH * Nq == 0) return FA_SUCCESS;
  if (Nk == 0) return FA_ERROR_INVALID_VALUE;  // softmax over no keys
  if (bad_ptr(Q) || bad_ptr(K) || bad_ptr(V) || bad_ptr(O) || L == nullptr ||
      (reinterpret_cast<uintptr_t>(L) & 3u) != 0)
    return FA_ERROR_INVALID_VALUE;
  const hipStream_t hs = stream;
  hipError_t e;
  if (dtype == FA_DTYPE_BF16)
    e = fa::launch_fwd_bf16(s, Q, K, V, O, L, static_cast<float*>(workspace), workspace_bytes,
                            hs);
  else
    e = fa::launch_fwd_f32(s, static_cast<const float*>(Q), static_cast<const float*>(K),
                           static_cast<const float*>(V), static_cast<float*>(O), L,
                           static_cast<float*>(workspace), workspace_bytes, hs);
  return e == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILED;
}

fa_status fa_forward(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                     const void* Q, const void* K, const void* V, int is_causal, float scale,
                     void* O, float* L, hipStream_t stream) {
  return fa_forward_with_workspace(dtype, B, H, Nq, Nk, d, Q, K, V, is_causal, scale, O, L,
                                   nullptr, 0, stream);
}

const char* fa_forward_kernel_name(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                   int64_t Nk, int64_t d, int is_causal,
                                   size_t workspace_bytes) {
  fa::Shape s;
  if (check_common(dtype, B, H, Nq, Nk, d, 1.f, is_causal, &s) != FA_SUCCESS) return "";
  return dtype == FA_DTYPE_BF16 ? fa::fwd_kernel_name_bf16(s, workspace_bytes)
                                : fa::fwd_kernel_name_f32(s);
}

const char* fa_backward_kernel_name(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                    int64_t Nk, int64_t d, int is_causal,
                                    size_t workspace_bytes) {
  fa::Shape s;
  if (check_common(dtype, B, H, Nq, Nk, d, 1.f, is_causal, &s) != FA_SUCCESS) return "";
  return dtype == FA_DTYPE_BF16 ? fa::bwd_kernel_name_bf16(s, workspace_bytes)
                                : fa::bwd_kernel_name_f32(s);
}

// Validation shared by fa_backward and fa_backward_main (which read the same arguments).
static fa_status check_backward(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                int64_t d, const void* Q, const void* K, const void* V,
                                const void* O, const float* L, const void* dO, int is_causal,
                                float scale, void* dQ, void* dK, void* dV, void* workspace,
                                size_t workspace_bytes, fa::Shape* s, bool* nothing,
                                bool check_workspace = true) {
  const fa_status st = check_common(dtype, B, H, Nq, Nk, d, scale, is_causal, s);
  if (st != FA_SUCCESS) return st;
  const size_t ws_need = backward_rows_bytes(dtype, *s);
  if (check_workspace) {
    if (workspace_bytes < ws_need) return FA_ERROR_INVALID_VALUE;
    if (ws_need > 0 &&
        (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0))
      return FA_ERROR_INVALID_VALUE;
  }
  const bool has_q = (int64_t)s->BH * Nq > 0, has_k = (int64_t)s->BH * Nk > 0;
  *nothing = !has_q && !has_k;
  if (*nothing) return FA_SUCCESS;
  if (has_q && Nk == 0) return FA_ERROR_INVALID_VALUE;  // softmax over no keys
  if (has_q && (bad_ptr(Q) || bad_ptr(O) || bad_ptr(dO) || bad_ptr(dQ) || L == nullptr ||
                (reinterpret_cast<uintptr_t>(L) & 3u) != 0))
    return FA_ERROR_INVALID_VALUE;
  if (has_k && (bad_ptr(K) || bad_ptr(V) || bad_ptr(dK) || bad_ptr(dV)))
    return FA_ERROR_INVALID_VALUE;
  return FA_SUCCESS;
}

fa_status fa_backward_preprocess(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t d,
                                 const void* O, const float* L, const void* dO,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa::Shape s;
  // Keys play no part here; Nk = 0 keeps the size checks to the query side.
  const fa_status st = check_common(dtype, B, H, Nq, 0, d, 1.f, 0, &s);
  if (st != FA_SUCCESS) return st;
  const size_t ws_need = backward_rows_bytes(dtype, s);
  if (workspace_bytes < ws_need) return FA_ERROR_INVALID_VALUE;
  if (ws_need == 0) return FA_SUCCESS;  // fp32, or no query rows: nothing to precompute
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0 ||
      bad_ptr(O) || bad_ptr(dO) || L == nullptr || (reinterpret_cast<uintptr_t>(L) & 3u) != 0)
    return FA_ERROR_INVALID_VALUE;
  const hipError_t e = fa::launch_bwd_prep_bf16(s, O, L, dO, static_cast<float*>(workspace),
                                                stream);
  return e == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILED;
}

fa_status fa_backward_main(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                           int64_t d, const void* Q, const void* K, const void* V,
                           const void* O, const float* L, const void* dO, int is_causal,
                           float scale, void* dQ, void* dK, void* dV, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  fa::Shape s;
  bool nothing = false;
  const fa_status st = check_backward(dtype, B, H, Nq, Nk, d, Q, K, V, O, L, dO, is_causal,
                                      scale, dQ, dK, dV, workspace, workspace_bytes, &s,
                                      &nothing);
  if (st != FA_SUCCESS || nothing) return st;
  const hipStream_t hs = stream;
  hipError_t e;
  if (dtype == FA_DTYPE_BF16)
    e = fa::launch_bwd_main_bf16(s, Q, K, V, dO, dQ, dK, dV,
                                 static_cast<const float*>(workspace), workspace_bytes, hs);
  else
    e = fa::launch_bwd_f32(s, static_cast<const float*>(Q), static_cast<const float*>(K),
                           static_cast<const float*>(V), static_cast<const float*>(O), L,
                           static_cast<const float*>(dO), static_cast<float*>(dQ),
                           static_cast<float*>(dK), static_cast<float*>(dV),
                           static_cast<float*>(workspace), workspace_bytes, hs);
  return e == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILED;
}

fa_status fa_backward(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                      const void* Q, const void* K, const void* V, const void* O,
                      const float* L, const void* dO, int is_causal, float scale, void* dQ,
                      void* dK, void* dV, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  fa::Shape s;
  bool nothing = false;
  fa_status st = check_backward(dtype, B, H, Nq, Nk, d, Q, K, V, O, L, dO, is_causal, scale,
                                dQ, dK, dV, workspace, workspace_bytes, &s, &nothing);
  if (st != FA_SUCCESS || nothing) return st;
  st = fa_backward_preprocess(dtype, B, H, Nq, d, O, L, dO, workspace, workspace_bytes, stream);
  if (st != FA_SUCCESS) return st;
  return fa_backward_main(dtype, B, H, Nq, Nk, d, Q, K, V, O, L, dO, is_causal, scale, dQ, dK,
                          dV, workspace, workspace_bytes, stream);
}

fa_status fa_backward_noalloc(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                              int64_t d, const void* Q, const void* K, const void* V,
                              const void* O, const float* L, const void* dO, int is_causal,
                              float scale, void* dQ, void* dK, void* dV, hipStream_t stream) {
  fa::Shape s;
  bool nothing = false;
  // Every argument is checked before the first HIP call.
  fa_status st = check_backward(dtype, B, H, Nq, Nk, d, Q, K, V, O, L, dO, is_causal, scale,
                                dQ, dK, dV, nullptr, 0, &s, &nothing, false);
  if (st != FA_SUCCESS) return st;
  if (backward_rows_bytes(dtype, s) > FA_BACKWARD_NOALLOC_MAX_BYTES)
    return FA_ERROR_SCRATCH_TOO_SMALL;
  if (nothing) return FA_SUCCESS;
  void* ws = nullptr;
  if (scratch_address(stream, &ws) != hipSuccess) return FA_ERROR_LAUNCH_FAILED;
  st = fa_backward_preprocess(dtype, B, H, Nq, d, O, L, dO, ws, FA_BACKWARD_NOALLOC_MAX_BYTES,
                              stream);
  if (st != FA_SUCCESS) return st;
  return fa_backward_main(dtype, B, H, Nq, Nk, d, Q, K, V, O, L, dO, is_causal, scale, dQ, dK,
                          dV, ws, FA_BACKWARD_NOALLOC_MAX_BYTES, stream);
}

size_t fa_backward_atomic_workspace_bytes(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                          int64_t Nk, int64_t d) {
  fa::Shape s;
  if (dtype != FA_DTYPE_BF16 || check_common(dtype, B, H, Nq, Nk, d, 1.f, 0, &s) != FA_SUCCESS)
    return 0;
  return fa::bwd_atomic_workspace_bytes_bf16(s);
}

fa_status fa_backward_atomic(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                             int64_t d, const void* Q, const void* K, const void* V,
                             const void* O, const float* L, const void* dO, int is_causal,
                             float scale, void* dQ, void* dK, void* dV, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  fa::Shape s;
  bool nothing = false;
  fa_status st = check_backward(dtype, B, H, Nq, Nk, d, Q, K, V, O, L, dO, is_causal, scale,
                                dQ, dK, dV, workspace, workspace_bytes, &s, &nothing);
  if (st != FA_SUCCESS || nothing) return st;
  if (dtype != FA_DTYPE_BF16) return FA_ERROR_NOT_SUPPORTED;
  if (workspace_bytes < fa::bwd_atomic_workspace_bytes_bf16(s)) return FA_ERROR_INVALID_VALUE;
  st = fa_backward_preprocess(dtype, B, H, Nq, d, O, L, dO, workspace, workspace_bytes, stream);
  if (st != FA_SUCCESS) return st;
  const hipError_t e =
      fa::launch_bwd_atomic_bf16(s, Q, K, V, dO, dQ, dK, dV, static_cast<float*>(workspace),
                                 stream);
  return e == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILED;
}

}  // extern "C"
