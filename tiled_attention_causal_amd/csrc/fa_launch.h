// Host-side launchers shared between the C ABI (fa_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kNumCUs = 256;  // MI355X

struct Shape {
  int BH;     // B * H
  int Nq;     // queries per head
  int Nk;     // keys per head
  int d;      // head dimension (16, 32, 64, 128)
  bool causal;
  float scale;
};

// Small causal grids spread each tile pair over several workgroups, whose partial results
// go to `workspace` (fwd_workspace_bytes_bf16 bytes) and are merged by a second launch. With a
// smaller workspace (or none) those grids run one workgroup per tile pair.
size_t fwd_workspace_bytes_bf16(const Shape& s);
hipError_t launch_fwd_bf16(const Shape& s, const void* Q, const void* K, const void* V, void* O,
                           float* L, float* workspace, size_t workspace_bytes,
                           hipStream_t stream);
// The bf16 backward is two launches sharing `workspace` (2 * BH * Nq floats): the first writes
// per-row terms (L log2(e) and -D) from O, L and dO, the second reads them.
hipError_t launch_bwd_prep_bf16(const Shape& s, const void* O, const float* L, const void* dO,
                                float* workspace, hipStream_t stream);
// Small square grids (Nq = Nk, a multiple of 128) spread each workgroup's steps over several
// workgroups when the workspace also holds bwd_split_workspace_bytes_bf16 bytes of fp32 partial
// sums after the per-row terms; a second launch adds them up.
size_t bwd_split_workspace_bytes_bf16(const Shape& s);
hipError_t launch_bwd_main_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                                const void* dO, void* dQ, void* dK, void* dV,
                                const float* workspace, size_t workspace_bytes,
                                hipStream_t stream);
// The nondeterministic bf16 backward main step: dQ accumulated with fp32 atomics in the
// workspace after the per-row terms (bwd_atomic_workspace_bytes_bf16 bytes in all), then
// scaled and rounded into dQ. Three launches: zero, main, convert.
size_t bwd_atomic_workspace_bytes_bf16(const Shape& s);
hipError_t launch_bwd_atomic_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                                  const void* dO, void* dQ, void* dK, void* dV, float* workspace,
                                  hipStream_t stream);
// Names of the main forward and backward kernels the launchers above run for these arguments
// and workspace sizes, as a profiler lists them (the launchers and these take the same plan).
const char* fwd_kernel_name_bf16(const Shape& s, size_t workspace_bytes);
const char* bwd_kernel_name_bf16(const Shape& s, size_t workspace_bytes);
// fp32: small grids likewise spread each workgroup's key (forward) or step (backward) range
// over several workgroups when the workspace holds fwd_workspace_bytes_f32 or
// bwd_split_workspace_bytes_f32 bytes; otherwise they run unsplit (fp32 needs no workspace).
size_t fwd_workspace_bytes_f32(const Shape& s);
size_t bwd_split_workspace_bytes_f32(const Shape& s);
// fp32 runs one forward and one backward kernel for every grid (plus a merge launch when split).
const char* fwd_kernel_name_f32(const Shape& s);
const char* bwd_kernel_name_f32(const Shape& s);
hipError_t launch_fwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          float* O, float* L, float* workspace, size_t workspace_bytes,
                          hipStream_t stream);
hipError_t launch_bwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          const float* O, const float* L, const float* dO, float* dQ, float* dK,
                          float* dV, float* workspace, size_t workspace_bytes,
                          hipStream_t stream);

}  // namespace fa
