// Host-side launchers shared between the C ABI (fa_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct Shape {
  int BH;     // B * H
  int Nq;     // queries per head
  int Nk;     // keys per head
  int d;      // head dimension (16, 32, 64, 128)
  bool causal;
  float scale;
};

hipError_t launch_fwd_bf16(const Shape& s, const void* Q, const void* K, const void* V, void* O,
                           float* L, hipStream_t stream);
// `workspace` holds 2 * BH * Nq floats: per-row terms written by the first of the two kernels
// this launches and read by the second.
hipError_t launch_bwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* O, const float* L, const void* dO, void* dQ, void* dK,
                           void* dV, float* workspace, hipStream_t stream);
hipError_t launch_fwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          float* O, float* L, hipStream_t stream);
hipError_t launch_bwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          const float* O, const float* L, const float* dO, float* dQ, float* dK,
                          float* dV, hipStream_t stream);

}  // namespace fa
