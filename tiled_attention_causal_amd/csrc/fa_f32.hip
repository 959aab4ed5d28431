// float32 attention forward and backward on the vector ALUs (no rounding below fp32
// anywhere). This is the exact-arithmetic path for fp32 inputs; the bf16 path in fa_bf16.hip
// is the one built for throughput.
//
// Method: "Systems and Parallelism" (CS336 field map, A2), section 1.2-1.3, problems
// flash_forward (online softmax over key tiles, L = m + log l) and flash_backward
// (P = exp(S - L), D = rowsum(dO o O), dS = P o (dP - D), scale in dQ and dK), with the
// two-pass backward split of section 1.3.3.
//
// Each row (a query, or a key in the dK/dV pass) is owned by TPR = d/16 consecutive lanes,
// each holding 16 of its d columns; dot products over d finish with group_sum<TPR>. The
// moving rows are staged 32 at a time in LDS.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kT = 32;  // moving rows per LDS tile

template <int D>
struct F32Cfg {
  static constexpr int TPR = D / 16;    // lanes per row
  static constexpr int RPB = 256 / TPR;  // rows per workgroup
};

__device__ __forceinline__ void ld16(float (&x)[16], const float* p) {
#pragma unroll
  for (int i = 0; i < 16; i += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
    x[i] = v[0];
    x[i + 1] = v[1];
    x[i + 2] = v[2];
    x[i + 3] = v[3];
  }
}

template <int D>
__device__ __forceinline__ void stage_rows(float* tile, const float* head, int row0, int nrows) {
  for (int i = threadIdx.x; i < kT * D / 4; i += 256) {
    const int row = i / (D / 4), c4 = i % (D / 4);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (row0 + row < nrows) v = *reinterpret_cast<const f32x4*>(head + (size_t)(row0 + row) * D + 4 * c4);
    *reinterpret_cast<f32x4*>(tile + row * D + 4 * c4) = v;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      float* __restrict__ O,
                                                      float* __restrict__ Lout, int Nq, int Nk,
                                                      float scale) {
  constexpr int TPR = F32Cfg<D>::TPR, RPB = F32Cfg<D>::RPB;
  __shared__ __attribute__((aligned(16))) float sK[kT * D];
  __shared__ __attribute__((aligned(16))) float sV[kT * D];
  const int nrt = (Nq + RPB - 1) / RPB;
  const int bh = blockIdx.x / nrt, rt = blockIdx.x % nrt;
  const int r0 = rt * RPB;
  const int row = r0 + threadIdx.x / TPR, part = threadIdx.x % TPR;
  const float* Qh = Q + (size_t)bh * Nq * D;
  const float* Kh = K + (size_t)bh * Nk * D;
  const float* Vh = V + (size_t)bh * Nk * D;

  float q[16], acc[16];
  if (row < Nq) ld16(q, Qh + (size_t)row * D + 16 * part);
  else
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(r0 + RPB, Nq));  // keys <= last row of this workgroup
  for (int k0 = 0; k0 < kend; k0 += kT) {
    __syncthreads();
    stage_rows<D>(sK, Kh, k0, Nk);
    stage_rows<D>(sV, Vh, k0, Nk);
    __syncthreads();
    float s[kT];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kT; ++j) {
      float kk[16];
      ld16(kk, sK + j * D + 16 * part);
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) dot = fmaf(q[i], kk[i], dot);
      dot = group_sum<TPR>(dot) * scale;
      const int key = k0 + j;
      if (key >= Nk || (CAUSAL && key > row)) dot = -INFINITY;
      s[j] = dot;
      mx = fmaxf(mx, dot);
    }
    const float mnew = fmaxf(m, mx);
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = expf(m - mref);
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kT; ++j) {
      const float p = expf(s[j] - mref);
      rs += p;
      float vv[16];
      ld16(vv, sV + j * D + 16 * part);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = fmaf(p, vv[i], acc[i]);
    }
    l = l * alpha + rs;
    m = mnew;
  }
  if (row < Nq) {
    const float inv = 1.f / l;
    float* Op = O + ((size_t)bh * Nq + row) * D + 16 * part;
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *reinterpret_cast<f32x4*>(Op + i) = f32x4{acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv,
                                                acc[i + 3] * inv};
    if (part == 0) Lout[(size_t)bh * Nq + row] = m + logf(l);
  }
}

// dK, dV: workgroup owns RPB keys and walks the query rows that can see them.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ O, const float* __restrict__ L, const float* __restrict__ dO,
    float* __restrict__ dK, float* __restrict__ dV, int Nq, int Nk, float scale) {
  constexpr int TPR = F32Cfg<D>::TPR, RPB = F32Cfg<D>::RPB;
  __shared__ __attribute__((aligned(16))) float sQ[kT * D];
  __shared__ __attribute__((aligned(16))) float sdO[kT * D];
  __shared__ float sL[kT], sD[kT];
  const int nrt = (Nk + RPB - 1) / RPB;
  const int bh = blockIdx.x / nrt, rt = blockIdx.x % nrt;
  const int r0 = rt * RPB;
  const int key = r0 + threadIdx.x / TPR, part = threadIdx.x % TPR;
  const size_t oq = (size_t)bh * Nq * D, ok = (size_t)bh * Nk * D;

  float k[16], v[16], dk[16], dv[16];
  if (key < Nk) {
    ld16(k, K + ok + (size_t)key * D + 16 * part);
    ld16(v, V + ok + (size_t)key * D + 16 * part);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) k[i] = v[i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) dk[i] = dv[i] = 0.f;

  const int qstart = CAUSAL ? (r0 / kT) * kT : 0;
  for (int m0 = qstart; m0 < Nq; m0 += kT) {
    __syncthreads();
    stage_rows<D>(sQ, Q + oq, m0, Nq);
    stage_rows<D>(sdO, dO + oq, m0, Nq);
    if (threadIdx.x < kT) {
      const int qi = m0 + threadIdx.x;
      float dsum = 0.f, lv = 0.f;
      if (qi < Nq) {
        const float* op = O + oq + (size_t)qi * D;
        const float* gp = dO + oq + (size_t)qi * D;
        for (int i = 0; i < D; ++i) dsum = fmaf(gp[i], op[i], dsum);
        lv = L[(size_t)bh * Nq + qi];
      }
      sL[threadIdx.x] = lv;
      sD[threadIdx.x] = dsum;
    }
    __syncthreads();
    for (int j = 0; j < kT; ++j) {
      const int qi = m0 + j;
      float qq[16], gg[16];
      ld16(qq, sQ + j * D + 16 * part);
      ld16(gg, sdO + j * D + 16 * part);
      float sdot = 0.f, pdot = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sdot = fmaf(qq[i], k[i], sdot);
        pdot = fmaf(gg[i], v[i], pdot);
      }
      sdot = group_sum<TPR>(sdot);
      pdot = group_sum<TPR>(pdot);
      const bool vis = qi < Nq && (!CAUSAL || key <= qi);
      const float p = vis ? expf(sdot * scale - sL[j]) : 0.f;
      const float ds = p * (pdot - sD[j]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dv[i] = fmaf(p, gg[i], dv[i]);
        dk[i] = fmaf(ds, qq[i], dk[i]);
      }
    }
  }
  if (key < Nk) {
    float* kp = dK + ok + (size_t)key * D + 16 * part;
    float* vp = dV + ok + (size_t)key * D + 16 * part;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      *reinterpret_cast<f32x4*>(kp + i) =
          f32x4{dk[i] * scale, dk[i + 1] * scale, dk[i + 2] * scale, dk[i + 3] * scale};
      *reinterpret_cast<f32x4*>(vp + i) = f32x4{dv[i], dv[i + 1], dv[i + 2], dv[i + 3]};
    }
  }
}

// dQ: workgroup owns RPB queries and walks the keys they can see.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ O, const float* __restrict__ L, const float* __restrict__ dO,
    float* __restrict__ dQ, int Nq, int Nk, float scale) {
  constexpr int TPR = F32Cfg<D>::TPR, RPB = F32Cfg<D>::RPB;
  __shared__ __attribute__((aligned(16))) float sK[kT * D];
  __shared__ __attribute__((aligned(16))) float sV[kT * D];
  const int nrt = (Nq + RPB - 1) / RPB;
  const int bh = blockIdx.x / nrt, rt = blockIdx.x % nrt;
  const int r0 = rt * RPB;
  const int row = r0 + threadIdx.x / TPR, part = threadIdx.x % TPR;
  const size_t oq = (size_t)bh * Nq * D, ok = (size_t)bh * Nk * D;

  float q[16], g[16], dq[16];
  float dsum = 0.f, lv = 0.f;
  if (row < Nq) {
    float o[16];
    ld16(q, Q + oq + (size_t)row * D + 16 * part);
    ld16(g, dO + oq + (size_t)row * D + 16 * part);
    ld16(o, O + oq + (size_t)row * D + 16 * part);
#pragma unroll
    for (int i = 0; i < 16; ++i) dsum = fmaf(g[i], o[i], dsum);
    lv = L[(size_t)bh * Nq + row];
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = g[i] = 0.f;
  }
  dsum = group_sum<TPR>(dsum);
#pragma unroll
  for (int i = 0; i < 16; ++i) dq[i] = 0.f;

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(r0 + RPB, Nq));
  for (int k0 = 0; k0 < kend; k0 += kT) {
    __syncthreads();
    stage_rows<D>(sK, K + ok, k0, Nk);
    stage_rows<D>(sV, V + ok, k0, Nk);
    __syncthreads();
    for (int j = 0; j < kT; ++j) {
      const int key = k0 + j;
      float kk[16], vv[16];
      ld16(kk, sK + j * D + 16 * part);
      ld16(vv, sV + j * D + 16 * part);
      float sdot = 0.f, pdot = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sdot = fmaf(q[i], kk[i], sdot);
        pdot = fmaf(g[i], vv[i], pdot);
      }
      sdot = group_sum<TPR>(sdot);
      pdot = group_sum<TPR>(pdot);
      const bool vis = row < Nq && key < Nk && (!CAUSAL || key <= row);
      const float p = vis ? expf(sdot * scale - lv) : 0.f;
      const float ds = p * (pdot - dsum);
#pragma unroll
      for (int i = 0; i < 16; ++i) dq[i] = fmaf(ds, kk[i], dq[i]);
    }
  }
  if (row < Nq) {
    float* qp = dQ + oq + (size_t)row * D + 16 * part;
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *reinterpret_cast<f32x4*>(qp + i) =
          f32x4{dq[i] * scale, dq[i + 1] * scale, dq[i + 2] * scale, dq[i + 3] * scale};
  }
}

template <int D, bool CAUSAL>
hipError_t fwd_t(const Shape& s, const float* Q, const float* K, const float* V, float* O,
                 float* L, hipStream_t stream) {
  const long long grid = (long long)((s.Nq + F32Cfg<D>::RPB - 1) / F32Cfg<D>::RPB) * s.BH;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, Q,
                     K, V, O, L, s.Nq, s.Nk, s.scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t bwd_t(const Shape& s, const float* Q, const float* K, const float* V, const float* O,
                 const float* L, const float* dO, float* dQ, float* dK, float* dV,
                 hipStream_t stream) {
  constexpr int RPB = F32Cfg<D>::RPB;
  const long long gkv = (long long)((s.Nk + RPB - 1) / RPB) * s.BH;
  if (gkv > 0) {
    hipLaunchKernelGGL((dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)gkv), dim3(256), 0, stream,
                       Q, K, V, O, L, dO, dK, dV, s.Nq, s.Nk, s.scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long gq = (long long)((s.Nq + RPB - 1) / RPB) * s.BH;
  if (gq > 0) {
    hipLaunchKernelGGL((dq_f32_kernel<D, CAUSAL>), dim3((unsigned)gq), dim3(256), 0, stream, Q,
                       K, V, O, L, dO, dQ, s.Nq, s.Nk, s.scale);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_fwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          float* O, float* L, hipStream_t stream) {
#define FA_F(DD)                                                 \
  case DD:                                                       \
    return s.causal ? fwd_t<DD, true>(s, Q, K, V, O, L, stream)  \
                    : fwd_t<DD, false>(s, Q, K, V, O, L, stream);
  switch (s.d) {
    FA_F(16)
    FA_F(32)
    FA_F(64)
    FA_F(128)
    default:
      return hipErrorInvalidValue;
  }
#undef FA_F
}

hipError_t launch_bwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          const float* O, const float* L, const float* dO, float* dQ, float* dK,
                          float* dV, hipStream_t stream) {
#define FA_B(DD)                                                                  \
  case DD:                                                                        \
    return s.causal ? bwd_t<DD, true>(s, Q, K, V, O, L, dO, dQ, dK, dV, stream)   \
                    : bwd_t<DD, false>(s, Q, K, V, O, L, dO, dQ, dK, dV, stream);
  switch (s.d) {
    FA_B(16)
    FA_B(32)
    FA_B(64)
    FA_B(128)
    default:
      return hipErrorInvalidValue;
  }
#undef FA_B
}

}  // namespace fa
