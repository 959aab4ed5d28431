// float32 attention forward and backward on the fp32 matrix cores (v_mfma_f32_32x32x2_f32:
// fp32 operands, fp32 accumulation; nothing is rounded below fp32).
//
// Method: "Systems and Parallelism" (CS336 field map, A2), section 1.2-1.3, problems
// flash_forward (online softmax over key tiles, L = m + log l) and flash_backward
// (P = exp(S - L), D = rowsum(dO o O), dS = P o (dP - D), scale in dQ and dK), with the
// two-pass backward split of section 1.3.3.
//
// The 32x32x2 instruction: lane l gives A[l%32][l/32] and B[l/32][l%32], and register r of
// lane l receives C[8(r/4) + 4(l/32) + r%4][l%32]. Every product here runs its reduction in
// steps sigma of two, lane half g supplying index perm(sigma, g) = 8(sigma/4) + 4g + sigma%4:
// over d that lets a lane read its operands as 16-byte groups (d = 8t + 4g .. +3 for steps
// 4t .. 4t+3), and over 32 keys or queries it is exactly the row order of a C fragment, so a
// product's output registers feed the next product as its B operand with no data movement:
//   forward:  S^T = K Q^T (keys in registers, queries on lanes), P^T from S^T, O^T += V^T P^T;
//   dK, dV:   S = Q K^T and dP = dO V^T (queries in registers, keys on lanes),
//             dV^T += dO^T P and dK^T += Q^T dS;
//   dQ:       S^T = K Q^T and dP^T = V dO^T, dQ^T += K^T dS^T.
// The stationary operand of each kernel (Q; K and V; Q and dO) sits in registers; the moving
// rows stream through double-buffered LDS tiles of 32 rows (direct loads, swizzled chunks).
// Rows past a head's end load as zeros and are masked or never stored.
#include <algorithm>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kMinSteps = 8, kMaxShares = 8;  // split grids: see f32_ways

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 32 fp32 rows of D columns in LDS: the bf16-unit Tile with twice the columns (same bytes).
template <int D>
struct FTile {
  using T = Tile<32, 2 * D>;
  static constexpr int NCH = D / 4;  // 16-byte chunks per row
  static constexpr int ELEMS = T::ELEMS;
  __device__ __forceinline__ static void load(rsrc_t src, int row0, bf16* t, int w, int lane) {
    T::template load<4>(src, row0, t, w, lane);
  }
  // Columns 4c .. 4c+3 of row r.
  __device__ __forceinline__ static f32x4 quad(const bf16* t, int r, int c) {
    return *reinterpret_cast<const f32x4*>(t + swz<NCH>(r, c));
  }
  // Column col of row r.
  __device__ __forceinline__ static float at(const bf16* t, int r, int col) {
    return *reinterpret_cast<const float*>(t + swz<NCH>(r, col >> 2) + 2 * (col & 3));
  }
};

// Row `row` of a head as this lane's operand groups: x[t] = columns 8t + 4g .. +3.
template <int D>
__device__ __forceinline__ void load_row_quads(f32x4 (&x)[D / 8], rsrc_t head, int row, int g) {
#pragma unroll
  for (int t = 0; t < D / 8; ++t)
    x[t] = __builtin_bit_cast(f32x4, buf_load16(head, (uint32_t)((row * D + 8 * t + 4 * g) * 4)));
}

// C^T += (rows from LDS)·(registers): c += sum over d of A[i][d] b[j][d], with A row i = lane
// l32 of the LDS tile and b this lane's register quads (perm order over d).
template <int D>
__device__ __forceinline__ f32x16 rows_times_regs(const bf16* tile, int l32, int g,
                                                  const f32x4 (&b)[D / 8], f32x16 c) {
#pragma unroll
  for (int t = 0; t < D / 8; ++t) {
    const f32x4 a = FTile<D>::quad(tile, l32, 2 * t + g);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = mfma_f32(a[e], b[t][e], c);
  }
  return c;
}

// acc[db] += (LDS tile rows transposed)·(32-row C fragment p): acc[db][d][j] += sum over the
// tile's 32 rows u of tile[u][32 db + d] p[u][j], with p this lane's registers (row perm order).
template <int D>
__device__ __forceinline__ void cols_times_frag(const bf16* tile, int l32, int g,
                                                const f32x16& p, f32x16 (&acc)[(D + 31) / 32]) {
#pragma unroll
  for (int db = 0; db < (D + 31) / 32; ++db) {
    int col = 32 * db + l32;
    if constexpr (D < 32) col &= D - 1;  // d = 16: the block's unused half re-reads valid columns
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int u = 8 * (s >> 2) + 4 * g + (s & 3);
      acc[db] = mfma_f32(FTile<D>::at(tile, u, col), p[s], acc[db]);
    }
  }
}

// Store a transposed accumulator as rows: lane owns row `row`, register r of block db holds
// column 32db + 8(r/4) + 4g + r%4.
template <int D>
__device__ __forceinline__ void store_rows_f32(float* out_row, const f32x16 (&acc)[(D + 31) / 32],
                                               float mul, int g) {
#pragma unroll
  for (int db = 0; db < (D + 31) / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * g;
      if (d0 < D)
        *reinterpret_cast<f32x4*>(out_row + d0) =
            f32x4{acc[db][4 * j] * mul, acc[db][4 * j + 1] * mul, acc[db][4 * j + 2] * mul,
                  acc[db][4 * j + 3] * mul};
    }
}

template <int D>
__device__ __forceinline__ void negate_quads(f32x4 (&x)[D / 8]) {
#pragma unroll
  for (int t = 0; t < D / 8; ++t) x[t] = -x[t];
}

// Runs step(n, cur) for n = first .. last-1 over tiles that fetch(n, dst) loads straight into
// LDS, one tile ahead, through two buffers. The loop is unrolled by two inside one function
// whose buffers are restrict parameters, so every access names its buffer statically: the
// compiler can tell that a step's LDS reads of `cur` do not alias the loads in flight into
// the other buffer and does not wait for those loads before reading.
template <class Fetch, class Step>
__device__ __forceinline__ void stream2(int first, int last, bf16* __restrict__ b0,
                                        bf16* __restrict__ b1, Fetch&& fetch, Step&& step) {
  if (first < last) fetch(first, b0);
  wait_vmem();
  __syncthreads();
  for (int n = first; n < last; n += 2) {
    if (n + 1 < last) fetch(n + 1, b1);
    step(n, b0);
    wait_vmem();
    __syncthreads();
    if (n + 1 < last) {
      if (n + 2 < last) fetch(n + 2, b0);
      step(n + 1, b1);
      wait_vmem();
      __syncthreads();
    }
  }
}

// Forward: 128 query rows per workgroup (32 per wave, one per lane; the lane halves split the
// keys of each tile), key tiles of 32.
//
// Small grids spread each query tile's key tiles over ns workgroups (consecutive blocks, in
// dispatch order, so that every XCD gets an even mix of long and short shares): share sw runs
// the sw-th of ns equal slices and writes its partial (unnormalised O, m, l) per lane to
// part + ((bh nqt + it) ns + sw) XS 256, component k of thread t at k 256 + t, for
// fwd_f32_combine_kernel to merge.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      float* __restrict__ O,
                                                      float* __restrict__ Lout, int Nq, int Nk,
                                                      float scale, int ns,
                                                      float* __restrict__ part) {
  constexpr int DB = (D + 31) / 32, NT = D / 8, XS = 16 * DB + 2;
  using FT = FTile<D>;
  constexpr int TE = FT::ELEMS;
  __shared__ __attribute__((aligned(1024))) bf16 buf0[2 * TE];  // K tile, then V tile
  __shared__ __attribute__((aligned(1024))) bf16 buf1[2 * TE];
  const int nqt = (Nq + 127) / 128;
  const int lid = ns > 1 ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  const int sw = lid % ns, pid = lid / ns;
  const int bh = pid / nqt, it = CAUSAL ? nqt - 1 - pid % nqt : pid % nqt;  // longest first
  const int q0 = it * 128;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int qw0 = q0 + 32 * w, qrow = qw0 + l32;
  const rsrc_t Qr = make_rsrc(Q + (size_t)bh * Nq * D, (uint32_t)Nq * D * 4);
  const rsrc_t Kr = make_rsrc(K + (size_t)bh * Nk * D, (uint32_t)Nk * D * 4);
  const rsrc_t Vr = make_rsrc(V + (size_t)bh * Nk * D, (uint32_t)Nk * D * 4);
  const float cs = fabsf(scale), c = exp2_coef(scale);

  // With a negative scale the scores are taken of -Q, so that every score below is
  // multiplied by |scale| and the row maxima stay maxima.
  f32x4 qf[NT];
  load_row_quads<D>(qf, Qr, qrow, g);
  if (scale < 0.f) negate_quads<D>(qf);
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  float m = -INFINITY, l = 0.f;  // row max of the raw scores, this lane half's sum of p

  const int kend = CAUSAL ? min(Nk, min(q0 + 128, Nq)) : Nk;  // keys the last row can see
  const int nkt = (kend + 31) / 32;
  const int lo = sw * nkt / ns, hi = (sw + 1) * nkt / ns;
  auto fetch = [&](int kt, bf16* dst) {
    FT::load(Kr, kt * 32, dst, w, lane);
    FT::load(Vr, kt * 32, dst + TE, w, lane);
  };
  auto step = [&](int kt, const bf16* cur) {
    const bf16* ck = cur;
    const bf16* cv = cur + TE;
    const int k0 = kt * 32;
    if (!CAUSAL || k0 <= qw0 + 31) {
      // S^T: register r holds key k0 + 8(r/4) + 4g + r%4 against this lane's query.
      f32x16 s[1] = {rows_times_regs<D>(ck, l32, g, qf, zero16())};
      if ((CAUSAL && k0 + 31 > qw0) || k0 + 32 > Nk)
        mask_scores<1>(s, 0, min(CAUSAL ? qrow - k0 - 4 * g : 1 << 30, Nk - 1 - k0 - 4 * g));
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
      const float mnew = fmaxf(m, halves_max(mx));
      const float mref = mnew == -INFINITY ? 0.f : mnew;  // no visible key yet: all p = 0
      const float alpha = fast_exp2((m - mref) * c);
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[0][r] = fast_exp2((s[0][r] - mref) * c);
        ps += s[0][r];
      }
      l = l * alpha + ps;
      m = mnew;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      cols_times_frag<D>(cv, l32, g, s[0], o);
    }
  };
  stream2(lo, hi, buf0, buf1, fetch, step);

  if (ns > 1) {
    float* x = part + ((size_t)(bh * nqt + it) * ns + sw) * XS * 256 + tid;
    asm volatile("" : "+v"(x));  // address formed here, not held through the loop
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[(16 * db + r) * 256] = o[db][r];
    x[16 * DB * 256] = m;
    x[(16 * DB + 1) * 256] = l;
    return;
  }
  const float lt = halves_sum(l);
  if (qrow < Nq) {
    store_rows_f32<D>(O + ((size_t)bh * Nq + qrow) * D, o, 1.f / lt, g);
    if (g == 0) Lout[(size_t)bh * Nq + qrow] = m * cs + logf(lt);
  }
}

// Merges the ns partial records fwd_f32_kernel wrote for each 128-row query tile, with the
// rescale the online softmax applies between key tiles, and stores O and L. Thread t takes
// record lane t % 256 (the kernel's lane and wave, so the two lane halves of a row sum their
// l as in the kernel) and 32-column block t / 256; all of its loads are independent. A share
// with no visible key for a row has m = -inf and l = O = 0: weight 0.
template <int D>
__global__ __launch_bounds__(256 * ((D + 31) / 32)) void fwd_f32_combine_kernel(
    const float* __restrict__ part, float* __restrict__ O, float* __restrict__ Lout, int Nq,
    float scale, int ns) {
  constexpr int DB = (D + 31) / 32, XS = 16 * DB + 2, MAXW = kMaxShares;
  const int nqt = (Nq + 127) / 128;
  const int bh = blockIdx.x / nqt, it = blockIdx.x % nqt;
  const int slot = threadIdx.x & 255, db = threadIdx.x >> 8;
  const int lane = slot & 63, w = slot >> 6, g = lane >> 5, l32 = lane & 31;
  const float cs = fabsf(scale), c = exp2_coef(scale);
  const float* x0 = part + (size_t)blockIdx.x * ns * XS * 256 + slot;
  // Loads are unconditional (shares past ns re-read the last one and get weight 0), so the
  // compiler can issue them all before the first use.
  float mw[MAXW], lw[MAXW];
#pragma unroll
  for (int sh = 0; sh < MAXW; ++sh) {
    const float* x = x0 + (size_t)min(sh, ns - 1) * XS * 256;
    mw[sh] = x[16 * DB * 256];
    lw[sh] = x[(16 * DB + 1) * 256];
  }
  float mm = mw[0];
#pragma unroll
  for (int sh = 1; sh < MAXW; ++sh) mm = fmaxf(mm, mw[sh]);
  const float mref = mm == -INFINITY ? 0.f : mm;
  f32x16 o = zero16();
  float l = 0.f;
#pragma unroll
  for (int sh = 0; sh < MAXW; ++sh) {
    const float f = sh < ns ? fast_exp2((mw[sh] - mref) * c) : 0.f;
    const float* x = x0 + (size_t)min(sh, ns - 1) * XS * 256 + 16 * db * 256;
    l += f * lw[sh];
#pragma unroll
    for (int r = 0; r < 16; ++r) o[r] += f * x[r * 256];
  }
  const float lt = halves_sum(l);
  const int qrow = it * 128 + 32 * w + l32;
  if (qrow < Nq) {
    float* orow = O + ((size_t)bh * Nq + qrow) * D;
    const float inv = 1.f / lt;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * g;
      if (d0 < D)
        *reinterpret_cast<f32x4*>(orow + d0) =
            f32x4{o[4 * j] * inv, o[4 * j + 1] * inv, o[4 * j + 2] * inv, o[4 * j + 3] * inv};
    }
    if (g == 0 && db == 0) Lout[(size_t)bh * Nq + qrow] = mm * cs + logf(lt);
  }
}

// Backward. Per head the workgroups run the dK/dV key tiles (128 keys each, longest first)
// and then the dQ query tiles (128 queries each, longest first).
template <int D>
struct F32Bwd {
  static constexpr int DB = (D + 31) / 32, NT = D / 8;
  static constexpr int TE = FTile<D>::ELEMS;
  // dK/dV: Q, dO and O tiles per buffer; dQ: K and V tiles per buffer.
  static constexpr int SMEM = 2 * 3 * TE;
};

// dK, dV for keys k0 .. k0+127. Per 32-query step: D_q = dO_q . O_q from the staged O and dO
// (each wave for itself, through its own 32 words of LDS), L for the step's queries from
// global memory (16 per lane), then the four products.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_f32(bf16* smem, float* sdelta, rsrc_t Qr, rsrc_t Kr,
                                         rsrc_t Vr, rsrc_t Or, rsrc_t Lr, rsrc_t dOr,
                                         float* dKh, float* dVh, int k0, int Nq, int Nk,
                                         float scale, int sw, int ns, float* part) {
  using B = F32Bwd<D>;
  using FT = FTile<D>;
  constexpr int DB = B::DB, NT = B::NT, TE = B::TE;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int kw0 = k0 + 32 * w, krow = kw0 + l32;
  const float c = exp2_coef(scale);

  f32x4 kf[NT], vf[NT];
  load_row_quads<D>(kf, Kr, krow, g);
  load_row_quads<D>(vf, Vr, krow, g);
  if (scale < 0.f) negate_quads<D>(kf);  // scores of -K: |scale| applies, as in the forward
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }
  float* wdelta = sdelta + 32 * w;

  const int nmt = (Nq + 31) / 32;
  const int mt0 = CAUSAL ? min(k0 / 32, nmt) : 0;
  const int lo = mt0 + sw * (nmt - mt0) / ns, hi = mt0 + (sw + 1) * (nmt - mt0) / ns;
  auto fetch = [&](int mt, bf16* dst) {
    FT::load(Qr, mt * 32, dst, w, lane);
    FT::load(dOr, mt * 32, dst + TE, w, lane);
    FT::load(Or, mt * 32, dst + 2 * TE, w, lane);
  };
  auto step = [&](int mt, const bf16* cur) {
    const bf16* cq = cur;
    const bf16* cdo = cur + TE;
    const bf16* co = cur + 2 * TE;
    const int m0 = mt * 32;
    if (!CAUSAL || m0 + 31 >= kw0) {
      // D for query m0 + l32 (lane halves take alternate column quads), to this wave's LDS.
      float dd = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 x = FT::quad(cdo, l32, 2 * t + g), y = FT::quad(co, l32, 2 * t + g);
        dd += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
      }
      dd = halves_sum(dd);
      if (g == 0) wdelta[l32] = dd;
      // L and D of this lane's 16 queries m0 + 8j + 4g + e (register 4j + e); L one word
      // at a time, so that a ragged end reads zeros past Nq only.
      f32x4 lq[4], dq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          lq[j][e] = buf_load_f32(Lr, (uint32_t)((m0 + 8 * j + 4 * g + e) * 4));
        dq[j] = *reinterpret_cast<const f32x4*>(wdelta + 8 * j + 4 * g);
      }
      // S = Q K^T and dP = dO V^T: register r holds query m0 + 8(r/4) + 4g + r%4, lane = key.
      f32x16 s[1] = {rows_times_regs<D>(cq, l32, g, kf, zero16())};
      f32x16 dp = rows_times_regs<D>(cdo, l32, g, vf, zero16());
      if ((CAUSAL && m0 < kw0 + 31) || m0 + 32 > Nq)
        mask_scores<1>(s, CAUSAL ? krow - m0 - 4 * g : -(1 << 30), Nq - 1 - m0 - 4 * g);
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[0][r] * c - lq[r >> 2][r & 3] * kLog2e);
        s[0][r] = p;
        ds[r] = p * (dp[r] - dq[r >> 2][r & 3]);
      }
      cols_times_frag<D>(cdo, l32, g, s[0], dv);  // dV^T += dO^T P
      cols_times_frag<D>(cq, l32, g, ds, dk);     // dK^T += Q^T dS
    }
  };
  stream2(lo, hi, smem, smem + 3 * TE, fetch, step);

  if (ns > 1) {  // Nq = Nk, a multiple of 128: every row exists
    float* x = part + (((size_t)(krow / 64) * ns + sw) * 2 * 64 + krow % 64) * D;
    asm volatile("" : "+v"(x));
    store_rows_f32<D>(x, dk, 1.f, g);
    store_rows_f32<D>(x + 64 * D, dv, 1.f, g);
  } else if (krow < Nk) {
    store_rows_f32<D>(dKh + (size_t)krow * D, dk, scale, g);
    store_rows_f32<D>(dVh + (size_t)krow * D, dv, 1.f, g);
  }
}

// dQ for queries q0 .. q0+127: Q, dO, L and D of the lane's query stay in registers.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_f32(bf16* smem, rsrc_t Qr, rsrc_t Kr, rsrc_t Vr, rsrc_t Or,
                                       rsrc_t Lr, rsrc_t dOr, float* dQh, int q0, int Nq,
                                       int Nk, float scale, int sw, int ns, float* part) {
  using B = F32Bwd<D>;
  using FT = FTile<D>;
  constexpr int DB = B::DB, NT = B::NT, TE = B::TE;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int qw0 = q0 + 32 * w, qrow = qw0 + l32;
  const float c = exp2_coef(scale);

  f32x4 qf[NT], dof[NT];
  load_row_quads<D>(qf, Qr, qrow, g);
  load_row_quads<D>(dof, dOr, qrow, g);
  float dd = 0.f;
  {
    f32x4 of[NT];
    load_row_quads<D>(of, Or, qrow, g);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      dd += dof[t][0] * of[t][0] + dof[t][1] * of[t][1] + dof[t][2] * of[t][2] +
            dof[t][3] * of[t][3];
  }
  dd = halves_sum(dd);
  const float l2 = buf_load_f32(Lr, (uint32_t)(qrow * 4)) * kLog2e;
  if (scale < 0.f) negate_quads<D>(qf);
  f32x16 dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = zero16();

  int nkt = (Nk + 31) / 32;
  if (CAUSAL) nkt = min(nkt, (min(q0 + 128, Nq) - 1) / 32 + 1);
  const int lo = sw * nkt / ns, hi = (sw + 1) * nkt / ns;
  auto fetch = [&](int kt, bf16* dst) {
    FT::load(Kr, kt * 32, dst, w, lane);
    FT::load(Vr, kt * 32, dst + TE, w, lane);
  };
  auto step = [&](int kt, const bf16* cur) {
    const bf16* ck = cur;
    const bf16* cv = cur + TE;
    const int k0 = kt * 32;
    if (!CAUSAL || k0 <= qw0 + 31) {
      // S^T and dP^T: register r holds key k0 + 8(r/4) + 4g + r%4, lane = query.
      f32x16 s[1] = {rows_times_regs<D>(ck, l32, g, qf, zero16())};
      f32x16 dp = rows_times_regs<D>(cv, l32, g, dof, zero16());
      if ((CAUSAL && k0 + 31 > qw0) || k0 + 32 > Nk)
        mask_scores<1>(s, 0, min(CAUSAL ? qrow - k0 - 4 * g : 1 << 30, Nk - 1 - k0 - 4 * g));
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(s[0][r] * c - l2) * (dp[r] - dd);
      cols_times_frag<D>(ck, l32, g, ds, dqa);  // dQ^T += K^T dS^T
    }
  };
  stream2(lo, hi, smem, smem + 3 * TE, fetch, step);
  if (ns > 1) {
    float* x = part + ((size_t)(qrow / 64) * ns + sw) * 64 * D + (size_t)(qrow % 64) * D;
    asm volatile("" : "+v"(x));
    store_rows_f32<D>(x, dqa, 1.f, g);
  } else if (qrow < Nq) {
    store_rows_f32<D>(dQh + (size_t)qrow * D, dqa, scale, g);
  }
}

// Small grids (Nq = Nk = N, N % 128 == 0) spread each workgroup's steps over ns workgroups,
// in dispatch order, as in the forward; share sw writes unscaled fp32 partial sums per 64-row
// tile t of head bh as [64][D] rows: dK^T and dV^T at kvpart + ((bh T + t) ns + sw) 2 * 64 D
// (dV^T after dK^T), dQ^T at qpart + ((bh T + t) ns + sw) 64 D, T = N / 64, for
// bwd_f32_combine_kernel to add up.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ O, const float* __restrict__ L, const float* __restrict__ dO,
    float* __restrict__ dQ, float* __restrict__ dK, float* __restrict__ dV, int Nq, int Nk,
    float scale, int ns, float* __restrict__ kvpart, float* __restrict__ qpart) {
  __shared__ __attribute__((aligned(1024))) bf16 smem[F32Bwd<D>::SMEM];
  __shared__ __attribute__((aligned(16))) float sdelta[4 * 32];
  const int nkv = (Nk + 127) / 128, nqw = (Nq + 127) / 128, per_head = nkv + nqw;
  const int lid = ns > 1 ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  const int sw = lid % ns, pid = lid / ns;
  const int bh = pid / per_head, idx = pid % per_head;
  const size_t head_part = (size_t)bh * (Nq / 64) * ns * 64 * D;  // one tensor's tiles per head
  const size_t oq = (size_t)bh * Nq * D, ok = (size_t)bh * Nk * D;
  const uint32_t bq = (uint32_t)Nq * D * 4, bk = (uint32_t)Nk * D * 4;
  const rsrc_t Qr = make_rsrc(Q + oq, bq), Or = make_rsrc(O + oq, bq), dOr = make_rsrc(dO + oq, bq);
  const rsrc_t Kr = make_rsrc(K + ok, bk), Vr = make_rsrc(V + ok, bk);
  const rsrc_t Lr = make_rsrc(L + (size_t)bh * Nq, (uint32_t)Nq * 4);
  if (idx < nkv) {
    dkdv_f32<D, CAUSAL>(smem, sdelta, Qr, Kr, Vr, Or, Lr, dOr, dK + ok, dV + ok, idx * 128, Nq,
                        Nk, scale, sw, ns, ns > 1 ? kvpart + 2 * head_part : nullptr);
  } else {
    const int it = CAUSAL ? nqw - 1 - (idx - nkv) : idx - nkv;
    dq_f32<D, CAUSAL>(smem, Qr, Kr, Vr, Or, Lr, dOr, dQ + oq, it * 128, Nq, Nk, scale, sw, ns,
                      ns > 1 ? qpart + head_part : nullptr);
  }
}

// Adds the ns partial [64][D] tiles bwd_f32_kernel wrote for each 64-row tile, scales dK and
// dQ, and stores dQ, dK and dV: one float4 of one tensor per thread, summed over the shares
// with independent loads; a tile's three tensors take 3 * 64 * D / 1024 workgroups.
template <int D>
__global__ __launch_bounds__(256) void bwd_f32_combine_kernel(
    const float* __restrict__ kvpart, const float* __restrict__ qpart, float* __restrict__ dQ,
    float* __restrict__ dK, float* __restrict__ dV, int N, float scale, int ns) {
  constexpr int MAXW = 8, TILE = 64 * D, BLOCKS = 3 * TILE / 1024;
  const int T = N / 64;
  const int tb = blockIdx.x / BLOCKS, blk = blockIdx.x % BLOCKS;
  const int tile = tb % T, bh = tb / T;
  const size_t base = ((size_t)bh * T + tile) * ns;
  const int e = blk * 1024 + 4 * threadIdx.x;
  const int tensor = e / TILE, k = e % TILE;  // 0: dK, 1: dV, 2: dQ
  const float* x = tensor < 2 ? kvpart + base * 2 * TILE + tensor * TILE + k
                              : qpart + base * TILE + k;
  const size_t stride = tensor < 2 ? 2 * TILE : TILE;
  f32x4 v[MAXW];
#pragma unroll
  for (int w = 0; w < MAXW; ++w)
    if (w < ns) v[w] = *reinterpret_cast<const f32x4*>(x + w * stride);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < MAXW; ++w)
    if (w < ns) acc += v[w];
  float* out = tensor == 0 ? dK : (tensor == 1 ? dV : dQ);
  *reinterpret_cast<f32x4*>(out + ((size_t)bh * N + 64 * tile) * D + k) =
      acc * (tensor == 1 ? 1.f : scale);
}

// Workgroups per workgroup for small fp32 grids: doubling (up to 8) while every share keeps
// at least kMinSteps steps of 32 rows and the grid stays within the CUs' room for the kernel's
// workgroups (two per CU at d <= 64, one at d = 128), or twice that for causal grids, whose
// shares differ in length: dispatched longest first, the short ones fill in behind the long.
int f32_ways(long long wgs, int steps, const Shape& s) {
  const long long room = (long long)kNumCUs * (s.d <= 64 ? 2 : 1) * (s.causal ? 2 : 1);
  int ns = 1;
  while (ns < kMaxShares && wgs * ns * 2 <= room && steps / (ns * 2) >= kMinSteps) ns *= 2;
  return ns;
}
int fwd_f32_ways(const Shape& s) {
  const int steps = ((s.causal ? std::min(s.Nq, s.Nk) : s.Nk) + 31) / 32;  // longest tile's
  return f32_ways((long long)((s.Nq + 127) / 128) * s.BH, steps, s);
}
int bwd_f32_ways(const Shape& s) {
  if (s.Nq != s.Nk || s.Nq % 128 != 0) return 1;  // partial sums come in 64-row tiles
  return f32_ways((long long)(s.Nq / 64) * s.BH, s.Nq / 32, s);
}

template <int D, bool CAUSAL>
hipError_t fwd_t(const Shape& s, const float* Q, const float* K, const float* V, float* O,
                 float* L, float* ws, size_t ws_bytes, hipStream_t stream) {
  const long long tiles = (long long)((s.Nq + 127) / 128) * s.BH;
  int ns = fwd_f32_ways(s);
  if (ns > 1 && (ws == nullptr || ws_bytes < fwd_workspace_bytes_f32(s))) ns = 1;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(tiles * ns)), dim3(256), 0,
                     stream, Q, K, V, O, L, s.Nq, s.Nk, s.scale, ns, ws);
  if (ns > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fwd_f32_combine_kernel<D>), dim3((unsigned)tiles),
                       dim3(256 * ((D + 31) / 32)), 0, stream, (const float*)ws, O, L, s.Nq,
                       s.scale, ns);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t bwd_t(const Shape& s, const float* Q, const float* K, const float* V, const float* O,
                 const float* L, const float* dO, float* dQ, float* dK, float* dV, float* ws,
                 size_t ws_bytes, hipStream_t stream) {
  const long long grid = (long long)((s.Nk + 127) / 128 + (s.Nq + 127) / 128) * s.BH;
  if (grid == 0) return hipSuccess;
  int ns = bwd_f32_ways(s);
  const size_t split_bytes = (size_t)(s.Nq / 64) * s.BH * ns * 3 * 64 * D * sizeof(float);
  if (ns > 1 && (ws == nullptr || ws_bytes < split_bytes ||
                 (reinterpret_cast<uintptr_t>(ws) & 15u) != 0))
    ns = 1;
  const long long tiles = (long long)(s.Nq / 64) * s.BH;
  float* kvpart = ws;
  float* qpart = ns > 1 ? ws + (size_t)tiles * ns * 2 * 64 * D : nullptr;
  hipLaunchKernelGGL((bwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(grid * ns)), dim3(256), 0,
                     stream, Q, K, V, O, L, dO, dQ, dK, dV, s.Nq, s.Nk, s.scale, ns, kvpart,
                     qpart);
  if (ns > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_f32_combine_kernel<D>), dim3((unsigned)(tiles * (3 * 64 * D / 1024))),
                       dim3(256), 0, stream, (const float*)kvpart, (const float*)qpart, dQ, dK,
                       dV, s.Nq, s.scale, ns);
  }
  return hipGetLastError();
}

}  // namespace

size_t fwd_workspace_bytes_f32(const Shape& s) {
  const int ns = fwd_f32_ways(s);
  if (ns == 1) return 0;
  const size_t xs = 16 * ((s.d + 31) / 32) + 2;  // floats per lane in a partial record
  return (size_t)((s.Nq + 127) / 128) * s.BH * ns * xs * 256 * sizeof(float);
}

size_t bwd_split_workspace_bytes_f32(const Shape& s) {
  // The size does not depend on the call being causal: room for either.
  Shape c = s, n = s;
  c.causal = true;
  n.causal = false;
  const int ns = std::max(bwd_f32_ways(c), bwd_f32_ways(n));
  if (ns == 1) return 0;
  return (size_t)(s.Nq / 64) * s.BH * ns * 3 * 64 * s.d * sizeof(float);
}

const char* fwd_kernel_name_f32(const Shape& s) {
  static const char* const names[2][4] = {
      {"fwd_f32_kernel<16, false>", "fwd_f32_kernel<32, false>", "fwd_f32_kernel<64, false>",
       "fwd_f32_kernel<128, false>"},
      {"fwd_f32_kernel<16, true>", "fwd_f32_kernel<32, true>", "fwd_f32_kernel<64, true>",
       "fwd_f32_kernel<128, true>"}};
  const int di = s.d == 16 ? 0 : s.d == 32 ? 1 : s.d == 64 ? 2 : 3;
  return names[s.causal ? 1 : 0][di];
}

const char* bwd_kernel_name_f32(const Shape& s) {
  static const char* const names[2][4] = {
      {"bwd_f32_kernel<16, false>", "bwd_f32_kernel<32, false>", "bwd_f32_kernel<64, false>",
       "bwd_f32_kernel<128, false>"},
      {"bwd_f32_kernel<16, true>", "bwd_f32_kernel<32, true>", "bwd_f32_kernel<64, true>",
       "bwd_f32_kernel<128, true>"}};
  const int di = s.d == 16 ? 0 : s.d == 32 ? 1 : s.d == 64 ? 2 : 3;
  return names[s.causal ? 1 : 0][di];
}

hipError_t launch_fwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          float* O, float* L, float* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
#define FA_F(DD)                                                                          \
  case DD:                                                                                \
    return s.causal ? fwd_t<DD, true>(s, Q, K, V, O, L, workspace, workspace_bytes, stream) \
                    : fwd_t<DD, false>(s, Q, K, V, O, L, workspace, workspace_bytes, stream);
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
                          float* dV, float* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
#define FA_B(DD)                                                                      \
  case DD:                                                                            \
    return s.causal ? bwd_t<DD, true>(s, Q, K, V, O, L, dO, dQ, dK, dV, workspace,    \
                                      workspace_bytes, stream)                        \
                    : bwd_t<DD, false>(s, Q, K, V, O, L, dO, dQ, dK, dV, workspace,   \
                                       workspace_bytes, stream);
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
