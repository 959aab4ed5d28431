// bf16 attention forward and backward for gfx950 (CDNA4): 32x32x16 bf16 MFMA with fp32
// accumulation; streaming tiles land in LDS straight from HBM (buffer loads with the LDS
// destination) and transposed MFMA operands are read with ds_read_b64_tr_b16.
//
// Method: "Systems and Parallelism" (CS336 field map, A2), section 1.2-1.3.
//   forward  (problem flash_forward): each workgroup owns one query tile and walks the key
//            tiles once, keeping a running row max m and row sum l, rescaling the output
//            accumulator by exp(m_prev - m_new), and writes O = acc / l and L = m + log l.
//            Causal: key tiles entirely above the diagonal are never visited and only tiles
//            that straddle it pay for the index comparison (section 1.3.3's early exit and
//            diagonal/full tile split).
//   backward (problem flash_backward, split as in section 1.3.3): P = exp(S - L) rebuilt from
//            Q, K and L; D = rowsum(dO o O); dS = P o (dP - D). One kind of workgroup owns a
//            key tile and walks query tiles for dK and dV, another owns a query tile and walks
//            key tiles for dQ, so nothing is accumulated atomically. Both kinds are one launch.
//
// Register layout used throughout (see mfma32 in fa_common.h): each wave owns 32 rows of the
// stationary side (queries in the forward and dQ pass, keys in the dK/dV pass) and holds
// them as MFMA B operands, so every score tile comes out with one stationary row per lane
// (lane % 32) and the moving rows spread over the 16 accumulator registers. Row statistics
// are then per lane, plus one exchange with lane ^ 32. The second product of each pass
// (P V, P^T dO, dS^T Q, dS K) takes the score registers directly as its B operand and reads
// its LDS operand transposed (Tile::tfrag).
#include <algorithm>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

__device__ __forceinline__ bf16x8 negate(bf16x8 x) {
  u32x4 u = __builtin_bit_cast(u32x4, x);
  u ^= 0x80008000u;
  return __builtin_bit_cast(bf16x8, u);
}

// Stationary-row fragments: lane holds row `row`, d = 16s + 8g .. +7 for every step s.
template <int D>
__device__ __forceinline__ void load_frags(bf16x8 (&f)[D / 16], rsrc_t head, int row, int g) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    f[s] = __builtin_bit_cast(bf16x8, buf_load16(head, (row * D + 16 * s + 8 * g) * 2));
}

// Store a transposed 32-wide output block: lane owns row `row`; register r of block db holds
// column 32db + 8(r/4) + 4g + r%4.
template <int D>
__device__ __forceinline__ void store_rows_from_acc(bf16* out_row,
                                                    const f32x16 (&acc)[(D + 31) / 32],
                                                    float mul, int g) {
#pragma unroll
  for (int db = 0; db < (D + 31) / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * g;
      if (d0 < D) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[db][4 * j + i] * mul);
        *reinterpret_cast<bf16x4*>(out_row + d0) = v;
      }
    }
}

// Online-softmax update of one 32-query x 64-key score tile held as in fwd_kernel: lane =
// query, register r of block kb = key offset 32kb + 8(r/4) + 4g + r%4 from the tile start;
// masked scores are -inf. Leaves p in sacc (the row sum is taken by p_operands). Rows rescale
// only when their max grows by more than 2^8 (in exp2 units): until then the stale max keeps
// every p <= 2^8, and O = acc / l does not depend on which max was used.
template <int DB>
__device__ __forceinline__ void softmax_tile(f32x16 (&sacc)[2], float& m, float& l,
                                             f32x16 (&o)[DB], float c, bool first) {
  constexpr float kLazy = 8.f;
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
  mx = halves_max(mx);
  if (first) {
    m = mx;  // every row sees key 0 in the first tile, so this is finite
  } else {
    const bool grow = (mx - m) * c > kLazy;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2((m - mx) * c) : 1.f;
      m = grow ? mx : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
  }
  const float nb = -m * c;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = fast_exp2(fmaf(sacc[kb][r], c, nb));
}

// P as the four bf16 operands of the P V product, and its fp32 row sum (L = m + log l must
// not pass through bf16).
__device__ __forceinline__ void p_operands(const f32x16 (&sacc)[2], bf16x8 (&pf)[4], float& l) {
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) rs += sacc[kb][r];
#pragma unroll
  for (int u = 0; u < 4; ++u) pf[u] = to_bf16x8(sacc[u >> 1], 8 * (u & 1));
  l += rs;
}

// ------------------------------------------------------------------------------ forward

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel(const bf16* __restrict__ Q,
                                                  const bf16* __restrict__ K,
                                                  const bf16* __restrict__ V,
                                                  bf16* __restrict__ O, float* __restrict__ Lout,
                                                  int Nq, int Nk, float scale, int neg) {
  constexpr int BQ = 128, BK = 64;
  constexpr int DS = D / 16, DB = (D + 31) / 32;
  using KTile = Tile<BK, D>;
  constexpr int BUF = 2 * KTile::ELEMS;  // K then V, both row-major
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * BUF];

  const int nqt = (Nq + BQ - 1) / BQ;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nqt;
  const int qt = CAUSAL ? nqt - 1 - lid % nqt : lid % nqt;  // longest rows first
  const int q0 = qt * BQ;
  const rsrc_t Qr = make_rsrc(Q + (size_t)bh * Nq * D, (uint32_t)Nq * D * 2);
  const rsrc_t Kr = make_rsrc(K + (size_t)bh * Nk * D, (uint32_t)Nk * D * 2);
  const rsrc_t Vr = make_rsrc(V + (size_t)bh * Nk * D, (uint32_t)Nk * D * 2);

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + l32;
  const float cs = fabsf(scale);
  const float c = exp2_coef(scale);

  int nkt = (Nk + BK - 1) / BK;
  if (CAUSAL) nkt = min(nkt, (min(q0 + BQ, Nq) - 1) / BK + 1);

  bf16x8 qf[DS];
  load_frags<D>(qf, Qr, qrow, g);
  if (neg)
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = negate(qf[s]);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  float m = 0.f, l = 0.f;

  KTile::template load<4>(Kr, 0, smem, w, lane);
  KTile::template load<4>(Vr, 0, smem + KTile::ELEMS, w, lane);
  wait_vmem();
  __syncthreads();

  // Each iteration issues its transposed V reads before the next tile's direct loads: the
  // compiler cannot tell that they do not alias and would otherwise wait for those loads (the
  // full memory latency) before the reads. Plain LDS reads do not have this problem.
  // One key tile; buf (0 or 1) holds it. Unrolled by two below so that buf is a constant in
  // each copy and every LDS address is a fixed register plus an immediate offset.
  auto step = [&](int kt, int buf) {
    const int k0 = kt * BK;
    const bool active = qw0 < Nq && (!CAUSAL || k0 <= qw0 + 31);
    const bf16* sK = smem + buf * BUF;
    const bf16* sV = sK + KTile::ELEMS;
    bf16x8 vfr[4][DB];
    if (active)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) vfr[u][db] = KTile::tfrag(sV, 32 * db, 16 * u, lane);
    if (kt + 1 < nkt) {
      bf16* nb = smem + (buf ^ 1) * BUF;
      KTile::template load<4>(Kr, (kt + 1) * BK, nb, w, lane);
      KTile::template load<4>(Vr, (kt + 1) * BK, nb + KTile::ELEMS, w, lane);
    }
    if (active) {
      // K fragments are read where they are used: requesting them up front with V's would
      // cost registers, and this kernel relies on two or three waves per SIMD.
      bf16x8 kfr[2][DS];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < DS; ++s) kfr[kb][s] = KTile::frag(sK, 32 * kb + l32, 2 * s + g);
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int s = 0; s < DS; ++s) sacc[kb] = mfma32(kfr[kb][s], qf[s], sacc[kb]);
      }
      // Score registers: key k0 + 32kb + 8(r/4) + 4g + r%4 against this lane's query. Only
      // tiles that straddle the diagonal or the ragged end of K compare indices.
      if ((CAUSAL && k0 + BK - 1 > qw0) || k0 + BK > Nk)
        mask_scores<2>(sacc, 0, min(CAUSAL ? qrow - k0 - 4 * g : 1 << 30, Nk - 1 - k0 - 4 * g));
      softmax_tile(sacc, m, l, o, c, kt == 0);
      bf16x8 pf[4];
      p_operands(sacc, pf, l);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma32(vfr[u][db], pf[u], o[db]);
    }
    wait_vmem();
    __syncthreads();
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    step(kt, 0);
    if (kt + 1 < nkt) step(kt + 1, 1);
  }

  const float lt = halves_sum(l);
  if (qrow < Nq) {
    store_rows_from_acc<D>(O + ((size_t)bh * Nq + qrow) * D, o, 1.f / lt, g);
    if (g == 0) Lout[(size_t)bh * Nq + qrow] = m * cs + logf(lt);
  }
}

// Causal forward with complementary tile pairing, for Nq = Nk = N, N % 128 == 0.
//
// With 64-row query tiles and 64-key tiles, query tile t sees key tiles 0..t, so tile t
// costs t + 1 steps and a plain one-tile-per-workgroup grid finishes when its last tile,
// N/64 steps long, does. Here each workgroup takes tiles A = T-1-i and B = i (T = N/64):
// T + 1 steps together, split evenly between its two wave pairs. Pair 0 runs A over key
// tiles [0, s); pair 1 runs B over [0, i+1) and then A over [s, T-i), with s = T/2 + 1.
// Both pairs step in lockstep (one barrier per step, each with its own K/V stream), and at
// the end pair 1 hands its partial (m, l, O) for A to pair 0 through LDS, which merges the
// two with the same rescale the online softmax uses between key tiles.
template <int D>
__global__ __launch_bounds__(256) void fwd_causal_paired_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ Lout, int N, float scale, int neg, int ns,
    float* __restrict__ part) {
  constexpr int BK = 64;
  constexpr int DS = D / 16, DB = (D + 31) / 32;
  using KTile = Tile<BK, D>;
  constexpr int KT = KTile::ELEMS;
  // Two statically distinct double buffers, so a step's direct loads into one provably do
  // not alias its LDS reads from the other. Index: [pair][K or V].
  __shared__ __attribute__((aligned(1024))) bf16 sb0[2][2][KT];
  __shared__ __attribute__((aligned(1024))) bf16 sb1[2][2][KT];

  const int T = N / 64;
  const int half = T / 2;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int sw = lid % ns, pid = lid / ns;  // this workgroup's share of tile pair pid
  const int bh = pid / half, i = pid % half;
  const int tA = T - 1 - i, tB = i, s = half + 1;
  const rsrc_t Qr = make_rsrc(Q + (size_t)bh * N * D, (uint32_t)N * D * 2);
  const rsrc_t Kr = make_rsrc(K + (size_t)bh * N * D, (uint32_t)N * D * 2);
  const rsrc_t Vr = make_rsrc(V + (size_t)bh * N * D, (uint32_t)N * D * 2);

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int pr = w >> 1, wp = w & 1;  // pair, wave within pair
  const float cs = fabsf(scale);
  const float c = exp2_coef(scale);

  // Steps of this pair: step n works on query tile qt(n) and key tile kt(n).
  //   pair 0: n in [0, s):           A, key tile n
  //   pair 1: n in [0, i+1):         B, key tile n;  n in [i+1, T-s+1): A, key tile n - (i+1) + s
  const int nsteps = pr == 0 ? s : T + 1 - s;
  // With ns > 1 each pair runs only steps [n_lo, n_hi) of its sequence, and the workgroup
  // writes partial (m, l, unnormalised O) records of A and B to `part` for
  // fwd_split_combine_kernel (the layout of fwd_causal_split_kernel's records).
  const int n_lo = sw * nsteps / ns, n_hi = (sw + 1) * nsteps / ns;
  constexpr int XS = 16 * DB + 2;  // per lane: O block(s), m, l

  auto qt_of = [&](int n) { return (pr == 0 || n > tB) ? tA : tB; };
  auto kt_of = [&](int n) { return (pr == 0 || n <= tB) ? n : n - (tB + 1) + s; };

  // Query fragments for both tiles this wave may own (rows 64 qt + 32 wp + lane % 32).
  bf16x8 qfA[DS], qfB[DS];
  load_frags<D>(qfA, Qr, 64 * tA + 32 * wp + l32, g);
  load_frags<D>(qfB, Qr, 64 * tB + 32 * wp + l32, g);
  if (neg)
#pragma unroll
    for (int q = 0; q < DS; ++q) {
      qfA[q] = negate(qfA[q]);
      qfB[q] = negate(qfB[q]);
    }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  float m = 0.f, l = 0.f;
  auto put_state = [&](bool tileA) {  // this wave's (m, l, O) as the share's record
    float* x = part + ((size_t)pid * ns + sw) * 2 * (XS * 128) + (tileA ? 0 : XS * 128) +
               wp * 64 + lane;
    // Opaque here, so the store addresses are formed at the store (this runs once) rather
    // than hoisted out of the step loop, where they would hold registers throughout.
    asm volatile("" : "+v"(x));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[(16 * db + r) * 128] = o[db][r];
    x[16 * DB * 128] = m;
    x[(16 * DB + 1) * 128] = l;
  };
  auto put_empty_B = [&]() {  // B's record from a share with no B step: m = -inf, l = O = 0
    float* x = part + ((size_t)pid * ns + sw) * 2 * (XS * 128) + XS * 128 + wp * 64 + lane;
    asm volatile("" : "+v"(x));
#pragma unroll
    for (int r = 0; r < 16 * DB; ++r) x[r * 128] = 0.f;
    x[16 * DB * 128] = -INFINITY;
    x[(16 * DB + 1) * 128] = 0.f;
  };

  auto fetch = [&](int n, bf16 (*dst)[KT]) {
    const int k0 = kt_of(n) * BK;
    KTile::template load_in_range<2>(Kr, k0, dst[0], wp, lane);
    KTile::template load_in_range<2>(Vr, k0, dst[1], wp, lane);
  };
  auto finish_B = [&]() {  // pair 1, after B's last key tile: B is complete
    if (ns > 1) {
      put_state(false);
    } else {
      const float lt = halves_sum(l);
      const int row = 64 * tB + 32 * wp + l32;
      store_rows_from_acc<D>(O + ((size_t)bh * N + row) * D, o, 1.f / lt, g);
      if (g == 0) Lout[(size_t)bh * N + row] = m * cs + logf(lt);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16();
    m = 0.f;
    l = 0.f;
  };
  auto step = [&](int n, const bf16 (*cur)[KT], bf16 (*nxt)[KT]) {
    // The transposed V reads come before the next tile's direct loads: the compiler cannot
    // tell that they do not alias and would otherwise wait for those loads to land first.
    // All of this step's LDS operands are requested up front, so the score MFMAs wait for the
    // first K fragment only (this kernel runs one wave per SIMD, so registers are plentiful).
    bf16x8 vfr[4][DB], kfr[2][DS];
    if (n < n_hi) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) vfr[u][db] = KTile::tfrag(cur[1], 32 * db, 16 * u, lane);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < DS; ++q) kfr[kb][q] = KTile::frag(cur[0], 32 * kb + l32, 2 * q + g);
    }
    if (n + 1 < n_hi) fetch(n + 1, nxt);
    __builtin_amdgcn_sched_barrier(0);
    if (n < n_hi) {
      const int qt = qt_of(n), kt = kt_of(n);
      const bool first = n == n_lo || (pr == 1 && n == tB + 1);
      const int qrow = 64 * qt + 32 * wp + l32;
      const int k0 = kt * BK;
      const bf16x8(&qf)[DS] = qt == tA ? qfA : qfB;
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int q = 0; q < DS; ++q) sacc[kb] = mfma32(kfr[kb][q], qf[q], sacc[kb]);
      }
      if (kt == qt) mask_scores<2>(sacc, 0, qrow - k0 - 4 * g);  // the diagonal tile
      softmax_tile(sacc, m, l, o, c, first);
      bf16x8 pf[4];
      p_operands(sacc, pf, l);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma32(vfr[u][db], pf[u], o[db]);
      if (pr == 1 && n == tB) finish_B();
    }
    wait_vmem();
    __syncthreads();
  };

  // Both pairs step in lockstep over the longer of their two shares; a pair past the end of
  // its share idles at the barriers.
  const int len0 = (sw + 1) * s / ns - sw * s / ns;
  const int len1 = (sw + 1) * (T + 1 - s) / ns - sw * (T + 1 - s) / ns;
  const int len = len0 > len1 ? len0 : len1;
  if (n_lo < n_hi) fetch(n_lo, sb0[pr]);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < len; j += 2) {
    step(n_lo + j, sb0[pr], sb1[pr]);
    if (j + 1 < len) step(n_lo + j + 1, sb1[pr], sb0[pr]);
  }

  // B's record when the share ends before B completes (pair 1's state is B's), or an empty
  // one when the share has no B step (pair 1's state, if any, is then A's, kept for the merge).
  if (ns > 1 && pr == 1) {
    if (n_lo > tB || n_lo >= n_hi) {
      put_empty_B();
    } else if (n_hi <= tB) {
      put_state(false);
    }
  }

  // Merge A: pair 1 holds A over key tiles [s, T - i) unless its share has no A step. Both
  // pairs decide this from pair 1's step range (n_lo and n_hi are each pair's own).
  const int lo1 = sw * (T + 1 - s) / ns, hi1 = (sw + 1) * (T + 1 - s) / ns;
  const bool p1_has_A = hi1 > (lo1 > tB + 1 ? lo1 : tB + 1);
  static_assert(2 * 64 * XS * sizeof(float) <= sizeof(sb0), "merge area must fit in sb0");
  // Component-major merge record (component k of wave wp's lane at k * 128 + wp * 64 + lane):
  // consecutive lanes write consecutive words, so the exchange is free of bank conflicts.
  float* xf = reinterpret_cast<float*>(&sb0[0][0][0]);
  if (pr == 1 && p1_has_A) {
    float* x = xf + wp * 64 + lane;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[(16 * db + r) * 128] = o[db][r];
    x[16 * DB * 128] = m;
    x[(16 * DB + 1) * 128] = l;
  }
  __syncthreads();
  if (pr == 0) {
    if (p1_has_A) {
      const float* x = xf + wp * 64 + lane;
      const float m1 = x[16 * DB * 128], l1 = x[(16 * DB + 1) * 128];
      const float mm = fmaxf(m, m1);
      const float a0 = fast_exp2((m - mm) * c), a1 = fast_exp2((m1 - mm) * c);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + x[(16 * db + r) * 128] * a1;
      l = l * a0 + l1 * a1;
      m = mm;
    }
    if (ns > 1) {
      put_state(true);
      return;
    }
    const float lt = halves_sum(l);
    const int row = 64 * tA + 32 * wp + l32;
    store_rows_from_acc<D>(O + ((size_t)bh * N + row) * D, o, 1.f / lt, g);
    if (g == 0) Lout[(size_t)bh * N + row] = m * cs + logf(lt);
  }
}

// Causal forward for Nq = Nk = N, N % 128 == 0, d = 16 or 32 (d = 64 takes
// fwd_causal_wide_kernel below), on eight waves (two per SIMD).
//
// As in fwd_causal_paired_kernel, workgroup i takes the 64-row query tiles A = T-1-i and
// B = i (T = N/64), which need T + 1 key steps together: A over key tiles 0 .. T-i-1, then
// B over key tiles 0 .. i. Here that sequence is cut into NP = 4 contiguous runs of equal
// length (within one), one per wave pair, and the pairs step in lockstep with their own K/V
// streams. A run that crosses from A into B parks its partial (m, l, O) for A in LDS and
// starts B afresh. At the end every pair parks its last partial; pair 0 merges those of A
// and pair NP-1 those of B, with the rescale the online softmax uses between key tiles, and
// stores O and L.
template <int D>
__global__ __launch_bounds__(512) void fwd_causal_split_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ Lout, int N, float scale, int neg, int ns,
    float* __restrict__ part) {
  constexpr int NP = 4, BK = 64;
  constexpr int DS = D / 16, DB = (D + 31) / 32;
  using KTile = Tile<BK, D>;
  constexpr int KT = KTile::ELEMS;
  constexpr int XS = 16 * DB + 2;  // parked partial: O registers, m, l (component-major)
  // K/V slots, padded where the parked partials need more room than the tiles (d = 16; the
  // pad keeps every slot at a multiple of 256 bytes, so the bank mapping is unchanged).
  constexpr int KTS = KT > 64 * XS ? KT : 64 * XS;
  static_assert(KTS * 2 % 256 == 0, "K/V slots must keep the bank mapping");
  __shared__ __attribute__((aligned(1024))) bf16 kv[NP][2][2][KTS];  // [pair][buffer][K | V]
  __shared__ __attribute__((aligned(16))) float park_cross[XS * 128];
  static_assert(NP * XS * 128 * sizeof(float) <= sizeof(kv), "parked partials must fit in kv");

  const int T = N / 64, half = T / 2;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int sw = lid % ns, pid = lid / ns;  // this workgroup's share of tile pair pid
  const int bh = pid / half, i = pid % half;
  const int tA = T - 1 - i, tB = i, nA = T - i, S = T + 1;
  const rsrc_t Qr = make_rsrc(Q + (size_t)bh * N * D, (uint32_t)N * D * 2);
  const rsrc_t Kr = make_rsrc(K + (size_t)bh * N * D, (uint32_t)N * D * 2);
  const rsrc_t Vr = make_rsrc(V + (size_t)bh * N * D, (uint32_t)N * D * 2);

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int pr = w >> 1, wp = w & 1;
  const int NR = NP * ns;  // runs per tile pair, over all ns workgroups
  const int st = (sw * NP + pr) * S / NR, en = (sw * NP + pr + 1) * S / NR;  // this pair's run
  const float cs = fabsf(scale);
  const float c = exp2_coef(scale);

  // qf holds the query tile of the current step: the run's first tile, then B's rows, copied
  // in once where the run crosses from A into B (a per-step select would cost DS * 4 VALU
  // instructions every step).
  bf16x8 qf[DS], qfB[DS];
  load_frags<D>(qf, Qr, 64 * (st < nA ? tA : tB) + 32 * wp + l32, g);
  load_frags<D>(qfB, Qr, 64 * tB + 32 * wp + l32, g);
  if (neg)
#pragma unroll
    for (int q = 0; q < DS; ++q) {
      qf[q] = negate(qf[q]);
      qfB[q] = negate(qfB[q]);
    }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  float m = 0.f, l = 0.f;

  // Park this wave's partial in a component-major record (consecutive lanes, consecutive
  // words) and start a fresh one.
  auto park = [&](float* rec) {
    float* x = rec + wp * 64 + lane;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[(16 * db + r) * 128] = o[db][r];
    x[16 * DB * 128] = m;
    x[(16 * DB + 1) * 128] = l;
  };
  auto fetch = [&](int n, int b) {
    const int k0 = (n < nA ? n : n - nA) * BK;
    KTile::template load_in_range<2>(Kr, k0, kv[pr][b][0], wp, lane);
    KTile::template load_in_range<2>(Vr, k0, kv[pr][b][1], wp, lane);
  };

  if (st < en) fetch(st, 0);
  wait_vmem();
  __syncthreads();
  const int jmax = (S + NP - 1) / NP;
  // One step of the run; b (0 or 1) is the buffer holding its K/V tile. The loop below is
  // unrolled by two so that b is a constant in each copy: every LDS address is then a fixed
  // register plus an immediate offset instead of being formed again on every step.
  auto step = [&](int j, int b) {
    const int n = st + j;
    const bool act = n < en;
    const bf16* sK = kv[pr][b][0];
    const bf16* sV = kv[pr][b][1];
    // All of this step's LDS operands are requested before the next tile's direct loads
    // (the compiler would otherwise wait for those loads ahead of the transposed reads).
    bf16x8 vfr[4][DB], kfr[2][DS];
    if (act) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) vfr[u][db] = KTile::tfrag(sV, 32 * db, 16 * u, lane);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < DS; ++q) kfr[kb][q] = KTile::frag(sK, 32 * kb + l32, 2 * q + g);
    }
    if (n + 1 < en) fetch(n + 1, b ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    if (act) {
      const bool isA = n < nA;
      const int qt = isA ? tA : tB, kt = isA ? n : n - nA;
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int q = 0; q < DS; ++q) sacc[kb] = mfma32(kfr[kb][q], qf[q], sacc[kb]);
      }
      if (kt == qt) mask_scores<2>(sacc, 0, 32 * wp + l32 - 4 * g);  // the diagonal tile
      softmax_tile(sacc, m, l, o, c, n == st || n == nA);
      bf16x8 pf[4];
      p_operands(sacc, pf, l);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma32(vfr[u][db], pf[u], o[db]);
      if (n + 1 == nA && n + 1 < en) {  // the run continues into B: park A's partial
        park(park_cross);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = zero16();
        m = 0.f;
        l = 0.f;
#pragma unroll
        for (int q = 0; q < DS; ++q) qf[q] = qfB[q];
      }
    }
    wait_vmem();
    __syncthreads();
  };
  for (int j = 0; j < jmax; j += 2) {
    step(j, 0);
    if (j + 1 < jmax) step(j + 1, 1);
  }

  // Every pair parks its last partial (of A if its run ends within A, else of B) in slot pr.
  float* slots = reinterpret_cast<float*>(&kv[0][0][0][0]);
  if (st < en) park(slots + pr * XS * 128);
  __syncthreads();
  if (pr != 0 && pr != NP - 1) return;
  const bool mergeA = pr == 0;
  // Partials of the tile being merged: slot p holds tile A iff p's run ends within A; the
  // crossing record holds A's part from the run that crosses into B, if one does.
  auto included = [&](int p) {
    const int sp = (sw * NP + p) * S / NR, ep = (sw * NP + p + 1) * S / NR;
    return sp < ep && (ep <= nA) == mergeA;
  };
  bool cross = false;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sp = (sw * NP + p) * S / NR, ep = (sw * NP + p + 1) * S / NR;
    cross |= sp < nA && nA < ep;
  }
  cross = cross && mergeA;
  float mm = -INFINITY;
#pragma unroll
  for (int p = 0; p < NP; ++p)
    if (included(p)) mm = fmaxf(mm, slots[p * XS * 128 + 16 * DB * 128 + wp * 64 + lane]);
  if (cross) mm = fmaxf(mm, park_cross[16 * DB * 128 + wp * 64 + lane]);
  float lsum = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  auto add = [&](const float* rec) {
    const float* x = rec + wp * 64 + lane;
    const float f = fast_exp2((x[16 * DB * 128] - mm) * c);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] += f * x[(16 * db + r) * 128];
    lsum += f * x[(16 * DB + 1) * 128];
  };
#pragma unroll
  for (int p = 0; p < NP; ++p)
    if (included(p)) add(slots + p * XS * 128);
  if (cross) add(park_cross);
  if (ns > 1) {
    // This workgroup's partial (m, l, unnormalised O) for the tile, in the component-major
    // record layout; fwd_split_combine_kernel merges the ns records. A workgroup with no
    // part of the tile writes m = -inf, l = 0.
    float* x = part + ((size_t)pid * ns + sw) * 2 * (XS * 128) + (mergeA ? 0 : XS * 128) +
               wp * 64 + lane;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[(16 * db + r) * 128] = o[db][r];
    x[16 * DB * 128] = mm;
    x[(16 * DB + 1) * 128] = lsum;
    return;
  }
  const float lt = halves_sum(lsum);
  const int row = 64 * (mergeA ? tA : tB) + 32 * wp + l32;
  store_rows_from_acc<D>(O + ((size_t)bh * N + row) * D, o, 1.f / lt, g);
  if (g == 0) Lout[(size_t)bh * N + row] = mm * cs + logf(lt);
}


// fwd_causal_split_kernel with one wave per run instead of a wave pair: eight waves, two per
// SIMD, each holding the query tile's 64 rows as two 32-row blocks, so the tile pair's T + 1
// key steps are cut into 8 ns runs. A wave reads each K/V fragment once for both blocks (half
// the LDS reads of a pair, which reads every fragment in both of its waves) and streams its
// own tiles through one LDS slot: it copies the tile's fragments into registers, then loads
// the next tile into the same slot while its second row block is computed. No other wave
// touches the slot, so the waves need no barrier between steps. At the end every wave parks
// its last partial (an empty run parks m = -inf, l = O = 0) and all eight merge, each one
// 32-column half of one 32-row block: waves 0-3 tile A, waves 4-7 tile B. Used for d = 64,
// where it is faster than the wave-pair kernel; the results differ from that kernel's only in
// the order of the merge's additions.
template <int D>
__global__ __launch_bounds__(512) void fwd_causal_wide_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ Lout, int N, float scale, int neg, int ns,
    float* __restrict__ part) {
  constexpr int NW = 8, BK = 64;
  constexpr int DS = D / 16, DB = (D + 31) / 32;
  using KTile = Tile<BK, D>;
  constexpr int KT = KTile::ELEMS;
  constexpr int XS = 16 * DB + 2;  // parked partial: O registers, m, l (component-major)
  // K/V slots, padded so that the eight parked partials fit in them.
  constexpr int KTS = KT > 128 * XS ? KT : 128 * XS;
  static_assert(KTS * 2 % 256 == 0, "K/V slots must keep the bank mapping");
  __shared__ __attribute__((aligned(1024))) bf16 kv[NW][2][KTS];  // [wave][K | V]
  __shared__ __attribute__((aligned(16))) float park_cross[XS * 128];
  static_assert(NW * XS * 128 * sizeof(float) <= sizeof(kv), "parked partials must fit in kv");

  const int T = N / 64, half = T / 2;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int sw = lid % ns, pid = lid / ns;  // this workgroup's share of tile pair pid
  const int bh = pid / half, i = pid % half;
  const int tA = T - 1 - i, tB = i, nA = T - i, S = T + 1;
  const rsrc_t Qr = make_rsrc(Q + (size_t)bh * N * D, (uint32_t)N * D * 2);
  const rsrc_t Kr = make_rsrc(K + (size_t)bh * N * D, (uint32_t)N * D * 2);
  const rsrc_t Vr = make_rsrc(V + (size_t)bh * N * D, (uint32_t)N * D * 2);

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int NR = NW * ns;  // runs per tile pair, over all ns workgroups
  // Run boundaries rounded up, so that the runs with an extra step come first. Run 0 starts
  // at A's first key step and reaches B only when A is shorter than it, so the run that
  // crosses into B (and waits there for B's query rows) is, on longer heads, a shorter run.
  auto run_start = [&](int r) { return ((sw * NW + r) * S + NR - 1) / NR; };
  const int st = run_start(w), en = run_start(w + 1);  // this wave's run
  const float cs = fabsf(scale);
  const float c = exp2_coef(scale);

  bf16x8 qf[2][DS];  // the current query tile's two row blocks
  auto load_q = [&](int qt) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      load_frags<D>(qf[rb], Qr, 64 * qt + 32 * rb + l32, g);
      if (neg)
#pragma unroll
        for (int q = 0; q < DS; ++q) qf[rb][q] = negate(qf[rb][q]);
    }
  };
  load_q(st < nA ? tA : tB);

  f32x16 o[2][DB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = zero16();
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  // A parked record in LDS: O in 16-byte chunks (four consecutive accumulator registers of
  // one lane; chunk j of row block rb at float ((rb * 4 DB + j) * 64 + lane) * 4, so a wave
  // writes or reads one chunk index with 128-bit accesses over consecutive addresses), then m
  // and l per (row block, lane). The partials written to global memory for ns > 1 keep
  // fwd_causal_split_kernel's component-major layout, which the combine kernel reads.
  constexpr int MOFF = 2 * 16 * DB * 64;
  auto park = [&](float* rec) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v = {o[rb][db][4 * j], o[rb][db][4 * j + 1], o[rb][db][4 * j + 2],
                     o[rb][db][4 * j + 3]};
          *reinterpret_cast<f32x4*>(rec + ((rb * 4 * DB + 4 * db + j) * 64 + lane) * 4) = v;
        }
      rec[MOFF + rb * 64 + lane] = m[rb];
      rec[MOFF + 128 + rb * 64 + lane] = l[rb];
    }
  };
  const bf16* sK = kv[w][0];
  const bf16* sV = kv[w][1];
  auto fetch = [&](int n) {
    const int k0 = (n < nA ? n : n - nA) * BK;
    KTile::template load_in_range<1>(Kr, k0, kv[w][0], 0, lane);
    KTile::template load_in_range<1>(Vr, k0, kv[w][1], 0, lane);
  };

  if (st < en) fetch(st);
  wait_vmem();
  for (int n = st; n < en; ++n) {
    bf16x8 vfr[4][DB], kfr[2][DS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < DS; ++q) kfr[kb][q] = KTile::frag(sK, 32 * kb + l32, 2 * q + g);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) vfr[u][db] = KTile::tfrag(sV, 32 * db, 16 * u, lane);
    const bool isA = n < nA;
    const int qt = isA ? tA : tB, kt = isA ? n : n - nA;
    const bool first = n == st || n == nA;
    f32x16 sacc[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[rb][kb] = zero16();
#pragma unroll
        for (int q = 0; q < DS; ++q) sacc[rb][kb] = mfma32(kfr[kb][q], qf[rb][q], sacc[rb][kb]);
      }
    // Every fragment of the tile is in registers once the LDS reads have returned. The next
    // tile goes into the same slot after row block 0's products are issued, while row block
    // 1's softmax and products run (this placement measured faster than right after the
    // score products, or later; so did waiting for the reads here rather than there).
    __builtin_amdgcn_sched_barrier(0);
    if (n + 1 < en) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if (kt == qt) mask_scores<2>(sacc[rb], 0, 32 * rb + l32 - 4 * g);  // the diagonal tile
      softmax_tile(sacc[rb], m[rb], l[rb], o[rb], c, first);
      bf16x8 pf[4];
      p_operands(sacc[rb], pf, l[rb]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] = mfma32(vfr[u][db], pf[u], o[rb][db]);
      if (rb == 0) {
        __builtin_amdgcn_sched_barrier(0);
        if (n + 1 < en) fetch(n + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (n + 1 == nA && n + 1 < en) {  // the run continues into B: park A's partial
      park(park_cross);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] = zero16();
        m[rb] = -INFINITY;
        l[rb] = 0.f;
      }
      load_q(tB);
    }
    wait_vmem();
  }

  // Every wave parks its last partial (of A if its run ends within A, else of B; empty if
  // its run is) in slot w, which is its own K/V slot: its reads of that slot have returned
  // and no other wave touches it, so it parks as soon as its run ends. Then each wave merges
  // one 32-column half (db) of one 32-row block (rb) of tile A (waves 0-3) or B (4-7).
  static_assert(XS * 128 * sizeof(float) == sizeof(kv[0]), "slot w is wave w's K/V slot");
  float* slots = reinterpret_cast<float*>(&kv[0][0][0]);
  park(slots + w * XS * 128);
  __syncthreads();
  static_assert(DB == 2, "the merge gives each wave one of the two 32-column halves");
  const bool mergeA = w < 4;
  const int rb = (w >> 1) & 1, db = w & 1;
  // Partials of the tile being merged: slot p holds tile A iff p's run ends within A; the
  // crossing record holds A's part from the run that crosses into B, if one does. A wave
  // loads only its tile's slots (the test is uniform over the wave), all of them into
  // registers before it adds any, so the loads need not wait for each other; reading every
  // slot with weight 0 for the others took twice the LDS reads and measured slower.
  bool inc[NW], cross = false;
#pragma unroll
  for (int p = 0; p < NW; ++p) {
    const int sp = run_start(p), ep = run_start(p + 1);
    inc[p] = sp < ep && (ep <= nA) == mergeA;
    cross |= sp < nA && nA < ep;
  }
  cross = cross && mergeA;
  const float* xc = park_cross + MOFF + rb * 64 + lane;
  auto chunk = [&](const float* rec, int j) {
    return *reinterpret_cast<const f32x4*>(rec + ((rb * 4 * DB + 4 * db + j) * 64 + lane) * 4);
  };
  float xm[NW], f[NW];
  float mm = cross ? xc[0] : -INFINITY;
#pragma unroll
  for (int p = 0; p < NW; ++p) {
    xm[p] = slots[p * XS * 128 + MOFF + rb * 64 + lane];
    if (inc[p]) mm = fmaxf(mm, xm[p]);
  }
  // An empty partial (m = -inf) weighs 0, also where every partial here is empty (ns > 1).
  auto weight = [&](bool in, float m_) {
    return in && m_ != -INFINITY ? fast_exp2((m_ - mm) * c) : 0.f;
  };
#pragma unroll
  for (int p = 0; p < NW; ++p) f[p] = weight(inc[p], xm[p]);
  float lsum = 0.f;
  f32x16 acc = zero16();
  float xv[NW][17];
#pragma unroll
  for (int p = 0; p < NW; ++p) {
    const float* x = slots + p * XS * 128;
    if (inc[p]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = chunk(x, j);
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[p][4 * j + e] = v[e];
      }
      xv[p][16] = x[MOFF + 128 + rb * 64 + lane];
    }
  }
#pragma unroll
  for (int p = 0; p < NW; ++p) {
    if (inc[p]) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += f[p] * xv[p][r];
      lsum += f[p] * xv[p][16];
    }
  }
  if (cross) {
    const float fc = weight(true, xc[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v = chunk(park_cross, j);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * j + e] += fc * v[e];
    }
    lsum += fc * xc[128];
  }
  if (ns > 1) {
    // This workgroup's partial for the tile, as fwd_causal_split_kernel writes it.
    float* x = part + ((size_t)pid * ns + sw) * 2 * (XS * 128) + (mergeA ? 0 : XS * 128) +
               rb * 64 + lane;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[(16 * db + r) * 128] = acc[r];
    if (db == 0) {
      x[16 * DB * 128] = mm;
      x[(16 * DB + 1) * 128] = lsum;
    }
    return;
  }
  const float lt = halves_sum(lsum);
  const int row = 64 * (mergeA ? tA : tB) + 32 * rb + l32;
  bf16* out = O + ((size_t)bh * N + row) * D + 32 * db;
  const float inv = 1.f / lt;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = (bf16)(acc[4 * j + k] * inv);
    *reinterpret_cast<bf16x4*>(out + 8 * j + 4 * g) = v;
  }
  if (db == 0 && g == 0) Lout[(size_t)bh * N + row] = mm * cs + logf(lt);
}

// Merges the ns partial records fwd_causal_split_kernel or fwd_causal_wide_kernel wrote for
// each 64-row tile (when it spreads a tile pair over ns <= kMaxWays workgroups) with the
// online-softmax rescale, and stores O and L. One workgroup per tile with 128 threads per 32-column block: thread t takes
// record lane t % 128 (lane = row, as in the split kernel) and column block t / 128, so every
// load is coalesced and all of a thread's loads are independent. A record from a workgroup
// with no part of the tile has m = -inf and l = O = 0, and so gets weight exp2(-inf) = 0.
template <int D>
__global__ __launch_bounds__(128 * ((D + 31) / 32)) void fwd_split_combine_kernel(
    const float* __restrict__ part, bf16* __restrict__ O, float* __restrict__ Lout, int N,
    float scale, int ns) {
  constexpr int DB = (D + 31) / 32, XS = 16 * DB + 2, MAXW = 8;
  const int T = N / 64, half = T / 2;
  const int tile = blockIdx.x % T, bh = blockIdx.x / T;
  const bool isA = tile >= half;  // tile pair i holds A = T-1-i and B = i
  const int i = isA ? T - 1 - tile : tile;
  const int slot = threadIdx.x & 127, db = threadIdx.x >> 7;
  const int lane = slot & 63, wp = slot >> 6, g = lane >> 5, l32 = lane & 31;
  const float c = exp2_coef(scale), cs = fabsf(scale);
  const float* x0 = part + (size_t)(bh * half + i) * ns * 2 * (XS * 128) +
                    (isA ? 0 : XS * 128) + slot;
  const size_t stride = 2 * (XS * 128);
  float mw[MAXW], lw[MAXW];
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
    mw[w] = w < ns ? x0[w * stride + 16 * DB * 128] : -INFINITY;
    lw[w] = w < ns ? x0[w * stride + (16 * DB + 1) * 128] : 0.f;
  }
  float mm = mw[0];
#pragma unroll
  for (int w = 1; w < MAXW; ++w) mm = fmaxf(mm, mw[w]);
  f32x16 o = zero16();
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
    if (w < ns) {
      const float f = fast_exp2((mw[w] - mm) * c);
      const float* x = x0 + w * stride + 16 * db * 128;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] += f * x[r * 128];
      lsum += f * lw[w];
    }
  }
  const float lt = halves_sum(lsum);
  const float inv = 1.f / lt;
  const int row = 64 * tile + 32 * wp + l32;
  bf16* orow = O + ((size_t)bh * N + row) * D;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d0 = 32 * db + 8 * j + 4 * g;
    if (d0 >= D) continue;  // d = 16: half of the block is padding
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[4 * j + e] * inv);
    *reinterpret_cast<bf16x4*>(orow + d0) = v;
  }
  if (db == 0 && g == 0) Lout[(size_t)bh * N + row] = mm * cs + logf(lt);
}

// ----------------------------------------------------------------------------- backward
//
// Both passes step through 32-row moving tiles. A dK/dV step takes 32 queries against the
// wave's 32 keys (key = lane % 32); a dQ step takes 32 keys against the wave's 32 queries.

template <int D>
struct Bwd {
  static constexpr int DS = D / 16, DB = (D + 31) / 32;
  using MTile = Tile<32, D>;
  static constexpr int T = MTile::ELEMS;
  // dK/dV stream buffer: Q and dO tiles, then 32 floats L log2e and 32 floats -D (written by
  // bwd_prep_kernel).
  static constexpr int KV_BUF = 2 * T + 2 * 32 * 2;
  // dQ stream buffer: K, V tiles.
  static constexpr int Q_BUF = 2 * T;
  static constexpr int NCH = D / 8;
};

// Per-row terms of the backward, one launch ahead of bwd_kernel: L2 = L log2(e) (the
// exponent offset of P = exp2(S scale log2(e) - L2)) and ND = -D with D = rowsum(dO o O)
// (problem flash_backward's preprocessing). ND starts the dP accumulators, so dS = P (dP - D)
// is one multiply. D_CH = d/8 lanes share a row, one 16-byte chunk of dO and of O each.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const bf16* __restrict__ O,
                                                       const bf16* __restrict__ dO,
                                                       const float* __restrict__ L,
                                                       float* __restrict__ L2,
                                                       float* __restrict__ ND, long long rows) {
  constexpr int CH = D / 8;
  const long long total = rows * CH;
  // Block-uniform stride loop: the grid is capped so its work-item count fits 32 bits, and
  // lane groups of one row stay together (CH divides 256).
  for (long long base = (long long)blockIdx.x * 256; base < total;
       base += (long long)gridDim.x * 256) {
    const long long t = base + threadIdx.x;
    const long long row = t / CH;
    const int ch = (int)(t % CH);
    // Lanes past the last row re-read it instead of branching around the loads: the lane
    // reduction below then follows straight-line code with the full wave active.
    const long long r = row < rows ? row : rows - 1;
    // L is loaded with dO and O (every lane of the row reads it), so the three loads share
    // one memory round trip instead of L waiting for the reduction.
    const float lr = L[r];
    const u32x4 a = *reinterpret_cast<const u32x4*>(dO + r * D + ch * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(O + r * D + ch * 8);
    asm volatile("" ::"v"(lr));  // keeps the L load here rather than after the reduction
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = dot2_bf16(a[i], b[i], acc);
    acc = group_sum<CH>(acc);
    if (row < rows && ch == 0) {
      L2[row] = lr * kLog2e;
      ND[row] = -acc;
    }
  }
}

// Direct loads of the dK/dV stream for moving tile m0.. (Q and dO rows, L2 and ND) into
// `buf`, by NW >= 2 waves (index w). Rows past Nq read as zeros: their Q, dO and ND are 0, so
// their P = exp2(0) = 1 meets dO = 0 and dP - D = 0 and adds nothing to dV or dK. IN_RANGE
// (the tile lies inside the head) takes the tile's offset as a wave-uniform operand.
template <int D, int NW, bool IN_RANGE = false>
__device__ __forceinline__ void kv_fetch(rsrc_t Qr, rsrc_t dOr, rsrc_t L2r, rsrc_t NDr, int m0,
                                         bf16* buf, int w, int lane) {
  static_assert(NW >= 2, "L2 and ND are fetched by waves 0 and 1");
  using B = Bwd<D>;
  if constexpr (IN_RANGE) {
    B::MTile::template load_in_range<NW>(Qr, m0, buf, w, lane);
    B::MTile::template load_in_range<NW>(dOr, m0, buf + B::T, w, lane);
    if (w < 2 && lane < 32)
      dma4_at(w == 0 ? L2r : NDr, (uint32_t)lane * 4, (uint32_t)m0 * 4, buf + 2 * B::T + 64 * w);
  } else {
    B::MTile::template load<NW>(Qr, m0, buf, w, lane);
    B::MTile::template load<NW>(dOr, m0, buf + B::T, w, lane);
    if (w < 2 && lane < 32)
      dma4(w == 0 ? L2r : NDr, (uint32_t)(m0 + lane) * 4, buf + 2 * B::T + 64 * w);
  }
}

// Transposed LDS operands of one dK/dV step (dO^T and Q^T, the A operands of dV^T and dK^T).
// The paired kernel requests them at the start of the step, right behind the reads its first
// products wait for (kv_step with EARLY = true), so that they are in flight while those
// products and the exponentials run. That costs 8 * DB registers for the whole step, which
// bwd_kernel cannot afford without dropping from three waves per SIMD to two, so there
// kv_step reads them where they are used (EARLY = false) and takes the wait, which the first
// half of the step overlaps.
template <int D>
struct KvOps {
  static constexpr int DB = (D + 31) / 32;
  bf16x8 dot[2][DB], qt[2][DB];
  __device__ __forceinline__ void read(const bf16* buf, int lane) {
    using B = Bwd<D>;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dot[st][db] = B::MTile::tfrag(buf + B::T, 32 * db, 16 * st, lane);
        qt[st][db] = B::MTile::tfrag(buf, 32 * db, 16 * st, lane);
      }
  }
};

// One dK/dV step for the 32 staged queries against this wave's 32 keys (kf, vf):
// S = Q K^T and dP - D = dO V^T - D (the dP accumulator starts at -D), with lane = key and
// register r = query 8(r/4) + 4g + r%4; P = exp2(S c - L2), dS = P (dP - D); then
// dV^T += dO^T P and dK^T += Q^T dS (lane = key, register = column of d). When `masked`,
// queries with offset 8(r/4) + r%4 below `lim` (earlier than this lane's key) get P = dS = 0.
//
// With DSOUT, dS (bf16, as the dK product takes it) is also written to dsT, a 32 x 32 LDS
// tile of this wave (Tile<32, 32> layout, row = key, column = query), for a dQ product.
template <int D, bool EARLY, bool DSOUT = false>
__device__ __forceinline__ void kv_step(const bf16* buf, KvOps<D>& op,
                                        const bf16x8 (&kf)[D / 16],
                                        const bf16x8 (&vf)[D / 16],
                                        f32x16 (&dvt)[(D + 31) / 32],
                                        f32x16 (&dkt)[(D + 31) / 32], float c, bool masked,
                                        int lim, int lane, int l32, int g,
                                        bf16* dsT = nullptr) {
  using B = Bwd<D>;
  constexpr int DS = D / 16, DB = (D + 31) / 32;
  // LDS reads in the order they are needed: dP's starting value, the score products' row
  // fragments, then (EARLY) the transposed operands of the last products.
  const float* sL2 = reinterpret_cast<const float*>(buf + 2 * B::T);
  f32x16 sp = zero16(), dp;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 n4 = *reinterpret_cast<const f32x4*>(sL2 + 32 + 8 * j + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) dp[4 * j + i] = n4[i];
  }
  bf16x8 qa[DS], da[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    qa[s] = B::MTile::frag(buf, l32, 2 * s + g);
    da[s] = B::MTile::frag(buf + B::T, l32, 2 * s + g);
  }
  // With registers to spare (EARLY), all of these reads are issued before the first MFMA,
  // so the score MFMAs wait for one LDS round trip rather than one per operand pair.
  if constexpr (EARLY) {
    op.read(buf, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    sp = mfma32(qa[s], kf[s], sp);
    dp = mfma32(da[s], vf[s], dp);
  }
  if (masked) {  // queries with offset below lim are earlier than this lane's key
    f32x16 t[1] = {sp};
    mask_scores<1>(t, lim, 1 << 30);
    sp = t[0];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(sL2 + 8 * j + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * j + i;
      const float p = fast_exp2(fmaf(sp[r], c, -l4[i]));
      sp[r] = p;
      dp[r] = p * dp[r];
    }
  }
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const bf16x8 pf = to_bf16x8(sp, 8 * st);
    const bf16x8 sf = to_bf16x8(dp, 8 * st);
    if constexpr (DSOUT) {
      // sf holds queries 16 st + 4g + 0..3 (elements 0..3) and 16 st + 8 + 4g + 0..3 (4..7)
      // of key l32: two 8-byte pieces of row l32, in chunks 2 st and 2 st + 1.
      const u32x4 u = __builtin_bit_cast(u32x4, sf);
      const u32x2 lo = {u[0], u[1]}, hi = {u[2], u[3]};
      *reinterpret_cast<u32x2*>(dsT + swz<4>(l32, 2 * st) + 4 * g) = lo;
      *reinterpret_cast<u32x2*>(dsT + swz<4>(l32, 2 * st + 1) + 4 * g) = hi;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if constexpr (EARLY) {
        dvt[db] = mfma32(op.dot[st][db], pf, dvt[db]);
        dkt[db] = mfma32(op.qt[st][db], sf, dkt[db]);
      } else {
        dvt[db] = mfma32(B::MTile::tfrag(buf + B::T, 32 * db, 16 * st, lane), pf, dvt[db]);
        dkt[db] = mfma32(B::MTile::tfrag(buf, 32 * db, 16 * st, lane), sf, dkt[db]);
      }
    }
  }
}

// Transposed LDS operands of one dQ step (K^T), requested early or late as in KvOps.
template <int D>
struct QOps {
  static constexpr int DB = (D + 31) / 32;
  bf16x8 kt[2][DB];
  __device__ __forceinline__ void read(const bf16* buf, int lane) {
    using B = Bwd<D>;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db) kt[s2][db] = B::MTile::tfrag(buf, 32 * db, 16 * s2, lane);
  }
};

// dQ step: S^T = K Q^T, dP^T - D = V dO^T - D (lane = query, register r = key
// 8(r/4) + 4g + r%4), P = exp2(S c - L2), dS = P (dP - D), dQ^T += K^T dS^T. When `masked`,
// keys with offset above hi get P = dS = 0.
template <int D, bool EARLY>
__device__ __forceinline__ void q_step(const bf16* buf, QOps<D>& op,
                                       const bf16x8 (&qf)[D / 16],
                                       const bf16x8 (&dof)[D / 16],
                                       f32x16 (&dqt)[(D + 31) / 32], float c, float l2,
                                       float nd, bool masked, int hi, int lane, int l32,
                                       int g) {
  using B = Bwd<D>;
  constexpr int DS = D / 16, DB = (D + 31) / 32;
  bf16x8 k[DS], v[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    k[s] = B::MTile::frag(buf, l32, 2 * s + g);
    v[s] = B::MTile::frag(buf + B::T, l32, 2 * s + g);
  }
  if constexpr (EARLY) {  // as in kv_step: the transposed operands after the row fragments
    op.read(buf, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  f32x16 st[1] = {zero16()};
  f32x16 dpt = splat16(nd);  // dP starts at -D of this lane's query
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    st[0] = mfma32(k[s], qf[s], st[0]);
    dpt = mfma32(v[s], dof[s], dpt);
  }
  if (masked) mask_scores<1>(st, 0, hi);  // keys with offset above hi are invisible
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = fast_exp2(fmaf(st[0][r], c, -l2));
    dpt[r] = p * dpt[r];
  }
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const bf16x8 sf = to_bf16x8(dpt, 8 * s2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if constexpr (EARLY)
        dqt[db] = mfma32(op.kt[s2][db], sf, dqt[db]);
      else
        dqt[db] = mfma32(B::MTile::tfrag(buf, 32 * db, 16 * s2, lane), sf, dqt[db]);
    }
  }
}

// Stationary state of a dQ wave: Q and dO fragments of query row `qrow`, its L2 and ND
// (rows past Nq read zeros and are never stored).
template <int D>
struct QRow {
  bf16x8 qf[D / 16], dof[D / 16];
  float l2, nd;
  // Issues the loads; finish() (after they have landed) applies the sign.
  __device__ __forceinline__ void issue(rsrc_t Qr, rsrc_t dOr, rsrc_t L2r, rsrc_t NDr,
                                        int qrow, int g) {
    load_frags<D>(qf, Qr, qrow, g);
    load_frags<D>(dof, dOr, qrow, g);
    l2 = buf_load_f32(L2r, qrow * 4);
    nd = buf_load_f32(NDr, qrow * 4);
  }
  __device__ __forceinline__ void finish(int neg) {
    if (neg)
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qf[s] = negate(qf[s]);
  }
  __device__ __forceinline__ void load(rsrc_t Qr, rsrc_t dOr, rsrc_t L2r, rsrc_t NDr, int qrow,
                                       int g, int neg) {
    issue(Qr, dOr, L2r, NDr, qrow, g);
    wait_vmem();
    finish(neg);
  }
};

template <int D>
__device__ __forceinline__ void load_kv_rows(bf16x8 (&kf)[D / 16], bf16x8 (&vf)[D / 16],
                                             rsrc_t Kr, rsrc_t Vr, int krow, int g, int neg) {
  load_frags<D>(kf, Kr, krow, g);
  load_frags<D>(vf, Vr, krow, g);
  wait_vmem();
  if (neg)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf[s] = negate(kf[s]);
}

// Partial sums of the split backward: an accumulator set stored unscaled as fp32 rows, the
// layout store_rows_from_acc gives bf16 outputs (lane owns row `out_row`; register r of block
// db holds column 32db + 8(r/4) + 4g + r%4), or zeros for a share with no step of the tile.
template <int D>
__device__ __forceinline__ void put_rows_f32(float* out_row, const f32x16 (&acc)[(D + 31) / 32],
                                             int g) {
#pragma unroll
  for (int db = 0; db < (D + 31) / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (32 * db + 8 * j + 4 * g >= D) continue;  // d = 16: half of the block is padding
      f32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc[db][4 * j + i];
      *reinterpret_cast<f32x4*>(out_row + 32 * db + 8 * j + 4 * g) = v;
    }
}
template <int D>
__device__ __forceinline__ void put_zero_rows_f32(float* out_row, int g) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < (D + 31) / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (32 * db + 8 * j + 4 * g < D)
        *reinterpret_cast<f32x4*>(out_row + 32 * db + 8 * j + 4 * g) = z;
}

// dK, dV for the 128 keys starting at k0 of one head (4 waves share one query stream). With
// ns > 1 this is share sw of the query steps, and the sums go unscaled to the fp32 partial
// tiles of the head at `part` (see bwd_kernel) instead of dK and dV.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_part(bf16* smem, rsrc_t Qr, rsrc_t Kr, rsrc_t Vr,
                                          rsrc_t L2r, rsrc_t NDr, rsrc_t dOr, bf16* dKh,
                                          bf16* dVh, int k0,
                                          int Nq, int Nk, float scale, int neg, int sw, int ns,
                                          float* part) {
  using B = Bwd<D>;
  constexpr int DS = B::DS, DB = B::DB;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int kw0 = k0 + 32 * w;
  const int krow = kw0 + l32;
  const float c = exp2_coef(scale);

  bf16x8 kf[DS], vf[DS];
  load_kv_rows<D>(kf, vf, Kr, Vr, krow, g, neg);
  f32x16 dvt[DB], dkt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dvt[db] = zero16();
    dkt[db] = zero16();
  }

  const int nmt = (Nq + 31) / 32;
  const int mt0 = CAUSAL ? min(k0 / 32, nmt) : 0;
  const int lo = mt0 + sw * (nmt - mt0) / ns, hi = mt0 + (sw + 1) * (nmt - mt0) / ns;
  if (lo < hi) kv_fetch<D, 4>(Qr, dOr, L2r, NDr, lo * 32, smem, w, lane);
  wait_vmem();
  __syncthreads();
  // One query step; buffer p (0 or 1) holds it. Unrolled by two below so that p is a
  // constant in each copy and every LDS address is a fixed register plus an immediate.
  auto step = [&](int mt, int p) {
    bf16* buf = smem + p * B::KV_BUF;
    bf16* nbuf = smem + (p ^ 1) * B::KV_BUF;
    const int m0 = mt * 32;
    const bool active = kw0 < Nk && (!CAUSAL || m0 + 31 >= kw0);
    KvOps<D> op;  // unused: transposed operands are read late (see KvOps)
    if (mt + 1 < hi) kv_fetch<D, 4>(Qr, dOr, L2r, NDr, m0 + 32, nbuf, w, lane);
    if (active)
      kv_step<D, false>(buf, op, kf, vf, dvt, dkt, c, CAUSAL && m0 < kw0 + 31,
                        krow - m0 - 4 * g, lane, l32, g);
    wait_vmem();
    __syncthreads();
  };
  for (int mt = lo; mt < hi; mt += 2) {
    step(mt, 0);
    if (mt + 1 < hi) step(mt + 1, 1);
  }

  if (ns > 1) {  // Nq = Nk, a multiple of 128: every row exists
    float* x = part + (((size_t)(krow / 64) * ns + sw) * 2 * 64 + krow % 64) * D;
    asm volatile("" : "+v"(x));  // address formed here, not held through the loop
    put_rows_f32<D>(x, dkt, g);
    put_rows_f32<D>(x + 64 * D, dvt, g);
  } else if (krow < Nk) {
    store_rows_from_acc<D>(dKh + (size_t)krow * D, dkt, scale, g);
    store_rows_from_acc<D>(dVh + (size_t)krow * D, dvt, 1.f, g);
  }
}

// dQ for the 128 queries starting at q0 of one head (4 waves share one key stream). With
// ns > 1 this is share sw of the key steps, summed into the head's fp32 partial tiles at `part`.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_part(bf16* smem, rsrc_t Qr, rsrc_t Kr, rsrc_t Vr,
                                        rsrc_t L2r, rsrc_t NDr, rsrc_t dOr, bf16* dQh, int q0,
                                        int Nq, int Nk,
                                        float scale, int neg, int sw, int ns, float* part) {
  using B = Bwd<D>;
  constexpr int DB = B::DB;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + l32;
  const float c = exp2_coef(scale);

  QRow<D> row;
  row.load(Qr, dOr, L2r, NDr, qrow, g, neg);
  f32x16 dqt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqt[db] = zero16();

  int nkt = (Nk + 31) / 32;
  if (CAUSAL) nkt = min(nkt, (min(q0 + 128, Nq) - 1) / 32 + 1);
  const int lo = sw * nkt / ns, hi = (sw + 1) * nkt / ns;
  if (lo < hi) {
    B::MTile::template load<4>(Kr, lo * 32, smem, w, lane);
    B::MTile::template load<4>(Vr, lo * 32, smem + B::T, w, lane);
  }
  wait_vmem();
  __syncthreads();
  // One key step; buffer p (0 or 1) holds it, unrolled by two as in dkdv_part.
  auto step = [&](int kt, int p) {
    const bf16* buf = smem + p * B::Q_BUF;
    bf16* nbuf = smem + (p ^ 1) * B::Q_BUF;
    const int n0 = kt * 32;
    const bool active = qw0 < Nq && (!CAUSAL || n0 <= qw0 + 31);
    QOps<D> op;  // unused: transposed operands are read late (see KvOps)
    if (kt + 1 < hi) {
      B::MTile::template load<4>(Kr, n0 + 32, nbuf, w, lane);
      B::MTile::template load<4>(Vr, n0 + 32, nbuf + B::T, w, lane);
    }
    if (active)
      q_step<D, false>(buf, op, row.qf, row.dof, dqt, c, row.l2, row.nd,
                       (CAUSAL && n0 + 31 > qw0) || n0 + 32 > Nk,
                       min(CAUSAL ? qrow - n0 - 4 * g : 1 << 30, Nk - 1 - n0 - 4 * g), lane,
                       l32, g);
    wait_vmem();
    __syncthreads();
  };
  for (int kt = lo; kt < hi; kt += 2) {
    step(kt, 0);
    if (kt + 1 < hi) step(kt + 1, 1);
  }

  if (ns > 1) {
    float* x = part + ((size_t)(qrow / 64) * ns + sw) * 64 * D + (size_t)(qrow % 64) * D;
    asm volatile("" : "+v"(x));
    put_rows_f32<D>(x, dqt, g);
  } else if (qrow < Nq) {
    store_rows_from_acc<D>(dQh + (size_t)qrow * D, dqt, scale, g);
  }
}

// One launch for the whole backward. Per head the workgroups run the dK/dV key tiles first
// and then the dQ query tiles, each kind longest first: the dK/dV tiles that finish first
// (few visible queries) free their CUs for the longest dQ tiles.
//
// Small grids (Nq = Nk = N, N % 128 == 0) spread each workgroup's steps over ns workgroups
// (consecutive blocks, so a tile's shares start together): share sw runs the sw-th of ns equal
// slices and writes fp32 partial sums, per 64-row tile t of head bh and share sw, as [64][D]
// rows of dK^T and dV^T at kvpart + ((bh T + t) ns + sw) 2 * 64 D (dV^T after dK^T) and of dQ^T
// at qpart + ((bh T + t) ns + sw) 64 D, T = N / 64; bwd_split_combine_kernel adds them up.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_kernel(const bf16* __restrict__ Q,
                                                  const bf16* __restrict__ K,
                                                  const bf16* __restrict__ V,
                                                  const float* __restrict__ L2,
                                                  const float* __restrict__ ND,
                                                  const bf16* __restrict__ dO,
                                                  bf16* __restrict__ dQ, bf16* __restrict__ dK,
                                                  bf16* __restrict__ dV, int Nq, int Nk,
                                                  float scale, int neg, int ns,
                                                  float* __restrict__ kvpart,
                                                  float* __restrict__ qpart) {
  constexpr int SM = Bwd<D>::KV_BUF > Bwd<D>::Q_BUF ? Bwd<D>::KV_BUF : Bwd<D>::Q_BUF;
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * SM];
  const int nkv = (Nk + 127) / 128, nqw = (Nq + 127) / 128;
  const int per_head = nkv + nqw;
  // Split grids keep the dispatch order: the hardware deals consecutive blocks to the eight
  // XCDs in turn, so every XCD gets its even share of the long and the short shares (by
  // XCD-contiguous ranges one XCD would take all the longest dK/dV tiles of a head).
  const int lid = ns > 1 ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  const int sw = lid % ns, pid = lid / ns;
  const int bh = pid / per_head, idx = pid % per_head;
  const size_t head_part = (size_t)bh * (Nq / 64) * ns * 64 * D;  // one tensor's tiles per head
  const size_t oq = (size_t)bh * Nq * D, ok = (size_t)bh * Nk * D;
  const uint32_t bq = (uint32_t)Nq * D * 2, bk = (uint32_t)Nk * D * 2;
  const rsrc_t Qr = make_rsrc(Q + oq, bq), dOr = make_rsrc(dO + oq, bq);
  const rsrc_t Kr = make_rsrc(K + ok, bk), Vr = make_rsrc(V + ok, bk);
  const rsrc_t L2r = make_rsrc(L2 + (size_t)bh * Nq, (uint32_t)Nq * 4);
  const rsrc_t NDr = make_rsrc(ND + (size_t)bh * Nq, (uint32_t)Nq * 4);
  if (idx < nkv) {
    dkdv_part<D, CAUSAL>(smem, Qr, Kr, Vr, L2r, NDr, dOr, dK + ok, dV + ok, idx * 128, Nq, Nk,
                         scale, neg, sw, ns, ns > 1 ? kvpart + 2 * head_part : nullptr);
  } else {
    const int it = CAUSAL ? nqw - 1 - (idx - nkv) : idx - nkv;
    dq_part<D, CAUSAL>(smem, Qr, Kr, Vr, L2r, NDr, dOr, dQ + oq, it * 128, Nq, Nk, scale, neg,
                       sw, ns, ns > 1 ? qpart + head_part : nullptr);
  }
}

// Backward with dQ accumulated atomically: the nondeterministic alternative to the two-pass
// split ("Systems and Parallelism" (CS336 field map, A2), section 1.3.3, names both). Only the
// dK/dV kind of workgroup runs: 128 keys each (four waves of 32), walking the visible 32-row
// query tiles as dkdv_part does. Each wave also stages its dS (bf16, transposed) in LDS and
// forms its keys' share of the tile's dQ, dS K, on the matrix cores; the four shares are
// summed in LDS and added into the fp32 accumulator dqacc ([B, H, Nq, d], zeroed beforehand)
// with hardware float atomics; dq_convert_kernel then scales and rounds it. The order of
// the additions, and so dQ's last bits, vary from run to run.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void bwd_atomic_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ L2, const float* __restrict__ ND, const bf16* __restrict__ dO,
    float* __restrict__ dqacc, bf16* __restrict__ dK, bf16* __restrict__ dV, int Nq, int Nk,
    float scale, int neg) {
  using B = Bwd<D>;
  using DTile = Tile<32, 32>;
  constexpr int DS = B::DS, DB = B::DB;
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * B::KV_BUF];
  __shared__ __attribute__((aligned(1024))) bf16 ktile[4][B::T];        // a wave's 32 keys
  __shared__ __attribute__((aligned(1024))) bf16 dstile[4][DTile::ELEMS];  // a wave's dS^T
  __shared__ __attribute__((aligned(16))) float red[4][32 * D];  // the waves' dQ shares
  const int nkv = (Nk + 127) / 128;
  // A head's workgroups on one XCD where the grid allows (they add into the same rows).
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nkv, k0 = (lid % nkv) * 128;
  const size_t oq = (size_t)bh * Nq * D, ok = (size_t)bh * Nk * D;
  const uint32_t bq = (uint32_t)Nq * D * 2, bk = (uint32_t)Nk * D * 2;
  const rsrc_t Qr = make_rsrc(Q + oq, bq), dOr = make_rsrc(dO + oq, bq);
  const rsrc_t Kr = make_rsrc(K + ok, bk), Vr = make_rsrc(V + ok, bk);
  const rsrc_t L2r = make_rsrc(L2 + (size_t)bh * Nq, (uint32_t)Nq * 4);
  const rsrc_t NDr = make_rsrc(ND + (size_t)bh * Nq, (uint32_t)Nq * 4);
  const int lane = threadIdx.x & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int kw0 = k0 + 32 * w;
  const int krow = kw0 + l32;
  const float c = exp2_coef(scale);

  bf16x8 kf[DS], vf[DS];
  load_kv_rows<D>(kf, vf, Kr, Vr, krow, g, neg);
  // This wave's K rows (unnegated; rows past Nk read as zeros), the B operand of dS K.
  B::MTile::template load<1>(Kr, kw0, ktile[w], 0, lane);
  f32x16 dvt[DB], dkt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dvt[db] = zero16();
    dkt[db] = zero16();
  }
  const int nmt = (Nq + 31) / 32;
  const int lo = CAUSAL ? min(k0 / 32, nmt) : 0, hi = nmt;
  if (lo < hi) kv_fetch<D, 4>(Qr, dOr, L2r, NDr, lo * 32, smem, w, lane);
  wait_vmem();
  __syncthreads();
  for (int mt = lo; mt < hi; ++mt) {
    bf16* buf = smem + ((mt - lo) & 1) * B::KV_BUF;
    bf16* nbuf = smem + (((mt - lo) & 1) ^ 1) * B::KV_BUF;
    const int m0 = mt * 32;
    const bool active = kw0 < Nk && (!CAUSAL || m0 + 31 >= kw0);
    KvOps<D> op;  // unused: transposed operands are read late (see KvOps)
    if (mt + 1 < hi) kv_fetch<D, 4>(Qr, dOr, L2r, NDr, m0 + 32, nbuf, w, lane);
    if (active) {
      kv_step<D, false, true>(buf, op, kf, vf, dvt, dkt, c, CAUSAL && m0 < kw0 + 31,
                              krow - m0 - 4 * g, lane, l32, g, dstile[w]);
      // dQ share of this wave's keys: register r of block db holds query 8(r/4) + 4g + r%4
      // of the tile and column 32 db + l32 (at d = 16 the upper half of the block is padding).
      f32x16 dq[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) dq[db] = zero16();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = DTile::tfrag(dstile[w], 0, 16 * ks, lane);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dq[db] = mfma32(a, B::MTile::tfrag(ktile[w], 32 * db, 16 * ks, lane), dq[db]);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + l32;
        if (col < D)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            red[w][(8 * (r >> 2) + 4 * g + (r & 3)) * D + col] = dq[db][r];
      }
    }
    // The four shares are summed in LDS and each wave adds 8 of the tile's rows (8 d
    // consecutive floats of the accumulator) to it: one atomic addition per element and tile
    // instead of four. Element e = 64 i + lane of the wave's block is row 8w + e/d, column
    // e%d, so each atomic instruction covers 64 consecutive floats.
    __syncthreads();
    {
      constexpr int NI = D / 8;  // atomic instructions per lane
      float acc[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[i] = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kv0 = k0 + 32 * v;
        if (kv0 < Nk && (!CAUSAL || m0 + 31 >= kv0))
#pragma unroll
          for (int i = 0; i < NI; ++i) acc[i] += red[v][8 * w * D + 64 * i + lane];
      }
      float* dst = dqacc + oq + (size_t)(m0 + 8 * w) * D;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int e = 64 * i + lane;
        if (m0 + 8 * w + e / D < Nq) unsafeAtomicAdd(dst + e, acc[i]);
      }
    }
    wait_vmem();
    __syncthreads();
  }
  if (krow < Nk) {
    store_rows_from_acc<D>(dK + ok + (size_t)krow * D, dkt, scale, g);
    store_rows_from_acc<D>(dV + ok + (size_t)krow * D, dvt, 1.f, g);
  }
}

// Zeroes n floats (the atomic dQ accumulator, which follows the per-row terms and so may be
// only 4-byte aligned).
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// dQ = bf16(scale * acc) elementwise (round to nearest even).
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc,
                                                         bf16* __restrict__ dQ, long long n,
                                                         float scale) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dQ[i] = (bf16)(acc[i] * scale);
}

// Runs step(n, cur) for n = first .. last-1 over tiles that fetch(n, dst) loads straight into
// LDS, two tiles ahead, through three buffers. Each step issues the loads of tile n+2, runs,
// then waits for tile n+1 only (vmcnt(KEEP), KEEP = vector-memory instructions one fetch
// issues per wave) and meets the other waves at an LDS-only barrier. The loop sits in one
// function whose buffers are restrict parameters and is unrolled by three, so every access
// names its buffer statically: the compiler can then tell that a step's (transposed) LDS
// reads of `cur` do not alias the loads in flight into the other two buffers, and inserts no
// wait for them. A step that issues other vector-memory instructions must wait for all of
// them itself before returning.
//
// ready() runs once after the first two tiles' loads have landed and before the first step:
// the caller issues its own first loads (stationary fragments) ahead of the call, so they
// share that one memory round trip, and finishes them in ready().
template <int KEEP, class Fetch, class Step, class Ready>
__device__ __forceinline__ void stream3(int first, int last, bf16* __restrict__ b0,
                                        bf16* __restrict__ b1, bf16* __restrict__ b2,
                                        Fetch&& fetch, Step&& step, Ready&& ready) {
  if (first < last) fetch(first, b0);
  if (first + 1 < last) fetch(first + 1, b1);
  wait_vmem();
  ready();
  __syncthreads();
  auto one = [&](int n, bf16* cur, bf16* pre) {
    const bool more = n + 2 < last;
    if (more) fetch(n + 2, pre);
    step(n, cur);
    if (more)
      wait_vmem_keep<KEEP>();
    else
      wait_vmem();
    lds_barrier();
  };
  for (int n = first; n < last; n += 3) {
    one(n, b0, b2);
    if (n + 1 < last) one(n + 1, b1, b0);
    if (n + 2 < last) one(n + 2, b2, b1);
  }
}

// Causal backward with complementary tile pairing, for Nq = Nk = N, N % 128 == 0 (the
// counterpart of fwd_causal_paired_kernel). Tiles are 64 rows, held by a wave pair (32 rows
// per wave); steps are 32-row moving tiles. Per head, T/2 workgroups do dK/dV and T/2 do dQ
// (T = N/64):
//   dK/dV workgroup j: key tile A = j sees query steps 2j .. 2T-1 (2(T-j) steps) and key tile
//     B = T-1-j sees 2(j+1) steps: 2(T+1) together. Pair 0 runs A's first T+1 steps; pair 1
//     runs B and then A's remaining T-2j-1 steps.
//   dQ workgroup i: query tile A = T-1-i sees key steps 0 .. 2(T-i)-1 and B = i sees
//     2(i+1): pair 0 runs A's first T+1 steps, pair 1 runs B and then A's rest.
// Both pairs make exactly T+1 steps in lockstep, each with its own stream; pair 1 then adds its
// partial sums for A into pair 0's through LDS.
//
// LEAN reads each step's transposed operands where the products use them instead of up front
// (kv_step and q_step with EARLY = false), which fits three workgroups per CU (168 VGPRs):
// bwd_causal_paired_lean_kernel runs grids of two to three workgroups per CU all at once,
// where two per CU would leave a second, half-empty wave of workgroups.
template <int D, bool LEAN>
__device__ __forceinline__ void bwd_paired_body(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ L2, const float* __restrict__ ND, const bf16* __restrict__ dO,
    bf16* __restrict__ dQ, bf16* __restrict__ dK, bf16* __restrict__ dV, int N, float scale,
    int neg, int ns, float* __restrict__ kvpart, float* __restrict__ qpart) {
  using B = Bwd<D>;
  constexpr int DS = B::DS, DB = B::DB;
  constexpr int SM = B::KV_BUF > B::Q_BUF ? B::KV_BUF : B::Q_BUF;
  __shared__ __attribute__((aligned(1024))) bf16 smem[2][3][SM];  // [pair][buffer]
  static_assert(B::MTile::NKIB % 2 == 0, "each wave of a pair loads the same number of blocks");

  const int T = N / 64, half = T / 2;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int sw = lid % ns, pid = lid / ns;  // this workgroup's share of workgroup pid's steps
  const int bh = pid / T, idx = pid % T;
  const size_t o = (size_t)bh * N * D;
  const uint32_t nb = (uint32_t)N * D * 2;
  const rsrc_t Qr = make_rsrc(Q + o, nb), dOr = make_rsrc(dO + o, nb);
  const rsrc_t Kr = make_rsrc(K + o, nb), Vr = make_rsrc(V + o, nb);
  const rsrc_t L2r = make_rsrc(L2 + (size_t)bh * N, (uint32_t)N * 4);
  const rsrc_t NDr = make_rsrc(ND + (size_t)bh * N, (uint32_t)N * 4);

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int pr = w >> 1, wp = w & 1;  // pair, wave in pair
  const float c = exp2_coef(scale);
  const int nsteps = T + 1;
  // With ns > 1 this workgroup runs steps [n_lo, n_hi) of both pairs' runs and writes fp32
  // partial sums per 64-row tile (records of component-major lanes, as the merge below) for
  // bwd_split_combine_kernel to add up.
  const int n_lo = sw * nsteps / ns, n_hi = (sw + 1) * nsteps / ns;
  constexpr int XS = 2 * 16 * DB;  // merge record per lane: up to two accumulator sets
  // Partial sums (ns > 1) are fp32 [64 rows][D] tiles: for key tile t and share sw, dK^T at
  // kvpart + ((bh T + t) ns + sw) 2 * 64 D and dV^T right after it; dQ^T at qpart + ((bh T +
  // t) ns + sw) 64 D. part_row gives this lane's row (32 wp + l32) in one of them.
  auto part_row = [&](float* base, int tile, int tensors, int which) {
    return base + ((((size_t)bh * T + tile) * ns + sw) * tensors + which) * (64 * D) +
           (32 * wp + l32) * D;
  };

  if (idx < half) {
    // ---------------------------------------------------------------- dK / dV workgroup
    const int tA = idx, tB = T - 1 - idx;
    const int nB = 2 * (tB == tA ? 0 : idx + 1);  // steps of B (pair 1), 2(j+1)
    // step n of this pair -> key tile and moving query tile
    auto kt_of = [&](int n) { return (pr == 0 || n >= nB) ? tA : tB; };
    auto mt_of = [&](int n) {
      return pr == 0 ? 2 * tA + n : (n < nB ? 2 * tB + n : 2 * tA + nsteps + (n - nB));
    };
    // The first tile, written out rather than as kt_of(n_lo): through the lambda, hipcc 7.2
    // keeps tA and tB in scratch memory and reloads them every step.
    int kt = (pr == 1 && n_lo < nB) ? tB + 0 : tA + 0;
    int krow = 64 * kt + 32 * wp + l32;
    bf16x8 kf[DS], vf[DS];
    load_frags<D>(kf, Kr, krow, g);  // lands with the first two tiles (stream3's ready)
    load_frags<D>(vf, Vr, krow, g);
    f32x16 dvt[DB], dkt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dvt[db] = zero16();
      dkt[db] = zero16();
    }
    // Per wave, one fetch issues NKIB/2 loads for each of Q and dO, and one for L2 or ND.
    constexpr int kKeep = B::MTile::NKIB + 1;
    stream3<kKeep>(
        n_lo, n_hi, smem[pr][0], smem[pr][1], smem[pr][2],
        [&](int n, bf16* dst) {
          kv_fetch<D, 2, true>(Qr, dOr, L2r, NDr, 32 * mt_of(n), dst, wp, lane);
        },
        [&](int n, bf16* buf) {
          const int m0 = 32 * mt_of(n);
          const int kw0 = 64 * kt + 32 * wp;
          if (m0 + 31 >= kw0) {
            KvOps<D> op;
            kv_step<D, !LEAN>(buf, op, kf, vf, dvt, dkt, c, m0 < kw0 + 31, krow - m0 - 4 * g,
                              lane, l32, g);
          }
          if (pr == 1 && n + 1 == nB) {  // B is complete: store it and switch to A
            if (ns > 1) {
              put_rows_f32<D>(part_row(kvpart, tB, 2, 0), dkt, g);
              put_rows_f32<D>(part_row(kvpart, tB, 2, 1), dvt, g);
            } else {
              store_rows_from_acc<D>(dK + o + (size_t)krow * D, dkt, scale, g);
              store_rows_from_acc<D>(dV + o + (size_t)krow * D, dvt, 1.f, g);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              dvt[db] = zero16();
              dkt[db] = zero16();
            }
            kt = tA;
            krow = 64 * kt + 32 * wp + l32;
            load_kv_rows<D>(kf, vf, Kr, Vr, krow, g, neg);  // waits for all its loads
          }
        },
        [&] {
          if (neg)
#pragma unroll
            for (int s = 0; s < DS; ++s) kf[s] = negate(kf[s]);
        });
    // Pair 1 holds A's partial sums unless its A range was empty (n == nB at the end). The
    // merge record is component-major (component k of wave wp's lane at k * 128 + wp * 64 +
    // lane), so the exchange is free of bank conflicts.
    const bool p1_has_A = n_hi > nB;
    // B's partial from this share: written at the switch when B completes inside the share
    // (n_lo < nB <= n_hi); here when the share ends before B completes (pair 1's sums are
    // B's), or as zeros when the share has no B step.
    if (ns > 1 && pr == 1) {
      if (n_lo >= nB) {
        put_zero_rows_f32<D>(part_row(kvpart, tB, 2, 0), g);
        put_zero_rows_f32<D>(part_row(kvpart, tB, 2, 1), g);
      } else if (n_hi < nB) {
        put_rows_f32<D>(part_row(kvpart, tB, 2, 0), dkt, g);
        put_rows_f32<D>(part_row(kvpart, tB, 2, 1), dvt, g);
      }
    }
    float* xf = reinterpret_cast<float*>(&smem[0][0][0]);
    static_assert(2 * 64 * XS * sizeof(float) <= sizeof(smem), "merge area must fit");
    if (pr == 1 && p1_has_A) {
      float* x = xf + wp * 64 + lane;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          x[(16 * db + r) * 128] = dkt[db][r];
          x[(16 * (DB + db) + r) * 128] = dvt[db][r];
        }
    }
    __syncthreads();
    if (pr == 0) {
      if (p1_has_A) {
        const float* x = xf + wp * 64 + lane;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            dkt[db][r] += x[(16 * db + r) * 128];
            dvt[db][r] += x[(16 * (DB + db) + r) * 128];
          }
      }
      if (ns > 1) {
        put_rows_f32<D>(part_row(kvpart, tA, 2, 0), dkt, g);
        put_rows_f32<D>(part_row(kvpart, tA, 2, 1), dvt, g);
      } else {
        store_rows_from_acc<D>(dK + o + (size_t)krow * D, dkt, scale, g);
        store_rows_from_acc<D>(dV + o + (size_t)krow * D, dvt, 1.f, g);
      }
    }
  } else {
    // ------------------------------------------------------------------------ dQ workgroup
    const int i = idx - half;
    const int tA = T - 1 - i, tB = i;
    const int nB = 2 * (i + 1);
    auto qt_of = [&](int n) { return (pr == 0 || n >= nB) ? tA : tB; };
    auto kt_of = [&](int n) { return pr == 0 ? n : (n < nB ? n : nsteps + (n - nB)); };
    int qt = (pr == 1 && n_lo < nB) ? tB + 0 : tA + 0;  // as kt above
    int qrow = 64 * qt + 32 * wp + l32;
    QRow<D> row;
    row.issue(Qr, dOr, L2r, NDr, qrow, g);  // lands with the first two tiles (stream3's ready)
    f32x16 dqt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dqt[db] = zero16();
    // Per wave, one fetch issues NKIB/2 loads for each of K and V.
    constexpr int kKeep = B::MTile::NKIB;
    stream3<kKeep>(
        n_lo, n_hi, smem[pr][0], smem[pr][1], smem[pr][2],
        [&](int n, bf16* dst) {
          B::MTile::template load_in_range<2>(Kr, 32 * kt_of(n), dst, wp, lane);
          B::MTile::template load_in_range<2>(Vr, 32 * kt_of(n), dst + B::T, wp, lane);
        },
        [&](int n, bf16* buf) {
          const int n0 = 32 * kt_of(n);
          const int qw0 = 64 * qt + 32 * wp;
          if (n0 <= qw0 + 31) {
            QOps<D> op;
            q_step<D, !LEAN>(buf, op, row.qf, row.dof, dqt, c, row.l2, row.nd, n0 + 31 > qw0,
                             qrow - n0 - 4 * g, lane, l32, g);
          }
          if (pr == 1 && n + 1 == nB) {  // B is complete: store it and switch to A
            if (ns > 1)
              put_rows_f32<D>(part_row(qpart, tB, 1, 0), dqt, g);
            else
              store_rows_from_acc<D>(dQ + o + (size_t)qrow * D, dqt, scale, g);
#pragma unroll
            for (int db = 0; db < DB; ++db) dqt[db] = zero16();
            qt = tA;
            qrow = 64 * qt + 32 * wp + l32;
            row.load(Qr, dOr, L2r, NDr, qrow, g, neg);  // waits for all its loads
          }
        },
        [&] { row.finish(neg); });
    const bool p1_has_A = n_hi > nB;
    if (ns > 1 && pr == 1) {  // as for dK/dV above
      if (n_lo >= nB)
        put_zero_rows_f32<D>(part_row(qpart, tB, 1, 0), g);
      else if (n_hi < nB)
        put_rows_f32<D>(part_row(qpart, tB, 1, 0), dqt, g);
    }
    float* xf = reinterpret_cast<float*>(&smem[0][0][0]);
    if (pr == 1 && p1_has_A) {
      float* x = xf + wp * 64 + lane;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[(16 * db + r) * 128] = dqt[db][r];
    }
    __syncthreads();
    if (pr == 0) {
      if (p1_has_A) {
        const float* x = xf + wp * 64 + lane;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) dqt[db][r] += x[(16 * db + r) * 128];
      }
      if (ns > 1)
        put_rows_f32<D>(part_row(qpart, tA, 1, 0), dqt, g);
      else
        store_rows_from_acc<D>(dQ + o + (size_t)qrow * D, dqt, scale, g);
    }
  }
}

#define FA_PAIRED_ARGS                                                                    \
  const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,       \
      const float *__restrict__ L2, const float *__restrict__ ND, const bf16 *__restrict__ dO, \
      bf16 *__restrict__ dQ, bf16 *__restrict__ dK, bf16 *__restrict__ dV, int N, float scale, \
      int neg, int ns, float *__restrict__ kvpart, float *__restrict__ qpart
template <int D>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void bwd_causal_paired_kernel(FA_PAIRED_ARGS) {
  bwd_paired_body<D, false>(Q, K, V, L2, ND, dO, dQ, dK, dV, N, scale, neg, ns, kvpart, qpart);
}
template <int D>
__global__ __launch_bounds__(256, 3) void bwd_causal_paired_lean_kernel(FA_PAIRED_ARGS) {
  bwd_paired_body<D, true>(Q, K, V, L2, ND, dO, dQ, dK, dV, N, scale, neg, ns, kvpart, qpart);
}
#undef FA_PAIRED_ARGS

// Adds the ns partial [64][D] fp32 tiles that bwd_causal_paired_kernel or bwd_kernel wrote for
// each 64-row tile when it spread every workgroup's steps over ns workgroups, scales dK and dQ,
// and stores dQ, dK and dV. Each thread sums one float4 of one tensor over the ns shares
// (independent loads, consecutive threads on consecutive addresses); a tile's three tensors
// take 3 * 64 * D / 1024 workgroups of 256 threads.
template <int D>
__global__ __launch_bounds__(256) void bwd_split_combine_kernel(
    const float* __restrict__ kvpart, const float* __restrict__ qpart, bf16* __restrict__ dQ,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int N, float scale, int ns) {
  constexpr int MAXW = 8, TILE = 64 * D, BLOCKS = 3 * TILE / 1024;  // per tile
  const int T = N / 64;
  const int tb = blockIdx.x / BLOCKS, part = blockIdx.x % BLOCKS;
  const int tile = tb % T, bh = tb / T;
  const size_t base = ((size_t)bh * T + tile) * ns;
  const int e = part * 1024 + 4 * threadIdx.x;
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
  const float mul = tensor == 1 ? 1.f : scale;
  bf16* out = tensor == 0 ? dK : (tensor == 1 ? dV : dQ);
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (bf16)(acc[i] * mul);
  *reinterpret_cast<bf16x4*>(out + ((size_t)bh * N + 64 * tile) * D + k) = o;
}

// The causal paired backward runs grids of up to three of its workgroups per CU (d = 32, 64).
bool bwd_uses_paired(const Shape& s) {
  return s.causal && s.d >= 32 && s.d <= 64 && s.Nq == s.Nk && s.Nq % 128 == 0 &&
         (long long)(s.Nq / 64) * s.BH <= 3 * kNumCUs;
}

// Workgroups per workgroup of the split backward (Nq = Nk, a multiple of 128). Small grids
// spread each workgroup's steps over up to 8 workgroups, doubling while every share keeps at
// least kMinShare steps and the grid stays within the CUs' room for the kernel's workgroups
// (two per CU for either kernel). Causal bwd_kernel grids may take twice that: their shares
// differ in length, and dispatched longest first, the short dK/dV shares free their CUs for
// the long dQ ones.
constexpr int kMinShare = 8;
int bwd_split_ways(const Shape& s) {
  if (s.Nq != s.Nk || s.Nq % 128 != 0) return 1;
  const bool paired = bwd_uses_paired(s);
  const long long wgs = (long long)(s.Nq / 64) * s.BH;  // either kernel: N / 64 per head
  const long long room = (long long)kNumCUs * 2 * (!paired && s.causal ? 2 : 1);
  const int steps = paired ? s.Nq / 64 + 1 : s.Nq / 32;  // the longest workgroup's steps
  int ns = 1;
  while (ns < 8 && wgs * ns * 2 <= room && steps / (ns * 2) >= kMinShare) ns *= 2;
  return ns;
}

// Workgroups per tile pair of the causal small-grid forward kernels (the split kernel at
// d = 16 and 32, the wide kernel at d = 64, the paired kernel at d = 128). Small grids spread each pair's key steps over up
// to kMaxWays workgroups, doubling while the grid still fits the CUs (one such workgroup per
// CU) and every wave pair keeps a run of at least kMinRun key steps; larger grids use one.
constexpr int kMinRun = 4, kMaxWays = 8;
static_assert(kMaxWays <= 8, "fwd_split_combine_kernel merges at most 8 records per tile");
int fwd_split_ways(const Shape& s) {
  if (!s.causal || s.Nq != s.Nk || s.Nq % 128 != 0) return 1;
  const long long pairs = (long long)(s.Nq / 128) * s.BH;
  if (pairs > kNumCUs) return 1;
  // Key steps of one wave pair's run per share: the split kernel cuts the pair's T + 1 steps
  // into 4 runs, the paired kernel's longer run is T/2 + 1. (The wide kernel at d = 64 cuts
  // them into 8 runs of half that length; the rule is kept the same for it.)
  const int steps = s.d <= 64 ? (s.Nq / 64 + 1) / 4 : s.Nq / 128 + 1;
  int ns = 1;
  while (ns < kMaxWays && pairs * ns * 2 <= kNumCUs && steps / (ns * 2) >= kMinRun) ns *= 2;
  return ns;
}

}  // namespace

size_t fwd_workspace_bytes_bf16(const Shape& s) {
  const int ns = fwd_split_ways(s);
  if (ns == 1) return 0;
  const size_t xs = 16 * ((s.d + 31) / 32) + 2;  // floats per lane in a partial record
  return (size_t)(s.Nq / 128) * s.BH * ns * 2 * xs * 128 * sizeof(float);
}

size_t bwd_split_workspace_bytes_bf16(const Shape& s) {
  // The size does not depend on the call being causal: room for either.
  Shape c = s, n = s;
  c.causal = true;
  n.causal = false;
  const int ns = std::max(bwd_split_ways(c), bwd_split_ways(n));
  if (ns == 1) return 0;
  // Per 64-row tile and share: fp32 [64][d] tiles of dK^T, dV^T and dQ^T.
  return (size_t)(s.Nq / 64) * s.BH * ns * 3 * 64 * s.d * sizeof(float);
}

namespace {

// Which forward kernel a call runs, and the workgroups per tile pair (ns > 1: the split
// launch whose partial results fwd_split_combine_kernel merges). Pairing pays off only when
// one 128-query tile per workgroup leaves CUs idle or runs a single wave per SIMD anyway;
// larger grids keep the plain kernel (shared K/V stream, two waves per SIMD). Up to one tile
// pair per CU, d <= 64 takes an eight-wave kernel (the wide kernel at d = 64, the split kernel
// below that) and d = 128 the paired kernel; up
// to two (d = 32, 64), the four-wave paired kernel (two fit a CU), whose balanced steps beat
// the plain kernel's longest-tile tail.
enum FwdKernel { kFwdPlain, kFwdPaired, kFwdSplit };
struct FwdPlan {
  FwdKernel kernel;
  int ns;
};

FwdPlan fwd_plan(const Shape& s, size_t ws_bytes) {
  const long long pairs = (long long)(s.Nq / 128) * s.BH;
  const bool square = s.causal && s.Nq == s.Nk && s.Nq % 128 == 0;
  if (square && s.d >= 32 && s.d <= 64 && pairs > kNumCUs && pairs <= 2 * kNumCUs)
    return {kFwdPaired, 1};
  if (square && pairs <= kNumCUs) {
    int ns = fwd_split_ways(s);
    if (ns > 1 && ws_bytes < fwd_workspace_bytes_bf16(s)) ns = 1;
    return {s.d <= 64 ? kFwdSplit : kFwdPaired, ns};
  }
  return {kFwdPlain, 1};
}

template <int D, bool CAUSAL>
hipError_t fwd_t(const Shape& s, const void* Q, const void* K, const void* V, void* O, float* L,
                 float* ws, size_t ws_bytes, hipStream_t stream) {
  const FwdPlan pl = fwd_plan(s, ws_bytes);
  const int neg = s.scale < 0.f ? 1 : 0;
  if constexpr (CAUSAL) {
    if (pl.kernel != kFwdPlain) {
      const unsigned grid = (unsigned)((long long)(s.Nq / 128) * s.BH * pl.ns);
      if (pl.kernel == kFwdSplit) {
        if constexpr (D == 64)
          hipLaunchKernelGGL((fwd_causal_wide_kernel<D>), dim3(grid), dim3(512), 0, stream,
                             (const bf16*)Q, (const bf16*)K, (const bf16*)V, (bf16*)O, L, s.Nq,
                             s.scale, neg, pl.ns, ws);
        else if constexpr (D <= 64)
          hipLaunchKernelGGL((fwd_causal_split_kernel<D>), dim3(grid), dim3(512), 0, stream,
                             (const bf16*)Q, (const bf16*)K, (const bf16*)V, (bf16*)O, L, s.Nq,
                             s.scale, neg, pl.ns, ws);
      } else {
        if constexpr (D >= 32)
          hipLaunchKernelGGL((fwd_causal_paired_kernel<D>), dim3(grid), dim3(256), 0, stream,
                             (const bf16*)Q, (const bf16*)K, (const bf16*)V, (bf16*)O, L, s.Nq,
                             s.scale, neg, pl.ns, ws);
      }
      if (pl.ns > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((fwd_split_combine_kernel<D>),
                           dim3((unsigned)((long long)s.BH * (s.Nq / 64))),
                           dim3(128 * ((D + 31) / 32)), 0, stream, (const float*)ws, (bf16*)O,
                           L, s.Nq, s.scale, pl.ns);
      }
      return hipGetLastError();
    }
  }
  const int nqt = (s.Nq + 127) / 128;
  const long long grid = (long long)nqt * s.BH;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const bf16*)Q, (const bf16*)K, (const bf16*)V, (bf16*)O, L, s.Nq, s.Nk,
                     s.scale, neg);
  return hipGetLastError();
}

// Workspace layout shared by the two backward launches: L2 for the B*H*Nq query rows, then
// ND for the same rows.
template <int D>
hipError_t bwd_prep_t(const Shape& s, const void* O, const float* L, const void* dO, float* ws,
                      hipStream_t stream) {
  const long long rows = (long long)s.BH * s.Nq;
  if (rows == 0) return hipSuccess;
  const long long grid = std::min((rows * (D / 8) + 255) / 256, 1LL << 16);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const bf16*)O, (const bf16*)dO, L, ws, ws + rows, rows);
  return hipGetLastError();
}

// Which backward main kernel a call runs, and the workgroups each workgroup's steps are
// spread over (ns > 1: fp32 partial sums after the per-row terms in the workspace, added up
// by bwd_split_combine_kernel). The paired kernel takes causal square grids of up to three
// of its workgroups per CU at d = 32 and 64, where the plain grid (two 128-row tiles per
// head per 128 rows) would leave the longest tile on the critical path (d = 128 grids at
// this size are rare, and hipcc 7.2 cannot register-allocate that instantiation, so it is
// not built).
enum BwdKernel { kBwdPlain, kBwdPaired };
struct BwdPlan {
  BwdKernel kernel;
  int ns;
  bool lean;  // paired grids of two to three workgroups per CU: the lean kernel, all resident
};

BwdPlan bwd_plan(const Shape& s, size_t ws_bytes, bool ws_aligned16) {
  const long long rows = (long long)s.BH * s.Nq;
  int ns = bwd_split_ways(s);
  const size_t split_bytes = (size_t)(s.Nq / 64) * s.BH * ns * 3 * 64 * s.d * sizeof(float);
  if (ns > 1 && (ws_bytes < (size_t)rows * 2 * sizeof(float) + split_bytes || !ws_aligned16))
    ns = 1;  // the partial tiles are written and read 16 bytes at a time
  const bool paired = bwd_uses_paired(s);
  const long long wgs = (long long)(s.Nq / 64) * s.BH * ns;
  return {paired ? kBwdPaired : kBwdPlain, ns, paired && wgs > 2 * kNumCUs};
}

template <int D, bool CAUSAL>
hipError_t bwd_t(const Shape& s, const void* Q, const void* K, const void* V, const void* dO,
                 void* dQ, void* dK, void* dV, const float* ws, size_t ws_bytes,
                 hipStream_t stream) {
  const long long rows = (long long)s.BH * s.Nq;
  const float* L2 = ws;
  const float* ND = ws + rows;
  const BwdPlan pl = bwd_plan(s, ws_bytes, (reinterpret_cast<uintptr_t>(ws) & 15u) == 0);
  const int ns = pl.ns;
  const long long tiles = (long long)(s.Nq / 64) * s.BH;  // 64-row tiles (when ns > 1)
  // Partial sums of split grids follow the two per-row arrays in the workspace.
  float* kvpart = const_cast<float*>(ws) + 2 * rows;
  float* qpart = kvpart + (size_t)tiles * ns * 2 * 64 * D;  // after dK^T, dV^T of every tile
  bool launched = false;
  if constexpr (CAUSAL && D >= 32 && D <= 64) {
    if (pl.kernel == kBwdPaired) {
      if (pl.lean)
        hipLaunchKernelGGL((bwd_causal_paired_lean_kernel<D>), dim3((unsigned)(tiles * ns)),
                           dim3(256), 0, stream, (const bf16*)Q, (const bf16*)K,
                           (const bf16*)V, L2, ND, (const bf16*)dO, (bf16*)dQ, (bf16*)dK,
                           (bf16*)dV, s.Nq, s.scale, s.scale < 0.f ? 1 : 0, ns, kvpart, qpart);
      else
        hipLaunchKernelGGL((bwd_causal_paired_kernel<D>), dim3((unsigned)(tiles * ns)),
                           dim3(256), 0, stream, (const bf16*)Q, (const bf16*)K,
                           (const bf16*)V, L2, ND, (const bf16*)dO, (bf16*)dQ, (bf16*)dK,
                           (bf16*)dV, s.Nq, s.scale, s.scale < 0.f ? 1 : 0, ns, kvpart, qpart);
      launched = true;
    }
  }
  if (!launched) {
    const long long grid = (long long)((s.Nk + 127) / 128 + (s.Nq + 127) / 128) * s.BH * ns;
    hipLaunchKernelGGL((bwd_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream,
                       (const bf16*)Q, (const bf16*)K, (const bf16*)V, L2, ND, (const bf16*)dO,
                       (bf16*)dQ, (bf16*)dK, (bf16*)dV, s.Nq, s.Nk, s.scale,
                       s.scale < 0.f ? 1 : 0, ns, kvpart, qpart);
  }
  if (ns > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_split_combine_kernel<D>), dim3((unsigned)(tiles * (3 * 64 * D / 1024))),
                       dim3(256), 0, stream, (const float*)kvpart, (const float*)qpart, (bf16*)dQ,
                       (bf16*)dK, (bf16*)dV, s.Nq, s.scale, ns);
  }
  return hipGetLastError();
}

// Kernel names as a profiler lists them, indexed by d (16, 32, 64, 128) and mask.
int d_index(int d) { return d == 16 ? 0 : d == 32 ? 1 : d == 64 ? 2 : 3; }
const char* const kFwdPlainNames[2][4] = {
    {"fwd_kernel<16, false>", "fwd_kernel<32, false>", "fwd_kernel<64, false>",
     "fwd_kernel<128, false>"},
    {"fwd_kernel<16, true>", "fwd_kernel<32, true>", "fwd_kernel<64, true>",
     "fwd_kernel<128, true>"}};
const char* const kFwdPairedNames[4] = {"", "fwd_causal_paired_kernel<32>",
                                        "fwd_causal_paired_kernel<64>",
                                        "fwd_causal_paired_kernel<128>"};
const char* const kFwdSplitNames[4] = {"fwd_causal_split_kernel<16>",
                                       "fwd_causal_split_kernel<32>",
                                       "fwd_causal_wide_kernel<64>", ""};
const char* const kBwdPlainNames[2][4] = {
    {"bwd_kernel<16, false>", "bwd_kernel<32, false>", "bwd_kernel<64, false>",
     "bwd_kernel<128, false>"},
    {"bwd_kernel<16, true>", "bwd_kernel<32, true>", "bwd_kernel<64, true>",
     "bwd_kernel<128, true>"}};
const char* const kBwdPairedLeanNames[4] = {"", "bwd_causal_paired_lean_kernel<32>",
                                            "bwd_causal_paired_lean_kernel<64>", ""};
const char* const kBwdPairedNames[4] = {"", "bwd_causal_paired_kernel<32>",
                                        "bwd_causal_paired_kernel<64>", ""};

}  // namespace

hipError_t launch_fwd_bf16(const Shape& s, const void* Q, const void* K, const void* V, void* O,
                           float* L, float* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
#define FA_FWD(DD)                                                                             \
  case DD:                                                                                     \
    return s.causal ? fwd_t<DD, true>(s, Q, K, V, O, L, workspace, workspace_bytes, stream)    \
                    : fwd_t<DD, false>(s, Q, K, V, O, L, workspace, workspace_bytes, stream);
  switch (s.d) {
    FA_FWD(16)
    FA_FWD(32)
    FA_FWD(64)
    FA_FWD(128)
    default:
      return hipErrorInvalidValue;
  }
#undef FA_FWD
}

hipError_t launch_bwd_prep_bf16(const Shape& s, const void* O, const float* L, const void* dO,
                                float* workspace, hipStream_t stream) {
  switch (s.d) {
    case 16:
      return bwd_prep_t<16>(s, O, L, dO, workspace, stream);
    case 32:
      return bwd_prep_t<32>(s, O, L, dO, workspace, stream);
    case 64:
      return bwd_prep_t<64>(s, O, L, dO, workspace, stream);
    case 128:
      return bwd_prep_t<128>(s, O, L, dO, workspace, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_main_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                                const void* dO, void* dQ, void* dK, void* dV,
                                const float* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
#define FA_BWD(DD)                                                                              \
  case DD:                                                                                      \
    return s.causal                                                                             \
               ? bwd_t<DD, true>(s, Q, K, V, dO, dQ, dK, dV, workspace, workspace_bytes, stream) \
               : bwd_t<DD, false>(s, Q, K, V, dO, dQ, dK, dV, workspace, workspace_bytes, stream);
  switch (s.d) {
    FA_BWD(16)
    FA_BWD(32)
    FA_BWD(64)
    FA_BWD(128)
    default:
      return hipErrorInvalidValue;
  }
#undef FA_BWD
}


namespace {
template <int D, bool CAUSAL>
hipError_t bwd_atomic_t(const Shape& s, const void* Q, const void* K, const void* V,
                        const void* dO, void* dQ, void* dK, void* dV, float* ws,
                        hipStream_t stream) {
  const long long rows = (long long)s.BH * s.Nq;
  const float* L2 = ws;
  const float* ND = ws + rows;
  float* acc = ws + 2 * rows;
  const long long n = rows * D;  // 0 when there are no query rows (dK = dV = 0 then)
  if (n > 0) {
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, acc, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long grid = (long long)((s.Nk + 127) / 128) * s.BH;
  if (grid > 0) {
    hipLaunchKernelGGL((bwd_atomic_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0,
                       stream, (const bf16*)Q, (const bf16*)K, (const bf16*)V, L2, ND,
                       (const bf16*)dO, acc, (bf16*)dK, (bf16*)dV, s.Nq, s.Nk, s.scale,
                       s.scale < 0.f ? 1 : 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n > 0)
    hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, (const float*)acc, (bf16*)dQ, n, s.scale);
  return hipGetLastError();
}
}  // namespace

const char* fwd_kernel_name_bf16(const Shape& s, size_t workspace_bytes) {
  const FwdPlan pl = fwd_plan(s, workspace_bytes);
  const int di = d_index(s.d);
  if (pl.kernel == kFwdSplit) return kFwdSplitNames[di];
  if (pl.kernel == kFwdPaired) return kFwdPairedNames[di];
  return kFwdPlainNames[s.causal ? 1 : 0][di];
}

const char* bwd_kernel_name_bf16(const Shape& s, size_t workspace_bytes) {
  const BwdPlan pl = bwd_plan(s, workspace_bytes, true);
  const int di = d_index(s.d);
  if (pl.kernel == kBwdPaired) return pl.lean ? kBwdPairedLeanNames[di] : kBwdPairedNames[di];
  return kBwdPlainNames[s.causal ? 1 : 0][di];
}

size_t bwd_atomic_workspace_bytes_bf16(const Shape& s) {
  return (size_t)s.BH * (size_t)s.Nq * (2 + (size_t)s.d) * sizeof(float);
}

hipError_t launch_bwd_atomic_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                                  const void* dO, void* dQ, void* dK, void* dV, float* ws,
                                  hipStream_t stream) {
#define FA_ATOMIC_CASE(DD)                                                                 \
  case DD:                                                                                 \
    return s.causal ? bwd_atomic_t<DD, true>(s, Q, K, V, dO, dQ, dK, dV, ws, stream)       \
                    : bwd_atomic_t<DD, false>(s, Q, K, V, dO, dQ, dK, dV, ws, stream);
  switch (s.d) {
    FA_ATOMIC_CASE(16)
    FA_ATOMIC_CASE(32)
    FA_ATOMIC_CASE(64)
    FA_ATOMIC_CASE(128)
  }
#undef FA_ATOMIC_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
