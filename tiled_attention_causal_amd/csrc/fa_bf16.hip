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
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kNumCUs = 256;  // MI355X

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

__device__ __forceinline__ bf16x8 negate(bf16x8 x) {
  u32x4 u = __builtin_bit_cast(u32x4, x);
  u ^= 0x80008000u;
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave index as a scalar, so LDS destinations of the direct loads stay uniform.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// 16 bytes per lane from a buffer straight into LDS: lane i's bytes land at dst + 16 i.
__device__ __forceinline__ void dma16(rsrc_t src, uint32_t byte_off, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)dst, 16, byte_off, 0, 0, 0);
}
// 4 bytes per lane (lane i's word lands at dst + 4 i).
__device__ __forceinline__ void dma4(rsrc_t src, uint32_t byte_off, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)dst, 4, byte_off, 0, 0, 0);
}

// Row-major R x C bf16 LDS tile with 16-byte chunks XOR-swizzled by row (swz in fa_common.h).
template <int R, int C>
struct Tile {
  static constexpr int NCH = C / 8;
  static constexpr int ELEMS = R * C;
  static constexpr int NKIB = ELEMS * 2 / 1024;  // one wave-wide direct load moves 1 KiB
  static_assert(ELEMS * 2 % 1024 == 0, "tile must be a whole number of KiB");

  // Rows [row0, row0 + R) of a head with C columns, spread over NW waves. LDS chunk p holds
  // the global chunk whose swizzled position is p; rows past the head's end read as zeros.
  template <int NW>
  __device__ __forceinline__ static void load(rsrc_t src, int row0, bf16* t, int w, int lane) {
    constexpr int M = NCH < 8 ? NCH - 1 : 7;
#pragma unroll
    for (int i = 0; i < (NKIB + NW - 1) / NW; ++i) {
      const int blk = w + i * NW;
      if (NKIB % NW == 0 || blk < NKIB) {
        const int p = blk * 64 + lane;
        const int row = p / NCH, cp = p % NCH;
        const int gc = cp ^ ((row ^ (row >> 3)) & M);
        dma16(src, (uint32_t)(((row0 + row) * C + gc * 8) * 2), t + blk * 512);
      }
    }
  }
  // Operand with k along columns: lane takes row r, columns 8c .. 8c+7.
  __device__ __forceinline__ static bf16x8 frag(const bf16* t, int r, int c) {
    return lds_frag<NCH>(t, r, c);
  }
  // Transposed operand: lane l takes column cbase + l%32 and the eight rows
  // kbase + 8h + 4g + j (h = 0, 1; j = 0..3; g = l/32) in element order 4h + j, which is the
  // row order of an MFMA C fragment's 16-row step. Each ds_read_b64_tr_b16 gathers, inside
  // a 16-lane group, the 4 x 4 block that lane 4a + b's column needs: lane k of the group
  // reads row base + k/4, columns 4(k%4) .. +3, and receives column 4a+b of rows base..+3.
  __device__ __forceinline__ static bf16x8 tfrag(const bf16* t, int cbase, int kbase, int lane) {
    const int g = lane >> 5, s = (lane >> 4) & 1, k = lane & 15;
    int col = cbase + 16 * s + 4 * (k & 3);
    if constexpr (C < 32) col &= C - 1;  // d = 16: the unused half-block re-reads valid columns
    const int row = kbase + 4 * g + (k >> 2);
    const bf16* p0 = t + swz<NCH>(row, col >> 3) + (col & 7);
    const bf16* p1 = t + swz<NCH>(row + 8, col >> 3) + (col & 7);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p1);
    const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
  }
};

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
// query, register r of block kb = key offset 32kb + 8(r/4) + 4g + r%4 from the tile start.
// Rows rescale only when their max grows by more than 2^8 (in exp2 units): until then the
// stale max keeps every p <= 2^8, and O = acc / l does not depend on which max was used.
template <bool MASKED, int DB>
__device__ __forceinline__ void softmax_tile(f32x16 (&sacc)[2], float& m, float& l,
                                             f32x16 (&o)[DB], float c, bool first, int qlim,
                                             int klim) {
  constexpr float kLazy = 8.f;
  auto vis = [&](int kb, int r) {
    const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
    return off <= qlim && off < klim;
  };
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      mx = fmaxf(mx, (!MASKED || vis(kb, r)) ? sacc[kb][r] : -INFINITY);
  mx = fmaxf(mx, swap_halves(mx));
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
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(fmaf(sacc[kb][r], c, nb));
      if (MASKED && !vis(kb, r)) p = 0.f;
      sacc[kb][r] = p;
      rs += p;
    }
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
  const float c = cs * kLog2e;

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
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
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
      // tiles that straddle the diagonal or the ragged end of K compare indices; masked
      // entries are left out of the row max and zeroed after the exponential, which stays
      // exact for any finite scale (including 0).
      if ((CAUSAL && k0 + BK - 1 > qw0) || k0 + BK > Nk) {
        const int qlim = CAUSAL ? qrow - k0 - 4 * g : 1 << 30;  // visible iff offset <= qlim
        const int klim = Nk - k0 - 4 * g;                       // and offset < klim
        softmax_tile<true>(sacc, m, l, o, c, kt == 0, qlim, klim);
      } else {
        softmax_tile<false>(sacc, m, l, o, c, kt == 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 pf = to_bf16x8(sacc[u >> 1], 8 * (u & 1));
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma32(vfr[u][db], pf, o[db]);
      }
    }
    wait_vmem();
    __syncthreads();
  }

  const float lt = l + swap_halves(l);
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
    bf16* __restrict__ O, float* __restrict__ Lout, int N, float scale, int neg) {
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
  const int bh = lid / half, i = lid % half;
  const int tA = T - 1 - i, tB = i, s = half + 1;
  const rsrc_t Qr = make_rsrc(Q + (size_t)bh * N * D, (uint32_t)N * D * 2);
  const rsrc_t Kr = make_rsrc(K + (size_t)bh * N * D, (uint32_t)N * D * 2);
  const rsrc_t Vr = make_rsrc(V + (size_t)bh * N * D, (uint32_t)N * D * 2);

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int pr = w >> 1, wp = w & 1;  // pair, wave within pair
  const float cs = fabsf(scale);
  const float c = cs * kLog2e;

  // Steps of this pair: step n works on query tile qt(n) and key tile kt(n).
  //   pair 0: n in [0, s):           A, key tile n
  //   pair 1: n in [0, i+1):         B, key tile n;  n in [i+1, T-s+1): A, key tile n - (i+1) + s
  const int nsteps = pr == 0 ? s : T + 1 - s;
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

  auto fetch = [&](int n, bf16 (*dst)[KT]) {
    const int k0 = kt_of(n) * BK;
    KTile::template load<2>(Kr, k0, dst[0], wp, lane);
    KTile::template load<2>(Vr, k0, dst[1], wp, lane);
  };
  auto finish_B = [&]() {  // pair 1, after B's last key tile: B is complete
    const float lt = l + swap_halves(l);
    const int row = 64 * tB + 32 * wp + l32;
    store_rows_from_acc<D>(O + ((size_t)bh * N + row) * D, o, 1.f / lt, g);
    if (g == 0) Lout[(size_t)bh * N + row] = m * cs + logf(lt);
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16();
    m = 0.f;
    l = 0.f;
  };
  auto step = [&](int n, const bf16 (*cur)[KT], bf16 (*nxt)[KT]) {
    // The transposed V reads come before the next tile's direct loads: the compiler cannot
    // tell that they do not alias and would otherwise wait for those loads to land first.
    bf16x8 vfr[4][DB];
    if (n < nsteps)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) vfr[u][db] = KTile::tfrag(cur[1], 32 * db, 16 * u, lane);
    if (n + 1 < nsteps) fetch(n + 1, nxt);
    if (n < nsteps) {
      const int qt = qt_of(n), kt = kt_of(n);
      const bool first = pr == 0 ? n == 0 : (n == 0 || n == tB + 1);
      const int qrow = 64 * qt + 32 * wp + l32;
      const int k0 = kt * BK;
      const bf16x8(&qf)[DS] = qt == tA ? qfA : qfB;
      bf16x8 kfr[2][DS];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < DS; ++q) kfr[kb][q] = KTile::frag(cur[0], 32 * kb + l32, 2 * q + g);
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int q = 0; q < DS; ++q) sacc[kb] = mfma32(kfr[kb][q], qf[q], sacc[kb]);
      }
      if (kt == qt)  // the diagonal tile: key offset <= query offset
        softmax_tile<true>(sacc, m, l, o, c, first, qrow - k0 - 4 * g, 1 << 30);
      else
        softmax_tile<false>(sacc, m, l, o, c, first, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 pf = to_bf16x8(sacc[u >> 1], 8 * (u & 1));
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma32(vfr[u][db], pf, o[db]);
      }
      if (pr == 1 && n == tB) finish_B();
    }
    wait_vmem();
    __syncthreads();
  };

  fetch(0, sb0[pr]);
  wait_vmem();
  __syncthreads();
  for (int n = 0; n < s; n += 2) {
    step(n, sb0[pr], sb1[pr]);
    if (n + 1 < s) step(n + 1, sb1[pr], sb0[pr]);
  }

  // Merge A: pair 1 holds A over key tiles [s, T - i) unless that range is empty.
  const bool p1_has_A = T - tB > s;
  constexpr int XS = 16 * DB + 2;  // per lane: O block(s), m, l
  static_assert(2 * 64 * XS * sizeof(float) <= sizeof(sb0), "merge area must fit in sb0");
  float* xf = reinterpret_cast<float*>(&sb0[0][0][0]);  // 2 waves x 64 lanes x XS
  if (pr == 1 && p1_has_A) {
    float* x = xf + (wp * 64 + lane) * XS;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[16 * db + r] = o[db][r];
    x[16 * DB] = m;
    x[16 * DB + 1] = l;
  }
  __syncthreads();
  if (pr == 0) {
    if (p1_has_A) {
      const float* x = xf + (wp * 64 + lane) * XS;
      const float m1 = x[16 * DB], l1 = x[16 * DB + 1];
      const float mm = fmaxf(m, m1);
      const float a0 = fast_exp2((m - mm) * c), a1 = fast_exp2((m1 - mm) * c);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + x[16 * db + r] * a1;
      l = l * a0 + l1 * a1;
      m = mm;
    }
    const float lt = l + swap_halves(l);
    const int row = 64 * tA + 32 * wp + l32;
    store_rows_from_acc<D>(O + ((size_t)bh * N + row) * D, o, 1.f / lt, g);
    if (g == 0) Lout[(size_t)bh * N + row] = m * cs + logf(lt);
  }
}

// ----------------------------------------------------------------------------- backward

// dK/dV pass: P = exp2(S c - L log2e) and dS = P (dP - D) in place, for score registers laid
// out with lane = key and register r of block qb = query offset 32qb + 8(r/4) + 4g + r%4.
// Masked (query < key) entries get P = dS = 0.
template <bool MASKED, int NB>
__device__ __forceinline__ void dkdv_scores(f32x16 (&sp)[NB], f32x16 (&dp)[NB],
                                            const f32x4 (&l4)[NB][4], const f32x4 (&d4)[NB][4],
                                            float c, int lim) {
#pragma unroll
  for (int qb = 0; qb < NB; ++qb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * j + i;
        float p = fast_exp2(fmaf(sp[qb][r], c, -l4[qb][j][i]));
        if (MASKED && 32 * qb + 8 * j + i < lim) p = 0.f;
        sp[qb][r] = p;
        dp[qb][r] = p * (dp[qb][r] - d4[qb][j][i]);
      }
}

// dQ pass: the same for lane = query and register r of block kb = key offset
// 32kb + 8(r/4) + 4g + r%4; visible iff offset <= qlim and offset < klim.
template <bool MASKED, int NB>
__device__ __forceinline__ void dq_scores(f32x16 (&st)[NB], f32x16 (&dpt)[NB], float c, float l2,
                                          float dsum, int qlim, int klim) {
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(fmaf(st[kb][r], c, -l2));
      const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
      if (MASKED && (off > qlim || off >= klim)) p = 0.f;
      dpt[kb][r] = p * (dpt[kb][r] - dsum);
    }
}

template <int D>
struct BwdCfg {
  static constexpr int MT = 32;  // moving-tile rows
  static constexpr int NB = MT / 32;
  static constexpr int DS = D / 16, DB = (D + 31) / 32;
  using MTile = Tile<MT, D>;
  static constexpr int T = MTile::ELEMS;
  // dK/dV staging: Q, dO, O (row-major), then L (-> L log2e) and D, 64 floats each.
  static constexpr int BUF_KV = 3 * T + 2 * 64 * 2;
  // dQ staging: K, V (row-major).
  static constexpr int BUF_Q = 2 * T;
  static constexpr int BUF = BUF_KV > BUF_Q ? BUF_KV : BUF_Q;
  // D = rowsum(dO o O) over the staged tile: CPT 16-byte chunks per thread, TPR threads per
  // row.
  static constexpr int NCH = D / 8;
  static constexpr int CPT = MT * NCH >= 512 ? 2 : 1;
  static constexpr int TPR = NCH / CPT;
};

__device__ __forceinline__ float dot_bf16x8(u32x4 a, u32x4 b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__builtin_bit_cast(float, a[i] << 16), __builtin_bit_cast(float, b[i] << 16),
               acc);
    acc = fmaf(__builtin_bit_cast(float, a[i] & 0xFFFF0000u),
               __builtin_bit_cast(float, b[i] & 0xFFFF0000u), acc);
  }
  return acc;
}

// dK, dV for the 128 keys starting at k0 of one head.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_part(bf16* smem, rsrc_t Qr, rsrc_t Kr, rsrc_t Vr, rsrc_t Or,
                                          rsrc_t Lr, rsrc_t dOr, bf16* dKh, bf16* dVh, int k0,
                                          int Nq, int Nk, float scale, int neg) {
  using C = BwdCfg<D>;
  using MTile = typename C::MTile;
  constexpr int MT = C::MT, NB = C::NB, DS = C::DS, DB = C::DB, T = C::T;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int kw0 = k0 + 32 * w;
  const int krow = kw0 + l32;
  const float c = fabsf(scale) * kLog2e;

  bf16x8 kf[DS], vf[DS];
  load_frags<D>(kf, Kr, krow, g);
  load_frags<D>(vf, Vr, krow, g);
  if (neg)
#pragma unroll
    for (int s = 0; s < DS; ++s) kf[s] = negate(kf[s]);

  f32x16 dvt[DB], dkt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dvt[db] = zero16();
    dkt[db] = zero16();
  }

  const int nmt = (Nq + MT - 1) / MT;
  const int mt0 = CAUSAL ? k0 / MT : 0;

  auto fetch = [&](int mt, bf16* base) {
    const int m0 = mt * MT;
    MTile::template load<4>(Qr, m0, base, w, lane);
    MTile::template load<4>(dOr, m0, base + T, w, lane);
    MTile::template load<4>(Or, m0, base + 2 * T, w, lane);
    if (w == 0) dma4(Lr, (uint32_t)(m0 + lane) * 4, base + 3 * T);
  };

  if (mt0 < nmt) fetch(mt0, smem);
  wait_vmem();
  __syncthreads();
  for (int mt = mt0; mt < nmt; ++mt) {
    const int buf = (mt - mt0) & 1;
    const int m0 = mt * MT;
    bf16* base = smem + buf * C::BUF;
    const bf16* sQ = base;
    const bf16* sdO = base + T;
    const bf16* sO = base + 2 * T;
    float* sL2 = reinterpret_cast<float*>(base + 3 * T);
    float* sD = sL2 + 64;
    const bool active = kw0 < Nk && (!CAUSAL || m0 + MT - 1 >= kw0);

    f32x16 sp[NB], dp[NB];
    if (active) {
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) {
        bf16x8 qa[DS], da[DS];
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          qa[s] = MTile::frag(sQ, 32 * qb + l32, 2 * s + g);
          da[s] = MTile::frag(sdO, 32 * qb + l32, 2 * s + g);
        }
        sp[qb] = zero16();
        dp[qb] = zero16();
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          sp[qb] = mfma32(qa[s], kf[s], sp[qb]);
          dp[qb] = mfma32(da[s], vf[s], dp[qb]);
        }
      }
    }
    // D and L log2e for the tile's rows, while the MFMAs above run.
    {
      const int row = tid / C::TPR, part = tid % C::TPR;
      float dsum = 0.f;
      if (row < MT) {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
          const int ch = part * C::CPT + i;
          const u32x4 a = *reinterpret_cast<const u32x4*>(sdO + swz<C::NCH>(row, ch));
          const u32x4 b = *reinterpret_cast<const u32x4*>(sO + swz<C::NCH>(row, ch));
          dsum = dot_bf16x8(a, b, dsum);
        }
      }
      dsum = group_sum<C::TPR>(dsum);
      if (row < MT && part == 0) {
        sD[row] = dsum;
        sL2[row] = m0 + row < Nq ? sL2[row] * kLog2e : INFINITY;
      }
    }
    __syncthreads();
    // Transposed dO and Q fragments and this tile's L log2e / D values, all read before the
    // next tile's direct loads are issued (see fwd_kernel); the loads themselves are issued
    // by every wave, outside the `active` branches, so no path reaches these reads with a
    // direct load in flight.
    bf16x8 ofr[2 * NB][DB], qfr[2 * NB][DB];
    f32x4 l4[NB][4], d4[NB][4];
    if (active) {
#pragma unroll
      for (int st = 0; st < 2 * NB; ++st)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          ofr[st][db] = MTile::tfrag(sdO, 32 * db, 16 * st, lane);
          qfr[st][db] = MTile::tfrag(sQ, 32 * db, 16 * st, lane);
        }
#pragma unroll
      for (int qb = 0; qb < NB; ++qb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          l4[qb][j] = *reinterpret_cast<const f32x4*>(sL2 + 32 * qb + 8 * j + 4 * g);
          d4[qb][j] = *reinterpret_cast<const f32x4*>(sD + 32 * qb + 8 * j + 4 * g);
        }
    }
    if (mt + 1 < nmt) fetch(mt + 1, smem + (buf ^ 1) * C::BUF);
    if (active) {
      // Registers: query m0 + 32qb + 8(r/4) + 4g + r%4 against this lane's key; the key is
      // visible iff query >= key, i.e. offset 32qb + 8(r/4) + r%4 >= krow - m0 - 4g.
      if (CAUSAL && m0 < kw0 + 31)
        dkdv_scores<true, NB>(sp, dp, l4, d4, c, krow - m0 - 4 * g);
      else
        dkdv_scores<false, NB>(sp, dp, l4, d4, c, 0);
#pragma unroll
      for (int st = 0; st < 2 * NB; ++st) {
        const bf16x8 pf = to_bf16x8(sp[st >> 1], 8 * (st & 1));
        const bf16x8 sf = to_bf16x8(dp[st >> 1], 8 * (st & 1));
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dvt[db] = mfma32(ofr[st][db], pf, dvt[db]);
          dkt[db] = mfma32(qfr[st][db], sf, dkt[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  }

  if (krow < Nk) {
    store_rows_from_acc<D>(dKh + (size_t)krow * D, dkt, scale, g);
    store_rows_from_acc<D>(dVh + (size_t)krow * D, dvt, 1.f, g);
  }
}

// dQ for the 128 queries starting at q0 of one head.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_part(bf16* smem, rsrc_t Qr, rsrc_t Kr, rsrc_t Vr, rsrc_t Or,
                                        rsrc_t Lr, rsrc_t dOr, bf16* dQh, int q0, int Nq, int Nk,
                                        float scale, int neg) {
  using C = BwdCfg<D>;
  using MTile = typename C::MTile;
  constexpr int MT = C::MT, NB = C::NB, DS = C::DS, DB = C::DB, T = C::T;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + l32;
  const float c = fabsf(scale) * kLog2e;

  bf16x8 qf[DS], dof[DS], of[DS];
  load_frags<D>(qf, Qr, qrow, g);
  load_frags<D>(dof, dOr, qrow, g);
  load_frags<D>(of, Or, qrow, g);
  const float lrow = buf_load_f32(Lr, qrow * 4);
  wait_vmem();
  float dsum = 0.f;
#pragma unroll
  for (int s = 0; s < DS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = fmaf((float)dof[s][e], (float)of[s][e], dsum);
  dsum += swap_halves(dsum);
  const float l2 = qrow < Nq ? lrow * kLog2e : INFINITY;
  if (neg)
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = negate(qf[s]);

  f32x16 dqt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqt[db] = zero16();

  int nkt = (Nk + MT - 1) / MT;
  if (CAUSAL) nkt = min(nkt, (min(q0 + 128, Nq) - 1) / MT + 1);

  auto fetch = [&](int kt, bf16* base) {
    MTile::template load<4>(Kr, kt * MT, base, w, lane);
    MTile::template load<4>(Vr, kt * MT, base + T, w, lane);
  };

  if (nkt > 0) fetch(0, smem);
  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const int n0 = kt * MT;
    const bool active = qw0 < Nq && (!CAUSAL || n0 <= qw0 + 31);
    // All LDS reads of this tile before the next tile's direct loads (see fwd_kernel).
    bf16x8 ka[NB][DS], va[NB][DS], ktf[2 * NB][DB];
    if (active) {
      const bf16* sK = smem + buf * C::BUF;
      const bf16* sV = sK + T;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          ka[kb][s] = MTile::frag(sK, 32 * kb + l32, 2 * s + g);
          va[kb][s] = MTile::frag(sV, 32 * kb + l32, 2 * s + g);
        }
#pragma unroll
      for (int s2 = 0; s2 < 2 * NB; ++s2)
#pragma unroll
        for (int db = 0; db < DB; ++db) ktf[s2][db] = MTile::tfrag(sK, 32 * db, 16 * s2, lane);
    }
    if (kt + 1 < nkt) fetch(kt + 1, smem + (buf ^ 1) * C::BUF);
    if (active) {
      f32x16 st[NB], dpt[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        st[kb] = zero16();
        dpt[kb] = zero16();
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          st[kb] = mfma32(ka[kb][s], qf[s], st[kb]);
          dpt[kb] = mfma32(va[kb][s], dof[s], dpt[kb]);
        }
      }
      // Registers: key n0 + 32kb + 8(r/4) + 4g + r%4 against this lane's query.
      if ((CAUSAL && n0 + MT - 1 > qw0) || n0 + MT > Nk)
        dq_scores<true, NB>(st, dpt, c, l2, dsum, CAUSAL ? qrow - n0 - 4 * g : 1 << 30,
                            Nk - n0 - 4 * g);
      else
        dq_scores<false, NB>(st, dpt, c, l2, dsum, 0, 0);
#pragma unroll
      for (int s2 = 0; s2 < 2 * NB; ++s2) {
        const bf16x8 sf = to_bf16x8(dpt[s2 >> 1], 8 * (s2 & 1));
#pragma unroll
        for (int db = 0; db < DB; ++db) dqt[db] = mfma32(ktf[s2][db], sf, dqt[db]);
      }
    }
    wait_vmem();
    __syncthreads();
  }

  if (qrow < Nq) store_rows_from_acc<D>(dQh + (size_t)qrow * D, dqt, scale, g);
}

// One launch for the whole backward. Per head the workgroups run the dK/dV key tiles first
// and then the dQ query tiles, each kind longest first: the dK/dV tiles that finish first
// (few visible queries) free their CUs for the longest dQ tiles.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_kernel(const bf16* __restrict__ Q,
                                                  const bf16* __restrict__ K,
                                                  const bf16* __restrict__ V,
                                                  const bf16* __restrict__ O,
                                                  const float* __restrict__ L,
                                                  const bf16* __restrict__ dO,
                                                  bf16* __restrict__ dQ, bf16* __restrict__ dK,
                                                  bf16* __restrict__ dV, int Nq, int Nk,
                                                  float scale, int neg) {
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * BwdCfg<D>::BUF];
  const int nkv = (Nk + 127) / 128, nqw = (Nq + 127) / 128;
  const int per_head = nkv + nqw;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / per_head, idx = lid % per_head;
  const size_t oq = (size_t)bh * Nq * D, ok = (size_t)bh * Nk * D;
  const uint32_t bq = (uint32_t)Nq * D * 2, bk = (uint32_t)Nk * D * 2;
  const rsrc_t Qr = make_rsrc(Q + oq, bq), Or = make_rsrc(O + oq, bq);
  const rsrc_t dOr = make_rsrc(dO + oq, bq);
  const rsrc_t Kr = make_rsrc(K + ok, bk), Vr = make_rsrc(V + ok, bk);
  const rsrc_t Lr = make_rsrc(L + (size_t)bh * Nq, (uint32_t)Nq * 4);
  if (idx < nkv) {
    dkdv_part<D, CAUSAL>(smem, Qr, Kr, Vr, Or, Lr, dOr, dK + ok, dV + ok, idx * 128, Nq, Nk,
                         scale, neg);
  } else {
    const int it = CAUSAL ? nqw - 1 - (idx - nkv) : idx - nkv;
    dq_part<D, CAUSAL>(smem, Qr, Kr, Vr, Or, Lr, dOr, dQ + oq, it * 128, Nq, Nk, scale, neg);
  }
}

template <int D, bool CAUSAL>
hipError_t fwd_t(const Shape& s, const void* Q, const void* K, const void* V, void* O, float* L,
                 hipStream_t stream) {
  // Pairing pays off only when one 128-query tile per workgroup leaves CUs idle or runs a
  // single wave per SIMD anyway; larger grids keep the plain kernel (shared K/V stream, two
  // waves per SIMD).
  if constexpr (CAUSAL && D >= 32) {
    if (s.Nq == s.Nk && s.Nq % 128 == 0 && (long long)(s.Nq / 128) * s.BH <= kNumCUs) {
      const long long grid = (long long)(s.Nq / 128) * s.BH;
      hipLaunchKernelGGL((fwd_causal_paired_kernel<D>), dim3((unsigned)grid), dim3(256), 0,
                         stream, (const bf16*)Q, (const bf16*)K, (const bf16*)V, (bf16*)O, L,
                         s.Nq, s.scale, s.scale < 0.f ? 1 : 0);
      return hipGetLastError();
    }
  }
  const int nqt = (s.Nq + 127) / 128;
  const long long grid = (long long)nqt * s.BH;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const bf16*)Q, (const bf16*)K, (const bf16*)V, (bf16*)O, L, s.Nq, s.Nk,
                     s.scale, s.scale < 0.f ? 1 : 0);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t bwd_t(const Shape& s, const void* Q, const void* K, const void* V, const void* O,
                 const float* L, const void* dO, void* dQ, void* dK, void* dV,
                 hipStream_t stream) {
  const long long grid = (long long)((s.Nk + 127) / 128 + (s.Nq + 127) / 128) * s.BH;
  hipLaunchKernelGGL((bwd_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const bf16*)Q, (const bf16*)K, (const bf16*)V, (const bf16*)O, L,
                     (const bf16*)dO, (bf16*)dQ, (bf16*)dK, (bf16*)dV, s.Nq, s.Nk, s.scale,
                     s.scale < 0.f ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const Shape& s, const void* Q, const void* K, const void* V, void* O,
                           float* L, hipStream_t stream) {
#define FA_FWD(DD)                                                              \
  case DD:                                                                      \
    return s.causal ? fwd_t<DD, true>(s, Q, K, V, O, L, stream)                 \
                    : fwd_t<DD, false>(s, Q, K, V, O, L, stream);
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

hipError_t launch_bwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* O, const float* L, const void* dO, void* dQ, void* dK,
                           void* dV, hipStream_t stream) {
#define FA_BWD(DD)                                                                   \
  case DD:                                                                           \
    return s.causal ? bwd_t<DD, true>(s, Q, K, V, O, L, dO, dQ, dK, dV, stream)      \
                    : bwd_t<DD, false>(s, Q, K, V, O, L, dO, dQ, dK, dV, stream);
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

}  // namespace fa
