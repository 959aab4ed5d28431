// bf16 attention forward and backward for gfx950 (CDNA4): 32x32x16 bf16 MFMA with fp32
// accumulation, K/V (forward), Q/dO (dK/dV pass) and K/V (dQ pass) tiles staged through
// LDS, online softmax in registers.
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
// (P V, P^T dO, dS^T Q, dS K) takes the score registers directly as its B operand; the LDS
// operand for it is stored transposed with the row permutation of tpos().
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

__device__ __forceinline__ bf16x8 negate(bf16x8 x) {
  u32x4 u = __builtin_bit_cast(u32x4, x);
  u ^= 0x80008000u;
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float lo_f(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float hi_f(uint32_t x) {
  return __builtin_bit_cast(float, x & 0xFFFF0000u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 8 rows (those of transposed chunk kc) x 4 columns of an [MT x D] bf16 tile.
template <int MT, int D>
struct TUnit {
  static constexpr int N = (MT / 8) * (D / 4);
  u32x2 r[8];

  __device__ __forceinline__ void load(rsrc_t head, int row0, int u) {
    const int d4 = u % (D / 4), kc = u / (D / 4);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      r[e] = buf_load8(head, ((row0 + chunk_row(kc, e)) * D + 4 * d4) * 2);
  }
  // Row-major copy: tile[MT][D].
  __device__ __forceinline__ void store_rows(bf16* tile, int u) const {
    const int d4 = u % (D / 4), kc = u / (D / 4);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<u32x2*>(tile + swz<D / 8>(chunk_row(kc, e), d4 >> 1) + 4 * (d4 & 1)) =
          r[e];
  }
  // Transposed copy: tile[d][tpos(row)], MT columns per row.
  __device__ __forceinline__ void store_trans(bf16* tile, int u) const {
    const int d4 = u % (D / 4), kc = u / (D / 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = (i & 2) ? r[2 * j].y : r[2 * j].x;
        const uint32_t b = (i & 2) ? r[2 * j + 1].y : r[2 * j + 1].x;
        v[j] = (i & 1) ? pack_hi(a, b) : pack_lo(a, b);
      }
      *reinterpret_cast<u32x4*>(tile + swz<MT / 8>(4 * d4 + i, kc)) = v;
    }
  }
};

// Row-major [MT x D] tile moved as 16-byte chunks by NT threads.
template <int MT, int D, int NT>
struct RChunks {
  static constexpr int NC = MT * D / 8;
  static constexpr int PER = (NC + NT - 1) / NT;
  u32x4 r[PER];

  __device__ __forceinline__ void load(rsrc_t head, int row0, int t) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = t + p * NT;
      if (NC % NT == 0 || c < NC)
        r[p] = buf_load16(head, ((row0 + c / (D / 8)) * D + 8 * (c % (D / 8))) * 2);
    }
  }
  __device__ __forceinline__ void store(bf16* tile, int t) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = t + p * NT;
      if (c < NC) *reinterpret_cast<u32x4*>(tile + swz<D / 8>(c / (D / 8), c % (D / 8))) = r[p];
    }
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
__device__ __forceinline__ void store_rows_from_acc(bf16* out_row, const f32x16 (&acc)[(D + 31) / 32],
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
  constexpr int DS = D / 16, DB = (D + 31) / 32, DP = 32 * DB;
  constexpr int KT = BK * D, VT = DP * BK, BUF = KT + VT;
  constexpr int NVU = TUnit<BK, D>::N;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * BUF];

  const int nqt = (Nq + BQ - 1) / BQ;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nqt;
  const int qt = CAUSAL ? nqt - 1 - lid % nqt : lid % nqt;  // longest rows first
  const int q0 = qt * BQ;
  const rsrc_t Qr = make_rsrc(Q + (size_t)bh * Nq * D, (uint32_t)Nq * D * 2);
  const rsrc_t Kr = make_rsrc(K + (size_t)bh * Nk * D, (uint32_t)Nk * D * 2);
  const rsrc_t Vr = make_rsrc(V + (size_t)bh * Nk * D, (uint32_t)Nk * D * 2);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + l32;
  const float cs = fabsf(scale);
  const float c = cs * kLog2e;

  int nkt = (Nk + BK - 1) / BK;
  if (CAUSAL) nkt = min(nkt, (min(q0 + BQ, Nq) - 1) / BK + 1);

  bf16x8 qf[DS];
  load_frags<D>(qf, Qr, qrow, g);
  wait_vmem();  // keeps the loop's own prefetch waits exact
  if (neg)
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = negate(qf[s]);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  float m = 0.f, l = 0.f;

  RChunks<BK, D, 256> kreg;
  TUnit<BK, D> vreg;
  kreg.load(Kr, 0, tid);
  if (tid < NVU) vreg.load(Vr, 0, tid);
  kreg.store(smem, tid);
  if (tid < NVU) vreg.store_trans(smem + KT, tid);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) {
      kreg.load(Kr, (kt + 1) * BK, tid);
      if (tid < NVU) vreg.load(Vr, (kt + 1) * BK, tid);
    }
    const int k0 = kt * BK;
    const bool active = qw0 < Nq && (!CAUSAL || k0 <= qw0 + 31);
    if (active) {
      const bf16* sK = smem + buf * BUF;
      const bf16* sV = sK + KT;
      // All K fragments of the tile first, so the LDS latency is paid once.
      bf16x8 kfr[2][DS];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < DS; ++s) kfr[kb][s] = lds_frag<D / 8>(sK, 32 * kb + l32, 2 * s + g);
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int s = 0; s < DS; ++s) sacc[kb] = mfma32(kfr[kb][s], qf[s], sacc[kb]);
      }
      bf16x8 vfr[4][DB];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) vfr[u][db] = lds_frag<BK / 8>(sV, 32 * db + l32, 2 * u + g);
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
    if (more) {
      bf16* nbuf = smem + (buf ^ 1) * BUF;
      kreg.store(nbuf, tid);
      if (tid < NVU) vreg.store_trans(nbuf + KT, tid);
    }
    __syncthreads();
  }

  const float lt = l + swap_halves(l);
  if (qrow < Nq) {
    store_rows_from_acc<D>(O + ((size_t)bh * Nq + qrow) * D, o, 1.f / lt, g);
    if (g == 0) Lout[(size_t)bh * Nq + qrow] = m * cs + logf(lt);
  }
}

// ----------------------------------------------------------------------------- backward

// dK/dV pass: P = exp2(S c - L log2e) and dS = P (dP - D) in place, for score registers laid
// out with lane = key and register r of block qb = query offset 32qb + 8(r/4) + 4g + r%4.
// Masked (query < key) entries get P = dS = 0.
template <bool MASKED, int NB>
__device__ __forceinline__ void dkdv_scores(f32x16 (&sp)[NB], f32x16 (&dp)[NB],
                                            const float* sL2, const float* sD, float c, int g,
                                            int lim) {
#pragma unroll
  for (int qb = 0; qb < NB; ++qb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(sL2 + 32 * qb + 8 * j + 4 * g);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(sD + 32 * qb + 8 * j + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * j + i;
        float p = fast_exp2(fmaf(sp[qb][r], c, -l4[i]));
        if (MASKED && 32 * qb + 8 * j + i < lim) p = 0.f;
        sp[qb][r] = p;
        dp[qb][r] = p * (dp[qb][r] - d4[i]);
      }
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
  static constexpr int MT = D >= 128 ? 32 : 64;  // moving-tile rows
  static constexpr int NB = MT / 32;
  static constexpr int DS = D / 16, DB = (D + 31) / 32, DP = 32 * DB;
  static constexpr int T_RM = MT * D;   // row-major tile, elements
  static constexpr int T_TR = DP * MT;  // transposed tile, elements
  // dK/dV staging: Q, dO (row-major), Q^T, dO^T, then L*log2e and D as MT floats each.
  static constexpr int BUF_KV = 2 * T_RM + 2 * T_TR + 4 * MT;
  // dQ staging: K, V (row-major), K^T.
  static constexpr int BUF_Q = 2 * T_RM + T_TR;
  static constexpr int BUF = BUF_KV > BUF_Q ? BUF_KV : BUF_Q;
  static constexpr int NU = TUnit<MT, D>::N;  // <= 128
};

// dK, dV for the 128 keys starting at k0 of one head.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_part(bf16* smem, rsrc_t Qr, rsrc_t Kr, rsrc_t Vr, rsrc_t Or,
                                          rsrc_t Lr, rsrc_t dOr, bf16* dKh, bf16* dVh, int k0,
                                          int Nq, int Nk, float scale, int neg) {
  using C = BwdCfg<D>;
  constexpr int MT = C::MT, NB = C::NB, DS = C::DS, DB = C::DB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int kw0 = k0 + 32 * w;
  const int krow = kw0 + l32;
  const float c = fabsf(scale) * kLog2e;

  bf16x8 kf[DS], vf[DS];
  load_frags<D>(kf, Kr, krow, g);
  load_frags<D>(vf, Vr, krow, g);
  wait_vmem();
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

  // Staging roles: threads [0, NU) move Q; threads [128, 128 + NU) move dO and O (for D);
  // threads [0, MT) also fetch L.
  const bool q_role = tid < C::NU;
  const bool do_role = tid >= 128 && tid - 128 < C::NU;
  const int u = do_role ? tid - 128 : tid;
  TUnit<MT, D> qreg, doreg, oreg;
  float lreg = 0.f;

  auto fetch = [&](int mt) {
    const int m0 = mt * MT;
    if (q_role) qreg.load(Qr, m0, u);
    if (do_role) {
      doreg.load(dOr, m0, u);
      oreg.load(Or, m0, u);
    }
    if (tid < MT) lreg = buf_load_f32(Lr, (m0 + tid) * 4);
  };
  auto stage = [&](int mt, bf16* base) {
    const int m0 = mt * MT;
    bf16* sQ = base;
    bf16* sdO = base + C::T_RM;
    bf16* sQt = base + 2 * C::T_RM;
    bf16* sdOt = sQt + C::T_TR;
    float* sL2 = reinterpret_cast<float*>(sdOt + C::T_TR);
    float* sD = sL2 + MT;
    if (q_role) {
      qreg.store_rows(sQ, u);
      qreg.store_trans(sQt, u);
    }
    if (do_role) {
      doreg.store_rows(sdO, u);
      doreg.store_trans(sdOt, u);
      const int d4 = u % (D / 4), kc = u / (D / 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const u32x2 a = doreg.r[e], b = oreg.r[e];
        float pd = lo_f(a.x) * lo_f(b.x);
        pd = fmaf(hi_f(a.x), hi_f(b.x), pd);
        pd = fmaf(lo_f(a.y), lo_f(b.y), pd);
        pd = fmaf(hi_f(a.y), hi_f(b.y), pd);
        pd = group_sum<D / 4>(pd);
        if (d4 == 0) sD[chunk_row(kc, e)] = pd;
      }
    }
    if (tid < MT) sL2[tid] = m0 + tid < Nq ? lreg * kLog2e : INFINITY;
  };

  if (mt0 < nmt) {
    fetch(mt0);
    stage(mt0, smem);
  }
  __syncthreads();
  for (int mt = mt0; mt < nmt; ++mt) {
    const int buf = (mt - mt0) & 1;
    const bool more = mt + 1 < nmt;
    if (more) fetch(mt + 1);
    const int m0 = mt * MT;
    const bool active = kw0 < Nk && (!CAUSAL || m0 + MT - 1 >= kw0);
    if (active) {
      const bf16* base = smem + buf * C::BUF;
      const bf16* sQ = base;
      const bf16* sdO = base + C::T_RM;
      const bf16* sQt = base + 2 * C::T_RM;
      const bf16* sdOt = sQt + C::T_TR;
      const float* sL2 = reinterpret_cast<const float*>(sdOt + C::T_TR);
      const float* sD = sL2 + MT;
      f32x16 sp[NB], dp[NB];
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) {
        bf16x8 qa[DS], da[DS];
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          qa[s] = lds_frag<D / 8>(sQ, 32 * qb + l32, 2 * s + g);
          da[s] = lds_frag<D / 8>(sdO, 32 * qb + l32, 2 * s + g);
        }
        sp[qb] = zero16();
        dp[qb] = zero16();
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          sp[qb] = mfma32(qa[s], kf[s], sp[qb]);
          dp[qb] = mfma32(da[s], vf[s], dp[qb]);
        }
      }
      // Registers: query m0 + 32qb + 8(r/4) + 4g + r%4 against this lane's key; the key is
      // visible iff query >= key, i.e. offset 32qb + 8(r/4) + r%4 >= krow - m0 - 4g.
      if (CAUSAL && m0 < kw0 + 31)
        dkdv_scores<true, NB>(sp, dp, sL2, sD, c, g, krow - m0 - 4 * g);
      else
        dkdv_scores<false, NB>(sp, dp, sL2, sD, c, g, 0);
#pragma unroll
      for (int st = 0; st < 2 * NB; ++st) {
        bf16x8 ofr[DB], qfr[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          ofr[db] = lds_frag<MT / 8>(sdOt, 32 * db + l32, 2 * st + g);
          qfr[db] = lds_frag<MT / 8>(sQt, 32 * db + l32, 2 * st + g);
        }
        const bf16x8 pf = to_bf16x8(sp[st >> 1], 8 * (st & 1));
        const bf16x8 sf = to_bf16x8(dp[st >> 1], 8 * (st & 1));
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dvt[db] = mfma32(ofr[db], pf, dvt[db]);
          dkt[db] = mfma32(qfr[db], sf, dkt[db]);
        }
      }
    }
    if (more) stage(mt + 1, smem + (buf ^ 1) * C::BUF);
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
  constexpr int MT = C::MT, NB = C::NB, DS = C::DS, DB = C::DB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
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

  const bool k_role = tid < C::NU;
  const bool v_role = tid >= 128;
  TUnit<MT, D> kreg;
  RChunks<MT, D, 128> vreg;

  auto fetch = [&](int kt) {
    if (k_role) kreg.load(Kr, kt * MT, tid);
    if (v_role) vreg.load(Vr, kt * MT, tid - 128);
  };
  auto stage = [&](bf16* base) {
    if (k_role) {
      kreg.store_rows(base, tid);
      kreg.store_trans(base + 2 * C::T_RM, tid);
    }
    if (v_role) vreg.store(base + C::T_RM, tid - 128);
  };

  if (nkt > 0) {
    fetch(0);
    stage(smem);
  }
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) fetch(kt + 1);
    const int n0 = kt * MT;
    const bool active = qw0 < Nq && (!CAUSAL || n0 <= qw0 + 31);
    if (active) {
      const bf16* sK = smem + buf * C::BUF;
      const bf16* sV = sK + C::T_RM;
      const bf16* sKt = sK + 2 * C::T_RM;
      f32x16 st[NB], dpt[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        bf16x8 ka[DS], va[DS];
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          ka[s] = lds_frag<D / 8>(sK, 32 * kb + l32, 2 * s + g);
          va[s] = lds_frag<D / 8>(sV, 32 * kb + l32, 2 * s + g);
        }
        st[kb] = zero16();
        dpt[kb] = zero16();
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          st[kb] = mfma32(ka[s], qf[s], st[kb]);
          dpt[kb] = mfma32(va[s], dof[s], dpt[kb]);
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
        bf16x8 kt_[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) kt_[db] = lds_frag<MT / 8>(sKt, 32 * db + l32, 2 * s2 + g);
        const bf16x8 sf = to_bf16x8(dpt[s2 >> 1], 8 * (s2 & 1));
#pragma unroll
        for (int db = 0; db < DB; ++db) dqt[db] = mfma32(kt_[db], sf, dqt[db]);
      }
    }
    if (more) stage(smem + (buf ^ 1) * C::BUF);
    __syncthreads();
  }

  if (qrow < Nq) store_rows_from_acc<D>(dQh + (size_t)qrow * D, dqt, scale, g);
}

// One launch for the whole backward: per head, workgroups alternate between a dK/dV key
// tile (fewest-visible-queries last) and a dQ query tile (most-visible-keys first).
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
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * BwdCfg<D>::BUF];
  const int nkv = (Nk + 127) / 128, nqw = (Nq + 127) / 128;
  const int per_head = nkv + nqw;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / per_head, idx = lid % per_head;
  const int mn = min(nkv, nqw);
  bool kv;
  int r;
  if (idx < 2 * mn) {
    kv = (idx & 1) == 0;
    r = idx >> 1;
  } else {
    kv = nkv > nqw;
    r = mn + (idx - 2 * mn);
  }
  const size_t oq = (size_t)bh * Nq * D, ok = (size_t)bh * Nk * D;
  const uint32_t bq = (uint32_t)Nq * D * 2, bk = (uint32_t)Nk * D * 2;
  const rsrc_t Qr = make_rsrc(Q + oq, bq), Or = make_rsrc(O + oq, bq), dOr = make_rsrc(dO + oq, bq);
  const rsrc_t Kr = make_rsrc(K + ok, bk), Vr = make_rsrc(V + ok, bk);
  const rsrc_t Lr = make_rsrc(L + (size_t)bh * Nq, (uint32_t)Nq * 4);
  if (kv) {
    dkdv_part<D, CAUSAL>(smem, Qr, Kr, Vr, Or, Lr, dOr, dK + ok, dV + ok, r * 128, Nq, Nk, scale,
                         neg);
  } else {
    const int it = CAUSAL ? nqw - 1 - r : r;
    dq_part<D, CAUSAL>(smem, Qr, Kr, Vr, Or, Lr, dOr, dQ + oq, it * 128, Nq, Nk, scale, neg);
  }
}

template <int D, bool CAUSAL>
hipError_t fwd_t(const Shape& s, const void* Q, const void* K, const void* V, void* O, float* L,
                 hipStream_t stream) {
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
