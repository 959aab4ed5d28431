// Shared device helpers for the gfx950 attention kernels: vector types, the bf16 MFMA,
// swizzled LDS tile addressing and direct-to-LDS tile loads, score masking, cross-lane
// reductions and the workgroup-to-XCD remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Buffer resource over `bytes` bytes at `base` (gfx9 raw buffer: stride 0, dword3 0x00020000).
// Loads whose bytes fall past `bytes` return zeros, which is how ragged tiles are padded:
// no branch, no select.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// v_dot2c_f32_bf16: acc + a.x * b.x + a.y * b.y for two bf16 pairs packed in 32 bits.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Wait until every outstanding vector-memory load of this wave has returned.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most K vector-memory instructions of this wave are outstanding (vmcnt(K)):
// they return in issue order, so this waits for everything but the K most recent. The 6-bit
// count is split in the encoding: bits 3:0 and 15:14.
template <int K>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(K >= 0 && K < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (K & 15) | ((K >> 4) << 14));
}

// Workgroup barrier that publishes this wave's LDS writes and completes its LDS reads
// (lgkmcnt(0)) but leaves its outstanding vector-memory loads, including loads into LDS, in
// flight; __syncthreads() would wait for those too. The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16) on the matrix cores.
// Fragment layout with g = lane / 32:
//   A: lane holds row (lane % 32), k = 8g .. 8g+7;  B: lane holds column (lane % 32), same k;
//   C: register r holds row 8*(r/4) + 4g + (r%4), column (lane % 32).
// The k order inside a fragment only has to agree between A and B, which it does for any
// tile this file reads with the same chunk index.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Eight consecutive fp32 accumulator registers -> one bf16 MFMA operand (RNE).
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)x[base + e];
  return r;
}

// XOR key of row r for an LDS tile with NCH 16-byte chunks per row. With 8 chunks (64
// columns) the key is 2(r%4) ^ ((r/4)%2) ^ 2((r/8)%2). The first two terms give four
// consecutive rows that read a pair of adjacent chunks (a transposed fragment,
// ds_read_b64_tr_b16) four disjoint chunk pairs; the last term separates rows r and r+8,
// which a 16-byte row-fragment read (ds_read_b128) otherwise puts on the same banks. With 16
// chunks (128 columns) the key also moves odd rows to the other half of the row: 8(r%2).
// Both were chosen by measurement on gfx950 (SQ_LDS_BANK_CONFLICT, both access patterns as
// the kernels issue them): no conflicts, where the obvious keys leave one pattern at 50%.
// Narrower tiles use (r ^ r/8) % NCH.
template <int NCH>
__device__ __forceinline__ int swz_key(int r) {
  const int k8 = ((r & 3) << 1) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
  if constexpr (NCH >= 16)
    return k8 ^ ((r & 1) << 3);
  else if constexpr (NCH == 8)
    return k8;
  else
    return (r ^ (r >> 3)) & (NCH - 1);
}

// Element offset of 16-byte chunk c of row r in an LDS tile with NCH chunks per row and no
// padding; chunk c of row r is stored at position c ^ swz_key(r).
template <int NCH>
__device__ __forceinline__ int swz(int r, int c) {
  return r * (NCH * 8) + ((c ^ swz_key<NCH>(r)) << 3);
}

template <int NCH>
__device__ __forceinline__ bf16x8 lds_frag(const bf16* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + swz<NCH>(r, c));
}

// All-reduce (sum) across aligned groups of N lanes (N = 1, 2, 4, 8, 16 or 32).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                            0xB1, 0xF, 0xF, false));
  if constexpr (N >= 4)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                            0x4E, 0xF, 0xF, false));
  if constexpr (N >= 8)  // row_half_mirror: lane i <- lane 7-i inside each 8
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                            0x141, 0xF, 0xF, false));
  if constexpr (N >= 16)  // row_mirror: lane i <- lane 15-i inside each 16
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                            0x140, 0xF, 0xF, false));
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// v_permlane32_swap: {a, b} -> {a[0..31] ++ b[0..31], a[32..63] ++ b[32..63]} (lane ranges of
// the two registers). Written as inline asm because hipcc 7.2 folds the second result of
// __builtin_amdgcn_permlane32_swap into the first in reductions such as max(r0, r1), which
// gives wrong results. The s_nop supplies the two wait states the instruction needs after a
// VALU write of its operands (the compiler cannot see inside the asm to insert them).
__device__ __forceinline__ void permlane32_swap(uint32_t& a, uint32_t& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// An MFMA accumulator with all sixteen registers equal to x, as eight 64-bit moves of one
// (x, x) pair: the compiler builds the same splat from sixteen or more 32-bit moves. The moves
// sit in one asm block, which the compiler cannot see as VALU writes, so the block ends with
// the two wait states an MFMA needs before reading a VGPR that a VALU instruction wrote. The
// outputs are early-clobber, so none shares a register with the pair.
__device__ __forceinline__ f32x16 splat16(float x) {
  typedef double f64x8 __attribute__((ext_vector_type(8)));
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const double p = __builtin_bit_cast(double, u32x2{b, b});
  double r0, r1, r2, r3, r4, r5, r6, r7;
  asm("v_mov_b64 %0, %8\n\tv_mov_b64 %1, %8\n\tv_mov_b64 %2, %8\n\tv_mov_b64 %3, %8\n\t"
      "v_mov_b64 %4, %8\n\tv_mov_b64 %5, %8\n\tv_mov_b64 %6, %8\n\tv_mov_b64 %7, %8\n\t"
      "s_nop 1"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(p));
  return __builtin_bit_cast(f32x16, f64x8{r0, r1, r2, r3, r4, r5, r6, r7});
}

// x[l] + x[l ^ 32] and max(x[l], x[l ^ 32]) in every lane: after the swap a holds the lower
// half's value and b the upper half's in every lane, so no lane select is needed and both
// halves get the bitwise identical result.
__device__ __forceinline__ float halves_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane32_swap(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
// The IEEE 754-2019 maximum (one v_maximum3_f32): fmaxf would first canonicalise both
// values, which come out of inline asm. The two differ only for NaN operands and for the sign
// of a zero maximum, and neither changes a softmax computed from the result.
__device__ __forceinline__ float halves_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane32_swap(a, b);
  return __builtin_elementwise_maximum(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// Workgroups are dispatched round-robin over the eight XCDs (workgroup b runs on XCD b % 8).
// Give each XCD one contiguous range of logical tiles so that the tiles of a head, which
// re-read the same K/V (or Q/dO) rows, share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  if ((n & 7) != 0) return bid;
  return (bid & 7) * (n >> 3) + (bid >> 3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// scale * log2(e) for the exponentials, floored at 1e-30 so that masked scores, set to -inf,
// give exp2(-inf * c) = 0 even for scale = 0. With c = 1e-30 every visible exponent is below
// 2^-80 in magnitude, whose exp2 rounds to exactly 1 in fp32: the same P as c = 0.
__device__ __forceinline__ float exp2_coef(float scale) {
  return fmaxf(fabsf(scale) * kLog2e, 1e-30f);
}

// Set score registers whose offset 8(r/4) + r%4 (+32 per block) is not visible to -inf:
// visible iff lo <= offset <= hi.
template <int NBLK>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[NBLK], int lo, int hi) {
#pragma unroll
  for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
      if (off < lo || off > hi) s[kb][r] = -INFINITY;
    }
}

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
// dma16 and dma4 with the offset split into a per-lane part and a wave-uniform part, which goes
// in the instruction's scalar offset operand. For loads that lie inside the buffer: the zero
// fill of bytes past its end, which dma16 and dma4 give, is not relied on here.
__device__ __forceinline__ void dma16_at(rsrc_t src, uint32_t lane_off, uint32_t uniform_off,
                                         void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)dst, 16, lane_off, (int)uniform_off,
                                           0, 0);
}
__device__ __forceinline__ void dma4_at(rsrc_t src, uint32_t lane_off, uint32_t uniform_off,
                                        void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)dst, 4, lane_off, (int)uniform_off,
                                           0, 0);
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
#pragma unroll
    for (int i = 0; i < (NKIB + NW - 1) / NW; ++i) {
      const int blk = w + i * NW;
      if (NKIB % NW == 0 || blk < NKIB) {
        const int p = blk * 64 + lane;
        const int row = p / NCH, cp = p % NCH;
        const int gc = cp ^ swz_key<NCH>(row);
        dma16(src, (uint32_t)(((row0 + row) * C + gc * 8) * 2), t + blk * 512);
      }
    }
  }
  // load() for a tile that lies wholly inside the head (row0 + R <= its rows): the row offset
  // is wave-uniform (dma16_at), so each lane's offset is the same for every tile and no vector
  // instruction forms it again per tile.
  template <int NW>
  __device__ __forceinline__ static void load_in_range(rsrc_t src, int row0, bf16* t, int w,
                                                       int lane) {
#pragma unroll
    for (int i = 0; i < (NKIB + NW - 1) / NW; ++i) {
      const int blk = w + i * NW;
      if (NKIB % NW == 0 || blk < NKIB) {
        const int p = blk * 64 + lane;
        const int row = p / NCH, cp = p % NCH;
        const int gc = cp ^ swz_key<NCH>(row);
        dma16_at(src, (uint32_t)((row * C + gc * 8) * 2), (uint32_t)row0 * (C * 2),
                 t + blk * 512);
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

}  // namespace fa
