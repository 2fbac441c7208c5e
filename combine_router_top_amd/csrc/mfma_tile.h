// Building blocks for bf16 MFMA tiles on gfx950 (v_mfma_f32_16x16x32_bf16).
//
// Operand layout used throughout (lane l of a 64-lane wave, i = l % 16,
// g = l / 16):
//   A fragment: 8 bf16 of row i of the 16-row tile, k = 8g .. 8g+7
//   B fragment: 8 bf16 of column i of the 16-column tile, same k = 8g .. 8g+7
//   D (f32x4):  rows 4g .. 4g+3 of column i
// The summation over k is order-free, so any k assignment that is the same for
// A and B gives the same product; only the row/column mapping of D matters.
//
// Weights are stored row-major as [K][N] (N contiguous), so a B fragment's 8
// k-values of one column are N elements apart.  Instead of staging through LDS,
// each lane loads 8 consecutive rows x CPL consecutive columns (2*CPL bytes per
// row) and transposes the 8 x CPL block in registers with byte permutes.  Lane
// i of group g then owns columns n0 + CPL*i + c (c = 0..CPL-1) for k rows
// 8g..8g+7, which makes n-tile c the strided column set {n0 + CPL*i + c}.  In
// the output each lane therefore holds CPL consecutive columns of each of its
// rows, so the epilogue stores CPL elements at once.
#pragma once

#include "common.h"

namespace moe {

// 8 k-rows x CPL columns of bf16, one register word per row for CPL = 2, two
// for CPL = 4.
template <int CPL>
struct BBlk;
template <>
struct BBlk<2> {
  uint32_t row[8];
};
template <>
struct BBlk<4> {
  u32x2 row[8];
};

template <int CPL>
__device__ __forceinline__ uint32_t bblk_word(const BBlk<CPL>& b, int r, int w);
template <>
__device__ __forceinline__ uint32_t bblk_word<2>(const BBlk<2>& b, int r, int) { return b.row[r]; }
template <>
__device__ __forceinline__ uint32_t bblk_word<4>(const BBlk<4>& b, int r, int w) { return b.row[r][w]; }

// Load the block at (k-row kb + 8g .. +7, column nc .. nc+CPL-1) of a
// row-major [K][ldb] bf16 matrix; rows >= K or a column group past N read as
// zeros.
template <int CPL>
__device__ __forceinline__ void load_b_block(BBlk<CPL>& br, const bf16_t* __restrict__ B,
                                             int64_t ldb, int kb, int K, int nc, int N) {
  const int g = __lane_id() >> 4;
  const int k0 = kb + 8 * g;
  const bool colok = nc < N;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int k = k0 + r;
    if (CPL == 2) {
      uint32_t v = 0u;
      if (colok && k < K) v = *reinterpret_cast<const uint32_t*>(B + (int64_t)k * ldb + nc);
      reinterpret_cast<uint32_t*>(&br)[r] = v;
    } else {
      u32x2 v = u32x2{0u, 0u};
      if (colok && k < K) v = *reinterpret_cast<const u32x2*>(B + (int64_t)k * ldb + nc);
      reinterpret_cast<u32x2*>(&br)[r] = v;
    }
  }
}

// Same, without bounds checks (caller guarantees the block is in range).
template <int CPL>
__device__ __forceinline__ void load_b_block_nocheck(BBlk<CPL>& br, const bf16_t* __restrict__ B,
                                                     int64_t ldb, int kb, int nc) {
  const int g = __lane_id() >> 4;
  const bf16_t* p = B + (int64_t)(kb + 8 * g) * ldb + nc;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (CPL == 2)
      reinterpret_cast<uint32_t*>(&br)[r] = *reinterpret_cast<const uint32_t*>(p + (int64_t)r * ldb);
    else
      reinterpret_cast<u32x2*>(&br)[r] = *reinterpret_cast<const u32x2*>(p + (int64_t)r * ldb);
  }
}

// Transpose the 8 x CPL block into CPL B fragments (one per n-tile c).
template <int CPL>
__device__ __forceinline__ void transpose_b(const BBlk<CPL>& br, bf16x8 (&frag)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    u32x4 t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = bblk_word<CPL>(br, 2 * q, c >> 1);
      const uint32_t hi = bblk_word<CPL>(br, 2 * q + 1, c >> 1);
      t[q] = __builtin_amdgcn_perm(hi, lo, sel);
    }
    frag[c] = __builtin_bit_cast(bf16x8, t);
  }
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace moe
