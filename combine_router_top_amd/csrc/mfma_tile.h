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
// each lane loads 8 consecutive rows x 4 consecutive columns (8 bytes per row)
// and transposes the 8x4 block in registers with byte permutes.  Lane i of
// group g then owns columns n0 + 4i + c (c = 0..3) for k rows 8g..8g+7, which
// makes n-tile c the strided column set {n0 + 4i + c : i = 0..15}.  In the
// output each lane therefore holds 4 consecutive columns of each of its rows,
// so the epilogue stores 4 elements at once.
#pragma once

#include "common.h"

namespace moe {

struct BRaw {
  u32x2 row[8];  // row r: columns c0..c3 of k-row 8g + r (bf16 pairs)
};

// Load the 8x4 block at (k-row kb + 8g .. +7, column nc .. nc+3) of a row-major
// [K][ldb] bf16 matrix; rows >= K or a column group past N read as zeros.
__device__ __forceinline__ void load_b_block(BRaw& br, const bf16_t* __restrict__ B, int64_t ldb,
                                             int kb, int K, int nc, int N) {
  const int g = __lane_id() >> 4;
  const int k0 = kb + 8 * g;
  const bool colok = nc < N;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int k = k0 + r;
    if (colok && k < K) {
      br.row[r] = *reinterpret_cast<const u32x2*>(B + (int64_t)k * ldb + nc);
    } else {
      br.row[r] = u32x2{0u, 0u};
    }
  }
}

// Same, without bounds checks (caller guarantees the block is in range).
__device__ __forceinline__ void load_b_block_nocheck(BRaw& br, const bf16_t* __restrict__ B,
                                                     int64_t ldb, int kb, int nc) {
  const int g = __lane_id() >> 4;
  const bf16_t* p = B + (int64_t)(kb + 8 * g) * ldb + nc;
#pragma unroll
  for (int r = 0; r < 8; ++r) br.row[r] = *reinterpret_cast<const u32x2*>(p + (int64_t)r * ldb);
}

// Transpose the 8x4 block into 4 B fragments (one per n-tile c).
__device__ __forceinline__ void transpose_b(const BRaw& br, bf16x8 frag[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    u32x4 t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = br.row[2 * q][c >> 1];
      const uint32_t hi = br.row[2 * q + 1][c >> 1];
      t[q] = __builtin_amdgcn_perm(hi, lo, sel);
    }
    frag[c] = __builtin_bit_cast(bf16x8, t);
  }
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace moe
