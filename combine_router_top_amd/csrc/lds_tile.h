// LDS-staged MFMA tiles shared by the expert GEMMs and the router: up to
// XT_BM rows of A against a 256-column block of a row-major [K][N] bf16
// matrix B, both operands through LDS.
//
// Each thread loads one 8 x 4 block of the 64-K stage of B (32 or 64 lanes side
// by side along a row of B, so every load instruction reads 256- or 512-byte
// runs of a row; 4-byte loads of 64-byte runs cap a compute unit near 28 GB/s
// on this part) and its share of the A rows, both with buffer loads, in a
// 3-slot register ring (two stages in flight).  At the end of a stage the
// next stage's A rows and transposed B block are written to the other LDS
// buffer.  The 8 waves form 2 row halves x 4 column slabs: wave (wm, wn)
// multiplies rows 16 MT wm .. + 16 MT - 1 by B^T rows 64 wn .. 64 wn + 63, so
// each wave reads only its half of the A tile from LDS.
#pragma once

#include "common.h"
#include "gemm_core.h"

namespace moe {

constexpr int XT_BM = 192;   // rows of A per tile at most (MT <= 6 per row half)
constexpr int XT_BN = 256;   // B columns per tile
constexpr int XT_NB = 3;     // register ring depth
constexpr int XT_LDS = 2 * (XT_BM + XT_BN) * GC_LDA;  // bf16: double-buffered A and B^T stages

// LDS row (within the 256-row B^T tile) of weight column c (0..3) of 4-column
// group nb.  GEMM-1: nb 0..31 are W1 columns 4 nb .., nb 32..63 the same W3
// columns; wave slab wn holds h columns 32 wn .. 32 wn + 31, lane i (< 8) of
// n-tile t the h column 32 wn + 4 i + t, lane i + 8 its W3 twin.  GEMM-2: wave
// slab wn holds weight columns 64 wn .. 64 wn + 63, lane i of n-tile t column
// 64 wn + 4 i + t.
template <bool SWIGLU>
__device__ __forceinline__ int tile_brow(int nb, int c) {
  if (SWIGLU) {
    const int m3 = nb >> 5;
    const int hc = 4 * (nb & 31) + c;   // 0..127
    const int wn = hc >> 5, hw = hc & 31;
    return 64 * wn + 16 * (hw & 3) + 8 * m3 + (hw >> 2);
  } else {
    const int wc = 4 * nb + c;          // 0..255
    const int wn = wc >> 6, cw = wc & 63;
    return 64 * wn + 16 * (cw & 3) + (cw >> 2);
  }
}


template <int MT>
struct MidPipe {
  static constexpr int AV = (MT + 1) / 2;   // 32 MT rows, 64 rows per 16-byte vector round
  struct Slot {
    u32x4 a[AV];
    u32x2 b[8];
  } s[XT_NB];
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t va[AV];
  uint32_t vb, ldb2;
  int kb, nb;
  int kbeg;   // first K of the loop
};

template <int J, int MT>
__device__ __forceinline__ void mid_issue(MidPipe<MT>& P, int k0) {
#pragma unroll
  for (int j = 0; j < MidPipe<MT>::AV; ++j)
    P.s[J].a[j] = __builtin_amdgcn_raw_buffer_load_b128(P.ra, P.va[j], (uint32_t)(k0 * 2), 0);
#pragma unroll
  for (int r = 0; r < 8; ++r)
    P.s[J].b[r] = __builtin_amdgcn_raw_buffer_load_b64(P.rb, P.vb, (uint32_t)(k0 + r) * P.ldb2, 0);
}

template <int J, bool SWIGLU, int MT>
__device__ __forceinline__ void mid_store(const MidPipe<MT>& P, bf16_t* As, bf16_t* Bs) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < MidPipe<MT>::AV; ++j)
    *reinterpret_cast<u32x4*>(As + ((t >> 3) + 64 * j) * GC_LDA + 8 * (t & 7)) = P.s[J].a[j];
#pragma unroll
  for (int col = 0; col < 4; ++col) {
    const uint32_t sel = (col & 1) ? 0x07060302u : 0x05040100u;
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = __builtin_amdgcn_perm(P.s[J].b[2 * q + 1][col >> 1], P.s[J].b[2 * q][col >> 1], sel);
    *reinterpret_cast<u32x4*>(Bs + tile_brow<SWIGLU>(P.nb, col) * GC_LDA + 8 * P.kb) = v;
  }
}

template <int MT>
__device__ __forceinline__ void mid_compute(const bf16_t* As, const bf16_t* Bs, int wm, int wn,
                                            f32x4 (&acc)[MT][4]) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const bf16_t* a0 = As + (16 * MT * wm + i) * GC_LDA + 8 * g;
  const bf16_t* b0 = Bs + (64 * wn + i) * GC_LDA + 8 * g;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    bf16x8 bf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      bf[t] = *reinterpret_cast<const bf16x8*>(b0 + 16 * t * GC_LDA + 32 * sub);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(a0 + 16 * mt * GC_LDA + 32 * sub);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = mfma16(af, bf[t], acc[mt][t]);
    }
  }
}

// Stage st in ring slot J = st % XT_NB: refill the slot of stage st - 1 with
// stage st + 2, multiply stage st, write stage st + 1 into the other LDS
// buffer, barrier.  GUARD as in gemm_core.h.
template <int J, bool GUARD, bool SWIGLU, int MT>
__device__ __forceinline__ void mid_step(MidPipe<MT>& P, int st, int nst, bf16_t* As, bf16_t* Bs,
                                         f32x4 (&acc)[MT][4], int wm, int wn) {
  if (GUARD && st >= nst) return;
  if (!GUARD || st + XT_NB - 1 < nst) mid_issue<(J + XT_NB - 1) % XT_NB>(P, P.kbeg + (st + XT_NB - 1) * GC_KS);
  __builtin_amdgcn_sched_barrier(0);
  mid_compute<MT>(As + (st & 1) * XT_BM * GC_LDA, Bs + (st & 1) * XT_BN * GC_LDA, wm, wn, acc);
  if (!GUARD || st + 1 < nst)
    mid_store<(J + 1) % XT_NB, SWIGLU>(P, As + ((st + 1) & 1) * XT_BM * GC_LDA,
                                       Bs + ((st + 1) & 1) * XT_BN * GC_LDA);
  __syncthreads();
}

template <int J, bool GUARD, bool SWIGLU, int MT>
__device__ __forceinline__ void mid_trip(MidPipe<MT>& P, int st, int nst, bf16_t* As, bf16_t* Bs,
                                         f32x4 (&acc)[MT][4], int wm, int wn) {
  mid_step<J, GUARD, SWIGLU>(P, st + J, nst, As, Bs, acc, wm, wn);
  if constexpr (J + 1 < XT_NB) mid_trip<J + 1, GUARD, SWIGLU>(P, st, nst, As, Bs, acc, wm, wn);
}


template <int J, int MT>
__device__ __forceinline__ void mid_prologue(MidPipe<MT>& P, int kbeg, int nst) {
  if constexpr (J < XT_NB - 1) {
    if (J < nst) mid_issue<J>(P, kbeg + J * GC_KS);
    mid_prologue<J + 1>(P, kbeg, nst);
  }
}

// The K loop over [kbeg, kend) (kbeg a multiple of 8; rows of B past the B
// descriptor read zero).  P holds the descriptors and lane offsets; As/Bs
// point at XT_BM / XT_BN double buffers of GC_LDA-strided rows.
template <bool SWIGLU, int MT>
__device__ __forceinline__ void mid_mainloop(MidPipe<MT>& P, int kbeg, int kend, bf16_t* As,
                                             bf16_t* Bs, f32x4 (&acc)[MT][4], int wm, int wn) {
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = (kend - kbeg + GC_KS - 1) / GC_KS;
  if (nst <= 0) return;
  P.kbeg = kbeg;
  mid_prologue<0>(P, kbeg, nst);  // stages 0 .. XT_NB - 2 into slots 0 .. XT_NB - 2
  mid_store<0, SWIGLU>(P, As, Bs);
  __syncthreads();
  int st = 0;
  for (; st + 2 * XT_NB - 1 <= nst; st += XT_NB)
    mid_trip<0, false, SWIGLU>(P, st, nst, As, Bs, acc, wm, wn);
  mid_trip<0, true, SWIGLU>(P, st, nst, As, Bs, acc, wm, wn);
  mid_trip<0, true, SWIGLU>(P, st + XT_NB, nst, As, Bs, acc, wm, wn);
}

}  // namespace moe
