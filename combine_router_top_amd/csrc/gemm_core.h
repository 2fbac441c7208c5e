// Pipelined bf16 MFMA main loop shared by the router and the expert GEMMs.
//
// A workgroup of NW waves computes C[rows, cols] += A[rows, K] * B[K, cols]
// for up to 16*MT rows.  A (row-major, K contiguous) is staged through a
// double-buffered LDS tile shared by the waves; each wave streams its own
// 16*CPL weight columns of B (row-major [K][ldb]) straight from memory into
// registers and transposes them there (mfma_tile.h).
//
// Pipeline: K advances in stages of 64.  A ring of 3 register slots holds, per
// stage, the lane's two 8 x CPL weight blocks and its share of the A tile.
// While stage s is multiplied, stages s+1 and s+2 are in flight.  Loads retire
// in order, so A and B of a stage are issued together: when A of stage s+1 is
// written to LDS at the end of stage s, B of stage s+1 has arrived as well and
// the two newer stages stay outstanding.  One barrier per stage.
//
// Register pressure decides whether this works: if the live ring, the
// accumulators and the temporaries do not fit, the allocator reuses
// registers that are still the targets of outstanding loads and the compiler
// then waits for those loads mid-stage, serialising the pipeline.  The
// configurations used keep well below the per-wave budget (e.g. 8 waves,
// 2 columns per lane, 160 rows: 80 accumulator AGPRs).
#pragma once

#include "common.h"
#include "mfma_tile.h"

namespace moe {

constexpr int GC_KS = 64;            // K per stage
constexpr int GC_LDA = GC_KS + 8;    // LDS row stride in bf16 (144 B): fragment reads hit distinct banks
constexpr int GC_NBUF = 3;           // register ring depth
#ifndef MOE_GC_STEADY
#define MOE_GC_STEADY 0              // 1: unguarded three-step loop body (one basic block)
#endif

struct GemmArgs {
  const bf16_t* A;   // first row of this block
  int64_t lda;       // A row stride (elements)
  int R;             // valid rows (1 .. 16*MT); rows >= R are clamped to R-1
  const bf16_t* B;   // weight matrix [K][ldb]
  int64_t ldb;
  int kbeg, kend;    // K range [kbeg, kend), kbeg a multiple of 8
  int N;             // valid columns of B
  int col;           // this lane's first column (CPL consecutive)
};

// The A share of a stage always covers whole slabs of 8*NW rows (16*MT
// rounded up), so every thread has the same number of vectors and no load is
// predicated.  Rows at or past R are clamped to row R-1: they read valid
// memory, produce finite values in accumulator rows that are never stored, and
// keep the loop free of exec-mask branches (branches make the compiler wait for
// all outstanding loads at their join points).
template <int NW, int CPL, int MT>
struct Pipe {
  static constexpr int NT = 64 * NW;                       // threads
  static constexpr int AV = (128 * MT + NT - 1) / NT;      // 16-byte A vectors per thread per stage
  static constexpr int AROWS = AV * NT / 8;                // rows per LDS stage buffer
  BBlk<CPL> b[GC_NBUF][2];
  u32x4 ar[GC_NBUF][AV];
};

// LDS bf16 elements needed by gemm_mainloop<NW, CPL, MT>.
template <int NW, int CPL, int MT>
constexpr int gc_lds_elems() { return 2 * Pipe<NW, CPL, MT>::AROWS * GC_LDA; }

template <int J, int NW, int CPL, int MT, bool CHECK>
__device__ __forceinline__ void gc_issue(Pipe<NW, CPL, MT>& P, int st, int nst, const GemmArgs& g) {
  if (st >= nst) return;
  const int k0 = g.kbeg + st * GC_KS;
  if (CHECK) {
    load_b_block<CPL>(P.b[J][0], g.B, g.ldb, k0, g.kend, g.col, g.N);
    load_b_block<CPL>(P.b[J][1], g.B, g.ldb, k0 + 32, g.kend, g.col, g.N);
  } else {
    load_b_block_nocheck<CPL>(P.b[J][0], g.B, g.ldb, k0, g.col);
    load_b_block_nocheck<CPL>(P.b[J][1], g.B, g.ldb, k0 + 32, g.col);
  }
#pragma unroll
  for (int q = 0; q < Pipe<NW, CPL, MT>::AV; ++q) {
    const int v = threadIdx.x + Pipe<NW, CPL, MT>::NT * q;
    const int r = min(v >> 3, g.R - 1);
    const int k = k0 + 8 * (v & 7);
    if (CHECK) {
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (k < g.kend) val = *reinterpret_cast<const u32x4*>(g.A + (int64_t)r * g.lda + k);
      P.ar[J][q] = val;
    } else {
      P.ar[J][q] = *reinterpret_cast<const u32x4*>(g.A + (int64_t)r * g.lda + k);
    }
  }
}

template <int J, int NW, int CPL, int MT>
__device__ __forceinline__ void gc_stash(Pipe<NW, CPL, MT>& P, int st, int nst, bf16_t* As) {
  if (st >= nst) return;
  bf16_t* dst = As + (st & 1) * (Pipe<NW, CPL, MT>::AROWS * GC_LDA);
#pragma unroll
  for (int q = 0; q < Pipe<NW, CPL, MT>::AV; ++q) {
    const int v = threadIdx.x + Pipe<NW, CPL, MT>::NT * q;
    *reinterpret_cast<u32x4*>(dst + (v >> 3) * GC_LDA + 8 * (v & 7)) = P.ar[J][q];
  }
}

template <int J, int NW, int CPL, int MT>
__device__ __forceinline__ void gc_compute(Pipe<NW, CPL, MT>& P, int st, const bf16_t* As,
                                           f32x4 (&acc)[MT][CPL]) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const bf16_t* src = As + (st & 1) * (Pipe<NW, CPL, MT>::AROWS * GC_LDA) + i * GC_LDA + 8 * g;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    bf16x8 bf[CPL];
    transpose_b<CPL>(P.b[J][sub], bf);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(src + 16 * mt * GC_LDA + 32 * sub);
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[mt][c] = mfma16(af, bf[c], acc[mt][c]);
    }
  }
}

template <int J, int NW, int CPL, int MT, bool CHECK, bool GUARD>
__device__ __forceinline__ void gc_step(Pipe<NW, CPL, MT>& P, int st, int nst, const GemmArgs& g,
                                        bf16_t* As, f32x4 (&acc)[MT][CPL]) {
  if (GUARD && st >= nst) return;
  if (!GUARD || st + 2 < nst) gc_issue<(J + 2) % GC_NBUF, NW, CPL, MT, CHECK>(P, st + 2, st + 3, g);
  gc_compute<J, NW, CPL, MT>(P, st, As, acc);
  if (!GUARD || st + 1 < nst) gc_stash<(J + 1) % GC_NBUF, NW, CPL, MT>(P, st + 1, st + 2, As);
  __syncthreads();
}

// acc[mt][c][r] receives rows 16 mt + 4 (lane / 16) + r, column g.col + c.
// As must hold gc_lds_elems<NW, CPL, MT>() bf16; g.R >= 1.  All 64*NW threads
// must call this.
//
// The steady-state loop runs three steps per trip with no conditions inside,
// so all of a trip is one basic block: the loads of stage s+2 cannot be sunk
// (by the compiler's sinking or scheduling passes) towards their use two
// steps later.  The last stages run through guarded steps.
template <int NW, int CPL, int MT, bool CHECK>
__device__ __forceinline__ void gemm_mainloop(const GemmArgs& g, bf16_t* As,
                                              f32x4 (&acc)[MT][CPL]) {
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = (g.kend - g.kbeg + GC_KS - 1) / GC_KS;
  if (nst <= 0) return;
  Pipe<NW, CPL, MT> P;
  gc_issue<0, NW, CPL, MT, CHECK>(P, 0, nst, g);
  gc_issue<1, NW, CPL, MT, CHECK>(P, 1, nst, g);
  gc_stash<0, NW, CPL, MT>(P, 0, nst, As);
  __syncthreads();
  int st = 0;
#if MOE_GC_STEADY
  for (; st + 5 <= nst; st += GC_NBUF) {
    gc_step<0, NW, CPL, MT, CHECK, false>(P, st, nst, g, As, acc);
    gc_step<1, NW, CPL, MT, CHECK, false>(P, st + 1, nst, g, As, acc);
    gc_step<2, NW, CPL, MT, CHECK, false>(P, st + 2, nst, g, As, acc);
  }
#else
  for (; st + 5 <= nst; st += GC_NBUF) {
    gc_step<0, NW, CPL, MT, CHECK, true>(P, st, nst, g, As, acc);
    gc_step<1, NW, CPL, MT, CHECK, true>(P, st + 1, nst, g, As, acc);
    gc_step<2, NW, CPL, MT, CHECK, true>(P, st + 2, nst, g, As, acc);
  }
#endif
  // at most 4 stages remain; slot of stage st is st % 3 == 0 here
  gc_step<0, NW, CPL, MT, CHECK, true>(P, st, nst, g, As, acc);
  gc_step<1, NW, CPL, MT, CHECK, true>(P, st + 1, nst, g, As, acc);
  gc_step<2, NW, CPL, MT, CHECK, true>(P, st + 2, nst, g, As, acc);
  gc_step<0, NW, CPL, MT, CHECK, true>(P, st + 3, nst, g, As, acc);
}

}  // namespace moe
