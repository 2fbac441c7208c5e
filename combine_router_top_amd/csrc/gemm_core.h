// Pipelined bf16 MFMA main loop shared by the router and the expert GEMMs.
//
// A workgroup of 4 waves computes C[rows, cols] += A[rows, K] * B[K, cols]
// for up to 16*MT rows.  A (row-major, K contiguous) is staged through a
// double-buffered LDS tile shared by the 4 waves; each wave streams its own
// 64 weight columns of B (row-major [K][ldb]) straight from memory into
// registers and transposes them there (mfma_tile.h).
//
// Pipeline: K advances in stages of 64.  A ring of 3 register slots holds, per
// stage, the lane's two 8x4 weight blocks and its share of the A tile.  While
// stage s is multiplied, stages s+1 and s+2 are in flight.  Loads retire in
// order, so A and B of a stage are issued together: when A of stage s+1 is
// written to LDS at the end of stage s, B of stage s+1 has arrived as well and
// the two newer stages stay outstanding.  One barrier per stage.
#pragma once

#include "common.h"
#include "mfma_tile.h"

namespace moe {

constexpr int GC_KS = 64;            // K per stage
constexpr int GC_LDA = GC_KS + 8;    // LDS row stride in bf16 (144 B): fragment reads hit distinct banks
constexpr int GC_NBUF = 3;           // register ring depth

struct GemmArgs {
  const bf16_t* A;   // first row of this block
  int64_t lda;       // A row stride (elements)
  int R;             // valid rows (<= 16*MT); rows >= R read as zero
  const bf16_t* B;   // weight matrix [K][ldb]
  int64_t ldb;
  int kbeg, kend;    // K range [kbeg, kend), kbeg a multiple of 8
  int N;             // valid columns of B
  int col;           // this lane's first column (4 consecutive)
};

template <int MT>
struct Pipe {
  static constexpr int AVEC = 16 * MT * (GC_KS / 8);  // 16-byte A vectors per stage
  static constexpr int AV = (AVEC + 255) / 256;       // per thread
  BRaw b[GC_NBUF][2];
  u32x4 ar[GC_NBUF][AV];
};

template <int J, int MT, bool CHECK>
__device__ __forceinline__ void gc_issue(Pipe<MT>& P, int st, int nst, const GemmArgs& g) {
  if (st >= nst) return;
  const int k0 = g.kbeg + st * GC_KS;
  if (CHECK) {
    load_b_block(P.b[J][0], g.B, g.ldb, k0, g.kend, g.col, g.N);
    load_b_block(P.b[J][1], g.B, g.ldb, k0 + 32, g.kend, g.col, g.N);
  } else {
    load_b_block_nocheck(P.b[J][0], g.B, g.ldb, k0, g.col);
    load_b_block_nocheck(P.b[J][1], g.B, g.ldb, k0 + 32, g.col);
  }
#pragma unroll
  for (int q = 0; q < Pipe<MT>::AV; ++q) {
    const int v = threadIdx.x + 256 * q;
    const int r = v >> 3, s = v & 7;
    const int k = k0 + 8 * s;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (v < Pipe<MT>::AVEC && r < g.R && (!CHECK || k < g.kend))
      val = *reinterpret_cast<const u32x4*>(g.A + (int64_t)r * g.lda + k);
    P.ar[J][q] = val;
  }
}

template <int J, int MT>
__device__ __forceinline__ void gc_stash(Pipe<MT>& P, int st, int nst, bf16_t* As) {
  if (st >= nst) return;
  bf16_t* dst = As + (st & 1) * (16 * MT * GC_LDA);
#pragma unroll
  for (int q = 0; q < Pipe<MT>::AV; ++q) {
    const int v = threadIdx.x + 256 * q;
    if (v < Pipe<MT>::AVEC) {
      const int r = v >> 3, s = v & 7;
      *reinterpret_cast<u32x4*>(dst + r * GC_LDA + 8 * s) = P.ar[J][q];
    }
  }
}

template <int J, int MT>
__device__ __forceinline__ void gc_compute(Pipe<MT>& P, int st, const bf16_t* As,
                                           f32x4 (&acc)[MT][4]) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const bf16_t* src = As + (st & 1) * (16 * MT * GC_LDA) + i * GC_LDA + 8 * g;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    bf16x8 bf[4];
    transpose_b(P.b[J][sub], bf);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(src + 16 * mt * GC_LDA + 32 * sub);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[mt][c] = mfma16(af, bf[c], acc[mt][c]);
    }
  }
}

template <int J, int MT, bool CHECK>
__device__ __forceinline__ void gc_step(Pipe<MT>& P, int st, int nst, const GemmArgs& g,
                                        bf16_t* As, f32x4 (&acc)[MT][4]) {
  if (st >= nst) return;
  gc_issue<(J + 2) % GC_NBUF, MT, CHECK>(P, st + 2, nst, g);
  gc_compute<J, MT>(P, st, As, acc);
  gc_stash<(J + 1) % GC_NBUF, MT>(P, st + 1, nst, As);
  __syncthreads();
}

// acc[mt][c][r] receives rows 16 mt + 4 (lane / 16) + r, column g.col + c.
// As must hold 2 * 16 * MT * GC_LDA bf16.  All 256 threads must call this.
template <int MT, bool CHECK>
__device__ __forceinline__ void gemm_mainloop(const GemmArgs& g, bf16_t* As, f32x4 (&acc)[MT][4]) {
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = (g.kend - g.kbeg + GC_KS - 1) / GC_KS;
  if (nst <= 0) return;
  Pipe<MT> P;
  gc_issue<0, MT, CHECK>(P, 0, nst, g);
  gc_issue<1, MT, CHECK>(P, 1, nst, g);
  gc_stash<0, MT>(P, 0, nst, As);
  __syncthreads();
  for (int st = 0; st < nst; st += GC_NBUF) {
    gc_step<0, MT, CHECK>(P, st, nst, g, As, acc);
    gc_step<1, MT, CHECK>(P, st + 1, nst, g, As, acc);
    gc_step<2, MT, CHECK>(P, st + 2, nst, g, As, acc);
  }
}

}  // namespace moe
