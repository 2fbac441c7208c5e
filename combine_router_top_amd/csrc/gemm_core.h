// Pipelined bf16 MFMA main loop shared by the router and the expert GEMMs.
//
// A workgroup of NW waves computes C[rows, cols] += A[rows, K] * B[K, cols]
// for up to 16*MT rows.  A (row-major, K contiguous) is staged through a
// double-buffered LDS tile shared by the waves; each wave streams its own
// 16*CPL weight columns of B (row-major [K][ldb]) straight from memory into
// registers and transposes them there (mfma_tile.h).
//
// All global loads are buffer loads: a per-lane VGPR offset that is fixed for
// the whole K loop plus a scalar offset that advances per stage.  The loop
// therefore does no per-lane address arithmetic (such arithmetic needs
// temporary registers, and when the allocator picks registers that are still
// the targets of outstanding loads the compiler must wait for those loads,
// which serialises the pipeline).  The buffer descriptors also bound every
// access in hardware: reads past the end of a descriptor return zero, which
// zero-fills the K tail of the weights (rows past kend) and lanes whose
// columns lie past N (their offset is pushed out of range).  A rows past the
// block and A columns past kend read finite values from inside the A
// descriptor; they only meet zero weights or land in accumulator rows that are
// never stored.
//
// Pipeline: K advances in stages of 64.  A ring of NB register slots holds, per
// stage, the lane's two 8 x CPL weight blocks and its share of the A tile.
// While stage s is multiplied, stages s+1 .. s+NB-1 are in flight.  Loads
// retire in order, so A and B of a stage are issued together: when A of stage
// s+1 is written to LDS at the end of stage s, B of stage s+1 has arrived as
// well and the newer stages stay outstanding.  One barrier per stage.
#pragma once

#include "common.h"
#include "mfma_tile.h"

namespace moe {

constexpr int GC_KS = 64;            // K per stage
constexpr int GC_LDA = GC_KS + 8;    // LDS row stride in bf16 (144 B): fragment reads hit distinct banks
constexpr int GC_NBUF = 3;           // default register ring depth
constexpr uint32_t GC_RSRC_W3 = 0x00020000u;  // buffer descriptor word 3 for gfx9-family raw buffers
constexpr uint32_t GC_OOR = 0x80000000u;      // lane offset that is outside every descriptor

struct GemmArgs {
  const bf16_t* A;   // first row of this block (or, with rows, the row-mapped matrix)
  int64_t lda;       // A row stride (elements)
  int R;             // rows of this block (>= 1); rows past R are never stored
  const bf16_t* B;   // weight matrix [K][ldb] (row 0 = k 0)
  int64_t ldb;
  int kbeg, kend;    // K range [kbeg, kend), kbeg a multiple of 8
  int N;             // valid columns of B
  int col;           // this lane's first column (CPL consecutive)
  // Optional row map: block row r is row rows[r] / rdiv of A, whose
  // descriptor then spans abytes (the whole matrix).  nullptr: rows are
  // consecutive from A.
  const int32_t* rows = nullptr;
  int rdiv = 1;
  uint32_t abytes = 0;
};

// Byte offset of block row r (clamped by the caller) inside the A descriptor.
__device__ __forceinline__ uint32_t gc_arow(const GemmArgs& g, int r) {
  const int64_t row = g.rows ? (int64_t)(g.rows[r] / g.rdiv) : (int64_t)r;
  return (uint32_t)(row * g.lda * 2);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gc_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)GC_RSRC_W3);
}

template <int NW, int CPL, int MT, int NB = GC_NBUF>
struct Pipe {
  static constexpr int NBUF = NB;                          // register ring slots
  static constexpr int NT = 64 * NW;                       // threads
  static constexpr int AV = (128 * MT + NT - 1) / NT;      // 16-byte A vectors per thread per stage
  static constexpr int AROWS = AV * NT / 8;                // rows per LDS stage buffer
  BBlk<CPL> b[NB][2];
  u32x4 ar[NB][AV];
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t va[AV];   // per-lane A offsets (bytes), fixed for the loop
  uint32_t vb;       // per-lane B offset (bytes), fixed for the loop
};

// LDS bf16 elements needed by gemm_mainloop<NW, CPL, MT>.
template <int NW, int CPL, int MT>
constexpr int gc_lds_elems() { return 2 * Pipe<NW, CPL, MT>::AROWS * GC_LDA; }

template <int NW, int CPL, int MT, int NB>
__device__ __forceinline__ void gc_setup(Pipe<NW, CPL, MT, NB>& P, const GemmArgs& g) {
  // A descriptor spans the block's rows (or the row-mapped matrix); B
  // descriptor spans rows [0, kend).
  P.ra = gc_rsrc(g.A, g.rows ? g.abytes : (uint32_t)((int64_t)g.R * g.lda * 2));
  P.rb = gc_rsrc(g.B, (uint32_t)((int64_t)g.kend * g.ldb * 2));
#pragma unroll
  for (int q = 0; q < Pipe<NW, CPL, MT, NB>::AV; ++q) {
    const int v = threadIdx.x + Pipe<NW, CPL, MT, NB>::NT * q;
    const int r = min(v >> 3, g.R - 1);
    P.va[q] = gc_arow(g, r) + (uint32_t)(16 * (v & 7));
  }
  const int grp = (threadIdx.x & 63) >> 4;
  P.vb = g.col < g.N ? (uint32_t)(((int64_t)(8 * grp) * g.ldb + g.col) * 2) : GC_OOR;
}

template <int J, int NW, int CPL, int MT, int NB>
__device__ __forceinline__ void gc_issue(Pipe<NW, CPL, MT, NB>& P, int st, const GemmArgs& g) {
  const int k0 = g.kbeg + st * GC_KS;
  const uint32_t row_bytes = (uint32_t)(g.ldb * 2);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t so = (uint32_t)(k0 + 32 * s + r) * row_bytes;
      if constexpr (CPL == 2)
        P.b[J][s].row[r] = __builtin_amdgcn_raw_buffer_load_b32(P.rb, P.vb, so, 0);
      else
        P.b[J][s].row[r] = __builtin_amdgcn_raw_buffer_load_b64(P.rb, P.vb, so, 0);
    }
  }
#pragma unroll
  for (int q = 0; q < Pipe<NW, CPL, MT, NB>::AV; ++q)
    P.ar[J][q] = __builtin_amdgcn_raw_buffer_load_b128(P.ra, P.va[q], (uint32_t)(k0 * 2), 0);
}

template <int J, int NW, int CPL, int MT, int NB>
__device__ __forceinline__ void gc_stash(Pipe<NW, CPL, MT, NB>& P, int st, bf16_t* As) {
  bf16_t* dst = As + (st & 1) * (Pipe<NW, CPL, MT, NB>::AROWS * GC_LDA);
#pragma unroll
  for (int q = 0; q < Pipe<NW, CPL, MT, NB>::AV; ++q) {
    const int v = threadIdx.x + Pipe<NW, CPL, MT, NB>::NT * q;
    *reinterpret_cast<u32x4*>(dst + (v >> 3) * GC_LDA + 8 * (v & 7)) = P.ar[J][q];
  }
}

template <int J, int NW, int CPL, int MT, int NB>
__device__ __forceinline__ void gc_compute(Pipe<NW, CPL, MT, NB>& P, int st, const bf16_t* As,
                                           f32x4 (&acc)[MT][CPL]) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const bf16_t* src = As + (st & 1) * (Pipe<NW, CPL, MT, NB>::AROWS * GC_LDA) + i * GC_LDA + 8 * g;
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

// Stage st uses ring slot J = st % NB; it refills the slot consumed by stage
// st-1 with stage st+NB-1, multiplies, then writes A of stage st+1 into LDS.
// GUARD selects the form with range conditions (prologue/tail); the
// steady-state form has none, so a whole trip of NB steps is one basic block
// and the loads cannot be sunk towards their use.  The scheduling barrier
// after the issue keeps the machine scheduler from doing the same.
template <int J, bool GUARD, int NW, int CPL, int MT, int NB>
__device__ __forceinline__ void gc_step(Pipe<NW, CPL, MT, NB>& P, int st, int nst, const GemmArgs& g,
                                        bf16_t* As, f32x4 (&acc)[MT][CPL]) {
  if (GUARD && st >= nst) return;
  if (!GUARD || st + NB - 1 < nst) gc_issue<(J + NB - 1) % NB>(P, st + NB - 1, g);
  __builtin_amdgcn_sched_barrier(0);
  gc_compute<J>(P, st, As, acc);
  if (!GUARD || st + 1 < nst) gc_stash<(J + 1) % NB>(P, st + 1, As);
  __syncthreads();
}

template <int J, bool GUARD, int NW, int CPL, int MT, int NB>
__device__ __forceinline__ void gc_trip(Pipe<NW, CPL, MT, NB>& P, int st, int nst, const GemmArgs& g,
                                        bf16_t* As, f32x4 (&acc)[MT][CPL]) {
  gc_step<J, GUARD>(P, st + J, nst, g, As, acc);
  if constexpr (J + 1 < NB) gc_trip<J + 1, GUARD>(P, st, nst, g, As, acc);
}

// Issue stage J into slot J for J = 0 .. NB - 2 (those that exist).
template <int J, int NW, int CPL, int MT, int NB>
__device__ __forceinline__ void gc_prologue(Pipe<NW, CPL, MT, NB>& P, int nst, const GemmArgs& g) {
  if constexpr (J < NB - 1) {
    if (J < nst) gc_issue<J>(P, J, g);
    gc_prologue<J + 1>(P, nst, g);
  }
}

// acc[mt][c][r] receives rows 16 mt + 4 (lane / 16) + r, column g.col + c.
// As must hold gc_lds_elems<NW, CPL, MT>() bf16; g.R >= 1.  All 64*NW threads
// must call this.  NB is the register ring depth (stages in flight + 1).
template <int NW, int CPL, int MT, int NB = GC_NBUF>
__device__ __forceinline__ void gemm_mainloop(const GemmArgs& g, bf16_t* As,
                                              f32x4 (&acc)[MT][CPL]) {
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = (g.kend - g.kbeg + GC_KS - 1) / GC_KS;
  if (nst <= 0) return;
  Pipe<NW, CPL, MT, NB> P;
  gc_setup(P, g);
  gc_prologue<0>(P, nst, g);  // stages 0 .. NB - 2 into slots 0 .. NB - 2
  gc_stash<0>(P, 0, As);
  __syncthreads();
  int st = 0;
  for (; st + 2 * NB - 1 <= nst; st += NB)   // stages st .. st + 2 NB - 2 exist
    gc_trip<0, false>(P, st, nst, g, As, acc);
  // fewer than 2 NB - 1 stages remain; the slot of stage st is 0 here
  gc_trip<0, true>(P, st, nst, g, As, acc);
  gc_trip<0, true>(P, st + NB, nst, g, As, acc);
}

}  // namespace moe
