// Large expert-GEMM tiles fed by buffer loads that write straight into LDS
// (gfx950): 256 rows of A against a 256-column block of a row-major [K][N]
// bf16 matrix B, 8 waves (two per SIMD).  Used where a segment is long enough
// for the product to be bound by the matrix cores rather than by the weight
// stream (dense routing), and by the GEMM with per-tile completion flags.
//
// Per 32-K stage the waves copy the weight block as two half-panels of 32 rows
// x 128 columns (GEMM-1: the W1 columns and the same W3 columns of 128 h
// columns; GEMM-2: two neighbouring 128-column halves of W2) and the stage's
// 32 K of all 256 A rows, each wave with two weight and two A copy
// instructions of 16 bytes per lane (weight copies read four 256-byte row
// runs, A copies sixteen 64-byte runs).  No register holds the data in transit
// and no instruction rewrites it.  The ring has BD_NS slots of 32 KB and a
// wave holds the fragments of the stage it multiplies in registers, so
// BD_NS - 1 stages are in flight; a stage is released by an explicit wait for
// the wave's own copies and one barrier (the copy/wait/barrier protocol of
// dma_tile.h).  Four slots measured as fast as five (all of LDS); the tile is
// bound by the rate at which a compute unit's copies complete (each spans 8 to
// 16 cache lines, and about one line in six misses L2), not by the matrix
// cores.
//
// Wave w = (wm, wn) = (w & 3, w >> 2) multiplies rows 64 wm .. 64 wm + 63 by
// 128 weight columns: GEMM-1 h columns 64 wn .. 64 wn + 63 of W1 (n-tiles
// 0..3) and of W3 (n-tiles 4..7), GEMM-2 half-panel wn (n-tiles 0..7).  The
// MFMA takes the weights as its 16-row operand: a lane's weight fragment (8
// consecutive k of one column) is two ds_read_b64_tr_b16 reads of the
// row-major half-panel, its A fragment one 16-byte read.  A product lane then
// holds 4 consecutive output columns of one row (8-byte stores), and the W1
// and W3 products of one h column sit in the same lane.
//
// LDS swizzle (16-byte pieces, applied on the copy side by choosing the source
// piece): half-panel row j keeps source piece q at q ^ 2 sigma(j), sigma(j) =
// (j & 3) | ((j >> 3) & 1) << 2, so the 32 lanes of a transposing read (8 rows
// x 32 bytes) cover all 64 banks once; A row r keeps piece q at q ^
// dt_swa(r), so that every pass of an A read meets 16 distinct 16-byte bank
// groups (dma_tile.h).
#pragma once

#include "common.h"
#include "gemm_core.h"
#include "dma_tile.h"

namespace moe {

constexpr int BD_BM = 256;                         // rows per tile
constexpr int BD_BN = 256;                         // weight columns per tile
constexpr int BD_HPROW = 256;                      // bytes per half-panel row (128 columns)
constexpr int BD_HP = DT_KS * BD_HPROW;            // bytes of one half-panel stage (8 KB)
constexpr int BD_AOFF = 2 * BD_HP;                 // A rows follow the two half-panels
constexpr int BD_SLOT = BD_AOFF + BD_BM * DT_KS * 2;  // bytes per ring slot (32 KB)
#ifndef MOE_BD_NS
#define MOE_BD_NS 4
#endif
constexpr int BD_NS = MOE_BD_NS;                   // ring slots
static_assert(BD_NS == 4 || BD_NS == 5, "ring of 4 or 5 slots");
// steps per unrolled trip: fragments alternate between two register sets, so
// a trip returns to the first set after an even number of steps
constexpr int BD_TL = BD_NS % 2 ? 2 * BD_NS : BD_NS;

// NW waves (8: two per SIMD, or 4: one per SIMD) in a (NW / 2) x 2 grid over
// the 256 x 256 tile: wave w = (wm, wn) = (w % WPH, w / WPH) multiplies rows
// 16 MT wm .. 16 MT wm + 16 MT - 1 by 128 weight columns (half wn).  Each
// wave copies RPW rows of its weight half-panel hp = w / WPH (CW copies of 4
// rows) and CA of the 16 A copies (16 rows each) per stage.
template <int NW>
struct BdCfg {
  static_assert(NW == 8 || NW == 4, "8 or 4 waves");
  static constexpr int WPH = NW / 2;        // waves per column half and per weight half-panel
  static constexpr int MT = 16 / WPH;       // m-tiles per wave
  static constexpr int RPW = 32 / WPH;      // weight rows a wave copies per stage
  static constexpr int CW = RPW / 4;        // weight copies per wave per stage
  static constexpr int CA = 16 / NW;        // A copies per wave per stage
  static constexpr int CNT = CW + CA;       // copy instructions per wave per stage
  static constexpr int NP = CW / 2;         // weight lane offsets: copies 2p, 2p + 1 share one
};

// Per-thread fixed state of the K loop.
template <int NW>
struct BdCtx {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t va[BdCfg<NW>::CA];   // A copies a = wave + NW v: lane source offsets (bytes) at k 0
  uint32_t vb[BdCfg<NW>::NP];   // weight copy 2p: lane source offset at stage row 0; copy
                                // 2p + 1 reads 4 rows further
  uint32_t ldb2;    // bytes per row of B
  int bdst;         // first weight destination of this wave inside a slot
  int adst;         // first A destination of this wave inside a slot
  int aoff;         // lane's A fragment offset inside the A region (m-tile 0)
  int wx;           // lane's weight fragment offset of the wave's n-tile 0
  uint32_t lbase;   // LDS address of the ring
};

// 16 bytes per lane from the buffer into LDS at byte address lds + 16 lane of
// the LDS aperture (lds wave-uniform); as dt_copy16, but with a 32-bit LDS
// address, so that no generic pointer per destination is kept in registers.
__device__ __forceinline__ void bd_copy16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff,
                                          uint32_t soff) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(lds), "v"(voff), "s"(r), "s"(soff)
      : "memory");
}

// Stage st into ring slot J.
template <int J, int NW>
__device__ __forceinline__ void bd_issue(const BdCtx<NW>& c, int st) {
  using Cfg = BdCfg<NW>;
  // recomputed per stage from one base, so that the unrolled loop does not
  // keep an address per slot and copy in scalar registers
  uint32_t b = c.lbase;
  asm volatile("" : "+s"(b));
  const uint32_t slot = b + (uint32_t)(J * BD_SLOT);
  const uint32_t k0 = (uint32_t)(st * DT_KS);
  const uint32_t sb = k0 * c.ldb2;
#pragma unroll
  for (int u = 0; u < Cfg::CW; ++u)
    bd_copy16(c.rb, slot + c.bdst + 1024 * u, c.vb[u >> 1], sb + (u & 1) * 4 * c.ldb2);
#pragma unroll
  for (int v = 0; v < Cfg::CA; ++v) bd_copy16(c.ra, slot + c.adst + NW * 1024 * v, c.va[v], k0 * 2);
}

// The fragments of one stage: MT A fragments (m-tiles) and 8 weight
// fragments (n-tiles).
template <int MT>
struct BdFrag {
  bf16x8 x[MT], w[8];
};

// Reads of the stage in slot J: the A fragments, and the weight fragment of
// n-tile t.  kleft < DT_KS (last stage only, MASK) zeroes both fragments for
// k past the end, whatever the slot holds there.
template <int J, bool MASK, int NW, int MT>
__device__ __forceinline__ void bd_read_x(const BdCtx<NW>& c, const char* ring, int kleft, BdFrag<MT>& f) {
  const char* slot = ring + J * BD_SLOT;
  const bool zero = MASK && 8 * ((threadIdx.x & 63) >> 4) >= kleft;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f.x[mt] = *reinterpret_cast<const bf16x8*>(slot + BD_AOFF + c.aoff + 1024 * mt);
    if (zero) f.x[mt] = bf16x8{};
  }
}
template <int J, bool MASK, bool SWIGLU, int MT>
__device__ __forceinline__ void bd_read_w(const char* ring, int wx, int t, int kleft, BdFrag<MT>& f) {
  const char* slot = ring + J * BD_SLOT;
  const bool zero = MASK && 8 * ((threadIdx.x & 63) >> 4) >= kleft;
  const int off = SWIGLU ? (wx ^ (32 * (t & 3))) + (t >> 2) * BD_HP : wx ^ (32 * t);
  const s16x4 lo = dt_tr16(slot + off);
  const s16x4 hi = dt_tr16(slot + off + 4 * BD_HPROW);
  f.w[t] = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  if (zero) f.w[t] = bf16x8{};
}

// Wait until at most N of this wave's copies are outstanding and its LDS
// reads have completed (so that the slot they read may be refilled), then
// barrier.
template <int N>
__device__ __forceinline__ void bd_sync() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// bd_sync with n (0..4) newer stages of CNT copies left in flight (n
// wave-uniform).
template <int CNT>
__device__ __forceinline__ void bd_sync_n(int n) {
  if (n >= 4) bd_sync<4 * CNT>();
  else if (n == 3) bd_sync<3 * CNT>();
  else if (n == 2) bd_sync<2 * CNT>();
  else if (n == 1) bd_sync<CNT>();
  else bd_sync<0>();
}

// Step st (slot J = st % BD_NS), F holding stage st's fragments: wait for
// stage st + 1 and barrier (every wave then holds stage st in registers, so
// slot J is free), refill slot J with stage st + BD_NS, then read stage st + 1
// into G while multiplying F.  GUARD: the form with range conditions (tail).
template <int J, bool GUARD, bool SWIGLU, int NW>
__device__ __forceinline__ void bd_step(const BdCtx<NW>& c, char* ring, int st, int nst, int K,
                                        BdFrag<BdCfg<NW>::MT>& F, BdFrag<BdCfg<NW>::MT>& G,
                                        f32x4 (&acc)[BdCfg<NW>::MT][8]) {
  using Cfg = BdCfg<NW>;
  constexpr int MT = Cfg::MT;
  if (GUARD && st >= nst) return;
  const bool next = !GUARD || st + 1 < nst;
  if (next) {
    // issued stages after st + 1: BD_NS - 2, fewer near the end
    if (!GUARD) bd_sync<(BD_NS - 2) * Cfg::CNT>();
    else bd_sync_n<Cfg::CNT>(min(nst - 2 - st, BD_NS - 2));
    if (!GUARD || st + BD_NS < nst) bd_issue<J % BD_NS>(c, st + BD_NS);
  }
  __builtin_amdgcn_sched_barrier(0);
  // stage st + 1's A fragments, then per n-tile t: the MT products of F's
  // fragment t and the reads of G's fragment t, which can take its registers
  const int kl = K - (st + 1) * DT_KS;
  int wx = c.wx;
  asm volatile("" : "+v"(wx));
  if (next) bd_read_x<(J + 1) % BD_NS, GUARD>(c, ring, kl, G);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt][t] = mfma16(F.w[t], F.x[mt], acc[mt][t]);
    if (next) bd_read_w<(J + 1) % BD_NS, GUARD, SWIGLU>(ring, wx, t, kl, G);
  }
  if (next) {
    __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int J, bool GUARD, bool SWIGLU, int NW>
__device__ __forceinline__ void bd_trip(const BdCtx<NW>& c, char* ring, int st, int nst, int K,
                                        BdFrag<BdCfg<NW>::MT>& F, BdFrag<BdCfg<NW>::MT>& G,
                                        f32x4 (&acc)[BdCfg<NW>::MT][8]) {
  // fragments alternate between F and G from step to step
  bd_step<J, GUARD, SWIGLU>(c, ring, st + J, nst, K, F, G, acc);
  if constexpr (J + 1 < BD_TL) bd_trip<J + 1, GUARD, SWIGLU>(c, ring, st, nst, K, G, F, acc);
}

template <int J, int NW>
__device__ __forceinline__ void bd_prologue(const BdCtx<NW>& c, int nst) {
  if constexpr (J < BD_NS) {
    if (J < nst) bd_issue<J>(c, J);
    bd_prologue<J + 1>(c, nst);
  }
}

// K loop of one 256 x 256 tile: acc = A[rows, 0 : klen] . B[0 : klen, cols],
// where A row r is A[(r0 + r) lda + k] or, with a row map, row rows[r0 + r] /
// rdiv of the abytes-byte matrix A (row stride lda), and B is row-major with
// N columns (row 0 = k 0) and brows readable rows; klen <= brows.  Columns:
// weight column block nt (GEMM-1: 128 columns of B1 and the same of B3).
// Rows past R, k past klen and columns past N read zeros or meet zeros.
// lda, N multiples of 8.  ring: BD_NS * BD_SLOT bytes of LDS.  All 64 NW
// threads call; the caller separates two tiles of one workgroup with a
// barrier.  acc[mt][t] of lane (i, g) of wave (wm, wn): row
// 16 MT wm + 16 mt + i, weight columns 16 t + 4 g .. + 3 of the wave's range
// (GEMM-1: h columns 128 nt + 64 wn + 16 (t & 3) + 4 g, of W1 for t < 4 and of
// W3 for t >= 4; otherwise columns 256 nt + 128 wn + 16 t + 4 g).
template <bool SWIGLU, int NW>
__device__ __forceinline__ void bd_accum(const bf16_t* __restrict__ A, int64_t lda,
                                         const bf16_t* __restrict__ B1, const bf16_t* __restrict__ B3,
                                         int64_t brows, int klen, int N, int r0, int R, int nt,
                                         const int32_t* __restrict__ rows, int rdiv, uint32_t abytes,
                                         char* ring, f32x4 (&acc)[BdCfg<NW>::MT][8]) {
  using Cfg = BdCfg<NW>;
  constexpr int MT = Cfg::MT;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = (klen + DT_KS - 1) / DT_KS;
  if (nst <= 0) return;
  BdCtx<NW> c;
  // weight copies: half-panel hp = wave / WPH, rows RPW (wave % WPH) .. + RPW
  // - 1, four rows (16 lanes each) per copy; rows j and j + 4 of a copy pair
  // share sigma
  const int hp = wave / Cfg::WPH, wq = wave % Cfg::WPH;
  const bf16_t* Bp = SWIGLU && hp ? B3 : B1;
  const int colbase = SWIGLU ? 128 * nt : 256 * nt + 128 * hp;
  c.rb = gc_rsrc(Bp, (uint32_t)(brows * N * 2));
  c.ldb2 = (uint32_t)(N * 2);
#pragma unroll
  for (int q = 0; q < Cfg::NP; ++q) {
    const int j = Cfg::RPW * wq + 8 * q + (lane >> 4);
    const int sig = (j & 3) | (((j >> 3) & 1) << 2);
    const int col = colbase + 8 * ((lane & 15) ^ (2 * sig));
    c.vb[q] = col < N ? (uint32_t)(((int64_t)j * N + col) * 2) : GC_OOR;
  }
  c.bdst = hp * BD_HP + Cfg::RPW * wq * BD_HPROW;
  c.lbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dt_lds_t*)ring);
  // A copies: copy a covers tile rows 16 a .. 16 a + 15, 4 lanes a row.
  // Without a row map the descriptor ends at the block's last element, k = klen
  // of row R - 1 (A may start inside a row: a K range of a wider matrix)
  c.ra = rows ? gc_rsrc(A, abytes)
              : gc_rsrc(A + (int64_t)r0 * lda, (uint32_t)(((int64_t)(R - 1) * lda + klen) * 2));
#pragma unroll
  for (int v = 0; v < Cfg::CA; ++v) {
    const int r = 16 * (wave + NW * v) + (lane >> 2);
    const int rr = min(r, R - 1);
    const uint32_t row = rows ? (uint32_t)(rows[r0 + rr] / rdiv) : (uint32_t)rr;
    c.va[v] = (row * (uint32_t)lda + 8u * (uint32_t)((lane & 3) ^ dt_swa(r))) * 2u;
  }
  c.adst = BD_AOFF + 1024 * wave;
  // fragment reads
  const int wm = wq, wn = hp;
  c.aoff = (16 * MT * wm + i) * 64 + 16 * (g ^ dt_swa(i));
  // weight fragment of n-tile ti of a half-panel: rows 8 g + i / 4 (and + 4),
  // columns 16 ti + 4 (i % 4) .. + 3 -> byte row * 256 + (32 (ti ^ sigma) +
  // 8 (i % 4)), sigma = (i / 4) | (g & 1) << 2; the XOR touches bits 5..7 only
  const int sig = (i >> 2) | ((g & 1) << 2);
  const int wlane = (8 * g + (i >> 2)) * BD_HPROW + 32 * sig + 8 * (i & 3);
  c.wx = SWIGLU ? (wlane ^ (32 * 4 * wn)) : wlane + wn * BD_HP;

  bd_prologue<0>(c, nst);   // stages 0 .. BD_NS - 1 into every slot
  bd_sync_n<Cfg::CNT>(min(nst - 1, BD_NS - 1));
  BdFrag<MT> F, G;
  bd_read_x<0, true>(c, ring, klen, F);
#pragma unroll
  for (int t = 0; t < 8; ++t) bd_read_w<0, true, SWIGLU>(ring, c.wx, t, klen, F);
  int st = 0;
  // an unguarded trip issues up to stage st + BD_TL - 1 + BD_NS
  for (; st + BD_TL + BD_NS <= nst; st += BD_TL) bd_trip<0, false, SWIGLU>(c, ring, st, nst, klen, F, G, acc);
  bd_trip<0, true, SWIGLU>(c, ring, st, nst, klen, F, G, acc);
  bd_trip<0, true, SWIGLU>(c, ring, st + BD_TL, nst, klen, F, G, acc);
}

// One 256 x 256 tile on NW waves: rows [r0, r0 + R) (1 <= R <= 256) of A,
// where A row r is A[r0 + r] or, with a row map, row rows[r0 + r] / rdiv of
// the abytes-byte matrix A; weight column block nt of expert e.  K and N
// multiples of 8.
//   SWIGLU: C[r0 + r][128 nt + h] = rnd(SiLU(A W1) * (A W3)), B1/B3 = [E][K][N]
//   else:   C[r0 + r][256 nt + n] = rnd(s (A W2)),             B1 = [E][K][N]
// with s = rscale[r0 + r], or 1 when rscale is NULL.
template <bool SWIGLU, int NW>
__device__ __forceinline__ void bd_tile(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B1,
                                        const bf16_t* __restrict__ B3, int K, int N,
                                        bf16_t* __restrict__ C, int e, int r0, int R, int nt,
                                        const int32_t* __restrict__ rows, int rdiv, uint32_t abytes,
                                        const float* __restrict__ rscale, char* ring) {
  constexpr int MT = BdCfg<NW>::MT;
  const int64_t estride = (int64_t)K * N;
  f32x4 acc[MT][8];
  bd_accum<SWIGLU, NW>(A, K, B1 + e * estride, SWIGLU ? B3 + e * estride : nullptr, K, K, N, r0, R,
                       nt, rows, rdiv, abytes, ring, acc);
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % BdCfg<NW>::WPH, wn = wave / BdCfg<NW>::WPH;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = 16 * MT * wm + 16 * mt + i;
    const float sc = !SWIGLU && rscale && row < R ? rscale[r0 + row] : 1.0f;
#pragma unroll
    for (int t = 0; t < (SWIGLU ? 4 : 8); ++t) {
      const int col = SWIGLU ? 128 * nt + 64 * wn + 16 * t + 4 * g : 256 * nt + 128 * wn + 16 * t + 4 * g;
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = acc[mt][t][r];
        o[r] = SWIGLU ? silu_mul(a, acc[mt][t + 4][r]) : a * sc;
      }
      if (row < R && col < N)
        *reinterpret_cast<u32x2*>(C + (int64_t)(r0 + row) * N + col) =
            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  }
}

}  // namespace moe
