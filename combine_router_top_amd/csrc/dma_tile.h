// Medium expert-GEMM tiles fed by buffer loads that write straight into LDS
// (gfx950): up to DT_BM rows of A against a 512-column block of a row-major
// [K][N] bf16 matrix B, 8 waves.
//
// Per 32-K stage the waves copy the weight block (32 rows x 512 columns, held
// as two 256-column panels) and the stage's 32 K of every A row from memory
// into LDS with 16-byte-per-lane load-to-LDS instructions, so no register
// holds the data in transit and no instruction rewrites it.  Each weight copy
// instruction reads two 512-byte runs of rows of B (long runs keep the load
// pipe of a compute unit near its streaming rate).  Three LDS slots form a
// ring: two stages are in flight while the third is multiplied.  A stage is
// released by an explicit wait for the wave's own copies (vmcnt) and one
// barrier.
//
// The MFMA runs with the weights as its 16-row operand: a lane's fragment, 8
// consecutive k of one weight column, comes from two ds_read_b64_tr_b16 reads
// of the row-major panel, and the A fragment (8 consecutive k of one row) from
// one 16-byte read.  Each lane of a product then holds 4 consecutive output
// columns of one row, which the epilogue stores as 8 bytes.  For GEMM-1 the
// W1 and W3 products of one h column land in the same lane and register.
//
// LDS is XOR-swizzled at 16-byte granularity; the swizzle is applied on the
// load side (each lane copies the source piece that belongs at its slot), so
// the transposing reads (8 rows x 32 bytes per 32 lanes) and the A reads (16
// rows x 16 bytes per 16 lanes) hit distinct banks.
//
// Wave w = (wm, wn) = (w & 1, w >> 1) multiplies rows 16 MT wm .. + 16 MT - 1
// by weight columns 128 wn .. 128 wn + 127 of the block (GEMM-1: h columns
// 64 wn .. 64 wn + 63 of W1 and the same of W3).
#pragma once

#include "common.h"
#include "gemm_core.h"

namespace moe {

constexpr int DT_KS = 32;                    // K per stage (one MFMA k-step)
constexpr int DT_MT = 5;                     // m-tiles per row half at most
constexpr int DT_BM = 32 * DT_MT;            // rows per tile at most
constexpr int DT_BN = 512;                   // weight columns per tile
constexpr int DT_PANEL = DT_KS * 256 * 2;    // bytes of one 256-column panel stage
constexpr int DT_AOFF = 2 * DT_PANEL;        // A rows follow the two panels
constexpr int DT_DUMMY = DT_AOFF + DT_BM * DT_KS * 2;  // 1 KB target of the unused A copies
constexpr int DT_SLOT = DT_DUMMY + 1024;              // bytes per ring slot

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void dt_lds_t;
typedef __attribute__((address_space(3))) s16x4 dt_lds4_t;

// 16 bytes per lane from the buffer into LDS at lds + 16 lane (lds wave-uniform).
// Written as inline assembly so that the compiler does not track these LDS
// writes: it would otherwise add its own vmcnt waits before LDS reads, and at
// loop heads those merge into waits that also drain the newer stages.  The
// ring's ordering is carried by dt_sync (an explicit vmcnt wait + barrier);
// loads the compiler does not know of can only make its own waits stricter,
// since loads retire in order.  M0 (the LDS base of the copy) is restored.
// (Plain functions: the templates below only call them.)
__device__ __forceinline__ void dt_copy16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                                          uint32_t soff) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dt_lds_t*)lds);
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(m), "v"(voff), "s"(r), "s"(soff)
      : "memory");
}
// ds_read_b64_tr_b16 at LDS address p.
__device__ __forceinline__ s16x4 dt_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((dt_lds4_t*)p);
}

constexpr int DT_AI = (2 * DT_MT + 7) / 8;   // A copy instructions per wave per stage, at most

// The three ring slots (distinct __shared__ arrays of DT_SLOT bytes) and a
// table of DT_AI * 512 words for the lanes' A copy offsets (each lane reads
// back only the entries it wrote, so the table needs no barrier).
struct DtSlots {
  char* s[3];
  uint32_t* tab;
};

// Weight panel row j (0..31) stores source piece q (16 bytes) at piece
// q ^ dt_swb(j); A row r stores piece q (0..3) at q ^ dt_swa(r).
__device__ __forceinline__ int dt_swb(int j) { return 2 * ((j & 3) | (((j >> 3) & 1) << 2)); }
__device__ __forceinline__ int dt_swa(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// Every wave issues the same copies per stage (4 weight copies, AI A copies),
// without branches: waves past the last A instruction copy from an offset
// outside the A descriptor (nothing is fetched) into the slot's dummy area.
// The per-stage count is then exact for the vmcnt waits.
template <int MT>
struct DtCtx {
  static constexpr int AI = (2 * MT + 7) / 8;   // A copy instructions per wave per stage
  static constexpr int CNT = 4 + AI;            // copy instructions per stage, every wave
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t vb[2];    // weight copies 0, 1: lane source offsets (bytes) at stage K row 0;
                     // copies 2, 3 read 4 rows further with the same offsets
  uint32_t ldb2;     // bytes per row of B
  int bdst;          // this wave's first weight destination inside a slot (bytes)
  int wave;
  int aoff;          // lane's A fragment offset inside the A region (m-tile 0)
  int wx;            // lane's weight fragment offset of the wave's first n-tile; n-tile
                     // t of a panel is at wx ^ (32 t) (plus DT_PANEL for GEMM-1's W3)
};

// Stage st into slot J: 4 weight copies per wave, then its A copies.
template <int J, int MT>
__device__ __forceinline__ void dt_issue(const DtCtx<MT>& c, const DtSlots& S, int st) {
  char* slot = S.s[J];
  const uint32_t k0 = (uint32_t)(st * DT_KS);
  const uint32_t sb = k0 * c.ldb2;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    dt_copy16(c.rb, slot + c.bdst + 1024 * u, c.vb[u & 1], sb + (u >> 1) * 4 * c.ldb2);
#pragma unroll
  for (int v = 0; v < DtCtx<MT>::AI; ++v) {
    const int a = c.wave + 8 * v;
    dt_copy16(c.ra, slot + (a < 2 * MT ? DT_AOFF + 1024 * a : DT_DUMMY), S.tab[512 * v + threadIdx.x],
              k0 * 2);
  }
}

// Wait until at most N of this wave's copies are outstanding, then barrier.
template <int N>
__device__ __forceinline__ void dt_sync() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Multiply the stage in slot J.  kleft < DT_KS (last stage only, MASK) zeroes
// both fragments for k past the end, whatever the slot holds there.
template <int J, bool MASK, bool SWIGLU, int MT>
__device__ __forceinline__ void dt_compute(const DtCtx<MT>& c, const DtSlots& S, int kleft,
                                           f32x4 (&acc)[MT][8]) {
  const char* slot = S.s[J];
  const int g = (threadIdx.x & 63) >> 4;
  const bool zero = MASK && 8 * g >= kleft;
  // the per-tile offsets are one XOR each; recomputing them every stage keeps
  // them out of the register file
  int wx = c.wx;
  asm volatile("" : "+v"(wx));
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 xf[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    xf[mt] = *reinterpret_cast<const bf16x8*>(slot + DT_AOFF + c.aoff + 1024 * mt);
    if (zero) xf[mt] = bf16x8{};
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int off = SWIGLU ? (wx ^ (32 * (t & 3))) + (t >> 2) * DT_PANEL : wx ^ (32 * t);
    const s16x4 lo = dt_tr16(slot + off);
    const s16x4 hi = dt_tr16(slot + off + 4 * 512);
    bf16x8 wf = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    if (zero) wf = bf16x8{};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt][t] = mfma16(wf, xf[mt], acc[mt][t]);
  }
  // order: A fragments and n-tiles 0, 1's reads, then per n-tile t its MFMAs
  // and n-tile t + 2's two reads (three weight fragments live at a time)
  __builtin_amdgcn_sched_group_barrier(0x100, MT + 4, 0);
#pragma unroll
  for (int t = 0; t < 6; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * MT, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Stage st in slot J = st % 3: wait for it, refill the slot of stage st - 1
// (every wave is past it) with stage st + 2, multiply.  GUARD: the form with
// range conditions (tail).  (Refilling a slot right after its own multiply,
// behind a second barrier, keeps three stages in flight but puts the multiply
// on the critical path; it measured slower.)
template <int J, bool GUARD, bool SWIGLU, int MT>
__device__ __forceinline__ void dt_step(const DtCtx<MT>& c, const DtSlots& S, int st, int nst, int K,
                                        f32x4 (&acc)[MT][8]) {
  if (GUARD && st >= nst) return;
  if (!GUARD || st + 1 < nst) dt_sync<DtCtx<MT>::CNT>();
  else dt_sync<0>();
  if (!GUARD || st + 2 < nst) dt_issue<(J + 2) % 3>(c, S, st + 2);
  dt_compute<J, GUARD, SWIGLU>(c, S, K - st * DT_KS, acc);
}

template <int J, bool GUARD, bool SWIGLU, int MT>
__device__ __forceinline__ void dt_trip(const DtCtx<MT>& c, const DtSlots& S, int st, int nst, int K,
                                        f32x4 (&acc)[MT][8]) {
  dt_step<J, GUARD, SWIGLU>(c, S, st + J, nst, K, acc);
  if constexpr (J < 2) dt_trip<J + 1, GUARD, SWIGLU>(c, S, st, nst, K, acc);
}

// One medium block: rows [r0, r0 + R) of expert e (32 (MT - 1) < R <= 32 MT,
// R >= 1), weight column block nb of mcols columns (a multiple of 64, at most
// DT_BN; GEMM-1: h columns mcols / 2 * nb .. + mcols / 2 - 1 of W1 and W3,
// GEMM-2: output columns mcols * nb .. + mcols - 1).  A row r is A[r0 + r] or, with a row map, row
// rows[r0 + r] / rdiv of the abytes-byte matrix A.  K and N multiples of 8.
//   SWIGLU: C[r0 + r][h] = rnd(SiLU(A W1) * (A W3)),  B1/B3 = [E][K][N]
//   else:   C[r0 + r][n] = rnd(s (A W2)),               B1 = [E][K][N]
// with s = rscale[r0 + r], or 1 when rscale is NULL.
template <bool SWIGLU, int MT>
__device__ __forceinline__ void dt_block(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B1,
                                         const bf16_t* __restrict__ B3, int K, int N,
                                         bf16_t* __restrict__ C, int e, int r0, int R, int nb, int mcols,
                                         const int32_t* __restrict__ rows, int rdiv, uint32_t abytes,
                                         const float* __restrict__ rscale, int wave, const DtSlots& S) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int64_t estride = (int64_t)K * N;
  DtCtx<MT> c;
  c.wave = wave;
  // weight copies: waves 0-3 fill panel 0, waves 4-7 panel 1; wave w copies
  // panel rows 8 (w & 3) .. + 7, two rows per instruction
  const int panel = wave >> 2;
  const bf16_t* Bp = (SWIGLU && panel ? B3 : B1) + e * estride;
  const int cblk = SWIGLU ? (mcols >> 1) * nb : mcols * nb;       // first column of the block
  const int cend = min(N, cblk + (SWIGLU ? mcols >> 1 : mcols));  // columns past it are not used
  const int colbase = SWIGLU ? cblk : cblk + 256 * panel;
  c.rb = gc_rsrc(Bp, (uint32_t)(estride * 2));
  c.ldb2 = (uint32_t)(N * 2);
  // rows j and j + 4 of a copy pair share dt_swb (it depends on j & 3 and j & 8)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = 8 * (wave & 3) + 2 * u + (lane >> 5);
    const int col = colbase + 8 * ((lane & 31) ^ dt_swb(j));
    c.vb[u] = col < cend ? (uint32_t)(((int64_t)j * N + col) * 2) : GC_OOR;
  }
  c.bdst = panel * DT_PANEL + 4096 * (wave & 3);
  // A copies: instruction a covers tile rows 16 a .. 16 a + 15, 4 lanes a row.
  // The lane source offsets (bytes, below 2^31: the A descriptor's size) go to
  // the table: across the K loop they would need registers.
  c.ra = rows ? gc_rsrc(A, abytes) : gc_rsrc(A + (int64_t)r0 * K, (uint32_t)((int64_t)R * K * 2));
#pragma unroll
  for (int v = 0; v < DtCtx<MT>::AI; ++v) {
    const int r = 16 * (wave + 8 * v) + (lane >> 2);
    const int rr = min(r, R - 1);
    const uint32_t row = rows ? (uint32_t)(rows[r0 + rr] / rdiv) : (uint32_t)rr;
    S.tab[512 * v + threadIdx.x] = wave + 8 * v < 2 * MT
        ? (row * (uint32_t)K + 8u * (uint32_t)((lane & 3) ^ dt_swa(r))) * 2u
        : GC_OOR;
  }
  // fragment reads
  const int wm = wave & 1, wn = wave >> 1;
  c.aoff = (16 * MT * wm + i) * 64 + 16 * (g ^ dt_swa(i));
  // weight fragment of n-tile ti (16 columns) of a panel: rows 8 g + i / 4
  // (and + 4), column 16 ti + 4 (i % 4) -> byte row 512 + 32 (ti ^ sig) +
  // 16 ((i % 4) / 2) + 8 (i % 2), sig = dt_swb(row) / 2; the XOR touches bits
  // 5..8 only, so the slab's first tile and the panel fold into one base
  const int sig = (i >> 2) | ((g & 1) << 2);
  const int wlane = (8 * g + (i >> 2)) * 512 + 32 * sig + 16 * ((i & 3) >> 1) + 8 * (i & 1);
  c.wx = SWIGLU ? (wlane ^ (32 * 4 * wn)) : (wlane ^ (32 * 8 * (wn & 1))) + (wn >> 1) * DT_PANEL;

  f32x4 acc[MT][8];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = (K + DT_KS - 1) / DT_KS;
  if (nst > 0) {
    dt_issue<0>(c, S, 0);
    if (nst > 1) dt_issue<1>(c, S, 1);
    int st = 0;
    for (; st + 5 <= nst; st += 3) dt_trip<0, false, SWIGLU>(c, S, st, nst, K, acc);
    dt_trip<0, true, SWIGLU>(c, S, st, nst, K, acc);
    dt_trip<0, true, SWIGLU>(c, S, st + 3, nst, K, acc);
  }

  // epilogue: lane (i, g), m-tile mt, n-tile t holds row 16 MT wm + 16 mt + i,
  // columns 16 t + 4 g .. + 3 of the wave's column range
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = 16 * MT * wm + 16 * mt + i;
    const float sc = !SWIGLU && rscale && row < R ? rscale[r0 + row] : 1.0f;
#pragma unroll
    for (int t = 0; t < (SWIGLU ? 4 : 8); ++t) {
      const int col = cblk + (SWIGLU ? 64 * wn : 128 * wn) + 16 * t + 4 * g;
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = acc[mt][t][r];
        o[r] = SWIGLU ? a / (1.0f + expf(-a)) * acc[mt][t + 4][r] : a * sc;
      }
      if (row < R && col < cend)
        *reinterpret_cast<u32x2*>(C + (int64_t)(r0 + row) * N + col) =
            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  }
}

}  // namespace moe
