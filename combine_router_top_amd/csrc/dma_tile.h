// Medium expert-GEMM tiles fed by buffer loads that write straight into LDS
// (gfx950): up to DT_BM rows of A against a 512-column block of a row-major
// [K][N] bf16 matrix B, 8 waves.
//
// Per 32-K stage the waves copy the weight block (32 rows x 512 columns, held
// as two 256-column panels) and the stage's 32 K of every A row from memory
// into LDS with 16-byte-per-lane load-to-LDS instructions, so no register
// holds the data in transit and no instruction rewrites it.  Each weight copy
// instruction reads two 512-byte runs of rows of B (long runs keep the load
// pipe of a compute unit near its streaming rate).  The weights and the A
// rows have rings of their own: four weight slots (three stages in flight
// while the fourth is multiplied) and three A slots (two in flight), 159 KB of
// LDS in all.  A wave's copies retire in issue order, so a copy's wait budget
// ends at the first later copy that some stage needs; issuing each step's A
// copies (stage st + 2) before its weight copies (stage st + 3) gives the
// weights, which come from HBM, three steps and the A rows, mostly L2 hits,
// two.  A stage is released by an explicit wait for the wave's own copies
// (vmcnt) and one barrier.
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
constexpr int DT_WSLOT = 2 * DT_PANEL;       // bytes of a weight stage (two panels)
constexpr int DT_ASLOT = DT_BM * DT_KS * 2;  // bytes of an A stage
constexpr int DT_NWS = 4;                    // weight slots
constexpr int DT_NAS = 3;                    // A slots
constexpr int DT_AREG = DT_NWS * DT_WSLOT;   // the A slots follow the weight slots
constexpr int DT_LDS = DT_AREG + DT_NAS * DT_ASLOT;    // bytes of LDS the ring takes
static_assert((DT_NWS & (DT_NWS - 1)) == 0, "weight slots rotate by a mask");
static_assert(DT_LDS <= 160 * 1024, "the ring fits the LDS of a compute unit");

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

// The ring: one __shared__ array of DT_LDS bytes (weight slot j at j DT_WSLOT,
// A slot j at DT_AREG + j DT_ASLOT).
struct DtSlots {
  char* ring;
};

// Weight panel row j (0..31) stores source piece q (16 bytes) at piece
// q ^ dt_swb(j); A row r stores piece q (0..3) at q ^ dt_swa(r).  A 16-byte
// fragment read (lane 16 g + i: row i, piece g; 64-byte rows) goes to the 64
// banks (a 256-byte window) in four passes of 16 lanes, and on this part a
// pass pairs rows 0..7 of one piece with rows 8..15 of a piece that differs
// in bit 0 (measured with the bank-conflict counter on single-pattern
// probes).  Rows i and i + 8 fall in the same 64-byte bank group, so they
// must keep the same swizzle (the two pieces of a pass then differ); rows i
// and i + 4 share a group too, and (i >> 1) & 3 sends them to pieces that
// differ in bit 1.  The A reads of both tiles are then conflict-free (an
// extra term (r >> 3) & 1 had cost four conflict cycles per read).
__device__ __forceinline__ int dt_swb(int j) { return 2 * ((j & 3) | (((j >> 3) & 1) << 2)); }
__device__ __forceinline__ int dt_swa(int r) { return (r >> 1) & 3; }

// Per stage every wave issues 4 weight copies and the first AFULL waves AI A
// copies, the others AI - 1: a copy instruction costs the compute unit's
// address unit its time whether or not it fetches anything, so a tile with
// fewer than 8 AI A instructions issues no padding copies.  The per-stage
// count of each wave is then exact for its vmcnt waits.
template <int MT>
struct DtCtx {
  static constexpr int AI = (2 * MT + 7) / 8;   // A copy instructions per wave per stage, at most
  static constexpr int AFULL = 2 * MT - 8 * (AI - 1);  // waves with AI of them
  static constexpr int CW = 4;                  // weight copy instructions per wave per stage
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t va[AI];   // A copies: lane source offsets (bytes) at stage K column 0
  uint32_t vb[2];    // weight copies 0, 1: lane source offsets (bytes) at stage K row 0;
                     // copies 2, 3 read 4 rows further with the same offsets
  uint32_t ldb2;     // bytes per row of B
  int bdst;          // this wave's first weight destination inside a slot (bytes)
  int wave;
  bool afull;        // wave < AFULL (wave-uniform)
  int aoff;          // lane's A fragment offset inside the A region (m-tile 0)
  int wx;            // lane's weight fragment offset of the wave's first n-tile; n-tile
                     // t of a panel is at wx ^ (32 t) (plus DT_PANEL for GEMM-1's W3)
};

// The weights of stage st into the weight slot at byte offset wo: 4 copies per wave.
template <int MT>
__device__ __forceinline__ void dt_issue_w(const DtCtx<MT>& c, const DtSlots& S, uint32_t wo, int st) {
  char* slot = S.ring + wo;
  const uint32_t sb = (uint32_t)(st * DT_KS) * c.ldb2;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    dt_copy16(c.rb, slot + c.bdst + 1024 * u, c.vb[u & 1], sb + (u >> 1) * 4 * c.ldb2);
}

// The A rows of stage st into the A slot at byte offset ao: AI or AI - 1
// copies per wave (instruction a = wave + 8 v covers rows 16 a .. 16 a + 15).
template <int MT>
__device__ __forceinline__ void dt_issue_a(const DtCtx<MT>& c, const DtSlots& S, uint32_t ao, int st) {
  char* slot = S.ring + ao;
#pragma unroll
  for (int v = 0; v < DtCtx<MT>::AI; ++v) {
    const int a = c.wave + 8 * v;   // wave-uniform
    if (a < 2 * MT) dt_copy16(c.ra, slot + 1024 * a, c.va[v], (uint32_t)(st * DT_KS * 2));
  }
}

// Wait until at most N of this wave's copies are outstanding, then barrier.
template <int N>
__device__ __forceinline__ void dt_sync() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Multiply the stage in the weight slot at wo and the A slot at ao.  kleft <
// DT_KS (last stage only, MASK) zeroes both fragments for k past the end,
// whatever the slots hold there.
template <bool MASK, bool SWIGLU, int MT>
__device__ __forceinline__ void dt_compute(const DtCtx<MT>& c, const DtSlots& S, uint32_t wo,
                                           uint32_t ao, int kleft, f32x4 (&acc)[MT][8]) {
  const char* slot = S.ring + wo;
  const char* aslot = S.ring + ao;
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
    xf[mt] = *reinterpret_cast<const bf16x8*>(aslot + c.aoff + 1024 * mt);
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

// One step: wait for stage st (KW stages of weight copies and KA of A copies
// may stay in flight), refill the slots of stage st - 1 (every wave is past
// them) with the A rows of stage st + 2 (IA) and the weights of stage st + 3
// (IW), multiply stage st.
template <int KW, int KA, bool IA, bool IW, bool MASK, bool SWIGLU, int MT>
__device__ __forceinline__ void dt_step(const DtCtx<MT>& c, const DtSlots& S, int st, uint32_t wo,
                                        uint32_t ao, int K, f32x4 (&acc)[MT][8]) {
  constexpr int CW = DtCtx<MT>::CW, AI = DtCtx<MT>::AI;
  if (c.afull) dt_sync<KW * CW + KA * AI>();
  else dt_sync<KW * CW + KA * (AI - 1)>();
  if constexpr (IA) dt_issue_a(c, S, DT_AREG + (ao == DT_AREG ? 2 * DT_ASLOT : ao - DT_AREG - DT_ASLOT), st + 2);
  if constexpr (IW) dt_issue_w(c, S, (wo + (DT_NWS - 1) * DT_WSLOT) & (DT_NWS * DT_WSLOT - 1), st + 3);
  dt_compute<MASK, SWIGLU>(c, S, wo, ao, K - st * DT_KS, acc);
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
  c.afull = wave < DtCtx<MT>::AFULL;
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
  // A copies: instruction a covers tile rows 16 a .. 16 a + 15, 4 lanes a row
  // (lane source offsets in bytes, below 2^31: the A descriptor's size).
  c.ra = rows ? gc_rsrc(A, abytes) : gc_rsrc(A + (int64_t)r0 * K, (uint32_t)((int64_t)R * K * 2));
#pragma unroll
  for (int v = 0; v < DtCtx<MT>::AI; ++v) {
    const int r = 16 * (wave + 8 * v) + (lane >> 2);
    const int rr = min(r, R - 1);
    const uint32_t row = rows ? (uint32_t)(rows[r0 + rr] / rdiv) : (uint32_t)rr;
    c.va[v] = wave + 8 * v < 2 * MT
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
  // Copies in issue order: W0 A0 W1 A1 W2, then per step st A(st + 2) W(st + 3).
  // The wait of step st needs A(st) (and W(st), issued before it); after A(st)
  // come W(st + 1), A(st + 1) and W(st + 2), those of them that exist.
  const int nst = (K + DT_KS - 1) / DT_KS;
  if (nst > 0) {
    dt_issue_w(c, S, 0, 0);
    dt_issue_a(c, S, DT_AREG, 0);
    if (nst > 1) {
      dt_issue_w(c, S, DT_WSLOT, 1);
      dt_issue_a(c, S, DT_AREG + DT_ASLOT, 1);
    }
    if (nst > 2) dt_issue_w(c, S, 2 * DT_WSLOT, 2);
    // wave-uniform slot offsets of stage st
    uint32_t wo = 0, ao = DT_AREG;
    int st = 0;
    for (; st + 3 < nst; ++st) {
      dt_step<2, 1, true, true, false, SWIGLU>(c, S, st, wo, ao, K, acc);
      wo = (wo + DT_WSLOT) & (DT_NWS * DT_WSLOT - 1);
      ao = ao == DT_AREG + 2 * DT_ASLOT ? DT_AREG : ao + DT_ASLOT;
    }
    // the last min(nst, 3) stages; only the last one can be partial in K (its
    // masked form zeroes nothing when it is whole: one form, no branch)
    if (st + 2 < nst) {
      dt_step<2, 1, true, false, false, SWIGLU>(c, S, st, wo, ao, K, acc);
      wo = (wo + DT_WSLOT) & (DT_NWS * DT_WSLOT - 1);
      ao = ao == DT_AREG + 2 * DT_ASLOT ? DT_AREG : ao + DT_ASLOT;
      ++st;
    }
    if (st + 1 < nst) {
      dt_step<1, 1, false, false, false, SWIGLU>(c, S, st, wo, ao, K, acc);
      wo = (wo + DT_WSLOT) & (DT_NWS * DT_WSLOT - 1);
      ao = ao == DT_AREG + 2 * DT_ASLOT ? DT_AREG : ao + DT_ASLOT;
      ++st;
    }
    dt_step<0, 0, false, false, true, SWIGLU>(c, S, st, wo, ao, K, acc);
  }

  // Epilogue: lane (i, g), m-tile mt, n-tile t holds row 16 MT wm + 16 mt + i,
  // columns 16 t + 4 g .. + 3 of the wave's WC columns.  Stored as they lie,
  // each instruction would write 16 rows x 32 bytes; instead each m-tile goes
  // through a wave-private 16-row LDS tile and leaves as whole row runs of the
  // wave's columns (16 bytes a lane, 128 or 256 bytes a row), several times
  // fewer and longer write requests.  The tile's 32-byte chunks are XOR-
  // swizzled by row so that the 8-byte writes of 16 rows spread over the banks.
  // The stores are non-temporal: h and y_packed are each read once, by the
  // next launch, and left dirty in the MALL they would be written back while
  // the next step's weight stream evicts them.  (Only whole row runs go out
  // this way: non-temporal 32-byte pieces, as the large and thin tiles store
  // them, miss the L2's write combining and cost more than they save.)
  constexpr int WC = SWIGLU ? 64 : 128;   // output columns per wave
  constexpr int RB = 2 * WC;              // bytes per staged row
  constexpr int NCH = RB / 32;            // 32-byte chunks per staged row
  constexpr int LPR = RB / 16;            // lanes per row in the read-back
  constexpr int RPI = 64 / LPR;           // rows per read-back instruction
  __syncthreads();                        // every wave is past the ring's last stage
  char* stg = S.ring + 4096 * wave;
  const int colw = cblk + WC * wn;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int rbase = 16 * MT * wm + 16 * mt;
    const float sc = !SWIGLU && rscale && rbase + i < R ? rscale[r0 + rbase + i] : 1.0f;
#pragma unroll
    for (int t = 0; t < WC / 16; ++t) {
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = acc[mt][t][r];
        o[r] = SWIGLU ? silu_mul(a, acc[mt][t + 4][r]) : a * sc;
      }
      *reinterpret_cast<u32x2*>(stg + i * RB + 32 * (t ^ (i & (NCH - 1))) + 8 * g) =
          u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < 16 / RPI; ++q) {
      const int row = RPI * q + lane / LPR;
      const int p = lane % LPR;   // 16-byte piece of the row: columns 8 p .. 8 p + 7
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * RB + 32 * ((p >> 1) ^ (row & (NCH - 1))) +
                                                      16 * (p & 1));
      const int col = colw + 8 * p;
      if (rbase + row < R && col < cend)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + (int64_t)(r0 + rbase + row) * N + col));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

}  // namespace moe
