// Router: logits = x . W_g (+ b) with fp32 accumulation, then per-token top-k
// softmax gating.  The routing step of the DeepSeek-V3 MoE layer in "CUCo: An
// Agentic Framework for Compute and Communication Co-design" (Abstract;
// Table 4, row "MoE Dispatch/Combine"); the pages give no formula, so this is
// the plain softmax top-k gate renormalised over the selected k, ties to the
// lower expert index.
//
// Kernels
//   router_dma          bf16, E % 8 == 0 and E >= 128, long batches (at least 8
//                       token blocks of 128): split-K MFMA GEMM with both operands
//                       copied straight from memory into a 3-slot LDS ring
//                       (64-K stages: 128-byte runs of every x row, 512-byte
//                       rows of W_g); 128 tokens x 256 experts per workgroup,
//                       8 waves of 64 x 64.  The split is the fastest-varying
//                       workgroup index, so with 8 splits each XCD streams one
//                       K slice of W_g, which stays in its L2.  Writes fp32
//                       partial sums per K split; can also zero the dispatch
//                       chunk histograms that top-k then fills.
//   router_wide_mfma    bf16, E % 4 == 0 and E > 16: split-K MFMA GEMM on the
//                       pipelined core (gemm_core.h); 8 waves, each 16 MT
//                       tokens x 32 experts, the workgroup 16 MT x 256 with
//                       MT = 10, or 5 when the 160-token grid would fill less
//                       than half the chip (short batches).  Writes fp32
//                       partial sums per K split.
//   router_narrow_mfma  bf16, E <= 16 and E*d <= 32K: W_g^T staged once in LDS,
//                       each wave streams its own 32 token rows with buffer
//                       loads straight into MFMA A fragments, one 128-K chunk
//                       in flight.  HBM-bound on x.
//   router_plain        any dtype/shape: one thread per logit (fp32 problems
//                       and shapes the MFMA kernels do not cover).
//   topk_softmax_multi  12 or more K splits (short batches): one workgroup
//                       per token, 4 waves each sum a quarter of the splits,
//                       quarters added in wave order, wave 0 selects.
//   topk_softmax_kernel one wave per token: sums the K splits in fixed order
//                       (loads of 8 splits x all of a lane's experts in
//                       flight together), adds the bias, optionally stores
//                       the logits, then k rounds of a wave-wide max of
//                       order-preserving 32-bit value keys (the lowest expert
//                       among equal maxima wins); optionally counts the
//                       selections into the dispatch chunk histograms.
#include <algorithm>

#include "common.h"
#include "gemm_core.h"
#include "dma_tile.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// wide router (bf16, MFMA, split-K) on the pipelined core of gemm_core.h
// ---------------------------------------------------------------------------
// 16 MT tokens x 256 experts per workgroup (8 waves, each 16 MT x 32), so
// that the gate matrix is re-read once per 16 MT tokens; K is split to fill
// the chip.  MT = 10 for long batches; a short batch (decode) has too few
// token blocks to fill the chip even with the deepest splits, and halving the
// block doubles its workgroups.
constexpr int RW_NW = 8;
constexpr int RW_CPL = 2;
constexpr int RW_MT_LONG = 10;     // m-tiles per workgroup
constexpr int RW_MT_SHORT = 5;
constexpr int RW_BN = 256;         // experts per workgroup (8 waves x 32)

template <int RW_MT>
__global__ __launch_bounds__(64 * RW_NW) void router_wide_mfma(const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ wg,
                                                               float* __restrict__ part, int T,
                                                               int d, int E, int kchunk) {
  constexpr int RW_BM = 16 * RW_MT;  // tokens per workgroup
  __shared__ __attribute__((aligned(16))) bf16_t As[gc_lds_elems<RW_NW, RW_CPL, RW_MT>()];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * RW_BM;
  const int split = blockIdx.y;
  const int kbeg = split * kchunk;
  const int kend = min(d, kbeg + kchunk);
  const int col = blockIdx.z * RW_BN + wave * 16 * RW_CPL + RW_CPL * i;
  const int R = min(RW_BM, T - m0);
  GemmArgs ga{x + (int64_t)m0 * d, d, R, wg, E, kbeg, kend, E, col};
  f32x4 acc[RW_MT][RW_CPL];
  gemm_mainloop<RW_NW, RW_CPL, RW_MT>(ga, As, acc);
  if (col >= E) return;
  float* out = part + (int64_t)split * T * E;
#pragma unroll
  for (int mt = 0; mt < RW_MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mt + 4 * g + r;
      if (row < R) {
        // read once by top-k: streamed past the caches (non-temporal)
        __builtin_nontemporal_store(f32x2{acc[mt][0][r], acc[mt][1][r]},
                                    reinterpret_cast<f32x2*>(out + (int64_t)(m0 + row) * E + col));
      }
    }
}

// ---------------------------------------------------------------------------
// wide router on direct-to-LDS copies (long batches)
// ---------------------------------------------------------------------------
// A workgroup multiplies 128 token rows of x by a 256-expert column block of
// W_g over one K range (a split).  Per 64-K stage every wave issues 4 weight
// copies (two 512-byte W_g rows each: the stage's 64 rows are 8 per wave) and
// 2 x copies (eight 128-byte row pieces each: 128 rows, 16 per wave), 16 bytes
// per lane, straight into a ring slot; no register holds the data in transit.
// The weights are the MFMA's row operand, read with transposing LDS reads from
// two 32-row panels per slot laid out and swizzled as the medium expert-GEMM
// tile's 256-column panels (dma_tile.h), so each lane's product holds 4
// consecutive experts of one token.  x rows are 128 bytes per stage, their
// eight 16-byte pieces XOR-swizzled by (row / 2) % 8 so that the 16 rows of a
// fragment read fall in distinct banks.  Wave w multiplies tokens
// 64 (w & 1) .. + 63 by experts 64 (w >> 1) .. + 63 of the block.
constexpr int RD_BM = 128;                           // tokens per workgroup
constexpr int RD_BN = 256;                           // experts per workgroup
constexpr int RD_KS = 64;                            // K per stage
constexpr int RD_PANEL = 32 * RD_BN * 2;             // 32 W_g rows (one MFMA k-step)
constexpr int RD_AOFF = 2 * RD_PANEL;                // x rows follow the two panels
constexpr int RD_SLOT = RD_AOFF + RD_BM * RD_KS * 2; // bytes per ring slot (48 KB)
constexpr int RD_CNT = 6;                            // copies per wave per stage
constexpr int RD_MIN_BLOCKS = 8;                     // token blocks from which router_dma is used

__device__ __forceinline__ int rd_swa(int r) { return (r >> 1) & 7; }

struct RdCtx {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t vb[2];    // weight copies 0, 1: lane source offsets (bytes) at stage row 0;
                     // copies 2, 3 read 4 rows further with the same offsets
  uint32_t va[2];    // x copies: lane source offsets (bytes) at the split's first column
  uint32_t b0, a0;   // scalar offsets of the split's first stage
  uint32_t bstage;   // bytes of 64 W_g rows
  uint32_t brow4;    // bytes of 4 W_g rows
  int wave;
};

// Stage st into slot J: 4 weight copies, then 2 x copies (every wave, always,
// so that the per-stage count is exact for the vmcnt waits).
template <int J>
__device__ __forceinline__ void rd_issue(const RdCtx& c, char* ring, int st) {
  char* slot = ring + J * RD_SLOT;
  const uint32_t sb = c.b0 + (uint32_t)st * c.bstage;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    dt_copy16(c.rb, slot + 4096 * c.wave + 1024 * u, c.vb[u & 1], sb + (u >> 1) * c.brow4);
  const uint32_t sa = c.a0 + (uint32_t)(st * RD_KS * 2);
#pragma unroll
  for (int v = 0; v < 2; ++v) dt_copy16(c.ra, slot + RD_AOFF + 1024 * (c.wave + 8 * v), c.va[v], sa);
}

// Multiply the stage in slot J (two 32-K steps).  MASK (last stage): k at or
// past kleft reads zero in both operands, whatever the slot holds there.
template <int J, bool MASK>
__device__ __forceinline__ void rd_compute(const char* ring, int aoff0, int aoff1, int wx0, int kleft,
                                           f32x4 (&acc)[4][4]) {
  const char* slot = ring + J * RD_SLOT;
  const int g = (threadIdx.x & 63) >> 4;
  int wx = wx0;
  asm volatile("" : "+v"(wx));
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bool zero = MASK && 32 * ks + 8 * g >= kleft;
    bf16x8 xf[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      xf[mt] = *reinterpret_cast<const bf16x8*>(slot + RD_AOFF + (ks ? aoff1 : aoff0) + 2048 * mt);
      if (zero) xf[mt] = bf16x8{};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int off = (wx ^ (32 * t)) + ks * RD_PANEL;
      const s16x4 lo = dt_tr16(slot + off);
      const s16x4 hi = dt_tr16(slot + off + 4 * 512);
      bf16x8 wf = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      if (zero) wf = bf16x8{};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][t] = mfma16(wf, xf[mt], acc[mt][t]);
    }
  }
}

// Stage st in slot J = st % 3: wait for it, refill the slot of stage st - 1
// (every wave is past it after the barrier) with stage st + 2, multiply.
template <int J, bool GUARD>
__device__ __forceinline__ void rd_step(const RdCtx& c, char* ring, int st, int nst, int nk, int aoff0,
                                        int aoff1, int wx, f32x4 (&acc)[4][4]) {
  if (GUARD && st >= nst) return;
  if (!GUARD || st + 1 < nst) dt_sync<RD_CNT>();
  else dt_sync<0>();
  if (!GUARD || st + 2 < nst) rd_issue<(J + 2) % 3>(c, ring, st + 2);
  rd_compute<J, GUARD>(ring, aoff0, aoff1, wx, nk - st * RD_KS, acc);
}

template <int J, bool GUARD>
__device__ __forceinline__ void rd_trip(const RdCtx& c, char* ring, int st, int nst, int nk, int aoff0,
                                        int aoff1, int wx, f32x4 (&acc)[4][4]) {
  rd_step<J, GUARD>(c, ring, st + J, nst, nk, aoff0, aoff1, wx, acc);
  if constexpr (J < 2) rd_trip<J + 1, GUARD>(c, ring, st, nst, nk, aoff0, aoff1, wx, acc);
}

// Grid: token blocks x column blocks x splits, the split varying fastest.
// part[s][t][e] receives split s's sums for every token and expert of the
// block (an empty split writes zeros).  zero[0 .. nzero) is cleared (the
// dispatch chunk histograms that top-k fills next), or zero is NULL.
__global__ __launch_bounds__(512, 1) void router_dma(const bf16_t* __restrict__ x,
                                                     const bf16_t* __restrict__ wg,
                                                     float* __restrict__ part, int T, int d, int E,
                                                     int S, int kc, int ncb,
                                                     int32_t* __restrict__ zero, int nzero) {
  __shared__ __attribute__((aligned(16))) char ring[3 * RD_SLOT];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int b = blockIdx.x;
  const int split = b % S, rest = b / S;
  const int cb = rest % ncb, tb = rest / ncb;
  const int m0 = tb * RD_BM;
  const int R = min(RD_BM, T - m0);
  const int kbeg = split * kc;
  const int kend = min(d, kbeg + kc);
  const int nk = kend - kbeg;
  const int nst = nk > 0 ? (nk + RD_KS - 1) / RD_KS : 0;

  RdCtx c;
  c.wave = wave;
  c.ra = gc_rsrc(x + (int64_t)m0 * d, (uint32_t)((int64_t)R * d * 2));
  c.rb = gc_rsrc(wg, (uint32_t)((int64_t)max(kend, 0) * E * 2));
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = 8 * wave + 2 * u + (lane >> 5);
    const int col = cb * RD_BN + 8 * ((lane & 31) ^ dt_swb(j));
    c.vb[u] = col < E ? (uint32_t)((j * E + col) * 2) : GC_OOR;
  }
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int r = 8 * (wave + 8 * v) + (lane >> 3);
    const int rr = min(r, R - 1);
    c.va[v] = (uint32_t)(((int64_t)rr * d + 8 * ((lane & 7) ^ rd_swa(r))) * 2);
  }
  c.b0 = (uint32_t)((int64_t)max(kbeg, 0) * E * 2);
  c.a0 = (uint32_t)(kbeg * 2);
  c.bstage = (uint32_t)(RD_KS * E * 2);
  c.brow4 = (uint32_t)(4 * E * 2);
  // fragment reads: x piece 4 ks + g of row 64 wm + 16 mt + i; weight n-tile
  // 4 wn + t of a panel (the medium tile's panel addressing)
  const int wm = wave & 1, wn = wave >> 1;
  const int arow = 64 * wm + i;
  const int aoff0 = arow * 128 + 16 * (g ^ rd_swa(i));
  const int aoff1 = arow * 128 + 16 * ((4 + g) ^ rd_swa(i));
  const int sig = (i >> 2) | ((g & 1) << 2);
  const int wlane = (8 * g + (i >> 2)) * 512 + 32 * sig + 16 * ((i & 3) >> 1) + 8 * (i & 1);
  const int wx = wlane ^ (128 * wn);

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nst > 0) {
    rd_issue<0>(c, ring, 0);
    if (nst > 1) rd_issue<1>(c, ring, 1);
    int st = 0;
    for (; st + 5 <= nst; st += 3) rd_trip<0, false>(c, ring, st, nst, nk, aoff0, aoff1, wx, acc);
    rd_trip<0, true>(c, ring, st, nst, nk, aoff0, aoff1, wx, acc);
    rd_trip<0, true>(c, ring, st + 3, nst, nk, aoff0, aoff1, wx, acc);
  }

  // lane (i, g) of m-tile mt, n-tile t: token 64 wm + 16 mt + i, experts
  // 64 wn + 16 t + 4 g .. + 3 of the block.  The partials are read once, by
  // top-k, so they are stored non-temporally; to leave as whole 1 KB rows
  // (non-temporal 64-byte pieces miss the L2's write combining: 1.5x the
  // bytes at the memory) the block goes through the idle ring first, 16-byte
  // pieces XOR-swizzled by row so that a 16-row write spreads over the banks.
  static_assert(RD_BM * RD_BN * 4 <= 3 * RD_SLOT, "the partial block fits the ring");
  __syncthreads();   // every wave is past the last stage
  float* stg = reinterpret_cast<float*>(ring);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = 64 * wm + 16 * mt + i;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int piece = (16 * wn + 4 * t + g) ^ (row & 15);   // 16-byte piece of the 1 KB row
      *reinterpret_cast<f32x4*>(stg + row * RD_BN + 4 * piece) = acc[mt][t];
    }
  }
  __syncthreads();
  float* out = part + ((int64_t)split * T + m0) * E;
  const int col = cb * RD_BN + 4 * lane;
  for (int row = wave; row < R; row += 8) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(stg + row * RD_BN + 4 * (lane ^ (row & 15)));
    if (col < E) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + (int64_t)row * E + col));
  }
  if (zero)
    for (int q = b * 512 + (int)threadIdx.x; q < nzero; q += gridDim.x * 512) zero[q] = 0;
}

// ---------------------------------------------------------------------------
// narrow router (bf16, MFMA, E <= 16)
// ---------------------------------------------------------------------------
// W_g^T is staged once per workgroup in LDS; each wave streams its own 32
// token rows with buffer loads (fixed lane offsets, scalar K offsets) straight
// into MFMA A fragments, 128 of K per chunk with the next chunk in flight.
// Rows past T and K past d read zeros (descriptor bounds / zero B fragments).
constexpr int RN_MT = 1;                 // m-tiles per wave (16 tokens)
constexpr int RN_ROWS = 4 * 16 * RN_MT;  // tokens per workgroup
constexpr int RN_KC = 256;               // K per chunk (8 MFMA k-steps)

struct NarrowChunk {
  u32x4 a[RN_MT][RN_KC / 32];
};

__device__ __forceinline__ void rn_issue(NarrowChunk& c, __amdgpu_buffer_rsrc_t rs,
                                         const uint32_t (&voff)[RN_MT], int k0) {
#pragma unroll
  for (int u = 0; u < RN_KC / 32; ++u)
#pragma unroll
    for (int mt = 0; mt < RN_MT; ++mt)
      c.a[mt][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[mt], (uint32_t)((k0 + 32 * u) * 2), 0);
}

__device__ __forceinline__ void rn_compute(const NarrowChunk& c, const bf16_t* WgT, int d, int E,
                                           int k0, f32x4 (&acc)[RN_MT]) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int u = 0; u < RN_KC / 32; ++u) {
    const int k = k0 + 32 * u + 8 * g;
    bf16x8 bfr = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    if (i < E && k < d) bfr = *reinterpret_cast<const bf16x8*>(WgT + i * d + k);
#pragma unroll
    for (int mt = 0; mt < RN_MT; ++mt)
      acc[mt] = mfma16(__builtin_bit_cast(bf16x8, c.a[mt][u]), bfr, acc[mt]);
  }
}

__global__ __launch_bounds__(256) void router_narrow_mfma(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wg,
                                                          float* __restrict__ logits, int T,
                                                          int d, int E) {
  extern __shared__ __attribute__((aligned(16))) bf16_t WgT[];  // [E][d]
  const int tid = threadIdx.x;
  // W_g is [d][E] row-major.  With E a multiple of 8 each thread takes 8 rows
  // x 8 experts, transposes the 8 x 8 block in registers and writes 8 x 16
  // bytes; otherwise it scatters 2-byte elements.
  if ((E & 7) == 0) {
    const int ng = E >> 3;
    for (int v = tid; v < (d >> 3) * ng; v += 256) {
      const int kg = v / ng, eg = v - kg * ng;
      u32x4 rowv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        rowv[r] = *reinterpret_cast<const u32x4*>(wg + (int64_t)(8 * kg + r) * E + 8 * eg);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = __builtin_amdgcn_perm(rowv[2 * q + 1][c >> 1], rowv[2 * q][c >> 1], sel);
        *reinterpret_cast<u32x4*>(WgT + (8 * eg + c) * d + 8 * kg) = o;
      }
    }
  } else {
    for (int v = tid; v < (E * d) >> 3; v += 256) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(wg + 8 * (int64_t)v);
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const int flat = 8 * v + h;
        const int kk = flat / E, e = flat - kk * E;
        WgT[e * d + kk] = (bf16_t)((h & 1) ? (q[h >> 1] >> 16) : (q[h >> 1] & 0xFFFFu));
      }
    }
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * RN_ROWS + wave * 16 * RN_MT;
  const int R = min(16 * RN_MT, T - m0);
  if (R <= 0) return;
  const __amdgpu_buffer_rsrc_t rs = gc_rsrc(x + (int64_t)m0 * d, (uint32_t)((int64_t)R * d * 2));
  uint32_t voff[RN_MT];
#pragma unroll
  for (int mt = 0; mt < RN_MT; ++mt) {
    const int r = 16 * mt + i;
    voff[mt] = r < R ? (uint32_t)(((int64_t)r * d + 8 * g) * 2) : GC_OOR;
  }
  f32x4 acc[RN_MT];
#pragma unroll
  for (int a = 0; a < RN_MT; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  NarrowChunk c0, c1;
  rn_issue(c0, rs, voff, 0);
  for (int k0 = 0; k0 < d; k0 += 2 * RN_KC) {
    if (k0 + RN_KC < d) rn_issue(c1, rs, voff, k0 + RN_KC);
    rn_compute(c0, WgT, d, E, k0, acc);
    if (k0 + RN_KC >= d) break;
    if (k0 + 2 * RN_KC < d) rn_issue(c0, rs, voff, k0 + 2 * RN_KC);
    rn_compute(c1, WgT, d, E, k0 + RN_KC, acc);
  }
  if (i >= E) return;
#pragma unroll
  for (int mt = 0; mt < RN_MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mt + 4 * g + r;
      if (row < R) logits[(int64_t)(m0 + row) * E + i] = acc[mt][r];
    }
}

// ---------------------------------------------------------------------------
// plain router (any dtype): one thread per (token, expert)
// ---------------------------------------------------------------------------
template <typename TIn>
__device__ __forceinline__ float load_val(const TIn* p, int64_t o);
template <>
__device__ __forceinline__ float load_val<float>(const float* p, int64_t o) { return p[o]; }
template <>
__device__ __forceinline__ float load_val<bf16_t>(const bf16_t* p, int64_t o) {
  return bf16_to_f32(p[o]);
}

template <typename TIn>
__global__ __launch_bounds__(256) void router_plain(const TIn* __restrict__ x,
                                                    const TIn* __restrict__ wg,
                                                    float* __restrict__ logits, int T, int d,
                                                    int E) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)T * E) return;
  const int t = (int)(id / E), e = (int)(id - (int64_t)t * E);
  float s = 0.f;
  for (int kk = 0; kk < d; ++kk) s = fmaf(load_val(x, (int64_t)t * d + kk), load_val(wg, (int64_t)kk * E + e), s);
  logits[id] = s;
}

// ---------------------------------------------------------------------------
// top-k + renormalised softmax: one wave per token
// ---------------------------------------------------------------------------
// Keys are order-preserving fp32 bits (f32_order_key, -0 folded to +0): a
// larger key is a larger logit, equal keys are equal logits, and a valid key
// is never 0, so 0 marks "taken/absent".  Each round takes the wave-wide
// maximum key; among the lanes holding it the lowest expert index wins (in
// the usual case of one such lane, that lane's own lowest index).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}

__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0xB1, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0x4E, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0x141, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0x140, 0xf, 0xf, false));
  const int a = min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16));
  const int b = min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48));
  return min(a, b);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), 0xB1, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), 0x4E, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), 0x141, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), 0x140, 0xf, 0xf, false));
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, v), 16 * r));
  return s;
}

__device__ __forceinline__ float key_to_f32(uint32_t ok) {
  const uint32_t u = (ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok;
  return __uint_as_float(u);
}

// The lane's best remaining key and its slot j (lowest j among equal keys:
// expert lane + 64 j grows with j).
template <int NV>
__device__ __forceinline__ void lane_best(const uint32_t (&key)[NV], uint32_t& bk, int& bj) {
  bk = key[0];
  bj = 0;
#pragma unroll
  for (int j = 1; j < NV; ++j)
    if (key[j] > bk) {
      bk = key[j];
      bj = j;
    }
}

// NV = values per lane = ceil(E / 64).
// Bias, optional logit store, k selection rounds and the softmax over the k
// selected: one wave, token t, with the lane's summed logits v[j] of experts
// lane + 64 j.  hist (or NULL): the dispatch chunk histograms [chunk][E] of
// 1024 assignments each, which receive one count per selection.
template <int NV>
__device__ __forceinline__ void topk_select(const float (&v)[NV], const float* __restrict__ bias,
                                            float* __restrict__ logits_out, int t, int E, int k,
                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                            int32_t* __restrict__ hist) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    key[j] = 0;
    const int e = lane + 64 * j;
    if (e < E) {
      float vj = v[j];
      if (bias) vj += bias[e];
      if (logits_out) logits_out[(int64_t)t * E + e] = vj;
      key[j] = f32_order_key(vj);
    }
  }
  uint32_t bk;
  int bj;
  lane_best<NV>(key, bk, bj);
  uint32_t myk = 0, k0 = 0;
  int mye = 0;
  for (int r = 0; r < k; ++r) {
    const uint32_t m = wave_max_u32(bk);
    const uint64_t holders = __ballot(bk == m);
    int e;
    if (__popcll(holders) == 1) {
      const int L = __builtin_ctzll(holders);
      e = L + 64 * __builtin_amdgcn_readlane(bj, L);
    } else {
      e = wave_min_i32(bk == m ? lane + 64 * bj : 0x7FFFFFFF);
    }
    if (r == 0) k0 = m;
    if (lane == r) {
      myk = m;
      mye = e;
    }
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (j == (e >> 6)) key[j] = 0;
      lane_best<NV>(key, bk, bj);
    }
  }
  const float v0 = key_to_f32(k0);
  const float ex = lane < k ? expf(key_to_f32(myk) - v0) : 0.f;
  const float sum = wave_sum_f32(ex);
  if (lane < k) {
    const int64_t a = (int64_t)t * k + lane;
    idx[a] = mye;
    w[a] = ex / sum;
    if (hist) atomicAdd(hist + (a >> 10) * E + mye, 1);
  }
}

template <int NV>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ part,
                                                           int nsplit, const float* __restrict__ bias,
                                                           float* __restrict__ logits_out, int T,
                                                           int E, int k, int32_t* __restrict__ idx,
                                                           float* __restrict__ w,
                                                           int32_t* __restrict__ hist) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // sum each expert's K splits in ascending order, starting from split 0;
  // the loads of up to 8 splits of all NV experts of the lane are issued
  // together, so a batch with at most 8 splits costs one round trip
  // Every load is unconditional (lanes past E read expert E - 1, splits past
  // the last read the last one, and the values are dropped by the adds), so
  // a batch goes out back to back instead of behind per-load branches.
  const int64_t sstride = (int64_t)T * E;
  const float* pt = part + (int64_t)t * E;
  int ej[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) ej[j] = min(lane + 64 * j, E - 1);
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = 0.f;
  for (int s = 0; s < nsplit; s += 8) {
    float q[8][NV];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* ps = pt + (int64_t)min(s + u, nsplit - 1) * sstride;
#pragma unroll
      for (int j = 0; j < NV; ++j) q[u][j] = ps[ej[j]];
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      v[j] = s == 0 ? q[0][j] : v[j] + q[0][j];
#pragma unroll
      for (int u = 1; u < 8; ++u) v[j] = s + u < nsplit ? v[j] + q[u][j] : v[j];
    }
  }
  topk_select<NV>(v, bias, logits_out, t, E, k, idx, w, hist);
}

// E a multiple of 4 in (192, 256] (4 values per lane): lane l holds the four
// consecutive experts 4 l .. 4 l + 3, so each split's values for a token
// arrive in one 16-byte load per lane, summed in ascending split order as in
// topk_softmax_kernel.  Among lanes holding the round's maximum the lowest
// lane holds the lowest expert index (and its own lowest slot among equal
// keys), so ties need no second reduction.
__global__ __launch_bounds__(256) void topk_softmax_vec4(const float* __restrict__ part, int nsplit,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits_out, int T, int E,
                                                         int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ w,
                                                         int32_t* __restrict__ hist) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int e0 = 4 * lane;
  const bool valid = e0 < E;
  // unconditional loads (lanes past E read the last quad), dropped below
  const float* pt = part + (int64_t)t * E + (valid ? e0 : E - 4);
  const int64_t sstride = (int64_t)T * E;
  f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; s += 8) {
    f32x4 q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      q[u] = *reinterpret_cast<const f32x4*>(pt + (int64_t)min(s + u, nsplit - 1) * sstride);
    v = s == 0 ? q[0] : v + q[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) v = s + u < nsplit ? v + q[u] : v;
  }
  uint32_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    key[j] = 0;
    if (valid) {
      float vj = v[j];
      if (bias) vj += bias[e0 + j];
      if (logits_out) logits_out[(int64_t)t * E + e0 + j] = vj;
      key[j] = f32_order_key(vj);
    }
  }
  uint32_t bk;
  int bj;
  lane_best<4>(key, bk, bj);
  uint32_t myk = 0, k0 = 0;
  int mye = 0;
  for (int r = 0; r < k; ++r) {
    const uint32_t m = wave_max_u32(bk);
    const int L = (int)__builtin_ctzll(__ballot(bk == m));
    const int jl = __builtin_amdgcn_readlane(bj, L);
    const int e = 4 * L + jl;
    if (r == 0) k0 = m;
    if (lane == r) {
      myk = m;
      mye = e;
    }
    if (lane == L) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == jl) key[j] = 0;
      lane_best<4>(key, bk, bj);
    }
  }
  const float v0 = key_to_f32(k0);
  const float ex = lane < k ? expf(key_to_f32(myk) - v0) : 0.f;
  const float sum = wave_sum_f32(ex);
  if (lane < k) {
    const int64_t a = (int64_t)t * k + lane;
    idx[a] = mye;
    w[a] = ex / sum;
    if (hist) atomicAdd(hist + (a >> 10) * E + mye, 1);
  }
}

// Deep K splits (short batches): one workgroup per token, each of its 4 waves
// sums a contiguous quarter of the splits (loads of up to 8 splits in flight
// together), the quarters are added in wave order through LDS, and wave 0
// selects.
constexpr int TK_MULTI_MIN_SPLITS = 12;

template <int NV>
__global__ __launch_bounds__(256) void topk_softmax_multi(const float* __restrict__ part,
                                                          int nsplit, const float* __restrict__ bias,
                                                          float* __restrict__ logits_out, int T,
                                                          int E, int k, int32_t* __restrict__ idx,
                                                          float* __restrict__ w,
                                                          int32_t* __restrict__ hist) {
  __shared__ float red[4][NV * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const int s0 = wave * nsplit / 4, s1 = (wave + 1) * nsplit / 4;
  const int64_t sstride = (int64_t)T * E;
  const float* pt = part + (int64_t)t * E + lane;
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = 0.f;
  for (int s = s0; s < s1; s += 8) {
    float q[NV][8];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        q[j][u] = (s + u < s1 && lane + 64 * j < E) ? pt[(int64_t)(s + u) * sstride + 64 * j] : 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u) v[j] += q[j][u];
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) red[wave][64 * j + lane] = v[j];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int j = 0; j < NV; ++j)
    v[j] = ((red[0][64 * j + lane] + red[1][64 * j + lane]) + red[2][64 * j + lane]) +
           red[3][64 * j + lane];
  topk_select<NV>(v, bias, logits_out, t, E, k, idx, w, hist);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
enum RouteKind { ROUTE_DMA = 0, ROUTE_WIDE = 1, ROUTE_NARROW = 2, ROUTE_PLAIN = 3 };

static int64_t rd_token_blocks(const Prob& p) { return (p.T + RD_BM - 1) / RD_BM; }
static int64_t rd_col_blocks(const Prob& p) { return (p.E + RD_BN - 1) / RD_BN; }

static RouteKind route_kind(const Prob& p) {
  if (p.dtype == 1 && p.E <= 16 && (int64_t)p.E * p.d <= 32768) return ROUTE_NARROW;
  if (p.dtype == 1 && p.E % 8 == 0 && p.E >= 128 && rd_token_blocks(p) >= RD_MIN_BLOCKS)
    return ROUTE_DMA;
  if (p.dtype == 1 && p.E % 4 == 0 && p.E > 16) return ROUTE_WIDE;
  return ROUTE_PLAIN;
}

// router_dma: as many K splits as fill one round of workgroups (one per
// compute unit), each at least 4 stages deep
static int rd_splits(const Prob& p) {
  int64_t s = 256 / (rd_token_blocks(p) * rd_col_blocks(p));
  const int64_t smax = std::max<int64_t>(1, p.d / (4 * RD_KS));
  return (int)std::max<int64_t>(1, std::min(s, smax));
}

static int64_t rw_blocks(const Prob& p, int mt) {
  return (int64_t)((p.T + 16 * mt - 1) / (16 * mt)) * ((p.E + RW_BN - 1) / RW_BN);
}

static int rw_splits(const Prob& p, int mt) {
  // at most one workgroup per compute unit (a second round of a few
  // workgroups would double the time), every split keeps >= 256 of K
  int64_t s = 256 / rw_blocks(p, mt);
  if (s < 1) s = 1;
  const int64_t smax = p.d / 256 > 1 ? p.d / 256 : 1;
  if (s > smax) s = smax;
  return (int)s;
}

// 160-token blocks when their grid fills at least half the chip, else 80
static int route_mt(const Prob& p) {
  return rw_blocks(p, RW_MT_LONG) * rw_splits(p, RW_MT_LONG) >= 128 ? RW_MT_LONG : RW_MT_SHORT;
}

static int route_splits(const Prob& p) {
  switch (route_kind(p)) {
    case ROUTE_DMA: return rd_splits(p);
    case ROUTE_WIDE: return rw_splits(p, route_mt(p));
    default: return 1;
  }
}

static int route_kchunk(const Prob& p, int S, int step) {
  const int kc = (p.d + S - 1) / S;
  return (kc + step - 1) / step * step;
}

size_t route_ws_bytes(const Prob& p) {
  // fp32 partial sums [splits][T][E]
  return (size_t)route_splits(p) * p.T * p.E * sizeof(float);
}

hipError_t launch_route(const Prob& p, const void* x, const void* wg, const float* bias,
                        float* logits, int32_t* idx, float* w, void* ws, hipStream_t st,
                        int32_t* chunk_hist, int64_t hist_elems, bool* hist_done) {
  float* part = reinterpret_cast<float*>(ws);
  const RouteKind kind = route_kind(p);
  const int S = route_splits(p);
  // the chunk histograms are filled by top-k only behind router_dma, which clears them first
  int32_t* hist = (kind == ROUTE_DMA && chunk_hist && hist_elems > 0) ? chunk_hist : nullptr;
  if (hist_done) *hist_done = hist != nullptr;
  if (kind == ROUTE_DMA) {
    const int kc = route_kchunk(p, S, RD_KS);
    const int ncb = (int)rd_col_blocks(p);
    dim3 grid((unsigned)(rd_token_blocks(p) * ncb * S));
    hipLaunchKernelGGL(router_dma, grid, dim3(512), 0, st, (const bf16_t*)x, (const bf16_t*)wg, part,
                       p.T, p.d, p.E, S, kc, ncb, hist, (int)(hist ? hist_elems : 0));
  } else if (kind == ROUTE_WIDE) {
    const int kchunk = route_kchunk(p, S, GC_KS);
    const int mt = route_mt(p);
    dim3 grid((p.T + 16 * mt - 1) / (16 * mt), S, (p.E + RW_BN - 1) / RW_BN);
    auto kern = mt == RW_MT_LONG ? router_wide_mfma<RW_MT_LONG> : router_wide_mfma<RW_MT_SHORT>;
    hipLaunchKernelGGL(kern, grid, dim3(64 * RW_NW), 0, st, (const bf16_t*)x, (const bf16_t*)wg,
                       part, p.T, p.d, p.E, kchunk);
  } else if (kind == ROUTE_NARROW) {
    dim3 grid((p.T + RN_ROWS - 1) / RN_ROWS);
    const size_t lds = (size_t)p.E * p.d * sizeof(bf16_t);
    hipLaunchKernelGGL(router_narrow_mfma, grid, dim3(256), lds, st, (const bf16_t*)x,
                       (const bf16_t*)wg, part, p.T, p.d, p.E);
  } else {
    const int64_t n = (int64_t)p.T * p.E;
    dim3 grid((unsigned)((n + 255) / 256));
    if (p.dtype == 1)
      hipLaunchKernelGGL(router_plain<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)x,
                         (const bf16_t*)wg, part, p.T, p.d, p.E);
    else
      hipLaunchKernelGGL(router_plain<float>, grid, dim3(256), 0, st, (const float*)x,
                         (const float*)wg, part, p.T, p.d, p.E);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nv = (p.E + 63) / 64;
  if (S >= TK_MULTI_MIN_SPLITS) {
    auto tk = nv <= 1 ? topk_softmax_multi<1>
            : nv <= 2 ? topk_softmax_multi<2>
            : nv <= 4 ? topk_softmax_multi<4>
            : nv <= 8 ? topk_softmax_multi<8>
                      : topk_softmax_multi<16>;
    hipLaunchKernelGGL(tk, dim3(p.T), dim3(256), 0, st, part, S, bias, logits, p.T, p.E, p.k, idx,
                       w, hist);
    return hipGetLastError();
  }
  if (nv == 4 && p.E % 4 == 0) {
    hipLaunchKernelGGL(topk_softmax_vec4, dim3((p.T + 3) / 4), dim3(256), 0, st, part, S, bias, logits,
                       p.T, p.E, p.k, idx, w, hist);
    return hipGetLastError();
  }
  auto tk = nv <= 1 ? topk_softmax_kernel<1>
          : nv <= 2 ? topk_softmax_kernel<2>
          : nv <= 4 ? topk_softmax_kernel<4>
          : nv <= 8 ? topk_softmax_kernel<8>
                    : topk_softmax_kernel<16>;
  hipLaunchKernelGGL(tk, dim3((p.T + 3) / 4), dim3(256), 0, st, part, S, bias, logits, p.T, p.E,
                     p.k, idx, w, hist);
  return hipGetLastError();
}

}  // namespace moe
