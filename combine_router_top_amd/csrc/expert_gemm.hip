// Local expert compute: SwiGLU expert FFNs as grouped GEMMs over the
// expert-contiguous, unpadded segments produced by dispatch (the "local
// compute" of the DeepSeek-V3 MoE layer in "CUCo: An Agentic Framework for
// Compute and Communication Co-design", Abstract and Table 4).
//
//   GEMM-1:  h[R]        = rnd(SiLU(x_packed[R] W1_e) * (x_packed[R] W3_e))
//   GEMM-2:  y_packed[R] = rnd(h[R] W2_e)
//
// bf16 path (grouped_gemm_bf16).  A workgroup owns one row block of one
// expert and one 512-column block of its weights; every weight byte of that
// column block is streamed from HBM exactly once per row block, which is the
// bound for the segment sizes of a sparse MoE layer (about 4..160 rows per
// expert).  Two tile classes share the kernel:
//   thin (segments of at most XG_THIN_MAX rows, decode): 8 waves (2 per SIMD)
//     share the A rows through LDS; each wave streams its own weight columns
//     (4 per lane) straight from HBM into registers and transposes them there
//     into MFMA B fragments (mfma_tile.h, gemm_core.h).  GEMM-1 pairs W1 and
//     W3: the lower half of the waves streams W1 columns and the upper half
//     the same W3 columns; after the K loop the upper half passes its products
//     to the lower half through LDS, which applies SiLU(x.W1)*(x.W3).
//   medium (up to XM_BM rows per block, prefill): both operands are copied
//     from memory straight into LDS rings (four weight slots, three A
//     slots) and multiplied with the weights as the MFMA row operand
//     (dma_tile.h); W1 and W3 products of an h column meet in one register.
// The row-block schedule is derived on the device from `offsets` in the
// workgroup prologue, so the number of local assignments never travels to the
// host; the grid is sized for the worst case and surplus workgroups exit
// after the prologue.  The intermediate products never reach memory.
//
// fp32 path (grouped_gemm_f32): one thread per output element, for the small
// fp32 problems only.
#include <stdint.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "gemm_core.h"
#include "dma_tile.h"
#include "dma_big.h"

namespace moe {

constexpr int XG_MAXN = 1024;             // max local experts

// Register-streamed tile configuration (the thin class): segments of a few
// rows (decode), where the kernel is a pure weight stream and 8-byte weight
// loads keep the load-instruction rate down: 80-row blocks, 4 columns per lane.
template <int NW_, int CPL_, int MTMAX_, int NB_>
struct XGCfg {
  static constexpr int NB = NB_;                 // register ring depth
  static constexpr int NW = NW_;                 // waves per workgroup
  static constexpr int CPL = CPL_;               // weight columns per lane
  static constexpr int MTMAX = MTMAX_;           // m-tiles per row block
  static constexpr int BM = 16 * MTMAX;          // rows per row block
  static constexpr int HW = 16 * CPL;            // h columns per wave in GEMM-1
  static constexpr int WG_H = (NW / 2) * HW;     // h columns per workgroup (W1 and W3 halves)
  static constexpr int OW = 16 * CPL;            // output columns per wave in GEMM-2
  static constexpr int WG_O = NW * OW;           // output columns per workgroup
  static constexpr int COLS = WG_O;              // weight columns per workgroup (both GEMMs)
  // LDS: the A stage buffers, reused after the K loop for the W3 -> W1
  // accumulator exchange of GEMM-1.
  static constexpr int XCH = (NW / 2) * MTMAX * CPL * 4 * 64;  // floats exchanged
  static constexpr int LDS = gc_lds_elems<NW, CPL, MTMAX>() > 2 * XCH
                                 ? gc_lds_elems<NW, CPL, MTMAX>() : 2 * XCH;
};
using XGThin = XGCfg<8, 4, 5, 2>;
// Medium class (more than XG_THIN_MAX rows): blocks of up to XM_BM rows and
// XM_COLS weight columns (dt_block, dma_tile.h).
constexpr int XM_BM = DT_BM;
constexpr int XM_COLS = DT_BN;

// Row block of this workgroup: expert e, rows [r0, r0 + R), column block nb,
// tile class (0: thin, 1: medium).
struct RowBlock {
  int e, r0, R, nb, cls;
};

// Optional A row map (GEMM-1 reading x directly instead of x_packed): packed
// row p is row rows[p] / div of A, a matrix of `bytes` bytes.
struct RowMap {
  const int32_t* rows;
  int div;
  uint32_t bytes;
  // Optional scale of every output row (down projection only): packed row p
  // is multiplied by scale[p] before its rounding (the routing weight of its
  // assignment, so that combine only sums).  nullptr: no scale.
  const float* scale = nullptr;
};

// Segments of at most XG_THIN_MAX rows stream through the thin tiles, larger
// ones (below the large-tile threshold) through the medium tiles.
#ifndef MOE_XG_THIN_MAX
#define MOE_XG_THIN_MAX 48
#endif
constexpr int XG_THIN_MAX = MOE_XG_THIN_MAX;

static_assert(XG_THIN_MAX <= XGThin::BM, "a thin segment is one row block");
// Work of a block in units of 64 weight columns: the path is bound by the
// weight stream, which grows with the block's column count.  Medium blocks
// span mcols weight columns (a multiple of 64, at most XM_COLS), chosen per
// launch by the host.
constexpr int XG_WUNIT = 64;
constexpr int XG_WT_THIN = XGThin::COLS / XG_WUNIT;
static_assert(XG_WT_THIN * XG_WUNIT == XGThin::COLS, "thin columns a multiple of the work unit");

// Blocks of class `cls` of one expert with `cnt` rows (0 for the other class);
// thin blocks span tcols weight columns, medium ones mcols.
__device__ __forceinline__ int xg_blocks(int cnt, int th, int ncols, int cls, int mcols, int tcols) {
  if (cnt <= 0 || cnt >= th || (cnt <= XG_THIN_MAX ? 0 : 1) != cls) return 0;
  if (cls == 0) return (ncols + tcols - 1) / tcols;
  return (cnt + XM_BM - 1) / XM_BM * ((ncols + mcols - 1) / mcols);
}

// Real workgroups per XCD of a streamed launch with these parameters: the
// number of blocks that start in XCD x's window of schedule() below, i.e.
// min(first(w1), blocks) - first(w0) with first(w) the first block starting
// at or after w.  Wave 0 of the calling workgroup; lane x < 8 writes cnt[x].
// GEMM-1 writes them for GEMM-2, whose surplus workgroups (the grid covers
// the worst routing) then exit after one load instead of the schedule.
__device__ void xg_xcd_counts(const int32_t* __restrict__ offsets, int e_begin, int e_end, int th,
                              int ncols, int mcols, int tcols, int* __restrict__ cnt) {
  const int lane = threadIdx.x & 63;
  const int ne = e_end - e_begin;
  int nth = 0, nwd = 0;
  for (int j = lane; j < ne; j += 64) {
    const int c = offsets[e_begin + j + 1] - offsets[e_begin + j];
    nth += xg_blocks(c, th, ncols, 0, mcols, tcols);
    nwd += xg_blocks(c, th, ncols, 1, mcols, tcols);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    nth += __shfl_xor(nth, off);
    nwd += __shfl_xor(nwd, off);
  }
  if (lane < 8) {
    const int wm = mcols / XG_WUNIT, wt = tcols / XG_WUNIT;
    const int wth = wt * nth, W = wth + wm * nwd;
    const int w0 = (lane * W + 7) >> 3, w1 = ((lane + 1) * W + 7) >> 3;
    const int f0 = w0 <= wth ? (w0 + wt - 1) / wt : nth + (w0 - wth + wm - 1) / wm;
    const int f1 = w1 <= wth ? (w1 + wt - 1) / wt : nth + (w1 - wth + wm - 1) / wm;
    cnt[lane] = max(0, min(f1, nth + nwd) - f0);
  }
}

// Schedule from `offsets` (computed by every workgroup, a few hundred cycles).
// Experts in [e_begin, e_end) with fewer than `th` rows contribute (row block,
// column block) pairs of their tile class.  The blocks are listed thin class
// first, then medium, each by ascending expert; a thin block weighs tcols /
// XG_WUNIT, a medium one mcols / XG_WUNIT, and block i starts at the running sum of the
// weights before it.  XCD x (workgroup id mod 8 on this part) takes the blocks that start in
// [ceil(x W / 8), ceil((x + 1) W / 8)) of the total work W, the q-th of them
// going to its q-th workgroup.  Every XCD thus gets an equal share of the
// weight stream, the blocks of one expert mostly share one L2 (an expert's
// blocks go by column block, its row blocks fastest), and within an XCD the
// longer thin blocks start first.  Block
// starts are at least the smaller weight apart, so the grid needs
// 8 ceil(ceil(W / 8) / min weight) workgroups at most.  R = 0 means "exit".
// `pre` holds 2 (XG_MAXN + 1) ints.
__device__ RowBlock schedule(const int32_t* __restrict__ offsets, int e_begin, int e_end,
                             int th, int ncols, int mcols, int tcols, int* pre) {
  const int ne = e_end - e_begin;
  int* prew = pre + XG_MAXN + 1;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int ct = 0, cw = 0;
    for (int j0 = 0; j0 < ne; j0 += 64) {
      const int j = j0 + lane;
      const int cnt = j < ne ? offsets[e_begin + j + 1] - offsets[e_begin + j] : 0;
      int xt = xg_blocks(cnt, th, ncols, 0, mcols, tcols);
      int xw = xg_blocks(cnt, th, ncols, 1, mcols, tcols);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int yt = __shfl_up(xt, off);
        const int yw = __shfl_up(xw, off);
        if (lane >= off) { xt += yt; xw += yw; }
      }
      if (j < ne) { pre[j] = ct + xt; prew[j] = cw + xw; }
      ct += __shfl(xt, 63);
      cw += __shfl(xw, 63);
    }
    if (lane == 0) { pre[XG_MAXN] = ct; prew[XG_MAXN] = cw; }
  }
  __syncthreads();
  RowBlock rb{0, 0, 0, 0, 0};
  const int nth = pre[XG_MAXN], nwd = prew[XG_MAXN];
  const int wm = mcols / XG_WUNIT;                   // work of a medium block
  const int wt = tcols / XG_WUNIT;                   // work of a thin block
  const int wth = wt * nth;                          // work of the thin blocks
  const int W = wth + wm * nwd;
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int w0 = (xcd * W + 7) >> 3, w1 = ((xcd + 1) * W + 7) >> 3;
  // first block starting at or after w0, then this workgroup's block
  const int i0 = w0 <= wth ? (w0 + wt - 1) / wt : nth + (w0 - wth + wm - 1) / wm;
  const int i = i0 + q;
  if (i >= nth + nwd) return rb;
  const int start = i < nth ? wt * i : wth + wm * (i - nth);
  if (start >= w1) return rb;
  rb.cls = i < nth ? 0 : 1;
  const int* P = rb.cls ? prew : pre;
  const int L = rb.cls ? i - nth : i;
  int lo = 0, hi = ne - 1;  // first j with P[j] > L
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (P[mid] > L) hi = mid; else lo = mid + 1;
  }
  const int e = e_begin + lo;
  const int local = L - (lo ? P[lo - 1] : 0);
  const int o = offsets[e];
  const int cnt = offsets[e + 1] - o;
  const int bm = rb.cls ? XM_BM : XGThin::BM;
  // an expert's blocks in column-block order, its row blocks fastest: the
  // row blocks of a long segment that run together on one XCD then share
  // each weight column block in its L2 (with column blocks fastest only the
  // two or so row blocks in flight did)
  const int nrb = (cnt + bm - 1) / bm;
  int jb;
  if (nrb > 1) {
    rb.nb = local / nrb;
    jb = local - rb.nb * nrb;
  } else {
    jb = 0;
    rb.nb = local;
  }
  rb.e = e;
  rb.r0 = o + jb * bm;
  rb.R = min(bm, cnt - jb * bm);
  return rb;
}

template <class Cfg, bool SWIGLU, int MT>
__device__ __forceinline__ void gemm_body(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bl,
                                          int K, int N, int col, bf16_t* __restrict__ C,
                                          const RowBlock& rb, const RowMap& rm, bf16_t* As,
                                          float* xch0, float* xch1) {
  constexpr int CPL = Cfg::CPL, NW = Cfg::NW;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  GemmArgs ga{A + (rm.rows ? 0 : (int64_t)rb.r0 * K), K, rb.R, Bl, N, 0, K, N, col};
  if (rm.rows) {
    ga.rows = rm.rows + rb.r0;
    ga.rdiv = rm.div;
    ga.abytes = rm.bytes;
  }
  f32x4 acc[MT][CPL];
  gemm_mainloop<NW, CPL, MT, Cfg::NB>(ga, As, acc);

  // GEMM-1: waves of the upper half hold the x.W3 products of the columns the
  // lower half holds x.W1 for; they hand them over through LDS (pairs
  // 0 .. NW/4 - 1 through xch0, the others through xch1).
  bool store_wave = true;
  if (SWIGLU) {
    store_wave = wave < NW / 2;
    const int pair = wave % (NW / 2);
    float* slot = (pair < NW / 4 ? xch0 : xch1) + (pair % (NW / 4)) * (Cfg::MTMAX * CPL * 4 * 64) + lane;
    if (!store_wave) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) slot[((mt * CPL + c) * 4 + r) * 64] = acc[mt][c][r];
    }
    __syncthreads();
    if (store_wave) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = acc[mt][c][r];
            const float b = slot[((mt * CPL + c) * 4 + r) * 64];
            acc[mt][c][r] = silu_mul(a, b);
          }
    }
  }
  // epilogue: lane holds CPL consecutive columns (c) of rows 16 mt + 4 g + r
  if (!store_wave || col >= N) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mt + 4 * g + r;
      if (row < rb.R) {
        if (!SWIGLU && rm.scale) {
          const float sc = rm.scale[rb.r0 + row];
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[mt][c][r] *= sc;
        }
        bf16_t* dst = C + (int64_t)(rb.r0 + row) * N + col;
        if constexpr (CPL == 2) {
          *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[mt][0][r], acc[mt][1][r]);
        } else {
          *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(acc[mt][0][r], acc[mt][1][r]),
                                                 pack_bf16x2(acc[mt][2][r], acc[mt][3][r])};
        }
      }
    }
  }
}

// One streamed row block of class Cfg.
template <class Cfg, bool SWIGLU>
__device__ __forceinline__ void stream_block(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B1,
                                             const bf16_t* __restrict__ B3, int K, int N,
                                             bf16_t* __restrict__ C, const RowBlock& rb,
                                             const RowMap& rm, int wave, int tcols, bf16_t* As,
                                             float* xch0, float* xch1) {
  const int i = threadIdx.x & 15;
  int col;
  const bf16_t* Bl;
  const int64_t estride = (int64_t)K * N;
  if (SWIGLU) {  // lower half of the waves streams W1, upper half the same columns of W3
    col = rb.nb * Cfg::WG_H + (wave % (Cfg::NW / 2)) * Cfg::HW + Cfg::CPL * i;
    Bl = ((wave < Cfg::NW / 2) ? B1 : B3) + rb.e * estride;
  } else {       // output columns per wave; a block of tcols < WG_O columns
                 // leaves its last waves idle (columns past N: zero loads, no stores)
    col = wave * Cfg::OW < tcols ? rb.nb * tcols + wave * Cfg::OW + Cfg::CPL * i : N;
    Bl = B1 + rb.e * estride;
  }
  const int mt = (rb.R + 15) >> 4;
  switch (mt) {
#define XG_CASE(n) \
  case n: if constexpr (n <= Cfg::MTMAX) gemm_body<Cfg, SWIGLU, n>(A, Bl, K, N, col, C, rb, rm, As, xch0, xch1); break;
    XG_CASE(1) XG_CASE(2) XG_CASE(3) XG_CASE(4) XG_CASE(5)
    XG_CASE(6) XG_CASE(7) XG_CASE(8) XG_CASE(9) XG_CASE(10)
#undef XG_CASE
    default: break;
  }
}

// ---------------------------------------------------------------------------
// large segments: 256 x 256 tiles, both operands through LDS
// ---------------------------------------------------------------------------
// For experts with at least XB_TH rows the weight-streaming kernel above would
// re-read the weights once per 160-row block; here a workgroup of 8 waves
// computes a 256-row x 256-weight-column tile (dma_big.h: both operands
// copied from memory straight into a ring of LDS slots, three 32-K stages in
// flight, weights read with transposing LDS reads, each wave 64 rows x 128
// weight columns, two waves per SIMD).
constexpr int XB_BM = BD_BM;
constexpr int XB_BN = BD_BN;    // weight columns per tile (GEMM-1: 128 of W1 + 128 of W3)
#ifndef MOE_XB_NW
#define MOE_XB_NW 8
#endif
constexpr int XB_NW = MOE_XB_NW;  // waves per workgroup (8: two per SIMD; 4: one per SIMD)
#ifndef MOE_XB_TH
#define MOE_XB_TH 320
#endif
constexpr int XB_TH = MOE_XB_TH; // row count from which an expert uses this kernel
#ifndef MOE_XB_GM
#define MOE_XB_GM 8
#endif
constexpr int XB_GM = MOE_XB_GM; // m-tiles grouped together along the XCD-local order


struct BigTile {
  int e, r0, R, nt;
};

// pre[j] = inclusive prefix of the m-tiles of the experts with at least XB_TH
// rows; returns the total.  All threads call; wave 0 scans.
__device__ int big_prefix(const int32_t* __restrict__ offsets, int e_begin, int ne, int* pre) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int j0 = 0; j0 < ne; j0 += 64) {
      const int j = j0 + lane;
      const int cnt = j < ne ? offsets[e_begin + j + 1] - offsets[e_begin + j] : 0;
      const int nb = cnt >= XB_TH ? (cnt + XB_BM - 1) / XB_BM : 0;
      int x = nb;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      if (j < ne) pre[j] = carry + x;
      carry += __shfl(x, 63);
    }
    if (lane == 0) pre[XG_MAXN] = carry;
  }
  __syncthreads();
  return pre[XG_MAXN];
}

// Tile L of tot_m * ntn: groups of XB_GM m-tiles, inside a group the m-tile
// index runs fastest, so consecutive tiles share weight columns.
__device__ BigTile big_tile_at(int L, const int32_t* __restrict__ offsets, int e_begin, int ne,
                               int ntn, int tot_m, const int* pre) {
  BigTile bt;
  const int mg = L / (XB_GM * ntn);
  const int rem = L - mg * XB_GM * ntn;
  const int gsz = min(XB_GM, tot_m - mg * XB_GM);
  bt.nt = rem / gsz;
  const int mt = mg * XB_GM + (rem - bt.nt * gsz);
  int lo = 0, hi = ne - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] > mt) hi = mid; else lo = mid + 1;
  }
  const int e = e_begin + lo;
  const int jb = mt - (lo ? pre[lo - 1] : 0);
  const int o = offsets[e];
  bt.e = e;
  bt.r0 = o + jb * XB_BM;
  bt.R = min(XB_BM, offsets[e + 1] - o - jb * XB_BM);
  return bt;
}

static_assert(XGThin::NW == 8, "one workgroup size for all streamed tile classes");
// The thin tiles borrow the medium ring: the A stages in its first third, the
// W3 -> W1 accumulator exchange in the other two (half of the pairs each).
// The schedule's prefix sums sit at the start of the ring until the row block
// is known.
constexpr int XG_TPART = DT_LDS / 3 / 16 * 16;
static_assert(2 * gc_lds_elems<XGThin::NW, XGThin::CPL, XGThin::MTMAX>() <= XG_TPART,
              "thin A stages fit a third of the ring");
static_assert(XGThin::XCH / 2 * 4 <= XG_TPART, "half of the thin exchange fits a third of the ring");
static_assert(2 * (XG_MAXN + 1) * 4 <= DT_LDS, "the schedule's prefix sums fit the ring");

// SWIGLU: A = x_packed [*, K = d], B1/B3 = w1/w3 [n][K][N = f], C = h [*, f]
// else:   A = h [*, K = f], B1 = w2 [n][K][N = d], C = y_packed [*, d]
// Segments with fewer than `th` rows; each picks its tile class by row count.
// K and N tails are bounded by the buffer descriptors (gemm_core.h).
template <bool SWIGLU>
__global__ __launch_bounds__(64 * XGThin::NW) void grouped_gemm_bf16(const bf16_t* __restrict__ A,
                                                                     const int32_t* __restrict__ offsets,
                                                                     int e_begin, int e_end,
                                                                     const bf16_t* __restrict__ B1,
                                                                     const bf16_t* __restrict__ B3,
                                                                     int K, int N,
                                                                     bf16_t* __restrict__ C, int th,
                                                                     int mcols, int tcols, RowMap rm,
                                                                     int* __restrict__ xcnt, int ncols2,
                                                                     int mcols2, int tcols2) {
  __shared__ __attribute__((aligned(16))) char ring[DT_LDS];
  // xcnt (or NULL): GEMM-1's workgroup 0 writes the down projection's real
  // workgroups per XCD (ncols2 output columns, mcols2 / tcols2 block widths);
  // the down projection's surplus workgroups leave at once
  if constexpr (SWIGLU) {
    if (xcnt && blockIdx.x == 0 && threadIdx.x < 64)
      xg_xcd_counts(offsets, e_begin, e_end, th, ncols2, mcols2, tcols2, xcnt);
  } else {
    if (xcnt && (int)(blockIdx.x >> 3) >= xcnt[blockIdx.x & 7]) return;
  }
  // GEMM-1 is counted in weight columns: each workgroup streams the columns of W1 and of W3
  const int ncols = SWIGLU ? 2 * N : N;
  RowBlock rb = schedule(offsets, e_begin, e_end, th, ncols, mcols, SWIGLU ? XGThin::COLS : tcols,
                         reinterpret_cast<int*>(ring));
  // values from LDS and the wave index are wave-uniform; say so, so that
  // pointers and buffer descriptors built from them live in scalar registers
  rb.e = __builtin_amdgcn_readfirstlane(rb.e);
  rb.r0 = __builtin_amdgcn_readfirstlane(rb.r0);
  rb.R = __builtin_amdgcn_readfirstlane(rb.R);
  rb.nb = __builtin_amdgcn_readfirstlane(rb.nb);
  rb.cls = __builtin_amdgcn_readfirstlane(rb.cls);
  if (rb.R <= 0) return;   // uniform over the workgroup
  __syncthreads();         // every wave has read the prefix sums before the ring is written
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (rb.cls == 0) {
    stream_block<XGThin, SWIGLU>(A, B1, B3, K, N, C, rb, rm, wave, SWIGLU ? XGThin::COLS : tcols,
                                 reinterpret_cast<bf16_t*>(ring), reinterpret_cast<float*>(ring + XG_TPART),
                                 reinterpret_cast<float*>(ring + 2 * XG_TPART));
    return;
  }
  const DtSlots slots{ring};
  switch ((rb.R + 31) >> 5) {
#define XM_CASE(n)                                                                              \
  case n:                                                                                       \
    dt_block<SWIGLU, n>(A, B1, B3, K, N, C, rb.e, rb.r0, rb.R, rb.nb, mcols, rm.rows, rm.div,    \
                        rm.bytes, rm.scale, wave, slots);                                       \
    break;
    XM_CASE(1) XM_CASE(2) XM_CASE(3) XM_CASE(4) XM_CASE(5)
#undef XM_CASE
    default: break;
  }
}

// SWIGLU: A = x_packed [*, K = d], B1/B3 = w1/w3 [n][K][N = f], C = h [*, f]
// else:   A = h [*, K = f], B1 = w2 [n][K][N = d], C = y_packed [*, d]
// K and N tails are bounded by the buffer descriptors.
//
// The tile order is cut into 8 contiguous ranges, one per XCD (workgroup id
// mod 8 on this part); workgroup (x, q) of the G = gridDim.x takes tiles
// q, q + G/8, ... of range x, so the tiles of a range start in order and
// neighbouring tiles share operands in that XCD's L2.  The host sizes G to
// cover every tile, so each workgroup takes at most one and the hardware
// balances the compute units.
template <bool SWIGLU>
__global__ __launch_bounds__(64 * XB_NW, 1) void grouped_gemm_bf16_big(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets, int e_begin, int e_end,
    const bf16_t* __restrict__ B1, const bf16_t* __restrict__ B3, int K, int N,
    bf16_t* __restrict__ C, int ntn, RowMap rm) {
  __shared__ __attribute__((aligned(16))) char ring[BD_NS * BD_SLOT];
  // the tile table lives in the ring until a tile's K loop starts
  static_assert((XG_MAXN + 1) * 4 <= BD_NS * BD_SLOT, "tile table fits the ring");
  int* pre = reinterpret_cast<int*>(ring);
  const int ne = e_end - e_begin;
  const int tot_m = big_prefix(offsets, e_begin, ne, pre);
  const int TT = tot_m * ntn;
  const int G = gridDim.x;
  int L, step, end;
  if ((G & 7) == 0) {
    const int x = blockIdx.x & 7;
    L = x * (TT >> 3) + min(x, TT & 7);
    end = L + (TT >> 3) + (x < (TT & 7) ? 1 : 0);
    L += blockIdx.x >> 3;
    step = G >> 3;
  } else {
    L = blockIdx.x;
    end = TT;
    step = G;
  }
  for (bool first = true; L < end; L += step, first = false) {
    if (!first) {
      // the previous tile's K loop overwrote the table: every wave must be
      // done with the ring and its epilogue stores retired (loads and stores
      // share the counter that the ring's waits count) before it is rebuilt
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      big_prefix(offsets, e_begin, ne, pre);
    }
    BigTile bt = big_tile_at(L, offsets, e_begin, ne, ntn, tot_m, pre);
    bt.e = __builtin_amdgcn_readfirstlane(bt.e);
    bt.r0 = __builtin_amdgcn_readfirstlane(bt.r0);
    bt.R = __builtin_amdgcn_readfirstlane(bt.R);
    bt.nt = __builtin_amdgcn_readfirstlane(bt.nt);
    __syncthreads();   // every wave has read the table before the copies overwrite it
    bd_tile<SWIGLU, XB_NW>(A, B1, B3, K, N, C, bt.e, bt.r0, bt.R, bt.nt, rm.rows, rm.div, rm.bytes,
                           rm.scale, ring);
  }
}

// ---------------------------------------------------------------------------
// GEMM with a completion signal per output tile: the compute half of the
// pages' GEMM + AllGather workload ("CUCo", Table 4, row "GEMM + AllGather":
// the broadcast starts from the device right after the GEMM, instead of the
// GPU idling until a host-launched collective).  C[M,N] = rnd(A[M,K] B[K,N]),
// bf16, fp32 accumulation, on the 256 x 256 large-tile core; once a tile's
// stores are complete and visible at the requested scope, flags[tile] is set
// to `epoch` with a release store, so a consumer (a tile forwarder, locally
// moe_tile_forward) can move each tile as soon as it exists.  Tiles are
// numbered row-major over ceil(M / 256) x ceil(N / 256); with epochs the flag
// array never needs clearing between calls.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * XB_NW, 1) void gemm_signal_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, bf16_t* __restrict__ C, int M,
    int N, int K, int ntn, uint32_t* __restrict__ flags, uint32_t epoch, int system_scope) {
  __shared__ __attribute__((aligned(16))) char ring[BD_NS * BD_SLOT];
  // Workgroup -> tile as in the grouped kernel: the G = gridDim.x tiles (one
  // workgroup each) are cut into 8 ranges, one per XCD (workgroup id mod 8),
  // and inside a range tiles run in groups of XB_GM m-tiles, m fastest, so
  // the tiles an XCD has in flight share A and B panels in its L2.  The flag
  // and the output keep the row-major tile number tm * ntn + tn.
  const int G = gridDim.x;
  const int L = (G & 7) == 0 ? (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int ntm = G / ntn;
  const int mg = L / (XB_GM * ntn);
  const int rem = L - mg * XB_GM * ntn;
  const int gsz = min(XB_GM, ntm - mg * XB_GM);
  const int tn = rem / gsz;
  const int tm = mg * XB_GM + (rem - tn * gsz);
  const int tile = tm * ntn + tn;
  BigTile bt;
  bt.e = 0;
  bt.r0 = tm * XB_BM;
  bt.R = min(XB_BM, M - bt.r0);
  bt.nt = tn;
  bd_tile<false, XB_NW>(A, B, nullptr, K, N, C, 0, bt.r0, bt.R, bt.nt, nullptr, 1, 0, nullptr, ring);
  // every thread's stores of the tile complete and visible at the scope,
  // then one release store of the flag
  if (system_scope) __threadfence_system();
  else __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (system_scope) __hip_atomic_store(flags + tile, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    else __hip_atomic_store(flags + tile, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

int64_t gemm_signal_tiles(int M, int N) {
  return (int64_t)((M + XB_BM - 1) / XB_BM) * ((N + XB_BN - 1) / XB_BN);
}

hipError_t launch_gemm_signal(int M, int N, int K, const void* A, const void* B, void* C,
                              uint32_t* flags, uint32_t epoch, int system_scope, hipStream_t st) {
  const int ntn = (N + XB_BN - 1) / XB_BN;
  const int64_t tiles = gemm_signal_tiles(M, N);
  hipLaunchKernelGGL(gemm_signal_kernel, dim3((unsigned)tiles), dim3(64 * XB_NW), 0, st,
                     (const bf16_t*)A, (const bf16_t*)B, (bf16_t*)C, M, N, K, ntn, flags, epoch,
                     system_scope);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32: one thread per output element
// ---------------------------------------------------------------------------
template <bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_gemm_f32(const float* __restrict__ A,
                                                        const int32_t* __restrict__ offsets,
                                                        int e_begin, int e_end,
                                                        const float* __restrict__ B1,
                                                        const float* __restrict__ B3, int K, int N,
                                                        float* __restrict__ C,
                                                        const float* __restrict__ rscale) {
  const int64_t p = (int64_t)offsets[e_begin] + blockIdx.x;
  if (p >= offsets[e_end]) return;
  const int n = blockIdx.y * 256 + threadIdx.x;
  if (n >= N) return;
  int lo = e_begin, hi = e_end - 1;  // last e with offsets[e] <= p
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid - 1;
  }
  const int64_t es = (int64_t)lo * K * N;
  const float* a = A + p * K;
  float s1 = 0.f, s3 = 0.f;
  for (int kk = 0; kk < K; ++kk) {
    s1 = fmaf(a[kk], B1[es + (int64_t)kk * N + n], s1);
    if (SWIGLU) s3 = fmaf(a[kk], B3[es + (int64_t)kk * N + n], s3);
  }
  C[p * N + n] = SWIGLU ? s1 / (1.0f + expf(-s1)) * s3 : (rscale ? s1 * rscale[p] : s1);
}

// Compute units of the current device.
static int big_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int* c = dev < 64 ? &cache[dev] : nullptr;
  if (c && *c) return *c;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (c) *c = n;
  return n;
}

// the down projection's real workgroups per XCD (8 ints), written by GEMM-1
size_t expert_gemm_ws_bytes(const Prob& p) { return p.dtype == 1 ? 256 : 0; }

hipError_t launch_expert_gemm(const Prob& p, const void* x_packed, const int32_t* offsets,
                              const void* w1, const void* w3, const void* w2, void* h,
                              void* y_packed, void* ws, int e_begin, int e_end, hipStream_t st,
                              const int32_t* perm, const float* rscale) {
  if (p.rows_max == 0 || e_end <= e_begin) return hipSuccess;
  if (p.dtype == 1) {
    // with perm, x_packed is x itself and GEMM-1 reads row perm[p] / k for packed row p
    const RowMap rm1 = perm ? RowMap{perm, p.k, (uint32_t)((int64_t)p.T * p.d * 2)} : RowMap{nullptr, 1, 0};
    const RowMap rm2{nullptr, 1, 0, rscale};
    // Dense-like routing (the mean segment reaches XB_TH rows, or every
    // segment does in the padded layout): experts with >= XB_TH rows go to the
    // 256 x 256 kernel.  Otherwise every segment, however long, streams
    // through the thin/medium tiles in one launch: a few long segments of a
    // skewed routing balance better there than in a second, serialized
    // launch (4096-token Zipf-skewed routing: 3.07 against 3.52 ms), and a
    // sparse routing skips the large-tile launches altogether.
    const bool dense_like = p.seg_rows ? p.seg_rows >= XB_TH : (int64_t)p.T * p.k >= (int64_t)XB_TH * p.E;
    const bool big = dense_like && p.T >= XB_TH;
    const int th = big ? XB_TH : INT32_MAX;
    const int ne = e_end - e_begin;
    // Medium column blocks: when the expected segment is a single medium row
    // block, pick the width (512, 448 or 384 weight columns) whose block count
    // fills the last round of workgroups best (one workgroup per compute
    // unit); e.g. 7168 output columns x 32 experts: 448 gives exactly 2 rounds
    // where 512 gives 1.75.
    const int cus = big_cus();
    const int64_t mean_rows = p.seg_rows ? p.seg_rows : (int64_t)p.T * p.k / std::max(1, p.E);
    auto pick_mcols = [&](int ncols) {
      if (mean_rows <= XG_THIN_MAX || mean_rows > XM_BM) return XM_COLS;
      int best = XM_COLS;
      double best_fill = 0.0;
      for (int cw = XM_COLS; cw >= 384; cw -= 64) {
        const int64_t nb = (int64_t)ne * ((ncols + cw - 1) / cw);
        const double fill = (double)nb / (double)(((nb + cus - 1) / cus) * cus);
        if (fill > best_fill + 1e-9) { best_fill = fill; best = cw; }
      }
      return best;
    };
    // Thin column blocks of the down projection: when the expected segment is
    // thin, the width (512, 448 or 384 output columns; the last waves of a
    // narrower block idle) whose block count fills the last round best, e.g.
    // 7168 columns x 32 experts: 448 gives exactly 2 rounds where 512 gives
    // 1.75.  GEMM-1 keeps 512 (its W1 and W3 halves pair 256 h columns).
    auto pick_tcols = [&](int ncols) {
      if (mean_rows > XG_THIN_MAX) return XGThin::COLS;
      int best = XGThin::COLS;
      double best_fill = 0.0;
      for (int cw = XGThin::COLS; cw >= 384; cw -= XGThin::OW) {
        const int64_t nb = (int64_t)ne * ((ncols + cw - 1) / cw);
        const double fill = (double)nb / (double)(((nb + cus - 1) / cus) * cus);
        if (fill > best_fill + 1e-9) { best_fill = fill; best = cw; }
      }
      return best;
    };
    // Streaming grid: the total work W of schedule() (units of XG_WUNIT
    // columns).  A thin expert is one row block of nt blocks of weight wt =
    // tcols / XG_WUNIT, a medium one ceil(cnt / BM) row blocks of nw blocks of
    // weight wm; a streamed expert has fewer than min(T + 1, th) rows, and the
    // local row counts add up to at most rows_max.  Each XCD's blocks start in
    // a window of ceil(W / 8) at least min(wt, wm) apart.
    const int64_t rbmax = (std::min<int64_t>(p.T, (int64_t)th - 1) + XM_BM - 1) / XM_BM;
    auto grid = [&](int ncols, int mcols, int tcols) {
      const int64_t wm = mcols / XG_WUNIT;
      const int64_t wt = tcols / XG_WUNIT;
      const int64_t nt = (ncols + tcols - 1) / tcols;
      const int64_t nw = (ncols + mcols - 1) / mcols;
      const int64_t per_e = std::max<int64_t>(wt * nt, wm * nw);
      const int64_t w_rows = ne * per_e + wm * ((p.rows_max * nw + XM_BM - 1) / XM_BM);
      const int64_t w_exp = ne * std::max<int64_t>(wt * nt, wm * rbmax * nw);
      const int64_t w = std::min(w_rows, w_exp);
      const int64_t wmin = std::min<int64_t>(wt, wm);
      return (unsigned)(8 * ((((w + 7) / 8) + wmin - 1) / wmin));
    };
    const int mc1 = pick_mcols(2 * p.f), mc2 = pick_mcols(p.d);
    const int tc1 = XGThin::COLS, tc2 = pick_tcols(p.d);
    // Large-tile grid (dense-like routing only): its tiles, the sum over
    // experts with n_e >= XB_TH of ceil(n_e / BM) <= rows_max / BM +
    // min(ne, rows_max / XB_TH) m-tiles, times ntn, each with its own
    // workgroup.
    const int64_t bblocks = (p.rows_max + XB_BM - 1) / XB_BM + std::min<int64_t>(ne, p.rows_max / XB_TH);
    auto big_grid = [&](int ntn) { return (unsigned)(bblocks * ntn); };
    hipError_t e;
    if (big) {
      const int ntn = (p.f + 127) / 128;
      hipLaunchKernelGGL(grouped_gemm_bf16_big<true>, dim3(big_grid(ntn)), dim3(64 * XB_NW), 0, st,
                         (const bf16_t*)x_packed, offsets, e_begin, e_end, (const bf16_t*)w1,
                         (const bf16_t*)w3, p.d, p.f, (bf16_t*)h, ntn, rm1);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    int* xcnt = reinterpret_cast<int*>(ws);
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3(grid(2 * p.f, mc1, tc1)), dim3(64 * XGThin::NW), 0, st,
                       (const bf16_t*)x_packed, offsets, e_begin, e_end, (const bf16_t*)w1,
                       (const bf16_t*)w3, p.d, p.f, (bf16_t*)h, th, mc1, tc1, rm1, xcnt, p.d, mc2, tc2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (big) {
      const int ntn = (p.d + 255) / 256;
      hipLaunchKernelGGL(grouped_gemm_bf16_big<false>, dim3(big_grid(ntn)), dim3(64 * XB_NW), 0, st,
                         (const bf16_t*)h, offsets, e_begin, e_end, (const bf16_t*)w2,
                         (const bf16_t*)nullptr, p.f, p.d, (bf16_t*)y_packed, ntn, rm2);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3(grid(p.d, mc2, tc2)), dim3(64 * XGThin::NW), 0, st,
                       (const bf16_t*)h, offsets, e_begin, e_end, (const bf16_t*)w2,
                       (const bf16_t*)nullptr, p.f, p.d, (bf16_t*)y_packed, th, mc2, tc2, rm2, xcnt,
                       0, 0, 0);
    return hipGetLastError();
  }
  dim3 g1((unsigned)p.rows_max, (p.f + 255) / 256);
  hipLaunchKernelGGL(grouped_gemm_f32<true>, g1, dim3(256), 0, st, (const float*)x_packed, offsets,
                     e_begin, e_end, (const float*)w1, (const float*)w3, p.d, p.f, (float*)h,
                     (const float*)nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)p.rows_max, (p.d + 255) / 256);
  hipLaunchKernelGGL(grouped_gemm_f32<false>, g2, dim3(256), 0, st, (const float*)h, offsets,
                     e_begin, e_end, (const float*)w2, (const float*)nullptr, p.f, p.d,
                     (float*)y_packed, rscale);
  return hipGetLastError();
}

}  // namespace moe
