// Local expert compute: SwiGLU expert FFNs as grouped GEMMs over the
// expert-contiguous, unpadded segments produced by dispatch (the "local
// compute" of the DeepSeek-V3 MoE layer in "CUCo: An Agentic Framework for
// Compute and Communication Co-design", Abstract and Table 4).
//
//   GEMM-1:  h[R]        = rnd(SiLU(x_packed[R] W1_e) * (x_packed[R] W3_e))
//   GEMM-2:  y_packed[R] = rnd(h[R] W2_e)
//
// bf16 path (grouped_gemm_bf16).  A workgroup owns one row block of one
// expert (up to 160 rows) and one column block; every weight byte of that
// column block is streamed from HBM exactly once per row block, which is the
// bound for the segment sizes of a sparse MoE layer (about 4..160 rows per
// expert).  8 waves (2 per SIMD) share the A rows through LDS; each wave
// streams its own weight columns (2 per lane) straight from HBM into
// registers and transposes them there into MFMA B fragments (mfma_tile.h,
// gemm_core.h).  The row-block schedule is derived on the
// device from `offsets` in the workgroup prologue, so the number of local
// assignments never travels to the host; the grid is sized for the worst case
// and surplus workgroups exit after the prologue.
//
// GEMM-1 pairs W1 and W3: the lower half of the waves streams W1 columns and
// the upper half the same W3 columns (each wave reads one weight matrix, so its
// buffer descriptor is wave-uniform); after the K loop the upper half passes
// its products to the lower half through LDS, which applies SiLU(x.W1)*(x.W3)
// and writes h.  The intermediate products never reach memory.
//
// fp32 path (grouped_gemm_f32): one thread per output element, for the small
// fp32 problems only.
#include <stdint.h>

#include "common.h"
#include "kernels.h"
#include "gemm_core.h"

namespace moe {

constexpr int XG_MTMAX = 10;              // m-tiles per row block
constexpr int XG_BM = 16 * XG_MTMAX;      // rows per row block
// Build-time tile shape (a tuning choice, not a behaviour switch).
#ifndef MOE_XG_NW
#define MOE_XG_NW 8
#endif
#ifndef MOE_XG_CPL
#define MOE_XG_CPL 2
#endif
constexpr int XG_NW = MOE_XG_NW;          // waves per workgroup
constexpr int XG_CPL = MOE_XG_CPL;        // weight columns per lane (2: 4-byte loads, 4: 8-byte)
constexpr int XG_HW = 256 / XG_NW;        // h columns per wave in GEMM-1 (128 per workgroup, W1 and W3 halves)
constexpr int XG_OW = 256 / XG_NW;        // output columns per wave in GEMM-2 (256 per workgroup)
static_assert(XG_HW == 16 * XG_CPL && XG_OW == 16 * XG_CPL, "tile shape");
constexpr int XG_MAXN = 1024;             // max local experts

// Row block of this workgroup: expert e, rows [r0, r0 + R), column block nb.
struct RowBlock {
  int e, r0, R, nb;
};

// Schedule from `offsets` (computed by every workgroup, a few hundred cycles):
// expert e in [e_begin, e_end) has ceil(count_e / XG_BM) row blocks, each with
// nblk_n column blocks.  The G = (total row blocks) * nblk_n live workgroups
// are renumbered so that every XCD (workgroup id mod 8 on this part) receives
// a contiguous range of (row block, column block) pairs: all column blocks of
// one row block then share one L2 for their A rows.  R = 0 means "exit".
__device__ RowBlock schedule(const int32_t* __restrict__ offsets, int e_begin, int e_end,
                             int nblk_n, int th, int* pre) {
  const int ne = e_end - e_begin;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int j0 = 0; j0 < ne; j0 += 64) {
      const int j = j0 + lane;
      const int cnt = j < ne ? offsets[e_begin + j + 1] - offsets[e_begin + j] : 0;
      const int nb = cnt < th ? (cnt + XG_BM - 1) / XG_BM : 0;
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
  RowBlock rb{0, 0, 0, 0};
  const int G = pre[XG_MAXN] * nblk_n;
  const int b = blockIdx.x;
  if (b >= G) return rb;
  const int xcd = b & 7, q = b >> 3;
  const int L = xcd * (G >> 3) + min(xcd, G & 7) + q;
  const int mb = L / nblk_n;
  rb.nb = L - mb * nblk_n;
  int lo = 0, hi = ne - 1;  // first j with pre[j] > mb
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] > mb) hi = mid; else lo = mid + 1;
  }
  const int e = e_begin + lo;
  const int jb = mb - (lo ? pre[lo - 1] : 0);
  const int o = offsets[e];
  const int cnt = offsets[e + 1] - o;
  rb.e = e;
  rb.r0 = o + jb * XG_BM;
  rb.R = min(XG_BM, cnt - jb * XG_BM);
  return rb;
}

// LDS bf16 elements of the streaming kernel: the A stage buffers, reused after
// the K loop for the W3 -> W1 accumulator exchange of GEMM-1.
constexpr int XG_XCH = (XG_NW / 2) * XG_MTMAX * XG_CPL * 4 * 64;  // floats exchanged
constexpr int XG_LDS = gc_lds_elems<XG_NW, XG_CPL, XG_MTMAX>() > 2 * XG_XCH
                           ? gc_lds_elems<XG_NW, XG_CPL, XG_MTMAX>() : 2 * XG_XCH;

template <bool SWIGLU, int MT>
__device__ __forceinline__ void gemm_body(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bl,
                                          int K, int N, int col, bf16_t* __restrict__ C,
                                          const RowBlock& rb, bf16_t* As) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  GemmArgs ga{A + (int64_t)rb.r0 * K, K, rb.R, Bl, N, 0, K, N, col};
  f32x4 acc[MT][XG_CPL];
  gemm_mainloop<XG_NW, XG_CPL, MT>(ga, As, acc);

  // GEMM-1: waves of the upper half hold the x.W3 products of the columns the
  // lower half holds x.W1 for; they hand them over through LDS.
  bool store_wave = true;
  float* xch = reinterpret_cast<float*>(As);
  if (SWIGLU) {
    store_wave = wave < XG_NW / 2;
    const int pair = wave % (XG_NW / 2);
    float* slot = xch + pair * (XG_MTMAX * XG_CPL * 4 * 64) + lane;
    if (!store_wave) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < XG_CPL; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) slot[((mt * XG_CPL + c) * 4 + r) * 64] = acc[mt][c][r];
    }
    __syncthreads();
    if (store_wave) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < XG_CPL; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = acc[mt][c][r];
            const float b = slot[((mt * XG_CPL + c) * 4 + r) * 64];
            acc[mt][c][r] = a / (1.0f + expf(-a)) * b;
          }
    }
  }
  // epilogue: lane holds XG_CPL consecutive columns (c) of rows 16 mt + 4 g + r
  if (!store_wave || col >= N) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mt + 4 * g + r;
      if (row < rb.R) {
        bf16_t* dst = C + (int64_t)(rb.r0 + row) * N + col;
        if (XG_CPL == 2) {
          *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[mt][0][r], acc[mt][1][r]);
        } else {
          *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(acc[mt][0][r], acc[mt][1][r]),
                                                 pack_bf16x2(acc[mt][XG_CPL - 2][r], acc[mt][XG_CPL - 1][r])};
        }
      }
    }
  }
}

// SWIGLU: A = x_packed [*, K = d], B1/B3 = w1/w3 [n][K][N = f], C = h [*, f]; 128 columns per WG.
// else:   A = h [*, K = f], B1 = w2 [n][K][N = d], C = y_packed [*, d];  256 columns per WG.
// K and N tails are bounded by the buffer descriptors (gemm_core.h).
template <bool SWIGLU>
__global__ __launch_bounds__(64 * XG_NW) void grouped_gemm_bf16(const bf16_t* __restrict__ A,
                                                                 const int32_t* __restrict__ offsets,
                                                                 int e_begin, int e_end,
                                                                 const bf16_t* __restrict__ B1,
                                                                 const bf16_t* __restrict__ B3,
                                                                 int K, int N,
                                                                 bf16_t* __restrict__ C,
                                                                 int nblk_n, int th) {
  __shared__ __attribute__((aligned(16))) bf16_t As[XG_LDS];
  __shared__ int pre[XG_MAXN + 1];
  RowBlock rb = schedule(offsets, e_begin, e_end, nblk_n, th, pre);
  // values from LDS and the wave index are wave-uniform; say so, so that
  // pointers and buffer descriptors built from them live in scalar registers
  rb.e = __builtin_amdgcn_readfirstlane(rb.e);
  rb.r0 = __builtin_amdgcn_readfirstlane(rb.r0);
  rb.R = __builtin_amdgcn_readfirstlane(rb.R);
  rb.nb = __builtin_amdgcn_readfirstlane(rb.nb);
  if (rb.R <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = threadIdx.x & 15;
  int col;
  const bf16_t* Bl;
  const int64_t estride = (int64_t)K * N;
  if (SWIGLU) {  // lower half of the waves streams W1, upper half the same columns of W3
    col = rb.nb * 128 + (wave % (XG_NW / 2)) * XG_HW + XG_CPL * i;
    Bl = ((wave < XG_NW / 2) ? B1 : B3) + rb.e * estride;
  } else {       // output columns per wave
    col = rb.nb * 256 + wave * XG_OW + XG_CPL * i;
    Bl = B1 + rb.e * estride;
  }
  const int mt = (rb.R + 15) >> 4;
  switch (mt) {
#define XG_CASE(n) \
  case n: gemm_body<SWIGLU, n>(A, Bl, K, N, col, C, rb, As); break;
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
// computes a 256-row x 256-weight-column tile, each wave 128 x 64
// (accumulators in AGPRs, two waves per SIMD).  Per 64-K stage every thread
// loads 4 A vectors and one 8 x 4 weight block with buffer loads (fixed lane
// offsets, scalar stage offsets); the next stage is in flight while the
// current one is multiplied; the weight block is transposed in registers and
// both are written into the other LDS buffer.  Weight columns are placed in
// LDS so that each lane's 4 n-tiles are 4 consecutive output columns (8-byte
// stores), and for GEMM-1 so that W1 and W3 of one column meet in lanes i and
// i ^ 8.  The lower four waves load W1 blocks, the upper four W3 blocks, so
// every buffer descriptor is wave-uniform.
constexpr int XB_BM = 256;
constexpr int XB_BN = 256;      // weight columns per tile (GEMM-1: 128 of W1 + 128 of W3)
constexpr int XB_NW = 8;        // waves per workgroup
constexpr int XB_TH = 320;      // row count from which an expert uses this kernel
#ifndef MOE_XB_GM
#define MOE_XB_GM 8
#endif
constexpr int XB_GM = MOE_XB_GM; // m-tiles grouped together along the XCD-local order

struct BigTile {
  int e, r0, R, nt;
};

__device__ BigTile schedule_big(const int32_t* __restrict__ offsets, int e_begin, int e_end,
                                int ntn, int* pre) {
  const int ne = e_end - e_begin;
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
  BigTile bt{0, 0, 0, 0};
  const int tot_m = pre[XG_MAXN];
  const int G = tot_m * ntn;
  const int b = blockIdx.x;
  if (b >= G) return bt;
  const int xcd = b & 7, q = b >> 3;
  const int L = xcd * (G >> 3) + min(xcd, G & 7) + q;
  // groups of XB_GM m-tiles; inside a group the m-tile index runs fastest
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

struct BigRegs {
  u32x4 a[4];
  u32x2 b[8];
};

// Per-thread fixed state of the large-tile loop: buffer descriptors (wave
// uniform) and byte offsets that do not change with K.
struct BigCtx {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t va[4];   // A rows (t >> 3) + 64 j, 16-byte chunk t & 7
  uint32_t vb;      // B block: k rows 8 kb .. 8 kb + 7 (via scalar offsets), 4 columns
  uint32_t ldb2;    // B row bytes
  int kb, nb;       // block coordinates inside the 64 x 256 weight stage (nb: 4-column group)
};

__device__ __forceinline__ void big_issue(BigRegs& R, const BigCtx& c, int k0) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    R.a[j] = __builtin_amdgcn_raw_buffer_load_b128(c.ra, c.va[j], (uint32_t)(k0 * 2), 0);
#pragma unroll
  for (int r = 0; r < 8; ++r)
    R.b[r] = __builtin_amdgcn_raw_buffer_load_b64(c.rb, c.vb, (uint32_t)(k0 + r) * c.ldb2, 0);
}

// LDS row (within the 256-row B^T tile) of weight column c (0..3) of 4-column
// group nb.  GEMM-1: nb 0..31 are W1 columns 4 nb .., nb 32..63 the same W3
// columns; wave slab wn holds h columns 32 wn .. 32 wn + 31, lane i (< 8) of
// n-tile t the h column 32 wn + 4 i + t, lane i + 8 its W3 twin.  GEMM-2: wave
// slab wn holds weight columns 64 wn .. 64 wn + 63, lane i of n-tile t column
// 64 wn + 4 i + t.
template <bool SWIGLU>
__device__ __forceinline__ int big_brow(int nb, int c) {
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

template <bool SWIGLU>
__device__ __forceinline__ void big_store(const BigRegs& R, const BigCtx& c, bf16_t* As, bf16_t* Bs) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<u32x4*>(As + ((t >> 3) + 64 * j) * GC_LDA + 8 * (t & 7)) = R.a[j];
#pragma unroll
  for (int col = 0; col < 4; ++col) {
    const uint32_t sel = (col & 1) ? 0x07060302u : 0x05040100u;
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = __builtin_amdgcn_perm(R.b[2 * q + 1][col >> 1], R.b[2 * q][col >> 1], sel);
    *reinterpret_cast<u32x4*>(Bs + big_brow<SWIGLU>(c.nb, col) * GC_LDA + 8 * c.kb) = v;
  }
}

__device__ __forceinline__ void big_compute(const bf16_t* As, const bf16_t* Bs, int wm, int wn,
                                            f32x4 (&acc)[8][4]) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const bf16_t* a0 = As + (128 * wm + i) * GC_LDA + 8 * g;
  const bf16_t* b0 = Bs + (64 * wn + i) * GC_LDA + 8 * g;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    bf16x8 bf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      bf[t] = *reinterpret_cast<const bf16x8*>(b0 + 16 * t * GC_LDA + 32 * sub);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(a0 + 16 * mt * GC_LDA + 32 * sub);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = mfma16(af, bf[t], acc[mt][t]);
    }
  }
}

// SWIGLU: A = x_packed [*, K = d], B1/B3 = w1/w3 [n][K][N = f], C = h [*, f]
// else:   A = h [*, K = f], B1 = w2 [n][K][N = d], C = y_packed [*, d]
// K and N tails are bounded by the buffer descriptors.
template <bool SWIGLU>
__global__ __launch_bounds__(64 * XB_NW, 1) void grouped_gemm_bf16_big(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets, int e_begin, int e_end,
    const bf16_t* __restrict__ B1, const bf16_t* __restrict__ B3, int K, int N,
    bf16_t* __restrict__ C, int ntn) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][XB_BM * GC_LDA];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][XB_BN * GC_LDA];
  __shared__ int pre[XG_MAXN + 1];
  BigTile bt = schedule_big(offsets, e_begin, e_end, ntn, pre);
  bt.e = __builtin_amdgcn_readfirstlane(bt.e);
  bt.r0 = __builtin_amdgcn_readfirstlane(bt.r0);
  bt.R = __builtin_amdgcn_readfirstlane(bt.R);
  bt.nt = __builtin_amdgcn_readfirstlane(bt.nt);
  if (bt.R <= 0) return;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t estride = (int64_t)K * N;
  BigCtx c;
  const bf16_t* Bp;
  int bcol;
  if (SWIGLU) {  // waves 0-3 load W1 blocks, waves 4-7 the same W3 blocks
    const int u = t & 255;
    c.kb = u >> 5;
    c.nb = (u & 31) + (wave >= 4 ? 32 : 0);
    Bp = (wave < 4 ? B1 : B3) + bt.e * estride;
    bcol = bt.nt * 128 + 4 * (u & 31);
  } else {
    c.kb = t >> 6;
    c.nb = t & 63;
    Bp = B1 + bt.e * estride;
    bcol = bt.nt * 256 + 4 * c.nb;
  }
  const bf16_t* Ablk = A + (int64_t)bt.r0 * K;
  c.ra = gc_rsrc(Ablk, (uint32_t)((int64_t)bt.R * K * 2));
  c.rb = gc_rsrc(Bp, (uint32_t)(estride * 2));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = min((t >> 3) + 64 * j, bt.R - 1);
    c.va[j] = (uint32_t)(((int64_t)r * K + 8 * (t & 7)) * 2);
  }
  c.vb = bcol < N ? (uint32_t)(((int64_t)(8 * c.kb) * N + bcol) * 2) : GC_OOR;
  c.ldb2 = (uint32_t)(N * 2);

  const int wm = wave & 1, wn = wave >> 1;
  f32x4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = (K + GC_KS - 1) / GC_KS;
  BigRegs R;
  big_issue(R, c, 0);
  big_store<SWIGLU>(R, c, As[0], Bs[0]);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    if (st + 1 < nst) big_issue(R, c, (st + 1) * GC_KS);
    __builtin_amdgcn_sched_barrier(0);
    big_compute(As[cur], Bs[cur], wm, wn, acc);
    if (st + 1 < nst) big_store<SWIGLU>(R, c, As[cur ^ 1], Bs[cur ^ 1]);
    __syncthreads();
  }
  // epilogue: lane (i, g) of wave (wm, wn) holds, for n-tile q, rows
  // 128 wm + 16 mt + 4 g + r of output column base + 4 (i or i & 7) + q
  const int lane = t & 63;
  const int i = lane & 15, g = lane >> 4;
  int ocol;
  if (SWIGLU) ocol = bt.nt * 128 + 32 * wn + 4 * (i & 7);
  else ocol = bt.nt * 256 + 64 * wn + 4 * i;
  const bool store_lane = (SWIGLU ? (i < 8) : true) && ocol < N;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = acc[mt][q][r];
        if (SWIGLU) {
          const float b = __shfl_xor(a, 8);
          o[q] = a / (1.0f + expf(-a)) * b;
        } else {
          o[q] = a;
        }
      }
      const int row = 128 * wm + 16 * mt + 4 * g + r;
      if (store_lane && row < bt.R)
        *reinterpret_cast<u32x2*>(C + (int64_t)(bt.r0 + row) * N + ocol) =
            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  }
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
                                                        float* __restrict__ C) {
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
  C[p * N + n] = SWIGLU ? s1 / (1.0f + expf(-s1)) * s3 : s1;
}

size_t expert_gemm_ws_bytes(const Prob&) { return 0; }

hipError_t launch_expert_gemm(const Prob& p, const void* x_packed, const int32_t* offsets,
                              const void* w1, const void* w3, const void* w2, void* h,
                              void* y_packed, void*, int e_begin, int e_end, hipStream_t st) {
  if (p.rows_max == 0 || e_end <= e_begin) return hipSuccess;
  if (p.dtype == 1) {
    // experts with >= XB_TH rows go to the 256 x 256 kernel; no expert can
    // exceed T rows (top-k picks distinct experts), so small T never needs it
    const bool big = p.T >= XB_TH;
    const int th = big ? XB_TH : INT32_MAX;
    const int64_t mblocks = (p.rows_max + XG_BM - 1) / XG_BM + (e_end - e_begin);
    const int64_t bblocks = (p.rows_max + XB_BM - 1) / XB_BM + (e_end - e_begin);
    hipError_t e;
    // GEMM-1 (SwiGLU)
    if (big) {
      const int ntn = (p.f + 127) / 128;
      hipLaunchKernelGGL(grouped_gemm_bf16_big<true>, dim3((unsigned)(bblocks * ntn)), dim3(64 * XB_NW), 0, st,
                         (const bf16_t*)x_packed, offsets, e_begin, e_end, (const bf16_t*)w1,
                         (const bf16_t*)w3, p.d, p.f, (bf16_t*)h, ntn);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int nb1 = (p.f + 127) / 128;
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3((unsigned)(mblocks * nb1)), dim3(64 * XG_NW), 0, st,
                       (const bf16_t*)x_packed, offsets, e_begin, e_end, (const bf16_t*)w1,
                       (const bf16_t*)w3, p.d, p.f, (bf16_t*)h, nb1, th);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // GEMM-2 (down projection)
    if (big) {
      const int ntn = (p.d + 255) / 256;
      hipLaunchKernelGGL(grouped_gemm_bf16_big<false>, dim3((unsigned)(bblocks * ntn)), dim3(64 * XB_NW), 0, st, (const bf16_t*)h,
                         offsets, e_begin, e_end, (const bf16_t*)w2, (const bf16_t*)nullptr, p.f,
                         p.d, (bf16_t*)y_packed, ntn);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int nb2 = (p.d + 255) / 256;
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3((unsigned)(mblocks * nb2)), dim3(64 * XG_NW), 0, st,
                       (const bf16_t*)h, offsets, e_begin, e_end, (const bf16_t*)w2,
                       (const bf16_t*)nullptr, p.f, p.d, (bf16_t*)y_packed, nb2, th);
    return hipGetLastError();
  }
  dim3 g1((unsigned)p.rows_max, (p.f + 255) / 256);
  hipLaunchKernelGGL(grouped_gemm_f32<true>, g1, dim3(256), 0, st, (const float*)x_packed, offsets,
                     e_begin, e_end, (const float*)w1, (const float*)w3, p.d, p.f, (float*)h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)p.rows_max, (p.d + 255) / 256);
  hipLaunchKernelGGL(grouped_gemm_f32<false>, g2, dim3(256), 0, st, (const float*)h, offsets,
                     e_begin, e_end, (const float*)w2, (const float*)nullptr, p.f, p.d,
                     (float*)y_packed);
  return hipGetLastError();
}

}  // namespace moe
