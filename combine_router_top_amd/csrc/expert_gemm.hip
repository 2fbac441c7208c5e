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
// expert).  A rows are staged through LDS (shared by the 4 waves); weights go
// straight from HBM into registers and are transposed there into MFMA B
// fragments (see mfma_tile.h).  The row-block schedule is derived on the
// device from `offsets` in the workgroup prologue, so the number of local
// assignments never travels to the host; the grid is sized for the worst case
// and surplus workgroups exit after the prologue.
//
// GEMM-1 pairs W1 and W3: in each 16-lane group, lanes 0..7 read W1 columns
// and lanes 8..15 the same W3 columns, so the epilogue combines a lane with
// lane ^ 8 and writes h directly; the two intermediate products never reach
// memory.
//
// fp32 path (grouped_gemm_f32): one thread per output element, for the small
// fp32 problems only.
#include "common.h"
#include "kernels.h"
#include "gemm_core.h"

namespace moe {

constexpr int XG_MTMAX = 10;              // m-tiles per row block
constexpr int XG_BM = 16 * XG_MTMAX;      // rows per row block
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
                             int nblk_n, int* pre) {
  const int ne = e_end - e_begin;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int j0 = 0; j0 < ne; j0 += 64) {
      const int j = j0 + lane;
      const int cnt = j < ne ? offsets[e_begin + j + 1] - offsets[e_begin + j] : 0;
      const int nb = (cnt + XG_BM - 1) / XG_BM;
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

template <bool SWIGLU, int MT, bool CHECK>
__device__ __forceinline__ void gemm_body(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bl,
                                          int K, int N, int col, bf16_t* __restrict__ C,
                                          const RowBlock& rb, bf16_t* As) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  GemmArgs ga{A + (int64_t)rb.r0 * K, K, rb.R, Bl, N, 0, K, N, col};
  f32x4 acc[MT][4];
  gemm_mainloop<MT, CHECK>(ga, As, acc);

  // epilogue: lane holds 4 consecutive columns (c = 0..3) of rows 16 mt + 4 g + r
  const bool store_lane = SWIGLU ? (i < 8) : true;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float a = acc[mt][c][r];
        if (SWIGLU) {
          const float b = __shfl_xor(a, 8);  // the W3 product of the same element
          o[c] = a / (1.0f + expf(-a)) * b;
        } else {
          o[c] = a;
        }
      }
      const int row = 16 * mt + 4 * g + r;
      if (store_lane && row < rb.R && col < N) {
        u32x2 pk = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(C + (int64_t)(rb.r0 + row) * N + col) = pk;
      }
    }
  }
}

// SWIGLU: A = x_packed [*, K = d], B1/B3 = w1/w3 [n][K][N = f], C = h [*, f]; 128 columns per WG.
// else:   A = h [*, K = f], B1 = w2 [n][K][N = d], C = y_packed [*, d];  256 columns per WG.
// CHECK:  bounds checks on K and N (needed unless K % 64 == 0 and the column
//         blocks tile N exactly).
template <bool SWIGLU, bool CHECK>
__global__ __launch_bounds__(256) void grouped_gemm_bf16(const bf16_t* __restrict__ A,
                                                         const int32_t* __restrict__ offsets,
                                                         int e_begin, int e_end,
                                                         const bf16_t* __restrict__ B1,
                                                         const bf16_t* __restrict__ B3, int K,
                                                         int N, bf16_t* __restrict__ C,
                                                         int nblk_n) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2 * XG_BM * GC_LDA];
  __shared__ int pre[XG_MAXN + 1];
  const RowBlock rb = schedule(offsets, e_begin, e_end, nblk_n, pre);
  if (rb.R <= 0) return;
  const int wave = threadIdx.x >> 6;
  const int i = threadIdx.x & 15;
  int col;
  const bf16_t* Bl;
  const int64_t estride = (int64_t)K * N;
  if (SWIGLU) {
    col = rb.nb * 128 + wave * 32 + 4 * (i & 7);
    Bl = ((i < 8) ? B1 : B3) + rb.e * estride;
  } else {
    col = rb.nb * 256 + wave * 64 + 4 * i;
    Bl = B1 + rb.e * estride;
  }
  const int mt = (rb.R + 15) >> 4;
  switch (mt) {
#define XG_CASE(n) \
  case n: gemm_body<SWIGLU, n, CHECK>(A, Bl, K, N, col, C, rb, As); break;
    XG_CASE(1) XG_CASE(2) XG_CASE(3) XG_CASE(4) XG_CASE(5)
    XG_CASE(6) XG_CASE(7) XG_CASE(8) XG_CASE(9) XG_CASE(10)
#undef XG_CASE
    default: break;
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
    const int64_t mblocks = (p.rows_max + XG_BM - 1) / XG_BM + (e_end - e_begin);
    const int nb1 = (p.f + 127) / 128;
    const bool chk1 = (p.d % GC_KS) != 0 || (p.f % 128) != 0;
    auto k1 = chk1 ? grouped_gemm_bf16<true, true> : grouped_gemm_bf16<true, false>;
    hipLaunchKernelGGL(k1, dim3((unsigned)(mblocks * nb1)), dim3(256), 0, st,
                       (const bf16_t*)x_packed, offsets, e_begin, e_end, (const bf16_t*)w1,
                       (const bf16_t*)w3, p.d, p.f, (bf16_t*)h, nb1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nb2 = (p.d + 255) / 256;
    const bool chk2 = (p.f % GC_KS) != 0 || (p.d % 256) != 0;
    auto k2 = chk2 ? grouped_gemm_bf16<false, true> : grouped_gemm_bf16<false, false>;
    hipLaunchKernelGGL(k2, dim3((unsigned)(mblocks * nb2)), dim3(256), 0, st,
                       (const bf16_t*)h, offsets, e_begin, e_end, (const bf16_t*)w2,
                       (const bf16_t*)nullptr, p.f, p.d, (bf16_t*)y_packed, nb2);
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
