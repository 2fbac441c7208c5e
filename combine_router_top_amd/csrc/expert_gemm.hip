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
#include "mfma_tile.h"

namespace moe {

constexpr int XG_MTMAX = 10;              // m-tiles per row block
constexpr int XG_BM = 16 * XG_MTMAX;      // rows per row block
constexpr int XG_KS = 64;                 // K per LDS stage
constexpr int XG_LDA = XG_KS + 8;         // LDS row stride (bf16), 16-byte pad
constexpr int XG_MAXN = 1024;             // max local experts

// Row block of this workgroup: expert e, rows [r0, r0 + R).
struct RowBlock {
  int e, r0, R;
};

// Wave 0 scans the per-expert block counts (ceil(count / XG_BM)) over
// [e_begin, e_end) and locates row block `mb`.  R = 0 when mb is past the end.
__device__ RowBlock find_row_block(const int32_t* __restrict__ offsets, int e_begin, int e_end,
                                   int mb, int* sh) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    if (lane == 0) {
      sh[0] = -1;
      sh[1] = 0;
      sh[2] = 0;
    }
    for (int e0 = e_begin; e0 < e_end; e0 += 64) {
      const int e = e0 + lane;
      int cnt = 0, o = 0;
      if (e < e_end) {
        o = offsets[e];
        cnt = offsets[e + 1] - o;
      }
      const int nb = (cnt + XG_BM - 1) / XG_BM;
      int x = nb;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      const int excl = carry + x - nb;
      if (e < e_end && mb >= excl && mb < excl + nb) {
        const int j = mb - excl;
        sh[0] = e;
        sh[1] = o + j * XG_BM;
        sh[2] = min(XG_BM, cnt - j * XG_BM);
      }
      carry += __shfl(x, 63);
    }
  }
  __syncthreads();
  RowBlock rb{sh[0], sh[1], sh[2]};
  return rb;
}

template <bool SWIGLU, int MT>
__device__ __forceinline__ void gemm_body(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bl,
                                          int K, int N, int col, bf16_t* __restrict__ C,
                                          const RowBlock& rb, bf16_t* As) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int rows_tile = 16 * MT;
  const bf16_t* Ablk = A + (int64_t)rb.r0 * K;

  f32x4 acc[MT][4];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += XG_KS) {
    BRaw br0, br1;
    load_b_block(br0, Bl, N, k0, K, col, N);
    load_b_block(br1, Bl, N, k0 + 32, K, col, N);
    __syncthreads();  // previous stage fully consumed
    for (int v = tid; v < rows_tile * (XG_KS / 8); v += 256) {
      const int r = v >> 3, s = v & 7;
      const int k = k0 + 8 * s;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (r < rb.R && k < K) val = *reinterpret_cast<const u32x4*>(Ablk + (int64_t)r * K + k);
      *reinterpret_cast<u32x4*>(As + r * XG_LDA + 8 * s) = val;
    }
    __syncthreads();
    bf16x8 bf[4];
    transpose_b(br0, bf);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(As + (16 * mt + i) * XG_LDA + 8 * g);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[mt][c] = mfma16(af, bf[c], acc[mt][c]);
    }
    transpose_b(br1, bf);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(As + (16 * mt + i) * XG_LDA + 32 + 8 * g);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[mt][c] = mfma16(af, bf[c], acc[mt][c]);
    }
  }

  // epilogue: lane holds 4 consecutive columns (c = 0..3) of rows 16 mt + 4 g + r
  const bool store_lane = SWIGLU ? (i < 8) : true;
  const int ocol = SWIGLU ? col : col;  // output column of element c = 0
  const int ldc = SWIGLU ? N : N;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float a = acc[mt][c][r];
        if (SWIGLU) {
          const float b = __shfl_xor(a, 8);
          o[c] = a / (1.0f + expf(-a)) * b;
        } else {
          o[c] = a;
        }
      }
      const int row = 16 * mt + 4 * g + r;
      if (store_lane && row < rb.R && ocol < N) {
        u32x2 pk = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(C + (int64_t)(rb.r0 + row) * ldc + ocol) = pk;
      }
    }
  }
}

// SWIGLU: A = x_packed [*, K = d], B1/B3 = w1/w3 [n][K][N = f], C = h [*, f]; 128 columns per WG.
// else:   A = h [*, K = f], B1 = w2 [n][K][N = d], C = y_packed [*, d];  256 columns per WG.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_gemm_bf16(const bf16_t* __restrict__ A,
                                                         const int32_t* __restrict__ offsets,
                                                         int e_begin, int e_end,
                                                         const bf16_t* __restrict__ B1,
                                                         const bf16_t* __restrict__ B3, int K,
                                                         int N, bf16_t* __restrict__ C,
                                                         int nblk_n) {
  __shared__ __attribute__((aligned(16))) bf16_t As[XG_BM * XG_LDA];
  __shared__ int sh[4];
  const int mb = blockIdx.x / nblk_n;
  const int nb = blockIdx.x - mb * nblk_n;
  const RowBlock rb = find_row_block(offsets, e_begin, e_end, mb, sh);
  if (rb.R <= 0) return;
  const int wave = threadIdx.x >> 6;
  const int i = threadIdx.x & 15;
  int col;
  const bf16_t* Bl;
  const int64_t estride = (int64_t)K * N;
  if (SWIGLU) {
    col = nb * 128 + wave * 32 + 4 * (i & 7);
    Bl = ((i < 8) ? B1 : B3) + rb.e * estride;
  } else {
    col = nb * 256 + wave * 64 + 4 * i;
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
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3((unsigned)(mblocks * nb1)), dim3(256), 0, st,
                       (const bf16_t*)x_packed, offsets, e_begin, e_end, (const bf16_t*)w1,
                       (const bf16_t*)w3, p.d, p.f, (bf16_t*)h, nb1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nb2 = (p.d + 255) / 256;
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3((unsigned)(mblocks * nb2)), dim3(256), 0, st,
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
