// Combine: y[t] = rnd(sum_j w[t,j] * y_packed[inv[t*k+j]]) over the token's
// local slots, fp32 accumulation in slot order; exact zeros for tokens with no
// local slot.  The un-permute and weighted sum of the pages' MoE combine
// ("CUCo: An Agentic Framework for Compute and Communication Co-design",
// Table 4, row "MoE Dispatch/Combine").
//
// One wave per token.  Lanes 0..k-1 fetch the slot indices and weights once;
// each lane then owns 16-byte column pieces of the row and reads the k source
// rows' pieces (all issued before the multiply-adds), so every load and store
// is a coalesced 16-byte access.
#include "common.h"
#include "kernels.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ yp,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w,
                                                      u32x4* __restrict__ y, int T, int k,
                                                      int nvec) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_row = -1;
  float my_w = 0.f;
  if (lane < k) {
    my_row = inv[(int64_t)t * k + lane];
    my_w = w[(int64_t)t * k + lane];
  }
  // compact the local slots, keeping slot order
  const uint64_t valid = __ballot(my_row >= 0);
  const int nloc = __popcll(valid);
  u32x4* dst = y + (int64_t)t * nvec;
  for (int v = lane; v < nvec; v += 64) {
    float acc[BF16 ? 8 : 4];
#pragma unroll
    for (int q = 0; q < (BF16 ? 8 : 4); ++q) acc[q] = 0.f;
    uint64_t rest = valid;
    for (int j0 = 0; j0 < nloc; j0 += 4) {
      u32x4 val[4];
      float wj[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wj[u] = 0.f;
        val[u] = u32x4{0u, 0u, 0u, 0u};
        if (j0 + u < nloc) {
          const int src = __ffsll((unsigned long long)rest) - 1;
          rest &= rest - 1;
          const int row = __shfl(my_row, src);
          wj[u] = __shfl(my_w, src);
          val[u] = yp[(int64_t)row * nvec + v];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j0 + u < nloc) {
          if (BF16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[2 * q] = fmaf(wj[u], bf16_lo(val[u][q]), acc[2 * q]);
              acc[2 * q + 1] = fmaf(wj[u], bf16_hi(val[u][q]), acc[2 * q + 1]);
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = fmaf(wj[u], __uint_as_float(val[u][q]), acc[q]);
          }
        }
      }
    }
    u32x4 o;
    if (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
    }
    dst[v] = o;
  }
}

hipError_t launch_combine(const Prob& p, const void* y_packed, const int32_t* inv,
                          const float* w, void* y, hipStream_t st) {
  const int nvec = (int)((int64_t)p.d * p.elem() / 16);
  dim3 grid((p.T + 3) / 4);
  if (p.dtype == 1)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, st, (const u32x4*)y_packed, inv, w,
                       (u32x4*)y, p.T, p.k, nvec);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, st, (const u32x4*)y_packed, inv,
                       w, (u32x4*)y, p.T, p.k, nvec);
  return hipGetLastError();
}

}  // namespace moe
