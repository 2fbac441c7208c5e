// Combine: y[t] = rnd(sum_j w[t,j] * y_packed[inv[t*k+j]]) over the token's
// local slots, fp32 accumulation in slot order; exact zeros for tokens with no
// local slot.  The un-permute and weighted sum of the pages' MoE combine
// ("CUCo: An Agentic Framework for Compute and Communication Co-design",
// Table 4, row "MoE Dispatch/Combine").
//
// One wave per (token, 128-vector column chunk): lanes 0..k-1 fetch the slot
// indices and weights and the wave compacts its local slots (in slot order)
// into LDS; each lane then owns two 16-byte pieces of the chunk and loads them
// for up to 8 slots at once before accumulating them in slot order, so a
// token with k local slots costs one round trip per 8 slots, and a short
// batch (decode) still spreads over T x ceil(d / 1024) waves.  y is stored
// non-temporally: the layer does not read it again, and left dirty in the
// MALL it would be written back while the next layer's weights stream in.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int CB_P = 2;   // 16-byte pieces per lane per slot (a chunk is 64 CB_P vectors)
constexpr int CB_G = 8;   // slots whose pieces are loaded together

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ yp,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w,
                                                      u32x4* __restrict__ y, int T, int k,
                                                      int nvec, int nchunk) {
  __shared__ int s_row[4][32];
  __shared__ float s_w[4][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  const int64_t t = gw / nchunk;
  const int ch = (int)(gw - t * nchunk);
  if (t >= T) return;
  int my_row = -1;
  float my_w = 0.f;
  if (lane < k) {
    my_row = inv[t * k + lane];
    my_w = w ? w[t * k + lane] : 1.0f;   // no weights: rows already weighted, a plain sum
  }
  // compact the local slots into LDS, keeping slot order
  const uint64_t valid = __ballot(my_row >= 0);
  const int nloc = __popcll(valid);
  if (my_row >= 0) {
    const int at = __popcll(valid & lanemask_lt());
    s_row[wave][at] = my_row;
    s_w[wave][at] = my_w;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int NQ = BF16 ? 8 : 4;
  const int v0 = ch * 64 * CB_P + lane;
  float acc[CB_P][NQ];
#pragma unroll
  for (int u = 0; u < CB_P; ++u)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[u][q] = 0.f;
  for (int j0 = 0; j0 < nloc; j0 += CB_G) {
    u32x4 val[CB_G][CB_P];
#pragma unroll
    for (int g = 0; g < CB_G; ++g) {
      const bool on = j0 + g < nloc;
      const u32x4* src = yp + (int64_t)(on ? s_row[wave][j0 + g] : 0) * nvec;
#pragma unroll
      for (int u = 0; u < CB_P; ++u) {
        const int v = v0 + 64 * u;
        val[g][u] = on && v < nvec ? src[v] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int g = 0; g < CB_G; ++g) {
      if (j0 + g >= nloc) break;
      const float wj = s_w[wave][j0 + g];
#pragma unroll
      for (int u = 0; u < CB_P; ++u) {
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[u][2 * q] = fmaf(wj, bf16_lo(val[g][u][q]), acc[u][2 * q]);
            acc[u][2 * q + 1] = fmaf(wj, bf16_hi(val[g][u][q]), acc[u][2 * q + 1]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[u][q] = fmaf(wj, __uint_as_float(val[g][u][q]), acc[u][q]);
        }
      }
    }
  }
  u32x4* dst = y + t * nvec;
#pragma unroll
  for (int u = 0; u < CB_P; ++u) {
    const int v = v0 + 64 * u;
    if (v >= nvec) continue;
    u32x4 o;
    if (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[u][q]);
    }
    __builtin_nontemporal_store(o, dst + v);
  }
}

hipError_t launch_combine(const Prob& p, const void* y_packed, const int32_t* inv,
                          const float* w, void* y, hipStream_t st) {
  const int nvec = (int)((int64_t)p.d * p.elem() / 16);
  const int nchunk = (nvec + 64 * CB_P - 1) / (64 * CB_P);
  const int64_t waves = (int64_t)p.T * nchunk;
  dim3 grid((unsigned)((waves + 3) / 4));
  if (p.dtype == 1)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, st, (const u32x4*)y_packed, inv, w,
                       (u32x4*)y, p.T, p.k, nvec, nchunk);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, st, (const u32x4*)y_packed, inv,
                       w, (u32x4*)y, p.T, p.k, nvec, nchunk);
  return hipGetLastError();
}

}  // namespace moe
