// Router: logits = x . W_g (+ b) with fp32 accumulation, then per-token top-k
// softmax gating.  The routing step of the DeepSeek-V3 MoE layer in "CUCo: An
// Agentic Framework for Compute and Communication Co-design" (Abstract;
// Table 4, row "MoE Dispatch/Combine"); the pages give no formula, so this is
// the plain softmax top-k gate renormalised over the selected k, ties to the
// lower expert index.
//
// Kernels
//   router_wide_mfma    bf16, E % 4 == 0 and E > 16: split-K MFMA GEMM on the
//                       pipelined core (gemm_core.h); each wave owns 64
//                       expert columns, the workgroup 64 tokens and 256
//                       experts.  Writes fp32 partial sums per K split.
//   router_narrow_mfma  bf16, E <= 16 and E*d <= 32K: W_g^T staged once in LDS,
//                       each wave streams its own 32 token rows straight from
//                       HBM into MFMA A fragments.  HBM-bound on x.
//   router_plain        any dtype/shape: one thread per logit (fp32 problems
//                       and shapes the MFMA kernels do not cover).
//   topk_softmax_kernel one wave per token: sums the K splits in fixed order,
//                       adds the bias, optionally stores the logits, then k
//                       rounds of a wave-wide max over (value, index) keys.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// wide router (bf16, MFMA, split-K) on the pipelined core of gemm_core.h
// ---------------------------------------------------------------------------
constexpr int RW_MT = 4;        // m-tiles per workgroup
constexpr int RW_BM = 16 * RW_MT;  // tokens per workgroup
constexpr int RW_BN = 256;      // experts per workgroup (4 waves x 64)

__global__ __launch_bounds__(256) void router_wide_mfma(const bf16_t* __restrict__ x,
                                                        const bf16_t* __restrict__ wg,
                                                        float* __restrict__ part, int T, int d,
                                                        int E, int kchunk) {
  __shared__ __attribute__((aligned(16))) bf16_t As[gc_lds_elems<4, 4, RW_MT>()];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * RW_BM;
  const int split = blockIdx.y;
  const int kbeg = split * kchunk;
  const int kend = min(d, kbeg + kchunk);
  const int col = blockIdx.z * RW_BN + wave * 64 + 4 * i;
  GemmArgs ga{x + (int64_t)m0 * d, d, min(RW_BM, T - m0), wg, E, kbeg, kend, E, col};
  f32x4 acc[RW_MT][4];
  gemm_mainloop<4, 4, RW_MT>(ga, As, acc);
  if (col >= E) return;
  float* out = part + (int64_t)split * T * E;
#pragma unroll
  for (int mt = 0; mt < RW_MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + 16 * mt + 4 * g + r;
      if (row < T) {
        f32x4 v = f32x4{acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
        *reinterpret_cast<f32x4*>(out + (int64_t)row * E + col) = v;
      }
    }
}

// ---------------------------------------------------------------------------
// narrow router (bf16, MFMA, E <= 16)
// ---------------------------------------------------------------------------
constexpr int RN_MT = 2;        // m-tiles per wave (32 tokens)
constexpr int RN_ROWS = 4 * 16 * RN_MT;  // tokens per workgroup

__global__ __launch_bounds__(256) void router_narrow_mfma(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wg,
                                                          float* __restrict__ logits, int T,
                                                          int d, int E) {
  extern __shared__ __attribute__((aligned(16))) bf16_t WgT[];  // [E][d]
  const int tid = threadIdx.x;
  // W_g is [d][E] row-major; read it in 16-byte pieces and scatter transposed.
  for (int v = tid; v < (E * d) >> 3; v += 256) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(wg + 8 * (int64_t)v);
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const int flat = 8 * v + h;
      const int kk = flat / E, e = flat - kk * E;
      WgT[e * d + kk] = (bf16_t)((h & 1) ? (q[h >> 1] >> 16) : (q[h >> 1] & 0xFFFFu));
    }
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * RN_ROWS + wave * 16 * RN_MT;
  f32x4 acc[RN_MT];
#pragma unroll
  for (int a = 0; a < RN_MT; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool colok = i < E;
  for (int k0 = 0; k0 < d; k0 += 32) {
    const int k = k0 + 8 * g;
    bf16x8 bfr;
    if (colok && k < d) {
      bfr = *reinterpret_cast<const bf16x8*>(WgT + i * d + k);
    } else {
      bfr = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int mt = 0; mt < RN_MT; ++mt) {
      const int row = m0 + 16 * mt + i;
      u32x4 a = u32x4{0u, 0u, 0u, 0u};
      if (row < T && k < d) a = *reinterpret_cast<const u32x4*>(x + (int64_t)row * d + k);
      acc[mt] = mfma16(__builtin_bit_cast(bf16x8, a), bfr, acc[mt]);
    }
  }
  if (!colok) return;
#pragma unroll
  for (int mt = 0; mt < RN_MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + 16 * mt + 4 * g + r;
      if (row < T) logits[(int64_t)row * E + i] = acc[mt][r];
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
// 64-bit keys: order-preserving fp32 bits in the high word, (1023 - expert) in
// the low word, so the maximum key is the largest logit with ties resolved to
// the lower expert index.  A logit key is never 0, so 0 marks "taken/absent".
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the wave, returned uniformly: butterfly inside each 16-lane row
// with DPP (quad swaps, half-row mirror, row mirror), then the four row maxima
// through readlane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<0xB1>(v));   // quad_perm 1,0,3,2
  v = umax64(v, dpp_u64<0x4E>(v));   // quad_perm 2,3,0,1
  v = umax64(v, dpp_u64<0x141>(v));  // row_half_mirror
  v = umax64(v, dpp_u64<0x140>(v));  // row_mirror
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 16 * r);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 16 * r);
    m = umax64(m, ((uint64_t)hi << 32) | lo);
  }
  return m;
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

// NV = values per lane = ceil(E / 64).
template <int NV>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ part,
                                                           int nsplit, const float* __restrict__ bias,
                                                           float* __restrict__ logits_out, int T,
                                                           int E, int k, int32_t* __restrict__ idx,
                                                           float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  uint64_t key[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    key[j] = 0;
    const int e = lane + 64 * j;
    if (e < E) {
      float v = part[(int64_t)t * E + e];
      for (int s = 1; s < nsplit; ++s) v += part[((int64_t)s * T + t) * E + e];
      if (bias) v += bias[e];
      if (logits_out) logits_out[(int64_t)t * E + e] = v;
      key[j] = ((uint64_t)f32_order_key(v) << 32) | (uint32_t)(1023 - e);
    }
  }
  float myv = 0.f, v0 = 0.f;
  int mye = 0;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) best = umax64(best, key[j]);
    best = wave_max_u64(best);
    const int e = 1023 - (int)(uint32_t)(best & 0xFFFFFFFFu);
    const float v = key_to_f32((uint32_t)(best >> 32));
    if (r == 0) v0 = v;
    if (lane == r) {
      myv = v;
      mye = e;
    }
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (j == (e >> 6)) key[j] = 0;
    }
  }
  const float ex = lane < k ? expf(myv - v0) : 0.f;
  const float sum = wave_sum_f32(ex);
  if (lane < k) {
    idx[(int64_t)t * k + lane] = mye;
    w[(int64_t)t * k + lane] = ex / sum;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
enum RouteKind { ROUTE_WIDE = 0, ROUTE_NARROW = 1, ROUTE_PLAIN = 2 };

static RouteKind route_kind(const Prob& p) {
  if (p.dtype == 1 && p.E <= 16 && (int64_t)p.E * p.d <= 32768) return ROUTE_NARROW;
  if (p.dtype == 1 && p.E % 4 == 0 && p.E > 16) return ROUTE_WIDE;
  return ROUTE_PLAIN;
}

static int route_splits(const Prob& p) {
  if (route_kind(p) != ROUTE_WIDE) return 1;
  // enough workgroups to cover the chip, every split keeps >= 256 of K
  const int64_t blocks = (int64_t)((p.T + RW_BM - 1) / RW_BM) * ((p.E + RW_BN - 1) / RW_BN);
  int64_t s = (256 + blocks - 1) / blocks;
  const int64_t smax = p.d / 256 > 1 ? p.d / 256 : 1;
  if (s > smax) s = smax;
  return (int)s;
}

static int route_kchunk(const Prob& p, int S) {
  const int kc = (p.d + S - 1) / S;
  return (kc + GC_KS - 1) / GC_KS * GC_KS;
}

size_t route_ws_bytes(const Prob& p) {
  // fp32 partial sums [splits][T][E]
  return (size_t)route_splits(p) * p.T * p.E * sizeof(float);
}

hipError_t launch_route(const Prob& p, const void* x, const void* wg, const float* bias,
                        float* logits, int32_t* idx, float* w, void* ws, hipStream_t st) {
  float* part = reinterpret_cast<float*>(ws);
  const RouteKind kind = route_kind(p);
  const int S = route_splits(p);
  if (kind == ROUTE_WIDE) {
    const int kchunk = route_kchunk(p, S);
    dim3 grid((p.T + RW_BM - 1) / RW_BM, S, (p.E + RW_BN - 1) / RW_BN);
    hipLaunchKernelGGL(router_wide_mfma, grid, dim3(256), 0, st, (const bf16_t*)x, (const bf16_t*)wg, part, p.T,
                       p.d, p.E, kchunk);
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
  auto tk = nv <= 1 ? topk_softmax_kernel<1>
          : nv <= 2 ? topk_softmax_kernel<2>
          : nv <= 4 ? topk_softmax_kernel<4>
          : nv <= 8 ? topk_softmax_kernel<8>
                    : topk_softmax_kernel<16>;
  hipLaunchKernelGGL(tk, dim3((p.T + 3) / 4), dim3(256), 0, st, part, S, bias, logits, p.T, p.E,
                     p.k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
