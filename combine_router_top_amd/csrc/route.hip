// Router: logits = x . W_g (+ b) with fp32 accumulation, then per-token top-k
// softmax gating.  The routing step of the DeepSeek-V3 MoE layer in "CUCo: An
// Agentic Framework for Compute and Communication Co-design" (Abstract;
// Table 4, row "MoE Dispatch/Combine"); the pages give no formula, so this is
// the plain softmax top-k gate renormalised over the selected k, ties to the
// lower expert index.
//
// Kernels
//   router_wide_mfma    bf16, E % 4 == 0 and E > 16: split-K MFMA GEMM, each
//                       wave owns 64 expert columns, the workgroup 64 tokens
//                       and 256 experts; A (x rows) staged through LDS, B
//                       (W_g) transposed in registers.  Writes fp32 partial
//                       sums per K split.
//   router_narrow_mfma  bf16, E <= 16 and E*d <= 32K: W_g^T staged once in LDS,
//                       each wave streams its own 32 token rows straight from
//                       HBM into MFMA A fragments.  HBM-bound on x.
//   router_plain        any dtype/shape: one thread per logit (fp32 problems
//                       and shapes the MFMA kernels do not cover).
//   topk_softmax_kernel one wave per token: sums the K splits in fixed order,
//                       adds the bias, optionally stores the logits, then k
//                       rounds of a wave-wide max over (value, index) keys.
#include "common.h"
#include "mfma_tile.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// wide router (bf16, MFMA, split-K)
// ---------------------------------------------------------------------------
constexpr int RW_BM = 64;       // tokens per workgroup (4 m-tiles)
constexpr int RW_BN = 256;      // experts per workgroup (4 waves x 64)
constexpr int RW_KS = 64;       // K per LDS stage
constexpr int RW_LDA = RW_KS + 8;  // LDS row stride in bf16 (16-byte pad)

__global__ __launch_bounds__(256) void router_wide_mfma(const bf16_t* __restrict__ x,
                                                        const bf16_t* __restrict__ wg,
                                                        float* __restrict__ part, int T, int d,
                                                        int E, int kchunk) {
  __shared__ __attribute__((aligned(16))) bf16_t As[RW_BM * RW_LDA];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * RW_BM;
  const int split = blockIdx.y;
  const int kbeg = split * kchunk;
  const int kend = min(d, kbeg + kchunk);
  const int nc = blockIdx.z * RW_BN + wave * 64 + 4 * i;  // this lane's 4 columns

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg; k0 < kend; k0 += RW_KS) {
    // stage A: 64 rows x 64 k, 16 bytes per thread per pass (2 passes)
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int v = tid + pass * 256;
      const int r = v >> 3, s = v & 7;
      const int row = m0 + r, k = k0 + 8 * s;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (row < T && k < kend) val = *reinterpret_cast<const u32x4*>(x + (int64_t)row * d + k);
      *reinterpret_cast<u32x4*>(As + r * RW_LDA + 8 * s) = val;
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kb = k0 + 32 * sub;
      BRaw br;
      load_b_block(br, wg, E, kb, kend, nc, E);
      bf16x8 bf[4];
      transpose_b(br, bf);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 af =
            *reinterpret_cast<const bf16x8*>(As + (16 * mt + i) * RW_LDA + 32 * sub + 8 * g);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[mt][c] = mfma16(af, bf[c], acc[mt][c]);
      }
    }
    __syncthreads();
  }
  if (nc >= E) return;
  float* out = part + (int64_t)split * T * E;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + 16 * mt + 4 * g + r;
      if (row < T) {
        f32x4 v = f32x4{acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
        *reinterpret_cast<f32x4*>(out + (int64_t)row * E + nc) = v;
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
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float key_to_f32(uint32_t ok) {
  const uint32_t u = (ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok;
  return __uint_as_float(u);
}

constexpr int TK_MAXV = 16;  // E <= 1024 = 16 values per lane

__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ part,
                                                           int nsplit, const float* __restrict__ bias,
                                                           float* __restrict__ logits_out, int T,
                                                           int E, int k, int32_t* __restrict__ idx,
                                                           float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nv = (E + 63) >> 6;
  uint64_t key[TK_MAXV];
#pragma unroll
  for (int j = 0; j < TK_MAXV; ++j) {
    key[j] = 0;
    const int e = lane + 64 * j;
    if (j < nv && e < E) {
      float v = part[(int64_t)t * E + e];
      for (int s = 1; s < nsplit; ++s) v += part[((int64_t)s * T + t) * E + e];
      if (bias) v += bias[e];
      if (logits_out) logits_out[(int64_t)t * E + e] = v;
      key[j] = ((uint64_t)f32_order_key(v) << 32) | (uint32_t)(1023 - e);
    }
  }
  float myv = 0.f;
  int mye = 0;
  float v0 = 0.f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < TK_MAXV; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int e = 1023 - (int)(uint32_t)(best & 0xFFFFFFFFu);
    const float v = key_to_f32((uint32_t)(best >> 32));
    if (r == 0) v0 = v;
    if (lane == r) {
      myv = v;
      mye = e;
    }
    // remove the winner from its owner lane
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < TK_MAXV; ++j)
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
  // enough workgroups to cover the chip; every split keeps >= 512 of K
  const int64_t mblocks = (p.T + RW_BM - 1) / RW_BM;
  const int64_t nblocks = (p.E + RW_BN - 1) / RW_BN;
  int s = 1;
  while (mblocks * nblocks * s < 256 && p.d / (2 * s) >= 512) s *= 2;
  return s;
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
    int kchunk = (p.d + S - 1) / S;
    kchunk = (kchunk + RW_KS - 1) / RW_KS * RW_KS;
    dim3 grid((p.T + RW_BM - 1) / RW_BM, S, (p.E + RW_BN - 1) / RW_BN);
    hipLaunchKernelGGL(router_wide_mfma, grid, dim3(256), 0, st, (const bf16_t*)x,
                       (const bf16_t*)wg, part, p.T, p.d, p.E, kchunk);
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
  hipLaunchKernelGGL(topk_softmax_kernel, dim3((p.T + 3) / 4), dim3(256), 0, st, part, S, bias,
                     logits, p.T, p.E, p.k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
