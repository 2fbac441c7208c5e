// Router: logits = x . W_g (+ b) with fp32 accumulation, then per-token top-k
// softmax gating.  The routing step of the DeepSeek-V3 MoE layer in "CUCo: An
// Agentic Framework for Compute and Communication Co-design" (Abstract;
// Table 4, row "MoE Dispatch/Combine"); the pages give no formula, so this is
// the plain softmax top-k gate renormalised over the selected k, ties to the
// lower expert index.
//
// Kernels
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
//                       the logits, then k rounds of a wave-wide max over
//                       (value, index) keys.
#include "common.h"
#include "gemm_core.h"
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
        f32x2 v = f32x2{acc[mt][0][r], acc[mt][1][r]};
        *reinterpret_cast<f32x2*>(out + (int64_t)(m0 + row) * E + col) = v;
      }
    }
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
// Bias, optional logit store, k rounds of a wave-wide max over (value, index)
// keys and the softmax over the k selected: one wave, token t, with the
// lane's summed logits v[j] of experts lane + 64 j.
template <int NV>
__device__ __forceinline__ void topk_select(const float (&v)[NV], const float* __restrict__ bias,
                                            float* __restrict__ logits_out, int t, int E, int k,
                                            int32_t* __restrict__ idx, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  uint64_t key[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    key[j] = 0;
    const int e = lane + 64 * j;
    if (e < E) {
      float vj = v[j];
      if (bias) vj += bias[e];
      if (logits_out) logits_out[(int64_t)t * E + e] = vj;
      key[j] = ((uint64_t)f32_order_key(vj) << 32) | (uint32_t)(1023 - e);
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

template <int NV>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ part,
                                                           int nsplit, const float* __restrict__ bias,
                                                           float* __restrict__ logits_out, int T,
                                                           int E, int k, int32_t* __restrict__ idx,
                                                           float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // sum each expert's K splits in ascending order; the loads of 8 splits of
  // all NV experts of the lane are issued together (one round trip per 8
  // splits, not per expert and 8 splits)
  const int64_t sstride = (int64_t)T * E;
  const float* pt = part + (int64_t)t * E + lane;
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = lane + 64 * j < E ? pt[64 * j] : 0.f;
  int s = 1;
  for (; s + 8 <= nsplit; s += 8) {
    float q[NV][8];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        q[j][u] = lane + 64 * j < E ? pt[(int64_t)(s + u) * sstride + 64 * j] : 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u) v[j] += q[j][u];
  }
  for (; s < nsplit; ++s) {
    float q[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) q[j] = lane + 64 * j < E ? pt[(int64_t)s * sstride + 64 * j] : 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] += q[j];
  }
  topk_select<NV>(v, bias, logits_out, t, E, k, idx, w);
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
                                                          float* __restrict__ w) {
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
  topk_select<NV>(v, bias, logits_out, t, E, k, idx, w);
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
  return route_kind(p) == ROUTE_WIDE ? rw_splits(p, route_mt(p)) : 1;
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
                       w);
    return hipGetLastError();
  }
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
