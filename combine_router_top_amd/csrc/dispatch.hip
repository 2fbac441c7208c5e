// Dispatch: per-expert histogram, prefix scan and stable permutation of the
// local (token, slot) assignments into expert-contiguous, unpadded segments,
// then the row gather x_packed[p] = x[perm[p] / k].  This is the one-GPU
// share of the pages' MoE dispatch with variable-size per-peer transfers and
// no padding ("CUCo: An Agentic Framework for Compute and Communication
// Co-design", Table 4, row "MoE Dispatch/Combine").
//
// The permutation is a stable counting sort computed without global atomics,
// so it is bitwise deterministic:
//   chunk_hist_kernel  one workgroup per chunk of 1024 assignments: LDS
//                      histogram over all E experts (integer atomics in LDS
//                      are order-free).
//   scatter_kernel     one workgroup per chunk: reads every chunk's histogram
//                      (a few KB), forms the global counts, the exclusive scan
//                      over local experts (offsets) and this chunk's base per
//                      expert, then ranks its assignments stably: four waves
//                      of 256 consecutive assignments each, wave-to-wave
//                      prefix in LDS, and inside a wave the rank among equal
//                      experts from ballots over the expert-id bits.
//   gather_rows_kernel one wave per packed row, 16-byte vector copies.
// A batch of at most 1024 assignments (one chunk, e.g. decode) launches only
// the scatter kernel, whose single workgroup builds the histogram itself.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int DCH = 1024;   // assignments per chunk
constexpr int DMAXE = 1024; // max experts
constexpr int DUN = 32;     // chunk histograms read per round in the scatter prologue (all of them at 4096 tokens)

__global__ __launch_bounds__(256) void chunk_hist_kernel(const int32_t* __restrict__ idx,
                                                         int64_t TK, int E,
                                                         int32_t* __restrict__ chunk_hist) {
  __shared__ int h[DMAXE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * DCH;
#pragma unroll
  for (int q = 0; q < DCH / 256; ++q) {
    const int64_t a = base + q * 256 + tid;
    if (a < TK) {
      const int e = idx[a];
      if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) chunk_hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// Exclusive scan over 256 threads; returns this thread's prefix, total in *tot.
__device__ __forceinline__ int block_excl_scan_256(int v, int* lds4, int* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) lds4[wave] = x;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += lds4[w];
  *tot = lds4[0] + lds4[1] + lds4[2] + lds4[3];
  __syncthreads();
  return wbase + x - v;
}

// ONE: the whole batch is one chunk (T k <= 1024) and this single workgroup
// builds the histogram itself in LDS, so chunk_hist_kernel is not launched.
template <bool ONE>
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ idx, int64_t TK,
                                                      int E, int lo, int n, int nchunks,
                                                      const int32_t* __restrict__ chunk_hist,
                                                      int32_t* __restrict__ counts_all,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ inv,
                                                      const float* __restrict__ w_in,
                                                      float* __restrict__ rscale) {
  __shared__ int base[DMAXE];
  __shared__ int wpos[4][DMAXE];
  __shared__ int scan_tmp[4];
  __shared__ int hl[ONE ? DMAXE : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;

  if constexpr (ONE) {
    for (int e = tid; e < E; e += 256) hl[e] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < DCH / 256; ++q) {
      const int64_t a = q * 256 + tid;
      if (a < TK) {
        const int e = idx[a];
        if ((unsigned)e < (unsigned)E) atomicAdd(&hl[e], 1);
      }
    }
    __syncthreads();
  }

  // this chunk's expert ids, loaded first so that their round trip overlaps
  // the histogram reads below
  const int64_t wbeg = (int64_t)c * DCH + wave * 256;
  int key[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t a = wbeg + r * 64 + lane;
    key[r] = a < TK ? idx[a] : -1;
  }

  // 1. per expert (all E: workgroup 0 also writes the global counts): total
  // count, and for the local experts the count in the chunks before this one
  // (DUN independent loads in flight per round instead of one round trip per chunk)
  for (int ge = tid; ge < E; ge += 256) {
    int tot = 0, pre = 0;
    int cc = ONE ? nchunks : 0;
    if constexpr (ONE) tot = hl[ge];
    for (; cc + DUN <= nchunks; cc += DUN) {
      int v[DUN];
#pragma unroll
      for (int u = 0; u < DUN; ++u) v[u] = chunk_hist[(int64_t)(cc + u) * E + ge];
#pragma unroll
      for (int u = 0; u < DUN; ++u) {
        pre += cc + u < c ? v[u] : 0;
        tot += v[u];
      }
    }
    for (; cc < nchunks; ++cc) {
      const int v = chunk_hist[(int64_t)cc * E + ge];
      pre += cc < c ? v : 0;
      tot += v;
    }
    if (c == 0) counts_all[ge] = tot;
    const int e = ge - lo;
    if ((unsigned)e < (unsigned)n) {
      base[e] = tot;
      wpos[0][e] = pre;
    }
  }
  __syncthreads();

  // 2. exclusive scan of the local totals: thread t owns experts 4t .. 4t+3
  int v4[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    v4[q] = e < n ? base[e] : 0;
    s += v4[q];
  }
  int total;
  int run = block_excl_scan_256(s, scan_tmp, &total);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    if (e < n) {
      if (c == 0) offsets[e] = run;
      base[e] = run + wpos[0][e];
    }
    run += v4[q];
  }
  if (c == 0 && tid == 0) offsets[n] = total;
  __syncthreads();

  // 3. per-wave counts of local experts over the wave's 256 assignments
  for (int e = lane; e < n; e += 64) wpos[wave][e] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int e = key[r];
    if (e >= 0) {
      e -= lo;
      if ((unsigned)e >= (unsigned)n) e = -1;
    }
    key[r] = e;
    if (e >= 0) atomicAdd(&wpos[wave][e], 1);
  }
  __syncthreads();

  // 4. turn the per-wave counts into per-wave starting positions
  for (int e = tid; e < n; e += 256) {
    int p = base[e];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int t = wpos[w][e];
      wpos[w][e] = p;
      p += t;
    }
  }
  __syncthreads();

  // 5. stable ranks inside each wave, rounds in assignment order
  const int nbits = n > 1 ? 32 - __clz(n - 1) : 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t a = wbeg + r * 64 + lane;
    const int e = key[r];
    const bool valid = e >= 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    int pos = -1;
    if (valid) {
      const int rank = __popcll(peers & lanemask_lt());
      pos = wpos[wave][e] + rank;
    }
    // all lanes have read their position before the leaders advance the counters
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers & lanemask_lt()) == 0) wpos[wave][e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (a < TK) {
      inv[a] = pos;
      if (valid) {
        perm[pos] = (int32_t)a;
        if (rscale) rscale[pos] = w_in[a];
      }
    }
  }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4* __restrict__ x,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ perm,
                                                          u32x4* __restrict__ xp, int nvec, int k,
                                                          int e_begin, int e_end) {
  const int lane = threadIdx.x & 63;
  const int64_t p = (int64_t)offsets[e_begin] + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= offsets[e_end]) return;
  const int t = perm[p] / k;
  const u32x4* src = x + (int64_t)t * nvec;
  u32x4* dst = xp + p * nvec;
  for (int v0 = lane; v0 < nvec; v0 += 256) {
    u32x4 buf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + 64 * u;
      if (v < nvec) buf[u] = src[v];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + 64 * u;
      if (v < nvec) dst[v] = buf[u];
    }
  }
}

// ---------------------------------------------------------------------------
// Padded fixed-capacity layout (an A/B against the unpadded segments): local
// expert e owns rows [e C, (e + 1) C); its first min(count_e, C) local
// assignments in ascending a fill them in order, later ones are dropped, and
// the remaining rows are padding (perm -1, zero rows).  Derived from the
// unpadded dispatch: rank r of an assignment inside its expert is its packed
// position minus offsets[e].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pad_rows_kernel(const int32_t* __restrict__ perm_u,
                                                       const int32_t* __restrict__ offsets_u, int n,
                                                       int C, int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ offsets) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q <= n) offsets[q] = (int32_t)(q * C);
  if (q >= (int64_t)n * C) return;
  const int e = (int)(q / C), r = (int)(q - (int64_t)e * C);
  const int o = offsets_u[e], cnt = offsets_u[e + 1] - o;
  perm[q] = r < cnt ? perm_u[o + r] : -1;
}

__global__ __launch_bounds__(256) void pad_inv_kernel(const int32_t* __restrict__ idx, int64_t TK,
                                                      const int32_t* __restrict__ offsets_u, int lo,
                                                      int C, int32_t* __restrict__ inv) {
  const int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a >= TK) return;
  const int pos = inv[a];
  if (pos < 0) return;
  const int e = idx[a] - lo;
  const int r = pos - offsets_u[e];
  inv[a] = r < C ? e * C + r : -1;
}

// x_packed[q] = x[perm[q] / k], or a zero row where perm[q] < 0; one wave per row.
__global__ __launch_bounds__(256) void gather_padded_kernel(const u32x4* __restrict__ x,
                                                            const int32_t* __restrict__ perm,
                                                            u32x4* __restrict__ xp, int nvec, int k,
                                                            int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t q = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= rows) return;
  const int a = perm[q];
  u32x4* dst = xp + q * nvec;
  if (a < 0) {
    for (int v = lane; v < nvec; v += 64) dst[v] = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const u32x4* src = x + (int64_t)(a / k) * nvec;
  for (int v0 = lane; v0 < nvec; v0 += 256) {
    u32x4 buf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + 64 * u;
      if (v < nvec) buf[u] = src[v];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + 64 * u;
      if (v < nvec) dst[v] = buf[u];
    }
  }
}

static int64_t n_chunks(const Prob& p) { return (p.tk() + DCH - 1) / DCH; }

size_t dispatch_ws_bytes(const Prob& p) { return (size_t)n_chunks(p) * p.E * sizeof(int32_t); }

// ---------------------------------------------------------------------------
// Scratch of the allocation-free dispatch: the per-chunk histograms live in a
// static device array instead of a caller workspace.  Each device holds its
// own copy for the life of the process; its device address is looked up once
// per device (with that device current) and kept.  In host code the array's
// name is only a registration handle, so kernels get the looked-up address.
// Every call on a device shares the array: calls that overlap on one device
// race.  The histogram kernel writes every entry that the scatter kernel later
// reads, so nothing has to start at zero.
// ---------------------------------------------------------------------------
constexpr size_t DISPATCH_SCRATCH_BYTES = size_t(1) << 20;
constexpr int SCRATCH_MAX_DEVICES = 64;
static __device__ __align__(256) int32_t scratch[DISPATCH_SCRATCH_BYTES / sizeof(int32_t)];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[SCRATCH_MAX_DEVICES] = {};

size_t dispatch_scratch_bytes() { return DISPATCH_SCRATCH_BYTES; }

hipError_t dispatch_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

// Empty batch: the histogram over all E experts and the local offsets are all
// zero; one workgroup writes them (a kernel rather than a memset, so that the
// call can be captured in a graph).
__global__ __launch_bounds__(256) void clear_index_kernel(int32_t* __restrict__ counts_all, int E,
                                                          int32_t* __restrict__ offsets, int n1) {
  for (int i = threadIdx.x; i < E; i += 256) counts_all[i] = 0;
  for (int i = threadIdx.x; i < n1; i += 256) offsets[i] = 0;
}

hipError_t launch_clear_index(const Prob& p, int32_t* counts_all, int32_t* offsets, hipStream_t st) {
  if (!counts_all && !offsets) return hipSuccess;
  hipLaunchKernelGGL(clear_index_kernel, dim3(1), dim3(256), 0, st, counts_all,
                     counts_all ? p.E : 0, offsets, offsets ? p.n + 1 : 0);
  return hipGetLastError();
}

hipError_t launch_dispatch_index(const Prob& p, const int32_t* idx, int32_t* counts_all,
                                 int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                                 hipStream_t st, bool hist_ready, const float* w_in, float* rscale) {
  if (p.tk() == 0) return launch_clear_index(p, counts_all, offsets, st);
  int32_t* chunk_hist = reinterpret_cast<int32_t*>(ws);
  const int64_t nc = n_chunks(p);
  if (nc == 1) {  // one workgroup does it all
    hipLaunchKernelGGL(scatter_kernel<true>, dim3(1), dim3(256), 0, st, idx, p.tk(), p.E, p.lo,
                       p.n, 1, (const int32_t*)nullptr, counts_all, offsets, perm, inv, w_in, rscale);
    return hipGetLastError();
  }
  if (!hist_ready) {
    hipLaunchKernelGGL(chunk_hist_kernel, dim3((unsigned)nc), dim3(256), 0, st, idx, p.tk(), p.E,
                       chunk_hist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(scatter_kernel<false>, dim3((unsigned)nc), dim3(256), 0, st, idx, p.tk(), p.E,
                     p.lo, p.n, (int)nc, chunk_hist, counts_all, offsets, perm, inv, w_in, rscale);
  return hipGetLastError();
}

hipError_t launch_gather(const Prob& p, const void* x, const int32_t* offsets,
                         const int32_t* perm, void* x_packed, int e_begin, int e_end,
                         hipStream_t st) {
  const int nvec = (int)((int64_t)p.d * p.elem() / 16);
  const int64_t rows = p.rows_max;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 3) / 4));
  hipLaunchKernelGGL(gather_rows_kernel, grid, dim3(256), 0, st, (const u32x4*)x, offsets, perm,
                     (u32x4*)x_packed, nvec, p.k, e_begin, e_end);
  return hipGetLastError();
}

size_t dispatch_padded_ws_bytes(const Prob& p) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  return up(dispatch_ws_bytes(p)) + up((size_t)(p.n + 1) * 4) + up((size_t)p.rows_max * 4);
}

hipError_t launch_dispatch_padded(const Prob& p, int capacity, const int32_t* idx,
                                  int32_t* counts_all, int32_t* offsets, int32_t* perm,
                                  int32_t* inv, const void* x, void* x_packed, void* ws,
                                  hipStream_t st) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  char* w = reinterpret_cast<char*>(ws);
  int32_t* offsets_u = reinterpret_cast<int32_t*>(w + up(dispatch_ws_bytes(p)));
  int32_t* perm_u = reinterpret_cast<int32_t*>(w + up(dispatch_ws_bytes(p)) + up((size_t)(p.n + 1) * 4));
  hipError_t e = launch_dispatch_index(p, idx, counts_all, offsets_u, perm_u, inv, ws, st);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.n * capacity;
  const int64_t tq = std::max<int64_t>(rows, p.n + 1);
  hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)((tq + 255) / 256)), dim3(256), 0, st, perm_u,
                     offsets_u, p.n, capacity, perm, offsets);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(pad_inv_kernel, dim3((unsigned)((p.tk() + 255) / 256)), dim3(256), 0, st, idx,
                     p.tk(), offsets_u, p.lo, capacity, inv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nvec = (int)((int64_t)p.d * p.elem() / 16);
  hipLaunchKernelGGL(gather_padded_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                     (const u32x4*)x, perm, (u32x4*)x_packed, nvec, p.k, rows);
  return hipGetLastError();
}

}  // namespace moe
