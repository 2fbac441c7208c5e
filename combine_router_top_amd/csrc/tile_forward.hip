// Tile forwarder: the consumer side of the signalled GEMM (gemm_signal_kernel).
// On several GPUs this is where the pages' GEMM + AllGather broadcast would
// start ("CUCo", Table 4, row "GEMM + AllGather": a device-initiated
// broadcast right after GEMM completion); here it copies each 256 x 256 bf16
// tile of C to dst (which could be a peer's mapped buffer) as soon as the
// tile's flag reads `epoch`.
//
// Workgroup g takes tiles g, g + G, ... in order.  Its first thread polls the
// flag with acquire loads (agent or system scope) and a short sleep between
// polls, at most spin_limit times; then the workgroup copies the tile with
// 16-byte loads and stores, or, if the flag never arrived, counts a timeout
// and moves on, so every wave always exits.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int TF_TILE = 256;   // tile edge, as the signalled GEMM's

__global__ __launch_bounds__(256) void tile_forward_kernel(const u32x4* __restrict__ C,
                                                           u32x4* __restrict__ dst,
                                                           const uint32_t* flags, uint32_t epoch,
                                                           uint32_t spin_limit, int system_scope,
                                                           uint32_t* timeouts, int M, int N,
                                                           int ntn, int tiles) {
  __shared__ int ready;
  const int nv = N / 8;   // 16-byte vectors per row
  for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
    if (threadIdx.x == 0) {
      uint32_t n = 0;
      uint32_t v;
      for (;;) {
        v = system_scope ? __hip_atomic_load(flags + t, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM)
                         : __hip_atomic_load(flags + t, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if (v == epoch || ++n >= spin_limit) break;
        __builtin_amdgcn_s_sleep(2);
      }
      ready = v == epoch;
      if (!ready) atomicAdd(timeouts, 1u);
    }
    __syncthreads();
    const bool go = ready;
    // the other waves order their loads after the first thread's acquire
    __atomic_thread_fence(__ATOMIC_ACQUIRE);
    if (go) {
      const int tm = t / ntn, tn = t - tm * ntn;
      const int r0 = tm * TF_TILE, c0 = tn * (TF_TILE / 8);
      const int rows = min(TF_TILE, M - r0), cols = min(TF_TILE / 8, nv - c0);
      for (int i = threadIdx.x; i < rows * (TF_TILE / 8); i += 256) {
        const int r = i / (TF_TILE / 8), c = i - r * (TF_TILE / 8);
        if (c < cols) {
          const int64_t off = (int64_t)(r0 + r) * nv + c0 + c;
          dst[off] = C[off];
        }
      }
    }
    __syncthreads();   // `ready` is rewritten for the next tile
  }
}

hipError_t launch_tile_forward(int M, int N, const void* C, void* dst, const uint32_t* flags,
                               uint32_t epoch, uint32_t spin_limit, int system_scope,
                               uint32_t* timeouts, int workgroups, hipStream_t st) {
  const int ntn = (N + TF_TILE - 1) / TF_TILE;
  const int tiles = ((M + TF_TILE - 1) / TF_TILE) * ntn;
  const int g = workgroups < tiles ? workgroups : tiles;
  hipLaunchKernelGGL(tile_forward_kernel, dim3((unsigned)g), dim3(256), 0, st, (const u32x4*)C,
                     (u32x4*)dst, flags, epoch, spin_limit, system_scope, timeouts, M, N, ntn, tiles);
  return hipGetLastError();
}

}  // namespace moe
