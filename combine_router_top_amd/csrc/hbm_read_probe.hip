// Streaming-read probe, for measurement only (built into its own library,
// libhbm_probe.so; the MoE path never calls it).
//
// Each lane reads 16-byte words at a grid-wide stride, once each, and folds
// them into one word that is stored only when it equals an unlikely constant,
// so the loads cannot be dropped and almost nothing is written.  Its rate is
// the HBM read bandwidth a plain, well-coalesced kernel reaches on the device:
// the practical ceiling beside the datasheet peak for the read-dominated
// expert GEMMs.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4* __restrict__ src, size_t n,
                                                       uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Reads n16 16-byte words from device memory src on the given HIP stream
// (nullptr = the default stream) with `grid` workgroups of 256 lanes.  sink is
// device memory of at least `grid` uint32 words; it is written only by chance.
// Returns 0, or a hipError_t code (hipErrorInvalidValue for a null pointer or
// a grid outside [1, 65536]).  Asynchronous: the caller synchronises.
extern "C" int hbm_read_probe(const void* src, size_t n16, void* sink, int grid, void* stream) {
    if (!src || !sink || grid < 1 || grid > 65536) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)src, n16, (uint32_t*)sink);
    return (int)hipGetLastError();
}
