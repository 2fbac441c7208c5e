// Internal launchers of libmoe (host functions defined next to their kernels).
// All take a validated problem and launch asynchronously on `st`.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace moe {

// route.hip
size_t route_ws_bytes(const Prob& p);
// chunk_hist (or NULL): the dispatch chunk histograms (hist_elems int32 =
// ceil(T k / 1024) * E).  Where the router kernel supports it, it clears them
// and top-k counts its selections into them; *hist_done (if given) says
// whether that happened, so that dispatch can skip its histogram kernel.
hipError_t launch_route(const Prob& p, const void* x, const void* wg, const float* bias,
                        float* logits, int32_t* idx, float* w, void* ws, hipStream_t st,
                        int32_t* chunk_hist = nullptr, int64_t hist_elems = 0,
                        bool* hist_done = nullptr);

// dispatch.hip
size_t dispatch_ws_bytes(const Prob& p);
// hist_ready: ws already holds the chunk histograms (filled by top-k), so the
// histogram kernel is skipped.
// w_in / rscale (both or neither): rscale[inv[a]] = w_in[a] for every local
// assignment a (the routing weight of each packed row).
hipError_t launch_dispatch_index(const Prob& p, const int32_t* idx, int32_t* counts_all,
                                 int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                                 hipStream_t st, bool hist_ready = false,
                                 const float* w_in = nullptr, float* rscale = nullptr);
// Zero counts_all [E] and offsets [n+1] (either may be NULL): the index of an
// empty batch.  launch_dispatch_index does this itself when T = 0.
hipError_t launch_clear_index(const Prob& p, int32_t* counts_all, int32_t* offsets, hipStream_t st);
// Static per-device scratch of the allocation-free dispatch: its size, and its
// device address on the current device (looked up once per device).
size_t dispatch_scratch_bytes();
hipError_t dispatch_scratch(void** out);
// Gather rows of the local experts [e_begin, e_end) (0-based local indices).
hipError_t launch_gather(const Prob& p, const void* x, const int32_t* offsets,
                         const int32_t* perm, void* x_packed, int e_begin, int e_end,
                         hipStream_t st);

// Padded fixed-capacity layout: n * capacity rows (see dispatch.hip); the
// workspace holds the unpadded index plus the dispatch workspace.
size_t dispatch_padded_ws_bytes(const Prob& p);
hipError_t launch_dispatch_padded(const Prob& p, int capacity, const int32_t* idx,
                                  int32_t* counts_all, int32_t* offsets, int32_t* perm,
                                  int32_t* inv, const void* x, void* x_packed, void* ws,
                                  hipStream_t st);

// expert_gemm.hip: GEMMs over the segments of local experts [e_begin, e_end).
// With perm (bf16 only, T * d * 2 < 2^32), x_packed is x itself and GEMM-1
// gathers its rows through perm (packed row p = token perm[p] / k).
size_t expert_gemm_ws_bytes(const Prob& p);
// With rscale (packed-row weights), y_packed row p is rnd(rscale[p] * (h W2)).
hipError_t launch_expert_gemm(const Prob& p, const void* x_packed, const int32_t* offsets,
                              const void* w1, const void* w3, const void* w2, void* h,
                              void* y_packed, void* ws, int e_begin, int e_end, hipStream_t st,
                              const int32_t* perm = nullptr, const float* rscale = nullptr);

// expert_gemm.hip: GEMM C = rnd(A B) with a release flag per 256 x 256 tile
int64_t gemm_signal_tiles(int M, int N);
hipError_t launch_gemm_signal(int M, int N, int K, const void* A, const void* B, void* C,
                              uint32_t* flags, uint32_t epoch, int system_scope, hipStream_t st);
// tile_forward.hip: copy each tile of C to dst once its flag reads epoch
hipError_t launch_tile_forward(int M, int N, const void* C, void* dst, const uint32_t* flags,
                               uint32_t epoch, uint32_t spin_limit, int system_scope,
                               uint32_t* timeouts, int workgroups, hipStream_t st);

// combine.hip
hipError_t launch_combine(const Prob& p, const void* y_packed, const int32_t* inv,
                          const float* w, void* y, hipStream_t st);

}  // namespace moe
