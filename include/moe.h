/*
 * moe.h -- C ABI of libmoe: one GPU's share of a Mixture-of-Experts layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the DeepSeek-V3 MoE workload of "CUCo: An Agentic Framework for
 * Compute and Communication Co-design" (Abstract; Table 4, row "MoE
 * Dispatch/Combine"): tokens are routed to experts, dispatched into
 * per-expert, variable-size, unpadded buffers, run through the local ("self")
 * experts, and combined back.  This library computes the share of one GPU that
 * owns experts [expert_lo, expert_lo + n_local) of E, for all T tokens:
 *
 *   moe_route        logits = x W_g (+ b); top-k softmax gating
 *   moe_dispatch     per-expert histogram, prefix scan, stable permutation,
 *                    row gather into expert-contiguous buffers
 *   moe_expert_gemm  SwiGLU expert FFNs as grouped GEMMs over the segments
 *   moe_combine      weighted un-permute and sum back to token order
 *   moe_layer        all of the above, stream-ordered
 *   moe_dispatch_padded, moe_expert_gemm_padded
 *                    the padded fixed-capacity layout, as an A/B
 *   moe_gemm_signal, moe_tile_forward
 *                    GEMM with per-tile completion flags and their consumer
 *                    (the local half of the pages' GEMM + AllGather)
 *
 * The pages state no formulas; the definitions below are the plain MoE layer
 * (softmax top-k gating renormalised over the selected k, ties to the lower
 * expert index; SwiGLU experts; weighted combine).
 *
 * Conventions for every call
 *   - Tensors are dense, row-major, and live in device memory.  Rows of x,
 *     x_packed, h, y_packed and y must start on 16-byte boundaries: the base
 *     pointers must be 16-byte aligned and d, f must be multiples of 8.
 *   - The caller owns all memory.  The library never allocates device memory
 *     and never frees caller memory.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Every call is asynchronous on its stream and never synchronises the
 *     device or the host.
 *   - Validation is host-side and shape-only.  On error nothing is launched,
 *     a status is returned and moe_last_error() describes it.  Data-dependent
 *     conditions are not checked: NaN/Inf inputs, expert indices outside
 *     [0, E) in a caller-supplied topk_idx, and a topk_idx row that names the
 *     same expert twice are undefined behaviour (the buffers sized from
 *     rows_max hold T*min(k, n_local) rows only because the k experts of a
 *     token are distinct, as moe_route produces them).
 *   - Results are bitwise deterministic for identical inputs and launch
 *     configuration (no floating-point atomics).
 *   - The calls are re-entrant; concurrent calls must not share workspace.
 *   - The number of local assignments A never leaves the device; a caller that
 *     wants it reads offsets[n_local].
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* NULL pointer, negative T or non-positive d/E/k/f, k > E, bad expert range */
  MOE_ERR_UNSUPPORTED = 2, /* d or f not a multiple of 8, k > 32, E > 1024, bad dtype, misaligned */
  MOE_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 4          /* a HIP launch/runtime call failed; message in moe_last_error() */
};

enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };

/* flags */
enum {
  MOE_F_WRITE_LOGITS = 1u, /* moe_layer: also write fp32 logits to routing_out->logits */
  MOE_F_OVERLAP = 2u,      /* moe_layer: pack the second half of the local experts on
                              stream2 while the first half's GEMMs run on stream */
  MOE_F_FOLD_WEIGHT = 4u   /* moe_layer: apply each assignment's routing weight in the
                              down projection's epilogue, y_packed[p] = rnd(w * (h W2)),
                              and combine the rows unweighted (one rounding point moves;
                              see moe_layer) */
};

/* Which call a workspace size is asked for. */
enum {
  MOE_CALL_ROUTE = 0,
  MOE_CALL_DISPATCH = 1,
  MOE_CALL_EXPERT_GEMM = 2,
  MOE_CALL_COMBINE = 3,
  MOE_CALL_LAYER = 4,
  MOE_CALL_DISPATCH_PADDED = 5,
  MOE_CALL_EXPERT_GEMM_PADDED = 6
};

/*
 * Problem description.
 *   T          tokens (rows of x), >= 0.  T = 0 is an empty batch (a GPU that
 *              received no tokens): the calls launch nothing but one small
 *              kernel that writes zeros to counts_all and offsets where the
 *              call has them; pointers to arrays with a T-sized dimension may
 *              be NULL, every workspace size is 0, and the padded calls reject
 *              it (their capacity must lie in 1 .. T).
 *   d          hidden size
 *   E          routed experts in total (1..1024)
 *   k          experts per token (1..min(E, 32))
 *   f          SwiGLU intermediate size per expert
 *   expert_lo  first expert owned by this GPU
 *   n_local    experts owned by this GPU (expert_lo + n_local <= E)
 *   dtype      MOE_DTYPE_BF16: x, w_gate, w1, w3, w2, x_packed, h, y_packed, y
 *              are bf16 and all sums accumulate in fp32;
 *              MOE_DTYPE_F32: all of them are fp32.
 *   flags      MOE_F_* (read by moe_layer only)
 * Derived: rows_max = T * min(k, n_local), an upper bound of A.
 */
typedef struct moe_problem_t {
  int32_t T, d, E, k, f, expert_lo, n_local;
  int32_t dtype;
  uint32_t flags;
} moe_problem_t;

/* Optional device outputs of moe_layer; any member may be NULL. */
typedef struct moe_routing_out_t {
  int32_t* topk_idx;   /* [T,k] */
  float* topk_w;       /* [T,k] */
  float* logits;       /* [T,E], written only with MOE_F_WRITE_LOGITS */
  int32_t* counts_all; /* [E] */
  int32_t* offsets;    /* [n_local+1] */
  int32_t* perm;       /* [rows_max], first A entries valid */
  int32_t* inv;        /* [T*k] */
} moe_routing_out_t;

/* Thread-local description of the last error on this thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

/*
 * Bytes of device scratch that `call` (MOE_CALL_*) needs for problem p, or 0
 * when p is invalid (then moe_last_error() says why) or the call needs none.
 * The workspace pointer passed to a call must be 256-byte aligned.
 */
size_t moe_workspace_bytes(const moe_problem_t* p, int32_t call);

/*
 * Router: logits[t,e] = sum_i x[t,i] * w_gate[i,e] (+ bias[e]) accumulated in
 * fp32; then per token the k largest logits in descending order, ties to the
 * lower expert index, and weights w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)
 * (softmax over all E renormalised over the selected k).  The pages call this
 * step the routing of the DeepSeek-V3 MoE layer (gist.science summary of the
 * CUCo paper, §4 Results: "imbalanced sparse routing").
 *   x        [T,d]   dtype
 *   w_gate   [d,E]   dtype
 *   bias     [E]     fp32, or NULL
 *   logits   [T,E]   fp32 output, or NULL
 *   topk_idx [T,k]   int32 output
 *   topk_w   [T,k]   fp32 output
 *   workspace of moe_workspace_bytes(p, MOE_CALL_ROUTE) bytes (may be NULL if 0)
 */
moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_gate,
                       const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dispatch (CUCo, Table 4, "MoE Dispatch/Combine": variable-size per-peer
 * transfers with no padding).  Assignment a = t*k + j is local when
 * expert_lo <= topk_idx[a] < expert_lo + n_local.  The k entries of a row of
 * topk_idx must be distinct experts in [0, E) (then A <= rows_max); anything
 * else is undefined behaviour and is not detected.
 *   counts_all [E]          counts_all[e] = #assignments to expert e (all E)
 *   offsets    [n_local+1]  offsets[0] = 0, offsets[e+1] = offsets[e] + counts_all[expert_lo+e]
 *   perm       [rows_max]   perm[p] = a, local assignments sorted by local expert,
 *                           ties in ascending a (stable); entries >= A untouched
 *   inv        [T*k]        inv[perm[p]] = p; -1 for non-local assignments
 *   x_packed   [rows_max,d] x_packed[p] = x[perm[p] / k]; rows >= A untouched
 *   workspace of moe_workspace_bytes(p, MOE_CALL_DISPATCH) bytes
 */
moe_status_t moe_dispatch(const moe_problem_t* p, const int32_t* topk_idx, const void* x,
                          int32_t* counts_all, int32_t* offsets, int32_t* perm, int32_t* inv,
                          void* x_packed, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_dispatch without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, outputs and contract as moe_dispatch
 * minus the workspace: its per-chunk histograms live in a static device array
 * of MOE_DISPATCH_NOALLOC_SCRATCH_BYTES that each device holds until the
 * process ends.  A problem needing more, ceil(T*k/1024) * E * 4 bytes (T*k up
 * to 2^20 at E = 256), is rejected with MOE_ERR_UNSUPPORTED before anything
 * is launched.  Every call on a device shares that array: calls that overlap
 * on one device (several streams or host threads) race, and the caller must
 * order them.  The call allocates nothing.
 */
#define MOE_DISPATCH_NOALLOC_SCRATCH_BYTES (1u << 20)
moe_status_t moe_dispatch_noalloc(const moe_problem_t* p, const int32_t* topk_idx, const void* x,
                                  int32_t* counts_all, int32_t* offsets, int32_t* perm,
                                  int32_t* inv, void* x_packed, void* stream);

/*
 * Local expert compute (CUCo, Abstract: "local compute" of the MoE layer).
 * For each local expert e and its rows R = [offsets[e], offsets[e+1]):
 *   h[R]        = rnd(SiLU(x_packed[R] w1[e]) * (x_packed[R] w3[e]))
 *   y_packed[R] = rnd(h[R] w2[e])
 * with SiLU(z) = z / (1 + exp(-z)), fp32 accumulation, and rnd = round to
 * nearest even into the problem dtype.
 *   w1, w3  [n_local,d,f]  dtype
 *   w2      [n_local,f,d]  dtype
 *   h       [rows_max,f]   dtype output (rows >= A untouched)
 *   y_packed[rows_max,d]   dtype output (rows >= A untouched)
 *   workspace of moe_workspace_bytes(p, MOE_CALL_EXPERT_GEMM) bytes
 */
moe_status_t moe_expert_gemm(const moe_problem_t* p, const void* x_packed, const int32_t* offsets,
                             const void* w1, const void* w3, const void* w2, void* h,
                             void* y_packed, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Combine (CUCo, Table 4, "MoE Dispatch/Combine"): un-permute and weighted sum,
 * over the unpadded or the padded layout (y_packed rows are read at inv),
 *   y[t] = rnd(sum over j < k with inv[t*k+j] >= 0 of topk_w[t,j] * y_packed[inv[t*k+j]])
 * accumulated in fp32 in slot order.  A token with no local slot gets an exact
 * zero row; every row of y is written.  topk_w = NULL sums the rows with unit
 * weights (rows that already carry their weight, as MOE_F_FOLD_WEIGHT makes).
 *   y_packed [rows_max,d] dtype;  inv [T*k];  topk_w [T,k] fp32 or NULL;  y [T,d] dtype
 */
moe_status_t moe_combine(const moe_problem_t* p, const void* y_packed, const int32_t* inv,
                         const float* topk_w, void* y, void* stream);

/*
 * Padded fixed-capacity dispatch: the layout with per-expert padding that CUCo
 * (Table 4, row "MoE Dispatch/Combine") names as a bottleneck on imbalanced
 * ranks, provided as an A/B against moe_dispatch's unpadded segments.  Local
 * expert e owns rows [e*capacity, (e+1)*capacity) of x_packed.  Its first
 * min(count_e, capacity) local assignments in ascending a fill them in that
 * order; later ones are dropped (inv = -1, so moe_combine leaves them out) and
 * the rows past count_e are padding.
 *   capacity   rows per local expert, 1 .. T
 *   counts_all [E]                  as moe_dispatch (before any drop)
 *   offsets    [n_local+1]          offsets[e] = e * capacity
 *   perm       [n_local*capacity]   perm[q] = a, or -1 for a padding row
 *   inv        [T*k]                inv[a] = q for kept local assignments, else -1
 *   x_packed   [n_local*capacity,d] x_packed[q] = x[perm[q] / k]; padding rows zero
 *   workspace of moe_workspace_bytes(p, MOE_CALL_DISPATCH_PADDED) bytes
 */
moe_status_t moe_dispatch_padded(const moe_problem_t* p, int32_t capacity, const int32_t* topk_idx,
                                 const void* x, int32_t* counts_all, int32_t* offsets, int32_t* perm,
                                 int32_t* inv, void* x_packed, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * moe_expert_gemm over the padded layout of moe_dispatch_padded: every local
 * expert's segment is its capacity rows (padding rows included, which give
 * zero rows of h and y_packed).  Same arguments as moe_expert_gemm with
 * x_packed, h and y_packed of n_local*capacity rows and offsets[e] = e*capacity;
 * workspace of moe_workspace_bytes(p, MOE_CALL_EXPERT_GEMM_PADDED) bytes.
 * moe_combine works on the padded y_packed unchanged (it reads rows inv[a]).
 */
moe_status_t moe_expert_gemm_padded(const moe_problem_t* p, int32_t capacity, const void* x_packed,
                                    const int32_t* offsets, const void* w1, const void* w3,
                                    const void* w2, void* h, void* y_packed, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * GEMM with per-tile completion signals: the local compute half of the pages'
 * GEMM + AllGather workload (CUCo, Table 4, row "GEMM + AllGather": a
 * device-initiated broadcast fused right after GEMM completion instead of a
 * host-launched collective after the whole GEMM).
 *   C[M,N] = rnd(A[M,K] B[K,N]), bf16 row-major, fp32 accumulation, RNE.
 * C is computed in 256 x 256 tiles numbered row-major over
 * ceil(M/256) x ceil(N/256) (moe_gemm_signal_tiles(M, N) of them).  When a
 * tile's stores are complete and visible at `scope` (MOE_SCOPE_AGENT: this
 * GPU; MOE_SCOPE_SYSTEM: also peers and host, which adds an L2 write-back),
 * flags[tile] is set to `epoch` by a release store.  `epoch` must be nonzero
 * and differ from what flags holds before the call (a zeroed array and
 * increasing epochs never need clearing).  N, K multiples of 8; K*N*2 < 2^31.
 */
enum { MOE_SCOPE_AGENT = 0, MOE_SCOPE_SYSTEM = 1 };
int64_t moe_gemm_signal_tiles(int32_t M, int32_t N);
moe_status_t moe_gemm_signal(int32_t M, int32_t N, int32_t K, const void* A, const void* B, void* C,
                             uint32_t* flags, uint32_t epoch, int32_t scope, void* stream);

/*
 * Tile forwarder, the consumer of moe_gemm_signal's flags (where the
 * broadcast of GEMM + AllGather would start; dst can be any device-visible
 * buffer).  Workgroup g of `workgroups` takes tiles g, g + workgroups, ...;
 * for each it polls flags[tile] with acquire loads at `scope`, at most
 * spin_limit times with a short sleep in between, then copies the tile of C
 * (same geometry as moe_gemm_signal) to dst, or, if the flag never read
 * `epoch`, adds 1 to *timeouts (a device counter the caller zeroes) and moves
 * on: the call always finishes.  Run concurrently with moe_gemm_signal on
 * another stream, keep `workgroups` small: polling workgroups hold compute
 * units.
 */
moe_status_t moe_tile_forward(int32_t M, int32_t N, const void* C, void* dst, const uint32_t* flags,
                              uint32_t epoch, uint32_t spin_limit, int32_t scope, uint32_t* timeouts,
                              int32_t workgroups, void* stream);

/*
 * The whole layer: moe_route, moe_dispatch, moe_expert_gemm, moe_combine in
 * stream order on `stream`, with all intermediates in `workspace`
 * (moe_workspace_bytes(p, MOE_CALL_LAYER) bytes).  No device-to-host
 * synchronisation.  routing_out may be NULL; its non-NULL members receive
 * copies of the routing and dispatch tensors.  With MOE_F_OVERLAP and a
 * non-NULL stream2, the row gather of the upper half of the local experts runs
 * on stream2 while the lower half's GEMMs run on `stream` (the two-stream
 * dispatch overlap of CUCo, Abstract and Table 4); stream2 is joined back into
 * `stream` before the call returns its work.  With MOE_F_FOLD_WEIGHT the
 * routing weight of each local assignment scales its expert output row before
 * that row is rounded (y_packed[p] = rnd(w[perm[p]] * (h[p] W2_e))) and the
 * combine sums rows unweighted, y[t] = rnd(sum of the token's local rows): the
 * same value in exact arithmetic, with the gate weight applied where the pages'
 * fused epilogues would apply it (CUCo, Table 4, row "MoE Dispatch/Combine").
 */
moe_status_t moe_layer(const moe_problem_t* p, const void* x, const void* w_gate,
                       const float* bias, const void* w1, const void* w3, const void* w2,
                       void* y, const moe_routing_out_t* routing_out, void* workspace,
                       size_t workspace_bytes, void* stream, void* stream2);

/*
 * Byte offset, inside a moe_layer workspace for problem p, of an intermediate
 * the layer leaves there: MOE_WS_H (h [rows_max,f]) or MOE_WS_Y_PACKED
 * (y_packed [rows_max,d]), in the problem dtype; after a moe_layer call the
 * first A rows hold that call's values (with MOE_F_FOLD_WEIGHT, y_packed rows
 * carry their weights).  For inspecting a layer stage by stage; (size_t)-1 for
 * an invalid p, an empty batch or an unknown region.
 */
enum { MOE_WS_H = 0, MOE_WS_Y_PACKED = 1 };
size_t moe_layer_ws_offset(const moe_problem_t* p, int32_t what);

/*
 * Measurement hook: the next moe_layer call on this host thread records the
 * HIP events `before` and `after` (hipEvent_t, created by the caller) on its
 * launch stream immediately before and after its expert-GEMM launches, so that
 * a benchmark can time the grouped GEMM inside the layer step it times.  The
 * hook is consumed by that call; NULL events record nothing.  Returns MOE_OK.
 */
moe_status_t moe_layer_set_gemm_events(void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
