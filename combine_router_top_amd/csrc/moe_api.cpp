// C ABI of libmoe: argument validation, workspace layout and launch order.
// Validation is shape-only and runs before any HIP call, so invalid calls are
// rejected (and testable) on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status_t ok() {
  g_err.clear();
  return MOE_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

moe_status_t check_problem(const moe_problem_t* p, moe::Prob* out) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "problem is NULL");
  if (p->T < 0 || p->d <= 0 || p->E <= 0 || p->k <= 0 || p->f <= 0)
    return fail(MOE_ERR_INVALID_ARG,
                "T must be >= 0 and d, E, k, f positive (T=%d d=%d E=%d k=%d f=%d)", p->T, p->d,
                p->E, p->k, p->f);
  if (p->k > p->E) return fail(MOE_ERR_INVALID_ARG, "k=%d exceeds E=%d", p->k, p->E);
  if (p->n_local <= 0 || p->expert_lo < 0 || (int64_t)p->expert_lo + p->n_local > p->E)
    return fail(MOE_ERR_INVALID_ARG, "local experts [%d, %d+%d) not inside [0, %d)", p->expert_lo,
                p->expert_lo, p->n_local, p->E);
  if (p->flags & ~(uint32_t)(MOE_F_WRITE_LOGITS | MOE_F_OVERLAP | MOE_F_FOLD_WEIGHT))
    return fail(MOE_ERR_INVALID_ARG, "unknown flag bits 0x%x", p->flags);
  if (p->dtype != MOE_DTYPE_F32 && p->dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "dtype %d not supported", p->dtype);
  if (p->k > 32) return fail(MOE_ERR_UNSUPPORTED, "k=%d > 32 not supported", p->k);
  if (p->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E=%d > 1024 not supported", p->E);
  if (p->d % 8 != 0 || p->f % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "d=%d and f=%d must be multiples of 8", p->d, p->f);
  const int64_t es = p->dtype == MOE_DTYPE_BF16 ? 2 : 4;
  if ((int64_t)p->d * p->f * es >= ((int64_t)1 << 31) || (int64_t)p->d * p->E * es >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "a weight matrix exceeds 2 GiB (d=%d f=%d E=%d)", p->d, p->f, p->E);
  const int64_t tk = (int64_t)p->T * p->k;
  if (tk >= (int64_t)1 << 30)
    return fail(MOE_ERR_UNSUPPORTED, "T*k=%lld too large", (long long)tk);
  moe::Prob q;
  q.T = p->T;
  q.d = p->d;
  q.E = p->E;
  q.k = p->k;
  q.f = p->f;
  q.lo = p->expert_lo;
  q.n = p->n_local;
  q.dtype = p->dtype;
  q.flags = p->flags;
  q.rows_max = (int64_t)p->T * (p->k < p->n_local ? p->k : p->n_local);
  *out = q;
  return MOE_OK;
}

#define NEED_PTR(ptr)                                                   \
  do {                                                                  \
    if (!(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #ptr);   \
  } while (0)
#define NEED_ALIGNED(ptr)                                                              \
  do {                                                                                 \
    if (!aligned16(ptr)) return fail(MOE_ERR_UNSUPPORTED, "%s is not 16-byte aligned", #ptr); \
  } while (0)

// Workspace layout of moe_layer (each region 256-byte aligned).
struct LayerWs {
  size_t route, idx, w, counts, offsets, perm, inv, disp, xp, h, yp, gemm, rs, total;
};

LayerWs layer_ws(const moe::Prob& p) {
  LayerWs L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  const size_t es = p.elem();
  L.route = take(moe::route_ws_bytes(p));
  L.idx = take(p.tk() * 4);
  L.w = take(p.tk() * 4);
  L.counts = take((size_t)p.E * 4);
  L.offsets = take((size_t)(p.n + 1) * 4);
  L.perm = take((size_t)p.rows_max * 4);
  L.inv = take(p.tk() * 4);
  L.disp = take(moe::dispatch_ws_bytes(p));
  L.xp = take((size_t)p.rows_max * p.d * es);
  L.h = take((size_t)p.rows_max * p.f * es);
  L.yp = take((size_t)p.rows_max * p.d * es);
  L.gemm = take(moe::expert_gemm_ws_bytes(p));
  L.rs = take((size_t)p.rows_max * 4);
  L.total = o;
  return L;
}

size_t call_ws_bytes(const moe::Prob& p, int32_t call) {
  if (p.T == 0) return 0;  // an empty batch launches no kernel that uses scratch
  switch (call) {
    case MOE_CALL_ROUTE: return moe::route_ws_bytes(p);
    case MOE_CALL_DISPATCH: return moe::dispatch_ws_bytes(p);
    case MOE_CALL_EXPERT_GEMM: return moe::expert_gemm_ws_bytes(p);
    case MOE_CALL_COMBINE: return 0;
    case MOE_CALL_LAYER: return layer_ws(p).total;
    case MOE_CALL_DISPATCH_PADDED: return moe::dispatch_padded_ws_bytes(p);
    case MOE_CALL_EXPERT_GEMM_PADDED: return moe::expert_gemm_ws_bytes(p);
    default: return 0;
  }
}

moe_status_t check_ws(const moe::Prob& p, int32_t call, const void* ws, size_t bytes) {
  const size_t need = call_ws_bytes(p, call);
  if (need == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  return MOE_OK;
}

// Capacity of the padded layout: 1 <= capacity <= T (no expert receives more
// than T assignments), and the padded buffers stay addressable.
moe_status_t check_capacity(const moe::Prob& q, int32_t capacity) {
  if (capacity <= 0 || capacity > q.T)
    return fail(MOE_ERR_INVALID_ARG, "capacity=%d outside [1, T=%d]", capacity, q.T);
  const int64_t rows = (int64_t)q.n * capacity;
  const int64_t wide = (int64_t)(q.d > q.f ? q.d : q.f) * q.elem();
  if (rows >= ((int64_t)1 << 31) || rows * wide >= ((int64_t)1 << 40))
    return fail(MOE_ERR_UNSUPPORTED, "n_local*capacity=%lld rows too large", (long long)rows);
  return MOE_OK;
}

// Shapes of the signalled GEMM: bf16 row-major A [M,K], B [K,N], C [M,N];
// N and K multiples of 8 (16-byte rows), B below 2 GiB and A's 256-row
// blocks below 4 GiB (32-bit buffer descriptors), M*N addressable.
moe_status_t check_signal_shape(int32_t M, int32_t N, int32_t K) {
  if (M <= 0 || N <= 0 || K <= 0)
    return fail(MOE_ERR_INVALID_ARG, "M=%d N=%d K=%d must be positive", M, N, K);
  if (N % 8 != 0 || K % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "N=%d and K=%d must be multiples of 8", N, K);
  if ((int64_t)K * N * 2 >= ((int64_t)1 << 31) || (int64_t)256 * K * 2 >= ((int64_t)1 << 32) ||
      (int64_t)M * N >= ((int64_t)1 << 40))
    return fail(MOE_ERR_UNSUPPORTED, "GEMM too large (M=%d N=%d K=%d)", M, N, K);
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct StreamEvents {
  hipEvent_t a = nullptr, b = nullptr;
  int device = -1;
};
thread_local StreamEvents g_ev;

hipError_t events_for_current_device(StreamEvents& ev) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (ev.device == dev && ev.a && ev.b) return hipSuccess;
  if (ev.a) (void)hipEventDestroy(ev.a);
  if (ev.b) (void)hipEventDestroy(ev.b);
  ev.a = ev.b = nullptr;
  e = hipEventCreateWithFlags(&ev.a, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ev.b, hipEventDisableTiming);
  if (e == hipSuccess) ev.device = dev;
  return e;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "libmoe 0.2 gfx950"; }

// events the next moe_layer call on this thread records around its expert GEMM
thread_local hipEvent_t g_gemm_ev[2] = {nullptr, nullptr};

moe_status_t moe_layer_set_gemm_events(void* before, void* after) {
  g_gemm_ev[0] = reinterpret_cast<hipEvent_t>(before);
  g_gemm_ev[1] = reinterpret_cast<hipEvent_t>(after);
  g_err.clear();
  return MOE_OK;
}

size_t moe_layer_ws_offset(const moe_problem_t* p, int32_t what) {
  moe::Prob q;
  if (check_problem(p, &q) != MOE_OK) return (size_t)-1;
  if (q.T == 0) {
    fail(MOE_ERR_INVALID_ARG, "an empty batch has no layer workspace");
    return (size_t)-1;
  }
  const LayerWs L = layer_ws(q);
  switch (what) {
    case MOE_WS_H: g_err.clear(); return L.h;
    case MOE_WS_Y_PACKED: g_err.clear(); return L.yp;
    default:
      fail(MOE_ERR_INVALID_ARG, "unknown workspace region %d", what);
      return (size_t)-1;
  }
}

size_t moe_workspace_bytes(const moe_problem_t* p, int32_t call) {
  moe::Prob q;
  if (check_problem(p, &q) != MOE_OK) return 0;
  if (call < MOE_CALL_ROUTE || call > MOE_CALL_EXPERT_GEMM_PADDED) {
    fail(MOE_ERR_INVALID_ARG, "unknown call %d", call);
    return 0;
  }
  g_err.clear();
  return call_ws_bytes(q, call);
}

moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_gate,
                       const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                       void* workspace, size_t workspace_bytes, void* stream) {
  moe::Prob q;
  moe_status_t st = check_problem(p, &q);
  if (st != MOE_OK) return st;
  NEED_PTR(w_gate);
  NEED_ALIGNED(w_gate);
  if (q.T == 0) return ok();  // empty batch: nothing to route
  NEED_PTR(x);
  NEED_PTR(topk_idx);
  NEED_PTR(topk_w);
  NEED_ALIGNED(x);
  if ((st = check_ws(q, MOE_CALL_ROUTE, workspace, workspace_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return hip_status(moe::launch_route(q, x, w_gate, bias, logits, topk_idx, topk_w, workspace,
                                      (hipStream_t)stream),
                    "moe_route");
}

moe_status_t moe_dispatch(const moe_problem_t* p, const int32_t* topk_idx, const void* x,
                          int32_t* counts_all, int32_t* offsets, int32_t* perm, int32_t* inv,
                          void* x_packed, void* workspace, size_t workspace_bytes, void* stream) {
  moe::Prob q;
  moe_status_t st = check_problem(p, &q);
  if (st != MOE_OK) return st;
  NEED_PTR(counts_all);
  NEED_PTR(offsets);
  if (q.T == 0) {  // empty batch: all counts and offsets are zero
    (void)hipGetLastError();
    return hip_status(moe::launch_clear_index(q, counts_all, offsets, (hipStream_t)stream),
                      "moe_dispatch");
  }
  NEED_PTR(topk_idx);
  NEED_PTR(x);
  NEED_PTR(perm);
  NEED_PTR(inv);
  NEED_PTR(x_packed);
  NEED_ALIGNED(x);
  NEED_ALIGNED(x_packed);
  if ((st = check_ws(q, MOE_CALL_DISPATCH, workspace, workspace_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = moe::launch_dispatch_index(q, topk_idx, counts_all, offsets, perm, inv, workspace, s);
  if (e == hipSuccess) e = moe::launch_gather(q, x, offsets, perm, x_packed, 0, q.n, s);
  return hip_status(e, "moe_dispatch");
}

moe_status_t moe_dispatch_noalloc(const moe_problem_t* p, const int32_t* topk_idx, const void* x,
                                  int32_t* counts_all, int32_t* offsets, int32_t* perm,
                                  int32_t* inv, void* x_packed, void* stream) {
  moe::Prob q;
  moe_status_t st = check_problem(p, &q);
  if (st != MOE_OK) return st;
  NEED_PTR(counts_all);
  NEED_PTR(offsets);
  if (q.T == 0) {  // empty batch: all counts and offsets are zero, no scratch used
    (void)hipGetLastError();
    return hip_status(moe::launch_clear_index(q, counts_all, offsets, (hipStream_t)stream),
                      "moe_dispatch_noalloc");
  }
  NEED_PTR(topk_idx);
  NEED_PTR(x);
  NEED_PTR(perm);
  NEED_PTR(inv);
  NEED_PTR(x_packed);
  NEED_ALIGNED(x);
  NEED_ALIGNED(x_packed);
  const size_t need = moe::dispatch_ws_bytes(q);
  if (need > moe::dispatch_scratch_bytes())
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_dispatch_noalloc: needs %zu bytes of scratch (ceil(T*k/1024)*E*4), the static "
                "array holds %zu",
                need, moe::dispatch_scratch_bytes());
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  void* scr = nullptr;
  hipError_t e = moe::dispatch_scratch(&scr);
  if (e == hipSuccess)
    e = moe::launch_dispatch_index(q, topk_idx, counts_all, offsets, perm, inv, scr, s);
  if (e == hipSuccess) e = moe::launch_gather(q, x, offsets, perm, x_packed, 0, q.n, s);
  return hip_status(e, "moe_dispatch_noalloc");
}

moe_status_t moe_expert_gemm(const moe_problem_t* p, const void* x_packed, const int32_t* offsets,
                             const void* w1, const void* w3, const void* w2, void* h,
                             void* y_packed, void* workspace, size_t workspace_bytes,
                             void* stream) {
  moe::Prob q;
  moe_status_t st = check_problem(p, &q);
  if (st != MOE_OK) return st;
  NEED_PTR(offsets);
  NEED_PTR(w1);
  NEED_PTR(w3);
  NEED_PTR(w2);
  NEED_ALIGNED(w1);
  NEED_ALIGNED(w3);
  NEED_ALIGNED(w2);
  if (q.T == 0) return ok();  // empty batch: no rows
  NEED_PTR(x_packed);
  NEED_PTR(h);
  NEED_PTR(y_packed);
  NEED_ALIGNED(x_packed);
  NEED_ALIGNED(h);
  NEED_ALIGNED(y_packed);
  if ((st = check_ws(q, MOE_CALL_EXPERT_GEMM, workspace, workspace_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return hip_status(moe::launch_expert_gemm(q, x_packed, offsets, w1, w3, w2, h, y_packed, workspace,
                                            0, q.n, (hipStream_t)stream),
                    "moe_expert_gemm");
}

moe_status_t moe_dispatch_padded(const moe_problem_t* p, int32_t capacity, const int32_t* topk_idx,
                                 const void* x, int32_t* counts_all, int32_t* offsets, int32_t* perm,
                                 int32_t* inv, void* x_packed, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  moe::Prob q;
  moe_status_t st = check_problem(p, &q);
  if (st != MOE_OK) return st;
  if ((st = check_capacity(q, capacity)) != MOE_OK) return st;
  NEED_PTR(topk_idx);
  NEED_PTR(x);
  NEED_PTR(counts_all);
  NEED_PTR(offsets);
  NEED_PTR(perm);
  NEED_PTR(inv);
  NEED_PTR(x_packed);
  NEED_ALIGNED(x);
  NEED_ALIGNED(x_packed);
  if ((st = check_ws(q, MOE_CALL_DISPATCH_PADDED, workspace, workspace_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return hip_status(moe::launch_dispatch_padded(q, capacity, topk_idx, counts_all, offsets, perm, inv,
                                                x, x_packed, workspace, (hipStream_t)stream),
                    "moe_dispatch_padded");
}

moe_status_t moe_expert_gemm_padded(const moe_problem_t* p, int32_t capacity, const void* x_packed,
                                    const int32_t* offsets, const void* w1, const void* w3,
                                    const void* w2, void* h, void* y_packed, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  moe::Prob q;
  moe_status_t st = check_problem(p, &q);
  if (st != MOE_OK) return st;
  if ((st = check_capacity(q, capacity)) != MOE_OK) return st;
  NEED_PTR(x_packed);
  NEED_PTR(offsets);
  NEED_PTR(w1);
  NEED_PTR(w3);
  NEED_PTR(w2);
  NEED_PTR(h);
  NEED_PTR(y_packed);
  NEED_ALIGNED(x_packed);
  NEED_ALIGNED(w1);
  NEED_ALIGNED(w3);
  NEED_ALIGNED(w2);
  NEED_ALIGNED(h);
  NEED_ALIGNED(y_packed);
  if ((st = check_ws(q, MOE_CALL_EXPERT_GEMM_PADDED, workspace, workspace_bytes)) != MOE_OK) return st;
  q.rows_max = (int64_t)q.n * capacity;
  q.seg_rows = capacity;
  (void)hipGetLastError();
  return hip_status(moe::launch_expert_gemm(q, x_packed, offsets, w1, w3, w2, h, y_packed, workspace,
                                            0, q.n, (hipStream_t)stream),
                    "moe_expert_gemm_padded");
}

int64_t moe_gemm_signal_tiles(int32_t M, int32_t N) {
  if (M <= 0 || N <= 0) {
    fail(MOE_ERR_INVALID_ARG, "M=%d and N=%d must be positive", M, N);
    return 0;
  }
  ok();
  return moe::gemm_signal_tiles(M, N);
}

moe_status_t moe_gemm_signal(int32_t M, int32_t N, int32_t K, const void* A, const void* B, void* C,
                             uint32_t* flags, uint32_t epoch, int32_t scope, void* stream) {
  moe_status_t st;
  if ((st = check_signal_shape(M, N, K)) != MOE_OK) return st;
  NEED_PTR(A);
  NEED_PTR(B);
  NEED_PTR(C);
  NEED_PTR(flags);
  NEED_ALIGNED(A);
  NEED_ALIGNED(B);
  NEED_ALIGNED(C);
  if (epoch == 0) return fail(MOE_ERR_INVALID_ARG, "epoch must be nonzero");
  if (scope != MOE_SCOPE_AGENT && scope != MOE_SCOPE_SYSTEM)
    return fail(MOE_ERR_INVALID_ARG, "scope %d is neither MOE_SCOPE_AGENT nor MOE_SCOPE_SYSTEM", scope);
  (void)hipGetLastError();
  return hip_status(moe::launch_gemm_signal(M, N, K, A, B, C, flags, epoch, scope, (hipStream_t)stream),
                    "moe_gemm_signal");
}

moe_status_t moe_tile_forward(int32_t M, int32_t N, const void* C, void* dst, const uint32_t* flags,
                              uint32_t epoch, uint32_t spin_limit, int32_t scope, uint32_t* timeouts,
                              int32_t workgroups, void* stream) {
  moe_status_t st;
  if ((st = check_signal_shape(M, N, 8)) != MOE_OK) return st;
  NEED_PTR(C);
  NEED_PTR(dst);
  NEED_PTR(flags);
  NEED_PTR(timeouts);
  NEED_ALIGNED(C);
  NEED_ALIGNED(dst);
  if (epoch == 0) return fail(MOE_ERR_INVALID_ARG, "epoch must be nonzero");
  if (spin_limit == 0) return fail(MOE_ERR_INVALID_ARG, "spin_limit must be positive");
  if (scope != MOE_SCOPE_AGENT && scope != MOE_SCOPE_SYSTEM)
    return fail(MOE_ERR_INVALID_ARG, "scope %d is neither MOE_SCOPE_AGENT nor MOE_SCOPE_SYSTEM", scope);
  if (workgroups <= 0 || workgroups > 1024)
    return fail(MOE_ERR_INVALID_ARG, "workgroups=%d outside [1, 1024]", workgroups);
  (void)hipGetLastError();
  return hip_status(moe::launch_tile_forward(M, N, C, dst, flags, epoch, spin_limit, scope, timeouts,
                                             workgroups, (hipStream_t)stream),
                    "moe_tile_forward");
}

moe_status_t moe_combine(const moe_problem_t* p, const void* y_packed, const int32_t* inv,
                         const float* topk_w, void* y, void* stream) {
  moe::Prob q;
  moe_status_t st = check_problem(p, &q);
  if (st != MOE_OK) return st;
  if (q.T == 0) return ok();  // empty batch: no output rows
  NEED_PTR(y_packed);
  NEED_PTR(inv);
  NEED_PTR(y);            // topk_w may be NULL: the rows are summed unweighted
  NEED_ALIGNED(y_packed);
  NEED_ALIGNED(y);
  (void)hipGetLastError();
  return hip_status(moe::launch_combine(q, y_packed, inv, topk_w, y, (hipStream_t)stream),
                    "moe_combine");
}

moe_status_t moe_layer(const moe_problem_t* p, const void* x, const void* w_gate,
                       const float* bias, const void* w1, const void* w3, const void* w2,
                       void* y, const moe_routing_out_t* routing_out, void* workspace,
                       size_t workspace_bytes, void* stream, void* stream2) {
  // the measurement hook is consumed by this call whatever its outcome
  const hipEvent_t ev_before = g_gemm_ev[0], ev_after = g_gemm_ev[1];
  g_gemm_ev[0] = g_gemm_ev[1] = nullptr;
  moe::Prob q;
  moe_status_t st = check_problem(p, &q);
  if (st != MOE_OK) return st;
  NEED_PTR(w_gate);
  NEED_PTR(w1);
  NEED_PTR(w3);
  NEED_PTR(w2);
  NEED_ALIGNED(w_gate);
  NEED_ALIGNED(w1);
  NEED_ALIGNED(w3);
  NEED_ALIGNED(w2);
  if (q.T == 0) {  // empty batch: only the caller's counts and offsets are written (zeros)
    (void)hipGetLastError();
    return hip_status(moe::launch_clear_index(q, routing_out ? routing_out->counts_all : nullptr,
                                              routing_out ? routing_out->offsets : nullptr,
                                              (hipStream_t)stream),
                      "moe_layer");
  }
  NEED_PTR(x);
  NEED_PTR(y);
  NEED_ALIGNED(x);
  NEED_ALIGNED(y);
  if ((q.flags & MOE_F_WRITE_LOGITS) && !(routing_out && routing_out->logits))
    return fail(MOE_ERR_INVALID_ARG, "MOE_F_WRITE_LOGITS needs routing_out->logits");
  if ((st = check_ws(q, MOE_CALL_LAYER, workspace, workspace_bytes)) != MOE_OK) return st;

  const LayerWs L = layer_ws(q);
  char* ws = static_cast<char*>(workspace);
  auto pick = [&](auto* user, size_t off) {
    using T = std::remove_pointer_t<decltype(user)>;
    return user ? user : reinterpret_cast<T*>(ws + off);
  };
  const moe_routing_out_t none{};
  const moe_routing_out_t& ro = routing_out ? *routing_out : none;
  const bool fold = (q.flags & MOE_F_FOLD_WEIGHT) != 0;
  int32_t* idx = pick(ro.topk_idx, L.idx);
  float* w = pick(ro.topk_w, L.w);
  int32_t* counts = pick(ro.counts_all, L.counts);
  int32_t* offsets = pick(ro.offsets, L.offsets);
  int32_t* perm = pick(ro.perm, L.perm);
  int32_t* inv = pick(ro.inv, L.inv);
  float* logits = (q.flags & MOE_F_WRITE_LOGITS) ? ro.logits : nullptr;
  void* xp = ws + L.xp;
  void* h = ws + L.h;
  void* yp = ws + L.yp;
  hipStream_t s0 = (hipStream_t)stream;
  hipStream_t s1 = (hipStream_t)stream2;
  const bool overlap = (q.flags & MOE_F_OVERLAP) && s1 != nullptr && q.n >= 2;

  (void)hipGetLastError();
  // top-k fills the dispatch chunk histograms where the router supports it,
  // which saves dispatch its histogram kernel
  bool hist_done = false;
  int32_t* chunk_hist = reinterpret_cast<int32_t*>(ws + L.disp);
  const int64_t hist_elems = (int64_t)(moe::dispatch_ws_bytes(q) / sizeof(int32_t));
  hipError_t e = moe::launch_route(q, x, w_gate, bias, logits, idx, w, ws + L.route, s0, chunk_hist,
                                   hist_elems, &hist_done);
  // with the weight folded into the down projection, the scatter also writes
  // each packed row's routing weight
  float* rscale = fold ? reinterpret_cast<float*>(ws + L.rs) : nullptr;
  if (e == hipSuccess)
    e = moe::launch_dispatch_index(q, idx, counts, offsets, perm, inv, ws + L.disp, s0, hist_done,
                                   fold ? w : nullptr, rscale);
  if (e != hipSuccess) return hip_status(e, "moe_layer routing");
  // bf16 with x inside one 32-bit buffer descriptor: GEMM-1 gathers the x rows
  // itself through perm, so x_packed is never written
  const bool fused = q.dtype == 1 && (int64_t)q.T * q.d * 2 < (int64_t(1) << 31);
  if (!overlap && fused) {
    if (ev_before) e = hipEventRecord(ev_before, s0);
    if (e == hipSuccess)
      e = moe::launch_expert_gemm(q, x, offsets, w1, w3, w2, h, yp, ws + L.gemm, 0, q.n, s0, perm,
                                rscale);
  } else if (!overlap) {
    e = moe::launch_gather(q, x, offsets, perm, xp, 0, q.n, s0);
    if (e == hipSuccess && ev_before) e = hipEventRecord(ev_before, s0);
    if (e == hipSuccess)
      e = moe::launch_expert_gemm(q, xp, offsets, w1, w3, w2, h, yp, ws + L.gemm, 0, q.n, s0,
                                  nullptr, rscale);
  } else {
    // two-stream dispatch overlap: the upper half of the local experts is
    // packed on s1 while the lower half's GEMMs run on s0.
    const int half = q.n / 2;
    e = events_for_current_device(g_ev);
    if (e == hipSuccess) e = hipEventRecord(g_ev.a, s0);
    if (e == hipSuccess) e = hipStreamWaitEvent(s1, g_ev.a, 0);
    if (e == hipSuccess) e = moe::launch_gather(q, x, offsets, perm, xp, half, q.n, s1);
    if (e == hipSuccess) e = hipEventRecord(g_ev.b, s1);
    if (e == hipSuccess) e = moe::launch_gather(q, x, offsets, perm, xp, 0, half, s0);
    if (e == hipSuccess)
      e = moe::launch_expert_gemm(q, xp, offsets, w1, w3, w2, h, yp, ws + L.gemm, 0, half, s0,
                                  nullptr, rscale);
    if (e == hipSuccess) e = hipStreamWaitEvent(s0, g_ev.b, 0);
    if (e == hipSuccess)
      e = moe::launch_expert_gemm(q, xp, offsets, w1, w3, w2, h, yp, ws + L.gemm, half, q.n, s0,
                                  nullptr, rscale);
  }
  if (e == hipSuccess && ev_after && !overlap) e = hipEventRecord(ev_after, s0);
  if (e == hipSuccess) e = moe::launch_combine(q, yp, inv, fold ? nullptr : w, y, s0);
  return hip_status(e, "moe_layer");
}

}  // extern "C"
