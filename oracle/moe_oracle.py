"""Plain, slow CPU oracle of one GPU's share of an MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What is computed.  The workload is the DeepSeek-V3 MoE layer of "CUCo: An
Agentic Framework for Compute and Communication Co-design" (Abstract; Table 4,
row "MoE Dispatch/Combine": dispatch, local ("self") expert compute, combine,
with variable-size unpadded per-peer transfers).  The pages give no formulas,
so every step below is the plain textbook MoE layer, restricted to this GPU's
local experts [expert_lo, expert_lo + n_local):

  1. logits  L = x . W_g (+ b)                  exact, rounded once to fp32
  2. top-k   the k largest logits per token, in descending order, ties to the
             lower expert index; weights = softmax over the selected k
  3. counts  per-expert histogram over all E experts
  4. offsets exclusive prefix sum of the local counts
  5. perm    stable counting sort of the local assignments a = t*k + j by
             local expert (ties in ascending a); inv[perm[p]] = p, else -1
  6. gather  x_packed[p] = x[perm[p] // k]
  7. experts h = rnd(SiLU(X W1) * (X W3)),  y_packed = rnd(h W2), per segment
  8. combine y[t] = rnd(sum over local slots j of w[t,j] * y_packed[inv[t,j]])

Arithmetic is float64 throughout.  ``rnd`` is round-to-nearest-even to bf16 for
bf16 workloads (the points where the GPU path stores bf16: h, y_packed, y) and
the identity for fp32 workloads.  bf16 tensors are held as uint16 bit patterns
and widened exactly.

Readings of points the pages leave open (each is listed with its reason in the
design notes): softmax top-k renormalised over the k selected experts; selection
on the fp32 logit (not on a rounded probability); bias added before both
selection and softmax; -0.0 equals +0.0 in comparisons; remote slots are dropped
without renormalising the local ones; a token with no local slot gets an exact
zero row; SiLU gates the x.W1 branch; the gate weight is applied in combine.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "widen",
    "round_bf16",
    "to_bf16_bits",
    "rnd",
    "router_logits",
    "topk_softmax",
    "expert_counts",
    "local_dispatch",
    "local_dispatch_padded",
    "gather_rows",
    "gather_rows_padded",
    "silu",
    "swiglu_experts",
    "down_projection",
    "combine",
    "moe_layer",
    "moe_layer_padded",
    "gemm",
    "token_outputs",
]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor (bf16 bit patterns or float32)."""
    a = np.asarray(a)
    if dtype == "bf16":
        u32 = a.astype(np.uint32) << np.uint32(16)
        return u32.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 has 8 significant bits and float32's exponent range.  A value with
    frexp exponent e (x = m * 2**e, 0.5 <= |m| < 1) sits on a grid of spacing
    2**(e-8); below the smallest normal (2**-126) the spacing stays 2**-133.
    Scaling by a power of two is exact, and ``np.rint`` rounds half to even.
    Magnitudes past the largest finite bf16 (whose own spacing is 2**120)
    round to +-inf, ties at the boundary included, as IEEE does.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.rint(x / q) * q
        big = np.abs(r) >= 2.0 ** 128
    r = np.where(big, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values that already lie on the bf16 grid."""
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)  # exact on the grid
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rnd(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# 1. router logits
# ---------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_gate: np.ndarray, dtype: str,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """L[t,e] = sum_i x[t,i] * W_g[i,e] (+ b[e]), exact in float64, rounded once
    to float32.  The pages name only "sparse routing" (gist.science summary,
    §4 Results); the projection itself is the standard MoE gate."""
    L = widen(x, dtype) @ widen(w_gate, dtype)
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return L.astype(np.float32)


# ---------------------------------------------------------------------------
# 2. top-k gating
# ---------------------------------------------------------------------------
def topk_softmax(logits: np.ndarray, k: int):
    """Top-k experts per token and their renormalised softmax weights.

    Selection: experts ordered by (logit descending, index ascending); the
    first k are slots 0..k-1.  Comparisons are IEEE (+0.0 equals -0.0).
    Weights: w_j = exp(l_j - m) / sum_{i<k} exp(l_i - m) with m the slot-0
    logit, in float64, rounded to float32.  This equals the full softmax over
    all E experts renormalised over the selected k (the full denominator
    cancels).
    """
    L = np.asarray(logits, dtype=np.float32).astype(np.float64) + 0.0  # -0 -> +0
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("k out of range")
    ar = np.broadcast_to(np.arange(E), L.shape)
    order = np.lexsort((ar, -L), axis=-1)          # primary: -L, secondary: index
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)


# ---------------------------------------------------------------------------
# 3-5. dispatch indices
# ---------------------------------------------------------------------------
def expert_counts(topk_idx: np.ndarray, E: int) -> np.ndarray:
    """counts_all[e] = number of (token, slot) assignments to expert e."""
    return np.bincount(np.asarray(topk_idx).ravel().astype(np.int64), minlength=E).astype(np.int32)


def local_dispatch(topk_idx: np.ndarray, E: int, expert_lo: int, n_local: int):
    """Histogram, prefix scan and stable permutation for the local experts.

    The pages' MoE strategy moves variable-size, unpadded per-peer blocks
    (CUCo, Table 4, "variable-size per-peer transfers"); on one GPU that is a
    packed buffer of expert-contiguous segments with no padding.

    Returns (counts_all int32[E], offsets int32[n_local+1], perm int32[A],
    inv int32[T*k]).
    """
    flat = np.asarray(topk_idx).ravel().astype(np.int64)
    counts_all = expert_counts(flat, E)
    le = flat - expert_lo
    local_a = np.nonzero((le >= 0) & (le < n_local))[0]
    order = np.argsort(le[local_a], kind="stable")
    perm = local_a[order].astype(np.int32)
    offsets = np.zeros(n_local + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts_all[expert_lo:expert_lo + n_local])
    inv = np.full(flat.shape[0], -1, dtype=np.int32)
    inv[perm] = np.arange(perm.shape[0], dtype=np.int32)
    return counts_all, offsets.astype(np.int32), perm, inv


def gather_rows(x: np.ndarray, perm: np.ndarray, k: int) -> np.ndarray:
    """x_packed[p] = x[perm[p] // k] (a plain copy of stored values)."""
    return np.asarray(x)[np.asarray(perm, dtype=np.int64) // k]


def local_dispatch_padded(topk_idx: np.ndarray, E: int, expert_lo: int, n_local: int,
                          capacity: int):
    """Padded fixed-capacity layout: the per-expert padded buffers that CUCo
    (Table 4, "MoE Dispatch/Combine") names as a bottleneck on imbalanced
    ranks.  Local expert e owns rows [e*C, (e+1)*C).  Walking the assignments
    a = t*k + j in ascending order, a local assignment takes the next free row
    of its expert while one is left; later ones are dropped.  Rows left over
    are padding.

    Returns (counts_all int32[E], offsets int32[n_local+1] = e*C,
    perm int32[n_local*C] with -1 for padding, inv int32[T*k] with -1 for
    non-local and dropped assignments).
    """
    flat = np.asarray(topk_idx).ravel().astype(np.int64)
    counts_all = expert_counts(flat, E)
    C = int(capacity)
    perm = np.full(n_local * C, -1, dtype=np.int32)
    inv = np.full(flat.shape[0], -1, dtype=np.int32)
    used = [0] * n_local
    for a in range(flat.shape[0]):
        e = int(flat[a]) - expert_lo
        if 0 <= e < n_local and used[e] < C:
            q = e * C + used[e]
            perm[q] = a
            inv[a] = q
            used[e] += 1
    offsets = (np.arange(n_local + 1, dtype=np.int64) * C).astype(np.int32)
    return counts_all, offsets, perm, inv


def gather_rows_padded(x: np.ndarray, perm: np.ndarray, k: int) -> np.ndarray:
    """x_packed[q] = x[perm[q] // k]; a padding row (perm -1) is all-zero bits."""
    x = np.asarray(x)
    perm = np.asarray(perm, dtype=np.int64)
    out = np.zeros((perm.shape[0],) + x.shape[1:], dtype=x.dtype)
    keep = perm >= 0
    out[keep] = x[perm[keep] // k]
    return out


# ---------------------------------------------------------------------------
# 6-7. SwiGLU experts
# ---------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def _expert_rows(X: np.ndarray, W1: np.ndarray, W3: np.ndarray, W2: np.ndarray, dtype: str,
                 rounded: bool = True):
    """One expert on float64 rows X: returns (h, y) after the rounding points
    (with ``rounded=False``, in plain float64 with no rounding point)."""
    r = dtype if rounded else "f64"
    a1 = X @ W1
    a3 = X @ W3
    h = rnd(silu(a1) * a3, r)
    y = rnd(h @ W2, r)
    return h, y


def swiglu_experts(x_packed: np.ndarray, offsets: np.ndarray, w1, w3, w2, dtype: str):
    """Per local expert e, rows [offsets[e], offsets[e+1]) of x_packed:
    h = rnd(SiLU(X W1_e) * (X W3_e)), y_packed = rnd(h W2_e).  float64 values."""
    Xp = widen(x_packed, dtype)
    A = Xp.shape[0]
    n_local = len(offsets) - 1
    f = np.asarray(w1).shape[2]
    d = np.asarray(w2).shape[2]
    h = np.zeros((A, f), dtype=np.float64)
    yp = np.zeros((A, d), dtype=np.float64)
    for e in range(n_local):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        h[r0:r1], yp[r0:r1] = _expert_rows(Xp[r0:r1], widen(w1[e], dtype), widen(w3[e], dtype),
                                           widen(w2[e], dtype), dtype)
    return h, yp


def down_projection(h: np.ndarray, offsets: np.ndarray, w2, dtype: str,
                    row_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """The second half of step 7 on its own: y_packed[R_e] = rnd(h[R_e] W2_e)
    for float64 values h (on the storage grid), per local expert segment.

    With ``row_scale`` (one float64 factor per packed row), each row's exact
    product is multiplied by its factor before the one rounding:
    y_packed[p] = rnd(s[p] * (h[p] W2_e)).  This is the layout in which the
    gate weight of a row's assignment is applied in the down projection's
    epilogue instead of in combine (the pages name the sequential
    dispatch/compute/combine phases as the MoE bottleneck, CUCo Table 4, row
    "MoE Dispatch/Combine"; folding the weight into the expert output lets
    combine be a plain sum)."""
    h = np.asarray(h, dtype=np.float64)
    n_local = len(offsets) - 1
    d = np.asarray(w2).shape[2]
    yp = np.zeros((h.shape[0], d), dtype=np.float64)
    for e in range(n_local):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        prod = h[r0:r1] @ widen(w2[e], dtype)
        if row_scale is not None:
            prod = np.asarray(row_scale, dtype=np.float64)[r0:r1, None] * prod
        yp[r0:r1] = rnd(prod, dtype)
    return yp


# ---------------------------------------------------------------------------
# 8. combine
# ---------------------------------------------------------------------------
def combine(y_packed: np.ndarray, inv: np.ndarray, topk_w: Optional[np.ndarray], dtype: str,
            k: Optional[int] = None) -> np.ndarray:
    """y[t] = rnd(sum_j w[t,j] * y_packed[inv[t*k+j]]) over local slots, in slot
    order, float64; exact zero rows for tokens with no local slot.  This is the
    pages' "combine" (CUCo, Table 4), un-permute plus weighted sum.

    ``topk_w=None`` is the plain sum of the local slots' rows (weights already
    applied in the down projection, see ``down_projection``); then ``k`` gives
    the slots per token."""
    if topk_w is None:
        if k is None:
            raise ValueError("k is needed when topk_w is None")
        T = np.asarray(inv).shape[0] // k
        W = np.ones((T, k), dtype=np.float64)
    else:
        W = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    T, k = W.shape
    inv2 = np.asarray(inv).reshape(T, k)
    d = y_packed.shape[1]
    acc = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        m = inv2[:, j] >= 0
        acc[m] += W[m, j:j + 1] * y_packed[inv2[m, j]]
    return rnd(acc, dtype)


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------
def moe_layer(p, inputs: Dict[str, np.ndarray], routing: Optional[Dict[str, np.ndarray]] = None,
              with_experts: bool = True, fold_weight: bool = False) -> Dict[str, np.ndarray]:
    """Steps 1-8 for problem ``p`` (fields T, d, E, k, f, expert_lo, n_local,
    dtype).  If ``routing`` supplies topk_idx/topk_w (for instance the GPU's),
    steps 3-8 follow that routing instead of the oracle's own (so that a
    legitimate near-tie flip in step 2 cannot cascade).

    ``fold_weight``: the gate weight of each packed row's assignment scales
    that row in the down projection, before its rounding
    (y_packed[p] = rnd(w[perm[p]] * (h[p] W2_e))), and combine sums the rows
    unweighted.  It moves one rounding point; the exact result is the same."""
    out: Dict[str, np.ndarray] = {}
    L = router_logits(inputs["x"], inputs["w_gate"], p.dtype, inputs.get("bias"))
    out["logits"] = L
    idx, w = topk_softmax(L, p.k)
    out["topk_idx"], out["topk_w"] = idx, w
    if routing is not None:
        idx, w = routing["topk_idx"], routing["topk_w"]
    counts_all, offsets, perm, inv = local_dispatch(idx, p.E, p.expert_lo, p.n_local)
    out.update(counts_all=counts_all, offsets=offsets, perm=perm, inv=inv)
    xp = gather_rows(inputs["x"], perm, p.k)
    out["x_packed"] = xp
    if with_experts:
        h, yp = swiglu_experts(xp, offsets, inputs["w1"], inputs["w3"], inputs["w2"], p.dtype)
        if fold_weight:
            wf = np.asarray(w, dtype=np.float32).astype(np.float64).ravel()
            yp = down_projection(h, offsets, inputs["w2"], p.dtype,
                                 row_scale=wf[np.asarray(perm, dtype=np.int64)])
            out["h"], out["y_packed"] = h, yp
            out["y"] = combine(yp, inv, None, p.dtype, k=p.k)
        else:
            out["h"], out["y_packed"] = h, yp
            out["y"] = combine(yp, inv, w, p.dtype)
    return out


def moe_layer_padded(p, inputs: Dict[str, np.ndarray], capacity: int,
                     routing: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """The layer over the padded fixed-capacity layout: as ``moe_layer`` with
    step 5-6 replaced by ``local_dispatch_padded`` / ``gather_rows_padded``
    (dropped assignments contribute nothing to y; padding rows run through
    the experts as zero rows)."""
    out: Dict[str, np.ndarray] = {}
    L = router_logits(inputs["x"], inputs["w_gate"], p.dtype, inputs.get("bias"))
    idx, w = topk_softmax(L, p.k)
    if routing is not None:
        idx, w = routing["topk_idx"], routing["topk_w"]
    out["topk_idx"], out["topk_w"] = idx, w
    counts_all, offsets, perm, inv = local_dispatch_padded(idx, p.E, p.expert_lo, p.n_local, capacity)
    out.update(counts_all=counts_all, offsets=offsets, perm=perm, inv=inv)
    xp = gather_rows_padded(inputs["x"], perm, p.k)
    out["x_packed"] = xp
    h, yp = swiglu_experts(xp, offsets, inputs["w1"], inputs["w3"], inputs["w2"], p.dtype)
    out["h"], out["y_packed"] = h, yp
    out["y"] = combine(yp, inv, w, p.dtype)
    return out


def gemm(A: np.ndarray, B: np.ndarray, dtype: str) -> np.ndarray:
    """C = rnd(A B): the plain product of the GEMM + AllGather workload's
    compute half (CUCo, Table 4, row "GEMM + AllGather"), float64, rounded once
    to the storage dtype."""
    return rnd(widen(A, dtype) @ widen(B, dtype), dtype)


def token_outputs(p, inputs: Dict[str, np.ndarray], topk_idx: np.ndarray, topk_w: np.ndarray,
                  tokens: Sequence[int], rounded: bool = True) -> np.ndarray:
    """Layer output rows y[t] for selected tokens only, under the given routing.

    Each token's output depends only on its own row of x and its own routing
    (the expert GEMM is row-independent), so this equals the corresponding
    rows of ``moe_layer`` and lets a full-size run be checked on a sample.

    ``rounded=False`` skips the three rounding points of steps 7-8 (h,
    y_packed, y) and returns the exact float64 layer on the same bf16 inputs:
    a diagnostic of how far the stored-precision result sits from the exact
    one, never a parity bar (the parity bar is the rounded result above).
    """
    dt = p.dtype
    rt = dt if rounded else "f64"
    tokens = list(tokens)
    X = widen(np.asarray(inputs["x"])[tokens], dt)
    idx = np.asarray(topk_idx)
    W = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    # expert output of every (sampled token, local slot), one expert at a time
    # so that only one expert's float64 weights are held at once
    yslot = {}
    for e in range(p.n_local):
        pairs = [(r, j) for r, t in enumerate(tokens) for j in range(p.k)
                 if int(idx[t, j]) - p.expert_lo == e]
        if not pairs:
            continue
        rows = np.array([r for r, _ in pairs])
        _, y = _expert_rows(X[rows], widen(inputs["w1"][e], dt), widen(inputs["w3"][e], dt),
                            widen(inputs["w2"][e], dt), dt, rounded)
        for q, rj in enumerate(pairs):
            yslot[rj] = y[q]
    out = np.zeros((len(tokens), p.d), dtype=np.float64)
    for r, t in enumerate(tokens):
        acc = np.zeros(p.d, dtype=np.float64)
        for j in range(p.k):                     # slot order
            if (r, j) in yslot:
                acc += W[t, j] * yslot[(r, j)]
        out[r] = rnd(acc, rt)
    return out
