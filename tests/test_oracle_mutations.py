"""Planted mistakes in the oracle (CPU only): each must make some pin fail.

Every mutation is a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, an unstable sort, a different rounding rule).  The
mutated function replaces the real one in the oracle module for the duration
of the test, so the oracle's internal calls see it too.
"""
import numpy as np
import pytest

import oracle.moe_oracle as O
from tests import oracle_pins

_real = {name: getattr(O, name) for name in O.__all__}


def _round_half_away(x):
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    return np.sign(x) * np.floor(np.abs(x / q) + 0.5) * q


def _round_via_f32(x):
    return _real["round_bf16"](np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64))


def _topk_ties_high(L, k):
    L = np.asarray(L, dtype=np.float32).astype(np.float64)
    E = L.shape[1]
    idx, w = _real["topk_softmax"](L[:, ::-1].copy(), k)
    idx = (E - 1 - idx).astype(np.int32)
    return idx, w


def _topk_full_softmax_no_renorm(L, k):
    idx, _ = _real["topk_softmax"](L, k)
    Lf = np.asarray(L, dtype=np.float64)
    p = np.exp(Lf - Lf.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return idx, np.take_along_axis(p, idx.astype(np.int64), 1).astype(np.float32)


def _topk_ascending(L, k):
    idx, w = _real["topk_softmax"](-np.asarray(L, dtype=np.float32), k)
    return idx, w


def _dispatch_unstable(topk_idx, E, lo, n):
    counts, offsets, perm, inv = _real["local_dispatch"](topk_idx, E, lo, n)
    perm = perm.copy()
    for e in range(n):                        # reverse order within each segment
        perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    inv = np.full_like(inv, -1)
    inv[perm] = np.arange(perm.shape[0], dtype=np.int32)
    return counts, offsets, perm, inv


def _dispatch_inclusive_offsets(topk_idx, E, lo, n):
    counts, offsets, perm, inv = _real["local_dispatch"](topk_idx, E, lo, n)
    off = offsets.copy()
    off[:-1] = offsets[1:]
    return counts, off, perm, inv


def _gather_token_index_mod(x, perm, k):
    return np.asarray(x)[np.asarray(perm, dtype=np.int64) % np.asarray(x).shape[0]]


def _logits_transposed(x, w_gate, dtype, bias=None):
    X = _real["widen"](x, dtype)
    G = _real["widen"](w_gate, dtype)
    L = X @ G[::-1]                 # rows of W_g taken in reverse (index slip)
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float32)[None, :]
    return L.astype(np.float32)


def _logits_bias_subtracted(x, w_gate, dtype, bias=None):
    if bias is None:
        return _real["router_logits"](x, w_gate, dtype)
    return _real["router_logits"](x, w_gate, dtype, -np.asarray(bias))


def _silu_wrong_sign(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _experts_gate_on_w3(x_packed, offsets, w1, w3, w2, dtype):
    return _real["swiglu_experts"](x_packed, offsets, w3, w1, w2, dtype)


def _experts_no_h_rounding(x_packed, offsets, w1, w3, w2, dtype):
    Xp = _real["widen"](x_packed, dtype)
    n = len(offsets) - 1
    h = np.zeros((Xp.shape[0], np.asarray(w1).shape[2]))
    y = np.zeros((Xp.shape[0], np.asarray(w2).shape[2]))
    for e in range(n):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        X = Xp[r0:r1]
        h[r0:r1] = _real["silu"](X @ _real["widen"](w1[e], dtype)) * (X @ _real["widen"](w3[e], dtype))
        y[r0:r1] = _real["rnd"](h[r0:r1] @ _real["widen"](w2[e], dtype), dtype)
    return h, y


def _combine_unweighted(y_packed, inv, topk_w, dtype, k=None):
    if topk_w is None:
        return _real["combine"](y_packed, inv, None, dtype, k=k)
    return _real["combine"](y_packed, inv, np.ones_like(topk_w), dtype)


def _combine_wrong_slot(y_packed, inv, topk_w, dtype, k=None):
    if topk_w is None:
        return _real["combine"](y_packed, inv, None, dtype, k=k)
    return _real["combine"](y_packed, inv, np.asarray(topk_w)[:, ::-1].copy(), dtype)


def _down_projection_ignores_scale(h, offsets, w2, dtype, row_scale=None):
    return _real["down_projection"](h, offsets, w2, dtype)


def _down_projection_scale_after_rounding(h, offsets, w2, dtype, row_scale=None):
    y = _real["down_projection"](h, offsets, w2, dtype)
    if row_scale is None:
        return y
    return _real["rnd"](np.asarray(row_scale, dtype=np.float64)[:, None] * y, dtype)


def _dispatch_padded_keeps_last(topk_idx, E, lo, n, C):
    """Keeps each expert's last C assignments instead of its first C."""
    flat = np.asarray(topk_idx).ravel().astype(np.int64)
    counts_all = np.bincount(flat, minlength=E).astype(np.int32)
    perm = np.full(n * C, -1, dtype=np.int32)
    inv = np.full(flat.shape[0], -1, dtype=np.int32)
    for e in range(n):
        ids = [a for a in range(flat.shape[0]) if flat[a] == lo + e][-C:]
        for r, a in enumerate(ids):
            perm[e * C + r] = a
            inv[a] = e * C + r
    return counts_all, (np.arange(n + 1) * C).astype(np.int32), perm, inv


def _gather_padded_copies_row0(x, perm, k):
    """Fills padding rows with x[0] instead of zeros."""
    x = np.asarray(x)
    perm = np.asarray(perm, dtype=np.int64)
    return x[np.where(perm >= 0, perm, 0) // k]


def _gemm_not_rounded(A, B, dtype):
    """Skips the rounding to the storage dtype."""
    from oracle.moe_oracle import widen
    return widen(A, dtype) @ widen(B, dtype)


MUTATIONS = {
    "gemm_not_rounded": ("gemm", _gemm_not_rounded),
    "dispatch_padded_keeps_last": ("local_dispatch_padded", _dispatch_padded_keeps_last),
    "gather_padded_nonzero_padding": ("gather_rows_padded", _gather_padded_copies_row0),
    "round_half_away_from_zero": ("round_bf16", _round_half_away),
    "round_double_via_f32": ("round_bf16", _round_via_f32),
    "topk_ties_to_high_index": ("topk_softmax", _topk_ties_high),
    "topk_no_renormalisation": ("topk_softmax", _topk_full_softmax_no_renorm),
    "topk_smallest_instead_of_largest": ("topk_softmax", _topk_ascending),
    "dispatch_unstable_within_segment": ("local_dispatch", _dispatch_unstable),
    "dispatch_inclusive_offsets": ("local_dispatch", _dispatch_inclusive_offsets),
    "gather_wrong_token_index": ("gather_rows", _gather_token_index_mod),
    "logits_transposed_operand": ("router_logits", _logits_transposed),
    "logits_bias_sign": ("router_logits", _logits_bias_subtracted),
    "silu_wrong_sign": ("silu", _silu_wrong_sign),
    "swiglu_gate_on_w3": ("swiglu_experts", _experts_gate_on_w3),
    "swiglu_h_not_rounded": ("swiglu_experts", _experts_no_h_rounding),
    "combine_drops_weight": ("combine", _combine_unweighted),
    "combine_wrong_slot_weight": ("combine", _combine_wrong_slot),
    "down_projection_ignores_scale": ("down_projection", _down_projection_ignores_scale),
    "down_projection_scale_after_rounding": ("down_projection", _down_projection_scale_after_rounding),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
