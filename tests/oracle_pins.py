"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` takes the oracle module ``O`` and raises AssertionError when the
oracle disagrees with an independent fact: a library routine (torch's bf16
cast, scipy's softmax, torch's SiLU, numpy integer matmul), a closed form, a
brute-force definition on tiny inputs, a hand-worked fixture under
``tests/golden/`` or an invariant.  ``test_oracle_pins.py`` runs them on the
real oracle; ``test_oracle_mutations.py`` plants plausible mistakes in the
oracle and checks that at least one pin fails for each.
"""
import itertools
import json
import math
import os
from types import SimpleNamespace

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _prob(T, d, E, k, f, lo, n, dtype="f32"):
    return SimpleNamespace(T=T, d=d, E=E, k=k, f=f, expert_lo=lo, n_local=n, dtype=dtype)


# ---------------------------------------------------------------------------
# number format
# ---------------------------------------------------------------------------
def pin_round_bf16_vs_torch(O):
    """RNE fp32->bf16 equals torch's bf16 cast (a library routine), over normal,
    subnormal, tie and large values."""
    import torch
    rng = np.random.default_rng(7)
    parts = [
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        (rng.standard_normal(5000) * 1e-39).astype(np.float32),     # fp32 subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38], dtype=np.float32),
    ]
    # exact ties: low 16 bits == 0x8000
    hi = rng.integers(0, 0x7F00, 4000, dtype=np.uint32)
    parts.append(((hi << np.uint32(16)) | np.uint32(0x8000)).view(np.float32))
    x = np.concatenate(parts)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.to_bf16_bits(O.round_bf16(x.astype(np.float64)))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r}"


def pin_round_bf16_hand(O):
    """Hand-derived cases, including a float64 value that double rounding via
    float32 would get wrong: 1 + 2^-8 + 2^-30 is above the tie, so it rounds up
    to 1 + 2^-7, while float32 first rounds it onto the tie 1 + 2^-8 (-> 1.0)."""
    cases = [
        (1.0 + 2.0 ** -8, 1.0),                     # tie -> even (mantissa 0)
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),     # tie -> even (mantissa 2)
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),
        (-(1.0 + 2.0 ** -8 + 2.0 ** -30), -(1.0 + 2.0 ** -7)),
        (2.0 ** -140, 0.0),                         # below half the smallest subnormal step 2^-133
        (3 * 2.0 ** -134, 2 * 2.0 ** -133),         # subnormal tie 1.5 steps -> 2 steps
        (2.0 ** 128 * (1 - 2.0 ** -9), math.inf),   # halfway past the largest finite -> inf
        (0.0, 0.0),
    ]
    for x, want in cases:
        got = float(O.round_bf16(np.array([x]))[0])
        assert got == want, (x, got, want)


# ---------------------------------------------------------------------------
# router logits
# ---------------------------------------------------------------------------
def pin_logits_integer_exact(O):
    """Small-integer x and W_g: logits are exact integers, equal to numpy's
    int64 matmul (exact integer arithmetic), with and without an integer bias;
    also through bf16 storage (small integers are exact in bf16)."""
    rng = np.random.default_rng(3)
    x = rng.integers(-2, 3, size=(37, 24))
    g = rng.integers(-2, 3, size=(24, 11))
    ref = (x.astype(np.int64) @ g.astype(np.int64)).astype(np.float64)
    got = O.router_logits(x.astype(np.float32), g.astype(np.float32), "f32")
    assert got.dtype == np.float32
    assert np.array_equal(got.astype(np.float64), ref)
    b = rng.integers(-3, 4, size=11).astype(np.float32)
    got_b = O.router_logits(x.astype(np.float32), g.astype(np.float32), "f32", b)
    assert np.array_equal(got_b.astype(np.float64), ref + b[None, :])
    # bf16 storage: integer v is stored as the top 16 bits of float32(v)
    xb = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    gb = (g.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.router_logits(xb, gb, "bf16").astype(np.float64), ref)


def pin_widen_bf16_hand(O):
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3FC0, 0x7F7F], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 1.5, (2 - 2.0 ** -7) * 2.0 ** 127]
    got = O.widen(bits, "bf16")
    assert list(got) == want
    assert math.copysign(1, got[3]) < 0


# ---------------------------------------------------------------------------
# top-k gating
# ---------------------------------------------------------------------------
def _brute_topk(L, k):
    """Expert e sits in slot r iff exactly r experts beat it under
    (logit descending, index ascending).  O(E^2) per token."""
    T, E = L.shape
    idx = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for e in range(E):
            r = sum(1 for o in range(E)
                    if L[t, o] > L[t, e] or (L[t, o] == L[t, e] and o < e))
            if r < k:
                idx[t, r] = e
    return idx


def pin_topk_brute_force(O):
    """Random integer-valued logits (many ties, including +0/-0) on tiny
    shapes: slots equal the brute-force rank definition."""
    rng = np.random.default_rng(11)
    for (T, E, k) in [(40, 8, 2), (30, 16, 5), (20, 5, 5), (25, 33, 8), (10, 1, 1)]:
        L = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
        L[L == 0] = np.where(rng.random(np.count_nonzero(L == 0)) < 0.5, -0.0, 0.0)
        idx, w = O.topk_softmax(L, k)
        assert idx.dtype == np.int32 and w.dtype == np.float32
        assert np.array_equal(idx.astype(np.int64), _brute_topk(L.astype(np.float64), k)), (T, E, k)


def pin_topk_weights_closed_forms(O):
    import scipy.special as sp
    rng = np.random.default_rng(5)
    L = rng.standard_normal((50, 12)).astype(np.float32)
    # k = E: plain softmax (scipy), in descending order
    idx, w = O.topk_softmax(L, 12)
    p = sp.softmax(L.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, idx.astype(np.int64), 1), rtol=2e-7, atol=0)
    # renormalised full softmax for k < E
    for k in (1, 2, 3, 7):
        idx, w = O.topk_softmax(L, k)
        sel = np.take_along_axis(p, idx.astype(np.int64), 1)
        assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=2e-7, atol=0), k
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 4 * 2.0 ** -24 * k)
        assert np.all(np.diff(w.astype(np.float64), axis=1) <= 0)
        assert np.all(w[:, 0] >= np.float32(1.0 / k) * (1 - 1e-7))
    # k = 1: weight exactly 1; k = 2: w0 = 1 / (1 + e^(l1 - l0))
    _, w1 = O.topk_softmax(L, 1)
    assert np.all(w1 == 1.0)
    idx2, w2 = O.topk_softmax(L, 2)
    l = L.astype(np.float64)
    l0 = np.take_along_axis(l, idx2[:, :1].astype(np.int64), 1)[:, 0]
    l1 = np.take_along_axis(l, idx2[:, 1:].astype(np.int64), 1)[:, 0]
    assert np.allclose(w2[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-7, atol=0)


def pin_topk_ties(O):
    """All-zero row: slots 0..k-1, weights exactly 1/k for k a power of two;
    -0.0 and +0.0 tie and the lower index wins; equal columns give the lower
    index first."""
    L = np.zeros((3, 8), dtype=np.float32)
    L[1, 0] = -0.0
    L[2] = [-1, -0.0, 0.0, -1, -2, -3, -4, -5]
    idx, w = O.topk_softmax(L, 4)
    assert idx[0].tolist() == [0, 1, 2, 3] and np.all(w[0] == 0.25)
    assert idx[1].tolist() == [0, 1, 2, 3]
    assert idx[2].tolist() == [1, 2, 0, 3]
    M = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], dtype=np.float32)
    assert O.topk_softmax(M, 3)[0][0].tolist() == [1, 2, 4]


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------
def pin_dispatch_brute_force(O):
    """Counts are plain tallies; position of a local assignment a is the
    number of local a' with (expert', a') < (expert, a); all invariants hold."""
    rng = np.random.default_rng(13)
    for (T, E, k, lo, n) in [(50, 8, 2, 0, 8), (64, 16, 4, 3, 6), (33, 12, 3, 11, 1),
                             (20, 10, 10, 2, 5), (7, 4, 1, 0, 1)]:
        L = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
        idx, _ = O.topk_softmax(L, k)
        counts, offsets, perm, inv = O.local_dispatch(idx, E, lo, n)
        flat = idx.ravel().tolist()
        assert counts.tolist() == [flat.count(e) for e in range(E)]
        assert int(counts.sum()) == T * k
        local = [a for a, e in enumerate(flat) if lo <= e < lo + n]
        pos = {a: sum(1 for b in local if (flat[b], b) < (flat[a], a)) for a in local}
        A = len(local)
        assert offsets.tolist() == [0] + list(itertools.accumulate(counts[lo:lo + n].tolist()))
        assert offsets[-1] == A and perm.shape == (A,)
        assert all(perm[pos[a]] == a for a in local)
        assert all(inv[a] == (pos[a] if a in pos else -1) for a in range(T * k))
        assert perm.dtype == np.int32 and inv.dtype == np.int32 and offsets.dtype == np.int32


def pin_dispatch_padded_reduces_to_unpadded(O):
    """With a capacity of at least the largest local count nothing is dropped
    and the padded layout is the unpadded one (already pinned above) spread to
    offsets e*C, with -1 padding rows after each segment."""
    rng = np.random.default_rng(19)
    for (T, E, k, lo, n) in [(50, 8, 2, 0, 8), (64, 16, 4, 3, 6), (33, 12, 3, 11, 1)]:
        L = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
        idx, _ = O.topk_softmax(L, k)
        cu, ou, pu, iu = O.local_dispatch(idx, E, lo, n)
        cnt = np.diff(ou)
        for C in (int(cnt.max()) if cnt.max() > 0 else 1, T):
            cp, op, pp, ip = O.local_dispatch_padded(idx, E, lo, n, C)
            assert np.array_equal(cp, cu)
            assert op.tolist() == [e * C for e in range(n + 1)]
            assert pp.shape == (n * C,)
            for e in range(n):
                seg = pp[e * C:(e + 1) * C]
                assert np.array_equal(seg[:cnt[e]], pu[ou[e]:ou[e + 1]])
                assert np.all(seg[cnt[e]:] == -1)
            for a in range(T * k):
                if iu[a] < 0:
                    assert ip[a] == -1
                else:
                    e = int(idx.ravel()[a]) - lo
                    assert ip[a] == e * C + iu[a] - ou[e]


def pin_dispatch_padded_capacity(O):
    """Small capacities: per expert the kept assignments are its C smallest
    assignment ids (computed here by sorting each expert's ids), in ascending
    order at the start of its segment; the rest of the segment is -1; perm and
    inv are inverse on the kept set and inv is -1 elsewhere."""
    rng = np.random.default_rng(23)
    for (T, E, k, lo, n, C) in [(40, 6, 2, 0, 6, 3), (64, 16, 4, 3, 6, 5), (30, 4, 4, 0, 4, 1),
                                (25, 8, 3, 2, 3, 7)]:
        L = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
        idx, _ = O.topk_softmax(L, k)
        flat = idx.ravel().tolist()
        counts, offsets, perm, inv = O.local_dispatch_padded(idx, E, lo, n, C)
        assert counts.tolist() == [flat.count(e) for e in range(E)]
        kept = set()
        for e in range(n):
            ids = sorted(a for a, x in enumerate(flat) if x == lo + e)[:C]
            kept.update(ids)
            seg = perm[e * C:(e + 1) * C].tolist()
            assert seg[:len(ids)] == ids and all(v == -1 for v in seg[len(ids):])
        for a in range(T * k):
            if a in kept:
                assert perm[inv[a]] == a
            else:
                assert inv[a] == -1
        assert int((perm >= 0).sum()) == len(kept)


def pin_gather_padded(O):
    """Padding rows are all-zero bits; kept rows are copies of x[perm // k]."""
    rng = np.random.default_rng(27)
    x = rng.integers(1, 65535, size=(9, 16), dtype=np.uint16)
    perm = np.array([5, -1, 17, -1, 8], dtype=np.int32)
    got = O.gather_rows_padded(x, perm, 2)
    want = np.stack([x[a // 2] if a >= 0 else np.zeros(16, np.uint16) for a in perm.tolist()])
    assert np.array_equal(got, want)


def pin_gather(O):
    rng = np.random.default_rng(17)
    x = rng.integers(0, 65535, size=(9, 16), dtype=np.uint16)
    perm = np.array([5, 0, 17, 3, 8], dtype=np.int32)
    got = O.gather_rows(x, perm, 2)
    assert np.array_equal(got, np.stack([x[a // 2] for a in perm.tolist()]))


def pin_hand_routing(O):
    """tests/golden/hand_routing.json: a tiny case worked out by hand."""
    g = _load("hand_routing.json")
    p = _prob(g["T"], g["d"], g["E"], g["k"], 1, g["expert_lo"], g["n_local"])
    x = np.array(g["x"], dtype=np.float32)
    L = O.router_logits(x, np.array(g["w_gate"], dtype=np.float32), "f32")
    assert L.tolist() == g["logits"]
    idx, w = O.topk_softmax(L, p.k)
    assert idx.tolist() == g["topk_idx"]
    wf = [eval(s, {"exp": math.exp}) for s in g["topk_w_formula"]]
    assert np.allclose(w.ravel(), wf, rtol=1e-7, atol=0)
    counts, offsets, perm, inv = O.local_dispatch(idx, p.E, p.expert_lo, p.n_local)
    assert counts.tolist() == g["counts_all"] and offsets.tolist() == g["offsets"]
    assert perm.tolist() == g["perm"] and inv.tolist() == g["inv"]
    xp = O.gather_rows(x, perm, p.k)
    assert xp.tolist() == g["x_packed"]
    y = O.combine(xp.astype(np.float64), inv, w, "f32")
    yf = [[eval(s, {"exp": math.exp}) for s in row] for row in g["y_identity_formula"]]
    assert np.allclose(y, yf, rtol=1e-7, atol=0)


# ---------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------
def _brute_swiglu(X, W1, W3, W2, rnd):
    """Scalar triple loops in float64 (pure Python)."""
    T, d = len(X), len(X[0])
    f = len(W1[0])
    h = [[0.0] * f for _ in range(T)]
    y = [[0.0] * d for _ in range(T)]
    for t in range(T):
        for j in range(f):
            a1 = sum(X[t][i] * W1[i][j] for i in range(d))
            a3 = sum(X[t][i] * W3[i][j] for i in range(d))
            h[t][j] = rnd((a1 / (1.0 + math.exp(-a1))) * a3)
        for c in range(d):
            y[t][c] = rnd(sum(h[t][j] * W2[j][c] for j in range(f)))
    return np.array(h), np.array(y)


def pin_swiglu_brute_force(O):
    """Tiny segments against scalar loops: fp32 (no rounding points) and bf16
    (rounding points at h and y; compared within one bf16 step since the two
    sides sum in different orders before rounding)."""
    rng = np.random.default_rng(19)
    d, f, n = 16, 24, 3
    counts = [5, 0, 3]
    offsets = np.array([0, 5, 5, 8], dtype=np.int32)
    for dtype in ("f32", "bf16"):
        def store(a):
            a = a.astype(np.float32)
            return (a.view(np.uint32) >> 16).astype(np.uint16) if dtype == "bf16" else a
        xp = store(rng.standard_normal((sum(counts), d)))
        w1 = store(rng.standard_normal((n, d, f)) / 4)
        w3 = store(rng.standard_normal((n, d, f)) / 4)
        w2 = store(rng.standard_normal((n, f, d)) / 4)
        h, yp = O.swiglu_experts(xp, offsets, w1, w3, w2, dtype)
        wid = lambda a: O.widen(a, dtype)
        rnd = (lambda v: float(O.round_bf16(np.array([v]))[0])) if dtype == "bf16" else (lambda v: v)
        for e in range(n):
            r0, r1 = offsets[e], offsets[e + 1]
            if r1 == r0:
                continue
            hb, yb = _brute_swiglu(wid(xp[r0:r1]).tolist(), wid(w1[e]).tolist(), wid(w3[e]).tolist(),
                                   wid(w2[e]).tolist(), rnd)
            if dtype == "f32":
                assert np.allclose(h[r0:r1], hb, rtol=1e-12, atol=1e-14)
                assert np.allclose(yp[r0:r1], yb, rtol=1e-12, atol=1e-14)
            else:
                assert np.all(np.abs(h[r0:r1] - hb) <= 2.0 ** -7 * np.abs(hb) + 1e-30)
                assert np.all(np.abs(yp[r0:r1] - yb) <= 2.0 ** -7 * np.abs(yb) + 1e-30)


def pin_dense_ffn_textbook(O):
    """E = 1, k = 1: the layer is a dense SwiGLU FFN, computed here with torch
    (F.silu, float64 matmul)."""
    import torch
    rng = np.random.default_rng(23)
    T, d, f = 12, 32, 40
    p = _prob(T, d, 1, 1, f, 0, 1)
    inp = {
        "x": rng.standard_normal((T, d)).astype(np.float32),
        "w_gate": rng.standard_normal((d, 1)).astype(np.float32),
        "w1": (rng.standard_normal((1, d, f)) / 5).astype(np.float32),
        "w3": (rng.standard_normal((1, d, f)) / 5).astype(np.float32),
        "w2": (rng.standard_normal((1, f, d)) / 5).astype(np.float32),
    }
    out = O.moe_layer(p, inp)
    assert np.all(out["topk_w"] == 1.0) and np.all(out["topk_idx"] == 0)
    X = torch.from_numpy(inp["x"]).double()
    ref = (torch.nn.functional.silu(X @ torch.from_numpy(inp["w1"][0]).double())
           * (X @ torch.from_numpy(inp["w3"][0]).double())) @ torch.from_numpy(inp["w2"][0]).double()
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-13)


def pin_hand_swiglu(O):
    g = _load("hand_swiglu.json")
    xp = np.array(g["x"], dtype=np.float32)
    h, y = O.swiglu_experts(xp, np.array([0, 1], dtype=np.int32), np.array(g["w1"], dtype=np.float32),
                            np.array(g["w3"], dtype=np.float32), np.array(g["w2"], dtype=np.float32), "f32")
    assert math.isclose(h[0, 0], eval(g["h_formula"], {"exp": math.exp}), rel_tol=1e-15)
    assert np.allclose(y[0], [eval(s, {"exp": math.exp}) for s in g["y_formula"]], rtol=1e-15)


def pin_down_projection_integer_exact(O):
    """Integer-valued h and W2 (exact in bf16): every product sum is a small
    integer, so y_packed equals numpy's int64 matmul exactly, per segment,
    also with power-of-two row scales (exact in binary); an empty segment
    writes nothing."""
    rng = np.random.default_rng(41)
    f, d, n = 24, 16, 3
    offsets = np.array([0, 4, 4, 9], dtype=np.int32)
    hi = rng.integers(-3, 4, size=(9, f))
    w2i = rng.integers(-2, 3, size=(n, f, d))
    store = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    scale = np.ldexp(1.0, rng.integers(-3, 2, size=9))
    for dtype in ("bf16", "f32"):
        w2 = store(w2i) if dtype == "bf16" else w2i.astype(np.float32)
        for rs in (None, scale):
            y = O.down_projection(hi.astype(np.float64), offsets, w2, dtype, row_scale=rs)
            for e in range(n):
                r0, r1 = offsets[e], offsets[e + 1]
                ref = (hi[r0:r1] @ w2i[e]).astype(np.float64)
                if rs is not None:
                    ref = ref * rs[r0:r1, None]
                assert np.array_equal(y[r0:r1], ref), (dtype, e)


def pin_down_projection_brute_force(O):
    """bf16 down projection with general row scales against scalar loops:
    y[p][c] = rnd(s[p] * sum_j h[p][j] W2[j][c]), the scale applied to the
    exact sum before the one rounding (scaling a rounded value would round
    twice)."""
    rng = np.random.default_rng(43)
    f, d = 20, 12
    offsets = np.array([0, 6], dtype=np.int32)
    store = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    h = O.widen(store(rng.standard_normal((6, f))), "bf16")
    w2 = store(rng.standard_normal((1, f, d)) / 4)
    W2 = O.widen(w2[0], "bf16").tolist()
    s = rng.uniform(0.05, 0.95, size=6)
    y = O.down_projection(h, offsets, w2, "bf16", row_scale=s)
    rb = lambda v: float(O.round_bf16(np.array([v]))[0])
    H = h.tolist()
    for p_ in range(6):
        for c in range(d):
            assert y[p_, c] == rb(s[p_] * math.fsum(H[p_][j] * W2[j][c] for j in range(f))), (p_, c)


def pin_fold_weight(O):
    """The gate weight folded into the down projection moves one rounding
    point: (a) with power-of-two gate weights rnd(w Y) = w rnd(Y) exactly, so
    the folded layer equals the weighted-combine layer bit for bit; (b) with
    the real weights each output element stays within two bf16 steps of the
    weighted-combine layer (one rounding moved per slot, plus the final one);
    (c) a pure-Python walk of one token: y[c] = rnd(sum over local slots of
    rnd(w_j (h_j W2_e)[c])) in slot order."""
    p, inp = _small_layer(O, "bf16", T=40, d=16, E=8, k=3, f=24, lo=1, n=5)
    base = O.moe_layer(p, inp)
    pw = np.ldexp(1.0, -np.arange(1, p.k + 1)).astype(np.float32)
    routing = {"topk_idx": base["topk_idx"], "topk_w": np.tile(pw, (p.T, 1))}
    a = O.moe_layer(p, inp, routing=routing)
    b = O.moe_layer(p, inp, routing=routing, fold_weight=True)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["h"], b["h"])
    f = O.moe_layer(p, inp, fold_weight=True)
    tol = 2.0 * 2.0 ** -7 * np.abs(base["y"]).max()
    assert np.abs(f["y"] - base["y"]).max() <= tol
    # (c) one token with two or more local slots, by hand
    inv = f["inv"].reshape(p.T, p.k)
    t = int(np.nonzero((inv >= 0).sum(1) >= 2)[0][0])
    rb = lambda v: float(O.round_bf16(np.array([v]))[0])
    X = O.widen(inp["x"], "bf16")[t]
    out = [0.0] * p.d
    for j in range(p.k):
        e = int(f["topk_idx"][t, j]) - p.expert_lo
        if not 0 <= e < p.n_local:
            continue
        W1, W3, W2 = (O.widen(inp[n_][e], "bf16") for n_ in ("w1", "w3", "w2"))
        hrow = []
        for q in range(p.f):
            a1 = math.fsum(X[i] * W1[i, q] for i in range(p.d))
            a3 = math.fsum(X[i] * W3[i, q] for i in range(p.d))
            hrow.append(rb(a1 / (1.0 + math.exp(-a1)) * a3))
        wj = float(f["topk_w"][t, j])
        for c in range(p.d):
            out[c] += rb(wj * math.fsum(hrow[q] * W2[q, c] for q in range(p.f)))
    ref = np.array([rb(v) for v in out])
    assert np.max(np.abs(f["y"][t] - ref)) <= 2.0 ** -7 * np.abs(ref).max(), t


def pin_combine_unweighted(O):
    """combine with no weights is the plain slot-order sum: equal to unit
    weights."""
    p, inp = _small_layer(O, "bf16")
    o = O.moe_layer(p, inp, with_experts=False)
    yp = O.widen(o["x_packed"], "bf16")
    a = O.combine(yp, o["inv"], None, "bf16", k=p.k)
    b = O.combine(yp, o["inv"], np.ones((p.T, p.k), dtype=np.float32), "bf16")
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# combine and the whole layer
# ---------------------------------------------------------------------------
def _small_layer(O, dtype, T=48, d=32, E=8, k=3, f=40, lo=2, n=4, seed=29):
    rng = np.random.default_rng(seed)

    def store(a):
        a = a.astype(np.float32)
        return (a.view(np.uint32) >> 16).astype(np.uint16) if dtype == "bf16" else a
    p = _prob(T, d, E, k, f, lo, n, dtype)
    inp = {"x": store(rng.standard_normal((T, d))),
           "w_gate": store(rng.standard_normal((d, E)) / math.sqrt(d)),
           "w1": store(rng.standard_normal((n, d, f)) / math.sqrt(d)),
           "w3": store(rng.standard_normal((n, d, f)) / math.sqrt(d)),
           "w2": store(rng.standard_normal((n, f, d)) / math.sqrt(d))}
    return p, inp


def pin_combine_identity_experts(O):
    """Identity experts (y_packed = x_packed): y[t] = rnd(x[t] * sum of the
    token's local weights); with all experts local the weights sum to 1 and
    bf16 outputs equal x bit for bit; tokens with no local slot get exact
    zeros; combine is linear under a power-of-two scale."""
    for dtype in ("f32", "bf16"):
        for lo, n in [(2, 4), (0, 8)]:
            p, inp = _small_layer(O, dtype, lo=lo, n=n)
            o = O.moe_layer(p, inp, with_experts=False)
            yp = O.widen(o["x_packed"], dtype)
            y = O.combine(yp, o["inv"], o["topk_w"], dtype)
            X = O.widen(inp["x"], dtype)
            inv = o["inv"].reshape(p.T, p.k)
            wsum = np.where(inv >= 0, o["topk_w"].astype(np.float64), 0.0).sum(1)
            assert np.allclose(y, O.rnd(X * wsum[:, None], dtype), rtol=2.0 ** -7, atol=0)
            none = ~(inv >= 0).any(1)
            assert np.all(y[none] == 0)
            if n == p.E and dtype == "bf16":
                assert np.array_equal(y, X)
            y2 = O.combine(2.0 * yp, o["inv"], o["topk_w"], dtype)
            assert np.array_equal(y2, 2.0 * y)


def pin_layer_token_shuffle(O):
    """Permuting the tokens permutes the routing and the outputs identically."""
    for dtype in ("f32", "bf16"):
        p, inp = _small_layer(O, dtype)
        o = O.moe_layer(p, inp)
        sh = np.random.default_rng(31).permutation(p.T)
        inp2 = dict(inp, x=inp["x"][sh])
        o2 = O.moe_layer(p, inp2)
        assert np.array_equal(o2["topk_idx"], o["topk_idx"][sh])
        assert np.array_equal(o2["topk_w"], o["topk_w"][sh])
        assert np.allclose(o2["y"], o["y"][sh], rtol=2.0 ** -7 if dtype == "bf16" else 1e-12, atol=1e-300)


def pin_layer_rows_vs_tokens(O):
    """The per-token path used for sampled checks equals the full layer."""
    for dtype in ("f32", "bf16"):
        p, inp = _small_layer(O, dtype)
        o = O.moe_layer(p, inp)
        toks = [0, 5, 17, 47]
        r = O.token_outputs(p, inp, o["topk_idx"], o["topk_w"], toks)
        assert np.allclose(r, o["y"][toks], rtol=2.0 ** -7 if dtype == "bf16" else 1e-12, atol=1e-300)


def pin_token_outputs_unrounded(O):
    """``token_outputs(rounded=False)`` is the exact float64 layer on the
    stored inputs: pure-Python SwiGLU with no rounding, weighted by the local
    gate weights in slot order; it differs from the rounded rows by at most a
    few bf16 ulps, and for fp32 workloads the two are identical."""
    for dtype in ("f32", "bf16"):
        p, inp = _small_layer(O, dtype)
        o = O.moe_layer(p, inp)
        toks = [0, 9, 30, 47]
        u = O.token_outputs(p, inp, o["topk_idx"], o["topk_w"], toks, rounded=False)
        r = O.token_outputs(p, inp, o["topk_idx"], o["topk_w"], toks)
        X = O.widen(inp["x"], dtype)
        for q, t in enumerate(toks):
            ref = np.zeros(p.d)
            for j in range(p.k):
                e = int(o["topk_idx"][t, j]) - p.expert_lo
                if not 0 <= e < p.n_local:
                    continue
                _, y = _brute_swiglu([list(X[t])], O.widen(inp["w1"][e], dtype).tolist(),
                                     O.widen(inp["w3"][e], dtype).tolist(),
                                     O.widen(inp["w2"][e], dtype).tolist(), lambda v: v)
                ref += float(o["topk_w"][t, j]) * y[0]
            assert np.allclose(u[q], ref, rtol=1e-12, atol=1e-12)
        if dtype == "f32":
            assert np.array_equal(u, r)
        else:
            assert not np.array_equal(u, r)
            assert np.allclose(u, r, rtol=2.0 ** -5, atol=2.0 ** -5 * np.abs(u).max())


def pin_empty_batch(O):
    """T = 0: no assignments, so every count and offset is zero and every
    T-sized output is empty (the degenerate batch of a GPU that received no
    tokens)."""
    for dtype in ("f32", "bf16"):
        p, inp = _small_layer(O, dtype, T=0)
        o = O.moe_layer(p, inp)
        assert np.array_equal(o["counts_all"], np.zeros(p.E, dtype=np.int32))
        assert np.array_equal(o["offsets"], np.zeros(p.n_local + 1, dtype=np.int32))
        for key, shape in (("topk_idx", (0, p.k)), ("topk_w", (0, p.k)), ("perm", (0,)),
                           ("inv", (0,)), ("y", (0, p.d))):
            assert np.asarray(o[key]).shape == shape, key


def pin_layer_padded(O):
    """The padded layer against the unpadded one: with C = the largest local
    count the outputs agree; with a smaller C they agree with the unpadded
    layer's packed rows combined without the dropped slots; padding rows of h
    and y_packed are exact zeros."""
    for dtype in ("f32", "bf16"):
        p, inp = _small_layer(O, dtype)
        u = O.moe_layer(p, inp)
        cnt = np.diff(u["offsets"])
        tol = 2.0 ** -7 if dtype == "bf16" else 1e-12
        for C in (int(cnt.max()), max(1, int(cnt.max()) // 2)):
            pd = O.moe_layer_padded(p, inp, C)
            pad = pd["perm"] < 0
            assert np.all(pd["h"][pad] == 0) and np.all(pd["y_packed"][pad] == 0)
            kept = pd["inv"] >= 0
            inv_u = np.where(kept, u["inv"], -1)
            want = O.combine(u["y_packed"], inv_u, u["topk_w"], dtype)
            assert np.allclose(pd["y"], want, rtol=tol, atol=1e-300)
            if C == int(cnt.max()):
                assert kept.sum() == (u["inv"] >= 0).sum()
                assert np.allclose(pd["y"], u["y"], rtol=tol, atol=1e-300)


def pin_gemm_integer_exact(O):
    """Integer-valued bf16 operands: the product equals numpy's int64 matmul
    and, where it is exactly representable in bf16 (|v| <= 256), rnd keeps it."""
    rng = np.random.default_rng(37)
    for (M, K, N) in [(5, 8, 3), (17, 40, 24), (1, 8, 8)]:
        a = rng.integers(-2, 3, size=(M, K))
        b = rng.integers(-2, 3, size=(K, N))
        store = lambda v: (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        c = O.gemm(store(a), store(b), "bf16")
        ref = (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float64)
        small = np.abs(ref) <= 256
        assert np.array_equal(c[small], ref[small])
        assert np.allclose(c, ref, rtol=2.0 ** -8, atol=0)
        c32 = O.gemm(a.astype(np.float32), b.astype(np.float32), "f32")
        assert np.array_equal(c32, ref)


def pin_gemm_vs_torch(O):
    """Random bf16 operands: float64 product equals torch's float64 matmul (a
    library routine) before rounding, and rnd is the bf16 rounding pinned above."""
    import torch
    rng = np.random.default_rng(41)
    a = (rng.standard_normal((33, 72)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b = (rng.standard_normal((72, 40)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ta = torch.from_numpy(O.widen(a, "bf16"))
    tb = torch.from_numpy(O.widen(b, "bf16"))
    exact = (ta @ tb).numpy()
    assert np.array_equal(O.gemm(a, b, "bf16"), O.round_bf16(exact))


def pin_skew_routing_shape(O):
    """With the Zipf-like bias b[e] = 1.5 ln(1/(e+1)) the low experts receive
    far more than the mean count and some experts receive none."""
    rng = np.random.default_rng(0)
    T, d, E, k = 512, 64, 64, 4
    x = rng.standard_normal((T, d)).astype(np.float32)
    g = (rng.standard_normal((d, E)) / math.sqrt(d)).astype(np.float32)
    b = (1.5 * np.log(1.0 / (np.arange(E) + 1.0))).astype(np.float32)
    idx, _ = O.topk_softmax(O.router_logits(x, g, "f32", b), k)
    c = O.expert_counts(idx, E)
    mean = T * k / E
    assert c[0] > 8 * mean and (c == 0).any() and c.sum() == T * k


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
