"""GPU parity: every call of libmoe against the CPU oracle, on seeded inputs
small enough for the full oracle but spanning several tiles and ragged tails.

Bars: routing indices, counts, offsets, permutation and gathered rows
bit-exact; logits and gate weights within 1e-5; expert and layer outputs within
the floored relative error 2e-2 (bf16) or 1e-5 (fp32).
"""
import numpy as np
import pytest

import combine_router_top_amd as M
import oracle.moe_oracle as O
import workloads
from tests.gpu_util import check_close, check_routing, dev, host

pytestmark = pytest.mark.gpu

W = workloads.Workload
SMALL = {
    # name: workload (shapes chosen to hit every kernel variant and tail)
    "tiny_fp32": workloads.get("tiny_fp32"),
    "wide_tails": W("wide_tails", 300, 264, 64, 6, 200, 8, 20, "bf16", seed=3),
    "wide_dsv3_like": W("wide_dsv3_like", 200, 512, 256, 8, 256, 0, 32, "bf16", seed=4),
    "narrow_multiblock": W("narrow_multiblock", 777, 256, 8, 2, 320, 0, 8, "bf16", seed=5),
    "skew": W("skew", 512, 128, 32, 4, 128, 0, 16, "bf16", skew=True, seed=6),
    "plain_router_bf16": W("plain_router_bf16", 100, 64, 22, 3, 64, 5, 10, "bf16", seed=7),
    "fp32_mid": W("fp32_mid", 130, 72, 12, 3, 40, 2, 7, "f32", seed=8),
    "one_token": W("one_token", 1, 64, 16, 1, 32, 0, 16, "bf16", seed=9),
    "one_local": W("one_local", 257, 128, 16, 4, 64, 15, 1, "bf16", seed=10),
    "dense_e1": W("dense_e1", 70, 96, 1, 1, 136, 0, 1, "bf16", seed=11),
    "k_equals_e": W("k_equals_e", 90, 64, 6, 6, 48, 1, 4, "bf16", seed=12),
    # large segments (256 x 256 tile kernel) with row, K and N tails
    "big_tails": W("big_tails", 1500, 328, 4, 2, 264, 0, 4, "bf16", seed=14),
    # skewed, not dense-like (mean 300 rows): every segment, up to ~1000 rows,
    # streams through the thin/medium tiles in one launch
    "big_mixed": W("big_mixed", 1200, 256, 16, 4, 256, 0, 8, "bf16", skew=True, seed=15),
    # skewed and dense-like (mean 500 rows): segments of 35 .. 1736 rows, the
    # ones >= 320 on the large-tile kernel next to thin and medium ones
    "big_dense_skew": W("big_dense_skew", 2000, 256, 8, 2, 256, 0, 8, "bf16", skew=True, seed=19),
    # thin (<= 48 rows) and medium segments, some past 320 rows, with column tails
    "mixed_classes": W("mixed_classes", 700, 264, 24, 4, 328, 0, 12, "bf16", skew=True, seed=16),
    # more than 8 local slots per token (combine loads slots in groups of 8):
    # k = 16 and the maximum k = 32, all experts local
    "many_slots_k16": W("many_slots_k16", 200, 136, 32, 16, 64, 0, 32, "bf16", seed=20),
    "many_slots_k32": W("many_slots_k32", 96, 64, 64, 32, 40, 0, 64, "bf16", seed=21),
    # ~60 rows per expert on 16 local experts: the host narrows the medium
    # column blocks so that they fill the last round of workgroups (GEMM-2:
    # 7168 columns in 448-column blocks; GEMM-1: 2 x 3072 weight columns in
    # 384-column blocks), thin and medium blocks mixed under the
    # column-weighted XCD split
    "narrow_mcols_down": W("narrow_mcols_down", 480, 7168, 16, 2, 128, 0, 16, "bf16", seed=17),
    "narrow_mcols_up": W("narrow_mcols_up", 480, 128, 16, 2, 3072, 0, 16, "bf16", seed=18),
    # wide router with two token blocks and four K splits (the last one 72
    # deep, a K tail), 40 experts inside a 256-column block
    "wide_ksplit": W("wide_ksplit", 300, 1032, 40, 4, 64, 8, 16, "bf16", seed=23),
    # wide router with E % 8 != 0
    "wide_e20": W("wide_e20", 150, 200, 20, 3, 96, 4, 8, "bf16", seed=22),
    # top-k with 2 (96 experts) and 8 (384 experts) values per lane
    "topk_e96": W("topk_e96", 130, 64, 96, 6, 32, 0, 16, "bf16", seed=24),
    "topk_e384": W("topk_e384", 70, 128, 384, 8, 32, 16, 32, "bf16", seed=25),
    # the largest E (16 values per lane in top-k, four 256-expert router
    # blocks) and, with it, the largest k on 1024 local experts: over a
    # thousand segments of 0..5 rows through the grouped GEMM schedule
    "topk_e1024": W("topk_e1024", 64, 64, 1024, 8, 32, 100, 16, "bf16", seed=27),
    # enough token blocks for the 160-token router tile (17 blocks x 8 K
    # splits of 320; the 7th is 184 deep, the 8th empty), ragged token tail
    "router_long": W("router_long", 2600, 2104, 32, 4, 64, 8, 8, "bf16", seed=29),
    # deep K splits (16 and 12): top-k sums them in four waves per token
    "topk_deep_e256": W("topk_deep_e256", 40, 4096, 256, 8, 32, 32, 32, "bf16", seed=30),
    "topk_deep_e1024": W("topk_deep_e1024", 20, 3072, 1024, 8, 32, 512, 16, "bf16", seed=31),
    "max_e1024_k32": W("max_e1024_k32", 48, 64, 1024, 32, 32, 0, 1024, "bf16", seed=28),
    # thin down-projection blocks of 448 and 384 output columns (the width
    # that fills the last round: 32 x 16 and 16 x 16 blocks)
    "thin_tcols448": W("thin_tcols448", 64, 7168, 32, 2, 64, 0, 32, "bf16", seed=26),
    "thin_tcols384": W("thin_tcols384", 48, 6144, 16, 2, 64, 0, 16, "bf16", seed=27),
    # router on direct-to-LDS copies (>= 8 token blocks of 128, E % 8 == 0,
    # E >= 128): ragged last token block (76 rows), 3 K splits with a K tail
    # (1000 = 15 x 64 + 40), skew bias; and two 256-expert column blocks, the
    # second with 64 valid experts
    "router_dma_tails": W("router_dma_tails", 1100, 1000, 256, 8, 64, 0, 32, "bf16", skew=True, seed=34),
    "router_dma_e320": W("router_dma_e320", 1030, 512, 320, 6, 48, 100, 40, "bf16", seed=35),
    # the same router with one K split of two stages (64 + 32 of K) and of a
    # single 40-deep stage: the pipelined loop's shortest forms
    # top-k with four consecutive experts per lane and lanes past E idle
    # (232 experts: lanes 58..63 hold none)
    "topk_e232": W("topk_e232", 300, 256, 232, 8, 32, 40, 32, "bf16", seed=38),
    "router_dma_k96": W("router_dma_k96", 1040, 96, 128, 4, 32, 0, 16, "bf16", seed=36),
    "router_dma_k40": W("router_dma_k40", 1030, 40, 128, 2, 32, 8, 16, "bf16", seed=37),
    # medium GEMM-1 blocks of the full 512 weight columns at a small size
    # (64 experts x 1024 h columns, ~50 rows each: 256 blocks fill one round)
    "medium_w512": W("medium_w512", 1600, 64, 64, 2, 1024, 0, 64, "bf16", seed=28),
}

_cache = {}


def case(name):
    if name not in _cache:
        w = SMALL[name]
        inp = workloads.generate(w)
        ref = O.moe_layer(w, inp)
        d = {k: dev(v) for k, v in inp.items()}
        _cache[name] = (w, inp, ref, d)
    return _cache[name]


@pytest.mark.parametrize("name", sorted(SMALL))
def test_route(name):
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    idx, wt, logits = M.route(p, d["x"], d["w_gate"], d["bias"], want_logits=True)
    check_routing(w, host(logits), host(idx), host(wt), ref["logits"])


@pytest.mark.parametrize("name", ["tiny_fp32", "wide_tails", "narrow_multiblock", "plain_router_bf16",
                                  "wide_ksplit", "wide_e20", "topk_e96",
                                  "topk_e384", "topk_e1024", "router_long", "topk_deep_e256",
                                  "topk_deep_e1024", "router_dma_tails", "router_dma_e320",
                                  "router_dma_k96", "router_dma_k40", "topk_e232"])
def test_route_integer_inputs_exact(name):
    """Small-integer x and W_g: logits are exact on both sides, so routing,
    including ties, must match with no exemption."""
    w = SMALL[name]
    ii = workloads.integer_inputs(w)
    p = M.Spec.of(w)
    idx, wt, logits = M.route(p, dev(ii["x"]), dev(ii["w_gate"]), None, want_logits=True)
    ref_l = O.router_logits(ii["x"], ii["w_gate"], w.dtype)
    assert np.array_equal(host(logits), ref_l)
    check_routing(w, host(logits), host(idx), host(wt), ref_l, tau=0)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_dispatch(name):
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    idx, _ = M.route(p, d["x"], d["w_gate"], d["bias"])
    o = M.dispatch(p, idx, d["x"])
    counts, offsets, perm, inv = O.local_dispatch(host(idx), w.E, w.expert_lo, w.n_local)
    A = int(offsets[-1])
    assert np.array_equal(host(o["counts_all"]), counts)
    assert np.array_equal(host(o["offsets"]), offsets)
    gp = host(o["perm"])
    assert np.array_equal(gp[:A], perm)
    assert np.all(gp[A:] == -7), "rows past A must be untouched"
    assert np.array_equal(host(o["inv"]), inv)
    xp = host(o["x_packed"])
    assert np.array_equal(xp[:A], O.gather_rows(inp["x"], perm, w.k))
    assert not np.any(xp[A:]), "rows past A must be untouched"


@pytest.mark.parametrize("pattern", ["random", "all_one_expert", "none_local", "sorted", "reversed"])
def test_dispatch_supplied_indices(pattern):
    """Dispatch on caller-supplied routing with extreme distributions."""
    T, d, E, k, lo, n = 3000, 64, 40, 5, 7, 13
    rng = np.random.default_rng(21)
    if pattern == "random":
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    elif pattern == "all_one_expert":
        idx = np.tile(np.array([lo + 3, 0, 1, 2, 3]), (T, 1))
    elif pattern == "none_local":
        idx = np.tile(np.array([0, 1, 2, 3, 4]), (T, 1))
    elif pattern == "sorted":
        idx = np.tile(np.arange(lo, lo + k), (T, 1))
    else:
        idx = np.tile(np.arange(lo + n - 1, lo + n - 1 - k, -1), (T, 1))
    idx = idx.astype(np.int32)
    x = rng.integers(0, 65535, size=(T, d), dtype=np.uint16) & np.uint16(0x7F7F)
    p = M.Spec(T, d, E, k, 64, lo, n, "bf16")
    o = M.dispatch(p, dev(idx), dev(x))
    counts, offsets, perm, inv = O.local_dispatch(idx, E, lo, n)
    A = int(offsets[-1])
    assert np.array_equal(host(o["counts_all"]), counts)
    assert np.array_equal(host(o["offsets"]), offsets)
    assert np.array_equal(host(o["perm"])[:A], perm)
    assert np.array_equal(host(o["inv"]), inv)
    assert np.array_equal(host(o["x_packed"])[:A], x[perm // k])


@pytest.mark.parametrize("name", sorted(SMALL))
def test_combine_identity_experts(name):
    """y_packed := x_packed gives y = rnd(x * sum of local weights); with all
    experts local the bf16 output equals x in value (a -0.0 in x comes back as
    +0.0: the weighted sum starts from +0)."""
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    idx, wt = M.route(p, d["x"], d["w_gate"], d["bias"])
    o = M.dispatch(p, idx, d["x"])
    y = host(M.combine(p, o["x_packed"], o["inv"], wt))
    yr = O.combine(O.widen(host(o["x_packed"]), w.dtype), host(o["inv"]), host(wt), w.dtype)
    check_close(O.widen(y, w.dtype), yr, w.dtype, "combine")
    inv = host(o["inv"]).reshape(w.T, w.k)
    none = ~(inv >= 0).any(1)
    assert np.all(O.widen(y, w.dtype)[none] == 0)
    if w.n_local == w.E and w.dtype == "bf16":
        assert np.array_equal(O.widen(y, w.dtype), O.widen(inp["x"], w.dtype))


@pytest.mark.parametrize("name", sorted(SMALL))
def test_expert_gemm(name):
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    idx, wt = M.route(p, d["x"], d["w_gate"], d["bias"])
    o = M.dispatch(p, idx, d["x"])
    h, yp = M.expert_gemm(p, o["x_packed"], o["offsets"], d["w1"], d["w3"], d["w2"])
    offsets = host(o["offsets"])
    A = int(offsets[-1])
    hr, ypr = O.swiglu_experts(host(o["x_packed"])[:A], offsets, inp["w1"], inp["w3"], inp["w2"], w.dtype)
    check_close(O.widen(host(h)[:A], w.dtype), hr, w.dtype, "h")
    check_close(O.widen(host(yp)[:A], w.dtype), ypr, w.dtype, "y_packed")
    assert not np.any(host(h)[A:]) and not np.any(host(yp)[A:]), "rows past A must be untouched"


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("overlap", [False, True])
def test_layer(name, overlap):
    import torch
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    s2 = torch.cuda.Stream() if overlap else None
    y, r = M.layer(p, d["x"], d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"], routing=True,
                   want_logits=True, overlap=overlap, stream2=s2)
    torch.cuda.synchronize()
    check_routing(w, host(r["logits"]), host(r["topk_idx"]), host(r["topk_w"]), ref["logits"])
    routing = {"topk_idx": host(r["topk_idx"]), "topk_w": host(r["topk_w"])}
    oref = O.moe_layer(w, inp, routing=routing)
    assert np.array_equal(host(r["counts_all"]), oref["counts_all"])
    assert np.array_equal(host(r["offsets"]), oref["offsets"])
    A = int(oref["offsets"][-1])
    assert np.array_equal(host(r["perm"])[:A], oref["perm"])
    assert np.array_equal(host(r["inv"]), oref["inv"])
    check_close(O.widen(host(y), w.dtype), oref["y"], w.dtype, "y")


@pytest.mark.parametrize("name", sorted(SMALL))
def test_layer_equals_separate_calls(name):
    """moe_layer gives bit for bit the y of its steps called one by one
    (route, dispatch, expert GEMM, weighted combine): the layer's fusions
    (top-k counting the dispatch histograms, GEMM-1 gathering x rows through
    perm) change no value."""
    import torch
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    y, r = M.layer(p, d["x"], d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"], routing=True)
    idx, wt = M.route(p, d["x"], d["w_gate"], d["bias"])
    o = M.dispatch(p, idx, d["x"])
    h, yp = M.expert_gemm(p, o["x_packed"], o["offsets"], d["w1"], d["w3"], d["w2"])
    ys = M.combine(p, yp, o["inv"], wt)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), host(r["topk_idx"]))
    assert np.array_equal(host(ys), host(y)), "separate calls differ from moe_layer"


@pytest.mark.parametrize("name", ["wide_dsv3_like", "medium_w512", "big_tails"])
def test_expert_gemm_large_activations(name):
    """x scaled by 64 (exact in bf16) so that GEMM-1's products reach a few
    hundred in magnitude: the SiLU of every epilogue (thin, medium and large
    tiles) passes through the range where e^-a overflows or underflows in
    fp32, and h and y_packed still match the oracle within the bar."""
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    xs = d["x"] * 64
    idx, wt = M.route(p, xs, d["w_gate"], d["bias"])
    o = M.dispatch(p, idx, xs)
    h, yp = M.expert_gemm(p, o["x_packed"], o["offsets"], d["w1"], d["w3"], d["w2"])
    offsets = host(o["offsets"])
    A = int(offsets[-1])
    xp = host(o["x_packed"])[:A]
    hr, ypr = O.swiglu_experts(xp, offsets, inp["w1"], inp["w3"], inp["w2"], w.dtype)
    a1 = O.widen(xp, w.dtype).astype(np.float64) @ O.widen(inp["w1"][0], w.dtype).astype(np.float64)
    assert np.abs(a1).max() > 100, "the scaled input should reach the exponential's saturation"
    hg = O.widen(host(h)[:A], w.dtype)
    assert np.all(np.isfinite(hg))
    check_close(hg, hr, w.dtype, "h (large activations)")
    check_close(O.widen(host(yp)[:A], w.dtype), ypr, w.dtype, "y_packed (large activations)")


@pytest.mark.parametrize("name", ["wide_dsv3_like", "router_dma_tails", "big_mixed", "thin_tcols448",
                                  "fp32_mid"])
def test_layer_graph_capture(name):
    """moe_layer captured into a HIP graph (it allocates nothing, clears its
    counters with kernels rather than memsets and waits on nothing): three
    replays, each behind an eager layer call on the same stream and a host
    synchronisation, each equal bit for bit to the eager result."""
    import torch
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    ws = M.alloc_workspace(p)
    st = torch.cuda.Stream()

    def run(out=None):
        return M.layer(p, d["x"], d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"], workspace=ws,
                       stream=st, out=out)

    with torch.cuda.stream(st):
        ye = run()
    torch.cuda.synchronize()
    y = torch.empty_like(ye)
    other = torch.empty_like(ye)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        run(y)
    for rep in range(3):
        with torch.cuda.stream(st):
            y.fill_(float("nan"))
            run(other)
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ye), f"replay {rep} differs from the eager layer"
        assert torch.equal(other, ye)
    del g


@pytest.mark.parametrize("name", sorted(SMALL))
def test_layer_fold_weight(name):
    """Routing weights folded into the down projection (MOE_F_FOLD_WEIGHT):
    routing and dispatch as the plain layer, y against the oracle's folded
    layer (y_packed[p] = rnd(w (h W2)), unweighted combine) on the GPU's
    routing; also with the two-stream overlap."""
    import torch
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    for overlap in (False, True):
        s2 = torch.cuda.Stream() if overlap else None
        y, r = M.layer(p, d["x"], d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"], routing=True,
                       fold_weight=True, overlap=overlap, stream2=s2)
        torch.cuda.synchronize()
        routing = {"topk_idx": host(r["topk_idx"]), "topk_w": host(r["topk_w"])}
        oref = O.moe_layer(w, inp, routing=routing, fold_weight=True)
        assert np.array_equal(host(r["offsets"]), oref["offsets"])
        A = int(oref["offsets"][-1])
        assert np.array_equal(host(r["perm"])[:A], oref["perm"])
        check_close(O.widen(host(y), w.dtype), oref["y"], w.dtype, f"y folded (overlap={overlap})")


@pytest.mark.parametrize("name", ["wide_dsv3_like", "many_slots_k16", "fp32_mid", "skew"])
def test_combine_unweighted(name):
    """combine with no weights sums the local rows in slot order."""
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    idx, wt = M.route(p, d["x"], d["w_gate"], d["bias"])
    o = M.dispatch(p, idx, d["x"])
    y = host(M.combine(p, o["x_packed"], o["inv"], None))
    yr = O.combine(O.widen(host(o["x_packed"]), w.dtype), host(o["inv"]), None, w.dtype, k=w.k)
    check_close(O.widen(y, w.dtype), yr, w.dtype, "unweighted combine")


# padded fixed-capacity layout (the A/B against the unpadded segments)
PADDED = ["skew", "narrow_multiblock", "mixed_classes", "big_mixed", "fp32_mid", "one_local"]


def _capacities(w, offsets):
    """No-drop (largest count), dropping (half the mean count, and 1) and the
    static worst case T."""
    cnt = np.diff(offsets)
    mx = max(1, int(cnt.max()) if cnt.size else 1)
    mean = max(1, (w.T * w.k) // w.E)
    return sorted({mx, max(1, mean // 2), 1, w.T})


@pytest.mark.parametrize("name", PADDED)
def test_dispatch_padded(name):
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    idx, _ = M.route(p, d["x"], d["w_gate"], d["bias"])
    idx_h = host(idx)
    _, off_u, _, _ = O.local_dispatch(idx_h, w.E, w.expert_lo, w.n_local)
    for C in _capacities(w, off_u):
        o = M.dispatch_padded(p, C, idx, d["x"])
        counts, offsets, perm, inv = O.local_dispatch_padded(idx_h, w.E, w.expert_lo, w.n_local, C)
        assert np.array_equal(host(o["counts_all"]), counts), C
        assert np.array_equal(host(o["offsets"]), offsets), C
        assert np.array_equal(host(o["perm"]), perm), C
        assert np.array_equal(host(o["inv"]), inv), C
        assert np.array_equal(host(o["x_packed"]), O.gather_rows_padded(inp["x"], perm, w.k)), C


@pytest.mark.parametrize("name", PADDED)
def test_padded_layer(name):
    """Padded dispatch, padded GEMM and combine against the oracle's padded
    layer on the GPU's routing; padding rows of h and y_packed are zeros."""
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    idx, wt = M.route(p, d["x"], d["w_gate"], d["bias"])
    routing = {"topk_idx": host(idx), "topk_w": host(wt)}
    _, off_u, _, _ = O.local_dispatch(routing["topk_idx"], w.E, w.expert_lo, w.n_local)
    for C in _capacities(w, off_u):
        o = M.dispatch_padded(p, C, idx, d["x"])
        h, yp = M.expert_gemm_padded(p, C, o["x_packed"], o["offsets"], d["w1"], d["w3"], d["w2"])
        y = M.combine(p, yp, o["inv"], wt, rows=w.n_local * C)
        r = O.moe_layer_padded(w, inp, C, routing=routing)
        pad = r["perm"] < 0
        assert not np.any(host(h)[pad]) and not np.any(host(yp)[pad]), C
        check_close(O.widen(host(h), w.dtype), r["h"], w.dtype, f"h C={C}")
        check_close(O.widen(host(yp), w.dtype), r["y_packed"], w.dtype, f"y_packed C={C}")
        check_close(O.widen(host(y), w.dtype), r["y"], w.dtype, f"y C={C}")


def test_layer_deterministic_and_overlap_identical():
    import torch
    w, inp, ref, d = case("wide_dsv3_like")
    p = M.Spec.of(w)
    outs = []
    for ov in (False, False, True):
        s2 = torch.cuda.Stream() if ov else None
        y, r = M.layer(p, d["x"], d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"], routing=True,
                       want_logits=True, overlap=ov, stream2=s2)
        torch.cuda.synchronize()
        outs.append({"y": host(y), **{k: host(v) for k, v in r.items()}})
    for o in outs[1:]:
        for k in outs[0]:
            assert np.array_equal(outs[0][k], o[k]), k


def test_layer_gemm_events_hook():
    """The measurement hook: the next moe_layer call records the two events
    around its expert GEMM (a positive interval inside the call's own), the
    output is unchanged, and the hook is consumed by that call."""
    import ctypes
    import torch
    w, inp, ref, d = case("wide_dsv3_like")
    p = M.Spec.of(w)
    hip = ctypes.CDLL("libamdhip64.so")
    ev = []
    for _ in range(4):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        ev.append(h.value)
    try:
        y0 = host(M.layer(p, d["x"], d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"]))
        st = torch.cuda.current_stream()
        assert hip.hipEventRecord(ctypes.c_void_p(ev[0]), ctypes.c_void_p(st.cuda_stream)) == 0
        M.layer_set_gemm_events(ev[1], ev[2])
        y1 = M.layer(p, d["x"], d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"], stream=st)
        assert hip.hipEventRecord(ctypes.c_void_p(ev[3]), ctypes.c_void_p(st.cuda_stream)) == 0
        torch.cuda.synchronize()
        ms = []
        for a, b in ((0, 3), (1, 2)):
            t = ctypes.c_float(0.0)
            assert hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(ev[a]), ctypes.c_void_p(ev[b])) == 0
            ms.append(t.value)
        assert 0.0 < ms[1] <= ms[0], ms
        assert np.array_equal(host(y1), y0)
        # consumed: a second call records nothing new (the events keep their times)
        M.layer(p, d["x"], d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"], stream=st)
        torch.cuda.synchronize()
        t = ctypes.c_float(0.0)
        assert hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(ev[1]), ctypes.c_void_p(ev[2])) == 0
        assert t.value == ms[1]
    finally:
        for h in ev:
            hip.hipEventDestroy(ctypes.c_void_p(h))


@pytest.mark.parametrize("name", ["wide_dsv3_like", "narrow_multiblock", "fp32_mid"])
def test_layer_token_shuffle_equivariance(name):
    """Permuting tokens permutes routing and outputs; bit-exact because each
    row's reductions do not depend on the other rows."""
    w, inp, ref, d = case(name)
    p = M.Spec.of(w)
    y, r = M.layer(p, d["x"], d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"], routing=True)
    sh = np.random.default_rng(5).permutation(w.T)
    x2 = dev(inp["x"][sh])
    y2, r2 = M.layer(p, x2, d["w_gate"], d["bias"], d["w1"], d["w3"], d["w2"], routing=True)
    assert np.array_equal(host(r2["topk_idx"]), host(r["topk_idx"])[sh])
    assert np.array_equal(host(r2["topk_w"]), host(r["topk_w"])[sh])
    assert np.array_equal(host(y2), host(y)[sh])


def test_layer_no_local_tokens():
    """A bias that keeps every token off the local experts: A = 0 and y = 0."""
    w = W("no_local", 64, 64, 16, 2, 32, 8, 8, "bf16", seed=13)
    inp = workloads.generate(w)
    bias = np.zeros(16, dtype=np.float32)
    bias[8:] = -1e4
    p = M.Spec.of(w)
    y, r = M.layer(p, dev(inp["x"]), dev(inp["w_gate"]), dev(bias), dev(inp["w1"]), dev(inp["w3"]),
                   dev(inp["w2"]), routing=True)
    assert int(host(r["offsets"])[-1]) == 0
    assert np.all(host(r["inv"]) == -1)
    assert not np.any(host(y))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_empty_batch(dtype):
    """T = 0 (a GPU that received no tokens): every call succeeds with empty
    outputs, no workspace, and dispatch and the layer write zero counts and
    offsets over what was there; the oracle gives the same."""
    import torch
    w = W("empty", 0, 64, 16, 2, 32, 4, 8, dtype, seed=26)
    inp = workloads.generate(w)
    ref = O.moe_layer(w, inp)
    p = M.Spec.of(w)
    for call in range(M.MOE_CALL_ROUTE, M.MOE_CALL_EXPERT_GEMM_PADDED + 1):
        assert M.workspace_bytes(p, call) == 0
    x, wg = dev(inp["x"]), dev(inp["w_gate"])
    w1, w3, w2 = dev(inp["w1"]), dev(inp["w3"]), dev(inp["w2"])
    idx, tw, logits = M.route(p, x, wg, want_logits=True)
    assert idx.shape == (0, w.k) and tw.shape == (0, w.k) and logits.shape == (0, w.E)
    stale = {
        "counts_all": torch.full((w.E,), -5, dtype=torch.int32, device="cuda"),
        "offsets": torch.full((w.n_local + 1,), -5, dtype=torch.int32, device="cuda"),
        "perm": torch.empty(0, dtype=torch.int32, device="cuda"),
        "inv": torch.empty(0, dtype=torch.int32, device="cuda"),
        "x_packed": torch.empty((0, w.d), dtype=x.dtype, device="cuda"),
    }
    o = M.dispatch(p, idx, x, out=stale)
    torch.cuda.synchronize()
    assert np.array_equal(host(o["counts_all"]), ref["counts_all"])
    assert np.array_equal(host(o["offsets"]), ref["offsets"])
    h, yp = M.expert_gemm(p, o["x_packed"], o["offsets"], w1, w3, w2)
    y = M.combine(p, yp, o["inv"], tw)
    assert h.shape == (0, w.f) and yp.shape == (0, w.d) and y.shape == (0, w.d)
    y2, r = M.layer(p, x, wg, None, w1, w3, w2, routing=True)
    torch.cuda.synchronize()
    assert y2.shape == (0, w.d)
    assert np.array_equal(host(r["counts_all"]), ref["counts_all"])
    assert np.array_equal(host(r["offsets"]), ref["offsets"])
    with pytest.raises(M.MoeError):
        M.dispatch_padded(p, 1, idx, x)

