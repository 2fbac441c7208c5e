"""moe_dispatch_noalloc (its scratch in a static per-device array, no
workspace) against moe_dispatch with a caller workspace, through the C ABI.

Dispatch is integer and byte work, so every output is compared bit for bit:
counts, offsets, the whole permutation buffer (rows past A must stay
untouched in both), the inverse and the gathered rows.  Two calls in a row
share the static array; the second is smaller, so stale histograms of the
first call lie in the array where the second one does not write.
"""
import numpy as np
import pytest

import combine_router_top_amd as M
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def _case(T, d, E, k, lo, n, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    x = rng.integers(0, 65535, size=(T, d), dtype=np.uint16) & np.uint16(0x7F7F)
    return M.Spec(T, d, E, k, 64, lo, n, "bf16"), idx, x


def test_dispatch_noalloc_matches_dispatch():
    import torch
    # 15000 then 4800 assignments: 15 and 5 chunk histograms in the static
    # array; then a one-chunk batch, which builds its histogram in LDS
    for T, d, E, k, lo, n, seed in [(3000, 64, 40, 5, 7, 13, 31), (1200, 128, 24, 4, 2, 9, 32),
                                    (100, 64, 16, 3, 0, 16, 33)]:
        p, idx, x = _case(T, d, E, k, lo, n, seed)
        di, dx = dev(idx), dev(x)
        ref = M.dispatch(p, di, dx)
        got = M.dispatch_noalloc(p, di, dx)
        torch.cuda.synchronize()
        for name in ("counts_all", "offsets", "perm", "inv", "x_packed"):
            assert np.array_equal(host(got[name]), host(ref[name])), (T, name)
        A = int(host(got["offsets"])[-1])
        assert A > 0 and np.all(host(got["perm"])[A:] == -7), T
