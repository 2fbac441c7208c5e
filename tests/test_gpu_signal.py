"""GEMM with per-tile completion signals and the tile forwarder (the local
half of the pages' GEMM + AllGather workload), against the oracle."""
import numpy as np
import pytest

import combine_router_top_amd as M
import oracle.moe_oracle as O
from tests.gpu_util import check_close, dev, host

pytestmark = pytest.mark.gpu


def _operands(Mr, N, K, seed):
    rng = np.random.default_rng(seed)
    store = lambda v: (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    A = store(rng.standard_normal((Mr, K)))
    B = store(rng.standard_normal((K, N)) / np.sqrt(K))
    return A, B


@pytest.mark.parametrize("shape", [(300, 520, 264), (256, 256, 64), (1000, 1024, 512), (1, 8, 8),
                                   (513, 264, 1000)])
def test_gemm_signal(shape):
    """C against the oracle within the bf16 bar; every tile's flag carries the
    epoch of the call that wrote it, also on a second call with a new epoch."""
    import torch
    Mr, N, K = shape
    A, B = _operands(Mr, N, K, seed=sum(shape))
    ref = O.gemm(A, B, "bf16")
    tiles = M.gemm_signal_tiles(Mr, N)
    assert tiles == -(-Mr // 256) * -(-N // 256)
    flags = torch.zeros(tiles, dtype=torch.int32, device="cuda")
    dA, dB = dev(A), dev(B)
    for epoch, scope in ((1, M.MOE_SCOPE_AGENT), (2, M.MOE_SCOPE_SYSTEM)):
        C = M.gemm_signal(dA, dB, flags, epoch, scope=scope)
        torch.cuda.synchronize()
        check_close(O.widen(host(C), "bf16"), ref, "bf16", f"C {shape}")
        assert np.all(host(flags) == epoch)


def test_tile_forward_concurrent():
    """The forwarder polls on a second stream while the GEMM runs: every tile
    it copies must already be final (dst == C bit for bit), none times out.
    Both streams start after the host synchronisation, so the forwarder can
    only overlap the GEMM, never precede its launch."""
    import torch
    Mr, N, K = 2048, 2048, 1024
    A, B = _operands(Mr, N, K, seed=3)
    dA, dB = dev(A), dev(B)
    tiles = M.gemm_signal_tiles(Mr, N)
    flags = torch.zeros(tiles, dtype=torch.int32, device="cuda")
    timeouts = torch.zeros(1, dtype=torch.int32, device="cuda")
    C = torch.empty((Mr, N), dtype=torch.bfloat16, device="cuda")
    dst = torch.zeros((Mr, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for epoch in (1, 2):
        dst.zero_()
        torch.cuda.synchronize()
        # the GEMM is enqueued first: if the two streams share a hardware
        # queue, the forwarder then runs after it (every flag already set)
        # instead of spinning in front of it
        M.gemm_signal(dA, dB, flags, epoch, stream=s1, out=C)
        M.tile_forward(C, dst, flags, epoch, spin_limit=1 << 22, timeouts=timeouts, workgroups=4,
                       stream=s2)
        torch.cuda.synchronize()
        assert int(host(timeouts)[0]) == 0
        assert np.array_equal(host(dst), host(C))
    check_close(O.widen(host(C), "bf16"), O.gemm(A, B, "bf16"), "bf16", "C")


def test_tile_forward_times_out():
    """Flags that never reach the epoch (forced from the host with a tiny
    spin limit): the forwarder counts a timeout per tile, copies nothing and
    finishes."""
    import torch
    Mr, N = 600, 520
    tiles = M.gemm_signal_tiles(Mr, N)
    flags = torch.zeros(tiles, dtype=torch.int32, device="cuda")
    timeouts = torch.zeros(1, dtype=torch.int32, device="cuda")
    C = torch.ones((Mr, N), dtype=torch.bfloat16, device="cuda")
    dst = torch.zeros((Mr, N), dtype=torch.bfloat16, device="cuda")
    M.tile_forward(C, dst, flags, 7, spin_limit=16, timeouts=timeouts, workgroups=3)
    torch.cuda.synchronize()
    assert int(host(timeouts)[0]) == tiles
    assert not np.any(host(dst))
