"""Helpers for GPU tests: numpy <-> device tensors and the routing protocol.

The routing check follows one rule: where floating point decides an integer
(which experts a token selects), both sides decide from the same fp32 values.
So the oracle's top-k is applied to the GPU's own fp32 logits and must match
bit for bit; against the oracle's own logits, only near-tie tokens may differ.
"""
import numpy as np

import oracle.moe_oracle as O
from tests.metrics import TOL, floored_rel_err

NEAR_TIE = 1e-4


def dev(a):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t):
    import torch
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def widen_out(a, dtype):
    return O.widen(a, dtype)


def near_tie_tokens(L, k, tau=NEAR_TIE):
    """Tokens whose sorted top k+1 logits have an adjacent gap below tau."""
    L = np.asarray(L, dtype=np.float64)
    E = L.shape[1]
    kk = min(k + 1, E)
    s = -np.sort(-L, axis=1)[:, :kk]
    if kk < 2:
        return np.zeros(L.shape[0], dtype=bool)
    return (np.diff(-s, axis=1) < tau).any(axis=1)


def check_routing(p, gpu_logits, gpu_idx, gpu_w, ref_logits, tau=NEAR_TIE):
    """Returns the number of near-tie tokens where the GPU differs from the
    oracle's own routing (asserts there is no other difference)."""
    err = floored_rel_err(gpu_logits, ref_logits)
    assert err <= 1e-5, f"logits err {err}"
    idx_g, w_g = O.topk_softmax(gpu_logits, p.k)
    assert np.array_equal(gpu_idx, idx_g), "top-k differs from the oracle on the GPU's own logits"
    assert np.allclose(gpu_w, w_g, rtol=2e-6, atol=1e-7), np.abs(gpu_w - w_g).max()
    idx_o, _ = O.topk_softmax(ref_logits, p.k)
    diff = ~(idx_o == gpu_idx).all(axis=1)
    if tau == 0:
        assert not diff.any(), f"{diff.sum()} tokens differ with exact logits"
        return 0
    nt = near_tie_tokens(ref_logits, p.k, tau)
    assert not (diff & ~nt).any(), f"{(diff & ~nt).sum()} tokens differ outside near ties"
    return int(diff.sum())


def check_close(got, ref, dtype, what, tol=None):
    err = floored_rel_err(got, ref)
    t = TOL[dtype] if tol is None else tol
    assert err <= t, f"{what}: err {err:.3e} > {t}"
    return err
