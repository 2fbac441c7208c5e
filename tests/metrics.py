"""Comparison metrics shared by the tests (no method arithmetic here).

Floating-point outputs are compared with a floored relative error: for each
element, |g - r| / max(|r|, rms(r)), with rms taken over the whole reference
tensor.  An unfloored elementwise relative error is unbounded next to zero and
a norm-wise error hides local mistakes; the floor at the tensor's rms keeps
the check elementwise while ignoring cancellation noise.  Bounds: 2e-2 for
bf16 outputs, 1e-5 for fp32 outputs.
"""
import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-5}

# One stage of the layer (h, y_packed or y) fed with the GPU's own stored
# input to that stage: the two sides differ only by fp32 accumulation order
# and the one rounding to the storage type, so at most one bf16 step (2^-7 of
# the value) plus accumulation error (below 1e-6 relative) for bf16 outputs.
STAGE_TOL = {"bf16": 1e-2, "f32": 1e-5}


def floored_rel_err(got, ref) -> float:
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), "non-finite values in result"
    rms = float(np.sqrt(np.mean(r * r)))
    floor = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(g - r) / floor))


def bf16_bits_to_f64(b) -> np.ndarray:
    u = np.asarray(b).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)
