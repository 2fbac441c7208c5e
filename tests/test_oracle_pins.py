"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle.moe_oracle as O
import workloads
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)


def test_generator_deterministic():
    w = workloads.get("tiny_fp32")
    a, b = workloads.generate(w), workloads.generate(w)
    for key in ("x", "w_gate", "w1", "w3", "w2"):
        assert a[key].tobytes() == b[key].tobytes()
    c = workloads.generate(w.replace(seed=1))
    assert c["x"].tobytes() != a["x"].tobytes()


def test_generator_bf16_conversion_is_rne():
    import torch
    x = np.random.default_rng(2).standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.f32_to_bf16_bits(x), ref)


def test_tiny_workload_layer_shapes():
    w = workloads.get("tiny_fp32")
    o = O.moe_layer(w, workloads.generate(w))
    assert o["y"].shape == (w.T, w.d)
    assert int(o["counts_all"].sum()) == w.T * w.k
    assert o["offsets"][-1] == w.T * w.k  # all experts local
