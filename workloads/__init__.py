"""Seeded synthetic inputs for the MoE layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds *no* arithmetic of the method itself (no gating, no
permutation, no expert math): it only defines workload shapes and draws the
input tensors from a seeded generator.

Workloads.  The subject is the DeepSeek-V3 MoE dispatch/combine workload of
"CUCo: An Agentic Framework for Compute and Communication Co-design"
(Abstract; Table 4, row "MoE Dispatch/Combine").  The pages print no shapes,
so the shapes below are the DeepSeek-V3 layer shapes (hidden 7168, 256 routed
experts, top-8, expert intermediate 2048) for one GPU's share of 32 experts,
plus a tiny fp32 case and a dense 8-expert case.  The skewed variants add a
Zipf-like per-expert bias to the gate logits, standing in for the pages'
"imbalanced sparse routing" (gist.science summary of the same paper, §4
Results).

Input recipe (one generator per workload, ``numpy.random.default_rng(seed)``,
PCG64, seed 0 unless stated):

* draw order: x[T,d], W_g[d,E], then per local expert W1[d,f], all W3[d,f],
  all W2[f,d], each with ``standard_normal(dtype=float32)``;
* x ~ N(0,1); every weight ~ N(0, 1/d): the float32 draw is multiplied by
  1/sqrt(d) in float64 and rounded to float32;
* bf16 workloads store every tensor as bf16 bit patterns (``uint16``), rounded
  from float32 to nearest-even; fp32 workloads store float32;
* optional gate bias b[e] = 1.5 * ln(1/(e+1)) in float64, stored as float32
  (expert index e is the 0-based global index).

Tensors are row-major: x[T,d], w_gate[d,E], w1/w3[n_local,d,f], w2[n_local,f,d].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get",
    "generate",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "skew_bias",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    d: int          # hidden size
    E: int          # routed experts (global)
    k: int          # experts per token
    f: int          # SwiGLU intermediate size per expert
    expert_lo: int  # first local expert
    n_local: int    # number of local experts
    dtype: str      # "f32" or "bf16"
    skew: bool = False
    seed: int = 0
    desc: str = ""

    @property
    def rows_max(self) -> int:
        return self.T * min(self.k, self.n_local)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 64, 128, 8, 2, 256, 0, 8, "f32",
                 desc="tiny fp32 layer, all experts local"),
        Workload("dsv3_decode", 128, 7168, 256, 8, 2048, 0, 32, "bf16",
                 desc="DeepSeek-V3-shaped decode share, experts 0-31 local"),
        Workload("dsv3_prefill", 4096, 7168, 256, 8, 2048, 0, 32, "bf16",
                 desc="DeepSeek-V3-shaped prefill share, experts 0-31 local"),
        Workload("dsv3_decode_skew", 128, 7168, 256, 8, 2048, 0, 32, "bf16", skew=True,
                 desc="decode share with Zipf-like gate bias (imbalanced routing)"),
        Workload("dsv3_prefill_skew", 4096, 7168, 256, 8, 2048, 0, 32, "bf16", skew=True,
                 desc="prefill share with Zipf-like gate bias (imbalanced routing)"),
        Workload("dense8_prefill", 16384, 4096, 8, 2, 14336, 0, 8, "bf16",
                 desc="dense-routing 8-expert layer, all local, compute-bound"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the uint16 bits.

    Storage conversion for generated inputs only.  NaN does not occur in
    generated data and is not handled specially.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def skew_bias(E: int) -> np.ndarray:
    """Zipf-like gate bias b[e] = 1.5 * ln(1/(e+1)), float64 then float32."""
    e = np.arange(E, dtype=np.float64)
    return (1.5 * np.log(1.0 / (e + 1.0))).astype(np.float32)


def _draw(rng: np.random.Generator, shape, scale: Optional[float], bf16: bool) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale is not None:
        a = (a.astype(np.float64) * scale).astype(np.float32)
    return f32_to_bf16_bits(a) if bf16 else a


def generate(w: Workload, with_experts: bool = True) -> Dict[str, np.ndarray]:
    """Draw all inputs of workload ``w``.

    Returns numpy arrays: x, w_gate, bias (or None), and, if ``with_experts``,
    w1, w3, w2.  bf16 tensors are uint16 bit patterns.
    """
    rng = np.random.default_rng(w.seed)
    bf = w.dtype == "bf16"
    s = 1.0 / math.sqrt(w.d)
    out: Dict[str, np.ndarray] = {}
    out["x"] = _draw(rng, (w.T, w.d), None, bf)
    out["w_gate"] = _draw(rng, (w.d, w.E), s, bf)
    out["bias"] = skew_bias(w.E) if w.skew else None
    if with_experts:
        et = np.uint16 if bf else np.float32
        w1 = np.empty((w.n_local, w.d, w.f), dtype=et)
        w3 = np.empty((w.n_local, w.d, w.f), dtype=et)
        w2 = np.empty((w.n_local, w.f, w.d), dtype=et)
        for e in range(w.n_local):
            w1[e] = _draw(rng, (w.d, w.f), s, bf)
        for e in range(w.n_local):
            w3[e] = _draw(rng, (w.d, w.f), s, bf)
        for e in range(w.n_local):
            w2[e] = _draw(rng, (w.f, w.d), s, bf)
        out["w1"], out["w3"], out["w2"] = w1, w3, w2
    return out


def integer_inputs(w: Workload, lo: int = -2, hi: int = 2, seed: int = 1) -> Dict[str, np.ndarray]:
    """Small-integer x and W_g (values in [lo, hi]) in the workload's dtype.

    Every partial sum of x.W_g is then a small integer, exact in float32 under
    any summation order, so the router logits are exact on every device.
    """
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=(w.T, w.d)).astype(np.float32)
    g = rng.integers(lo, hi + 1, size=(w.d, w.E)).astype(np.float32)
    if w.dtype == "bf16":
        return {"x": f32_to_bf16_bits(x), "w_gate": f32_to_bf16_bits(g)}
    return {"x": x, "w_gate": g}
