"""Seeded synthetic workloads for the MoE layer.

This module only *draws* inputs.  It holds none of the layer's arithmetic: no
routing, no scheduling, no quantisation, no GEMM.  Both the CPU oracle and the
GPU path receive exactly the arrays produced here, so the two sides always see
the same values.

Every tensor is drawn in fp32 from ``numpy.random.default_rng(seed)`` (PCG64)
in the fixed order listed in each function, then rounded to bf16 by torch's
CPU cast (round-to-nearest-even).  bf16 tensors are returned as ``uint16`` bit
patterns; ``bf16_to_f32`` widens them for the oracle.

Weight storage follows the row-per-output-feature convention:

* ``w_router`` [E, H]        logits z = x . w_router[e]
* ``w_gate``   [E, I, H]     g = x @ w_gate[e].T
* ``w_up``     [E, I, H]     u = x @ w_up[e].T
* ``w_down``   [E, H, I]     y = a @ w_down[e].T

Initialisation is N(0, 1/fan_in) for every projection (fan_in = H for the
router, gate and up, I for down) and x, dY ~ N(0, 1).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = [
    "FullLayerShape", "ExpertShareShape", "FULL_LAYER", "EXPERT_SHARE",
    "bf16_bits", "bf16_to_f32", "zipf_local_weights",
    "make_full_layer", "make_expert_share",
]


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), via torch's CPU RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class FullLayerShape:
    """A whole MoE layer on one GPU: T tokens routed top-k over E local experts."""
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    renorm: int          # 1: weights renormalised over the k chosen experts
    bias_var: float      # variance of the per-expert router logit offset (0: none)
    seed: int

    @property
    def R(self) -> int:
        return self.T * self.k


@dataclasses.dataclass(frozen=True)
class ExpertShareShape:
    """One GPU's expert share under expert parallelism: R routed rows already
    resident in arrival order, E local experts with Zipf-skewed popularity."""
    name: str
    R: int
    H: int
    I: int
    E: int
    sources: int         # simulated source ranks, R/sources consecutive rows each
    zipf_s: float
    seed: int


FULL_LAYER = {
    "tiny": FullLayerShape("tiny", T=256, H=256, I=128, E=8, k=2, renorm=0,
                           bias_var=0.0, seed=0),
    "full": FullLayerShape("full", T=4096, H=2048, I=768, E=128, k=8, renorm=1,
                           bias_var=0.5, seed=1),
    # micro shapes for brute force and finite differences
    "micro": FullLayerShape("micro", T=8, H=64, I=32, E=4, k=2, renorm=1,
                            bias_var=0.5, seed=11),
}

EXPERT_SHARE = {
    "ep64_fwd": ExpertShareShape("ep64_fwd", R=16384, H=7168, I=2048, E=4,
                                 sources=64, zipf_s=1.2, seed=2),
    "ep_bwd": ExpertShareShape("ep_bwd", R=24576, H=7168, I=2048, E=8,
                               sources=64, zipf_s=1.2, seed=4),
    # reduced shapes: same recipe, sizes the oracle finishes in seconds while
    # still spanning several GEMM tiles and ragged tails
    "small": ExpertShareShape("small", R=1000, H=512, I=256, E=4,
                              sources=8, zipf_s=1.2, seed=21),
    "small8": ExpertShareShape("small8", R=1536, H=768, I=512, E=8,
                               sources=8, zipf_s=1.2, seed=22),
    "micro": ExpertShareShape("micro", R=48, H=64, I=32, E=4,
                              sources=4, zipf_s=1.2, seed=23),
}


def zipf_local_weights(E: int, s: float) -> np.ndarray:
    """Popularity of global expert ranks 1..E under Zipf(s), renormalised over
    those E (the local experts of EP rank 0 with contiguous placement)."""
    q = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    return q / q.sum()


def _normal(rng, shape, std):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def make_full_layer(shape: FullLayerShape | str, seed: int | None = None) -> dict:
    """Draw order: x, w_router, bias (if any), w_gate, w_up, w_down, dY."""
    if isinstance(shape, str):
        shape = FULL_LAYER[shape]
    rng = np.random.default_rng(shape.seed if seed is None else seed)
    T, H, I, E = shape.T, shape.H, shape.I, shape.E
    out = {"shape": shape}
    out["x"] = bf16_bits(_normal(rng, (T, H), 1.0))
    out["w_router"] = bf16_bits(_normal(rng, (E, H), 1.0 / math.sqrt(H)))
    if shape.bias_var > 0:
        out["bias"] = _normal(rng, (E,), math.sqrt(shape.bias_var))
    else:
        out["bias"] = None
    out["w_gate"] = bf16_bits(_normal(rng, (E, I, H), 1.0 / math.sqrt(H)))
    out["w_up"] = bf16_bits(_normal(rng, (E, I, H), 1.0 / math.sqrt(H)))
    out["w_down"] = bf16_bits(_normal(rng, (E, H, I), 1.0 / math.sqrt(I)))
    out["dY"] = bf16_bits(_normal(rng, (T, H), 1.0))
    return out


def make_expert_share(shape: ExpertShareShape | str, seed: int | None = None,
                      with_dy: bool = True) -> dict:
    """Draw order: row_expert, row_w, x_rows, w_gate, w_up, w_down, dY.

    ``row_expert[r]`` is drawn i.i.d. from the local Zipf weights; ``row_w[r]``
    is the first entry of a softmax over 8 standard-normal logits (the weight
    a top-8 router would give that row; the draw is input data, not routing).
    Arrival order is source-major: row r comes from source rank r // (R/sources).
    """
    if isinstance(shape, str):
        shape = EXPERT_SHARE[shape]
    rng = np.random.default_rng(shape.seed if seed is None else seed)
    R, H, I, E = shape.R, shape.H, shape.I, shape.E
    out = {"shape": shape}
    q = zipf_local_weights(E, shape.zipf_s)
    out["row_expert"] = rng.choice(E, size=R, p=q).astype(np.int32)
    lg = rng.standard_normal((R, 8)).astype(np.float64)
    ex = np.exp(lg - lg.max(axis=1, keepdims=True))
    out["row_w"] = (ex[:, 0] / ex.sum(axis=1)).astype(np.float32)
    out["x"] = bf16_bits(_normal(rng, (R, H), 1.0))
    out["w_gate"] = bf16_bits(_normal(rng, (E, I, H), 1.0 / math.sqrt(H)))
    out["w_up"] = bf16_bits(_normal(rng, (E, I, H), 1.0 / math.sqrt(H)))
    out["w_down"] = bf16_bits(_normal(rng, (E, H, I), 1.0 / math.sqrt(I)))
    if with_dy:
        out["dY"] = bf16_bits(_normal(rng, (R, H), 1.0))
    return out
