"""Top-k softmax router (oracle; test infrastructure only).

The pages take the routing result as an input: [CARD] "Use the functional
API" passes ``topk_experts`` into ``build_schedule``.  Routing itself is the
standard softmax top-k router of an MoE transformer layer; this module states
the reading used here:

* logits z[t, e] = sum_h x[t, h] * W_r[e, h] (+ b[e]), accumulated in fp32
  in ascending h starting from +0.0, then the bias added in fp32.  The product
  of two bf16 values is exact in fp32, so a fused multiply-add and a separate
  multiply and add give the same sum; only the order matters, and it is fixed.
  The top-k decision is an integer decided by float values, so it is taken in
  the precision the kernel uses (fp32, this order) on both sides.
* top-k: experts sorted by descending z, ties to the lower expert id; slot 0
  holds the largest.  +0 and -0 compare equal.
* weights: renorm=1 -> softmax over the k chosen logits; renorm=0 -> the full
  softmax over all E experts, read at the chosen ones.  Computed in fp64 and
  rounded to fp32.
"""
from __future__ import annotations

import numpy as np


def logits_fp32(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """x [T,H] fp32 (bf16 values), w_router [E,H] fp32 (bf16 values), bias [E]
    fp32 or None -> z [T,E] fp32, summed in ascending h."""
    x = np.asarray(x, dtype=np.float32)
    w = np.asarray(w_router, dtype=np.float32)
    T, H = x.shape
    E = w.shape[0]
    acc = np.zeros((T, E), dtype=np.float32)
    for h in range(H):
        acc = acc + x[:, h, None] * w[None, :, h]     # fp32 ops, product exact
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float32)[None, :]
    return acc


def topk(z: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, descending, ties -> lower id."""
    T, E = z.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -z.astype(np.float64)), axis=-1)
    return order[:, :k].astype(np.int32)


def weights(z: np.ndarray, idx: np.ndarray, renorm: int) -> np.ndarray:
    """Router weights for the chosen experts, fp64 math rounded to fp32."""
    z64 = z.astype(np.float64)
    zsel = np.take_along_axis(z64, idx.astype(np.int64), axis=1)
    if renorm:
        ex = np.exp(zsel - zsel[:, :1])
        w = ex / ex.sum(axis=1, keepdims=True)
    else:
        ex = np.exp(z64 - z64.max(axis=1, keepdims=True))
        p = ex / ex.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return w.astype(np.float32)


def route(x, w_router, bias, k: int, renorm: int):
    """-> (topk_idx [T,k] int32, topk_w [T,k] fp32, z [T,E] fp32)."""
    z = logits_fp32(x, w_router, bias)
    idx = topk(z, k)
    return idx, weights(z, idx, renorm), z
