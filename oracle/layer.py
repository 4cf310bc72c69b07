"""MoE layer forward and backward (oracle; test infrastructure only).

What is computed ([MTP] "Three design decisions that matter" and the
paragraph after them; [CARD] "Use the functional API"): routed token rows go
to their expert, each expert is a SwiGLU feed-forward block evaluated as an
expert-grouped GEMM (gate/up projection, SwiGLU, down projection), and the
expert outputs are combined back to token order weighted by the router
weights.  The backward computes dX and all weight gradients, and the gradient
of the router weight inside the SwiGLU backward (the SonicMoE-style
calculation the pages name).  No token is dropped ([MTP] "Key Takeaways").

Notation (weights stored one row per output feature, see ``workloads``):
    g = x W_g[e]^T,  u = x W_u[e]^T,  a = silu(g) * u,  y = a W_d[e]^T
    silu(g) = g * sigmoid(g)
Full layer: out[t] = sum_j w[t, j] * y(t, j), j ascending.
Expert share (one GPU under expert parallelism): out_rows[r] = w[r] * y(r);
the sum over a token's k experts happens at the token's source GPU and is not
part of this share.

Everything here is fp64 on exact bf16 inputs, except where a step's own
precision is part of the method (the MXFP8 path rounds a to bf16 before
quantising it).  Results are returned unrounded (fp64) unless noted.
"""
from __future__ import annotations

import numpy as np

from . import bf16, mxfp8
from .route import route as _route


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def silu(v):
    return v * sigmoid(v)


def expert_ffn(x, wg, wu, wd):
    """One expert on rows x [n, H]: -> (g, u, a, y), fp64."""
    g = x @ wg.T
    u = x @ wu.T
    a = silu(g) * u
    y = a @ wd.T
    return g, u, a, y


def _weights(inp):
    return (bf16.decode(inp["w_gate"]), bf16.decode(inp["w_up"]), bf16.decode(inp["w_down"]))


def rows_ffn(x_rows, row_expert, wg, wu, wd):
    """FFN of each row under its own expert, arrival order.  Rows whose expert
    id is out of range get zeros."""
    R, H = x_rows.shape
    I = wg.shape[1]
    g = np.zeros((R, I)); u = np.zeros((R, I)); a = np.zeros((R, I)); y = np.zeros((R, H))
    for e in range(wg.shape[0]):
        sel = np.nonzero(row_expert == e)[0]
        if sel.size == 0:
            continue
        g[sel], u[sel], a[sel], y[sel] = expert_ffn(x_rows[sel], wg[e], wu[e], wd[e])
    return g, u, a, y


def forward_full(inp, renorm: int | None = None):
    """Full layer, bf16 mode: route, expert FFN, combine.  -> dict."""
    sh = inp["shape"]
    x = bf16.decode(inp["x"])
    bias = inp["bias"]
    idx, w, z = _route(x.astype(np.float32), bf16.decode(inp["w_router"]).astype(np.float32),
                       bias, sh.k, sh.renorm if renorm is None else renorm)
    wg, wu, wd = _weights(inp)
    row_expert = idx.reshape(-1)
    x_rows = np.repeat(x, sh.k, axis=0)                 # row r = t*k + j comes from token t
    g, u, a, y = rows_ffn(x_rows, row_expert, wg, wu, wd)
    T, H = x.shape
    out = np.zeros((T, H))
    yk = y.reshape(T, sh.k, H)
    for j in range(sh.k):                               # fixed ascending order
        out += w[:, j, None].astype(np.float64) * yk[:, j]
    return {"topk_idx": idx, "topk_w": w, "logits": z, "row_expert": row_expert,
            "g": g, "u": u, "a": a, "y": y, "out": out}


def forward_share(inp):
    """Expert share, bf16 mode: out_rows[r] = w[r] * y(r), arrival order."""
    x = bf16.decode(inp["x"])
    wg, wu, wd = _weights(inp)
    re = inp["row_expert"]
    g, u, a, y = rows_ffn(x, re, wg, wu, wd)
    w = inp["row_w"].astype(np.float64)
    return {"g": g, "u": u, "a": a, "y": y, "out": w[:, None] * y}


def quantized_weights(inp):
    """MXFP8 weights: gate/up rows quantised along H, down rows along I."""
    wg, wu, wd = _weights(inp)
    return {"gate": mxfp8.quantize(wg), "up": mxfp8.quantize(wu), "down": mxfp8.quantize(wd)}


def forward_share_mxfp8(inp, qw=None):
    """Expert share, MXFP8 mode.

    x rows and the gate/up weights are quantised along H, the down weights
    along I (blocks of 32 along each GEMM's K).  g and u are exact products of
    the dequantised operands (fp64); a = silu(g) * u is rounded to bf16 and
    then quantised along I; y = D(a_q) D(W_d)^T; out_rows = w * y.
    """
    x = bf16.decode(inp["x"])
    re = inp["row_expert"]
    qw = quantized_weights(inp) if qw is None else qw
    xc, xs = mxfp8.quantize(x)
    xd = mxfp8.dequantize(xc, xs)
    wg = mxfp8.dequantize(*qw["gate"]); wu = mxfp8.dequantize(*qw["up"])
    wd = mxfp8.dequantize(*qw["down"])
    R, H = x.shape
    I = wg.shape[1]
    a_bits = np.zeros((R, I), dtype=np.uint16)
    y = np.zeros((R, H))
    for e in range(wg.shape[0]):
        sel = np.nonzero(re == e)[0]
        if sel.size == 0:
            continue
        g = xd[sel] @ wg[e].T
        u = xd[sel] @ wu[e].T
        a_bits[sel] = bf16.encode(silu(g) * u)
        ac, as_ = mxfp8.quantize(bf16.decode(a_bits[sel]))
        y[sel] = mxfp8.dequantize(ac, as_) @ wd[e].T
    w = inp["row_w"].astype(np.float64)
    return {"x_codes": xc, "x_scales": xs, "a_bits": a_bits, "y": y, "out": w[:, None] * y}


def backward_share(inp):
    """Expert share backward, bf16 mode, loss L = sum_r <dY[r], out_rows[r]>.

    dA' = dY W_d[e]            (gradient w.r.t. a, before the router weight)
    dw[r] = <dA'[r], a[r]>     (= <dY[r], y[r]>: router-weight gradient)
    dA  = w * dA'
    dg  = dA * u * s * (1 + g (1 - s)),  s = sigmoid(g)
    du  = dA * silu(g)
    dX  = dg W_g[e] + du W_u[e]
    dW_g[e] = dg_e^T X_e,  dW_u[e] = du_e^T X_e,  dW_d[e] = (w dY)_e^T a_e
    """
    x = bf16.decode(inp["x"])
    wg, wu, wd = _weights(inp)
    re = inp["row_expert"]
    w = inp["row_w"].astype(np.float64)
    dY = bf16.decode(inp["dY"])
    R, H = x.shape
    E, I, _ = wg.shape
    dX = np.zeros((R, H)); dw = np.zeros(R); dw_alt = np.zeros(R)
    dWg = np.zeros((E, I, H)); dWu = np.zeros((E, I, H)); dWd = np.zeros((E, H, I))
    for e in range(E):
        sel = np.nonzero(re == e)[0]
        if sel.size == 0:
            continue
        xe = x[sel]
        g, u, a, y = expert_ffn(xe, wg[e], wu[e], wd[e])
        dYe = dY[sel]
        dAp = dYe @ wd[e]
        dw[sel] = np.einsum("ri,ri->r", dAp, a)
        dw_alt[sel] = np.einsum("rh,rh->r", dYe, y)
        dA = w[sel, None] * dAp
        s = sigmoid(g)
        dg = dA * u * s * (1.0 + g * (1.0 - s))
        du = dA * silu(g)
        dX[sel] = dg @ wg[e] + du @ wu[e]
        dWg[e] = dg.T @ xe
        dWu[e] = du.T @ xe
        dWd[e] = (w[sel, None] * dYe).T @ a
    return {"dX": dX, "dW_gate": dWg, "dW_up": dWu, "dW_down": dWd,
            "d_row_w": dw, "d_row_w_alt": dw_alt}


def ring_contents(sched, x_bits, src_of_row):
    """Final ring state after the forward permute: minibatches are written in
    order, so a slot ends up holding the last minibatch that mapped to it.
    Slots never written stay zero."""
    H = x_bits.shape[1]
    ring = np.zeros((sched.ring_rows, H), dtype=x_bits.dtype)
    written = np.zeros(sched.ring_rows, dtype=bool)
    for r in np.argsort(sched.sorted_pos, kind="stable"):
        p = sched.sorted_pos[r]
        if p < 0:
            continue
        ring[p % sched.ring_rows] = x_bits[src_of_row[r]]
        written[p % sched.ring_rows] = True
    return ring, written
