"""MoE layer forward and backward (oracle; test infrastructure only).

What is computed ([MTP] "Three design decisions that matter" and the
paragraph after them; [CARD] "Use the functional API"): routed token rows go
to their expert, each expert is a SwiGLU feed-forward block evaluated as an
expert-grouped GEMM (gate/up projection, SwiGLU, down projection), and the
expert outputs are combined back to token order weighted by the router
weights.  The backward computes dX and all weight gradients, and the gradient
of the router weight inside the SwiGLU backward (the SonicMoE-style
calculation the pages name).  No token is dropped ([MTP] "Key Takeaways").
The full-layer backward also carries the gradient through the router (the
pages take routing as an input, so this part is the plain chain rule through
the softmax top-k router that the route module states: softmax Jacobian,
then the linear logit map).

Notation (weights stored one row per output feature, see ``workloads``):
    g = x W_g[e]^T,  u = x W_u[e]^T,  a = silu(g) * u,  y = a W_d[e]^T
    silu(g) = g * sigmoid(g)
Full layer: out[t] = sum_j w[t, j] * y(t, j), j ascending.
Expert share (one GPU under expert parallelism): out_rows[r] = w[r] * y(r);
the sum over a token's k experts happens at the token's source GPU and is not
part of this share.

Precision.  The pages' BF16 mode (and the MXFP8 mode's "accumulate in fp32,
bf16 output") is read as: every GEMM operand is a bf16 tensor, every GEMM
accumulates exactly (here fp64, on the device fp32), and the layer's outputs
are bf16 tensors.  With ``bf16_mode=True`` (the default) the oracle therefore
rounds, once each and to nearest even, exactly the values that are bf16
tensors in that reading -- the SwiGLU output a (GEMM2 operand), the layer
output, and in the backward dg/du (operands of the dX and gate/up weight
GEMMs), w*a (operand of the down weight GEMM) and dX -- and computes all
else in fp64.  ``bf16_mode=False`` is the exact-math layer, pinned by finite
differences and autograd; the bf16 mode is pinned against it within bf16's
error bound.
"""
from __future__ import annotations

import numpy as np

from . import bf16, mxfp8
from .route import route as _route


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def silu(v):
    return v * sigmoid(v)


def rnd(v, on: bool):
    """Round to bf16 (nearest even) when on, else leave exact."""
    return bf16.round_rne(v) if on else v


def expert_ffn(x, wg, wu, wd, bf16_mode: bool = False):
    """One expert on rows x [n, H]: -> (g, u, a, y), fp64.  In bf16 mode a is
    the bf16 GEMM2 operand."""
    g = x @ wg.T
    u = x @ wu.T
    a = rnd(silu(g) * u, bf16_mode)
    y = a @ wd.T
    return g, u, a, y


def _weights(inp):
    return (bf16.decode(inp["w_gate"]), bf16.decode(inp["w_up"]), bf16.decode(inp["w_down"]))


def rows_ffn(x_rows, row_expert, wg, wu, wd, bf16_mode: bool = False):
    """FFN of each row under its own expert, arrival order.  Rows whose expert
    id is out of range get zeros."""
    R, H = x_rows.shape
    I = wg.shape[1]
    g = np.zeros((R, I)); u = np.zeros((R, I)); a = np.zeros((R, I)); y = np.zeros((R, H))
    for e in range(wg.shape[0]):
        sel = np.nonzero(row_expert == e)[0]
        if sel.size == 0:
            continue
        g[sel], u[sel], a[sel], y[sel] = expert_ffn(x_rows[sel], wg[e], wu[e], wd[e], bf16_mode)
    return g, u, a, y


def forward_full(inp, renorm: int | None = None, bf16_mode: bool = True):
    """Full layer: route, expert FFN, combine.  -> dict (out in bf16 mode is
    the bf16 output, out_exact the value before that rounding)."""
    sh = inp["shape"]
    x = bf16.decode(inp["x"])
    bias = inp["bias"]
    idx, w, z = _route(x.astype(np.float32), bf16.decode(inp["w_router"]).astype(np.float32),
                       bias, sh.k, sh.renorm if renorm is None else renorm)
    wg, wu, wd = _weights(inp)
    row_expert = idx.reshape(-1)
    x_rows = np.repeat(x, sh.k, axis=0)                 # row r = t*k + j comes from token t
    g, u, a, y = rows_ffn(x_rows, row_expert, wg, wu, wd, bf16_mode)
    T, H = x.shape
    out = np.zeros((T, H))
    yk = y.reshape(T, sh.k, H)
    for j in range(sh.k):                               # fixed ascending order
        out += w[:, j, None].astype(np.float64) * yk[:, j]
    return {"topk_idx": idx, "topk_w": w, "logits": z, "row_expert": row_expert,
            "g": g, "u": u, "a": a, "y": y, "out": rnd(out, bf16_mode), "out_exact": out}


def forward_share(inp, bf16_mode: bool = True):
    """Expert share: out_rows[r] = w[r] * y(r), arrival order."""
    x = bf16.decode(inp["x"])
    wg, wu, wd = _weights(inp)
    re = inp["row_expert"]
    g, u, a, y = rows_ffn(x, re, wg, wu, wd, bf16_mode)
    w = inp["row_w"].astype(np.float64)
    out = w[:, None] * y
    return {"g": g, "u": u, "a": a, "y": y, "out": rnd(out, bf16_mode), "out_exact": out}


def quantized_weights(inp):
    """MXFP8 weights: gate/up rows quantised along H, down rows along I."""
    wg, wu, wd = _weights(inp)
    return {"gate": mxfp8.quantize(wg), "up": mxfp8.quantize(wu), "down": mxfp8.quantize(wd)}


def forward_share_mxfp8(inp, qw=None, allow: bool = False):
    """Expert share, MXFP8 mode.

    x rows and the gate/up weights are quantised along H, the down weights
    along I (blocks of 32 along each GEMM's K).  g and u are exact products of
    the dequantised operands (fp64); a = silu(g) * u is rounded to bf16 and
    then quantised along I; y = D(a_q) D(W_d)^T; out_rows = w * y.
    With ``allow`` also out_allow: how far out_rows may move because a is a
    GEMM output whose E4M3 codes another correct evaluation may decide
    differently (``qd_spread`` of a, through |W_d|, times |w|).
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
    G = np.zeros((R, I)); U = np.zeros((R, I))
    y = np.zeros((R, H)); y_allow = np.zeros((R, H))
    for e in range(wg.shape[0]):
        sel = np.nonzero(re == e)[0]
        if sel.size == 0:
            continue
        g = xd[sel] @ wg[e].T
        u = xd[sel] @ wu[e].T
        G[sel], U[sel] = g, u
        a_bits[sel] = bf16.encode(silu(g) * u)
        ac, as_ = mxfp8.quantize(bf16.decode(a_bits[sel]))
        y[sel] = mxfp8.dequantize(ac, as_) @ wd[e].T
        if allow:
            y_allow[sel] = qd_spread(silu(g) * u) @ np.abs(wd[e]).T
    w = inp["row_w"].astype(np.float64)
    out = w[:, None] * y
    res = {"x_codes": xc, "x_scales": xs, "a_bits": a_bits, "g": G, "u": U, "y": y, "out": bf16.round_rne(out),
           "out_exact": out}
    if allow:
        res["out_allow"] = np.abs(w)[:, None] * y_allow
    return res


def bf16_spread(v, rel: float | None = None):
    """How far bf16(v') may lie from bf16(v), per element, over all v' with
    |v'_i - v_i| <= rel |v_i| (rel defaults to DECISION_REL): v are the exact
    values of a GEMM output that is rounded to bf16 as the next GEMM's
    operand, and another correct evaluation of that GEMM may land on the
    other side of a rounding midpoint.  Rounding is monotone, so the
    interval's two ends bound every reachable value; 0 where no decision can
    change."""
    rel = DECISION_REL if rel is None else rel
    v = np.asarray(v, dtype=np.float64)
    ref = bf16.round_rne(v)
    return np.maximum(np.abs(bf16.round_rne(v * (1.0 - rel)) - ref), np.abs(bf16.round_rne(v * (1.0 + rel)) - ref))


def _backward_rows(x, re, w, dY, wg, wu, wd, bf16_mode: bool, allow: bool = False):
    """Expert backward of routed rows (arrival order), loss
    L = sum_r <dY[r], w[r] y(r)>:

    dA' = dY W_d[e]            (gradient w.r.t. a, before the router weight)
    dw[r] = <dA'[r], a[r]>     (= <dY[r], y[r]>: router-weight gradient)
    dA  = w * dA'
    dg  = dA * u * s * (1 + g (1 - s)),  s = sigmoid(g)
    du  = dA * silu(g)
    dX_rows = dg W_g[e] + du W_u[e]          (not rounded here)
    dW_g[e] = dg_e^T X_e,  dW_u[e] = du_e^T X_e,  dW_d[e] = dY_e^T (w a)_e
    In bf16 mode dg, du and w*a are bf16 tensors (GEMM operands); g, u, a,
    dA' and the fp32 outputs dW, dw are exact.  Rows whose expert id is out
    of range get zeros.  With ``allow`` (bf16 mode) also dW_gate_allow,
    dW_up_allow, dW_down_allow and dX_rows_allow: how far each may move
    because dg, du and w*a are GEMM outputs whose bf16 rounding another
    correct evaluation may decide the other way (``bf16_spread`` through
    |X|, |dY| and |W|).
    """
    R, H = x.shape
    E, I, _ = wg.shape
    dX = np.zeros((R, H)); dw = np.zeros(R); dw_alt = np.zeros(R)
    dWg = np.zeros((E, I, H)); dWu = np.zeros((E, I, H)); dWd = np.zeros((E, H, I))
    allow = allow and bf16_mode
    if allow:
        A = {"dW_gate": np.zeros_like(dWg), "dW_up": np.zeros_like(dWu), "dW_down": np.zeros_like(dWd),
             "dX_rows": np.zeros((R, H))}
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
        dgx, dux, wax = dA * u * s * (1.0 + g * (1.0 - s)), dA * silu(g), w[sel, None] * a
        dg = rnd(dgx, bf16_mode)
        du = rnd(dux, bf16_mode)
        dX[sel] = dg @ wg[e] + du @ wu[e]
        dWg[e] = dg.T @ xe
        dWu[e] = du.T @ xe
        dWd[e] = dYe.T @ rnd(wax, bf16_mode)
        if allow:
            sg, su = bf16_spread(dgx), bf16_spread(dux)
            A["dW_gate"][e] = sg.T @ np.abs(xe)
            A["dW_up"][e] = su.T @ np.abs(xe)
            A["dW_down"][e] = np.abs(dYe).T @ bf16_spread(wax)
            A["dX_rows"][sel] = sg @ np.abs(wg[e]) + su @ np.abs(wu[e])
    res = {"dX_rows": dX, "dW_gate": dWg, "dW_up": dWu, "dW_down": dWd, "d_row_w": dw, "d_row_w_alt": dw_alt}
    if allow:
        res.update({k + "_allow": v for k, v in A.items()})
    return res


def backward_share(inp, bf16_mode: bool = True, allow: bool = False):
    """Expert share backward (rows in arrival order), see ``_backward_rows``;
    dX is each row's dX_rows, a bf16 tensor in bf16 mode.  With ``allow``
    also the decision allowances of ``_backward_rows`` (dX_allow for dX)."""
    wg, wu, wd = _weights(inp)
    g = _backward_rows(bf16.decode(inp["x"]), inp["row_expert"], inp["row_w"].astype(np.float64),
                       bf16.decode(inp["dY"]), wg, wu, wd, bf16_mode, allow)
    g["dX_exact"] = g.pop("dX_rows")
    g["dX"] = rnd(g["dX_exact"], bf16_mode)
    if "dX_rows_allow" in g:
        g["dX_allow"] = g.pop("dX_rows_allow")
    return g


def router_logit_grad(z, idx, d_w, renorm: int):
    """Gradient of the loss w.r.t. the router logits z [T, E], given its
    gradient d_w [T, k] w.r.t. the router weights of the chosen experts idx.

    The choice itself is piecewise constant in z (no gradient).  With
    renorm=1 the weights are the softmax q of the chosen logits, so the chosen
    logits get J_q^T d_w with the softmax Jacobian J_q = diag(q) - q q^T and
    the others get 0; with renorm=0 they are the full softmax p read at the
    chosen experts, so with g = d_w scattered into an E-vector (0 elsewhere),
    dz = (diag(p) - p p^T) g.  Both written out as matrices, fp64.
    """
    z = np.asarray(z, dtype=np.float64)
    T, E = z.shape
    dz = np.zeros((T, E))
    for t in range(T):
        sel = idx[t].astype(np.int64)
        if renorm:
            ex = np.exp(z[t, sel] - z[t, sel].max())
            q = ex / ex.sum()
            J = np.diag(q) - np.outer(q, q)
            dz[t, sel] = J.T @ d_w[t]
        else:
            ex = np.exp(z[t] - z[t].max())
            p = ex / ex.sum()
            gfull = np.zeros(E)
            gfull[sel] = d_w[t]
            J = np.diag(p) - np.outer(p, p)
            dz[t] = J.T @ gfull
    return dz


def backward_full(inp, renorm: int | None = None, bf16_mode: bool = True, router: bool = True,
                  allow: bool = False):
    """Full-layer backward, loss L = sum_t <dY[t], out[t]>.

    Routing (indices, weights, logits) is recomputed as in the forward.  Row
    r = t*k + j carries token t to its j-th expert with dY_rows[r] = dY[t];
    the expert part is ``_backward_rows`` on these rows, and
        d_topk_w[t, j] = dw[t*k + j]
        dX[t] = sum_j dX_rows[t*k + j]            (j ascending)
    With ``router`` the gradient also flows through the router:
        dz = router_logit_grad(z, idx, d_topk_w)  [T, E]
        dW_router = dz^T x  [E, H],  d_bias = sum_t dz[t]
        dX[t] += dz[t] W_router
    In bf16 mode dX (after both sums) is one bf16 tensor; dz, dW_router and
    d_bias are exact.  With ``allow`` also the decision allowances of
    ``_backward_rows`` (dX_allow: the sum of the token's rows' allowances).
    """
    sh = inp["shape"]
    rn = sh.renorm if renorm is None else renorm
    k = sh.k
    x = bf16.decode(inp["x"])
    wr = bf16.decode(inp["w_router"])
    idx, w, z = _route(x.astype(np.float32), wr.astype(np.float32), inp["bias"], k, rn)
    wg, wu, wd = _weights(inp)
    T, H = x.shape
    g = _backward_rows(np.repeat(x, k, axis=0), idx.reshape(-1), w.reshape(-1).astype(np.float64),
                       np.repeat(bf16.decode(inp["dY"]), k, axis=0), wg, wu, wd, bf16_mode, allow)
    if "dX_rows_allow" in g:
        g["dX_allow"] = g.pop("dX_rows_allow").reshape(T, k, H).sum(axis=1)
    d_topk_w = g["d_row_w"].reshape(T, k)
    dXr = g.pop("dX_rows").reshape(T, k, H)
    dX = np.zeros((T, H))
    for j in range(k):                                   # fixed ascending order
        dX += dXr[:, j]
    out = dict(g, topk_idx=idx, topk_w=w, logits=z, d_topk_w=d_topk_w)
    if router:
        dz = router_logit_grad(z, idx, d_topk_w, rn)
        dX += dz @ wr
        out.update(dz=dz, dW_router=dz.T @ x, d_bias=dz.sum(axis=0))
    out["dX"] = rnd(dX, bf16_mode)
    out["dX_exact"] = dX
    return out


def backward_full_tokens(inp, idx, w, z, tokens, renorm: int):
    """backward_full's per-token results (bf16 mode) for the given tokens
    only, under routing (idx, w, z): dX, d_topk_w and the logit gradient dz.
    Each depends only on the token's own k rows."""
    tokens = np.asarray(tokens)
    k = idx.shape[1]
    wg, wu, wd = _weights(inp)
    x = bf16.decode(inp["x"][tokens])
    wr = bf16.decode(inp["w_router"])
    g = _backward_rows(np.repeat(x, k, axis=0), idx[tokens].reshape(-1), w[tokens].reshape(-1).astype(np.float64),
                       np.repeat(bf16.decode(inp["dY"][tokens]), k, axis=0), wg, wu, wd, True)
    n, H = x.shape
    d_topk_w = g["d_row_w"].reshape(n, k)
    dXr = g["dX_rows"].reshape(n, k, H)
    dX = np.zeros((n, H))
    for j in range(k):                                   # fixed ascending order
        dX += dXr[:, j]
    dz = router_logit_grad(z[tokens], idx[tokens], d_topk_w, renorm)
    dX += dz @ wr
    return {"dX": rnd(dX, True), "dX_exact": dX, "d_topk_w": d_topk_w, "dz": dz}


def backward_full_expert(inp, idx, w, z, e, renorm: int):
    """backward_full's gradients of expert e's weights and router row (bf16
    mode), from the rows routed to e and, for the router row, the tokens
    whose logit gradient at e is nonzero: with renorm=1 those that chose e,
    with renorm=0 every token."""
    k = idx.shape[1]
    T = idx.shape[0]
    wg, wu, wd = _weights(inp)
    rows = np.nonzero(idx.reshape(-1) == e)[0]
    tok = rows // k
    g = _backward_rows(bf16.decode(inp["x"][tok]), np.full(rows.size, e),
                       w.reshape(-1)[rows].astype(np.float64), bf16.decode(inp["dY"][tok]), wg, wu, wd, True)
    toks = np.unique(tok) if renorm else np.arange(T)
    dz_e = backward_full_tokens(inp, idx, w, z, toks, renorm)["dz"][:, e]
    x = bf16.decode(inp["x"][toks])
    return {"dW_gate": g["dW_gate"][e], "dW_up": g["dW_up"][e], "dW_down": g["dW_down"][e],
            "dW_router": dz_e @ x, "d_bias": dz_e.sum()}


def qd(v):
    """MXFP8 quantise-dequantise along the last axis (blocks of 32)."""
    return mxfp8.dequantize(*mxfp8.quantize(v))


# Relative change of a GEMM output that another correct fp32 evaluation (the
# block-scaled MFMA sums in their own order, an fp32 SiLU) may bring; about
# four times what the device shows (near 2^-15).
DECISION_REL = 2.0 ** -13


def qd_spread(v, rel: float = DECISION_REL):
    """How far D(Q(bf16(v'))) may lie from D(Q(bf16(v))), per element, over all
    v' with |v'_i - v_i| <= rel |v_i| (v: exact values of a GEMM output that is
    rounded to bf16 and then MXFP8-quantised along its last axis).  0 where
    no E4M3 code and no block scale can change.

    bf16 rounding and the E4M3 element rule are monotone, so at one block
    scale every reachable code lies between those of the interval's two ends;
    the block scale follows the block's largest magnitude, so it lies between
    the scales of the two ends' blocks (at most one power of two apart).  The
    largest distance over both ends at both scales bounds every reachable
    value.
    """
    v = np.asarray(v, dtype=np.float64)
    ref = qd(bf16.round_rne(v))
    small = bf16.round_rne(v * (1.0 - rel))
    big = bf16.round_rne(v * (1.0 + rel))
    spread = np.zeros_like(v)
    for sc in (mxfp8.block_scale_codes(small), mxfp8.block_scale_codes(big)):
        for end in (small, big):
            d = mxfp8.dequantize(mxfp8.quantize_with_scales(end, sc), sc)
            spread = np.maximum(spread, np.abs(d - ref))
    return spread


def _dact_mxfp8(dYq, wdTq, g, u, w):
    """dA' = D(Q_H(dY)) D(Q_H(W_d^T))^T and the SwiGLU backward from the
    forward's g, u: -> dA', a (exact silu(g) u), dw, dg, du (bf16), and dg,
    du before that rounding."""
    dAp = dYq @ wdTq.T
    a = silu(g) * u
    dw = np.einsum("ri,ri->r", dAp, a)
    dA = w[:, None] * dAp
    s = sigmoid(g)
    dgx = dA * u * s * (1.0 + g * (1.0 - s))
    dux = dA * silu(g)
    return dAp, a, dw, bf16.round_rne(dgx), bf16.round_rne(dux), dgx, dux


def qd_rows(v):
    """MXFP8 quantise-dequantise along the first axis: each column of v is cut
    into blocks of 32 consecutive rows, the last one completed with zero rows
    (which change neither its largest magnitude nor the other codes and are
    dropped again).  The MX format itself is the one the pages name for the
    MXFP8 mode ([CARD] "Core concepts"; [MTP] "Key Takeaways"), with the
    element and scale rule of ``mxfp8``."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    pad = (-n) % 32
    if pad:
        v = np.concatenate([v, np.zeros((pad,) + v.shape[1:])], axis=0)
    return qd(v.T).T[:n]


def qd_spread_rows(v):
    """``qd_spread`` with the blocks of 32 taken down the rows of v (as
    ``qd_rows``; zero pad rows have no spread)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    pad = (-n) % 32
    if pad:
        v = np.concatenate([v, np.zeros((pad,) + v.shape[1:])], axis=0)
    return qd_spread(v.T).T[:n]


def minibatch_of(rows, R: int, mb: int):
    """Minibatch index of arrival rows (mb <= 0 or mb >= R: one minibatch)."""
    rows = np.asarray(rows)
    return np.zeros_like(rows) if mb <= 0 or mb >= R else rows // mb


def wgrad_mx_allow(A_exact, A_fixed, B_exact, B_fixed, mbs):
    """How far ``wgrad_mx`` may move when an operand is a GEMM output rounded
    to bf16 and then quantised: per segment, the spread of each such operand's
    codes (``qd_spread_rows`` of its exact values, A_exact / B_exact; None for
    an operand that is an input) through |the other operand|, both spreads
    added.  A_fixed / B_fixed: the operands as ``wgrad_mx`` takes them."""
    out = np.zeros((A_fixed.shape[1], B_fixed.shape[1]))
    for b in np.unique(mbs):
        k = mbs == b
        qa, qb = np.abs(qd_rows(A_fixed[k])), np.abs(qd_rows(B_fixed[k]))
        if A_exact is not None:
            out += qd_spread_rows(A_exact[k]).T @ qb
        if B_exact is not None:
            out += qa.T @ qd_spread_rows(B_exact[k])
    return out


def wgrad_mx(A, B, mbs):
    """sum over segments s of D(Q_rows(A_s))^T D(Q_rows(B_s)): the MXFP8
    weight-gradient contraction over one expert's rows.  A [n, M] and B [n, N]
    hold the expert's rows in arrival order, mbs their minibatch; a segment is
    the rows of one minibatch, and the MX blocks of 32 rows never cross a
    segment boundary.  The pages report an MXFP8 backward ([MTP] "Results")
    but give no recipe for it; the reading taken here blocks along each
    GEMM's contraction as the forward does, and takes the minibatch ([MTP]
    "Three design decisions that matter": minibatch granularity) as the unit
    a block may not cross, since a minibatch's rows arrive together and a
    block is complete once its minibatch is."""
    out = np.zeros((A.shape[1], B.shape[1]))
    for b in np.unique(mbs):
        k = mbs == b
        out += qd_rows(A[k]).T @ qd_rows(B[k])
    return out


def _backward_rows_mxfp8(x, re, w, dY, G, U, wg, wu, wd, allow: bool = False, wgrad_mx_mb: int | None = None):
    """MXFP8 expert backward of routed rows (arrival order) given the
    forward's g = G and u = U: the rows of ``backward_share_mxfp8`` with
    dX_rows not rounded (see there).  With ``allow`` also dX_rows_allow: how
    far dX_rows may move because [dg | du] is a GEMM output whose E4M3 codes
    another correct evaluation may decide differently (``qd_spread`` through
    |W_P|).  ``wgrad_mx_mb``: None = bf16 weight gradients; else MXFP8 ones
    (``wgrad_mx``) with minibatches of that many rows (0 = one minibatch),
    and with ``allow`` also dW_gate_allow, dW_up_allow, dW_down_allow
    (``wgrad_mx_allow``: dg, du and w a are GEMM outputs)."""
    dYq = qd(dY)
    R, H = x.shape
    E, I, _ = wg.shape
    dX = np.zeros((R, H)); dw = np.zeros(R); dX_allow = np.zeros((R, H))
    dWg = np.zeros((E, I, H)); dWu = np.zeros((E, I, H)); dWd = np.zeros((E, H, I))
    W_allow = {"dW_gate": np.zeros_like(dWg), "dW_up": np.zeros_like(dWu), "dW_down": np.zeros_like(dWd)}
    for e in range(E):
        sel = np.nonzero(re == e)[0]
        if sel.size == 0:
            continue
        g, u = G[sel], U[sel]
        _, a, dw[sel], dg, du, dgx, dux = _dact_mxfp8(dYq[sel], qd(wd[e].T), g, u, w[sel])
        P = np.concatenate([dg, du], axis=1)                        # [n, 2I]: the I gate, then the I up features
        WP = np.concatenate([wg[e], wu[e]], axis=0)                 # [2I, H], the same feature order
        WPq = qd(WP.T)
        dX[sel] = qd(P) @ WPq.T
        if allow:
            dX_allow[sel] = qd_spread(np.concatenate([dgx, dux], axis=1)) @ np.abs(WPq).T
        xe = x[sel]
        wa = bf16.round_rne(w[sel, None] * a)
        if wgrad_mx_mb is None:
            dWg[e] = dg.T @ xe
            dWu[e] = du.T @ xe
            dWd[e] = dY[sel].T @ wa
        else:
            mbs = minibatch_of(sel, R, wgrad_mx_mb)
            dWg[e] = wgrad_mx(dg, xe, mbs)
            dWu[e] = wgrad_mx(du, xe, mbs)
            dWd[e] = wgrad_mx(dY[sel], wa, mbs)
            if allow:
                # dg, du and w a are GEMM outputs whose codes may be decided
                # differently; x and dY are inputs
                W_allow["dW_gate"][e] = wgrad_mx_allow(dgx, dg, None, xe, mbs)
                W_allow["dW_up"][e] = wgrad_mx_allow(dux, du, None, xe, mbs)
                W_allow["dW_down"][e] = wgrad_mx_allow(None, dY[sel], w[sel, None] * a, wa, mbs)
    res = {"dX_rows": dX, "dW_gate": dWg, "dW_up": dWu, "dW_down": dWd, "d_row_w": dw}
    if allow:
        res["dX_rows_allow"] = dX_allow
        if wgrad_mx_mb is not None:
            res.update({k + "_allow": v for k, v in W_allow.items()})
    return res


def backward_share_mxfp8(inp, fwd=None, allow: bool = False, wgrad_mx_mb: int | None = None):
    """Expert share backward in MXFP8 mode, loss L = sum_r <dY[r], out_rows[r]>
    with out_rows from forward_share_mxfp8.

    The two data-gradient GEMMs take MXFP8 operands quantised along their
    contraction, blocks of 32 (the forward's rule carried to the backward):
        dA' = D(Q_H(dY)) . D(Q_H(W_d[e]^T))^T
        dX  = bf16( D(Q(P)) . D(Q(W_P[e]^T))^T ),  P = [dg | du] (the I gate
              features, then the I up features) and W_P = [W_g[e] ; W_u[e]]
              in the same order; since I is a multiple of 32, every MX block
              of 32 along this contraction is 32 consecutive gate features or
              32 consecutive up features, i.e. dg and du are quantised along
              I each on their own, as are W_g[e]^T and W_u[e]^T
    g and u are the MXFP8 forward's (exact products of its dequantised
    operands); a = silu(g) u; dw, dA, dg, du (bf16) as in the bf16 backward.
    With ``wgrad_mx_mb`` None the weight gradients are bf16 GEMMs, as in the
    bf16 backward:
        dW_g[e] = dg_e^T X_e,  dW_u[e] = du_e^T X_e,  dW_d[e] = dY_e^T bf16(w a)_e
    With an integer (the minibatch rows; 0 = one minibatch) they are MXFP8
    GEMMs too, each operand quantised along their contraction, the expert's
    rows, in blocks of 32 rows of one minibatch (``wgrad_mx``):
        dW_g[e] = sum_s D(Q_rows(dg_s))^T D(Q_rows(X_s)), dW_u likewise,
        dW_d[e] = sum_s D(Q_rows(dY_s))^T D(Q_rows(bf16(w a)_s))
    With ``allow`` also dX_allow (see ``_backward_rows_mxfp8``).
    """
    fwd = forward_share_mxfp8(inp) if fwd is None else fwd
    wg, wu, wd = _weights(inp)
    g = _backward_rows_mxfp8(bf16.decode(inp["x"]), inp["row_expert"], inp["row_w"].astype(np.float64),
                             bf16.decode(inp["dY"]), fwd["g"], fwd["u"], wg, wu, wd, allow, wgrad_mx_mb)
    g["dX_exact"] = g.pop("dX_rows")
    g["dX"] = bf16.round_rne(g["dX_exact"])
    if allow:
        g["dX_allow"] = g.pop("dX_rows_allow")
    return g


def _expanded_rows(inp, idx, w):
    """Routed rows r = t*k + j of the full layer as an expert-share input."""
    k = idx.shape[1]
    return {"x": np.repeat(inp["x"], k, axis=0), "w_gate": inp["w_gate"], "w_up": inp["w_up"],
            "w_down": inp["w_down"], "row_expert": idx.reshape(-1), "row_w": w.reshape(-1)}


def forward_full_mxfp8(inp, renorm: int | None = None, allow: bool = False):
    """Full layer in MXFP8 mode: the router of ``forward_full``, the routed
    rows r = t*k + j through the MXFP8 expert arithmetic of
    ``forward_share_mxfp8`` (unweighted y), and the combine of
    ``forward_full`` (sum over j ascending, one bf16 rounding).  With
    ``allow`` also out_allow, the sum of the token's rows' allowances."""
    sh = inp["shape"]
    x = bf16.decode(inp["x"])
    idx, w, z = _route(x.astype(np.float32), bf16.decode(inp["w_router"]).astype(np.float32),
                       inp["bias"], sh.k, sh.renorm if renorm is None else renorm)
    f = forward_share_mxfp8(_expanded_rows(inp, idx, w), allow=allow)
    T, H = x.shape
    out = np.zeros((T, H))
    yk = f["y"].reshape(T, sh.k, H)
    for j in range(sh.k):
        out += w[:, j, None].astype(np.float64) * yk[:, j]
    res = {"topk_idx": idx, "topk_w": w, "logits": z, "g": f["g"], "u": f["u"], "a_bits": f["a_bits"],
           "y": f["y"], "out": bf16.round_rne(out), "out_exact": out}
    if allow:
        res["out_allow"] = f["out_allow"].reshape(T, sh.k, H).sum(axis=1)
    return res


def backward_full_mxfp8(inp, renorm: int | None = None, router: bool = True, fwd=None, allow: bool = False,
                        wgrad_mx_mb: int | None = None):
    """Full-layer backward in MXFP8 mode: ``backward_full`` with the expert
    part of ``backward_share_mxfp8`` (weight gradients per ``wgrad_mx_mb``,
    minibatches over the routed rows r = t k + j) on the routed rows (g, u from
    ``forward_full_mxfp8``); the k-sum, the router gradient and the single
    bf16 rounding of dX as in ``backward_full``.  With ``allow`` also
    dX_allow, the sum of the token's rows' allowances."""
    sh = inp["shape"]
    rn = sh.renorm if renorm is None else renorm
    k = sh.k
    fwd = forward_full_mxfp8(inp, rn) if fwd is None else fwd
    idx, w, z = fwd["topk_idx"], fwd["topk_w"], fwd["logits"]
    x = bf16.decode(inp["x"])
    wr = bf16.decode(inp["w_router"])
    wg, wu, wd = _weights(inp)
    T, H = x.shape
    g = _backward_rows_mxfp8(np.repeat(x, k, axis=0), idx.reshape(-1), w.reshape(-1).astype(np.float64),
                             np.repeat(bf16.decode(inp["dY"]), k, axis=0), fwd["g"], fwd["u"], wg, wu, wd, allow,
                             wgrad_mx_mb)
    if allow:
        g["dX_allow"] = g.pop("dX_rows_allow").reshape(T, k, H).sum(axis=1)
    d_topk_w = g["d_row_w"].reshape(T, k)
    dXr = g.pop("dX_rows").reshape(T, k, H)
    dX = np.zeros((T, H))
    for j in range(k):
        dX += dXr[:, j]
    out = dict(g, topk_idx=idx, topk_w=w, logits=z, d_topk_w=d_topk_w)
    if router:
        dz = router_logit_grad(z, idx, d_topk_w, rn)
        dX += dz @ wr
        out.update(dz=dz, dW_router=dz.T @ x, d_bias=dz.sum(axis=0))
    out["dX"] = bf16.round_rne(dX)
    out["dX_exact"] = dX
    return out


def backward_share_mxfp8_sampled(inp, rows, gate_up_rows, down_cols, wgrad_mx_mb: int | None = None):
    """Entries of backward_share_mxfp8 computed one by one (each needs only
    its own rows, or the rows of one expert), with dX_allow for the rows;
    ``wgrad_mx_mb`` as there."""
    re = inp["row_expert"]
    w = inp["row_w"].astype(np.float64)
    out = {"dX": [], "dX_exact": [], "dX_allow": [], "d_row_w": [], "dW_gate": [], "dW_up": [], "dW_down": [],
           "dW_gate_allow": [], "dW_up_allow": [], "dW_down_allow": []}
    cache = {}

    def expert(e):
        if e not in cache:
            wg = bf16.decode(inp["w_gate"][e]); wu = bf16.decode(inp["w_up"][e]); wd = bf16.decode(inp["w_down"][e])
            q = quantized_weights_expert(inp, e)
            cache[e] = {"gq": mxfp8.dequantize(*q["gate"]), "uq": mxfp8.dequantize(*q["up"]),
                        "wdTq": qd(wd.T), "WPTq": qd(np.concatenate([wg, wu], axis=0).T)}
        return cache[e]

    def fwd_gu(e, sel):
        c = expert(e)
        xd = qd(bf16.decode(inp["x"][sel]))
        return xd @ c["gq"].T, xd @ c["uq"].T

    for r in rows:
        e = int(re[r])
        c = expert(e)
        g, u = fwd_gu(e, [r])
        _, _, dw, dg, du, dgx, dux = _dact_mxfp8(qd(bf16.decode(inp["dY"][r:r + 1])), c["wdTq"], g, u, w[[r]])
        P = np.concatenate([dg, du], axis=1)
        dx = (qd(P) @ c["WPTq"].T)[0]
        out["dX"].append(bf16.round_rne(dx))
        out["dX_exact"].append(dx)
        out["dX_allow"].append((qd_spread(np.concatenate([dgx, dux], axis=1)) @ np.abs(c["WPTq"]).T)[0])
        out["d_row_w"].append(float(dw[0]))
    rows_q = {}

    def expert_rows(e):
        # the rows of expert e: x and dY (bf16) and their MXFP8 forms
        if e not in rows_q:
            sel = np.nonzero(re == e)[0]
            X = bf16.decode(inp["x"][sel]); dY = bf16.decode(inp["dY"][sel])
            rows_q[e] = [sel, X, dY, qd(X), qd(dY)]
            if wgrad_mx_mb is not None:
                # weight-gradient operands quantised along the rows, per segment
                mbs = minibatch_of(sel, re.size, wgrad_mx_mb)
                xs = np.zeros_like(X); ds = np.zeros_like(dY)
                for b in np.unique(mbs):
                    kk = mbs == b
                    xs[kk] = qd_rows(X[kk]); ds[kk] = qd_rows(dY[kk])
                rows_q[e] += [mbs, xs, ds]
        return rows_q[e]

    def seg_q(v, mbs, f=qd_rows):
        # one column, quantised along the rows per segment (f = qd_spread_rows:
        # the spread of its codes)
        out = np.zeros_like(v)
        for b in np.unique(mbs):
            kk = mbs == b
            out[kk] = f(v[kk, None])[:, 0]
        return out

    for key, pairs in (("gate_up", gate_up_rows), ("down", down_cols)):
        for (e, i) in pairs:
            # feature i only: one column of g, u and dA' (as _dact_mxfp8 computes
            # them); the weights are quantised per row along H, so the rows
            # for feature i are quantised alone
            sel, X, dY, xd, dyq = expert_rows(e)[:5]
            g = xd @ qd(bf16.decode(inp["w_gate"][e, i]))
            u = xd @ qd(bf16.decode(inp["w_up"][e, i]))
            dAp = dyq @ qd(bf16.decode(inp["w_down"][e][:, i]))
            s = sigmoid(g)
            dA = w[sel] * dAp
            dgx, dux, wax = dA * u * s * (1.0 + g * (1.0 - s)), dA * silu(g), w[sel] * silu(g) * u
            dg, du, wa = bf16.round_rne(dgx), bf16.round_rne(dux), bf16.round_rne(wax)
            if wgrad_mx_mb is None:
                if key == "gate_up":
                    out["dW_gate"].append(dg @ X)
                    out["dW_up"].append(du @ X)
                else:
                    out["dW_down"].append(wa @ dY)
            else:
                mbs, xs, ds = expert_rows(e)[5:]
                if key == "gate_up":
                    out["dW_gate"].append(seg_q(dg, mbs) @ xs)
                    out["dW_up"].append(seg_q(du, mbs) @ xs)
                    out["dW_gate_allow"].append(seg_q(dgx, mbs, qd_spread_rows) @ np.abs(xs))
                    out["dW_up_allow"].append(seg_q(dux, mbs, qd_spread_rows) @ np.abs(xs))
                else:
                    out["dW_down"].append(seg_q(wa, mbs) @ ds)
                    out["dW_down_allow"].append(seg_q(wax, mbs, qd_spread_rows) @ np.abs(ds))
    return {k: np.asarray(v) for k, v in out.items()}


def forward_share_rows(inp, rows, exact: bool = False):
    """forward_share's out for the given arrival rows only (each row is
    independent of every other); with ``exact`` the value before its bf16
    rounding (forward_share's out_exact)."""
    rows = np.asarray(rows)
    re = inp["row_expert"]
    out = np.zeros((len(rows), inp["x"].shape[1]))
    for e in np.unique(re[rows]):
        e = int(e)
        sel = np.nonzero(re[rows] == e)[0]
        x = bf16.decode(inp["x"][rows[sel]])
        _, _, _, y = expert_ffn(x, bf16.decode(inp["w_gate"][e]), bf16.decode(inp["w_up"][e]),
                                bf16.decode(inp["w_down"][e]), bf16_mode=True)
        out[sel] = inp["row_w"][rows[sel], None].astype(np.float64) * y
    return out if exact else bf16.round_rne(out)


def forward_full_tokens(inp, idx, w, tokens, exact: bool = False):
    """Full-layer out for the given tokens under routing (idx, w); with
    ``exact`` the value before its bf16 rounding."""
    tokens = np.asarray(tokens)
    x = bf16.decode(inp["x"][tokens])
    out = np.zeros((len(tokens), x.shape[1]))
    sub = idx[tokens]
    ys = {}
    for e in np.unique(sub):
        e = int(e)
        _, _, _, ys[e] = expert_ffn(x, bf16.decode(inp["w_gate"][e]), bf16.decode(inp["w_up"][e]),
                                    bf16.decode(inp["w_down"][e]), bf16_mode=True)
    for n, t in enumerate(tokens):
        for j in range(idx.shape[1]):                    # fixed ascending order
            out[n] += float(w[t, j]) * ys[int(idx[t, j])][n]
    return out if exact else bf16.round_rne(out)


def quantized_weights_expert(inp, e):
    """MXFP8 codes/scales of one expert's weights (gate/up along H, down along I)."""
    return {"gate": mxfp8.quantize(bf16.decode(inp["w_gate"][e])),
            "up": mxfp8.quantize(bf16.decode(inp["w_up"][e])),
            "down": mxfp8.quantize(bf16.decode(inp["w_down"][e]))}


def forward_share_mxfp8_rows(inp, rows, allow: bool = False, exact: bool = False):
    """forward_share_mxfp8's out for the given arrival rows only (with
    ``exact`` the value before its bf16 rounding); with ``allow`` the pair
    (out, out_allow)."""
    rows = np.asarray(rows)
    re = inp["row_expert"]
    H = inp["x"].shape[1]
    out = np.zeros((len(rows), H)); out_allow = np.zeros((len(rows), H))
    for e in np.unique(re[rows]):
        q = quantized_weights_expert(inp, int(e))
        wg = mxfp8.dequantize(*q["gate"]); wu = mxfp8.dequantize(*q["up"]); wd = mxfp8.dequantize(*q["down"])
        sel = np.nonzero(re[rows] == e)[0]
        xc, xs = mxfp8.quantize(bf16.decode(inp["x"][rows[sel]]))
        xd = mxfp8.dequantize(xc, xs)
        g = xd @ wg.T
        u = xd @ wu.T
        a = bf16.decode(bf16.encode(silu(g) * u))
        ad = mxfp8.dequantize(*mxfp8.quantize(a))
        wr = inp["row_w"][rows[sel], None].astype(np.float64)
        out[sel] = wr * (ad @ wd.T)
        if allow:
            out_allow[sel] = np.abs(wr) * (qd_spread(silu(g) * u) @ np.abs(wd).T)
    res = out if exact else bf16.round_rne(out)
    return (res, out_allow) if allow else res


def backward_share_sampled(inp, rows, gate_up_rows, down_cols):
    """Entries of backward_share (bf16 mode) computed one by one.

    rows          arrival rows r -> dX[r], d_row_w[r]
    gate_up_rows  (e, i) pairs   -> dW_gate[e, i, :], dW_up[e, i, :]
    down_cols     (e, i) pairs   -> dW_down[e, :, i]
    """
    re = inp["row_expert"]
    w = inp["row_w"].astype(np.float64)
    out = {"dX": [], "dX_exact": [], "d_row_w": [], "dW_gate": [], "dW_up": [], "dW_down": []}
    for r in rows:
        e = int(re[r])
        x = bf16.decode(inp["x"][r:r + 1]); dY = bf16.decode(inp["dY"][r:r + 1])
        wg = bf16.decode(inp["w_gate"][e]); wu = bf16.decode(inp["w_up"][e]); wd = bf16.decode(inp["w_down"][e])
        g, u, a, y = expert_ffn(x, wg, wu, wd)
        dAp = dY @ wd
        s = sigmoid(g)
        dA = w[r] * dAp
        dg = bf16.round_rne(dA * u * s * (1.0 + g * (1.0 - s)))
        du = bf16.round_rne(dA * silu(g))
        dx = (dg @ wg + du @ wu)[0]
        out["dX"].append(bf16.round_rne(dx))
        out["dX_exact"].append(dx)
        out["d_row_w"].append(float(np.sum(dAp * a)))
    for (e, i) in gate_up_rows:
        sel = np.nonzero(re == e)[0]
        X = bf16.decode(inp["x"][sel]); dY = bf16.decode(inp["dY"][sel])
        g = X @ bf16.decode(inp["w_gate"][e, i]); u = X @ bf16.decode(inp["w_up"][e, i])
        dAp = dY @ bf16.decode(inp["w_down"][e][:, i])
        s = sigmoid(g)
        dA = w[sel] * dAp
        out["dW_gate"].append(bf16.round_rne(dA * u * s * (1.0 + g * (1.0 - s))) @ X)
        out["dW_up"].append(bf16.round_rne(dA * silu(g)) @ X)
    for (e, i) in down_cols:
        sel = np.nonzero(re == e)[0]
        X = bf16.decode(inp["x"][sel]); dY = bf16.decode(inp["dY"][sel])
        a = silu(X @ bf16.decode(inp["w_gate"][e, i])) * (X @ bf16.decode(inp["w_up"][e, i]))
        out["dW_down"].append(bf16.round_rne(w[sel] * a) @ dY)
    return {k: np.asarray(v) for k, v in out.items()}


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


# ---------------------------------------------------------------------------
# Single GEMM steps fed given operands.  Each is the definition of one step of
# the layer written out on its own, so that a result computed from another
# implementation's intermediate tensor (the bf16 a, dg/du, w a, or their
# MXFP8 codes) can be checked step by step, without the roundings and E4M3
# decisions that the earlier steps take on GEMM outputs.
# ---------------------------------------------------------------------------

def swiglu_rows(x_rows, row_expert, wg, wu):
    """g, u and the exact a = silu(g) u of each row under its expert (fp64;
    zeros for an expert id out of range)."""
    g, u, _, _ = rows_ffn(x_rows, row_expert, wg, wu, np.zeros((wg.shape[0], 1, wg.shape[1])))
    return g, u, silu(g) * u


def down_rows(a_rows, row_expert, wd):
    """y[r] = a[r] W_d[e]^T for given GEMM2 operands a (arrival order)."""
    y = np.zeros((a_rows.shape[0], wd.shape[1]))
    for e in range(wd.shape[0]):
        sel = np.nonzero(row_expert == e)[0]
        if sel.size:
            y[sel] = a_rows[sel] @ wd[e].T
    return y


def combine_tokens(y_rows, w, k):
    """out[t] = sum over j ascending of w[t, j] y[t k + j] (exact)."""
    T = y_rows.shape[0] // k
    yk = y_rows.reshape(T, k, -1)
    out = np.zeros((T, yk.shape[2]))
    for j in range(k):
        out += np.asarray(w, dtype=np.float64).reshape(T, k)[:, j, None] * yk[:, j]
    return out


def dact_rows(dY_rows, g, u, row_expert, wd, w, dYq=None, wdT=None):
    """dA' = dY W_d[e] (or, MXFP8, dYq wdT[e]^T with the given dequantised
    operands) and the exact SwiGLU backward from g, u: -> dict of dA', dw,
    dg and du before their bf16 rounding, and w a."""
    R = dY_rows.shape[0]
    I = g.shape[1]
    dAp = np.zeros((R, I))
    for e in range(wd.shape[0]):
        sel = np.nonzero(row_expert == e)[0]
        if sel.size:
            dAp[sel] = dY_rows[sel] @ wd[e] if dYq is None else dYq[sel] @ wdT[e].T
    s = sigmoid(g)
    w = np.asarray(w, dtype=np.float64)
    dA = w[:, None] * dAp
    return {"dAp": dAp, "dw": np.einsum("ri,ri->r", dAp, silu(g) * u),
            "dg": dA * u * s * (1.0 + g * (1.0 - s)), "du": dA * silu(g), "wa": w[:, None] * silu(g) * u}


def dx_rows_from(dg, du, row_expert, wg, wu):
    """dX_rows[r] = dg[r] W_g[e] + du[r] W_u[e] for given operands (exact)."""
    dX = np.zeros((dg.shape[0], wg.shape[2]))
    for e in range(wg.shape[0]):
        sel = np.nonzero(row_expert == e)[0]
        if sel.size:
            dX[sel] = dg[sel] @ wg[e] + du[sel] @ wu[e]
    return dX


def dx_rows_from_mx(p_codes, p_scales, row_expert, wg, wu):
    """MXFP8 dX rows from given codes of P = [dg | du] (quantised along the
    2I features, the I gate ones then the I up ones): D(P) D(Q([W_g; W_u]^T))^T."""
    P = mxfp8.dequantize(p_codes, p_scales)
    dX = np.zeros((P.shape[0], wg.shape[2]))
    for e in range(wg.shape[0]):
        sel = np.nonzero(row_expert == e)[0]
        if sel.size:
            dX[sel] = P[sel] @ qd(np.concatenate([wg[e], wu[e]], axis=0).T).T
    return dX


def wgrads_from(x_rows, dY_rows, dg, du, wa, row_expert, E):
    """bf16-mode weight gradients from given GEMM operands (exact sums):
    dW_g[e] = dg_e^T X_e, dW_u[e] = du_e^T X_e, dW_d[e] = dY_e^T (w a)_e."""
    I, H = dg.shape[1], x_rows.shape[1]
    dWg = np.zeros((E, I, H)); dWu = np.zeros((E, I, H)); dWd = np.zeros((E, H, I))
    for e in range(E):
        sel = np.nonzero(row_expert == e)[0]
        if sel.size:
            dWg[e] = dg[sel].T @ x_rows[sel]
            dWu[e] = du[sel].T @ x_rows[sel]
            dWd[e] = dY_rows[sel].T @ wa[sel]
    return {"dW_gate": dWg, "dW_up": dWu, "dW_down": dWd}


def wgrads_from_mx(x_rows, dY_rows, dg, du, wa, row_expert, E, mb: int):
    """MXFP8 weight gradients (``wgrad_mx``, minibatches of mb rows, 0 = one)
    from given bf16 operands."""
    I, H = dg.shape[1], x_rows.shape[1]
    R = x_rows.shape[0]
    dWg = np.zeros((E, I, H)); dWu = np.zeros((E, I, H)); dWd = np.zeros((E, H, I))
    for e in range(E):
        sel = np.nonzero(row_expert == e)[0]
        if sel.size:
            mbs = minibatch_of(sel, R, mb)
            dWg[e] = wgrad_mx(dg[sel], x_rows[sel], mbs)
            dWu[e] = wgrad_mx(du[sel], x_rows[sel], mbs)
            dWd[e] = wgrad_mx(dY_rows[sel], wa[sel], mbs)
    return {"dW_gate": dWg, "dW_up": dWu, "dW_down": dWd}
