"""GPU parity over seeded random configurations: forward and backward of the
expert share and of the full layer (router included), in bf16 and MXFP8, with
random H, I, expert count, top-k, row and token counts, minibatch sizes that
cut across tiles and experts, and rings of one, a few or many minibatches;
and for the bf16 cases the fused forward against the phase-by-phase one,
bit for bit.  The configurations are drawn once from fixed seeds, so every
run checks the same cases; each case's id names its configuration."""
import dataclasses

import numpy as np
import torch
import pytest

import workloads
from helpers import BF16_TOL, MXFP8_TOL, assert_close, dev, host_bf16, say
from oracle import layer

pytestmark = pytest.mark.gpu

from mixture_experts_layer_device_amd import binding as B  # noqa: E402
from mixture_experts_layer_device_amd.layer import MoELayer  # noqa: E402


def _draw_share(rng):
    H = int(rng.choice([256, 512, 768]))
    I = int(rng.choice([256, 512]))
    E = int(rng.choice([1, 2, 3, 5, 8, 13]))
    R = int(rng.integers(1, 1400))
    prec = str(rng.choice(["bf16", "mxfp8"]))
    mxw = prec == "mxfp8" and bool(rng.integers(0, 2))
    MB = int(rng.choice([0, 64, 100, 256, 512]))
    ring_mbs = int(rng.choice([1, 2, 3, 64]))
    seed = int(rng.integers(0, 1 << 30))
    return dict(R=R, H=H, I=I, E=E, prec=prec, mxw=mxw, MB=MB, ring_mbs=ring_mbs if MB else 0, seed=seed)


def _draw_full(rng):
    T = int(rng.integers(1, 300))
    H = int(rng.choice([256, 512]))
    I = int(rng.choice([256, 512]))
    E = int(rng.choice([1, 2, 4, 7, 8, 16]))
    k = int(rng.integers(1, min(E, 8) + 1))
    renorm = int(rng.integers(0, 2))
    bias_var = float(rng.choice([0.0, 0.5]))
    prec = str(rng.choice(["bf16", "mxfp8"]))
    mxw = prec == "mxfp8" and bool(rng.integers(0, 2))
    MB = int(rng.choice([0, 16, 50, 128])) * k
    ring_mbs = int(rng.choice([1, 2, 64]))
    seed = int(rng.integers(0, 1 << 30))
    return dict(T=T, H=H, I=I, E=E, k=k, renorm=renorm, bias_var=bias_var, prec=prec, mxw=mxw, MB=MB,
                ring_mbs=ring_mbs if MB else 0, seed=seed)


def _cases(draw, seed, n):
    rng = np.random.default_rng(seed)
    return [draw(rng) for _ in range(n)]


def _id(c):
    return "-".join(f"{k}{v}" for k, v in c.items() if k != "seed")


SHARE_CASES = _cases(_draw_share, 2, 12)
FULL_CASES = _cases(_draw_full, 11, 10)


def _ring(c, row_bytes):
    return c["ring_mbs"] * c["MB"] * row_bytes if c["MB"] else 256 << 20


def _mb_eff(MB, R):
    """Rows per minibatch as the layer cuts them (0 or above R: one minibatch)."""
    return R if MB == 0 or MB >= R else MB


@pytest.mark.parametrize("c", SHARE_CASES, ids=[_id(c) for c in SHARE_CASES])
def test_random_expert_share(c):
    R, H, I, E, prec, mxw, MB = c["R"], c["H"], c["I"], c["E"], c["prec"], c["mxw"], c["MB"]
    say(f"[random share] {c}")
    sh = workloads.ExpertShareShape("random", R=R, H=H, I=I, E=E, sources=max(1, min(8, R)), zipf_s=1.2,
                                    seed=c["seed"])
    inp = workloads.make_expert_share(sh)
    row_bytes = H + H // 32 if prec == "mxfp8" else 2 * H
    L = MoELayer(H=H, I=I, E=E, k=8, max_rows=R, precision=prec, minibatch_rows=MB, ring_bytes=_ring(c, row_bytes),
                 enable_backward=True, wgrad_mxfp8=mxw)
    x, row_w = dev(inp["x"]), dev(inp["row_w"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
    L.build_schedule(dev(inp["row_expert"]), R)
    ctx = L.new_fwd_ctx()
    out = L.forward(B.MK_EXPERT_SHARE, x, row_w, packed, R, fwd_ctx=ctx)
    g = L.backward(ctx, x, row_w, packed, dev(inp["dY"]), R)
    if prec == "bf16":
        fo = layer.forward_share(inp)
        ref = layer.backward_share(inp, allow=True)
        tol, out_allow = BF16_TOL, None
    else:
        fo = layer.forward_share_mxfp8(inp, allow=True)
        ref = layer.backward_share_mxfp8(inp, fo, allow=True, wgrad_mx_mb=_mb_eff(MB, R) if mxw else None)
        tol, out_allow = MXFP8_TOL, fo["out_allow"]
    assert_close(host_bf16(out), fo["out_exact"], tol, "out", bf16_out=True, allow=out_allow)
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], tol, "dX", bf16_out=True, allow=ref["dX_allow"])
    assert_close(g["d_row_w"].cpu().numpy(), ref["d_row_w"], tol, "d_row_w")
    for key in ("dW_gate", "dW_up", "dW_down"):
        assert_close(g[key].cpu().numpy(), ref[key], tol, key, allow=ref.get(key + "_allow"))
    assert L.device_error() == 0
    L.close()


@pytest.mark.parametrize("c", FULL_CASES, ids=[_id(c) for c in FULL_CASES])
def test_random_full_layer(c):
    T, H, I, E, k, prec, mxw, MB = c["T"], c["H"], c["I"], c["E"], c["k"], c["prec"], c["mxw"], c["MB"]
    R = T * k
    say(f"[random full layer] {c}")
    sh = dataclasses.replace(workloads.FULL_LAYER["tiny"], T=T, H=H, I=I, E=E, k=k, renorm=c["renorm"],
                             bias_var=c["bias_var"], seed=c["seed"])
    inp = workloads.make_full_layer(sh)
    row_bytes = H + H // 32 if prec == "mxfp8" else 2 * H
    L = MoELayer(H=H, I=I, E=E, k=k, max_rows=R, renorm=c["renorm"], minibatch_rows=MB,
                 ring_bytes=_ring(c, row_bytes), enable_backward=True, precision=prec, wgrad_mxfp8=mxw)
    x, wr = dev(inp["x"]), dev(inp["w_router"])
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
    idx, w = L.route(x, wr, bias, T)
    L.build_schedule(idx.view(-1), R)
    ctx = L.new_fwd_ctx()
    out = L.forward(B.MK_FULL_LAYER, x, w.view(-1), packed, T, fwd_ctx=ctx)
    g = L.backward_layer(ctx, x, wr, bias, idx, w, packed, dev(inp["dY"]), T)
    if prec == "bf16":
        fo = layer.forward_full(inp)
        ref = layer.backward_full(inp, allow=True)
        tol, out_allow = BF16_TOL, None
    else:
        fo = layer.forward_full_mxfp8(inp, allow=True)
        ref = layer.backward_full_mxfp8(inp, fwd=fo, allow=True, wgrad_mx_mb=_mb_eff(MB, R) if mxw else None)
        tol, out_allow = MXFP8_TOL, fo["out_allow"]
    assert np.array_equal(idx.cpu().numpy(), ref["topk_idx"])
    assert_close(host_bf16(out), fo["out_exact"], tol, "out", bf16_out=True, allow=out_allow)
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], tol, "dX", bf16_out=True, allow=ref["dX_allow"])
    for key in ("dW_gate", "dW_up", "dW_down"):
        assert_close(g[key].cpu().numpy(), ref[key], tol, key, allow=ref.get(key + "_allow"))
    assert_close(g["d_row_w"].cpu().numpy(), ref["d_topk_w"].reshape(-1), tol, "d_topk_w")
    assert_close(g["dW_router"].cpu().numpy(), ref["dW_router"], tol, "dW_router")
    if bias is not None:
        assert_close(g["d_bias"].cpu().numpy(), ref["d_bias"], tol, "d_bias")
    assert L.device_error() == 0
    L.close()


def _fused_run(c, full, fused):
    """Forward (with its context) and backward of a case, with or without
    the fused forward; every output cloned."""
    if full:
        T, H, I, E, k, MB = c["T"], c["H"], c["I"], c["E"], c["k"], c["MB"]
        R = T * k
        sh = dataclasses.replace(workloads.FULL_LAYER["tiny"], T=T, H=H, I=I, E=E, k=k, renorm=c["renorm"],
                                 bias_var=c["bias_var"], seed=c["seed"])
        inp = workloads.make_full_layer(sh)
        L = MoELayer(H=H, I=I, E=E, k=k, max_rows=R, renorm=c["renorm"], minibatch_rows=MB,
                     ring_bytes=_ring(c, 2 * H), enable_backward=True, fused_forward=fused)
        x, wr = dev(inp["x"]), dev(inp["w_router"])
        bias = dev(inp["bias"]) if inp["bias"] is not None else None
        packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
        idx, w = L.route(x, wr, bias, T)
        L.build_schedule(idx.view(-1), R)
        ctx = L.new_fwd_ctx().zero_()      # (positions past the rows are not written)
        out = L.forward(B.MK_FULL_LAYER, x, w.view(-1), packed, T, fwd_ctx=ctx)
        g = L.backward_layer(ctx, x, wr, bias, idx, w, packed, dev(inp["dY"]), T)
    else:
        R, H, I, E, MB = c["R"], c["H"], c["I"], c["E"], c["MB"]
        sh = workloads.ExpertShareShape("random", R=R, H=H, I=I, E=E, sources=max(1, min(8, R)), zipf_s=1.2,
                                        seed=c["seed"])
        inp = workloads.make_expert_share(sh)
        L = MoELayer(H=H, I=I, E=E, k=8, max_rows=R, minibatch_rows=MB, ring_bytes=_ring(c, 2 * H),
                     enable_backward=True, fused_forward=fused)
        x, row_w = dev(inp["x"]), dev(inp["row_w"])
        packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
        L.build_schedule(dev(inp["row_expert"]), R)
        ctx = L.new_fwd_ctx().zero_()
        out = L.forward(B.MK_EXPERT_SHARE, x, row_w, packed, R, fwd_ctx=ctx)
        g = L.backward(ctx, x, row_w, packed, dev(inp["dY"]), R)
    assert L.device_error() == 0
    res = {"out": out.clone(), "ctx": ctx.clone()}
    res.update({key: v.clone() for key, v in g.items() if v is not None})
    L.close()
    return res


FUSED_CASES = [(c, False) for c in SHARE_CASES if c["prec"] == "bf16"] + \
              [(c, True) for c in FULL_CASES if c["prec"] == "bf16"]


@pytest.mark.parametrize("c,full", FUSED_CASES, ids=[("full-" if f else "share-") + _id(c) for c, f in FUSED_CASES])
def test_random_fused_forward_equals_phase_by_phase(c, full):
    """The fused forward (one persistent launch; in the full layer GEMM1
    gathers the token rows itself and leaves the ring alone) gives the
    phase-by-phase forward's output and context bit for bit, and the
    backward after it every gradient bit for bit (the expert share falls
    back to the phase-by-phase launches when the ring cannot hold every
    minibatch)."""
    say(f"[random fused] {'full layer' if full else 'expert share'} {c}")
    a = _fused_run(c, full, True)
    b = _fused_run(c, full, False)
    assert a.keys() == b.keys()
    for key in a:
        assert torch.equal(a[key], b[key]), key
