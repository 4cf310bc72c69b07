"""GPU parity at the limits and in the degenerate cases of the layer: the
largest expert count and top-k the workspace takes, one expert (the layer is
then a dense SwiGLU MLP and the router carries no gradient), every expert
chosen (k = E), and MXFP8 weight gradients over many tiny minibatch segments."""
import dataclasses

import numpy as np
import pytest

import workloads
from helpers import BF16_TOL, ROUTER_W_ATOL, assert_close, dev, host_bf16, say
from oracle import bf16, layer, route, schedule

pytestmark = pytest.mark.gpu

from mixture_experts_layer_device_amd import binding as B  # noqa: E402
from mixture_experts_layer_device_amd.layer import MoELayer  # noqa: E402

MAX_E, MAX_K = 1024, 32


@pytest.mark.parametrize("renorm", [0, 1])
def test_route_at_max_experts_and_topk(renorm):
    T, H = 64, 256
    say(f"[limits] route T={T} H={H} E={MAX_E} k={MAX_K} renorm={renorm}, biased")
    rng = np.random.default_rng(31 + renorm)
    x = bf16.encode(rng.standard_normal((T, H)))
    wr = bf16.encode(rng.standard_normal((MAX_E, H)) / 16.0)
    bias = (rng.standard_normal(MAX_E) * np.sqrt(0.5)).astype(np.float32)
    idx_ref, w_ref, _ = route.route(bf16.decode(x).astype(np.float32), bf16.decode(wr).astype(np.float32), bias,
                                    MAX_K, renorm)
    L = MoELayer(H=H, I=128, E=MAX_E, k=MAX_K, max_rows=T * MAX_K, renorm=renorm)
    idx, w = L.route(dev(x), dev(wr), dev(bias), T)
    idx = idx.cpu().numpy()
    assert np.array_equal(idx, idx_ref)
    assert all(len(set(row)) == MAX_K for row in idx.tolist())
    err = float(np.max(np.abs(w.cpu().numpy().astype(np.float64) - w_ref)))
    say(f"  router weights max|err| = {err:.2e}")
    assert err <= ROUTER_W_ATOL
    L.close()


def test_schedule_at_max_experts():
    R, MB = 8192, 2048
    say(f"[limits] schedule R={R} E={MAX_E} MB={MB}")
    rng = np.random.default_rng(33)
    re = rng.choice(MAX_E, size=R, p=workloads.zipf_local_weights(MAX_E, 1.2)).astype(np.int32)
    L = MoELayer(H=256, I=128, E=MAX_E, k=1, max_rows=R, minibatch_rows=MB, ring_bytes=2 * MB * 512)
    L.build_schedule(dev(re), R)
    ref = schedule.build(re, MAX_E, MB, L.query("ring_rows"), L.query("tile_m"))
    nb = R // MB
    for name, n, want in (("counts", MAX_E, ref.counts), ("offsets", MAX_E + 1, ref.offsets),
                          ("sorted_pos", R, ref.sorted_pos), ("inv", nb * MB, ref.inv),
                          ("mb_offsets", nb * (MAX_E + 1), ref.mb_offsets)):
        assert np.array_equal(L.table(name, n).cpu().numpy(), np.asarray(want).reshape(-1)), name
    assert L.device_error() == 0
    L.close()


def _full_layer(sh, precision="bf16"):
    inp = workloads.make_full_layer(sh)
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, enable_backward=True,
                 precision=precision)
    x, wr = dev(inp["x"]), dev(inp["w_router"])
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
    idx, w = L.route(x, wr, bias, sh.T)
    L.build_schedule(idx.view(-1), sh.R)
    ctx = L.new_fwd_ctx()
    out = L.forward(B.MK_FULL_LAYER, x, w.view(-1), packed, sh.T, fwd_ctx=ctx)
    g = L.backward_layer(ctx, x, wr, bias, idx, w, packed, dev(inp["dY"]), sh.T)
    return inp, L, idx, w, out, g


@pytest.mark.parametrize("renorm", [0, 1])
def test_single_expert_is_a_dense_swiglu_mlp(renorm):
    """E = 1, k = 1: every token goes to expert 0 with weight exactly 1, so
    the output is the dense SwiGLU MLP, and the softmax Jacobian of one logit
    is zero: dW_router and d_bias are exactly 0."""
    sh = dataclasses.replace(workloads.FULL_LAYER["tiny"], E=1, k=1, I=256, renorm=renorm, bias_var=0.5, seed=35)
    say(f"[limits] single expert T={sh.T} H={sh.H} I={sh.I} renorm={renorm}")
    inp, L, idx, w, out, g = _full_layer(sh)
    assert not np.any(idx.cpu().numpy())
    assert np.all(w.cpu().numpy() == 1.0)
    # the dense MLP written out: a rounded to bf16 (a GEMM operand), y exact, out rounded once
    x = bf16.decode(inp["x"])
    wg, wu, wd = (bf16.decode(inp[n])[0] for n in ("w_gate", "w_up", "w_down"))
    gg, uu = x @ wg.T, x @ wu.T
    a = bf16.round_rne(gg / (1.0 + np.exp(-gg)) * uu)
    assert_close(host_bf16(out), a @ wd.T, BF16_TOL, "out vs dense SwiGLU MLP", bf16_out=True)
    ref = layer.backward_full(inp, allow=True)
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], BF16_TOL, "dX", bf16_out=True, allow=ref["dX_allow"])
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert_close(g[k].cpu().numpy(), ref[k], BF16_TOL, k)
    assert not np.any(g["dW_router"].cpu().numpy()) and not np.any(g["d_bias"].cpu().numpy())
    assert L.device_error() == 0
    L.close()


def test_every_expert_chosen():
    """k = E: each token's rows go to all experts, in descending logit order."""
    sh = dataclasses.replace(workloads.FULL_LAYER["tiny"], k=8, I=256, renorm=1, bias_var=0.5, seed=37)
    say(f"[limits] k = E = {sh.E}, T={sh.T} H={sh.H} I={sh.I}")
    inp, L, idx, w, out, g = _full_layer(sh)
    idx = idx.cpu().numpy()
    assert all(sorted(row) == list(range(sh.E)) for row in idx.tolist())
    fwd = layer.forward_full(inp)
    assert np.array_equal(idx, fwd["topk_idx"])
    assert_close(host_bf16(out), fwd["out_exact"], BF16_TOL, "out", bf16_out=True)
    ref = layer.backward_full(inp, allow=True)
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], BF16_TOL, "dX", bf16_out=True, allow=ref["dX_allow"])
    for k in ("dW_gate", "dW_up", "dW_down", "dW_router", "d_bias"):
        assert_close(g[k].cpu().numpy(), ref[k], BF16_TOL, k, allow=ref.get(k + "_allow"))
    assert L.device_error() == 0
    L.close()


def test_mxfp8_weight_gradients_many_experts_and_minibatches():
    """E = 64 experts over 32 minibatches of 128 rows: most (minibatch, expert)
    segments hold a handful of rows or none, so nearly every MX block of the
    weight gradients is a padded segment tail."""
    sh = workloads.ExpertShareShape("wide", R=4096, H=256, I=256, E=64, sources=8, zipf_s=1.2, seed=41)
    inp = workloads.make_expert_share(sh)
    MB = 128
    say(f"[limits] MXFP8 weight gradients R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB} ({sh.R // MB} minibatches)")
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=8, max_rows=sh.R, precision="mxfp8", minibatch_rows=MB,
                 ring_bytes=4 * MB * (sh.H + sh.H // 32), enable_backward=True, wgrad_mxfp8=True)
    x, row_w = dev(inp["x"]), dev(inp["row_w"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
    L.build_schedule(dev(inp["row_expert"]), sh.R)
    ctx = L.new_fwd_ctx()
    L.forward(B.MK_EXPERT_SHARE, x, row_w, packed, sh.R, fwd_ctx=ctx)
    g = L.backward(ctx, x, row_w, packed, dev(inp["dY"]), sh.R)
    fwd = layer.forward_share_mxfp8(inp, allow=True)
    ref = layer.backward_share_mxfp8(inp, fwd, allow=True, wgrad_mx_mb=MB)
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert_close(g[k].cpu().numpy(), ref[k], 6e-2, k, allow=ref[k + "_allow"])
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], 6e-2, "dX", bf16_out=True, allow=ref["dX_allow"])
    assert L.device_error() == 0
    L.close()


def test_route_order_decides_the_top_k():
    """The hand-worked golden case whose top-2 depends on the logits'
    summation order (tests/test_oracle_route_schedule.py
    ascending_order_case): the device's ascending-h fp32 chains give z0 = 0
    exactly and rank expert 1 first, as the oracle does; any other order
    ranks expert 0 first."""
    from tests.test_oracle_route_schedule import ascending_order_case
    T, H, E, k = 48, 256, 8, 2
    say(f"[limits] route, summation-order golden case T={T} H={H} E={E} k={k}")
    xb, wb = ascending_order_case(T=T, H=H, E=E)
    L = MoELayer(H=H, I=128, E=E, k=k, max_rows=T * k, renorm=1)
    idx, w = L.route(dev(xb), dev(wb), None, T)
    got = idx.cpu().numpy()
    L.close()
    assert got.tolist() == [[1, 0]] * T
