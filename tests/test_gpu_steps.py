"""GPU parity step by step: each GEMM of the device path checked against the
oracle fed the device's OWN operands of that GEMM.

The end-to-end parity tests compare the layer with the oracle's independent
evaluation, where a GEMM output that is rounded to bf16 (a, dg/du, w a) or
quantised to MXFP8 can land on the other side of a rounding or E4M3
boundary than the oracle's fp64 value; those tests carry the oracle's
allowance for such decisions.  Here the device's intermediate tensors are
read back (mk_workspace_copy) and
  1. each is checked against the oracle's exact value of it (bf16 rule);
  2. MXFP8 codes and scales the device took from its own bf16 tensors must be
     the oracle quantiser's codes of those tensors, bit for bit, every element;
  3. every next GEMM is recomputed by the oracle from the device's operands
     and compared with no allowance at all, on every element, at the
     workload sizes.
Every step check uses the stated rule (2e-2 x RMS for bf16 paths, 6e-2 x RMS
for MXFP8) with no allowance; from identical operands only the fp32
accumulation differs, and the printed ratios (about 1e-4 .. 2e-3 of RMS
beyond half a bf16 step) show how far inside the rule the device lands.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import bf16, layer, mxfp8, route
from tests.helpers import BF16_TOL, MXFP8_TOL, assert_close, dev, host_bf16, say

pytestmark = pytest.mark.gpu

from mixture_experts_layer_device_amd import binding as B  # noqa: E402
from mixture_experts_layer_device_amd.layer import MoELayer  # noqa: E402

_CACHE = {}


def share_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = workloads.make_expert_share(name)
    return _CACHE[name]


def sync():
    torch.cuda.synchronize()


def by_row(L, name, width, dtype, sp, npos):
    """Workspace buffer `name` ([positions, width]) read back, in arrival row
    order (row r at its sorted position sp[r])."""
    t = L.table(name, npos * width, dtype).cpu().numpy()
    if dtype == torch.int16:
        t = bf16.decode(t.view(np.uint16))
    elif dtype == torch.uint8:
        t = t.view(np.uint8)
    return t.reshape(npos, width)[sp]


def weights(inp):
    return bf16.decode(inp["w_gate"]), bf16.decode(inp["w_up"]), bf16.decode(inp["w_down"])


def share_mb(sh):
    """The minibatch the benchmarks run the full-size expert shares with (the
    two-wave floor of 256 x 256 tiles at H=7168, I=2048 on 256 compute
    units), 256 rows for the small shapes (several minibatches there too)."""
    return 8192 if sh.R > 8192 else 256


def run_share(inp, precision, MB, backward=False, wgrad_mxfp8=False, fused=False):
    sh = inp["shape"]
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=8, max_rows=sh.R, precision=precision, minibatch_rows=MB,
                 enable_backward=backward, wgrad_mxfp8=wgrad_mxfp8, fused_forward=fused)
    x, row_w = dev(inp["x"]), dev(inp["row_w"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=backward)
    L.build_schedule(dev(inp["row_expert"]), sh.R)
    ctx = L.new_fwd_ctx() if backward else None
    out = L.forward(B.MK_EXPERT_SHARE, x, row_w, packed, sh.R, fwd_ctx=ctx)
    g = L.backward(ctx, x, row_w, packed, dev(inp["dY"]), sh.R) if backward else None
    sync()
    sp = L.table("sorted_pos", sh.R).cpu().numpy()
    npos = L.sched_query("num_mb") * L.query("minibatch_rows")
    assert np.all(sp >= 0) and L.device_error() == 0
    return L, out, g, sp, npos


# ------------------------------------------------------------ forward --
@pytest.mark.parametrize("name,fused", [("small", False), ("small", True), ("ep64_fwd", False), ("ep64_fwd", True)])
def test_forward_share_bf16_steps(name, fused):
    inp = share_inputs(name)
    sh = inp["shape"]
    MB = share_mb(sh)
    say(f"[steps, forward bf16{' fused' if fused else ''}] {name} R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB}: "
        f"every element")
    L, out, _, sp, npos = run_share(inp, "bf16", MB, fused=fused)
    a_dev = by_row(L, "a", sh.I, torch.int16, sp, npos)
    L.close()
    wg, wu, wd = weights(inp)
    x, re = bf16.decode(inp["x"]), inp["row_expert"]
    _, _, a_exact = layer.swiglu_rows(x, re, wg, wu)
    assert_close(a_dev, a_exact, BF16_TOL, "a = silu(g) u (GEMM1 + SwiGLU, bf16)", bf16_out=True)
    del a_exact
    out_exact = inp["row_w"][:, None].astype(np.float64) * layer.down_rows(a_dev, re, wd)
    assert_close(host_bf16(out), out_exact, BF16_TOL, "out_rows from the device's a (GEMM2 + weighted unpermute)",
                 bf16_out=True)


@pytest.mark.parametrize("name", ["small", "ep64_fwd"])
def test_forward_share_mxfp8_steps(name):
    inp = share_inputs(name)
    sh = inp["shape"]
    MB = share_mb(sh)
    say(f"[steps, forward MXFP8] {name} R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB}: every element")
    L, out, _, sp, npos = run_share(inp, "mxfp8", MB)
    a_dev = by_row(L, "a", sh.I, torch.int16, sp, npos)
    ac_dev = by_row(L, "a_codes", sh.I, torch.uint8, sp, npos)
    as_dev = by_row(L, "a_scales", sh.I // 32, torch.uint8, sp, npos)
    rr = L.query("ring_rows")
    raw = L.table("ring", rr * (sh.H + sh.H // 32) // 4).cpu().numpy().view(np.uint8)
    ring_pos = sp % rr
    xc_dev = raw[: rr * sh.H].reshape(rr, sh.H)[ring_pos]
    xs_dev = raw[rr * sh.H:].reshape(rr, sh.H // 32)[ring_pos]
    L.close()
    # the permute's quantise of every x row (the ring does not wrap here)
    assert sh.R <= rr
    xc, xs = mxfp8.quantize(bf16.decode(inp["x"]))
    assert np.array_equal(xs_dev, xs) and np.array_equal(xc_dev, xc), "x ring codes / scales"
    ref = layer.forward_share_mxfp8(inp)
    assert_close(a_dev, layer.silu(ref["g"]) * ref["u"], MXFP8_TOL, "a = silu(g) u from MXFP8 operands (bf16)",
                 bf16_out=True)
    # the device's codes of its own a, bit for bit
    rc, rs = mxfp8.quantize(a_dev)
    bad = np.count_nonzero(ac_dev != rc) + np.count_nonzero(as_dev != rs)
    say(f"  a codes: {ac_dev.size} codes and {as_dev.size} scales, {bad} differ from the oracle quantiser's")
    assert bad == 0
    wdq = np.stack([layer.qd(w) for w in bf16.decode(inp["w_down"])])
    y = layer.down_rows(mxfp8.dequantize(ac_dev, as_dev), inp["row_expert"], wdq)
    out_exact = inp["row_w"][:, None].astype(np.float64) * y
    assert_close(host_bf16(out), out_exact, MXFP8_TOL, "out_rows from the device's a codes (MXFP8 GEMM2)",
                 bf16_out=True)


# ----------------------------------------------------------- backward --
def _backward_steps(inp, L, g, sp, npos, mx, wgrad_mx_mb=None):
    sh = inp["shape"]
    I = sh.I
    STEP_TOL = MXFP8_TOL if mx else BF16_TOL
    dgdu = by_row(L, "dgdu", 2 * I, torch.int16, sp, npos)
    wa = by_row(L, "wa", I, torch.int16, sp, npos)
    if mx:
        gc = by_row(L, "dgdu_codes", 2 * I, torch.uint8, sp, npos)
        gs = by_row(L, "dgdu_scales", 2 * I // 32, torch.uint8, sp, npos)
        yc = by_row(L, "dy_codes", sh.H, torch.uint8, sp, npos)
        ys = by_row(L, "dy_scales", sh.H // 32, torch.uint8, sp, npos)
    dX_dev = host_bf16(g["dX"])
    got = {k: g[k].cpu().numpy() for k in ("dW_gate", "dW_up", "dW_down", "d_row_w")}
    L.close()
    wg, wu, wd = weights(inp)
    x, re, w = bf16.decode(inp["x"]), inp["row_expert"], inp["row_w"]
    dY = bf16.decode(inp["dY"])
    if mx:
        yq, ysc = mxfp8.quantize(dY)
        assert np.array_equal(yc, yq) and np.array_equal(ys, ysc), "dY codes / scales"
        f = layer.forward_share_mxfp8(inp)
        G, U = f["g"], f["u"]
        d = layer.dact_rows(dY, G, U, re, wd, w, dYq=mxfp8.dequantize(yq, ysc),
                            wdT=np.stack([layer.qd(wd[e].T) for e in range(sh.E)]))
    else:
        G, U, _ = layer.swiglu_rows(x, re, wg, wu)
        d = layer.dact_rows(dY, G, U, re, wd, w)
    # 1. the dA' GEMM and the SwiGLU backward: dg, du, w a (bf16) and dw
    assert_close(dgdu[:, :I], d["dg"], STEP_TOL, "dg (dA' GEMM + SwiGLU backward)", bf16_out=True)
    assert_close(dgdu[:, I:], d["du"], STEP_TOL, "du", bf16_out=True)
    assert_close(wa, d["wa"], STEP_TOL, "w a", bf16_out=True)
    assert_close(got["d_row_w"], d["dw"], STEP_TOL, "d_row_w (router-weight gradient)")
    del d, G, U
    # 2. the dX GEMM from the device's dg/du (MXFP8: its codes of them)
    if mx:
        pc, ps = mxfp8.quantize(dgdu)
        bad = np.count_nonzero(gc != pc) + np.count_nonzero(gs != ps)
        say(f"  dg/du codes: {gc.size} codes and {gs.size} scales, {bad} differ from the oracle quantiser's")
        assert bad == 0
        dX = layer.dx_rows_from_mx(gc, gs, re, wg, wu)
    else:
        dX = layer.dx_rows_from(dgdu[:, :I], dgdu[:, I:], re, wg, wu)
    assert_close(dX_dev, dX, STEP_TOL, "dX from the device's dg/du", bf16_out=True)
    del dX
    # 3. the weight gradients from the device's operands
    if wgrad_mx_mb is None:
        wgr = layer.wgrads_from(x, dY, dgdu[:, :I], dgdu[:, I:], wa, re, sh.E)
    else:
        wgr = layer.wgrads_from_mx(x, dY, dgdu[:, :I], dgdu[:, I:], wa, re, sh.E, wgrad_mx_mb)
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert_close(got[k], wgr[k], STEP_TOL, k + " from the device's operands")


@pytest.mark.parametrize("name", ["small8", "ep_bwd"])
def test_backward_share_bf16_steps(name):
    inp = share_inputs(name)
    sh = inp["shape"]
    MB = share_mb(sh)
    say(f"[steps, backward bf16] {name} R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB}: every element")
    L, out, g, sp, npos = run_share(inp, "bf16", MB, backward=True)
    _backward_steps(inp, L, g, sp, npos, mx=False)


@pytest.mark.parametrize("name,wmx", [("small8", False), ("small8", True), ("ep_bwd", False), ("ep_bwd", True)])
def test_backward_share_mxfp8_steps(name, wmx):
    inp = share_inputs(name)
    sh = inp["shape"]
    MB = share_mb(sh)
    say(f"[steps, backward MXFP8{' + MXFP8 weight gradients' if wmx else ''}] {name} R={sh.R} H={sh.H} "
        f"I={sh.I} E={sh.E} MB={MB}: every element")
    L, out, g, sp, npos = run_share(inp, "mxfp8", MB, backward=True, wgrad_mxfp8=wmx)
    _backward_steps(inp, L, g, sp, npos, mx=True, wgrad_mx_mb=MB if wmx else None)


# --------------------------------------------------------- full layer --
def test_full_layer_steps():
    """Full layer T=4096 H=2048 I=768 E=128 k=8, forward and backward with
    the router, every element: a from the device's routing, y from the
    device's a, out from the device's y and weights (the combine), then
    dg/du, w a, the fp32 dX rows from the device's dg/du, and dX, dW_router
    and d_bias from the device's dX rows and router-weight gradient (the
    softmax Jacobian and the router GEMMs)."""
    inp = workloads.make_full_layer("full")
    sh = inp["shape"]
    T, H, I, E, k, R = sh.T, sh.H, sh.I, sh.E, sh.k, sh.R
    say(f"[steps, full layer] T={T} H={H} I={I} E={E} k={k}: every element")
    # the forward as the benchmark's main line runs it: one fused launch
    L = MoELayer(H=H, I=I, E=E, k=k, max_rows=R, renorm=sh.renorm, enable_backward=True, fused_forward=True)
    x_d, wr_d, bias_d = dev(inp["x"]), dev(inp["w_router"]), dev(inp["bias"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
    idx, w = L.route(x_d, wr_d, bias_d, T)
    L.build_schedule(idx.view(-1), R)
    ctx = L.new_fwd_ctx()
    out = L.forward(B.MK_FULL_LAYER, x_d, w.view(-1), packed, T, fwd_ctx=ctx)
    sync()
    sp = L.table("sorted_pos", R).cpu().numpy()
    npos = L.sched_query("num_mb") * L.query("minibatch_rows")
    a_dev = by_row(L, "a", I, torch.int16, sp, npos)
    y_dev = L.table("y", npos * H, torch.float32).cpu().numpy().reshape(npos, H)[sp].astype(np.float64)
    g = L.backward_layer(ctx, x_d, wr_d, bias_d, idx, w, packed, dev(inp["dY"]), T)
    sync()
    dgdu = by_row(L, "dgdu", 2 * I, torch.int16, sp, npos)
    wa = by_row(L, "wa", I, torch.int16, sp, npos)
    dx32 = L.table("y", npos * H, torch.float32).cpu().numpy().reshape(npos, H)[sp].astype(np.float64)
    got = {kk: (v.cpu().numpy() if v is not None else None) for kk, v in g.items()}
    idx_d, w_d, out_d = idx.cpu().numpy(), w.cpu().numpy(), host_bf16(out)
    assert L.device_error() == 0
    L.close()
    x = bf16.decode(inp["x"])
    wr = bf16.decode(inp["w_router"])
    idx_r, w_r, z = route.route(x.astype(np.float32), wr.astype(np.float32), inp["bias"], k, sh.renorm)
    assert np.array_equal(idx_d, idx_r)
    wg, wu, wd = weights(inp)
    re = idx_d.reshape(-1)
    x_rows = np.repeat(x, k, axis=0)
    G, U, a_exact = layer.swiglu_rows(x_rows, re, wg, wu)
    assert_close(a_dev, a_exact, BF16_TOL, "a (GEMM1 + SwiGLU)", bf16_out=True)
    assert_close(y_dev, layer.down_rows(a_dev, re, wd), BF16_TOL, "y from the device's a (GEMM2, fp32)")
    assert_close(out_d, layer.combine_tokens(y_dev, w_d, k), BF16_TOL, "out from the device's y and w (combine)",
                 bf16_out=True)
    dY_rows = np.repeat(bf16.decode(inp["dY"]), k, axis=0)
    d = layer.dact_rows(dY_rows, G, U, re, wd, w_d.reshape(-1))
    assert_close(dgdu[:, :I], d["dg"], BF16_TOL, "dg", bf16_out=True)
    assert_close(dgdu[:, I:], d["du"], BF16_TOL, "du", bf16_out=True)
    assert_close(wa, d["wa"], BF16_TOL, "w a", bf16_out=True)
    assert_close(got["d_row_w"], d["dw"], BF16_TOL, "d_topk_w")
    del d, G, U, a_exact
    assert_close(dx32, layer.dx_rows_from(dgdu[:, :I], dgdu[:, I:], re, wg, wu), BF16_TOL,
                 "dX rows from the device's dg/du (fp32)")
    dz = layer.router_logit_grad(z, idx_d, got["d_row_w"].astype(np.float64).reshape(T, k), sh.renorm)
    dX = dx32.reshape(T, k, H).sum(axis=1) + dz @ wr
    assert_close(bf16.decode(got["dX"].view(np.uint16)), dX, BF16_TOL,
                 "dX from the device's dX rows and d_topk_w (k-sum + router term)", bf16_out=True)
    assert_close(got["dW_router"], dz.T @ x, BF16_TOL, "dW_router from the device's d_topk_w")
    assert_close(got["d_bias"], dz.sum(axis=0), BF16_TOL, "d_bias from the device's d_topk_w")
    wgr = layer.wgrads_from(x_rows, dY_rows, dgdu[:, :I], dgdu[:, I:], wa, re, E)
    for kk in ("dW_gate", "dW_up", "dW_down"):
        assert_close(got[kk], wgr[kk], BF16_TOL, kk + " from the device's operands")
