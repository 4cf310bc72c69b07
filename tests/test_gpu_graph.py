"""The layer's step captured as one HIP graph and replayed.

Every call of the boundary only enqueues work on the caller's stream: no
host synchronisation, no device-to-host copy, no allocation and no memset
(counters and flags are cleared by kernels) -- the property that lets a
training step run without the CPU in the loop ([MTP] "Three design decisions
that matter": the ring removes CPU-GPU synchronisation).  Here route,
schedule build, forward and combine (and in the training step the backward
with the router) are captured from one stream into a graph; each replay,
with eager work and different inputs in between, must equal the eager step
bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.helpers import dev, say

pytestmark = pytest.mark.gpu

from mixture_experts_layer_device_amd import binding as B  # noqa: E402
from mixture_experts_layer_device_amd.layer import MoELayer  # noqa: E402


def _replays_match(step, outputs, inputs, other_inputs):
    """Eager results on the inputs and on other_inputs, then the captured
    step replayed three times: on the inputs, on other_inputs copied into
    the same buffers, and on the inputs again (outputs cleared before each
    run, so that bytes a step does not write -- the forward context of the
    padding positions -- read the same; an eager step on the other inputs
    between the replays)."""
    s = torch.cuda.current_stream()
    saved = [t.clone() for t in inputs]
    for t in outputs:
        t.zero_()
    step(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    for t, o in zip(inputs, other_inputs):
        t.copy_(o)
    for t in outputs:
        t.zero_()
    step(s)
    torch.cuda.synchronize()
    ref_other = [t.clone() for t in outputs]
    for t, o in zip(inputs, saved):
        t.copy_(o)
    assert any(not torch.equal(a, b) for a, b in zip(ref, ref_other)), "other inputs gave the same outputs"

    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep, (data, want) in enumerate([(saved, ref), (other_inputs, ref_other), (saved, ref)]):
        for t, o in zip(inputs, data):
            t.copy_(o)
        for t in outputs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, w) in enumerate(zip(outputs, want)):
            assert torch.equal(got, w), f"replay {rep}: output {i} differs from the eager step"
        # eager work between the replays (the other inputs, then back)
        for t, o in zip(inputs, other_inputs):
            t.copy_(o)
        step(s)
        torch.cuda.synchronize()
        for t, o in zip(inputs, saved):
            t.copy_(o)
    del g


def test_full_layer_step_as_one_graph():
    inp = workloads.make_full_layer("full")
    sh = inp["shape"]
    say(f"[graph] full layer fused forward T={sh.T} H={sh.H} I={sh.I} E={sh.E} k={sh.k}")
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, fused_forward=True)
    x, wr, bias = dev(inp["x"]), dev(inp["w_router"]), dev(inp["bias"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
    out = torch.empty((sh.T, sh.H), dtype=torch.int16, device="cuda")
    idx = torch.empty((sh.T, sh.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((sh.T, sh.k), dtype=torch.float32, device="cuda")
    x_other = torch.roll(x, shifts=1, dims=0)    # the same rows, another token order

    def step(s):
        B.mk_route(L.ws, x, wr, bias, sh.T, idx, wts, s)
        B.mk_build_schedule(L.ws, L.sched.handle, idx, sh.R, s)
        B.mk_forward(L.ws, L.sched.handle, B.MK_FULL_LAYER, x, wts, packed, out, None, s)

    _replays_match(step, [out, idx, wts], [x], [x_other])
    assert L.device_error() == 0
    L.close()


def test_expert_share_wrapping_ring_as_one_graph():
    inp = workloads.make_expert_share("small")
    sh = inp["shape"]
    MB = 256
    say(f"[graph] expert share, phase-by-phase launches, R={sh.R} H={sh.H} E={sh.E} MB={MB}, ring of 2 minibatches")
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=8, max_rows=sh.R, minibatch_rows=MB, ring_bytes=2 * MB * 2 * sh.H)
    x, w, rows = dev(inp["x"]), dev(inp["row_w"]), dev(inp["row_expert"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
    out = torch.empty((sh.R, sh.H), dtype=torch.int16, device="cuda")
    rng = np.random.default_rng(5)
    rows_other = torch.from_numpy(rng.permutation(inp["row_expert"]).astype(np.int32)).cuda()

    def step(s):
        B.mk_build_schedule(L.ws, L.sched.handle, rows, sh.R, s)
        B.mk_forward(L.ws, L.sched.handle, B.MK_EXPERT_SHARE, x, w, packed, out, None, s)

    _replays_match(step, [out], [rows], [rows_other])
    assert L.device_error() == 0
    L.close()


def test_full_layer_training_step_as_one_graph():
    """Forward with its context and the backward including the router, one graph."""
    inp = workloads.make_full_layer("full")
    sh = inp["shape"]
    say(f"[graph] full layer forward + backward T={sh.T} H={sh.H} I={sh.I} E={sh.E} k={sh.k}")
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, fused_forward=True,
                 enable_backward=True)
    x, wr, bias, dY = dev(inp["x"]), dev(inp["w_router"]), dev(inp["bias"]), dev(inp["dY"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
    f32 = dict(dtype=torch.float32, device="cuda")
    out = torch.empty((sh.T, sh.H), dtype=torch.int16, device="cuda")
    idx = torch.empty((sh.T, sh.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((sh.T, sh.k), **f32)
    ctx = L.new_fwd_ctx()
    dX = torch.empty((sh.T, sh.H), dtype=torch.int16, device="cuda")
    dWg, dWu = torch.empty((sh.E, sh.I, sh.H), **f32), torch.empty((sh.E, sh.I, sh.H), **f32)
    dWd, dWr = torch.empty((sh.E, sh.H, sh.I), **f32), torch.empty((sh.E, sh.H), **f32)
    db, dw = torch.empty((sh.E,), **f32), torch.empty((sh.R,), **f32)

    def step(s):
        B.mk_route(L.ws, x, wr, bias, sh.T, idx, wts, s)
        B.mk_build_schedule(L.ws, L.sched.handle, idx, sh.R, s)
        B.mk_forward(L.ws, L.sched.handle, B.MK_FULL_LAYER, x, wts, packed, out, ctx, s)
        B.mk_backward_layer(L.ws, L.sched.handle, ctx, x, wr, bias, idx, wts, packed, dY, dX, dWg, dWu, dWd, dWr,
                            db, dw, s)

    _replays_match(step, [out, idx, wts, ctx, dX, dWg, dWu, dWd, dWr, db, dw], [x, dY],
                   [torch.roll(x, shifts=1, dims=0), torch.roll(dY, shifts=3, dims=0)])
    assert L.device_error() == 0
    L.close()


def test_expert_share_mxfp8_training_step_as_one_graph():
    """MXFP8: the quantising permute, the MXFP8 GEMMs, and the backward with
    MXFP8 weight gradients (operand quantisers included), one graph."""
    inp = workloads.make_expert_share("small")
    sh = inp["shape"]
    MB = 256
    say(f"[graph] expert share MXFP8 forward + backward R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB}")
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=8, max_rows=sh.R, minibatch_rows=MB, precision="mxfp8",
                 enable_backward=True, wgrad_mxfp8=True)
    x, w, rows, dY = dev(inp["x"]), dev(inp["row_w"]), dev(inp["row_expert"]), dev(inp["dY"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
    f32 = dict(dtype=torch.float32, device="cuda")
    out = torch.empty((sh.R, sh.H), dtype=torch.int16, device="cuda")
    ctx = L.new_fwd_ctx()
    dX = torch.empty((sh.R, sh.H), dtype=torch.int16, device="cuda")
    dWg, dWu = torch.empty((sh.E, sh.I, sh.H), **f32), torch.empty((sh.E, sh.I, sh.H), **f32)
    dWd, dw = torch.empty((sh.E, sh.H, sh.I), **f32), torch.empty((sh.R,), **f32)

    def step(s):
        B.mk_build_schedule(L.ws, L.sched.handle, rows, sh.R, s)
        B.mk_forward(L.ws, L.sched.handle, B.MK_EXPERT_SHARE, x, w, packed, out, ctx, s)
        B.mk_backward(L.ws, L.sched.handle, B.MK_EXPERT_SHARE, ctx, x, w, packed, dY, dX, dWg, dWu, dWd, dw, s)

    _replays_match(step, [out, ctx, dX, dWg, dWu, dWd, dw], [x, dY],
                   [torch.roll(x, shifts=5, dims=0), torch.roll(dY, shifts=2, dims=0)])
    assert L.device_error() == 0
    L.close()
