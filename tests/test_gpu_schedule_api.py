"""The schedule as a handle ([CARD] "Use the functional API": build_schedule
returns the schedule that forward and backward take): several microbatches'
forwards before their backwards, in any order, give the same bits as one
after the other; and the host-side state checks refuse a backward that has
no matching forward instead of computing from stale buffers."""
import numpy as np
import pytest
import torch

import workloads
from oracle import layer
from tests.helpers import BF16_TOL, MXFP8_TOL, assert_close, dev, host_bf16, say

pytestmark = pytest.mark.gpu

from mixture_experts_layer_device_amd import binding as B  # noqa: E402
from mixture_experts_layer_device_amd.layer import MoELayer  # noqa: E402


def sync():
    torch.cuda.synchronize()


def _micro_inputs(seed_a, seed_b):
    sa = workloads.ExpertShareShape("mbA", R=1536, H=768, I=512, E=8, sources=8, zipf_s=1.2, seed=seed_a)
    sb = workloads.ExpertShareShape("mbB", R=1100, H=768, I=512, E=8, sources=8, zipf_s=1.2, seed=seed_b)
    return workloads.make_expert_share(sa), workloads.make_expert_share(sb)


def _layer(prec, R, MB=256, ring_mbs=2, wmx=False):
    H = 768
    row_bytes = H + H // 32 if prec == "mxfp8" else 2 * H
    return MoELayer(H=H, I=512, E=8, k=8, max_rows=R, precision=prec, minibatch_rows=MB,
                    ring_bytes=ring_mbs * MB * row_bytes, enable_backward=True, wgrad_mxfp8=wmx)


class Micro:
    """Device copies of one microbatch's inputs and its own schedule / ctx."""

    def __init__(self, L, inp, packed):
        self.inp = inp
        self.R = inp["shape"].R
        self.x, self.w, self.dY = dev(inp["x"]), dev(inp["row_w"]), dev(inp["dY"])
        self.re = dev(inp["row_expert"])
        self.sched = L.new_schedule()
        self.ctx = L.new_fwd_ctx()
        self.packed = packed

    def forward(self, L):
        L.build_schedule(self.re, self.R, sched=self.sched)
        return L.forward(B.MK_EXPERT_SHARE, self.x, self.w, self.packed, self.R, fwd_ctx=self.ctx, sched=self.sched)

    def backward(self, L):
        return L.backward(self.ctx, self.x, self.w, self.packed, self.dY, self.R, sched=self.sched)


@pytest.mark.parametrize("prec,wmx", [("bf16", False), ("mxfp8", False), ("mxfp8", True)])
def test_interleaved_microbatches_match_sequential(prec, wmx):
    """forward(A), forward(B), backward(A), backward(B) on one workspace: A's
    rows left the ring when B's forward ran, so A's backward gathers every
    minibatch again; every output equals, bit for bit, the order
    forward(A), backward(A), forward(B), backward(B), and both match the
    oracle."""
    inA, inB = _micro_inputs(51, 52)
    say(f"[schedule handles] {prec}{' + MXFP8 weight gradients' if wmx else ''}: two microbatches "
        f"(R={inA['shape'].R}, {inB['shape'].R}), MB=256, ring of 2 minibatches")
    res = {}
    for order in ("sequential", "interleaved"):
        L = _layer(prec, max(inA["shape"].R, inB["shape"].R), wmx=wmx)
        packed = L.prepare_weights(dev(inA["w_gate"]), dev(inA["w_up"]), dev(inA["w_down"]), for_backward=True)
        A, Bm = Micro(L, inA, packed), Micro(L, inB, packed)
        if order == "sequential":
            oA = A.forward(L); gA = A.backward(L)
            oB = Bm.forward(L); gB = Bm.backward(L)
        else:
            oA = A.forward(L); oB = Bm.forward(L)
            gA = A.backward(L); gB = Bm.backward(L)
        sync()
        assert L.device_error(sched=A.sched) == 0 and L.device_error(sched=Bm.sched) == 0
        res[order] = (oA.clone(), oB.clone(), {k: v.clone() for k, v in gA.items()},
                      {k: v.clone() for k, v in gB.items()})
        L.close()
    s, i = res["sequential"], res["interleaved"]
    assert torch.equal(s[0], i[0]) and torch.equal(s[1], i[1])
    for gs, gi in ((s[2], i[2]), (s[3], i[3])):
        for k in gs:
            assert torch.equal(gs[k], gi[k]), k
    # and the oracle agrees (microbatch B's weights are A's: same packed weights)
    inB = dict(inB, w_gate=inA["w_gate"], w_up=inA["w_up"], w_down=inA["w_down"])
    for inp, (o, g) in ((inA, (i[0], i[2])), (inB, (i[1], i[3]))):
        if prec == "bf16":
            fo = layer.forward_share(inp)
            ref = layer.backward_share(inp, allow=True)
            tol, oa = BF16_TOL, None
        else:
            fo = layer.forward_share_mxfp8(inp, allow=True)
            ref = layer.backward_share_mxfp8(inp, fo, allow=True, wgrad_mx_mb=256 if wmx else None)
            tol, oa = MXFP8_TOL, fo["out_allow"]
        assert_close(host_bf16(o), fo["out_exact"], tol, "out", bf16_out=True, allow=oa)
        assert_close(host_bf16(g["dX"]), ref["dX_exact"], tol, "dX", bf16_out=True, allow=ref["dX_allow"])
        assert_close(g["d_row_w"].cpu().numpy(), ref["d_row_w"], tol, "d_row_w")
        for k in ("dW_gate", "dW_up", "dW_down"):
            assert_close(g[k].cpu().numpy(), ref[k], tol, k, allow=ref.get(k + "_allow"))


def _status(fn, *a):
    try:
        fn(*a)
    except B.MkError as e:
        return e.status
    return B.MK_OK


def test_backward_without_a_matching_forward_is_refused():
    """Host-side checks, no kernel runs for a refused call: a backward
    (1) right after build_schedule, (2) after a forward without fwd_ctx,
    (3) in the other mode than the forward, (4) with another schedule's
    fwd_ctx, (5) after the schedule was rebuilt, or (6) with a schedule of
    another workspace returns MK_ERR_STATE; a matching one runs."""
    inA, inB = _micro_inputs(53, 54)
    say("[schedule handles] backward sequences without a matching forward")
    L = _layer("bf16", 1536)
    L2 = _layer("bf16", 1536)
    packed = L.prepare_weights(dev(inA["w_gate"]), dev(inA["w_up"]), dev(inA["w_down"]), for_backward=True)
    A, Bm = Micro(L, inA, packed), Micro(L, inB, packed)
    R = A.R
    g = L._grads(R, R)

    def bwd(sched, ctx, mode=B.MK_EXPERT_SHARE, ws=None):
        B.mk_backward((ws or L).ws, sched.handle, mode, ctx, A.x, A.w, packed, A.dY, g["dX"], g["dW_gate"],
                      g["dW_up"], g["dW_down"], g["d_row_w"], torch.cuda.current_stream().cuda_stream)

    L.build_schedule(A.re, R, sched=A.sched)
    assert _status(bwd, A.sched, A.ctx) == B.MK_ERR_STATE                          # (1)
    L.forward(B.MK_EXPERT_SHARE, A.x, A.w, packed, R, sched=A.sched)
    assert _status(bwd, A.sched, A.ctx) == B.MK_ERR_STATE                          # (2)
    L.forward(B.MK_EXPERT_SHARE, A.x, A.w, packed, R, fwd_ctx=A.ctx, sched=A.sched)
    assert _status(bwd, A.sched, A.ctx, B.MK_FULL_LAYER) == B.MK_ERR_STATE        # (3)
    assert _status(bwd, A.sched, Bm.ctx) == B.MK_ERR_STATE                         # (4)
    other = L2.new_schedule()
    assert _status(bwd, other, A.ctx) == B.MK_ERR_STATE                            # (6)
    assert _status(B.mk_build_schedule, L.ws, other.handle, A.re, R, None) == B.MK_ERR_STATE
    assert _status(bwd, A.sched, A.ctx) == B.MK_OK                                 # the matching backward
    L.build_schedule(A.re, R, sched=A.sched)
    assert _status(bwd, A.sched, A.ctx) == B.MK_ERR_STATE                          # (5)
    sync()
    L.close()
    L2.close()
