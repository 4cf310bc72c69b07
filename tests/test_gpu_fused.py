"""The fused forward (mk_config.fused_forward: permute, GEMM1 + SwiGLU and
GEMM2 in one persistent launch, minibatches overlapping through device
counters; the full layer's combine follows as a launch of its own) against
the phase-by-phase launches,
bit for bit, and against the oracle: several minibatches, one minibatch, the
expert share and the full layer.  In the expert share a ring that cannot
hold every minibatch falls back to the phase-by-phase launches; the full
layer's fused launch reads the token rows through the inverse map and needs
no ring, so it runs fused whatever the ring holds."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from oracle import layer, route
from tests.helpers import BF16_TOL, assert_close, dev, host_bf16, say
from oracle import bf16

pytestmark = pytest.mark.gpu

from mixture_experts_layer_device_amd import binding as B  # noqa: E402
from mixture_experts_layer_device_amd.layer import MoELayer  # noqa: E402


def _share(inp, fused, MB, ring_mbs, fwd_ctx=False):
    sh = inp["shape"]
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * 2 * sh.H
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=8, max_rows=sh.R, minibatch_rows=MB, ring_bytes=ring,
                 fused_forward=fused, enable_backward=fwd_ctx)
    x, w = dev(inp["x"]), dev(inp["row_w"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=fwd_ctx)
    L.build_schedule(dev(inp["row_expert"]), sh.R)
    ctx = L.new_fwd_ctx() if fwd_ctx else None
    B.mk_timing_read(L.ws)
    B.mk_timing_enable(L.ws, True)
    outs = [L.forward(B.MK_EXPERT_SHARE, x, w, packed, sh.R, fwd_ctx=ctx) for _ in range(2)]
    torch.cuda.synchronize()
    B.mk_timing_enable(L.ws, False)
    L.fused_launches = B.mk_timing_read(L.ws)["fused_fwd"][1]
    return L, outs, ctx, (x, w, packed)


@pytest.mark.parametrize("name,MB,ring_mbs", [("small8", 256, None), ("small8", 0, None), ("small", 128, None),
                                               ("ep64_fwd", 4096, None), ("small8", 256, 2)],
                         ids=["small8_6mb", "small8_one_mb", "small_8mb", "ep64_4mb", "small8_ring2_fallback"])
def test_fused_share_equals_phase_by_phase(name, MB, ring_mbs):
    inp = workloads.make_expert_share(name, with_dy=False)
    sh = inp["shape"]
    say(f"[fused forward] expert share {name} R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB} ring_mbs={ring_mbs}")
    Lf, of, _, _ = _share(inp, True, MB, ring_mbs)
    assert Lf.device_error() == 0
    # fused when the ring holds every minibatch, else one launch per phase
    assert Lf.fused_launches == (0 if ring_mbs else 2)
    assert torch.equal(of[0], of[1]), "fused forward not repeatable"
    ring_f = Lf.table("ring", Lf.query("ring_rows") * sh.H, torch.int16).cpu()
    Lf.close()
    Lp, op, _, _ = _share(inp, False, MB, ring_mbs)
    ring_p = Lp.table("ring", Lp.query("ring_rows") * sh.H, torch.int16).cpu()
    Lp.close()
    assert torch.equal(of[0], op[0]), "fused and phase-by-phase outputs differ"
    assert torch.equal(ring_f, ring_p), "ring contents differ"
    if sh.R <= 2048:
        ref = layer.forward_share(inp)["out_exact"]
        assert_close(host_bf16(of[0]), ref, BF16_TOL, "out_rows (fused)", bf16_out=True)
    else:
        rows = np.sort(np.random.default_rng(7).choice(sh.R, 48, replace=False))
        ref = layer.forward_share_rows(inp, rows, exact=True)
        assert_close(host_bf16(of[0])[rows], ref, BF16_TOL, "out_rows (fused, 48 sampled rows)", bf16_out=True)


@pytest.mark.parametrize("name,MB,ring_mbs", [("tiny", 128, None), ("tiny", 0, None), ("full", 0, None),
                                               ("full", 8192, None), ("tiny", 128, 1)],
                         ids=["tiny_4mb", "tiny_one_mb", "full_one_mb", "full_4mb", "tiny_4mb_ring1"])
def test_fused_full_layer_equals_phase_by_phase(name, MB, ring_mbs):
    inp = workloads.make_full_layer(name)
    sh = inp["shape"]
    say(f"[fused forward] full layer {name} T={sh.T} H={sh.H} I={sh.I} E={sh.E} k={sh.k} MB={MB} "
        f"ring_mbs={ring_mbs}")
    res = []
    for fused in (True, False):
        ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * 2 * sh.H
        L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, minibatch_rows=MB,
                     ring_bytes=ring, fused_forward=fused)
        x = dev(inp["x"])
        packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
        bias = dev(inp["bias"]) if inp["bias"] is not None else None
        idx, w = L.route(x, dev(inp["w_router"]), bias, sh.T)
        L.build_schedule(idx.view(-1), sh.R)
        B.mk_timing_read(L.ws)
        B.mk_timing_enable(L.ws, True)
        outs = [L.forward(B.MK_FULL_LAYER, x, w.view(-1), packed, sh.T) for _ in range(2)]
        torch.cuda.synchronize()
        B.mk_timing_enable(L.ws, False)
        assert B.mk_timing_read(L.ws)["fused_fwd"][1] == (2 if fused else 0)
        assert L.device_error() == 0
        assert torch.equal(outs[0], outs[1])
        res.append((idx.cpu().numpy(), w.cpu().numpy(), outs[0]))
        L.close()
    assert torch.equal(res[0][2], res[1][2]), "fused and phase-by-phase outputs differ"
    idx, w, out = res[0]
    x32 = bf16.decode(inp["x"]).astype(np.float32)
    idx_r, w_r, _ = route.route(x32, bf16.decode(inp["w_router"]).astype(np.float32), inp["bias"], sh.k, sh.renorm)
    assert np.array_equal(idx, idx_r)
    toks = np.arange(sh.T) if sh.T <= 256 else np.sort(np.random.default_rng(8).choice(sh.T, 64, replace=False))
    ref = layer.forward_full_tokens(inp, idx_r, w_r, toks, exact=True)
    assert_close(host_bf16(out)[toks], ref, BF16_TOL, "out (fused)", bf16_out=True)


def test_fused_forward_context_feeds_the_backward():
    """The fused forward writes the same forward context as the phase-by-phase
    one, and the backward taken after it gives the same gradients."""
    inp = workloads.make_expert_share("small8")
    sh = inp["shape"]
    say(f"[fused forward] fwd_ctx and backward, small8 R={sh.R} MB=256 (6 minibatches)")
    g = []
    ctxs = []
    for fused in (True, False):
        L, outs, ctx, (x, w, packed) = _share(inp, fused, 256, None, fwd_ctx=True)
        assert L.fused_launches == (2 if fused else 0)
        gr = L.backward(ctx, x, w, packed, dev(inp["dY"]), sh.R)
        torch.cuda.synchronize()
        g.append({k: v.clone() for k, v in gr.items()})
        ctxs.append(ctx.clone())
        L.close()
    assert torch.equal(ctxs[0], ctxs[1]), "forward contexts differ"
    for k in g[0]:
        assert torch.equal(g[0][k], g[1][k]), k



@pytest.mark.parametrize("name,MB", [("tiny", 128), ("tiny", 0)], ids=["tiny_4mb", "tiny_one_mb"])
def test_fused_full_layer_backward_replays_the_token_rows(name, MB):
    """The full layer's fused forward gathers the token rows through the
    inverse map and leaves the ring alone, so the backward of its schedule
    gathers the x rows again: its forward context and every gradient
    (router included) equal those after the phase-by-phase forward, which
    left the rows in the ring, bit for bit."""
    # (the backward needs I a multiple of 256)
    inp = workloads.make_full_layer(dataclasses.replace(workloads.FULL_LAYER[name], I=256))
    sh = inp["shape"]
    say(f"[fused forward] full layer {name} (I=256) backward after the fused forward, MB={MB}")
    res = []
    for fused in (True, False):
        L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, minibatch_rows=MB,
                     enable_backward=True, fused_forward=fused)
        x, wr = dev(inp["x"]), dev(inp["w_router"])
        bias = dev(inp["bias"]) if inp["bias"] is not None else None
        packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
        idx, w = L.route(x, wr, bias, sh.T)
        L.build_schedule(idx.view(-1), sh.R)
        ctx = L.new_fwd_ctx()
        B.mk_timing_read(L.ws)
        B.mk_timing_enable(L.ws, True)
        out = L.forward(B.MK_FULL_LAYER, x, w.view(-1), packed, sh.T, fwd_ctx=ctx)
        torch.cuda.synchronize()
        B.mk_timing_enable(L.ws, False)
        assert B.mk_timing_read(L.ws)["fused_fwd"][1] == (1 if fused else 0)
        g = L.backward_layer(ctx, x, wr, bias, idx, w, packed, dev(inp["dY"]), sh.T)
        torch.cuda.synchronize()
        assert L.device_error() == 0
        res.append((out.clone(), ctx.clone(), {k: v.clone() for k, v in g.items() if v is not None}))
        L.close()
    assert torch.equal(res[0][0], res[1][0]), "outputs differ"
    assert torch.equal(res[0][1], res[1][1]), "forward contexts differ"
    assert res[0][2].keys() == res[1][2].keys()
    for k in res[0][2]:
        assert torch.equal(res[0][2][k], res[1][2][k]), k


@pytest.mark.parametrize("mode", ["full", "share"])
def test_fused_wait_bound_reports_timeout_and_recovers(mode):
    """The fused launch's dependency waits are bounded polls of device
    counters.  Forced from the host (mk_debug_fused_waits: a bound of 64 polls
    and targets one above what the producers count), every wait ends at its
    bound, the launch runs to its end, and the schedule's error word carries
    MK_DEVERR_WAIT_TIMEOUT; with the hook cleared, the next schedule build
    clears the word and the forward gives the same output as before."""
    if mode == "full":
        inp = workloads.make_full_layer("tiny")
        sh = inp["shape"]
        MB = 128
        L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, minibatch_rows=MB,
                     fused_forward=True)
        x = dev(inp["x"])
        packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
        bias = dev(inp["bias"]) if inp["bias"] is not None else None
        idx, w = L.route(x, dev(inp["w_router"]), bias, sh.T)
        rows, w, n, kind = idx.view(-1), w.view(-1), sh.T, B.MK_FULL_LAYER
    else:
        inp = workloads.make_expert_share("small")
        sh = inp["shape"]
        MB = 256
        L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=8, max_rows=sh.R, minibatch_rows=MB, fused_forward=True)
        x, w = dev(inp["x"]), dev(inp["row_w"])
        packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
        rows, n, kind = dev(inp["row_expert"]), sh.R, B.MK_EXPERT_SHARE
    say(f"[fused forward] bounded waits forced to time out: {mode} H={sh.H} I={sh.I} E={sh.E} MB={MB}")
    L.build_schedule(rows, sh.R)
    ref = L.forward(kind, x, w, packed, n).clone()
    torch.cuda.synchronize()
    assert L.device_error() == 0
    B.mk_debug_fused_waits(L.ws, 64, True)
    L.forward(kind, x, w, packed, n)
    torch.cuda.synchronize()
    assert L.device_error() & B.MK_DEVERR_WAIT_TIMEOUT
    B.mk_debug_fused_waits(L.ws, 0, False)
    L.build_schedule(rows, sh.R)
    out = L.forward(kind, x, w, packed, n)
    torch.cuda.synchronize()
    assert L.device_error() == 0
    assert torch.equal(out, ref)
    L.close()
