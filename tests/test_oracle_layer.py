"""Pins for the oracle's layer forward/backward (CPU only).

Independent references: scalar per-token loops in plain Python (brute force),
the dense SwiGLU MLP as torch CPU computes it (E=1, k=1, w=1), bit-exact
reproduction of y under one-hot weights, central finite differences, torch
autograd in fp64, and the two-way router-weight-gradient identity.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import bf16, layer, mxfp8, schedule


def rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def scalar_silu(v):
    return v / (1.0 + math.exp(-v))


def test_forward_full_brute_force_micro():
    inp = workloads.make_full_layer("micro")
    sh = inp["shape"]
    ref = layer.forward_full(inp, bf16_mode=False)
    x = bf16.decode(inp["x"]); wg = bf16.decode(inp["w_gate"]); wu = bf16.decode(inp["w_up"])
    wd = bf16.decode(inp["w_down"])
    idx, w = ref["topk_idx"], ref["topk_w"]
    for t in range(sh.T):
        out = [0.0] * sh.H
        for j in range(sh.k):
            e = int(idx[t, j])
            a = []
            for i in range(sh.I):
                g = sum(x[t, h] * wg[e, i, h] for h in range(sh.H))
                u = sum(x[t, h] * wu[e, i, h] for h in range(sh.H))
                a.append(scalar_silu(g) * u)
            for h in range(sh.H):
                y = sum(a[i] * wd[e, h, i] for i in range(sh.I))
                out[h] += float(w[t, j]) * y
        assert np.allclose(ref["out"][t], out, rtol=0, atol=1e-12 * max(1.0, rms(ref["out"])))


def test_forward_reduces_to_dense_swiglu_mlp():
    rng = np.random.default_rng(0)
    R, H, I = 37, 48, 24
    inp = {
        "shape": None,
        "x": workloads.bf16_bits(rng.standard_normal((R, H)).astype(np.float32)),
        "w_gate": workloads.bf16_bits(rng.standard_normal((1, I, H)).astype(np.float32) / 7),
        "w_up": workloads.bf16_bits(rng.standard_normal((1, I, H)).astype(np.float32) / 7),
        "w_down": workloads.bf16_bits(rng.standard_normal((1, H, I)).astype(np.float32) / 5),
        "row_expert": np.zeros(R, dtype=np.int32),
        "row_w": np.ones(R, dtype=np.float32),
    }
    out = layer.forward_share(inp, bf16_mode=False)["out"]
    tx = torch.from_numpy(bf16.decode(inp["x"]))
    g = tx @ torch.from_numpy(bf16.decode(inp["w_gate"])[0]).T
    u = tx @ torch.from_numpy(bf16.decode(inp["w_up"])[0]).T
    y = (torch.nn.functional.silu(g) * u) @ torch.from_numpy(bf16.decode(inp["w_down"])[0]).T
    assert np.allclose(out, y.numpy(), rtol=1e-12, atol=1e-12)


def test_combine_one_hot_weights_reproduce_y_bitwise():
    inp = workloads.make_full_layer("tiny")
    sh = inp["shape"]
    ref = layer.forward_full(inp, bf16_mode=False)
    # with one-hot weights the combine is a copy of the chosen expert's row
    T, k, H = sh.T, sh.k, sh.H
    yk = ref["y"].reshape(T, k, H)
    for j in range(k):
        onehot = np.zeros((T, k), dtype=np.float32); onehot[:, j] = 1.0
        out = np.zeros((T, H))
        for jj in range(k):
            out += onehot[:, jj, None].astype(np.float64) * yk[:, jj]
        assert np.array_equal(out, yk[:, j])


def test_forward_share_invariant_to_schedule_and_rows():
    """The oracle computes per row; each row's output only depends on that row."""
    inp = workloads.make_expert_share("micro")
    ref = layer.forward_share(inp)
    perm = np.random.default_rng(1).permutation(inp["shape"].R)
    inp2 = dict(inp)
    inp2["x"] = inp["x"][perm]; inp2["row_expert"] = inp["row_expert"][perm]; inp2["row_w"] = inp["row_w"][perm]
    ref2 = layer.forward_share(inp2)
    assert np.allclose(ref2["out"], ref["out"][perm], rtol=1e-13, atol=1e-13)


def loss_share(inp, x, wg, wu, wd, w):
    re = inp["row_expert"]
    dY = bf16.decode(inp["dY"])
    tot = 0.0
    for e in range(wg.shape[0]):
        sel = np.nonzero(re == e)[0]
        _, _, _, y = layer.expert_ffn(x[sel], wg[e], wu[e], wd[e])
        tot += float(np.sum(dY[sel] * (w[sel, None] * y)))
    return tot


def test_backward_finite_differences():
    inp = workloads.make_expert_share("micro")
    g = layer.backward_share(inp, bf16_mode=False)
    x = bf16.decode(inp["x"]); wg = bf16.decode(inp["w_gate"]); wu = bf16.decode(inp["w_up"])
    wd = bf16.decode(inp["w_down"]); w = inp["row_w"].astype(np.float64)
    rng = np.random.default_rng(9)
    args = {"x": x, "wg": wg, "wu": wu, "wd": wd, "w": w}
    grads = {"x": g["dX"], "wg": g["dW_gate"], "wu": g["dW_up"], "wd": g["dW_down"], "w": g["d_row_w"]}
    eps = 1e-5
    for name, val in args.items():
        d = rng.standard_normal(val.shape)
        plus = dict(args); plus[name] = val + eps * d
        minus = dict(args); minus[name] = val - eps * d
        fd = (loss_share(inp, **plus) - loss_share(inp, **minus)) / (2 * eps)
        an = float(np.sum(grads[name] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), name


def test_backward_matches_torch_autograd():
    inp = workloads.make_expert_share("micro")
    g = layer.backward_share(inp, bf16_mode=False)
    re = torch.from_numpy(inp["row_expert"].astype(np.int64))
    x = torch.tensor(bf16.decode(inp["x"]), requires_grad=True)
    wg = torch.tensor(bf16.decode(inp["w_gate"]), requires_grad=True)
    wu = torch.tensor(bf16.decode(inp["w_up"]), requires_grad=True)
    wd = torch.tensor(bf16.decode(inp["w_down"]), requires_grad=True)
    w = torch.tensor(inp["row_w"].astype(np.float64), requires_grad=True)
    gsel = torch.einsum("rh,rih->ri", x, wg[re])
    usel = torch.einsum("rh,rih->ri", x, wu[re])
    a = torch.nn.functional.silu(gsel) * usel
    y = torch.einsum("ri,rhi->rh", a, wd[re])
    out = w[:, None] * y
    (out * torch.from_numpy(bf16.decode(inp["dY"]))).sum().backward()
    assert np.allclose(g["dX"], x.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["dW_gate"], wg.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["dW_up"], wu.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["dW_down"], wd.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["d_row_w"], w.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_router_weight_gradient_two_ways():
    inp = workloads.make_expert_share("small")
    g = layer.backward_share(inp)
    assert np.allclose(g["d_row_w"], g["d_row_w_alt"], rtol=1e-9, atol=1e-9)


def test_mxfp8_forward_brute_force_rows():
    inp = workloads.make_expert_share("micro")
    ref = layer.forward_share_mxfp8(inp)
    x = bf16.decode(inp["x"])
    qg = mxfp8.quantize(bf16.decode(inp["w_gate"])); qu = mxfp8.quantize(bf16.decode(inp["w_up"]))
    qd = mxfp8.quantize(bf16.decode(inp["w_down"]))
    for r in range(0, inp["shape"].R, 5):
        e = int(inp["row_expert"][r])
        xc, xs = mxfp8.quantize(x[r:r + 1])
        assert np.array_equal(xc, ref["x_codes"][r:r + 1]) and np.array_equal(xs, ref["x_scales"][r:r + 1])
        xd = mxfp8.e4m3_decode(xc[0]) * np.repeat(2.0 ** (xs[0].astype(np.float64) - 127), 32)
        I = qg[0].shape[1]
        a = np.zeros(I)
        for i in range(I):
            wgd = mxfp8.e4m3_decode(qg[0][e, i]) * np.repeat(2.0 ** (qg[1][e, i].astype(np.float64) - 127), 32)
            wud = mxfp8.e4m3_decode(qu[0][e, i]) * np.repeat(2.0 ** (qu[1][e, i].astype(np.float64) - 127), 32)
            gg = math.fsum(xd * wgd); uu = math.fsum(xd * wud)
            a[i] = bf16.decode(bf16.encode(np.array(scalar_silu(gg) * uu)))
        assert np.array_equal(bf16.encode(a), ref["a_bits"][r])
        ac, as_ = mxfp8.quantize(a[None, :])
        ad = mxfp8.e4m3_decode(ac[0]) * np.repeat(2.0 ** (as_[0].astype(np.float64) - 127), 32)
        for h in range(0, inp["shape"].H, 7):
            wdd = mxfp8.e4m3_decode(qd[0][e, h]) * np.repeat(2.0 ** (qd[1][e, h].astype(np.float64) - 127), 32)
            y = math.fsum(ad * wdd)
            assert abs(ref["y"][r, h] - y) <= 1e-12 * max(1.0, abs(y))


def test_mxfp8_forward_close_to_bf16_forward():
    """Quantisation error of the whole MXFP8 layer stays near E4M3's ~2^-4
    relative precision (a sanity band, not the parity bound)."""
    inp = workloads.make_expert_share("small")
    q = layer.forward_share_mxfp8(inp)["out"]
    b = layer.forward_share(inp)["out"]
    assert rms(q - b) < 0.1 * rms(b)


def test_ring_contents_wrap():
    inp = workloads.make_full_layer("tiny")
    ref = layer.forward_full(inp)
    re = ref["row_expert"]
    MB = 128
    s = schedule.build(re, 8, MB, 2 * MB, 64)
    src = np.arange(len(re)) // 2
    ring, written = layer.ring_contents(s, inp["x"], src)
    assert written.all()
    # the ring ends up holding the last two minibatches
    for p in range(2 * MB, 4 * MB):
        r = s.inv[p]
        assert np.array_equal(ring[p % (2 * MB)], inp["x"][src[r]])


def test_sampled_helpers_match_full_oracle():
    inp = workloads.make_expert_share("small")
    full = layer.forward_share(inp)["out"]
    rows = np.array([0, 7, 500, 999])
    assert np.allclose(layer.forward_share_rows(inp, rows), full[rows], rtol=1e-12, atol=1e-12)
    fq = layer.forward_share_mxfp8(inp)["out"]
    assert np.allclose(layer.forward_share_mxfp8_rows(inp, rows), fq[rows], rtol=1e-12, atol=1e-12)
    g = layer.backward_share(inp)
    pairs = [(0, 3), (2, 255), (3, 0)]
    smp = layer.backward_share_sampled(inp, rows, pairs, pairs)
    assert np.allclose(smp["dX"], g["dX"][rows], rtol=1e-10, atol=1e-12)
    assert np.allclose(smp["d_row_w"], g["d_row_w"][rows], rtol=1e-10, atol=1e-12)
    for n, (e, i) in enumerate(pairs):
        assert np.allclose(smp["dW_gate"][n], g["dW_gate"][e, i], rtol=1e-10, atol=1e-12)
        assert np.allclose(smp["dW_up"][n], g["dW_up"][e, i], rtol=1e-10, atol=1e-12)
        assert np.allclose(smp["dW_down"][n], g["dW_down"][e, :, i], rtol=1e-10, atol=1e-12)


def test_full_layer_token_helper_matches_full_oracle():
    inp = workloads.make_full_layer("tiny")
    ref = layer.forward_full(inp)
    toks = [0, 5, 255]
    got = layer.forward_full_tokens(inp, ref["topk_idx"], ref["topk_w"], toks)
    assert np.allclose(got, ref["out"][toks], rtol=1e-12, atol=1e-12)


def ulp_bf16(v):
    """Spacing of bf16 values at |v| (2^-133 below the normal range)."""
    _, e = np.frexp(np.abs(v))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def test_bf16_mode_forward_within_rounding_bound_of_exact():
    """bf16 mode differs from the exact layer only by the roundings it names:
    |out - out_exact| <= half an output ulp + |w| sum_i |W_d[h, i]| half-ulp(a_i)."""
    inp = workloads.make_expert_share("small")
    b = layer.forward_share(inp, bf16_mode=True)
    x = layer.forward_share(inp, bf16_mode=False)
    assert np.array_equal(bf16.round_rne(b["out"]), b["out"])            # outputs are bf16 values
    assert np.array_equal(bf16.round_rne(b["a"]), b["a"])                # a is a bf16 operand
    wd = bf16.decode(inp["w_down"])
    w = np.abs(inp["row_w"].astype(np.float64))
    re = inp["row_expert"]
    bound = np.zeros_like(b["out"])
    for e in range(wd.shape[0]):
        sel = np.nonzero(re == e)[0]
        bound[sel] = w[sel, None] * ((0.5 * ulp_bf16(x["a"][sel])) @ np.abs(wd[e]).T)
    err = np.abs(b["out"] - x["out"])
    assert np.all(err <= bound * (1 + 1e-9) + 0.5 * ulp_bf16(b["out"]) + 1e-300)
    assert np.any(err > 0)


def test_bf16_mode_backward_close_to_exact():
    inp = workloads.make_expert_share("small")
    b = layer.backward_share(inp, bf16_mode=True)
    x = layer.backward_share(inp, bf16_mode=False)
    for k in ("dX", "dW_gate", "dW_up", "dW_down", "d_row_w"):
        rel = np.linalg.norm(b[k] - x[k]) / np.linalg.norm(x[k])
        assert rel < 4e-3, (k, rel)
        if k != "d_row_w":
            assert rel > 0, k          # the roundings really happen
    assert np.array_equal(bf16.round_rne(b["dX"]), b["dX"])


def test_bf16_spread_bounds_perturbed_roundings():
    """bf16_spread: every value within the relative margin of v rounds to a
    bf16 value no farther from bf16(v) than the spread, the spread is zero
    where the whole interval rounds alike, and it reaches one bf16 step for
    values on a rounding midpoint."""
    rng = np.random.default_rng(17)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, size=20000))
    # plant exact midpoints between adjacent bf16 values
    b = bf16.round_rne(v[:200])
    _, e = np.frexp(np.abs(b))
    v[:200] = b + np.sign(b) * np.ldexp(1.0, e - 9)
    sp = layer.bf16_spread(v)
    ref = bf16.round_rne(v)
    for t in np.linspace(-1.0, 1.0, 21):
        moved = np.abs(bf16.round_rne(v * (1.0 + t * layer.DECISION_REL)) - ref)
        assert np.all(moved <= sp)
    assert np.all(sp[:200] > 0)
    assert np.mean(sp[200:] == 0) > 0.9          # a margin of 2^-13 against steps of 2^-8 .. 2^-7


def test_bf16_backward_allowances_bound_perturbed_gemm_outputs(monkeypatch):
    """With dg, du and w a perturbed within the margin before their bf16
    rounding, the bf16 backward's weight gradients stay within the oracle's
    allowance."""
    inp = workloads.make_expert_share("small")
    ref = layer.backward_share(inp, allow=True)
    rng = np.random.default_rng(19)
    real_rnd = layer.rnd

    def jitter(v, on):
        if not on:
            return real_rnd(v, on)
        return real_rnd(v * (1.0 + layer.DECISION_REL * rng.uniform(-1, 1, size=np.shape(v))), on)

    monkeypatch.setattr(layer, "rnd", jitter)
    got = layer.backward_share(inp)
    monkeypatch.undo()
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert np.all(np.abs(got[k] - ref[k]) <= ref[k + "_allow"] * (1 + 1e-9) + 1e-12), k
    assert np.mean(ref["dW_up_allow"]) < 0.01 * np.sqrt(np.mean(ref["dW_up"] ** 2))


def _rne_bf16(v: float) -> float:
    """Round one float to the nearest bf16 value, ties to even (8 significant
    bits; Python's round() breaks ties to even).  Normal range only."""
    if v == 0.0:
        return v
    m, e = math.frexp(v)                 # v = m 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0), e - 8)


def test_bf16_backward_rounding_points_by_scalar_loops():
    """The bf16-mode backward rounds exactly dg, du, w a and dX, once each
    (the GEMM operands and the output), and nothing else: a scalar loop on
    the micro shape that rounds at those points and computes all else in
    exact double arithmetic must reproduce the oracle bit for bit (dX) and to
    the last few double ulps (dW, dw).  A rounding moved (on dA' or dA
    instead of dg, on a, or one missing) changes dW by ~1e-3 relative."""
    inp = workloads.make_expert_share("micro")
    ref = layer.backward_share(inp, bf16_mode=True)
    x = bf16.decode(inp["x"]); dY = bf16.decode(inp["dY"])
    wg = bf16.decode(inp["w_gate"]); wu = bf16.decode(inp["w_up"]); wd = bf16.decode(inp["w_down"])
    re = inp["row_expert"]; w = inp["row_w"].astype(np.float64)
    R, H = x.shape
    E, I, _ = wg.shape
    dWg = np.zeros((E, I, H)); dWu = np.zeros((E, I, H)); dWd = np.zeros((E, H, I))
    for r in range(R):
        e = int(re[r])
        dg = [0.0] * I; du = [0.0] * I; wa = [0.0] * I; dw = 0.0
        for i in range(I):
            g = math.fsum(x[r, h] * wg[e, i, h] for h in range(H))
            u = math.fsum(x[r, h] * wu[e, i, h] for h in range(H))
            dap = math.fsum(dY[r, h] * wd[e, h, i] for h in range(H))
            s = 1.0 / (1.0 + math.exp(-g))
            a = g * s * u
            dw += dap * a
            dg[i] = _rne_bf16(w[r] * dap * u * s * (1.0 + g * (1.0 - s)))
            du[i] = _rne_bf16(w[r] * dap * g * s)
            wa[i] = _rne_bf16(w[r] * a)
        dx = [_rne_bf16(math.fsum(dg[i] * wg[e, i, h] + du[i] * wu[e, i, h] for i in range(I))) for h in range(H)]
        assert np.array_equal(np.array(dx), ref["dX"][r]), r
        assert math.isclose(dw, ref["d_row_w"][r], rel_tol=1e-12, abs_tol=1e-15)
        for i in range(I):
            dWg[e, i] += dg[i] * x[r]
            dWu[e, i] += du[i] * x[r]
            dWd[e, :, i] += dY[r] * wa[i]
    for k, v in (("dW_gate", dWg), ("dW_up", dWu), ("dW_down", dWd)):
        assert np.allclose(v, ref[k], rtol=1e-12, atol=1e-15), k


def test_single_steps_compose_to_the_layer():
    """The one-GEMM step functions (fed given operands) rebuild the whole
    layer from its own intermediates: bf16 and MXFP8, forward and backward,
    expert share and full layer.  The layer itself is pinned by brute force,
    finite differences and autograd; these pin the step functions to it."""
    inp = workloads.make_expert_share("small8")
    x, dY = bf16.decode(inp["x"]), bf16.decode(inp["dY"])
    wg, wu, wd = (bf16.decode(inp[n]) for n in ("w_gate", "w_up", "w_down"))
    re, w = inp["row_expert"], inp["row_w"].astype(np.float64)
    E, I, H = wg.shape
    f = layer.forward_share(inp)
    G, U, a = layer.swiglu_rows(x, re, wg, wu)
    assert np.allclose(G, f["g"], rtol=1e-13, atol=1e-13) and np.array_equal(bf16.round_rne(a), f["a"])
    assert np.allclose(w[:, None] * layer.down_rows(f["a"], re, wd), f["out_exact"], rtol=1e-12, atol=1e-13)
    b = layer.backward_share(inp)
    d = layer.dact_rows(dY, G, U, re, wd, w)
    assert np.allclose(d["dw"], b["d_row_w"], rtol=1e-12, atol=1e-13)
    dg, du, wa = bf16.round_rne(d["dg"]), bf16.round_rne(d["du"]), bf16.round_rne(d["wa"])
    assert np.allclose(layer.dx_rows_from(dg, du, re, wg, wu), b["dX_exact"], rtol=1e-12, atol=1e-13)
    wgr = layer.wgrads_from(x, dY, dg, du, wa, re, E)
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert np.allclose(wgr[k], b[k], rtol=1e-12, atol=1e-13), k
    # MXFP8
    fm = layer.forward_share_mxfp8(inp)
    ac, as_ = mxfp8.quantize(bf16.decode(fm["a_bits"]))
    wdq = np.stack([layer.qd(m) for m in wd])
    assert np.allclose(w[:, None] * layer.down_rows(mxfp8.dequantize(ac, as_), re, wdq), fm["out_exact"],
                       rtol=1e-12, atol=1e-13)
    bm = layer.backward_share_mxfp8(inp, fm, wgrad_mx_mb=256)
    dm = layer.dact_rows(dY, fm["g"], fm["u"], re, wd, w, dYq=layer.qd(dY),
                         wdT=np.stack([layer.qd(wd[e].T) for e in range(E)]))
    assert np.allclose(dm["dw"], bm["d_row_w"], rtol=1e-12, atol=1e-13)
    dgm, dum, wam = bf16.round_rne(dm["dg"]), bf16.round_rne(dm["du"]), bf16.round_rne(dm["wa"])
    pc, ps = mxfp8.quantize(np.concatenate([dgm, dum], axis=1))
    assert np.allclose(layer.dx_rows_from_mx(pc, ps, re, wg, wu), bm["dX_exact"], rtol=1e-12, atol=1e-13)
    wm = layer.wgrads_from_mx(x, dY, dgm, dum, wam, re, E, 256)
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert np.allclose(wm[k], bm[k], rtol=1e-12, atol=1e-13), k
    # full layer: the combine
    fi = workloads.make_full_layer("tiny")
    ff = layer.forward_full(fi)
    assert np.allclose(layer.combine_tokens(ff["y"], ff["topk_w"], fi["shape"].k), ff["out_exact"],
                       rtol=1e-12, atol=1e-13)
