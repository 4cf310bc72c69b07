"""Pins for the oracle's MXFP8 expert-share backward (CPU only).

Independent references: with the quantiser replaced by the identity the
MXFP8 backward must be the bf16 backward (pinned by autograd and finite
differences elsewhere), so only the quantise-dequantise steps are new; a
power-of-two scaling of one dY row must scale exactly that row's dX and
router-weight gradient (every quantised operand is blocked along its own
row, and power-of-two scales commute with E4M3/E8M0 quantisation and bf16
rounding); and the MXFP8 result stays within E4M3's error of the bf16 one.
"""
import numpy as np
import pytest

import workloads
from oracle import bf16, layer, mxfp8


def test_identity_quantiser_gives_the_bf16_backward(monkeypatch):
    inp = workloads.make_expert_share("small")
    monkeypatch.setattr(mxfp8, "quantize", lambda v: (np.asarray(v, dtype=np.float64), None))
    monkeypatch.setattr(mxfp8, "dequantize", lambda c, s: c)
    m = layer.backward_share_mxfp8(inp)
    monkeypatch.undo()
    b = layer.backward_share(inp)
    for k in ("dW_gate", "dW_up", "dW_down", "d_row_w"):
        assert np.allclose(m[k], b[k], rtol=1e-11, atol=1e-12), k
    # dX: the same exact value summed in another order, rounded once to bf16
    d = np.abs(m["dX"] - b["dX"])
    _, e = np.frexp(np.abs(b["dX"]))
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    assert np.all(d <= ulp) and np.mean(d > 0) < 1e-3


def test_scaling_one_dy_row_scales_only_that_row():
    inp = dict(workloads.make_expert_share("small"))
    base = layer.backward_share_mxfp8(inp)
    r = 123
    dY = bf16.decode(inp["dY"]).copy()
    dY[r] *= 4.0
    inp["dY"] = bf16.encode(dY)
    m = layer.backward_share_mxfp8(inp)
    assert np.array_equal(m["dX"][r], 4.0 * base["dX"][r])
    assert m["d_row_w"][r] == 4.0 * base["d_row_w"][r]
    others = np.arange(inp["x"].shape[0]) != r
    assert np.array_equal(m["dX"][others], base["dX"][others])
    assert np.array_equal(m["d_row_w"][others], base["d_row_w"][others])


def test_mxfp8_backward_within_e4m3_error_of_bf16():
    inp = workloads.make_expert_share("small")
    m = layer.backward_share_mxfp8(inp)
    b = layer.backward_share(inp)
    for k in ("dX", "dW_gate", "dW_up", "dW_down", "d_row_w"):
        rel = np.linalg.norm(m[k] - b[k]) / np.linalg.norm(b[k])
        assert 5e-3 < rel < 0.12, (k, rel)     # E4M3 step 2^-3: a few % RMS after a few quantisations


def test_dx_blocks_cut_from_dg_and_du_each_alone():
    """The dX contraction runs over the I gate features then the I up
    features, so its MX blocks of 32 are cut from dg alone and from du alone
    (I is a multiple of 32), and the weights likewise: dX must equal the sum
    of two separately blocked contractions, D(Q(dg)) D(Q(W_g^T))^T +
    D(Q(du)) D(Q(W_u^T))^T, each quantised along I on its own.  A blocking
    that mixed gate and up features in one block (any interleave) changes
    the shared scales and fails this."""
    inp = workloads.make_expert_share("small8")
    fwd = layer.forward_share_mxfp8(inp)
    ref = layer.backward_share_mxfp8(inp, fwd)
    x = bf16.decode(inp["x"]); dY = bf16.decode(inp["dY"]); w = inp["row_w"].astype(np.float64)
    wg = bf16.decode(inp["w_gate"]); wu = bf16.decode(inp["w_up"]); wd = bf16.decode(inp["w_down"])
    re = inp["row_expert"]
    dX = np.zeros_like(x)
    for e in range(wg.shape[0]):
        sel = np.nonzero(re == e)[0]
        g, u = fwd["g"][sel], fwd["u"][sel]
        dAp = layer.qd(dY[sel]) @ layer.qd(wd[e].T).T
        s = 1.0 / (1.0 + np.exp(-g))
        dA = w[sel, None] * dAp
        dg = bf16.round_rne(dA * u * s * (1.0 + g * (1.0 - s)))
        du = bf16.round_rne(dA * g * s)
        dX[sel] = layer.qd(dg) @ layer.qd(wg[e].T).T + layer.qd(du) @ layer.qd(wu[e].T).T
    dX = bf16.round_rne(dX)
    # the same value summed in another order, rounded once: at most one bf16 step apart
    d = np.abs(dX - ref["dX"])
    _, ex = np.frexp(np.maximum(np.abs(dX), np.abs(ref["dX"])))
    assert np.all(d <= np.ldexp(1.0, np.maximum(ex, -125) - 8)) and np.mean(d > 0) < 1e-3
    # control: an interleaved blocking (16 gate, then the same 16 up) differs
    I = wg.shape[1]
    mix = np.concatenate([np.r_[16 * b:16 * b + 16, I + 16 * b:I + 16 * b + 16] for b in range(I // 16)])
    e = int(re[0]); sel = np.nonzero(re == e)[0][:64]
    g, u = fwd["g"][sel], fwd["u"][sel]
    dAp = layer.qd(dY[sel]) @ layer.qd(wd[e].T).T
    s = 1.0 / (1.0 + np.exp(-g))
    dA = w[sel, None] * dAp
    P = bf16.round_rne(np.concatenate([dA * u * s * (1.0 + g * (1.0 - s)), dA * g * s], axis=1))
    WP = np.concatenate([wg[e], wu[e]], axis=0)
    alt = bf16.round_rne(layer.qd(P[:, mix]) @ layer.qd(WP[mix].T).T)
    assert np.mean(alt != ref["dX"][sel]) > 0.05


def test_sampled_mxfp8_backward_helper_matches_full_oracle():
    inp = workloads.make_expert_share("small")
    m = layer.backward_share_mxfp8(inp)
    rows = np.array([0, 7, 500, 999])
    pairs = [(0, 3), (2, 255), (3, 0)]
    s = layer.backward_share_mxfp8_sampled(inp, rows, pairs, pairs)
    assert np.allclose(s["dX"], m["dX"][rows], rtol=1e-12, atol=1e-12)
    assert np.allclose(s["d_row_w"], m["d_row_w"][rows], rtol=1e-12, atol=1e-12)
    for n, (e, i) in enumerate(pairs):
        assert np.allclose(s["dW_gate"][n], m["dW_gate"][e, i], rtol=1e-10, atol=1e-12)
        assert np.allclose(s["dW_up"][n], m["dW_up"][e, i], rtol=1e-10, atol=1e-12)
        assert np.allclose(s["dW_down"][n], m["dW_down"][e, :, i], rtol=1e-10, atol=1e-12)


def _q_blocks(v):
    """Quantise-dequantise a 1-D vector in consecutive blocks of 32 (loop)."""
    out = np.empty(len(v))
    for b0 in range(0, len(v), 32):
        c, s = mxfp8.quantize(np.asarray(v[b0:b0 + 32], dtype=np.float64)[None, :])
        out[b0:b0 + 32] = mxfp8.dequantize(c, s)[0]
    return out


def test_mxfp8_backward_brute_force_micro():
    """dX and the router-weight gradient of a few rows by plain loops: every
    GEMM operand cut into 32-blocks along that GEMM's contraction by hand."""
    inp = workloads.make_expert_share("micro")
    ref = layer.backward_share_mxfp8(inp)
    fwd = layer.forward_share_mxfp8(inp)
    R, H = inp["x"].shape
    E, I, _ = inp["w_gate"].shape
    wg = bf16.decode(inp["w_gate"]); wu = bf16.decode(inp["w_up"]); wd = bf16.decode(inp["w_down"])
    for r in (0, 17, R - 1):
        e = int(inp["row_expert"][r]); w = float(inp["row_w"][r])
        dyq = _q_blocks(bf16.decode(inp["dY"][r]))                       # along h
        g, u = fwd["g"][r], fwd["u"][r]
        dg = np.zeros(I); du = np.zeros(I); dw = 0.0
        for i in range(I):
            col = _q_blocks(wd[e][:, i])                                   # W_d column i along h
            dap = sum(dyq[h] * col[h] for h in range(H))
            s = 1.0 / (1.0 + np.exp(-g[i]))
            dw += dap * (g[i] * s * u[i])
            dg[i] = bf16.round_rne(np.array([w * dap * u[i] * s * (1.0 + g[i] * (1.0 - s))]))[0]
            du[i] = bf16.round_rne(np.array([w * dap * g[i] * s]))[0]
        # contraction over the I gate features, then the I up features: the
        # blocks of 32 are cut from dg and du each on their own, and from each
        # weight column's gate part and up part
        pq = np.concatenate([_q_blocks(dg), _q_blocks(du)])
        dx = np.zeros(H)
        for h in range(H):
            colq = np.concatenate([_q_blocks(wg[e][:, h]), _q_blocks(wu[e][:, h])])
            dx[h] = sum(pq[c] * colq[c] for c in range(2 * I))
        dx = bf16.round_rne(dx)
        assert np.isclose(dw, ref["d_row_w"][r], rtol=1e-10, atol=1e-12)
        assert np.allclose(dx, ref["dX"][r], rtol=0, atol=0) or \
            np.max(np.abs(dx - ref["dX"][r]) / np.maximum(np.abs(ref["dX"][r]), 1e-30)) <= 2 ** -8


def _beyond(got, ref, allow):
    """Largest excess of |got - ref| over one bf16 ulp (at the larger of the
    two magnitudes) plus allow."""
    _, e = np.frexp(np.maximum(np.abs(got), np.abs(ref)))
    return np.max(np.maximum(np.abs(got - ref) - np.ldexp(1.0, np.maximum(e, -125) - 8) - allow, 0.0))


def test_dx_within_decision_allowance_when_dact_changes_slightly(monkeypatch):
    """dg, du come from a GEMM output, so another correct evaluation decides
    some of their E4M3 codes differently: with dA' changed by a relative
    2^-15 (near what the device shows; clipped at 2^-13), dX leaves
    6e-2 * RMS of the oracle in places, yet every element stays within one
    bf16 ulp plus the oracle's dX_allow; without the allowance it does not."""
    inp = workloads.make_expert_share("small8")
    fwd = layer.forward_share_mxfp8(inp)
    ref = layer.backward_share_mxfp8(inp, fwd, allow=True)
    orig = layer._dact_mxfp8
    rng = np.random.default_rng(0)

    def perturbed(dYq, wdTq, g, u, w):
        dAp = orig(dYq, wdTq, g, u, w)[0]
        dAp = dAp * (1.0 + 2.0 ** -15 * np.clip(rng.standard_normal(dAp.shape), -4.0, 4.0))
        a = layer.silu(g) * u
        s = layer.sigmoid(g)
        dA = w[:, None] * dAp
        dgx = dA * u * s * (1.0 + g * (1.0 - s))
        dux = dA * layer.silu(g)
        return dAp, a, np.einsum("ri,ri->r", dAp, a), bf16.round_rne(dgx), bf16.round_rne(dux), dgx, dux

    monkeypatch.setattr(layer, "_dact_mxfp8", perturbed)
    alt = layer.backward_share_mxfp8(inp, fwd)
    monkeypatch.undo()
    r = ref["dX"]
    rms = np.sqrt(np.mean(r ** 2))
    assert _beyond(alt["dX"], r, 0.0) > 0.06 * rms                # flips exceed the plain bound
    assert _beyond(alt["dX"], r, ref["dX_allow"]) == 0.0             # and the allowance covers them
    # not a blanket widening: most elements keep (nearly) the plain bound
    assert np.quantile(ref["dX_allow"], 0.9) < 0.01 * rms


def test_out_within_decision_allowance_when_a_changes_slightly():
    """The forward's a = silu(g) u is a GEMM output quantised to MXFP8: a
    changed by a relative 2^-15 (clipped at 2^-13) moves out_rows by more than
    6e-2 * RMS in places, but within one bf16 ulp plus out_allow everywhere."""
    inp = workloads.make_expert_share("small8")
    ref = layer.forward_share_mxfp8(inp, allow=True)
    rng = np.random.default_rng(1)
    qw = layer.quantized_weights(inp)
    wd = mxfp8.dequantize(*qw["down"])
    a = layer.silu(ref["g"]) * ref["u"]
    a = a * (1.0 + 2.0 ** -15 * np.clip(rng.standard_normal(a.shape), -4.0, 4.0))
    aq = layer.qd(bf16.round_rne(a))
    re = inp["row_expert"]
    y = np.zeros_like(ref["y"])
    for e in range(wd.shape[0]):
        sel = np.nonzero(re == e)[0]
        y[sel] = aq[sel] @ wd[e].T
    alt = bf16.round_rne(inp["row_w"][:, None].astype(np.float64) * y)
    r = ref["out"]
    rms = np.sqrt(np.mean(r ** 2))
    assert _beyond(alt, r, 0.0) > 0.06 * rms
    assert _beyond(alt, r, ref["out_allow"]) == 0.0
    assert np.quantile(ref["out_allow"], 0.9) < 0.01 * rms


def test_qd_spread_bounds_every_reachable_value():
    """qd_spread against brute force: random values (some on E4M3 code
    boundaries, some blocks with their largest element at a power of two)
    moved within rel, element by element, all at once to either end, and at
    random; every result lies within the spread.  rel = 0 gives 0."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 128))
    # exact E4M3 midpoints at the block scale (bf16 values), and amax at 2^k
    v[:8, ::7] = (1.0 + 1.0 / 16.0) * 2.0 ** rng.integers(-3, 3, v[:8, ::7].shape)
    v[8:16, 0] = 2.0; v[8:16, 1:32] = np.clip(v[8:16, 1:32], -1.9, 1.9)
    v[16:24, 0] = 2.0 * (1.0 - 2.0 ** -9)
    rel = 2.0 ** -9
    assert np.all(layer.qd_spread(v, 0.0) == 0.0)
    sp = layer.qd_spread(v, rel)
    ref = layer.qd(bf16.round_rne(v))
    assert np.mean(sp > 0) > 0.01
    tries = [v * (1 - rel), v * (1 + rel)]
    tries += [v * (1 + rel * rng.uniform(-1, 1, v.shape)) for _ in range(20)]
    tries += [v * (1 + rel * rng.choice([-1.0, 1.0], v.shape)) for _ in range(20)]
    for t in tries:
        d = np.abs(layer.qd(bf16.round_rne(t)) - ref)
        assert np.all(d <= sp), np.max(d - sp)


# ------------------------------------------------------ full layer, MXFP8 --
def _full(name="tiny", **over):
    import dataclasses
    sh = workloads.FULL_LAYER[name]
    return workloads.make_full_layer(dataclasses.replace(sh, **over) if over else sh)


def _identity_quantiser(monkeypatch):
    monkeypatch.setattr(mxfp8, "quantize", lambda v: (np.asarray(v, dtype=np.float64), None))
    monkeypatch.setattr(mxfp8, "dequantize", lambda c, s: c)


@pytest.mark.parametrize("renorm", [0, 1])
def test_full_layer_identity_quantiser_gives_the_bf16_layer(monkeypatch, renorm):
    """With Q = identity the MXFP8 full layer is the bf16 full layer (pinned by
    autograd and finite differences), forward and backward with the router."""
    inp = _full(renorm=renorm, bias_var=0.5)
    _identity_quantiser(monkeypatch)
    mf = layer.forward_full_mxfp8(inp)
    mb = layer.backward_full_mxfp8(inp, fwd=mf)
    monkeypatch.undo()
    bf = layer.forward_full(inp)
    bb = layer.backward_full(inp)
    assert np.array_equal(mf["topk_idx"], bf["topk_idx"])
    assert np.allclose(mf["out_exact"], bf["out_exact"], rtol=1e-11, atol=1e-12)
    for k in ("dW_gate", "dW_up", "dW_down", "d_topk_w", "dz", "dW_router", "d_bias"):
        assert np.allclose(mb[k], bb[k], rtol=1e-10, atol=1e-12), k
    d = np.abs(mb["dX"] - bb["dX"])
    _, e = np.frexp(np.abs(bb["dX"]))
    assert np.all(d <= np.ldexp(1.0, np.maximum(e, -125) - 8)) and np.mean(d > 0) < 1e-3


def test_full_layer_scaling_one_token_dy_scales_only_that_token():
    """dY enters linearly and every quantised operand derived from it is
    blocked along its own row, so a power-of-two factor on one token's dY
    scales exactly that token's dX, d_topk_w and logit gradient."""
    inp = dict(_full(renorm=1, bias_var=0.5))
    fwd = layer.forward_full_mxfp8(inp)
    base = layer.backward_full_mxfp8(inp, fwd=fwd)
    t = 77
    dY = bf16.decode(inp["dY"]).copy()
    dY[t] *= 0.25
    inp["dY"] = bf16.encode(dY)
    m = layer.backward_full_mxfp8(inp, fwd=fwd)
    for k in ("dX", "d_topk_w", "dz"):
        assert np.array_equal(m[k][t], 0.25 * base[k][t]), k
        others = np.arange(base[k].shape[0]) != t
        assert np.array_equal(m[k][others], base[k][others]), k


def test_full_layer_mxfp8_within_e4m3_error_of_bf16():
    inp = _full()
    mf = layer.forward_full_mxfp8(inp)
    mb = layer.backward_full_mxfp8(inp, fwd=mf)
    bf = layer.forward_full(inp)
    bb = layer.backward_full(inp)
    assert 5e-3 < np.linalg.norm(mf["out_exact"] - bf["out_exact"]) / np.linalg.norm(bf["out_exact"]) < 0.12
    for k in ("dX", "dW_gate", "dW_up", "dW_down", "d_topk_w", "dW_router", "d_bias"):
        rel = np.linalg.norm(mb[k] - bb[k]) / np.linalg.norm(bb[k])
        assert 5e-3 < rel < 0.12, (k, rel)
