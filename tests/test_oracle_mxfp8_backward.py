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


def test_gu_order_is_the_packed_interleave():
    I = 64
    o = layer.gu_order(I)
    assert sorted(o.tolist()) == list(range(2 * I))
    # each MX block of 32 holds 16 gate features and the same 16 up features
    for b in range(2 * I // 32):
        blk = o[32 * b:32 * b + 32]
        assert np.array_equal(blk[16:] - I, blk[:16])


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
        # contraction over features in groups of 16 gate then 16 up
        p = []; wrows = []
        for b in range(I // 16):
            p += list(dg[16 * b:16 * b + 16]) + list(du[16 * b:16 * b + 16])
            wrows += [wg[e][i] for i in range(16 * b, 16 * b + 16)] + [wu[e][i] for i in range(16 * b, 16 * b + 16)]
        pq = _q_blocks(np.array(p))
        wrows = np.array(wrows)                                            # [2I, H]
        dx = np.zeros(H)
        for h in range(H):
            colq = _q_blocks(wrows[:, h])                                  # along the feature order
            dx[h] = sum(pq[c] * colq[c] for c in range(2 * I))
        dx = bf16.round_rne(dx)
        assert np.isclose(dw, ref["d_row_w"][r], rtol=1e-10, atol=1e-12)
        assert np.allclose(dx, ref["dX"][r], rtol=0, atol=0) or \
            np.max(np.abs(dx - ref["dX"][r]) / np.maximum(np.abs(ref["dX"][r]), 1e-30)) <= 2 ** -8


def test_mxfp8_backward_dx_bound_covers_one_flipped_code():
    """The MXFP8 backward's dX tolerance: its GEMM's A operand (dg, du) is
    quantised from a GEMM output, so a 2^-16 relative change of dA' (far below
    fp32 accumulation differences over hundreds of terms) already flips E4M3
    codes and moves dX beyond the forward's 6e-2 * RMS; the bound used for it
    must cover that and stay well under an error of the operand itself."""
    from tests.helpers import MXFP8_BWD_DX_TOL, MXFP8_TOL
    inp = workloads.make_expert_share("small8")
    fwd = layer.forward_share_mxfp8(inp)
    ref = layer.backward_share_mxfp8(inp, fwd)
    orig = layer._dact_mxfp8
    rng = np.random.default_rng(0)

    def perturbed(dYq, wdTq, g, u, w):
        dAp, a, dw, _, _ = orig(dYq, wdTq, g, u, w)
        dAp = dAp * (1.0 + 2.0 ** -16 * rng.standard_normal(dAp.shape))
        s = 1.0 / (1.0 + np.exp(-g))
        dA = w[:, None] * dAp
        return dAp, a, dw, bf16.round_rne(dA * u * s * (1.0 + g * (1.0 - s))), bf16.round_rne(dA * g * s)

    layer._dact_mxfp8 = perturbed
    try:
        alt = layer.backward_share_mxfp8(inp, fwd)
    finally:
        layer._dact_mxfp8 = orig
    r = ref["dX"]
    _, e = np.frexp(np.abs(r))
    beyond = np.max(np.maximum(np.abs(alt["dX"] - r) - np.ldexp(1.0, np.maximum(e, -125) - 8), 0.0))
    ratio = beyond / np.sqrt(np.mean(r ** 2))
    assert MXFP8_TOL < ratio < MXFP8_BWD_DX_TOL, ratio
