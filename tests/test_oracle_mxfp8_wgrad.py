"""Pins for the oracle's MXFP8 weight gradients (CPU only).

The pages leave the blocking of these GEMMs open; the reading pinned here:
both operands of dW_gate, dW_up and dW_down are quantised along the
contraction (the expert's rows), 32 rows per block, and a block never holds
rows of two minibatches (each minibatch's last block is completed with zero
rows).  Independent references: blocks cut by hand and quantised through the
element quantiser (pinned exhaustively in test_oracle_codecs); the identity
quantiser, which must give back the bf16 weight gradients (pinned by
autograd and finite differences elsewhere), so every routed row enters
exactly once; exact linearity in a power-of-two factor on one minibatch's
loss gradient, which holds only if no block mixes minibatches; and E4M3's
error against the bf16 gradients.
"""
import numpy as np
import pytest

import workloads
from oracle import bf16, layer, mxfp8


def _q_col_blocks(col):
    """Quantise-dequantise a column in consecutive 32-row blocks by hand, the
    last block completed with zeros."""
    n = len(col)
    out = np.empty(n)
    for b0 in range(0, n, 32):
        blk = np.zeros(32)
        m = min(32, n - b0)
        blk[:m] = col[b0:b0 + m]
        c, s = mxfp8.quantize(blk[None, :])
        out[b0:b0 + m] = mxfp8.dequantize(c, s)[0, :m]
    return out


def test_qd_rows_is_per_column_blocks_of_32_rows():
    rng = np.random.default_rng(11)
    n, C = 70, 6                                 # 3 blocks, the last with 6 rows
    v = rng.standard_normal((n, C)) * np.exp2(rng.integers(-20, 20, size=C))
    v[40:64, 2] = 0.0                            # a block that is zero but for its first 8 rows
    v[64:, 3] = 0.0                              # an all-zero (padded) block
    v[5, 4] = 1e4                                # one outlier dominating its block's scale
    got = layer.qd_rows(v)
    for c in range(C):
        assert np.array_equal(got[:, c], _q_col_blocks(v[:, c])), c
    assert np.all(got[64:, 3] == 0.0)
    # rows outside the outlier's block keep their own, finer scale
    assert np.array_equal(got[32:, 4], _q_col_blocks(v[32:, 4]))


def test_wgrad_mx_brute_force():
    """C[m, n] = sum over minibatches b of sum over the segment's rows of the
    hand-quantised columns of A and B, by loops."""
    rng = np.random.default_rng(12)
    n, M, N = 90, 3, 4
    A = rng.standard_normal((n, M))
    B = rng.standard_normal((n, N)) * 3.0
    mbs = np.repeat([0, 1, 3], [37, 20, 33])     # segments of 37, 20 and 33 rows
    got = layer.wgrad_mx(A, B, mbs)
    ref = np.zeros((M, N))
    for b in (0, 1, 3):
        rows = np.nonzero(mbs == b)[0]
        qa = [_q_col_blocks(A[rows, m]) for m in range(M)]
        qb = [_q_col_blocks(B[rows, q]) for q in range(N)]
        for m in range(M):
            for q in range(N):
                ref[m, q] += sum(qa[m][i] * qb[q][i] for i in range(len(rows)))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def _identity_quantiser(monkeypatch):
    monkeypatch.setattr(mxfp8, "quantize", lambda v: (np.asarray(v, dtype=np.float64), None))
    monkeypatch.setattr(mxfp8, "dequantize", lambda c, s: c)


@pytest.mark.parametrize("mb", [0, 256, 100])
def test_identity_quantiser_gives_the_bf16_weight_gradients(monkeypatch, mb):
    inp = workloads.make_expert_share("small")
    _identity_quantiser(monkeypatch)
    m = layer.backward_share_mxfp8(inp, wgrad_mx_mb=mb)
    b = layer.backward_share_mxfp8(inp)
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert np.allclose(m[k], b[k], rtol=1e-11, atol=1e-12), k
    assert np.array_equal(m["dX"], b["dX"]) and np.array_equal(m["d_row_w"], b["d_row_w"])


def test_full_layer_identity_quantiser_gives_the_bf16_weight_gradients(monkeypatch):
    sh = workloads.FULL_LAYER["tiny"]
    inp = workloads.make_full_layer("tiny")
    _identity_quantiser(monkeypatch)
    m = layer.backward_full_mxfp8(inp, wgrad_mx_mb=64 * sh.k)
    b = layer.backward_full_mxfp8(inp)
    for k in ("dW_gate", "dW_up", "dW_down", "dW_router", "d_bias"):
        assert np.allclose(m[k], b[k], rtol=1e-11, atol=1e-12), k


def _scaled_minibatch(inp, mb, b, f):
    out = dict(inp)
    dY = bf16.decode(inp["dY"]).copy()
    dY[b * mb:(b + 1) * mb] *= f
    out["dY"] = bf16.encode(dY)
    return out


def test_weight_gradients_are_linear_in_one_minibatchs_dy():
    """A power-of-two factor f on the loss gradient of minibatch 1 scales dY,
    dA', dg, du (bf16 rounding and E8M0/E4M3 quantisation commute with it) of
    exactly that minibatch's rows, so each weight gradient is C0 + f C1 with
    C1 the minibatch's own part -- as long as no MX block holds rows of two
    minibatches (a shared block scale would couple them)."""
    inp = workloads.make_expert_share("small")
    mb = 300
    fwd = layer.forward_share_mxfp8(inp)
    res = {f: layer.backward_share_mxfp8(_scaled_minibatch(inp, mb, 1, f), fwd=fwd, wgrad_mx_mb=mb)
           for f in (1.0, 4.0, 0.5)}
    for k in ("dW_gate", "dW_up", "dW_down"):
        c1 = (res[4.0][k] - res[1.0][k]) / 3.0
        c0 = res[1.0][k] - c1
        assert np.allclose(res[0.5][k], c0 + 0.5 * c1, rtol=1e-9, atol=1e-9 * np.abs(res[1.0][k]).max()), k
        assert np.abs(c1).max() > 0.1 * np.abs(res[1.0][k]).max(), k


def test_linearity_fails_when_blocks_cross_minibatches():
    """Control for the test above: blocking over the expert's rows as a whole
    (one minibatch) while scaling rows of the middle of it breaks linearity."""
    inp = workloads.make_expert_share("small")
    mb = 300
    fwd = layer.forward_share_mxfp8(inp)
    res = {f: layer.backward_share_mxfp8(_scaled_minibatch(inp, mb, 1, f), fwd=fwd, wgrad_mx_mb=0)
           for f in (1.0, 4.0, 0.5)}
    k = "dW_down"
    c1 = (res[4.0][k] - res[1.0][k]) / 3.0
    c0 = res[1.0][k] - c1
    assert not np.allclose(res[0.5][k], c0 + 0.5 * c1, rtol=1e-9, atol=1e-9 * np.abs(res[1.0][k]).max())


@pytest.mark.parametrize("mb", [0, 256])
def test_mx_weight_gradients_within_e4m3_error_of_bf16(mb):
    inp = workloads.make_expert_share("small")
    m = layer.backward_share_mxfp8(inp, wgrad_mx_mb=mb)
    b = layer.backward_share(inp)
    for k in ("dW_gate", "dW_up", "dW_down"):
        rel = np.linalg.norm(m[k] - b[k]) / np.linalg.norm(b[k])
        assert 5e-3 < rel < 0.12, (k, rel)


def test_sampled_helper_matches_full_oracle_with_mx_weight_gradients():
    inp = workloads.make_expert_share("small")
    mb = 256
    m = layer.backward_share_mxfp8(inp, wgrad_mx_mb=mb)
    pairs = [(0, 3), (2, 255), (3, 0)]
    s = layer.backward_share_mxfp8_sampled(inp, [0, 999], pairs, pairs, wgrad_mx_mb=mb)
    for n, (e, i) in enumerate(pairs):
        assert np.allclose(s["dW_gate"][n], m["dW_gate"][e, i], rtol=1e-10, atol=1e-12)
        assert np.allclose(s["dW_up"][n], m["dW_up"][e, i], rtol=1e-10, atol=1e-12)
        assert np.allclose(s["dW_down"][n], m["dW_down"][e, :, i], rtol=1e-10, atol=1e-12)


def test_weight_gradient_allowance_bounds_perturbed_gemm_outputs():
    """dg, du and w a are GEMM outputs rounded to bf16 and then quantised: a
    relative change within DECISION_REL of their exact values may flip codes
    and block scales, and the result must stay within the oracle's allowance
    (which is zero where no decision can change)."""
    inp = workloads.make_expert_share("small")
    mb = 256
    fwd = layer.forward_share_mxfp8(inp)
    ref = layer.backward_share_mxfp8(inp, fwd, allow=True, wgrad_mx_mb=mb)
    rng = np.random.default_rng(21)
    re = inp["row_expert"]
    w = inp["row_w"].astype(np.float64)
    wd = bf16.decode(inp["w_down"])
    x = bf16.decode(inp["x"]); dY = bf16.decode(inp["dY"])
    e = 1
    sel = np.nonzero(re == e)[0]
    _, a, _, dg, du, dgx, dux = layer._dact_mxfp8(layer.qd(dY[sel]), layer.qd(wd[e].T), fwd["g"][sel],
                                                  fwd["u"][sel], w[sel])
    mbs = layer.minibatch_of(sel, re.size, mb)
    for trial in range(3):
        f = 1.0 + layer.DECISION_REL * rng.uniform(-1, 1, size=dgx.shape)
        dgp = bf16.round_rne(dgx * f)
        got = layer.wgrad_mx(dgp, x[sel], mbs)
        d = np.abs(got - ref["dW_gate"][e])
        assert np.all(d <= ref["dW_gate_allow"][e] * (1 + 1e-9) + 1e-12), trial
        wax = w[sel, None] * a * (1.0 + layer.DECISION_REL * rng.uniform(-1, 1, size=a.shape))
        got = layer.wgrad_mx(dY[sel], bf16.round_rne(wax), mbs)
        d = np.abs(got - ref["dW_down"][e])
        assert np.all(d <= ref["dW_down_allow"][e] * (1 + 1e-9) + 1e-12), trial
    # the allowance is a small share of the gradient's size
    r = np.sqrt(np.mean(ref["dW_gate"] ** 2))
    assert np.mean(ref["dW_gate_allow"]) < 0.05 * r


def test_sampled_helper_allowances_match_full_oracle():
    inp = workloads.make_expert_share("small")
    mb = 256
    m = layer.backward_share_mxfp8(inp, allow=True, wgrad_mx_mb=mb)
    pairs = [(0, 3), (3, 0)]
    s = layer.backward_share_mxfp8_sampled(inp, [0], pairs, pairs, wgrad_mx_mb=mb)
    for n, (e, i) in enumerate(pairs):
        assert np.allclose(s["dW_gate_allow"][n], m["dW_gate_allow"][e, i], rtol=1e-10, atol=1e-14)
        assert np.allclose(s["dW_up_allow"][n], m["dW_up_allow"][e, i], rtol=1e-10, atol=1e-14)
        assert np.allclose(s["dW_down_allow"][n], m["dW_down_allow"][e, :, i], rtol=1e-10, atol=1e-14)


def test_segments_of_whole_blocks_equal_one_segment():
    """When every minibatch segment holds a multiple of 32 rows, the blocks
    of the per-segment rule are exactly the consecutive 32-row blocks of the
    expert's rows, so the result equals blocking the rows as one segment."""
    rng = np.random.default_rng(13)
    n = 32 * 7
    A = rng.standard_normal((n, 5)) * np.exp2(rng.integers(-6, 6, size=(n, 1)))
    B = rng.standard_normal((n, 3))
    mbs = np.repeat([0, 2, 3, 5], [64, 32, 96, 32])
    assert np.array_equal(layer.wgrad_mx(A, B, mbs), layer.wgrad_mx(A, B, np.zeros(n, dtype=int)))
    # and a segment that is not a whole number of blocks changes the result
    mbs2 = np.repeat([0, 1], [40, n - 40])
    assert not np.array_equal(layer.wgrad_mx(A, B, mbs2), layer.wgrad_mx(A, B, np.zeros(n, dtype=int)))


def test_full_layer_weight_gradients_linear_in_one_minibatchs_dy():
    """Full layer (routed rows r = t k + j, minibatches of whole tokens): a
    power-of-two factor on the loss gradient of the tokens of one minibatch
    scales exactly that minibatch's part of every weight gradient."""
    sh = workloads.FULL_LAYER["tiny"]
    inp = workloads.make_full_layer("tiny")
    mb_tok = 64
    mb = mb_tok * sh.k
    fwd = layer.forward_full_mxfp8(inp)
    res = {}
    for f in (1.0, 4.0, 0.5):
        sub = dict(inp)
        dY = bf16.decode(inp["dY"]).copy()
        dY[mb_tok:2 * mb_tok] *= f
        sub["dY"] = bf16.encode(dY)
        res[f] = layer.backward_full_mxfp8(sub, fwd=fwd, wgrad_mx_mb=mb)
    for k in ("dW_gate", "dW_up", "dW_down"):
        c1 = (res[4.0][k] - res[1.0][k]) / 3.0
        c0 = res[1.0][k] - c1
        assert np.allclose(res[0.5][k], c0 + 0.5 * c1, rtol=1e-9, atol=1e-9 * np.abs(res[1.0][k]).max()), k
        assert np.abs(c1).max() > 0.05 * np.abs(res[1.0][k]).max(), k
