"""Pins for the oracle's full-layer backward with the router backward (CPU only).

Independent references: torch autograd in fp64 through a full-layer forward
written here (routing choice held fixed, since it is piecewise constant),
central finite differences of the same forward, checked first against the
oracle's own forward; and the invariants of the softmax Jacobian (rows of
dz sum to zero; renorm=1 gives no gradient to unchosen experts; with k = E
the renormalised and the full softmax coincide, so both branches agree).
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from oracle import bf16, layer, route


def _inputs(name, renorm=None, **over):
    sh = workloads.FULL_LAYER[name]
    if over:
        sh = dataclasses.replace(sh, **over)
    inp = workloads.make_full_layer(sh)
    rn = sh.renorm if renorm is None else renorm
    return inp, rn


def _forward_t(inp, idx, renorm, x, wr, b, wg, wu, wd):
    """Full layer in torch fp64 with the routing choice idx held fixed."""
    T, H = x.shape
    k = idx.shape[1]
    z = x @ wr.T + b
    it = torch.from_numpy(idx.astype(np.int64))
    if renorm:
        w = torch.softmax(torch.gather(z, 1, it), dim=1)
    else:
        w = torch.gather(torch.softmax(z, dim=1), 1, it)
    re = it.reshape(-1)
    xr = x.repeat_interleave(k, dim=0)
    g = torch.einsum("rh,rih->ri", xr, wg[re])
    u = torch.einsum("rh,rih->ri", xr, wu[re])
    y = torch.einsum("ri,rhi->rh", torch.nn.functional.silu(g) * u, wd[re])
    out = (w.reshape(-1, 1) * y).reshape(T, k, H).sum(dim=1)
    return out, w


def _leaves(inp):
    E = inp["w_router"].shape[0]
    bias = inp["bias"] if inp["bias"] is not None else np.zeros(E, dtype=np.float32)
    vals = {"x": bf16.decode(inp["x"]), "wr": bf16.decode(inp["w_router"]),
            "b": bias.astype(np.float64), "wg": bf16.decode(inp["w_gate"]),
            "wu": bf16.decode(inp["w_up"]), "wd": bf16.decode(inp["w_down"])}
    return vals


GRAD_KEY = {"x": "dX", "wr": "dW_router", "b": "d_bias", "wg": "dW_gate", "wu": "dW_up", "wd": "dW_down"}


@pytest.mark.parametrize("name,renorm", [("micro", 1), ("micro", 0), ("tiny", 0), ("tiny", 1)])
def test_full_backward_matches_torch_autograd(name, renorm):
    inp, rn = _inputs(name, renorm)
    g = layer.backward_full(inp, renorm=rn, bf16_mode=False)
    vals = _leaves(inp)
    ts = {n: torch.tensor(v, requires_grad=True) for n, v in vals.items()}
    out, w = _forward_t(inp, g["topk_idx"], rn, **ts)
    w.retain_grad()
    # the forward written here is the oracle's forward (up to its fp32 logits)
    ref = layer.forward_full(inp, renorm=rn, bf16_mode=False)
    assert np.allclose(out.detach().numpy(), ref["out_exact"], rtol=1e-5, atol=1e-6)
    (out * torch.from_numpy(bf16.decode(inp["dY"]))).sum().backward()
    for n, t in ts.items():
        a, b = g[GRAD_KEY[n]], t.grad.numpy()
        scale = max(np.abs(b).max(), 1e-30)
        assert np.abs(a - b).max() <= 2e-5 * scale, (n, np.abs(a - b).max() / scale)
    dw = w.grad.numpy()
    assert np.abs(g["d_topk_w"] - dw).max() <= 2e-5 * np.abs(dw).max()


@pytest.mark.parametrize("renorm", [1, 0])
def test_full_backward_finite_differences(renorm):
    inp, rn = _inputs("micro", renorm)
    g = layer.backward_full(inp, renorm=rn, bf16_mode=False)
    vals = _leaves(inp)
    dY = torch.from_numpy(bf16.decode(inp["dY"]))
    idx = g["topk_idx"]

    def loss(v):
        with torch.no_grad():
            out, _ = _forward_t(inp, idx, rn, **{n: torch.from_numpy(a) for n, a in v.items()})
        return float((out * dY).sum())

    rng = np.random.default_rng(5)
    eps = 1e-5
    for n, v in vals.items():
        d = rng.standard_normal(v.shape)
        plus = dict(vals); plus[n] = v + eps * d
        minus = dict(vals); minus[n] = v - eps * d
        fd = (loss(plus) - loss(minus)) / (2 * eps)
        an = float(np.sum(g[GRAD_KEY[n]] * d))
        assert abs(fd - an) <= 2e-5 * max(1.0, abs(an)), (n, fd, an)


@pytest.mark.parametrize("name,renorm", [("micro", 1), ("micro", 0), ("tiny", 0)])
def test_router_logit_grad_invariants(name, renorm):
    inp, rn = _inputs(name, renorm)
    g = layer.backward_full(inp, renorm=rn, bf16_mode=False)
    dz = g["dz"]
    # softmax is shift invariant: every row of its Jacobian sums to zero
    assert np.abs(dz.sum(axis=1)).max() <= 1e-12 * max(1.0, np.abs(dz).max())
    assert abs(g["d_bias"].sum()) <= 1e-11 * max(1.0, np.abs(g["d_bias"]).max())
    if rn:
        mask = np.zeros_like(dz, dtype=bool)
        np.put_along_axis(mask, g["topk_idx"].astype(np.int64), True, axis=1)
        assert np.all(dz[~mask] == 0)
    else:
        assert np.all(dz != 0)          # every expert's logit gets a gradient
    x = bf16.decode(inp["x"])
    assert np.allclose(g["dW_router"], dz.T @ x, rtol=1e-12, atol=1e-14)


def test_renorm_branches_agree_when_all_experts_chosen():
    inp, _ = _inputs("micro", k=4)             # E = 4 = k
    g1 = layer.backward_full(inp, renorm=1, bf16_mode=False)
    g0 = layer.backward_full(inp, renorm=0, bf16_mode=False)
    assert np.array_equal(g1["topk_idx"], g0["topk_idx"])
    for key in ("dz", "dW_router", "d_bias", "dX", "d_topk_w"):
        assert np.allclose(g1[key], g0[key], rtol=1e-6, atol=1e-9), key


def test_expert_part_is_share_backward_of_the_expanded_rows():
    """Without the router term, dX is the fixed-order k-sum of the expert
    share backward's dX rows for the rows r = t*k + j, dY_rows[r] = dY[t]."""
    inp, rn = _inputs("micro")
    sh = inp["shape"]
    g = layer.backward_full(inp, bf16_mode=False, router=False)
    share = {"x": np.repeat(inp["x"], sh.k, axis=0), "w_gate": inp["w_gate"], "w_up": inp["w_up"],
             "w_down": inp["w_down"], "row_expert": g["topk_idx"].reshape(-1),
             "row_w": g["topk_w"].reshape(-1), "dY": np.repeat(inp["dY"], sh.k, axis=0)}
    s = layer.backward_share(share, bf16_mode=False)
    assert np.allclose(g["dX"], s["dX"].reshape(sh.T, sh.k, sh.H).sum(axis=1), rtol=1e-12, atol=1e-13)
    for key in ("dW_gate", "dW_up", "dW_down"):
        assert np.allclose(g[key], s[key], rtol=1e-12, atol=1e-13)
    assert np.allclose(g["d_topk_w"].reshape(-1), s["d_row_w"], rtol=1e-12, atol=1e-13)


def test_full_backward_bf16_mode_close_to_exact():
    inp, rn = _inputs("tiny")
    b = layer.backward_full(inp, bf16_mode=True)
    x = layer.backward_full(inp, bf16_mode=False)
    for key in ("dX", "dW_gate", "dW_up", "dW_down", "d_topk_w", "dW_router", "d_bias"):
        rel = np.linalg.norm(b[key] - x[key]) / np.linalg.norm(x[key])
        assert rel < 4e-3, (key, rel)
    assert np.array_equal(bf16.round_rne(b["dX"]), b["dX"])


@pytest.mark.parametrize("renorm", [0, 1])
def test_sampled_full_backward_helpers_match_full_oracle(renorm):
    inp, rn = _inputs("tiny", renorm, bias_var=0.5)
    g = layer.backward_full(inp, renorm=rn)
    idx, w, z = g["topk_idx"], g["topk_w"], g["logits"]
    toks = np.array([0, 17, 255])
    t = layer.backward_full_tokens(inp, idx, w, z, toks, rn)
    assert np.allclose(t["dX"], g["dX"][toks], rtol=1e-12, atol=1e-12)
    assert np.allclose(t["d_topk_w"], g["d_topk_w"][toks], rtol=1e-12, atol=1e-13)
    assert np.allclose(t["dz"], g["dz"][toks], rtol=1e-12, atol=1e-13)
    for e in (0, 5):
        x = layer.backward_full_expert(inp, idx, w, z, e, rn)
        for key in ("dW_gate", "dW_up", "dW_down", "dW_router"):
            assert np.allclose(x[key], g[key][e], rtol=1e-10, atol=1e-12), key
        assert np.isclose(x["d_bias"], g["d_bias"][e], rtol=1e-10, atol=1e-13)
