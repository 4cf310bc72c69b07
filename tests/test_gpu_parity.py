"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer results (routing indices, schedule tables, ring contents, MXFP8 codes
and scales) must match bit for bit; bf16 outputs and gradients within
max|err| <= 2e-2 * RMS(oracle tensor), MXFP8 outputs within 6e-2 * RMS of the
MXFP8-emulating oracle.  At full workload sizes the oracle evaluates sampled
rows / columns one by one (each output row depends only on its own inputs).
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from oracle import bf16, layer, mxfp8, route, schedule
from tests.helpers import (BF16_TOL, MXFP8_TOL, ROUTER_W_ATOL, assert_close, dev, host_bf16,
                           rms, say)

pytestmark = pytest.mark.gpu

from mixture_experts_layer_device_amd import binding as B  # noqa: E402
from mixture_experts_layer_device_amd.layer import MoELayer  # noqa: E402

_CACHE = {}


def share_inputs(name):
    if name not in _CACHE:
        _CACHE[name] = workloads.make_expert_share(name)
    return _CACHE[name]


def full_inputs(name):
    key = "full:" + name
    if key not in _CACHE:
        _CACHE[key] = workloads.make_full_layer(name)
    return _CACHE[key]


def sync():
    torch.cuda.synchronize()


def sched_tables(L, R, E, MB):
    nb = -(-R // MB) if R else 0
    t = {
        "counts": L.table("counts", E), "offsets": L.table("offsets", E + 1),
        "mb_counts": L.table("mb_counts", nb * E), "mb_offsets": L.table("mb_offsets", nb * (E + 1)),
        "sorted_pos": L.table("sorted_pos", R), "inv": L.table("inv", nb * MB),
        "mb_items": L.table("mb_items", nb + 1),
    }
    t["items"] = L.table("items", 4 * L.query("item_capacity"))
    sync()
    return {k: v.cpu().numpy() for k, v in t.items()}


def check_schedule(L, re, E, MB, ring_rows):
    R = len(re)
    ref = schedule.build(re, E, MB, ring_rows, L.query("tile_m"))
    got = sched_tables(L, R, E, MB)
    for k in ("counts", "offsets", "sorted_pos", "inv", "mb_items"):
        assert np.array_equal(got[k], getattr(ref, k).reshape(-1)), k
    assert np.array_equal(got["mb_counts"], ref.mb_counts.reshape(-1))
    assert np.array_equal(got["mb_offsets"], ref.mb_offsets.reshape(-1))
    n_items = len(ref.items)
    assert np.array_equal(got["items"][: 4 * n_items], ref.items.reshape(-1))
    return ref


# ----------------------------------------------------------------- schedule --
SCHED_CASES = [
    # (name, R, E, MB, seed)
    ("zipf4_mb4096", 16384, 4, 4096, 2),
    ("zipf8_mb4096", 24576, 8, 4096, 4),
    ("uniform128_one_mb", 32768, 128, 32768, 1),
    ("ragged37", 1000, 37, 300, 7),
    ("single_row", 1, 3, 1, 8),
    # (b, e) tables past the scan's LDS copy (10 minibatches x 1025 > 8192)
    ("e1024_ten_mbs", 20000, 1024, 2048, 9),
    # runs of more than 16 chunks per scan lane (256 chunks of 256 rows)
    ("mb65536_long_runs", 70000, 16, 65536, 10),
]


@pytest.mark.parametrize("case", SCHED_CASES, ids=[c[0] for c in SCHED_CASES])
def test_schedule_bit_exact(case):
    name, R, E, MB, seed = case
    say(f"[schedule] {name} R={R} E={E} MB={MB}")
    rng = np.random.default_rng(seed)
    re = rng.choice(E, size=R, p=workloads.zipf_local_weights(E, 1.2)).astype(np.int32)
    L = MoELayer(H=256, I=128, E=E, k=1, max_rows=R, minibatch_rows=MB, ring_bytes=2 * MB * 512)
    L.build_schedule(dev(re), R)
    sync()
    check_schedule(L, re, E, MB, L.query("ring_rows"))
    assert L.device_error() == 0
    L.close()


def test_schedule_empty_and_invalid_ids():
    say("[schedule] empty input and out-of-range ids")
    L = MoELayer(H=256, I=128, E=4, k=1, max_rows=64, minibatch_rows=16)
    L.build_schedule(None, 0)
    sync()
    assert L.table("mb_items", 1).cpu().item() == 0
    re = np.array([0, 5, 1, -1, 3, 3, 0, 2, 9, 1], dtype=np.int32)
    L.build_schedule(dev(re), len(re))
    sync()
    check_schedule(L, re, 4, 16, L.query("ring_rows"))
    assert L.device_error() == B.MK_DEVERR_EXPERT_RANGE
    L.build_schedule(dev(np.zeros(4, np.int32)), 4)      # the next schedule clears the error word
    sync()
    assert L.device_error() == 0
    L.close()


def test_schedule_capacity_overflow_flags_and_returns():
    say("[schedule] work-table overflow")
    R, E = 4096, 16
    re = np.arange(R, dtype=np.int32) % E
    L = MoELayer(H=256, I=128, E=E, k=1, max_rows=R, minibatch_rows=256, capacity_mult=0.1)
    L.build_schedule(dev(re), R)
    sync()
    assert L.device_error() & B.MK_DEVERR_SCHED_OVERFLOW
    L.close()


# -------------------------------------------------------------------- route --
@pytest.mark.parametrize("name", ["tiny", "full"])
def test_route_bit_exact(name):
    inp = full_inputs(name)
    sh = inp["shape"]
    say(f"[route] {name} T={sh.T} H={sh.H} E={sh.E} k={sh.k} renorm={sh.renorm}")
    x = bf16.decode(inp["x"]).astype(np.float32)
    wr = bf16.decode(inp["w_router"]).astype(np.float32)
    idx_ref, w_ref, _ = route.route(x, wr, inp["bias"], sh.k, sh.renorm)
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm)
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    idx, w = L.route(dev(inp["x"]), dev(inp["w_router"]), bias, sh.T)
    sync()
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    err = float(np.max(np.abs(w.cpu().numpy().astype(np.float64) - w_ref)))
    say(f"  router weights max|err| = {err:.2e}")
    assert err <= ROUTER_W_ATOL
    L.close()


@pytest.mark.parametrize("T,H,E,k,renorm,bias_var", [(1000, 512, 37, 3, 1, 0.5), (77, 256, 200, 5, 0, 0.0)],
                         ids=["T1000_E37", "T77_E200"])
def test_route_bit_exact_ragged(T, H, E, k, renorm, bias_var):
    """Token counts off the router's 16-token blocks, an expert count off its
    4-expert groups (E=37) and a second, partial 128-expert chunk (E=200)."""
    sh = dataclasses.replace(workloads.FULL_LAYER["tiny"], T=T, H=H, E=E, k=k, renorm=renorm, bias_var=bias_var,
                             seed=41 + E)
    inp = workloads.make_full_layer(sh)
    say(f"[route] ragged T={T} H={H} E={E} k={k} renorm={renorm}")
    x = bf16.decode(inp["x"]).astype(np.float32)
    wr = bf16.decode(inp["w_router"]).astype(np.float32)
    idx_ref, w_ref, _ = route.route(x, wr, inp["bias"], k, renorm)
    L = MoELayer(H=H, I=sh.I, E=E, k=k, max_rows=T * k, renorm=renorm)
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    idx, w = L.route(dev(inp["x"]), dev(inp["w_router"]), bias, T)
    sync()
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    err = float(np.max(np.abs(w.cpu().numpy().astype(np.float64) - w_ref)))
    say(f"  router weights max|err| = {err:.2e}")
    assert err <= ROUTER_W_ATOL
    L.close()


# -------------------------------------------------------------- quantiser --
def test_mxfp8_quantize_bit_exact():
    say("[mxfp8_quantize] all finite bf16 patterns + wide-range random rows")
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    allbits = allbits[((allbits >> 7) & 0xFF) != 0xFF]
    rng = np.random.default_rng(5)
    allbits = rng.permutation(allbits)
    allbits = allbits[: (len(allbits) // 256) * 256].reshape(-1, 256)
    wide = workloads.bf16_bits((rng.standard_normal((512, 1024)) * np.exp(rng.standard_normal((512, 32)).repeat(32, 1)
                                * 6)).astype(np.float32))
    special = np.zeros((4, 256), dtype=np.uint16)
    special[1, :] = 0x8000                                # -0 block
    special[2, :32] = 0x0001                              # smallest subnormal
    special[3, :] = 0x7F7F                                # largest finite
    for bits in (allbits, wide, special):
        rows, K = bits.shape
        codes = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
        B.mk_mxfp8_quantize(dev(bits), rows, K, codes, scales, torch.cuda.current_stream())
        sync()
        rc, rs = mxfp8.quantize(bf16.decode(bits))
        assert np.array_equal(scales.cpu().numpy(), rs)
        assert np.array_equal(codes.cpu().numpy(), rc)


def test_mxfp8_quantize_every_value_at_every_scale():
    """Every finite bf16 magnitude (both signs) quantised at every block scale
    that can hold it: a power-of-two anchor 2^fl in slot 0 fixes the block's
    largest magnitude and so its E8M0 scale, the other 31 slots run through
    all patterns no larger than the anchor.  fl spans the whole bf16 range
    (-133 .. 127), which covers every scale code the encoder can produce."""
    say("[mxfp8_quantize] every (value, scale) pair, 8.6M elements")
    mag = np.arange(0x7F80, dtype=np.uint32)
    blocks = []
    for fl in range(-133, 128):
        a = (fl + 127) << 7 if fl >= -126 else 1 << (fl + 133)
        vals = mag[mag <= a]
        vals = np.concatenate([vals, vals | 0x8000]).astype(np.uint16)
        n = (len(vals) + 30) // 31
        body = np.resize(vals, n * 31).reshape(n, 31)
        blocks.append(np.concatenate([np.full((n, 1), a, dtype=np.uint16), body], axis=1).reshape(-1))
    bits = np.concatenate(blocks)
    bits = np.concatenate([bits, np.zeros((-len(bits)) % 256, dtype=np.uint16)]).reshape(-1, 256)
    rows, K = bits.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
    B.mk_mxfp8_quantize(dev(bits), rows, K, codes, scales, torch.cuda.current_stream())
    sync()
    rc, rs = mxfp8.quantize(bf16.decode(bits))
    got_s, got_c = scales.cpu().numpy(), codes.cpu().numpy()
    assert np.array_equal(got_s, rs)
    bad = np.argwhere(got_c != rc)
    assert len(bad) == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}: bits {bits[tuple(bad[0])]:#06x} got {got_c[tuple(bad[0])]:#04x} want {rc[tuple(bad[0])]:#04x}"


# ------------------------------------------------------------ full layer --
def run_full_layer(inp, precision="bf16", MB=0, ring_bytes=256 << 20):
    sh = inp["shape"]
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, precision=precision,
                 minibatch_rows=MB, ring_bytes=ring_bytes)
    x = dev(inp["x"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    idx, w = L.route(x, dev(inp["w_router"]), bias, sh.T)
    L.build_schedule(idx.view(-1), sh.R)
    out = L.forward(B.MK_FULL_LAYER, x, w.view(-1), packed, sh.T)
    sync()
    return L, idx, w, out


def test_forward_full_layer_tiny():
    inp = full_inputs("tiny")
    say("[forward full layer] tiny T=256 H=256 I=128 E=8 k=2, one minibatch and a wrapping ring")
    ref = layer.forward_full(inp)
    for MB, ring in ((0, 256 << 20), (128, 2 * 128 * 512)):
        L, idx, w, out = run_full_layer(inp, MB=MB, ring_bytes=ring)
        assert np.array_equal(idx.cpu().numpy(), ref["topk_idx"])
        assert_close(host_bf16(out), ref["out_exact"], BF16_TOL, f"out (MB={MB})", bf16_out=True)
        if MB:
            # ring after the forward: the last two minibatches, bit-exact
            s = schedule.build(ref["row_expert"], 8, MB, L.query("ring_rows"), L.query("tile_m"))
            ring_ref, written = layer.ring_contents(s, inp["x"], np.arange(512) // 2)
            ring = L.table("ring", L.query("ring_rows") * 256 // 2).cpu().numpy().view(np.uint16)
            ring = ring.reshape(-1, 256)
            assert written.all() and np.array_equal(ring, ring_ref)
        L.close()


def test_forward_full_layer_full_sampled():
    inp = full_inputs("full")
    sh = inp["shape"]
    say("[forward full layer] T=4096 H=2048 I=768 E=128 k=8 renorm, biased router")
    x = bf16.decode(inp["x"]).astype(np.float32)
    idx_ref, w_ref, _ = route.route(x, bf16.decode(inp["w_router"]).astype(np.float32), inp["bias"], sh.k,
                                    sh.renorm)
    L, idx, w, out = run_full_layer(inp)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    toks = np.random.default_rng(0).choice(sh.T, 96, replace=False)
    ref = layer.forward_full_tokens(inp, idx_ref, w_ref, toks, exact=True)
    assert_close(host_bf16(out)[toks], ref, BF16_TOL, "out (96 sampled tokens)", bf16_out=True)
    L.close()


# ---------------------------------------------------------- expert share --
def run_share(inp, precision="bf16", MB=0, ring_bytes=256 << 20, fwd_ctx=False, backward=False, wgrad_mxfp8=False):
    sh = inp["shape"]
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=8, max_rows=sh.R, precision=precision, minibatch_rows=MB,
                 ring_bytes=ring_bytes, enable_backward=backward, wgrad_mxfp8=wgrad_mxfp8)
    x = dev(inp["x"])
    row_w = dev(inp["row_w"])
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=backward)
    L.build_schedule(dev(inp["row_expert"]), sh.R)
    ctx = L.new_fwd_ctx() if fwd_ctx else None
    out = L.forward(B.MK_EXPERT_SHARE, x, row_w, packed, sh.R, fwd_ctx=ctx)
    sync()
    return L, out, (x, row_w, packed, ctx)


@pytest.mark.parametrize("MB,ring_mbs", [(0, None), (256, 2)], ids=["one_mb", "mb256_ring2"])
def test_forward_share_bf16_small(MB, ring_mbs):
    inp = share_inputs("small")
    sh = inp["shape"]
    say(f"[forward share bf16] small R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB}")
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * 2 * sh.H
    L, out, _ = run_share(inp, MB=MB, ring_bytes=ring)
    ref = layer.forward_share(inp)["out_exact"]
    assert_close(host_bf16(out), ref, BF16_TOL, "out_rows", bf16_out=True)
    L.close()


def test_forward_share_bf16_ep64_sampled():
    inp = share_inputs("ep64_fwd")
    sh = inp["shape"]
    say(f"[forward share bf16] EP=64 share R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB=4096, 256 MiB ring")
    L, out, _ = run_share(inp, MB=4096)
    rows = np.sort(np.random.default_rng(1).choice(sh.R, 64, replace=False))
    ref = layer.forward_share_rows(inp, rows, exact=True)
    assert_close(host_bf16(out)[rows], ref, BF16_TOL, "out_rows (64 sampled rows)", bf16_out=True)
    # ring holds every row, bit-exact, at sorted_pos mod ring_rows
    sp = L.table("sorted_pos", sh.R).cpu().numpy()
    ring = L.table("ring", L.query("ring_rows") * sh.H // 2).cpu().numpy().view(np.uint16).reshape(-1, sh.H)
    s = schedule.build(inp["row_expert"], sh.E, 4096, L.query("ring_rows"), L.query("tile_m"))
    assert np.array_equal(sp, s.sorted_pos)
    assert np.array_equal(ring[s.ring_pos], inp["x"])
    L.close()


@pytest.mark.parametrize("MB,ring_mbs", [(0, None), (256, 2)], ids=["one_mb", "mb256_ring2"])
def test_forward_share_mxfp8_small(MB, ring_mbs):
    inp = share_inputs("small")
    sh = inp["shape"]
    say(f"[forward share mxfp8] small R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB}")
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * (sh.H + sh.H // 32)
    L, out, _ = run_share(inp, precision="mxfp8", MB=MB, ring_bytes=ring)
    ref = layer.forward_share_mxfp8(inp, allow=True)
    assert_close(host_bf16(out), ref["out_exact"], MXFP8_TOL, "out_rows", bf16_out=True, allow=ref["out_allow"])
    if not MB:
        rr = L.query("ring_rows")
        raw = L.table("ring", rr * (sh.H + sh.H // 32) // 4).cpu().numpy().view(np.uint8)
        codes = raw[: rr * sh.H].reshape(rr, sh.H)
        scales = raw[rr * sh.H:].reshape(rr, sh.H // 32)
        sp = L.table("sorted_pos", sh.R).cpu().numpy()
        assert np.array_equal(codes[sp], ref["x_codes"])
        assert np.array_equal(scales[sp], ref["x_scales"])
    L.close()


def test_forward_share_mxfp8_ep64_sampled():
    inp = share_inputs("ep64_fwd")
    sh = inp["shape"]
    say(f"[forward share mxfp8] EP=64 share R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB=4096")
    L, out, _ = run_share(inp, precision="mxfp8", MB=4096)
    rows = np.sort(np.random.default_rng(2).choice(sh.R, 48, replace=False))
    ref, allow = layer.forward_share_mxfp8_rows(inp, rows, allow=True, exact=True)
    assert_close(host_bf16(out)[rows], ref, MXFP8_TOL, "out_rows (48 sampled rows)", bf16_out=True, allow=allow)
    rr = L.query("ring_rows")
    raw = L.table("ring", rr * (sh.H + sh.H // 32) // 4).cpu().numpy().view(np.uint8)
    codes = raw[: rr * sh.H].reshape(rr, sh.H)
    scales = raw[rr * sh.H:].reshape(rr, sh.H // 32)
    sp = L.table("sorted_pos", sh.R).cpu().numpy()
    xc, xs = mxfp8.quantize(bf16.decode(inp["x"][rows]))
    assert np.array_equal(codes[sp[rows]], xc)
    assert np.array_equal(scales[sp[rows]], xs)
    L.close()


# ---------------------------------------------------------------- backward --
def run_backward(inp, MB=0, ring_bytes=256 << 20):
    sh = inp["shape"]
    L, out, (x, row_w, packed, ctx) = run_share(inp, MB=MB, ring_bytes=ring_bytes, fwd_ctx=True, backward=True)
    g = L.backward(ctx, x, row_w, packed, dev(inp["dY"]), sh.R)
    sync()
    return L, out, g


@pytest.mark.parametrize("MB,ring_mbs", [(0, None), (256, 2)], ids=["one_mb", "mb256_ring2_replay"])
def test_backward_small8(MB, ring_mbs):
    inp = share_inputs("small8")
    sh = inp["shape"]
    say(f"[backward] small8 R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB}")
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * 2 * sh.H
    L, out, g = run_backward(inp, MB=MB, ring_bytes=ring)
    # dg, du and w a are GEMM outputs rounded to bf16: each element also gets
    # the oracle's allowance for roundings another correct evaluation decides
    # the other way
    ref = layer.backward_share(inp, allow=True)
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], BF16_TOL, "dX", bf16_out=True, allow=ref["dX_allow"])
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert_close(g[k].cpu().numpy(), ref[k], BF16_TOL, k, allow=ref[k + "_allow"])
    assert_close(g["d_row_w"].cpu().numpy(), ref["d_row_w"], BF16_TOL, "d_row_w")
    L.close()


def test_backward_ep_bwd_sampled():
    inp = share_inputs("ep_bwd")
    sh = inp["shape"]
    say(f"[backward] EP share R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB=4096, 256 MiB ring (wraps: replay)")
    L, out, g = run_backward(inp, MB=4096)
    assert L.query("ring_rows") < sh.R
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(sh.R, 32, replace=False))
    pairs = [(0, 5), (3, 2047), (7, 1000)]
    ref = layer.backward_share_sampled(inp, rows, pairs, pairs)
    assert_close(host_bf16(g["dX"])[rows], ref["dX_exact"], BF16_TOL, "dX (32 sampled rows)", bf16_out=True)
    assert_close(g["d_row_w"].cpu().numpy()[rows], ref["d_row_w"], BF16_TOL, "d_row_w (32 sampled rows)")
    gate = np.stack([g["dW_gate"][e, i].cpu().numpy() for e, i in pairs])
    up = np.stack([g["dW_up"][e, i].cpu().numpy() for e, i in pairs])
    down = np.stack([g["dW_down"][e, :, i].cpu().numpy() for e, i in pairs])
    assert_close(gate, ref["dW_gate"], BF16_TOL, "dW_gate (3 rows)")
    assert_close(up, ref["dW_up"], BF16_TOL, "dW_up (3 rows)")
    assert_close(down, ref["dW_down"], BF16_TOL, "dW_down (3 columns)")
    L.close()


# ----------------------------------------------------- MXFP8 backward --
def run_backward_mxfp8(inp, MB=0, ring_bytes=256 << 20, wgrad_mxfp8=False):
    sh = inp["shape"]
    L, out, (x, row_w, packed, ctx) = run_share(inp, precision="mxfp8", MB=MB, ring_bytes=ring_bytes, fwd_ctx=True,
                                               backward=True, wgrad_mxfp8=wgrad_mxfp8)
    g = L.backward(ctx, x, row_w, packed, dev(inp["dY"]), sh.R)
    sync()
    return L, out, g


@pytest.mark.parametrize("MB,ring_mbs", [(0, None), (256, 2)], ids=["one_mb", "mb256_ring2"])
def test_backward_mxfp8_small8(MB, ring_mbs):
    inp = share_inputs("small8")
    sh = inp["shape"]
    say(f"[backward mxfp8] small8 R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB}")
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * (sh.H + sh.H // 32)
    L, out, g = run_backward_mxfp8(inp, MB=MB, ring_bytes=ring)
    fwd = layer.forward_share_mxfp8(inp, allow=True)
    ref = layer.backward_share_mxfp8(inp, fwd, allow=True)
    assert_close(host_bf16(out), fwd["out_exact"], MXFP8_TOL, "out (mxfp8 forward)", bf16_out=True,
                 allow=fwd["out_allow"])
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], MXFP8_TOL, "dX", bf16_out=True, allow=ref["dX_allow"])
    for k in ("dW_gate", "dW_up", "dW_down", "d_row_w"):
        assert_close(g[k].cpu().numpy(), ref[k], MXFP8_TOL, k)
    L.close()


def test_backward_mxfp8_ep_bwd_sampled():
    inp = share_inputs("ep_bwd")
    sh = inp["shape"]
    say(f"[backward mxfp8] EP share R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB=4096, sampled from experts 3 and 7")
    L, out, g = run_backward_mxfp8(inp, MB=4096)
    rng = np.random.default_rng(5)
    re = inp["row_expert"]
    rows = np.sort(np.concatenate([rng.choice(np.nonzero(re == e)[0], 12, replace=False) for e in (3, 7)]))
    pairs = [(3, 5), (7, 2047), (7, 1000)]
    ref = layer.backward_share_mxfp8_sampled(inp, rows, pairs, pairs)
    assert_close(host_bf16(g["dX"])[rows], ref["dX_exact"], MXFP8_TOL, "dX (24 sampled rows)", bf16_out=True,
                 allow=ref["dX_allow"])
    assert_close(g["d_row_w"].cpu().numpy()[rows], ref["d_row_w"], MXFP8_TOL, "d_row_w (24 sampled rows)")
    gate = np.stack([g["dW_gate"][e, i].cpu().numpy() for e, i in pairs])
    up = np.stack([g["dW_up"][e, i].cpu().numpy() for e, i in pairs])
    down = np.stack([g["dW_down"][e, :, i].cpu().numpy() for e, i in pairs])
    assert_close(gate, ref["dW_gate"], MXFP8_TOL, "dW_gate (3 rows)")
    assert_close(up, ref["dW_up"], MXFP8_TOL, "dW_up (3 rows)")
    assert_close(down, ref["dW_down"], MXFP8_TOL, "dW_down (3 columns)")
    L.close()


# ------------------------------------- MXFP8 weight gradients --
@pytest.mark.parametrize("MB,ring_mbs", [(0, None), (256, 2), (200, 3)], ids=["one_mb", "mb256_ring2", "mb200_ragged"])
def test_backward_mxfp8_wgrad_small8(MB, ring_mbs):
    """All six backward GEMMs on MXFP8 operands; the weight gradients' operands
    quantised along the rows in 32-row blocks of one minibatch (MB = 200:
    segments of every length, blocks padded at each minibatch's end)."""
    inp = share_inputs("small8")
    sh = inp["shape"]
    say(f"[backward mxfp8, MXFP8 weight gradients] small8 R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={MB}")
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * (sh.H + sh.H // 32)
    L, out, g = run_backward_mxfp8(inp, MB=MB, ring_bytes=ring, wgrad_mxfp8=True)
    fwd = layer.forward_share_mxfp8(inp, allow=True)
    ref = layer.backward_share_mxfp8(inp, fwd, allow=True, wgrad_mx_mb=MB)
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], MXFP8_TOL, "dX", bf16_out=True, allow=ref["dX_allow"])
    assert_close(g["d_row_w"].cpu().numpy(), ref["d_row_w"], MXFP8_TOL, "d_row_w")
    # dg, du and w a are GEMM outputs quantised again: each element also gets the
    # oracle's allowance for the E4M3 codes another correct evaluation may decide
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert_close(g[k].cpu().numpy(), ref[k], MXFP8_TOL, k, allow=ref[k + "_allow"])
    # the bf16 weight gradients lie E4M3's error away: the MXFP8 path really ran
    bw = layer.backward_share_mxfp8(inp, fwd)
    rel = np.linalg.norm(g["dW_down"].double().cpu().numpy() - bw["dW_down"]) / np.linalg.norm(bw["dW_down"])
    assert rel > 5e-3, rel
    assert L.device_error() == 0
    L.close()


def test_backward_mxfp8_wgrad_absent_experts():
    """Experts 2 and 5 get no rows and expert 6 only rows of the last
    minibatch: their K ranges are empty or one segment, and the gradients of
    the absent experts are exactly zero."""
    inp = dict(share_inputs("small8"))
    sh = inp["shape"]
    re = inp["row_expert"].copy()
    re[(re == 2) | (re == 5)] = 0
    MB = 256
    last = (np.arange(sh.R) // MB) == (sh.R - 1) // MB
    re[(re == 6) & ~last] = 1
    inp["row_expert"] = re
    say(f"[backward mxfp8, MXFP8 weight gradients] small8 with experts 2, 5 absent, 6 in the last minibatch only, "
        f"MB={MB}")
    L, out, g = run_backward_mxfp8(inp, MB=MB, wgrad_mxfp8=True)
    fwd = layer.forward_share_mxfp8(inp, allow=True)
    ref = layer.backward_share_mxfp8(inp, fwd, allow=True, wgrad_mx_mb=MB)
    for k in ("dW_gate", "dW_up", "dW_down"):
        got = g[k].cpu().numpy()
        assert not np.any(got[[2, 5]]), k
        assert_close(got, ref[k], MXFP8_TOL, k, allow=ref[k + "_allow"])
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], MXFP8_TOL, "dX", bf16_out=True, allow=ref["dX_allow"])
    assert L.device_error() == 0
    L.close()


def test_backward_mxfp8_wgrad_ep_bwd_sampled():
    inp = share_inputs("ep_bwd")
    sh = inp["shape"]
    say(f"[backward mxfp8, MXFP8 weight gradients] EP share R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB=4096, "
        f"sampled from experts 0, 3 and 7")
    L, out, g = run_backward_mxfp8(inp, MB=4096, wgrad_mxfp8=True)
    pairs = [(0, 17), (3, 5), (7, 2047), (7, 1000)]
    ref = layer.backward_share_mxfp8_sampled(inp, [0], pairs, pairs, wgrad_mx_mb=4096)
    gate = np.stack([g["dW_gate"][e, i].cpu().numpy() for e, i in pairs])
    up = np.stack([g["dW_up"][e, i].cpu().numpy() for e, i in pairs])
    down = np.stack([g["dW_down"][e, :, i].cpu().numpy() for e, i in pairs])
    assert_close(gate, ref["dW_gate"], MXFP8_TOL, "dW_gate (4 rows)", allow=ref["dW_gate_allow"])
    assert_close(up, ref["dW_up"], MXFP8_TOL, "dW_up (4 rows)", allow=ref["dW_up_allow"])
    assert_close(down, ref["dW_down"], MXFP8_TOL, "dW_down (4 columns)", allow=ref["dW_down_allow"])
    L.close()


def test_backward_mxfp8_wgrad_repeatable():
    inp = share_inputs("small8")
    sh = inp["shape"]
    say("[determinism] small8 MXFP8 weight gradients: two runs bitwise equal")
    ring = 2 * 256 * (sh.H + sh.H // 32)
    L1, _, g1 = run_backward_mxfp8(inp, MB=256, ring_bytes=ring, wgrad_mxfp8=True)
    L2, _, g2 = run_backward_mxfp8(inp, MB=256, ring_bytes=ring, wgrad_mxfp8=True)
    for k in ("dW_gate", "dW_up", "dW_down", "dX", "d_row_w"):
        assert torch.equal(g1[k], g2[k]), k
    L1.close()
    L2.close()


# ------------------------------------------------- full-layer backward --
def full_variant(name, **over):
    key = "full:" + name + repr(sorted(over.items()))
    if key not in _CACHE:
        sh = workloads.FULL_LAYER[name]
        _CACHE[key] = workloads.make_full_layer(dataclasses.replace(sh, **over) if over else sh)
    return _CACHE[key]


def run_full_backward(inp, MB=0, ring_bytes=256 << 20, router=True, precision="bf16", wgrad_mxfp8=False):
    sh = inp["shape"]
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, minibatch_rows=MB,
                 ring_bytes=ring_bytes, enable_backward=True, precision=precision, wgrad_mxfp8=wgrad_mxfp8)
    x = dev(inp["x"])
    wr = dev(inp["w_router"])
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
    idx, w = L.route(x, wr, bias, sh.T)
    L.build_schedule(idx.view(-1), sh.R)
    ctx = L.new_fwd_ctx()
    out = L.forward(B.MK_FULL_LAYER, x, w.view(-1), packed, sh.T, fwd_ctx=ctx)
    dY = dev(inp["dY"])
    if router:
        g = L.backward_layer(ctx, x, wr, bias, idx, w, packed, dY, sh.T)
    else:
        g = L.backward(ctx, x, w.view(-1), packed, dY, sh.R, mode=B.MK_FULL_LAYER)
    sync()
    return L, idx, w, out, g, (x, wr, bias, packed, ctx, dY)


# the backward tiles I by 256: the tiny shape with I = 256
FULL_BWD_CASES = [("renorm0", {"I": 256}), ("renorm1_bias", {"I": 256, "renorm": 1, "bias_var": 0.5})]


@pytest.mark.parametrize("MB,ring_mbs", [(0, None), (128, 2)], ids=["one_mb", "mb128_ring2_replay"])
@pytest.mark.parametrize("case", FULL_BWD_CASES, ids=[c[0] for c in FULL_BWD_CASES])
def test_backward_full_layer_tiny(case, MB, ring_mbs):
    inp = full_variant("tiny", **case[1])
    sh = inp["shape"]
    say(f"[backward full layer] tiny {case[0]} T={sh.T} H={sh.H} I={sh.I} E={sh.E} k={sh.k} "
        f"renorm={sh.renorm} MB={MB}")
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * 2 * sh.H
    L, idx, w, out, g, (x, wr, bias, packed, ctx, dY) = run_full_backward(inp, MB=MB, ring_bytes=ring)
    ref = layer.backward_full(inp, allow=True)
    assert np.array_equal(idx.cpu().numpy(), ref["topk_idx"])
    if MB:
        assert L.query("ring_rows") < sh.R          # the walk replays evicted minibatches
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], BF16_TOL, "dX", bf16_out=True, allow=ref["dX_allow"])
    for key in ("dW_gate", "dW_up", "dW_down", "dW_router"):
        assert_close(g[key].cpu().numpy(), ref[key], BF16_TOL, key, allow=ref.get(key + "_allow"))
    assert_close(g["d_row_w"].cpu().numpy(), ref["d_topk_w"].reshape(-1), BF16_TOL, "d_topk_w")
    if bias is not None:
        assert_close(g["d_bias"].cpu().numpy(), ref["d_bias"], BF16_TOL, "d_bias")
    # the same call again on the same workspace: bitwise equal
    g2 = L.backward_layer(ctx, x, wr, bias, idx, w, packed, dY, sh.T)
    sync()
    for key, t in g.items():
        if t is not None:
            assert torch.equal(t, g2[key]), key
    L.close()


def test_backward_full_layer_router_external_tiny():
    inp = full_variant("tiny", I=256, renorm=1, bias_var=0.5)
    sh = inp["shape"]
    say("[backward full layer] tiny (I=256), router as an external input (mk_backward, MK_FULL_LAYER)")
    L, idx, w, out, g, _ = run_full_backward(inp, router=False)
    ref = layer.backward_full(inp, router=False, allow=True)
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], BF16_TOL, "dX (expert part)", bf16_out=True,
                 allow=ref["dX_allow"])
    assert_close(g["d_row_w"].cpu().numpy(), ref["d_topk_w"].reshape(-1), BF16_TOL, "d_topk_w")
    for key in ("dW_gate", "dW_up", "dW_down"):
        assert_close(g[key].cpu().numpy(), ref[key], BF16_TOL, key, allow=ref[key + "_allow"])
    L.close()


def test_backward_full_layer_full_sampled():
    inp = full_inputs("full")
    sh = inp["shape"]
    say(f"[backward full layer] T={sh.T} H={sh.H} I={sh.I} E={sh.E} k={sh.k} renorm={sh.renorm}, biased router")
    x = bf16.decode(inp["x"]).astype(np.float32)
    idx_ref, w_ref, z_ref = route.route(x, bf16.decode(inp["w_router"]).astype(np.float32), inp["bias"], sh.k,
                                        sh.renorm)
    L, idx, w, out, g, _ = run_full_backward(inp)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    toks = np.sort(np.random.default_rng(4).choice(sh.T, 48, replace=False))
    t = layer.backward_full_tokens(inp, idx_ref, w_ref, z_ref, toks, sh.renorm)
    assert_close(host_bf16(g["dX"])[toks], t["dX_exact"], BF16_TOL, "dX (48 sampled tokens)", bf16_out=True)
    assert_close(g["d_row_w"].cpu().numpy().reshape(sh.T, sh.k)[toks], t["d_topk_w"], BF16_TOL,
                 "d_topk_w (48 sampled tokens)")
    counts = np.bincount(idx_ref.reshape(-1), minlength=sh.E)
    order = np.argsort(counts, kind="stable")
    experts = [int(order[sh.E // 2]), int(order[3])]
    db_ref = []
    for e in experts:
        say(f"  expert {e}: {counts[e]} rows")
        r = layer.backward_full_expert(inp, idx_ref, w_ref, z_ref, e, sh.renorm)
        for key in ("dW_gate", "dW_up", "dW_down", "dW_router"):
            assert_close(g[key][e].cpu().numpy(), r[key], BF16_TOL, f"{key}[{e}]")
        db_ref.append(r["d_bias"])
    assert_close(g["d_bias"].cpu().numpy()[experts], np.array(db_ref), BF16_TOL, "d_bias (2 experts)")
    # every row of the softmax Jacobian sums to zero, so d_bias does too
    db = g["d_bias"].double().cpu().numpy()
    assert abs(db.sum()) <= 1e-4 * np.abs(db).sum()
    L.close()


@pytest.mark.parametrize("MB,ring_mbs", [(0, None), (128, 2), (64, 2)], ids=["one_mb", "mb128_ring2", "mb64_ring2"])
@pytest.mark.parametrize("case", FULL_BWD_CASES, ids=[c[0] for c in FULL_BWD_CASES])
def test_full_layer_mxfp8_tiny(case, MB, ring_mbs):
    """MXFP8 precision in full-layer mode: forward, then the backward with the
    router, against the oracle's MXFP8 full layer.  With the token rows
    fitting the ring (one_mb, mb128_ring2) GEMM1 reads the token rows' codes
    through the inverse map; with a ring of fewer rows than tokens
    (mb64_ring2) the routed rows are quantised into the ring minibatch by
    minibatch."""
    inp = full_variant("tiny", **case[1])
    sh = inp["shape"]
    say(f"[full layer mxfp8] tiny {case[0]} T={sh.T} H={sh.H} I={sh.I} E={sh.E} k={sh.k} "
        f"renorm={sh.renorm} MB={MB}")
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * (sh.H + sh.H // 32)
    L, idx, w, out, g, (x, wr, bias, packed, ctx, dY) = run_full_backward(inp, MB=MB, ring_bytes=ring,
                                                                          precision="mxfp8")
    fwd = layer.forward_full_mxfp8(inp, allow=True)
    ref = layer.backward_full_mxfp8(inp, fwd=fwd, allow=True)
    assert np.array_equal(idx.cpu().numpy(), ref["topk_idx"])
    if MB:
        assert L.query("ring_rows") < sh.R
    assert_close(host_bf16(out), fwd["out_exact"], MXFP8_TOL, "out", bf16_out=True, allow=fwd["out_allow"])
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], MXFP8_TOL, "dX", bf16_out=True, allow=ref["dX_allow"])
    for key in ("dW_gate", "dW_up", "dW_down", "dW_router"):
        assert_close(g[key].cpu().numpy(), ref[key], MXFP8_TOL, key)
    assert_close(g["d_row_w"].cpu().numpy(), ref["d_topk_w"].reshape(-1), MXFP8_TOL, "d_topk_w")
    if bias is not None:
        assert_close(g["d_bias"].cpu().numpy(), ref["d_bias"], MXFP8_TOL, "d_bias")
    L.close()


@pytest.mark.parametrize("MB,ring_mbs", [(0, None), (128, 2)], ids=["one_mb", "mb128_ring2"])
def test_full_layer_mxfp8_token_codes_in_the_ring(MB, ring_mbs):
    """MXFP8 full layer with the token rows fitting the ring: the forward
    quantises each token row once into the ring (a routed row's codes are its
    token's, the quantisation running along H) and GEMM1 reads them through
    the inverse map.  The ring's first T rows are the oracle quantiser's codes
    and scales of x, bit for bit, and the output is within the MXFP8 rule."""
    inp = full_variant("tiny")
    sh = inp["shape"]
    say(f"[full layer mxfp8] token codes in the ring: tiny T={sh.T} H={sh.H} E={sh.E} k={sh.k} MB={MB}")
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * (sh.H + sh.H // 32)
    L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, minibatch_rows=MB,
                 ring_bytes=ring, precision="mxfp8")
    x = dev(inp["x"])
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    packed = L.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
    idx, w = L.route(x, dev(inp["w_router"]), bias, sh.T)
    L.build_schedule(idx.view(-1), sh.R)
    out = L.forward(B.MK_FULL_LAYER, x, w.view(-1), packed, sh.T)
    rr = L.query("ring_rows")
    assert sh.T <= rr
    raw = L.table("ring", rr * (sh.H + sh.H // 32) // 4).cpu().numpy().view(np.uint8)
    codes = raw[: rr * sh.H].reshape(rr, sh.H)[: sh.T]
    scales = raw[rr * sh.H:].reshape(rr, sh.H // 32)[: sh.T]
    xc, xs = mxfp8.quantize(bf16.decode(inp["x"]))
    assert np.array_equal(codes, xc)
    assert np.array_equal(scales, xs)
    fwd = layer.forward_full_mxfp8(inp, allow=True)
    assert_close(host_bf16(out), fwd["out_exact"], MXFP8_TOL, "out", bf16_out=True, allow=fwd["out_allow"])
    assert L.device_error() == 0
    L.close()


@pytest.mark.parametrize("MB,ring_mbs", [(0, None), (128, 2)], ids=["one_mb", "mb128_ring2"])
def test_full_layer_mxfp8_wgrad_tiny(MB, ring_mbs):
    """Full layer in MXFP8 with MXFP8 weight gradients (x rows pulled again
    from the token rows for the gate/up gradient's operand)."""
    case = FULL_BWD_CASES[1]
    inp = full_variant("tiny", **case[1])
    sh = inp["shape"]
    say(f"[full layer mxfp8, MXFP8 weight gradients] tiny {case[0]} T={sh.T} H={sh.H} I={sh.I} E={sh.E} "
        f"k={sh.k} MB={MB}")
    ring = 256 << 20 if ring_mbs is None else ring_mbs * MB * (sh.H + sh.H // 32)
    L, idx, w, out, g, _ = run_full_backward(inp, MB=MB, ring_bytes=ring, precision="mxfp8", wgrad_mxfp8=True)
    fwd = layer.forward_full_mxfp8(inp, allow=True)
    ref = layer.backward_full_mxfp8(inp, fwd=fwd, allow=True, wgrad_mx_mb=MB)
    assert np.array_equal(idx.cpu().numpy(), ref["topk_idx"])
    assert_close(host_bf16(g["dX"]), ref["dX_exact"], MXFP8_TOL, "dX", bf16_out=True, allow=ref["dX_allow"])
    for key in ("dW_gate", "dW_up", "dW_down"):
        assert_close(g[key].cpu().numpy(), ref[key], MXFP8_TOL, key, allow=ref[key + "_allow"])
    assert_close(g["dW_router"].cpu().numpy(), ref["dW_router"], MXFP8_TOL, "dW_router")
    L.close()


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp8_wgrad"])
def test_empty_schedule_forward_and_backward(precision):
    """T = R = 0: route and forward launch nothing, every backward writes its
    weight gradients as zeros, and no device error is raised."""
    H, I, E, k = 256, 256, 8, 2
    say(f"[empty] {precision} R = 0: share and full-layer forward/backward, backward with the router")
    rng = np.random.default_rng(9)
    w = [dev(bf16.encode(0.05 * rng.standard_normal(s))) for s in ((E, I, H), (E, I, H), (E, H, I))]
    wr = dev(bf16.encode(0.05 * rng.standard_normal((E, H))))
    L = MoELayer(H=H, I=I, E=E, k=k, max_rows=512, precision=precision.split("_")[0], enable_backward=True,
                 wgrad_mxfp8=precision.endswith("_wgrad"))
    packed = L.prepare_weights(*w, for_backward=True)
    x = torch.empty((0, H), dtype=torch.int16, device="cuda")
    idx, tw = L.route(x, wr, None, 0)
    L.build_schedule(idx.view(-1), 0)
    ctx = L.new_fwd_ctx()

    def nan_grads():
        g = L._grads(0, 0)
        for key in ("dW_gate", "dW_up", "dW_down"):
            g[key].fill_(float("nan"))
        return g

    for mode in (B.MK_EXPERT_SHARE, B.MK_FULL_LAYER):
        L.forward(mode, x, tw.view(-1), packed, 0, fwd_ctx=ctx)
        g = L.backward(ctx, x, tw.view(-1), packed, x, 0, grads=nan_grads(), mode=mode)
        sync()
        for key in ("dW_gate", "dW_up", "dW_down"):
            assert torch.count_nonzero(g[key]).item() == 0, (mode, key)
    g = nan_grads()
    g["dW_router"] = torch.full((E, H), float("nan"), dtype=torch.float32, device="cuda")
    g["d_bias"] = torch.full((E,), float("nan"), dtype=torch.float32, device="cuda")
    bias = torch.zeros(E, dtype=torch.float32, device="cuda")
    g = L.backward_layer(ctx, x, wr, bias, idx, tw, packed, x, 0, grads=g)
    sync()
    for key in ("dW_gate", "dW_up", "dW_down", "dW_router", "d_bias"):
        assert torch.count_nonzero(g[key]).item() == 0, key
    assert L.device_error() == 0
    L.close()


# ----------------------------------------------------- determinism, errors --
def test_repeat_runs_bitwise_and_minibatch_invariance():
    inp = share_inputs("small8")
    sh = inp["shape"]
    say("[determinism] small8: repeated forward/backward, and MB / ring size invariance")
    L1, out1, g1 = run_backward(inp, MB=256, ring_bytes=2 * 256 * 2 * sh.H)
    # repeat on the same workspace
    x = dev(inp["x"]); row_w = dev(inp["row_w"])
    packed = L1.prepare_weights(dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]), for_backward=True)
    L1.build_schedule(dev(inp["row_expert"]), sh.R)
    ctx = L1.new_fwd_ctx()
    out1b = L1.forward(B.MK_EXPERT_SHARE, x, row_w, packed, sh.R, fwd_ctx=ctx)
    g1b = L1.backward(ctx, x, row_w, packed, dev(inp["dY"]), sh.R)
    sync()
    assert torch.equal(out1, out1b)
    for k in g1:
        assert torch.equal(g1[k], g1b[k]), k
    # another minibatch size and ring: out, dX and d_row_w bitwise equal
    L2, out2, g2 = run_backward(inp, MB=512, ring_bytes=256 << 20)
    assert torch.equal(out1, out2)
    assert torch.equal(g1["dX"], g2["dX"])
    assert torch.equal(g1["d_row_w"], g2["d_row_w"])
    L1.close()
    L2.close()


def test_invalid_expert_rows_are_zero_and_flagged():
    inp = dict(share_inputs("small"))
    sh = inp["shape"]
    say("[errors] out-of-range expert ids in an expert-share forward")
    re = inp["row_expert"].copy()
    bad = np.array([3, 400, 999])
    re[bad] = [-1, 4, 1 << 20]
    inp["row_expert"] = re
    L, out, _ = run_share(inp)
    assert L.device_error() == B.MK_DEVERR_EXPERT_RANGE
    got = host_bf16(out)
    assert np.all(got[bad] == 0)
    ref = layer.forward_share(inp)["out_exact"]
    assert_close(got, ref, BF16_TOL, "out_rows with dropped rows", bf16_out=True)
    L.close()
