"""Pins for the oracle's router, schedule and sizing rule (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import workloads
from oracle import bf16, route, schedule, sizing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_two_wave_floor_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "two_wave_floor.json")))
    assert sizing.two_wave_rows(g["H"], g["I"], g["n_cu"], g["tile_m"], g["tile_n"]) == g["rows"]


def test_two_wave_floor_other_cases():
    # min(2I, H) picks the narrower GEMM: with H < 2I the down GEMM's N = H decides
    assert sizing.two_wave_rows(2048, 2048, 256, 128, 256) == 2 * 256 * 128 * 256 // 2048
    assert sizing.two_wave_rows(7168, 2048, 256, 256, 256) == 8192


@pytest.mark.parametrize("name", ["micro", "tiny"])
def test_router_brute_force(name):
    inp = workloads.make_full_layer(name)
    sh = inp["shape"]
    x = bf16.decode(inp["x"]); w = bf16.decode(inp["w_router"])
    idx, wts, z = route.route(x.astype(np.float32), w.astype(np.float32), inp["bias"], sh.k, sh.renorm)
    # fp32 pinned-order sums stay within H ulps of the exact (fsum) logits
    for t in range(0, sh.T, max(1, sh.T // 16)):
        for e in range(sh.E):
            exact = math.fsum(float(x[t, h]) * float(w[e, h]) for h in range(sh.H))
            if inp["bias"] is not None:
                exact += float(inp["bias"][e])
            assert abs(z[t, e] - exact) <= sh.H * np.spacing(np.float32(abs(exact) + 1.0)) * 4
    # brute force top-k on exact fp64 logits agrees wherever the top-k gap is wide
    z64 = x @ w.T + (0 if inp["bias"] is None else inp["bias"].astype(np.float64))
    for t in range(sh.T):
        order = sorted(range(sh.E), key=lambda e: (-z64[t, e], e))
        srt = np.sort(z64[t])[::-1]
        gaps = np.abs(np.diff(srt[: sh.k + 1]))
        if gaps.min() > 1e-4:
            assert list(idx[t]) == order[: sh.k]
    # invariants
    assert np.all(np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1])
    assert np.all(wts > 0)
    if sh.renorm:
        assert np.allclose(wts.sum(axis=1), 1.0, atol=1e-6)
    else:
        assert np.all(wts.sum(axis=1) <= 1.0 + 1e-6)
    # slot order is descending logit
    zs = np.take_along_axis(z, idx, axis=1)
    assert np.all(zs[:, :-1] >= zs[:, 1:])


def test_router_ties_go_to_lower_id():
    T, H, E, k = 4, 8, 6, 3
    x = np.zeros((T, H), dtype=np.float32)
    w = np.ones((E, H), dtype=np.float32)
    x[1, 0] = 1.0                         # token 1: all logits equal 1.0
    w[4, 0] = 2.0                         # expert 4 wins for token 1
    x[2, 0] = -0.0                        # signed zeros compare equal
    idx, wts, _ = route.route(x, w, None, k, 1)
    assert list(idx[0]) == [0, 1, 2]
    assert list(idx[1]) == [4, 0, 1]
    assert list(idx[2]) == [0, 1, 2]
    assert np.allclose(wts[0], 1.0 / 3)


def test_router_full_softmax_reading():
    """renorm=0 returns full-softmax probabilities at the chosen experts."""
    z = np.array([[2.0, 1.0, 0.0, -1.0]], dtype=np.float32)
    idx = route.topk(z, 2)
    w = route.weights(z, idx, 0)
    p = np.exp(z[0].astype(np.float64)); p /= p.sum()
    assert list(idx[0]) == [0, 1]
    assert np.allclose(w[0], p[:2], rtol=1e-7)
    w1 = route.weights(z, idx, 1)
    assert np.allclose(w1[0], [1 / (1 + math.exp(-1)), math.exp(-1) / (1 + math.exp(-1))], rtol=1e-7)


def brute_schedule(re, E, MB):
    """Positions by explicit enumeration: walk minibatches, then experts, then
    rows in arrival order, handing out consecutive slots."""
    R = len(re)
    pos = [-1] * R
    nb = -(-R // MB)
    for b in range(nb):
        p = b * MB
        for e in range(E):
            for r in range(b * MB, min(R, (b + 1) * MB)):
                if re[r] == e:
                    pos[r] = p
                    p += 1
    return np.array(pos)


@pytest.mark.parametrize("R,E,MB,tile", [(512, 8, 512, 256), (500, 8, 128, 64), (97, 3, 40, 16),
                                         (1000, 4, 256, 256), (0, 4, 16, 16)])
def test_schedule_brute_force_and_invariants(R, E, MB, tile):
    rng = np.random.default_rng(R + E)
    re = rng.choice(E, size=R, p=workloads.zipf_local_weights(E, 1.2)).astype(np.int32)
    ring_rows = 2 * MB
    s = schedule.build(re, E, MB, ring_rows, tile)
    assert np.array_equal(s.sorted_pos, brute_schedule(re, E, MB))
    assert s.counts.sum() == R and np.array_equal(s.counts, np.bincount(re, minlength=E))
    assert s.offsets[0] == 0 and s.offsets[-1] == R and np.all(np.diff(s.offsets) >= 0)
    # bijection onto the occupied positions; inv o sorted_pos = id
    assert np.array_equal(s.inv[s.sorted_pos], np.arange(R))
    assert len(set(s.sorted_pos.tolist())) == R
    # stability: within (minibatch, expert) positions increase with r
    for b in range(s.nb):
        for e in range(E):
            rows = [r for r in range(b * MB, min(R, (b + 1) * MB)) if re[r] == e]
            assert np.all(np.diff(s.sorted_pos[rows]) == 1)
    # items tile every (b, e) run exactly once
    cover = np.zeros(s.nb * MB, dtype=int)
    for (rb, rc, e, b) in s.items:
        assert 0 < rc <= tile
        assert np.all(re[s.inv[rb:rb + rc]] == e)
        assert np.all(s.inv[rb:rb + rc] // MB == b)
        cover[rb:rb + rc] += 1
    assert np.array_equal(cover[s.sorted_pos], np.ones(R, dtype=int))
    assert cover.sum() == R
    assert s.mb_items[-1] == len(s.items)
    assert np.array_equal(s.ring_pos, s.sorted_pos % ring_rows)


def test_schedule_single_minibatch_is_stable_argsort():
    rng = np.random.default_rng(5)
    re = rng.integers(0, 16, 3000).astype(np.int32)
    s = schedule.build(re, 16, 4096, 4096, 256)
    assert np.array_equal(s.inv[:3000], np.argsort(re, kind="stable"))


def test_schedule_sorted_input_is_identity():
    re = np.repeat(np.arange(5), [3, 0, 7, 1, 9]).astype(np.int32)
    s = schedule.build(re, 5, 64, 64, 4)
    assert np.array_equal(s.sorted_pos, np.arange(len(re)))


def test_schedule_invalid_rows_dropped():
    re = np.array([0, 5, 1, -1, 1, 0], dtype=np.int32)
    s = schedule.build(re, 2, 8, 8, 4)
    assert s.invalid_rows == 2
    assert s.sorted_pos[1] == -1 and s.sorted_pos[3] == -1
    assert list(s.sorted_pos[[0, 5, 2, 4]]) == [0, 1, 2, 3]
    assert s.counts.sum() == 4


def test_ring_rows_rule():
    # 256 MiB ring, bf16 rows of H=7168: 18724 rows -> 4 minibatches of 4096
    assert schedule.ring_rows_for(256 << 20, 4096, schedule.row_bytes_for(7168, "bf16")) == 16384
    assert schedule.ring_rows_for(256 << 20, 8192, schedule.row_bytes_for(7168, "bf16")) == 16384
    # MXFP8 rows: 7168 codes + 224 scales
    assert schedule.row_bytes_for(7168, "mxfp8") == 7392
    assert schedule.ring_rows_for(256 << 20, 4096, 7392) == 32768
    with pytest.raises(ValueError):
        schedule.build(np.zeros(10, np.int32), 1, 8, 4, 4)


def ascending_order_case(T=1, H=256, E=8):
    """Router input whose top-2 depends on the summation order of the logits.

    Token 0: x[0, :4] = (1, 2^-12, 2^-12, -1), the rest 0.  Expert 0's router
    row starts (1, 2^-12, 2^-12, 1), so its products are (1, 2^-24, 2^-24, -1):
    summed in fp32 in ascending h from +0, 1 + 2^-24 is a tie that rounds to
    even, i.e. to 1, twice, and the last product cancels it: z0 = 0 exactly.
    In exact arithmetic (and summed in descending h) z0 = 2^-23; summed in
    pairs, 2^-24.  Expert 1's row is (2^-25, 0, ...): z1 = 2^-25 in every
    order.  Experts 2..7 have row (-1, 0, ...): z = -1.  So the ascending-h
    fp32 sum ranks expert 1 first (2^-25 > 0) where any of the other orders
    ranks expert 0 first.  Further tokens, if any, repeat token 0."""
    x = np.zeros((T, H)); wr = np.zeros((E, H))
    x[:, :4] = [1.0, 2.0 ** -12, 2.0 ** -12, -1.0]
    wr[0, :4] = [1.0, 2.0 ** -12, 2.0 ** -12, 1.0]
    wr[1, 0] = 2.0 ** -25
    wr[2:, 0] = -1.0
    return bf16.encode(x), bf16.encode(wr)


def test_logits_are_summed_in_ascending_h_from_zero():
    """Golden case worked by hand from IEEE fp32 round-to-nearest-even (see
    ascending_order_case): the logits and the top-2 the router reading takes
    (fp32, ascending h, from +0) differ from those of the exact sum."""
    xb, wb = ascending_order_case(T=2)
    x = bf16.decode(xb).astype(np.float32); w = bf16.decode(wb).astype(np.float32)
    z = route.logits_fp32(x, w, None)
    assert z[0, 0] == 0.0 and z[0, 1] == 2.0 ** -25 and np.all(z[0, 2:] == -1.0)
    idx, wts, _ = route.route(x, w, None, 2, 1)
    assert idx.tolist() == [[1, 0], [1, 0]]
    # the exact sum would rank them the other way
    z64 = bf16.decode(xb) @ bf16.decode(wb).T
    assert z64[0, 0] == 2.0 ** -23 and z64[0, 0] > z64[0, 1]
