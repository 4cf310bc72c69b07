"""Pins for the oracle's bf16 and MXFP8 codecs (CPU only).

Independent references: torch's CPU casts (bf16 RNE; float8_e4m3fn RNE without
saturation, so inputs are clamped to +-448 first), brute-force nearest-code
search over the E4M3 code table, and hand-worked blocks from the OCP MX v1.0
definition (tests/golden/mxfp8_blocks.json).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import bf16, mxfp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def test_bf16_decode_encode_roundtrip_all_patterns():
    bits = all_finite_bf16()
    v = bf16.decode(bits)
    back = bf16.encode(v)
    # -0 and +0 both encode from their value; compare values, then sign
    assert np.array_equal(bf16.decode(back), v)
    assert np.array_equal(np.signbit(bf16.decode(back)), np.signbit(v))


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),    # subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
    ])
    # exact ties: bf16 value + half an ulp
    base = bf16.decode(rng.integers(0x0080, 0x7F00, 20000).astype(np.uint16))
    _, e = np.frexp(base)
    ties = (base + np.ldexp(1.0, e - 9)).astype(np.float32)
    v = np.concatenate([v, ties, -ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.encode(v.astype(np.float64))
    assert np.array_equal(got, ref)


def e4m3_table():
    codes = np.arange(256, dtype=np.uint8)
    vals = mxfp8.e4m3_decode(codes)
    return codes, vals


def test_e4m3_decode_table():
    codes, vals = e4m3_table()
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert vals[0x7E] == 448.0 and vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6
    assert vals[0x38] == 1.0 and vals[0x78] == 256.0
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(vals)
    assert np.array_equal(vals[fin], ref[fin])


def brute_force_encode(v):
    """Nearest of the finite non-negative E4M3 codes, ties to the even code,
    saturating at 448; sign taken from v."""
    codes = np.arange(0x7F, dtype=np.int64)       # 0x00..0x7E
    vals = mxfp8.e4m3_decode(codes.astype(np.uint8))
    a = np.minimum(np.abs(v), 448.0)
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates pick the even code (there are at most two, adjacent)
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (pick | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


@pytest.mark.parametrize("shift", [0, -3, 5, -9])
def test_e4m3_encode_exhaustive_bf16(shift):
    """Every finite bf16 value, scaled by 2^shift, through the element encoder."""
    v = bf16.decode(all_finite_bf16()) * 2.0 ** shift
    got = mxfp8.e4m3_encode(v)
    assert np.array_equal(got, brute_force_encode(v))
    clamped = np.clip(v, -448.0, 448.0)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nz = v != 0          # torch keeps -0 as 0x80 too, but compare the nonzero set strictly
    assert np.array_equal(got[nz], ref[nz])
    assert np.array_equal(got[~nz], np.where(np.signbit(v[~nz]), 0x80, 0x00).astype(np.uint8))


def test_e4m3_roundtrip_representable():
    codes, vals = e4m3_table()
    fin = ~np.isnan(vals)
    assert np.array_equal(mxfp8.e4m3_encode(vals[fin]), codes[fin])


def test_mx_golden_blocks():
    d = json.load(open(os.path.join(GOLDEN, "mxfp8_blocks.json")))
    for b in d["blocks"]:
        v = np.full(32, b["fill"], dtype=np.float64)
        for i, x in b["special"].items():
            v[int(i)] = x
        codes, scales = mxfp8.quantize(v[None, :])
        assert scales[0, 0] == b["scale"], b["name"]
        exp = np.full(32, b["fill_code"], dtype=np.uint8)
        for i, c in b["special_codes"].items():
            exp[int(i)] = c
        assert np.array_equal(codes[0], exp), b["name"]


def test_mx_scale_matches_torch_e8m0_on_powers_of_two():
    """torch's float8_e8m0fnu cast is exact on powers of two: the scale code of
    a block whose amax is 2^p is the E8M0 code of 2^(p-8)."""
    for p in range(-100, 120, 7):
        v = np.zeros((1, 32)); v[0, 5] = 2.0 ** p; v[0, 6] = -2.0 ** (p - 1)
        _, s = mxfp8.quantize(v)
        ref = torch.tensor([2.0 ** (p - 8)], dtype=torch.float32).to(torch.float8_e8m0fnu).view(torch.uint8).item()
        assert s[0, 0] == ref


def test_mx_quantize_error_bound_and_saturation():
    rng = np.random.default_rng(3)
    v = bf16.decode(bf16.encode(rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)) * 4)))
    codes, scales = mxfp8.quantize(v)
    d = mxfp8.dequantize(codes, scales)
    blk = v.reshape(64, 8, 32)
    amax = np.abs(blk).max(axis=-1, keepdims=True)
    step = 2.0 ** (np.floor(np.log2(amax)) - 3)                # ulp of the block's top binade
    err = np.abs(d.reshape(64, 8, 32) - blk)
    # below saturation: at most half an ulp of the value's own binade (<= half top ulp)
    sat = np.abs(blk) / 2.0 ** (np.floor(np.log2(amax)) - 8) > 448
    assert np.all(err[~sat] <= 0.5 * step.repeat(32, axis=-1)[~sat] + 1e-300)
    # saturated elements come out at exactly +-448 * scale
    assert np.all(np.abs(d.reshape(64, 8, 32)[sat]) == (448 * 2.0 ** (np.floor(np.log2(amax)) - 8)).repeat(32, axis=-1)[sat])
    # about 1/8 of random blocks have amax mantissa >= 1.75 and clip
    assert sat.any()


def test_mx_zero_and_negative_zero():
    v = np.zeros((2, 32)); v[1] = -0.0
    c, s = mxfp8.quantize(v)
    assert np.all(s == 0) and np.all(c[0] == 0) and np.all(c[1] == 0x80)
