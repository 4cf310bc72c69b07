"""Shared helpers of the GPU tests: device upload, result download, the
float-tolerance rule.  No arithmetic of the layer lives here."""
import sys

import numpy as np
import torch

from oracle import bf16

BF16_TOL = 2e-2     # max |err| <= 2e-2 * RMS(oracle tensor), bf16 outputs and gradients
MXFP8_TOL = 6e-2    # same rule for MXFP8 outputs against the MXFP8-emulating oracle; where an
# MXFP8 operand is quantised from a GEMM output (a in the forward, dg/du in
# the backward) the oracle also gives each element an allowance for the E4M3
# codes another correct evaluation may decide differently (``layer.qd_spread``)
ROUTER_W_ATOL = 2e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(bits_or_array, device="cuda"):
    a = np.ascontiguousarray(bits_or_array)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    """Device bf16 bits (int16) -> fp64 values."""
    return bf16.decode(t.cpu().numpy().view(np.uint16))


def rms(a):
    return float(np.sqrt(np.mean(np.square(np.asarray(a, dtype=np.float64)))))


def ulp_bf16(v):
    """Spacing of bf16 values at |v|."""
    _, e = np.frexp(np.abs(np.asarray(v, dtype=np.float64)))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def assert_close(got, ref, tol, what, bf16_out=False, allow=None):
    """max|got - ref| <= tol * RMS(ref).

    bf16_out: got is a bf16 tensor and ref the oracle's exact value of it,
    before the rounding to bf16 that the layer's output format applies.
    That rounding alone moves a correct result by up to half a bf16 step
    (far more than 2e-2 * RMS where |v| is many times the RMS), so each
    element's error less half a bf16 step (at the larger of the two
    magnitudes) must stay within tol * RMS(ref); an implementation that
    rounds its fp32 value of the exact result once passes with the fp32
    error alone.  allow: a per-element allowance from the oracle (roundings
    and E4M3 codes decided on GEMM outputs) that is subtracted as well.  The
    raw ratio, the share of differing elements and the allowance are printed
    alongside."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    r = rms(ref)
    d = np.abs(got - ref)
    err = float(np.max(d)) if ref.size else 0.0
    msg = f"  {what}: max|err| = {err:.3e}, RMS(ref) = {r:.3e}, ratio = {err / max(r, 1e-300):.3e} (tol {tol})"
    a = np.zeros_like(ref) if allow is None else np.broadcast_to(np.asarray(allow, dtype=np.float64), ref.shape)
    if not bf16_out:
        ex = float(np.max(np.maximum(d - a, 0.0))) if ref.size else 0.0
        say(msg + (f"; beyond allowance: {ex / max(r, 1e-300):.3e}" if allow is not None else ""))
        assert ex <= tol * r, f"{what}: max|err| beyond allowance {ex:.4e} > {tol} * RMS {r:.4e}"
        return
    h = 0.5 * ulp_bf16(np.maximum(np.abs(got), np.abs(ref)))
    beyond = np.maximum(d - h - a, 0.0)
    ex = float(np.max(beyond)) if ref.size else 0.0
    extra = ""
    if allow is not None and ref.size:
        extra = (f"; allowance > 0 on {np.mean(a > 0):.1%}, p90 {np.quantile(a, 0.9) / max(r, 1e-300):.2e}"
                 f", max {np.max(a) / max(r, 1e-300):.2e} of RMS")
    say(msg + f"; beyond half a bf16 step: {np.max(np.maximum(d - h, 0.0)) / max(r, 1e-300) if ref.size else 0:.3e}"
        f" of RMS on {np.mean(d > h):.4%} of elements" + extra + f"; beyond the allowance too: {ex / max(r, 1e-300):.3e}")
    assert ex <= tol * r, f"{what}: error beyond half a bf16 step and the allowance {ex:.4e} > {tol} * RMS {r:.4e}"
