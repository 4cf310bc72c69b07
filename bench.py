"""Benchmark of the one-GPU MoE layer hot path on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-breakdown] [--no-cpu-baseline]

Prints ONE JSON line.  ``value`` is routed rows/s of the full single-GPU layer
forward (T=4096 tokens, H=2048, I=768, 128 experts, top-8 renormalised router
with a biased logit): one step = route + build_schedule + forward (permute,
expert GEMMs, combine), inputs resident in HBM.  ``breakdown`` adds the
expert-share shapes (EP=64 forward and the backward, each in bf16 and MXFP8)
and the full-layer backward including the router, each with rows/s,
grouped-GEMM TFLOP/s and per-kernel roofline fractions.  Kernel
durations come from HIP events the library records around each phase on the
stream it launches on, over the timed steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # dense MFMA flop/s
PEAK_FP8 = 5.0e15
PEAK_FP32_VALU = 157.3e12  # vector fp32 flop/s (published; counts packed FMA)
METRIC = "MoE layer routed rows/s + grouped-GEMM TFLOP/s (fwd/bwd, bf16 & MXFP8), 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma-separated workloads to run (full, full_unfused, full_fused, full_mxfp8, ep64_fwd, "
                         "ep64_fwd_fused, ep64_mxfp8, ep_bwd, ep_bwd_mxfp8, ep_bwd_mxfp8_dgrad, full_bwd, "
                         "full_bwd_mxfp8)")
    ap.add_argument("--main-fused", type=int, default=1,
                    help="1: the main line runs the forward as one fused launch (mk_config.fused_forward), "
                         "0: one launch per phase")
    ap.add_argument("--share-mb", type=int, default=0,
                    help="minibatch rows of the expert-share workloads (0: the two-wave floor of the GEMMs' "
                         "256 x 256 tiles on this GPU's compute units, mk_two_wave_rows)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (torch) 3 times: the known-size reference that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return ap.parse_args()


# --------------------------------------------------------------------------
# algorithmic work per phase (flops, bytes) -- minimum traffic: every operand
# read once and every result written once
# --------------------------------------------------------------------------
def phase_work(kind, R, T, H, I, E, k, mx=False, save_ctx=False, share=True, replay_rows=0, mx_wgrad=False):
    ab = 1 if mx else 2                       # bytes per GEMM operand element
    sc = 1.0 / 32 if mx else 0.0             # MXFP8 scale bytes per element
    w = {}
    if kind == "forward":
        w["route"] = (2.0 * T * E * H, T * H * 2 + E * H * 2 + T * k * 8)
        # (MXFP8 full layer: the T token rows are quantised once and GEMM1
        # reads their codes through the inverse map, x codes read once)
        xr = T if mx and not share else R
        w["permute"] = (0.0, xr * H * 2 + xr * H * (ab + sc))
        w["gemm1"] = (4.0 * R * H * I, xr * H * (ab + sc) + E * 2 * I * H * (ab + sc) + R * I * 2
                      + (R * 2 * I * 4 if save_ctx else 0))
        if mx:
            w["quant_a"] = (0.0, R * I * 2 + R * I * (1 + 1 / 32))
        w["gemm2"] = (2.0 * R * I * H, R * I * (ab + sc) + E * H * I * (ab + sc) + (R * H * 2 if share else R * H * 4))
        if not share:
            w["combine"] = (0.0, R * H * 4 + T * H * 2 + R * 8)
            # the same k-sum if the y rows were bf16 (2 bytes an element):
            # the floor of a design without the fp32 y round trip
            w["combine_y_bf16"] = (0.0, R * H * 2 + T * H * 2 + R * 8)
        # the fused forward: permute, GEMM1 and GEMM2 in one launch (the full
        # layer's combine stays a launch of its own); in the full layer's
        # launch GEMM1 gathers the token rows through the inverse map instead
        # of a permute, x read once
        if share:
            parts = [w[p] for p in ("permute", "gemm1", "gemm2")]
            w["fused_fwd"] = (sum(f for f, _ in parts), sum(b for _, b in parts))
        else:
            g1f, g1b = w["gemm1"]
            g1b += T * H * 2 - R * H * (ab + sc)
            w["fused_fwd"] = (g1f + w["gemm2"][0], g1b + w["gemm2"][1])
    else:
        # share: dY rows [R, H] in; full layer: dY [T, H] read once, rows written
        # (MXFP8: read twice, written as bf16 rows and as codes + scales)
        src = (R if share else T) * H * 2
        # (MXFP8 weight gradients: no bf16 copy; their dY operand is read from
        # the rows; in the full layer the T token rows are quantised once and
        # the dA' GEMM reads their codes)
        yr = T if mx_wgrad and not share else R
        w["bwd_gather"] = (0.0, src + (yr * H * (ab + sc) if mx_wgrad else
                                       R * H * 2 + (src + R * H * (ab + sc) if mx else 0)))
        w["bwd_dact"] = (2.0 * R * H * I, yr * H * (ab + sc) + E * I * H * (ab + sc) + R * 2 * I * 4 + R * 2 * I * 2
                         + R * I * 2)
        if mx:
            w["quant_a"] = (0.0, R * 2 * I * 2 + R * 2 * I * (1 + 1 / 32))     # dg/du quantised along 2I
        # share: bf16 rows to arrival order; full layer: fp32 rows for the k-sum
        w["bwd_dx"] = (4.0 * R * I * H, R * 2 * I * (ab + sc) + E * H * 2 * I * (ab + sc)
                       + R * H * (2 if share else 4))
        if mx_wgrad:
            # operands quantised along the rows: bf16 rows in, codes + scales out
            # (dY, w a, dg/du, x), then the GEMMs read codes + scales
            q = 1 + 1 / 32
            w["wgrad_quant"] = (0.0, R * (H + I + 2 * I + H) * (2 + q))
            w["wgrad_down"] = (2.0 * R * H * I, R * (H + I) * q + E * H * I * 4)
            w["wgrad_gate_up"] = (4.0 * R * H * I, R * (2 * I + H) * q + E * 2 * I * H * 4)
        else:
            w["wgrad_down"] = (2.0 * R * H * I, R * H * 2 + R * I * 2 + E * H * I * 4)
            w["wgrad_gate_up"] = (4.0 * R * H * I, R * 2 * I * 2 + R * H * 2 + E * 2 * I * H * 4)
        # x rows of the minibatches evicted from the ring gathered again
        w["replay"] = (0.0, replay_rows * H * 2 * 2)
        if not share:
            # k-sum of fp32 rows + router term (k rows of W_r per token, L2-resident)
            w["bwd_combine"] = (2.0 * R * H, R * H * 4 + T * H * 2 + R * 4 + T * E * 4 + E * H * 2)
            # logit gradient + dW_router = dz^T x (k nonzeros per token) + d_bias
            w["router_bwd"] = (2.0 * R * H, T * k * 12 + T * E * 4 * 2 + T * H * 2 + E * H * 4)
    return w


def roofline_alu(flops, nbytes, ms):
    """Vector-ALU work (the router's fp32 FMA chains): against the fp32 vector
    peak unless HBM takes longer."""
    if nbytes / PEAK_HBM > flops / PEAK_FP32_VALU:
        return roofline(0.0, nbytes, ms)
    ach = flops / (ms * 1e-3) / 1e12
    return {"bound": "alu", "achieved": round(ach, 2), "peak": PEAK_FP32_VALU / 1e12, "unit": "TFLOP/s",
            "frac": round(ach / (PEAK_FP32_VALU / 1e12), 4)}


def roofline(flops, nbytes, ms, mx=False):
    peak_f = PEAK_FP8 if mx else PEAK_BF16
    t_f = flops / peak_f
    t_b = nbytes / PEAK_HBM
    s = ms * 1e-3
    if t_f >= t_b and flops > 0:
        ach = flops / s / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_f / 1e12, "unit": "TFLOP/s",
                "frac": round(ach / (peak_f / 1e12), 4)}
    ach = nbytes / s / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(ach / (PEAK_HBM / 1e9), 4)}


def src_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "mixture_experts_layer_device_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        e = d[workload][kernel]
        if e["src_hash"] != src_hash(e["src_files"]):
            return None
        return e["bytes_per_launch"]
    except Exception:
        return None


# --------------------------------------------------------------------------
def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this layer runs on one GPU only; --gpus must be 1 "
                          "(sharding across GPUs is a design note, not built)"}))
        sys.exit(2)
    import torch

    import workloads
    from mixture_experts_layer_device_amd import binding as B
    from mixture_experts_layer_device_amd.layer import MoELayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"

    def up(x):
        x = np.ascontiguousarray(x)
        return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()

    def log(*m):
        print(*m, file=sys.stderr, flush=True)

    def timed(step, L, steps, warmup, outputs=()):
        """Warm-up; a breakdown pass of `steps` steps with events around every
        phase (they cost a few microseconds each, ~5% of a full-layer step);
        then the timed region: exactly `steps` steps, wall clock around the
        block, HIP events between steps for the median, and the library's
        events only around the phase that took longest in the breakdown (its
        figure in the returned breakdown is replaced by this live one).
        `outputs`: tensors the step writes; their bits after the timed steps
        are compared with a snapshot taken after warm-up (bitwise
        repeatability)."""
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        snap = [t.clone() for t in outputs]
        B.mk_timing_read(L.ws)                      # drop warm-up events
        B.mk_timing_phases(L.ws, None)
        B.mk_timing_enable(L.ws, True)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        B.mk_timing_enable(L.ws, False)
        ph = B.mk_timing_read(L.ws)
        per = {k: (v[0] / steps, v[1] / steps) for k, v in ph.items() if v[1] > 0}
        dom = max(per, key=lambda k: per[k][0])
        B.mk_timing_phases(L.ws, [dom])
        B.mk_timing_enable(L.ws, True)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            step()
            ev[i + 1].record()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        B.mk_timing_enable(L.ws, False)
        B.mk_timing_phases(L.ws, None)
        live = B.mk_timing_read(L.ws)[dom]
        per[dom] = (live[0] / steps, live[1] / steps)
        step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        extra = {"step_ms_median": round(step_ms[steps // 2], 4), "timed_phase": dom}
        if outputs:
            extra["repeatable"] = all(torch.equal(a, b) for a, b in zip(snap, outputs))
        # cold: the 256 MB last-level cache evicted before each step by writing
        # 512 MB elsewhere (the write is outside the timed interval)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold = []
        for _ in range(5):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush
        extra["step_ms_cold_median"] = round(sorted(cold)[2], 4)
        return dt, per, extra

    def summarize(name, R, T, H, I, E, k, dt, per, steps, kind, mx=False, share=True, save_ctx=False, replay_rows=0,
                  mx_wgrad=False):
        work = phase_work(kind, R, T, H, I, E, k, mx=mx, save_ctx=save_ctx, share=share, replay_rows=replay_rows,
                          mx_wgrad=mx_wgrad)
        mx_phases = ("gemm1", "gemm2", "bwd_dact", "bwd_dx") + (("wgrad_down", "wgrad_gate_up") if mx_wgrad else ())
        phases = {}
        gemm_flops = gemm_ms = 0.0
        for p, (ms, n) in per.items():
            f, b = work.get(p, (0.0, 0.0))
            ent = {"ms": round(ms, 4), "launches": n}
            if p == "route":
                ent["roofline"] = roofline_alu(f, b, ms)
            elif f or b:
                ent["roofline"] = roofline(f, b, ms, mx=mx and p in mx_phases)
            if p == "combine" and "combine_y_bf16" in work:
                ent["roofline_y_bf16_bytes"] = roofline(0.0, work["combine_y_bf16"][1], ms)
            phases[p] = ent
            if f and p not in ("route", "bwd_combine", "router_bwd"):
                gemm_flops += f
                gemm_ms += ms
        ms_step = dt / steps * 1e3
        return {
            "workload": name, "routed_rows": R, "ms_per_step": round(ms_step, 4),
            "rows_per_s": round(R / (ms_step * 1e-3), 1),
            "gemm_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 2) if gemm_ms else None,
            "gemm_tflops_over_step": round(gemm_flops / (ms_step * 1e-3) / 1e12, 2),
            "phases": phases,
        }

    results = {}
    want = set(a.only.split(",")) if a.only else {"full", "full_unfused", "full_mxfp8", "ep64_fwd",
                                                   "ep64_fwd_fused", "ep64_mxfp8", "ep_bwd", "ep_bwd_mxfp8",
                                                   "full_bwd", "full_bwd_mxfp8"}
    if a.no_breakdown:
        want = {"full"}

    # ---- main line: full single-GPU layer forward ------------------------
    main = None
    full_inp = None

    def run_full(key, fused, prec="bf16"):
        nonlocal full_inp
        log(f"[bench] full layer forward {prec}{' (fused: one launch)' if fused else ''}: T=4096 H=2048 I=768 "
            f"E=128 k=8")
        inp = full_inp = full_inp or workloads.make_full_layer("full")
        sh = inp["shape"]
        L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, fused_forward=fused,
                     precision=prec)
        x = up(inp["x"]); wr = up(inp["w_router"]); bias = up(inp["bias"])
        packed = L.prepare_weights(up(inp["w_gate"]), up(inp["w_up"]), up(inp["w_down"]))
        out = torch.empty((sh.T, sh.H), dtype=torch.int16, device="cuda")
        idx = torch.empty((sh.T, sh.k), dtype=torch.int32, device="cuda")
        wts = torch.empty((sh.T, sh.k), dtype=torch.float32, device="cuda")
        s = torch.cuda.current_stream()

        def step():
            B.mk_route(L.ws, x, wr, bias, sh.T, idx, wts, s)
            B.mk_build_schedule(L.ws, L.sched.handle, idx, sh.R, s)
            B.mk_forward(L.ws, L.sched.handle, B.MK_FULL_LAYER, x, wts, packed, out, None, s)

        dt, per, extra = timed(step, L, a.steps, a.warmup, outputs=(out, idx, wts))
        res = summarize(key, sh.R, sh.T, sh.H, sh.I, sh.E, sh.k, dt, per, a.steps, "forward", share=False,
                        mx=prec == "mxfp8")
        res.update(extra)
        res["err"] = L.device_error()
        L.close()
        del packed
        log(json.dumps(res))
        return res

    if "full" in want:
        main = run_full("full", a.main_fused)
    if "full_unfused" in want:
        results["full_unfused"] = run_full("full_unfused", False)
    if "full_fused" in want:
        results["full_fused"] = run_full("full_fused", True)
    if "full_mxfp8" in want:
        results["full_mxfp8"] = run_full("full_mxfp8", False, "mxfp8")

    # ---- expert-share shapes ---------------------------------------------
    # minibatches sized for at least two waves of 256 x 256 output tiles over
    # the compute units ([MTP] "Three design decisions that matter")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    share_mb = a.share_mb or B.mk_two_wave_rows(7168, 2048, n_cu // 8 * 8, 256, 256)
    if want & {"ep64_fwd", "ep64_fwd_fused", "ep64_mxfp8"}:
        inp = workloads.make_expert_share("ep64_fwd", with_dy=False)
        sh = inp["shape"]
        x = up(inp["x"]); re = up(inp["row_expert"]); rw = up(inp["row_w"])
        wg, wu, wd = up(inp["w_gate"]), up(inp["w_up"]), up(inp["w_down"])
        for prec, key, fused in (("bf16", "ep64_fwd", False), ("bf16", "ep64_fwd_fused", True),
                                 ("mxfp8", "ep64_mxfp8", False)):
            if key not in want:
                continue
            log(f"[bench] EP=64 expert share forward {prec}{' (fused: one launch)' if fused else ''}: R={sh.R} "
                f"H={sh.H} I={sh.I} E={sh.E} MB={share_mb}")
            L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=8, max_rows=sh.R, precision=prec, minibatch_rows=share_mb,
                         fused_forward=fused)
            packed = L.prepare_weights(wg, wu, wd)
            out = torch.empty((sh.R, sh.H), dtype=torch.int16, device="cuda")
            s = torch.cuda.current_stream()

            def step():
                B.mk_build_schedule(L.ws, L.sched.handle, re, sh.R, s)
                B.mk_forward(L.ws, L.sched.handle, B.MK_EXPERT_SHARE, x, rw, packed, out, None, s)

            dt, per, extra = timed(step, L, a.steps, a.warmup, outputs=(out,))
            results[key] = summarize(key, sh.R, 0, sh.H, sh.I, sh.E, 8, dt, per, a.steps, "forward",
                                     mx=prec == "mxfp8")
            results[key].update(extra)
            results[key]["minibatch_rows"] = share_mb
            results[key]["err"] = L.device_error()
            L.close()
            del packed
            log(json.dumps(results[key]))
        del x, wg, wu, wd

    # ep_bwd_mxfp8: every backward GEMM on MXFP8 operands; ep_bwd_mxfp8_dgrad:
    # MXFP8 data gradients with bf16 weight gradients (not run by default)
    for prec, key, mxw in (("bf16", "ep_bwd", False), ("mxfp8", "ep_bwd_mxfp8", True),
                           ("mxfp8", "ep_bwd_mxfp8_dgrad", False)):
        if key not in want:
            continue
        inp = workloads.make_expert_share("ep_bwd")
        sh = inp["shape"]
        log(f"[bench] expert share backward {prec}{' (MXFP8 weight gradients)' if mxw else ''}: "
            f"R={sh.R} H={sh.H} I={sh.I} E={sh.E} MB={share_mb} (ring wraps)")
        L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=8, max_rows=sh.R, precision=prec, minibatch_rows=share_mb,
                     enable_backward=True, wgrad_mxfp8=mxw)
        x = up(inp["x"]); re = up(inp["row_expert"]); rw = up(inp["row_w"]); dY = up(inp["dY"])
        packed = L.prepare_weights(up(inp["w_gate"]), up(inp["w_up"]), up(inp["w_down"]), for_backward=True)
        out = torch.empty((sh.R, sh.H), dtype=torch.int16, device="cuda")
        ctx = L.new_fwd_ctx()
        s = torch.cuda.current_stream()
        B.mk_build_schedule(L.ws, L.sched.handle, re, sh.R, s)
        B.mk_forward(L.ws, L.sched.handle, B.MK_EXPERT_SHARE, x, rw, packed, out, ctx, s)     # fwd_ctx, untimed
        g = {"dX": torch.empty((sh.R, sh.H), dtype=torch.int16, device="cuda"),
             "dW_gate": torch.empty((sh.E, sh.I, sh.H), dtype=torch.float32, device="cuda"),
             "dW_up": torch.empty((sh.E, sh.I, sh.H), dtype=torch.float32, device="cuda"),
             "dW_down": torch.empty((sh.E, sh.H, sh.I), dtype=torch.float32, device="cuda"),
             "d_row_w": torch.empty((sh.R,), dtype=torch.float32, device="cuda")}

        def step():
            B.mk_backward(L.ws, L.sched.handle, B.MK_EXPERT_SHARE, ctx, x, rw, packed, dY, g["dX"], g["dW_gate"], g["dW_up"],
                          g["dW_down"], g["d_row_w"], s)

        dt, per, extra = timed(step, L, a.steps, a.warmup, outputs=tuple(g.values()))
        MB = L.query("minibatch_rows")
        nb = -(-sh.R // MB)
        replay_mbs = 0 if mxw else nb if prec == "mxfp8" else max(0, nb - L.query("ring_rows") // MB)
        results[key] = summarize(key, sh.R, 0, sh.H, sh.I, sh.E, 8, dt, per, a.steps, "backward",
                                 mx=prec == "mxfp8", replay_rows=min(sh.R, replay_mbs * MB), mx_wgrad=mxw)
        results[key].update(extra)
        results[key]["minibatch_rows"] = share_mb
        results[key]["err"] = L.device_error()
        L.close()
        del packed, g, x, dY
        log(json.dumps(results[key]))

    for key in ("full_bwd", "full_bwd_mxfp8"):
        if key not in want:
            continue
        mxw = key == "full_bwd_mxfp8"
        prec = "mxfp8" if mxw else "bf16"
        inp = workloads.make_full_layer("full")
        sh = inp["shape"]
        log(f"[bench] full layer backward incl. router {prec}{' (MXFP8 weight gradients)' if mxw else ''}: "
            f"T={sh.T} H={sh.H} I={sh.I} E={sh.E} k={sh.k}")
        L = MoELayer(H=sh.H, I=sh.I, E=sh.E, k=sh.k, max_rows=sh.R, renorm=sh.renorm, enable_backward=True,
                     precision=prec, wgrad_mxfp8=mxw)
        x = up(inp["x"]); wr = up(inp["w_router"]); bias = up(inp["bias"]); dY = up(inp["dY"])
        packed = L.prepare_weights(up(inp["w_gate"]), up(inp["w_up"]), up(inp["w_down"]), for_backward=True)
        out = torch.empty((sh.T, sh.H), dtype=torch.int16, device="cuda")
        ctx = L.new_fwd_ctx()
        s = torch.cuda.current_stream()
        idx, wts = L.route(x, wr, bias, sh.T)                                 # forward, untimed
        B.mk_build_schedule(L.ws, L.sched.handle, idx, sh.R, s)
        B.mk_forward(L.ws, L.sched.handle, B.MK_FULL_LAYER, x, wts, packed, out, ctx, s)
        g = {"dX": torch.empty((sh.T, sh.H), dtype=torch.int16, device="cuda"),
             "dW_gate": torch.empty((sh.E, sh.I, sh.H), dtype=torch.float32, device="cuda"),
             "dW_up": torch.empty((sh.E, sh.I, sh.H), dtype=torch.float32, device="cuda"),
             "dW_down": torch.empty((sh.E, sh.H, sh.I), dtype=torch.float32, device="cuda"),
             "dW_router": torch.empty((sh.E, sh.H), dtype=torch.float32, device="cuda"),
             "d_bias": torch.empty((sh.E,), dtype=torch.float32, device="cuda"),
             "d_topk_w": torch.empty((sh.R,), dtype=torch.float32, device="cuda")}

        def step():
            B.mk_backward_layer(L.ws, L.sched.handle, ctx, x, wr, bias, idx, wts, packed, dY, g["dX"], g["dW_gate"], g["dW_up"],
                                g["dW_down"], g["dW_router"], g["d_bias"], g["d_topk_w"], s)

        dt, per, extra = timed(step, L, a.steps, a.warmup, outputs=tuple(g.values()))
        results[key] = summarize(key, sh.R, sh.T, sh.H, sh.I, sh.E, sh.k, dt, per, a.steps, "backward",
                                 share=False, mx=mxw, mx_wgrad=mxw)
        results[key].update(extra)
        results[key]["err"] = L.device_error()
        L.close()
        del packed
        log(json.dumps(results[key]))

    if a.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 3 x 1 GiB read + 1 GiB written")
        del src, dst

    # ---- CPU baseline: the oracle on a bounded sample of the main workload --
    cpu = None
    if main is not None and not a.no_cpu_baseline:
        cpu = cpu_baseline(log, full_inp)

    if main is None:
        main = next(iter(results.values()))
    # the dominant kernel: the phase whose events ran inside the timed region
    tp = main.get("timed_phase")
    dom = (tp, main["phases"][tp]) if tp in main["phases"] and "roofline" in main["phases"][tp] else \
        max(((p, v) for p, v in main["phases"].items() if "roofline" in v), key=lambda kv: kv[1]["ms"])
    roof = dict(dom[1]["roofline"])
    roof["kernel"] = dom[0]
    f, b = phase_work("forward", 32768, 4096, 2048, 768, 128, 8, share=False)[dom[0]] if main["workload"] == "full" \
        else (None, None)
    tr = traffic_for(dom[0], main["workload"])
    roof["traffic"] = tr
    roof["algorithmic"] = b if roof["bound"] == "hbm" else f
    line = {
        "metric": METRIC, "value": main["rows_per_s"], "unit": "rows/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": main["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full single-GPU MoE layer forward: route + build_schedule + permute (the "
                               "fused launch gathers the token rows inside GEMM1) + expert GEMMs (SwiGLU) + "
                               "combine; T=4096 tokens, H=2048, I=768, 128 experts, top-8 renormalised "
                               "softmax router with per-expert logit bias",
                   "tokens": 4096, "routed_rows": 32768, "H": 2048, "I": 768, "E": 128, "k": 8,
                   "forward_launches": "one fused persistent launch" if a.main_fused else "one launch per phase"},
        "gemm_tflops": main["gemm_tflops"],
        "protocol": {k: main.get(k) for k in ("step_ms_median", "step_ms_cold_median", "repeatable", "timed_phase")},
        "roofline": roof,
        "cpu_baseline": cpu,
        "phases": main["phases"],
        "breakdown": results,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(log, inp):
    """The oracle, as it stands, on the host cores.

    Main figure (``value``): the main workload's full-layer forward on all
    4096 tokens -- route, schedule (``oracle.schedule.build``), expert FFN and
    combine, each timed on its own -- in routed rows/s.  ``others``: the
    expert-share forward (bf16 and MXFP8) and backward on bounded samples of
    their workloads (the first rows of each, about a second or two of CPU
    work each), rows/s over the sample.  About 15-25 s of CPU in all."""
    import threadpoolctl

    import workloads
    from oracle import bf16, layer, route, schedule

    sh = inp["shape"]
    n_tok = sh.T
    toks = np.arange(n_tok)
    with threadpoolctl.threadpool_limits(limits=None):
        info = threadpoolctl.threadpool_info()
    blas_threads = max([i.get("num_threads", 1) for i in info] or [1])
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    x = bf16.decode(inp["x"][:n_tok]).astype(np.float32)
    idx, w, _ = route.route(x, bf16.decode(inp["w_router"]).astype(np.float32), inp["bias"], sh.k, sh.renorm)
    t1 = time.perf_counter()
    schedule.build(idx.reshape(-1), sh.E, n_tok * sh.k, n_tok * sh.k, 256)
    t2 = time.perf_counter()
    layer.forward_full_tokens(inp, idx, w, toks)
    t3 = time.perf_counter()
    rows = n_tok * sh.k
    log(f"[bench] cpu oracle, full layer: route {t1 - t0:.2f}s, schedule {t2 - t1:.2f}s, ffn+combine {t3 - t2:.2f}s "
        f"for {rows} routed rows")

    def sub(d, n):
        o = dict(d)
        for key in ("x", "row_expert", "row_w", "dY"):
            if key in o:
                o[key] = o[key][:n]
        return o

    others = {}
    ep = workloads.make_expert_share("ep64_fwd", with_dy=False)
    n = 2048
    d = sub(ep, n)
    ta = time.perf_counter()
    schedule.build(d["row_expert"], ep["shape"].E, 4096, 4096, 256)
    tb = time.perf_counter()
    layer.forward_share(d)
    tc = time.perf_counter()
    others["ep64_fwd"] = {"rows_per_s": round(n / (tc - ta), 1), "schedule_s": round(tb - ta, 3),
                          "forward_s": round(tc - tb, 3), "sample_rows": n, "of_rows": ep["shape"].R}
    # MXFP8: weights are quantised ahead (as on the device, outside the
    # timing); to bound that untimed work the sample is the first 1024 rows
    # routed to expert 0, with that expert's weights only
    sel = np.nonzero(ep["row_expert"] == 0)[0][:1024]
    d = {"x": ep["x"][sel], "row_expert": np.zeros(sel.size, np.int32), "row_w": ep["row_w"][sel],
         "w_gate": ep["w_gate"][:1], "w_up": ep["w_up"][:1], "w_down": ep["w_down"][:1]}
    qw = layer.quantized_weights(d)
    ta = time.perf_counter()
    layer.forward_share_mxfp8(d, qw=qw)
    tb = time.perf_counter()
    others["ep64_mxfp8"] = {"rows_per_s": round(sel.size / (tb - ta), 1), "forward_s": round(tb - ta, 3),
                            "sample_rows": int(sel.size), "of_rows": ep["shape"].R,
                            "sample": "rows of expert 0, weights quantised before the timing"}
    del ep
    bw = workloads.make_expert_share("ep_bwd")
    d = sub(bw, n)
    ta = time.perf_counter()
    layer.backward_share(d)
    tb = time.perf_counter()
    others["ep_bwd"] = {"rows_per_s": round(n / (tb - ta), 1), "backward_s": round(tb - ta, 3), "sample_rows": n,
                        "of_rows": bw["shape"].R}
    del bw
    log(f"[bench] cpu oracle, expert share samples: {json.dumps(others)}")
    return {"value": round(rows / (t3 - t0), 1), "unit": "rows/s", "cores": cores, "blas_threads": int(blas_threads),
            "kind": "oracle",
            "sample": f"full-layer forward of all {n_tok} tokens ({rows} routed rows): route, schedule and expert "
                      f"FFN + combine in fp64 numpy; cores = len(os.sched_getaffinity(0)), BLAS threads as listed",
            "phases_s": {"route": round(t1 - t0, 3), "schedule": round(t2 - t1, 3), "forward": round(t3 - t2, 3)},
            "others": others}


if __name__ == "__main__":
    main()
