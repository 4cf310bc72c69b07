"""ctypes binding of libmk.so (declared in include/mk.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmk.so.  Functions keep the C names; device pointers are passed as
integers (``tensor.data_ptr()``) and ``stream`` is a hipStream_t handle
(``torch.cuda.current_stream().cuda_stream``) or None for the default stream.
A missing library raises at import: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

# torch ships its own HIP runtime with the same SONAME (libamdhip64.so.7) as
# the one libmk.so links against; loading torch first makes the dynamic
# linker bind libmk.so to that already-loaded runtime, so the process has one
# HIP runtime and torch's device memory and streams are valid here.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmk.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "mk.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_device_amd.build`")

lib = ctypes.CDLL(LIB_PATH)


def _constants() -> dict:
    out = {}
    for line in open(HEADER):
        m = re.match(r"#define\s+(MK_\w+)\s+(-?0x[0-9a-fA-F]+|-?\d+)u?\b", line)
        if m:
            out[m.group(1)] = int(m.group(2), 0)
    return out


C = _constants()
globals().update(C)


class MkConfig(ctypes.Structure):
    _fields_ = [
        ("minibatch_rows", ctypes.c_int32),
        ("precision", ctypes.c_int32),
        ("ring_bytes", ctypes.c_int64),
        ("sched_capacity_mult", ctypes.c_float),
        ("renorm", ctypes.c_int32),
        ("enable_backward", ctypes.c_int32),
        ("wgrad_mxfp8", ctypes.c_int32),
        ("fused_forward", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64

_SIGS = {
    "mk_config_default": (None, [ctypes.POINTER(MkConfig)]),
    "mk_workspace_create": (ctypes.c_int, [ctypes.POINTER(MkConfig), _i32, _i32, _i32, _i32, _i32,
                                           ctypes.POINTER(_vp)]),
    "mk_workspace_destroy": (ctypes.c_int, [_vp]),
    "mk_query": (_i64, [_vp, _i32]),
    "mk_route": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "mk_schedule_create": (ctypes.c_int, [_vp, ctypes.POINTER(_vp)]),
    "mk_schedule_destroy": (ctypes.c_int, [_vp]),
    "mk_schedule_query": (_i64, [_vp, _i32]),
    "mk_build_schedule": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp]),
    "mk_build_schedule_static": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32] + [_vp] * 10),
    "mk_schedule_copy": (ctypes.c_int, [_vp, _i32, _vp, _i64, _vp]),
    "mk_workspace_copy": (ctypes.c_int, [_vp, _i32, _vp, _i64, _vp]),
    "mk_mxfp8_quantize": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _vp]),
    "mk_prepare_weights": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp]),
    "mk_forward": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mk_backward": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mk_backward_layer": (ctypes.c_int, [_vp] * 18),
    "mk_device_error": (ctypes.c_int, [_vp, _vp, _vp]),
    "mk_debug_fused_waits": (ctypes.c_int, [_vp, _i32, _i32]),
    "mk_timing_enable": (ctypes.c_int, [_vp, _i32]),
    "mk_timing_phases": (ctypes.c_int, [_vp, ctypes.c_uint32]),
    "mk_timing_read": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_i32)]),
    "mk_two_wave_rows": (_i64, [_i32, _i32, _i32, _i32, _i32]),
    "mk_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class MkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({lib.mk_status_string(status).decode()})")
        self.status = status


def _check(fn: str, rc: int) -> int:
    if rc < 0:
        raise MkError(fn, rc)
    return rc


def _p(t) -> int | None:
    """Device pointer of a tensor (or an int), None for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream) -> int | None:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def declared_functions() -> list[str]:
    """Function names include/mk.h declares."""
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(mk_\w+)\s*\(", src, re.M)))


# ---- thin wrappers, same names as the C ABI ------------------------------

def mk_config_default() -> MkConfig:
    cfg = MkConfig()
    lib.mk_config_default(ctypes.byref(cfg))
    return cfg


def mk_workspace_create(cfg: MkConfig, max_rows: int, H: int, I: int, E: int, k: int) -> int:
    h = _vp()
    _check("mk_workspace_create", lib.mk_workspace_create(ctypes.byref(cfg), max_rows, H, I, E, k, ctypes.byref(h)))
    return h.value


def mk_workspace_destroy(ws: int) -> None:
    _check("mk_workspace_destroy", lib.mk_workspace_destroy(ws))


def mk_query(ws: int, what: int) -> int:
    return _check("mk_query", lib.mk_query(ws, what))


def mk_route(ws, x, w_router, bias, T, topk_idx, topk_w, stream=None):
    _check("mk_route", lib.mk_route(ws, _p(x), _p(w_router), _p(bias), T, _p(topk_idx), _p(topk_w), _s(stream)))


def mk_schedule_create(ws: int) -> int:
    h = _vp()
    _check("mk_schedule_create", lib.mk_schedule_create(ws, ctypes.byref(h)))
    return h.value


def mk_schedule_destroy(sched: int) -> None:
    _check("mk_schedule_destroy", lib.mk_schedule_destroy(sched))


def mk_schedule_query(sched: int, what: int) -> int:
    return _check("mk_schedule_query", lib.mk_schedule_query(sched, what))


def mk_build_schedule(ws, sched, row_expert, R, stream=None):
    _check("mk_build_schedule", lib.mk_build_schedule(ws, sched, _p(row_expert), R, _s(stream)))


def mk_build_schedule_static(row_expert, R, E, MB, item_cap, counts, offsets, mb_counts, mb_offsets, sorted_pos,
                             inv, items, mb_items, err, stream=None):
    _check("mk_build_schedule_static",
           lib.mk_build_schedule_static(_p(row_expert), R, E, MB, item_cap, _p(counts), _p(offsets), _p(mb_counts),
                                        _p(mb_offsets), _p(sorted_pos), _p(inv), _p(items), _p(mb_items), _p(err),
                                        _s(stream)))


def mk_schedule_copy(sched, table, dst, nbytes, stream=None):
    _check("mk_schedule_copy", lib.mk_schedule_copy(sched, table, _p(dst), nbytes, _s(stream)))


def mk_workspace_copy(ws, buffer, dst, nbytes, stream=None):
    _check("mk_workspace_copy", lib.mk_workspace_copy(ws, buffer, _p(dst), nbytes, _s(stream)))


def mk_mxfp8_quantize(x, rows, K, codes, scales, stream=None):
    _check("mk_mxfp8_quantize", lib.mk_mxfp8_quantize(_p(x), rows, K, _p(codes), _p(scales), _s(stream)))


def mk_prepare_weights(ws, w_gate, w_up, w_down, for_backward, packed, stream=None):
    _check("mk_prepare_weights", lib.mk_prepare_weights(ws, _p(w_gate), _p(w_up), _p(w_down), int(for_backward),
                                                        _p(packed), _s(stream)))


def mk_forward(ws, sched, mode, x_src, row_w, packed, out, fwd_ctx=None, stream=None):
    _check("mk_forward", lib.mk_forward(ws, sched, mode, _p(x_src), _p(row_w), _p(packed), _p(out), _p(fwd_ctx),
                                        _s(stream)))


def mk_backward(ws, sched, mode, fwd_ctx, x_src, row_w, packed, dY, dX, dW_gate, dW_up, dW_down, d_row_w,
                stream=None):
    _check("mk_backward", lib.mk_backward(ws, sched, mode, _p(fwd_ctx), _p(x_src), _p(row_w), _p(packed), _p(dY),
                                          _p(dX), _p(dW_gate), _p(dW_up), _p(dW_down), _p(d_row_w), _s(stream)))


def mk_backward_layer(ws, sched, fwd_ctx, x, w_router, bias, topk_idx, topk_w, packed, dY, dX, dW_gate, dW_up,
                      dW_down, dW_router, d_bias, d_topk_w, stream=None):
    _check("mk_backward_layer", lib.mk_backward_layer(ws, sched, _p(fwd_ctx), _p(x), _p(w_router), _p(bias),
                                                      _p(topk_idx), _p(topk_w), _p(packed), _p(dY), _p(dX),
                                                      _p(dW_gate), _p(dW_up), _p(dW_down), _p(dW_router),
                                                      _p(d_bias), _p(d_topk_w), _s(stream)))


def mk_device_error(sched, dst, stream=None):
    _check("mk_device_error", lib.mk_device_error(sched, _p(dst), _s(stream)))


def mk_debug_fused_waits(ws, spin_limit: int = 0, unreachable: bool = False) -> None:
    _check("mk_debug_fused_waits", lib.mk_debug_fused_waits(ws, int(spin_limit), int(unreachable)))


def mk_timing_enable(ws, on: bool) -> None:
    _check("mk_timing_enable", lib.mk_timing_enable(ws, int(on)))


def mk_timing_phases(ws, phases=None) -> None:
    """Record events only for the named phases while timing is on (None: all)."""
    mask = 0xFFFFFFFF if phases is None else sum(1 << PHASES.index(p) for p in phases)
    _check("mk_timing_phases", lib.mk_timing_phases(ws, mask))


PHASES = ["route", "schedule", "permute", "gemm1", "quant_a", "gemm2", "combine", "bwd_gather", "bwd_dact",
          "bwd_dw", "bwd_dx", "wgrad_down", "wgrad_gate_up", "bwd_combine", "router_bwd", "replay", "wgrad_quant",
          "fused_fwd"]


def mk_timing_read(ws) -> dict:
    """Host call: {phase: (ms, launches)} since the last read."""
    n = C["MK_PH_COUNT"]
    ms = (ctypes.c_float * n)()
    cnt = (_i32 * n)()
    _check("mk_timing_read", lib.mk_timing_read(ws, ms, cnt))
    return {PHASES[i]: (float(ms[i]), int(cnt[i])) for i in range(n)}


def mk_two_wave_rows(H, I, n_cu, tile_m, tile_n) -> int:
    return _check("mk_two_wave_rows", lib.mk_two_wave_rows(H, I, n_cu, tile_m, tile_n))


def mk_status_string(status: int) -> str:
    return lib.mk_status_string(status).decode()
