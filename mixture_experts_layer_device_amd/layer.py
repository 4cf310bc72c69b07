"""Device-memory plumbing around the C ABI: torch tensors as buffers, the
current torch stream as the HIP stream.  No arithmetic of the layer happens
here; every call below is one libmk.so entry point.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

PRECISION = {"bf16": B.MK_BF16, "mxfp8": B.MK_MXFP8}
TABLE = {
    "counts": B.MK_TAB_COUNTS, "offsets": B.MK_TAB_OFFSETS, "mb_counts": B.MK_TAB_MB_COUNTS,
    "mb_offsets": B.MK_TAB_MB_OFFSETS, "sorted_pos": B.MK_TAB_SORTED_POS, "inv": B.MK_TAB_INV,
    "items": B.MK_TAB_ITEMS, "mb_items": B.MK_TAB_MB_ITEMS,
}
BUFFER = {
    "ring": B.MK_BUF_RING, "a": B.MK_BUF_A, "a_codes": B.MK_BUF_A_CODES, "a_scales": B.MK_BUF_A_SCALES,
    "y": B.MK_BUF_Y, "dgdu": B.MK_BUF_DGDU, "dgdu_codes": B.MK_BUF_DGDU_CODES, "dgdu_scales": B.MK_BUF_DGDU_SCALES,
    "wa": B.MK_BUF_WA, "dy_codes": B.MK_BUF_DY_CODES, "dy_scales": B.MK_BUF_DY_SCALES,
}


def to_device_bits(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 patterns -> device int16 tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def stream():
    return torch.cuda.current_stream().cuda_stream


class Schedule:
    """One dispatch schedule (mk_schedule) of a workspace."""

    def __init__(self, ws: int):
        self.handle = B.mk_schedule_create(ws)

    def close(self):
        if self.handle:
            B.mk_schedule_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class MoELayer:
    """A workspace plus the calls that use it (one per model, reused), with a
    default schedule; calls take ``sched=`` to use another one."""

    def __init__(self, H, I, E, k, max_rows, precision="bf16", minibatch_rows=0, ring_bytes=256 << 20,
                 renorm=1, enable_backward=False, capacity_mult=1.0, wgrad_mxfp8=False, fused_forward=False,
                 device="cuda"):
        cfg = B.mk_config_default()
        cfg.minibatch_rows = minibatch_rows
        cfg.precision = PRECISION[precision]
        cfg.ring_bytes = ring_bytes
        cfg.sched_capacity_mult = capacity_mult
        cfg.renorm = renorm
        cfg.enable_backward = int(enable_backward)
        cfg.wgrad_mxfp8 = int(wgrad_mxfp8)
        cfg.fused_forward = int(fused_forward)
        self.H, self.I, self.E, self.k = H, I, E, k
        self.precision = precision
        self.device = device
        self.ws = B.mk_workspace_create(cfg, max_rows, H, I, E, k)
        self.sched = Schedule(self.ws)
        self._scheds = [self.sched]

    def new_schedule(self) -> Schedule:
        s = Schedule(self.ws)
        self._scheds.append(s)
        return s

    def _sc(self, sched) -> int:
        return (sched or self.sched).handle

    def close(self):
        for s in getattr(self, "_scheds", []):
            s.close()
        if self.ws:
            B.mk_workspace_destroy(self.ws)
            self.ws = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def query(self, what: str) -> int:
        return B.mk_query(self.ws, getattr(B, "MK_Q_" + what.upper()))

    # ---- calls ---------------------------------------------------------
    def prepare_weights(self, w_gate, w_up, w_down, for_backward=False) -> torch.Tensor:
        nbytes = self.query("packed_bytes_bwd" if for_backward else "packed_bytes")
        packed = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        B.mk_prepare_weights(self.ws, w_gate, w_up, w_down, for_backward, packed, stream())
        return packed

    def route(self, x, w_router, bias, T):
        idx = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        B.mk_route(self.ws, x, w_router, bias, T, idx, w, stream())
        return idx, w

    def build_schedule(self, row_expert, R, sched=None):
        B.mk_build_schedule(self.ws, self._sc(sched), row_expert, R, stream())

    def forward(self, mode, x_src, row_w, packed, n_out, out=None, fwd_ctx=None, sched=None):
        if out is None:
            out = torch.empty((n_out, self.H), dtype=torch.int16, device=self.device)
        B.mk_forward(self.ws, self._sc(sched), mode, x_src, row_w, packed, out, fwd_ctx, stream())
        return out

    def new_fwd_ctx(self) -> torch.Tensor:
        return torch.empty(self.query("fwd_ctx_bytes"), dtype=torch.uint8, device=self.device)

    def _grads(self, n_x, R):
        E, H, I = self.E, self.H, self.I
        return {
            "dX": torch.empty((n_x, H), dtype=torch.int16, device=self.device),
            "dW_gate": torch.empty((E, I, H), dtype=torch.float32, device=self.device),
            "dW_up": torch.empty((E, I, H), dtype=torch.float32, device=self.device),
            "dW_down": torch.empty((E, H, I), dtype=torch.float32, device=self.device),
            "d_row_w": torch.empty((R,), dtype=torch.float32, device=self.device),
        }

    def backward(self, fwd_ctx, x_src, row_w, packed, dY, R, grads=None, mode=B.MK_EXPERT_SHARE, sched=None):
        """mk_backward; full-layer mode takes x/dY/dX as [R/k, H] token rows."""
        g = grads if grads is not None else self._grads(R if mode == B.MK_EXPERT_SHARE else R // self.k, R)
        B.mk_backward(self.ws, self._sc(sched), mode, fwd_ctx, x_src, row_w, packed, dY, g["dX"], g["dW_gate"],
                      g["dW_up"], g["dW_down"], g["d_row_w"], stream())
        return g

    def backward_layer(self, fwd_ctx, x, w_router, bias, topk_idx, topk_w, packed, dY, T, grads=None, sched=None):
        """mk_backward_layer: full layer including the router; d_row_w is the
        gradient w.r.t. topk_w (flattened), d_bias is None without a bias."""
        if grads is None:
            grads = self._grads(T, T * self.k)
            grads["dW_router"] = torch.empty((self.E, self.H), dtype=torch.float32, device=self.device)
            grads["d_bias"] = (torch.empty((self.E,), dtype=torch.float32, device=self.device)
                               if bias is not None else None)
        g = grads
        B.mk_backward_layer(self.ws, self._sc(sched), fwd_ctx, x, w_router, bias, topk_idx, topk_w, packed, dY, g["dX"],
                            g["dW_gate"], g["dW_up"], g["dW_down"], g["dW_router"], g["d_bias"], g["d_row_w"],
                            stream())
        return g

    def table(self, name: str, n: int, dtype=torch.int32, sched=None) -> torch.Tensor:
        """A schedule table (``TABLE``) or a workspace buffer (``BUFFER``), n
        elements of dtype."""
        item = torch.empty(0, dtype=dtype).element_size()
        t = torch.empty(n, dtype=dtype, device=self.device)
        if name in BUFFER:
            B.mk_workspace_copy(self.ws, BUFFER[name], t, n * item, stream())
        else:
            B.mk_schedule_copy(self._sc(sched), TABLE[name], t, n * item, stream())
        return t

    def sched_query(self, what: str, sched=None) -> int:
        return B.mk_schedule_query(self._sc(sched), getattr(B, "MK_Q_" + what.upper()))

    def device_error(self, sched=None) -> int:
        t = torch.zeros(1, dtype=torch.int32, device=self.device)
        B.mk_device_error(self._sc(sched), t, stream())
        return int(t.item()) & 0xFFFFFFFF
