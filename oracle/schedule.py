"""Dispatch schedule and ring placement (oracle; test infrastructure only).

What the pages fix ([MTP] "Three design decisions that matter"): one schedule
table serves dispatch, combine and both backward directions; rows move in
minibatches ("tokens per transfer", [WIKI] item 2) through a fixed-size ring
token buffer cycled at minibatch granularity ([WIKI] item 3, [MTP] third
design decision), and no token is dropped ([MTP] "Key Takeaways").

Readings used here (the pages give no table layout):

* A minibatch is MB consecutive routed rows in arrival order; the last one may
  be short.  Inside a minibatch rows are grouped by expert, stably (arrival
  order kept within an expert) -- a counting sort.
* sorted_pos[r] = b*MB + mb_offsets[b][e] + rank[r], where mb_offsets[b] is the
  exclusive scan over experts of minibatch b's counts and rank[r] counts the
  earlier rows of the same minibatch routed to the same expert.
* The ring holds ring_rows = MB * floor(ring_bytes / (MB * row_bytes)) rows, a
  whole number of minibatches; row r lives in ring slot sorted_pos[r] mod
  ring_rows.  A ring smaller than one minibatch is an error.
* Work items for the expert-grouped GEMMs: for each minibatch b, expert e and
  m-tile of tile_m rows, (row_begin, row_count, e, b), ordered by (b, e, m).
  mb_items[b] is the index of minibatch b's first item.
* A row whose expert id is outside [0, E) is left out of the schedule
  (sorted_pos = -1) and flagged; every other row is placed as above.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class Schedule:
    R: int
    E: int
    MB: int
    nb: int
    ring_rows: int
    tile_m: int
    counts: np.ndarray        # [E]        rows per expert (valid rows only)
    offsets: np.ndarray       # [E+1]      exclusive scan of counts
    mb_counts: np.ndarray     # [nb, E]
    mb_offsets: np.ndarray    # [nb, E+1]  exclusive scan within each minibatch
    sorted_pos: np.ndarray    # [R]        -1 for a dropped (invalid) row
    inv: np.ndarray           # [nb*MB]    row at each sorted position, -1 if none
    ring_pos: np.ndarray      # [R]        -1 for a dropped row
    items: np.ndarray         # [n_items, 4] (row_begin, row_count, expert, minibatch)
    mb_items: np.ndarray      # [nb+1]
    invalid_rows: int


def ring_rows_for(ring_bytes: int, MB: int, row_bytes: int) -> int:
    """Rows the ring holds: a whole number of minibatches (0 if not one fits)."""
    return MB * (ring_bytes // (MB * row_bytes))


def row_bytes_for(H: int, precision: str) -> int:
    """Bytes one ring row takes: bf16 values, or E4M3 codes plus one E8M0
    scale per 32 values."""
    if precision == "bf16":
        return 2 * H
    if precision == "mxfp8":
        return H + H // 32
    raise ValueError(precision)


def build(row_expert: np.ndarray, E: int, MB: int, ring_rows: int, tile_m: int) -> Schedule:
    re = np.asarray(row_expert, dtype=np.int64)
    R = re.shape[0]
    if MB <= 0 or ring_rows < MB or ring_rows % MB:
        raise ValueError("ring must hold a whole, non-zero number of minibatches")
    nb = -(-R // MB) if R else 0
    valid = (re >= 0) & (re < E)
    counts = np.zeros(E, dtype=np.int64)
    mb_counts = np.zeros((nb, E), dtype=np.int64)
    sorted_pos = np.full(R, -1, dtype=np.int64)
    inv = np.full(nb * MB, -1, dtype=np.int64)
    mb_offsets = np.zeros((nb, E + 1), dtype=np.int64)
    for b in range(nb):
        lo, hi = b * MB, min(R, (b + 1) * MB)
        for r in range(lo, hi):
            if valid[r]:
                mb_counts[b, re[r]] += 1
        mb_offsets[b, 1:] = np.cumsum(mb_counts[b])
        seen = np.zeros(E, dtype=np.int64)
        for r in range(lo, hi):
            if not valid[r]:
                continue
            e = re[r]
            p = b * MB + mb_offsets[b, e] + seen[e]
            seen[e] += 1
            sorted_pos[r] = p
            inv[p] = r
    counts = mb_counts.sum(axis=0) if nb else counts
    offsets = np.concatenate([[0], np.cumsum(counts)])
    ring_pos = np.where(sorted_pos >= 0, sorted_pos % ring_rows, -1)
    items = []
    mb_items = [0]
    for b in range(nb):
        for e in range(E):
            c = int(mb_counts[b, e])
            for m in range(-(-c // tile_m)):
                items.append((b * MB + mb_offsets[b, e] + m * tile_m,
                              min(tile_m, c - m * tile_m), e, b))
        mb_items.append(len(items))
    return Schedule(
        R=R, E=E, MB=MB, nb=nb, ring_rows=ring_rows, tile_m=tile_m,
        counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
        mb_counts=mb_counts.astype(np.int32), mb_offsets=mb_offsets.astype(np.int32),
        sorted_pos=sorted_pos.astype(np.int32), inv=inv.astype(np.int32),
        ring_pos=ring_pos.astype(np.int32),
        items=np.asarray(items, dtype=np.int32).reshape(-1, 4),
        mb_items=np.asarray(mb_items, dtype=np.int32),
        invalid_rows=int((~valid).sum()),
    )
