"""Minibatch sizing rule (oracle; test infrastructure only).

[MTP] "Three design decisions that matter", overlap granularity: the
minibatch is sized so that each expert-grouped GEMM gets at least two full
waves over the GPU's compute units; for the Kimi 2.5 shapes the floor is
2,368 tokens.  [WIKI] item 2 prints the rule with numerator and denominator
swapped (it would give a fraction of a token).  The reading used here, which
reproduces 2,368, is

    T >= 2 * C * tile_m * tile_n / min(2*I, H)

tokens per minibatch, for C compute units and tile_m x tile_n output tiles:
an expert-grouped GEMM over T rows with N = min(2I, H) output columns (the
narrower of the up/gate and down GEMMs) produces T*N/(tile_m*tile_n) tiles,
and two waves need 2*C of them.
"""
from __future__ import annotations


def two_wave_rows(H: int, I: int, n_cu: int, tile_m: int = 128, tile_n: int = 256) -> int:
    """Smallest whole number of rows meeting the two-wave rule."""
    num = 2 * n_cu * tile_m * tile_n
    den = min(2 * I, H)
    return -(-num // den)
