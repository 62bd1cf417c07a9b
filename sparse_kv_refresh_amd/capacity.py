"""Hardware-aware refresh capacity (RealtimeWAM §3 "Token capacity": the
latency of a forward pass is flat over ranges of token counts because of tile
and wave quantisation; the upper end of the plateau holding the required
count is the execution capacity, and the spare slots are filled with the next
most useful tokens at almost no latency cost).

Host-side policy only: it reads a measured latency curve (for example the
per-layer curve of `bench.py --plateau`) and returns a row count; the refresh
itself is the ordinary selection with that count, which already fills by
rank.
"""
from __future__ import annotations

import bisect
from typing import Sequence


def plateau_capacity(rows: Sequence[int], ms: Sequence[float], k: int, tol: float = 0.02) -> int:
    """Largest profiled row count r >= k such that every profiled latency from
    the first profiled count >= k up to r stays within (1 + tol) of the
    latency at that first count.  `rows` ascending; returns k when k lies
    beyond the profile or the next profiled count already costs more."""
    if len(rows) != len(ms) or not rows:
        raise ValueError("rows and ms must be non-empty and of equal length")
    if any(b <= a for a, b in zip(rows, rows[1:])):
        raise ValueError("rows must be strictly ascending")
    if k < 0:
        raise ValueError("k must be >= 0")
    i = bisect.bisect_left(rows, k)
    if i == len(rows):
        return k
    base = ms[i]
    cap = max(k, rows[i]) if ms[i] <= (1.0 + tol) * base else k
    for j in range(i + 1, len(rows)):
        if ms[j] > (1.0 + tol) * base:
            break
        cap = rows[j]
    return cap
