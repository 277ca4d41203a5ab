"""CPU oracle for Stochastic Length (SL) sampling of jagged training sequences.

TEST INFRASTRUCTURE ONLY: the test suite is the only user. The GPU library never
imports, calls or falls back to it.

Source: the HSTU chapter of chenhuiyu.github.io, "Three more scaling components",
paragraph "Stochastic Length". Long histories are cut to a random sub-sequence
whose length is set by alpha, and a few are left whole; the page's worked number is
4,096 -> 776 at alpha = 1.6, which is floor(4096 ** 0.8) = floor(4096 ** (alpha / 2)).

Readings taken where the page is silent:

* target length: L = floor(N ** (alpha / 2)) for the maximum sequence length N
  (4096 -> 776 at alpha = 1.6). It is computed in float64 as
  floor(N ** (alpha / 2) + 1e-9), so that exact powers (4096 ** 0.75 = 512) do
  not land one below.
* a sequence of n <= L actions is kept whole.
* a longer one is kept whole with probability (L / n) ** 2 ("occasionally"; with
  it the expected cost of a user's n^2 attention term is at most 2 L^2), decided by
  a per-sequence uniform draw u_keep: whole iff u_keep < (L / n) ** 2.
* otherwise it becomes a uniformly random subsequence of exactly L actions that
  keeps their order. It is the L positions with the smallest (key, position) pairs
  under per-action uniform 32-bit keys. With i.i.d. keys every L-subset is equally
  likely.

The random numbers (u_keep per sequence, keys per action) are inputs, so the
oracle and the GPU take the same decisions.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["target_length", "keep_whole", "sl_lengths", "sl_select", "sl_gather"]


def target_length(N: int, alpha: float) -> int:
    """L = floor(N ** (alpha / 2)), in float64 with a 1e-9 guard against exact powers."""
    return int(math.floor(float(N) ** (float(np.float32(alpha)) / 2.0) + 1e-9))


def keep_whole(n: int, L: int, u: float) -> bool:
    """True when a sequence of n actions is kept whole: n <= L, or u < (L / n) ** 2."""
    if n <= L:
        return True
    return float(np.float32(u)) < (float(L) * float(L)) / (float(n) * float(n))


def sl_lengths(offsets, N: int, alpha: float, u_keep) -> np.ndarray:
    """New jagged offsets after Stochastic Length: each sequence keeps n or L actions."""
    off = np.asarray(offsets, np.int64)
    L = target_length(N, alpha)
    new = np.zeros_like(off)
    for b in range(len(off) - 1):
        n = int(off[b + 1] - off[b])
        new[b + 1] = new[b] + (n if keep_whole(n, L, u_keep[b]) else L)
    return new


def sl_select(offsets, new_offsets, keys) -> np.ndarray:
    """Source row (global index into the input) of every kept action, in order.
    A sequence whose new length equals its length is kept whole; otherwise the kept
    positions are those of the m smallest (key, position) pairs, m = new length,
    listed in increasing position."""
    off = np.asarray(offsets, np.int64)
    new = np.asarray(new_offsets, np.int64)
    keys = np.asarray(keys, np.uint32)
    src = np.zeros(int(new[-1]), np.int64)
    for b in range(len(off) - 1):
        s, e = int(off[b]), int(off[b + 1])
        n, m = e - s, int(new[b + 1] - new[b])
        if m == n:
            pos = np.arange(n)
        else:
            order = np.lexsort((np.arange(n), keys[s:e]))  # by key, then by position
            pos = np.sort(order[:m])
        src[new[b]:new[b + 1]] = s + pos
    return src


def sl_gather(x, ts, src):
    """Rows of x (and timestamps) at the kept source rows."""
    x = np.asarray(x)
    out_ts = None if ts is None else np.asarray(ts, np.int64)[src]
    return x[src], out_ts
