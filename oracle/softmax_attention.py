"""CPU oracle for the softmax variant of the jagged causal attention.

TEST INFRASTRUCTURE ONLY. Only the test suite and the benchmark's CPU-baseline leg use
this module. The GPU library never imports it, calls it or falls back to it.

The HSTU chapter of chenhuiyu.github.io ("What an HSTU layer changes", "No
sequence-wise softmax") contrasts HSTU's pointwise SiLU with softmax attention,
which normalises every row to total mass one. It reports an ablation that replaces
the pointwise activation with softmax. This module is that ablation, taken as
plainly as possible. The scores are the HSTU scores, z_ij = q_i.k_j + rab(i, j),
with the same buckets and tables as the forward oracle and no 1/sqrt(d), because
only the activation changes. Each query row i is normalised over its visible keys
j <= i:

    A_ij = exp(z_ij) / sum_{k <= i} exp(z_ik)   (j <= i), else 0;     O_i = sum_j A_ij v_j

It is computed in fp64, densely per sequence and head, with the row maximum
subtracted before exp, which leaves the value unchanged.
"""
from __future__ import annotations

import numpy as np

from . import hstu_oracle as F

__all__ = ["softmax_attention", "softmax_attention_rows"]


def _row_softmax_av(z, v):
    """softmax over the last axis of z (rows fully visible), then times v."""
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)) @ v


def softmax_attention(offsets, ts, q, k, v, rab_pos, rab_time):
    """Causal softmax attention over a jagged batch. q, k [T_tot, H, d_qk];
    v [T_tot, H, d_v]. Returns fp64 [T_tot, H, d_v]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    Ttot, H, dv = v.shape
    out = np.zeros((Ttot, H, dv))
    for b in range(len(offsets) - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        n = e - s
        if n == 0:
            continue
        pos = np.arange(n, dtype=np.int64)
        t = None if ts is None else np.asarray(ts, np.int64)[s:e]
        hidden = pos[None, :] > pos[:, None]
        for h in range(H):
            z = q[s:e, h] @ k[s:e, h].T + F.bias_matrix(h, pos, pos, t, t, rab_pos, rab_time)
            z = np.where(hidden, -np.inf, z)
            out[s:e, h] = _row_softmax_av(z, v[s:e, h])
    return out


def softmax_attention_rows(offsets, ts, q, k, v, rab_pos, rab_time, rows):
    """Selected global rows of softmax_attention, each from its own prefix (keys 0..i)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    H, dv = v.shape[1], v.shape[2]
    out = np.zeros((len(rows), H, dv))
    for idx, r in enumerate(rows):
        r = int(r)
        b = int(np.searchsorted(offsets, r, side="right")) - 1
        s = int(offsets[b])
        i = r - s
        kpos = np.arange(i + 1, dtype=np.int64)
        qts = None if ts is None else np.asarray(ts, np.int64)[r:r + 1]
        kts = None if ts is None else np.asarray(ts, np.int64)[s:r + 1]
        for h in range(H):
            bias = F.bias_matrix(h, np.array([i]), kpos, qts, kts, rab_pos, rab_time)[0]
            z = k[s:r + 1, h] @ q[r, h] + bias
            out[idx, h] = _row_softmax_av(z[None, :], v[s:r + 1, h])[0]
    return out
