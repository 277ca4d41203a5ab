"""Pins of the softmax-variant oracle (CPU): closed forms (prefix mean, one action,
rows of mass one), shift invariance of softmax, a dominant key, and an independent
route through scipy's softmax on a small case."""
import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import softmax_attention as SA
from oracle import hstu_oracle as F
from hstu_jagged_pointwise_amd import synth


def _case(seed, lens=(6, 1, 0, 9), H=2, d=4, P=4, T=3):
    rng = np.random.default_rng(seed)
    off = synth.offsets_from_lengths(np.array(lens))
    n = int(off[-1])
    q, k, v = (rng.standard_normal((n, H, d)) for _ in range(3))
    rp = rng.standard_normal((H, P))
    rt = rng.standard_normal((H, T))
    ts = np.concatenate([np.cumsum(rng.integers(0, 6, size=m)) for m in lens if m]).astype(np.int64)
    return off, ts, q, k, v, rp, rt


def test_zero_queries_give_prefix_means():
    off, ts, q, k, v, rp, rt = _case(1)
    o = SA.softmax_attention(off, None, np.zeros_like(q), k, v, None, None)
    for b in range(len(off) - 1):
        s, e = int(off[b]), int(off[b + 1])
        for i in range(s, e):
            assert np.allclose(o[i], v[s:i + 1].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_one_action_returns_its_value_and_rows_have_mass_one():
    off, ts, q, k, v, rp, rt = _case(2)
    o = SA.softmax_attention(off, ts, q, k, v, rp, rt)
    assert np.allclose(o[6], v[6], rtol=1e-14)  # the one-action sequence
    ones = SA.softmax_attention(off, ts, q, k, np.ones_like(v), rp, rt)
    assert np.allclose(ones, 1.0, rtol=1e-13)


def test_shift_invariance():
    off, ts, q, k, v, rp, rt = _case(3)
    a = SA.softmax_attention(off, ts, q, k, v, rp, rt)
    b = SA.softmax_attention(off, ts, q, k, v, rp + 7.5, rt - 2.0)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def test_dominant_key_wins():
    off, ts, q, k, v, rp, rt = _case(4, lens=(5,), H=1)
    k = k.copy()
    k[2, 0] = 40.0 * q[4, 0] / np.linalg.norm(q[4, 0])  # row 4 scores key 2 far above the rest
    o = SA.softmax_attention(off, None, q, k, v, None, None)
    assert np.allclose(o[4, 0], v[2, 0], atol=1e-6)


def test_against_scipy_softmax_by_loops():
    off, ts, q, k, v, rp, rt = _case(5)
    o = SA.softmax_attention(off, ts, q, k, v, rp, rt)
    P, T = rp.shape[1], rt.shape[1]
    for b in range(len(off) - 1):
        s, e = int(off[b]), int(off[b + 1])
        for i in range(e - s):
            for h in range(q.shape[1]):
                z = []
                for j in range(i + 1):
                    dt = int(ts[s + i]) - int(ts[s + j])
                    bt = min((max(dt, 0) + 1).bit_length() - 1, T - 1)
                    z.append(float(q[s + i, h] @ k[s + j, h]) + rp[h, min(i - j, P - 1)] + rt[h, bt])
                w = sp_softmax(np.array(z))
                want = w @ v[s:s + i + 1, h]
                assert np.allclose(o[s + i, h], want, rtol=1e-12, atol=1e-13)


def test_sampled_rows_equal_full():
    off, ts, q, k, v, rp, rt = _case(6)
    o = SA.softmax_attention(off, ts, q, k, v, rp, rt)
    rows = np.arange(int(off[-1]))
    assert np.allclose(SA.softmax_attention_rows(off, ts, q, k, v, rp, rt, rows), o, rtol=1e-13,
                       atol=1e-14)
