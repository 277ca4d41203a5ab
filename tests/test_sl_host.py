"""Stochastic Length on the host side of the C ABI (no GPU): hstu_sl_lengths
against the oracle, and hstu_sl_sample's argument checks, which reject before
any HIP call."""
import ctypes
import os

import numpy as np
import pytest

from oracle import stochastic_length as SL
from hstu_jagged_pointwise_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "hstu_jagged_pointwise_amd", "libhstu.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libhstu.so not built")


@pytest.fixture(scope="module")
def ops():
    from hstu_jagged_pointwise_amd import ops as o
    return o


@pytest.mark.parametrize("N", [1, 2, 7, 64, 200, 1000, 4096, 8192, 65536])
@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0, 1.2, 1.5, 1.6, 1.8, 2.0])
def test_target_length_matches_oracle(ops, N, alpha):
    _, L = ops.hstu_sl_lengths(np.array([0], np.int64), N, alpha, np.zeros(0, np.float32))
    assert L == SL.target_length(N, alpha)


def test_page_example(ops):
    _, L = ops.hstu_sl_lengths(np.array([0, 4096], np.int64), 4096, 1.6, np.array([0.9], np.float32))
    assert L == 776


@pytest.mark.parametrize("seed", range(4))
def test_lengths_match_oracle(ops, seed):
    def lens(r):
        n = synth.lengths_power_law(r, 300, 1.2, 1, 4096)
        n[::17] = 0  # a few empty sequences
        return n
    x = synth.make_sl(seed, lens, 16, 4096, 1.6, "f32")
    new, L = ops.hstu_sl_lengths(x.offsets, 4096, 1.6, x.u_keep)
    assert np.array_equal(new, SL.sl_lengths(x.offsets, 4096, 1.6, x.u_keep))


def test_keep_whole_boundary(ops):
    # u just below / above (L/n)^2, as float32, around the exact rational
    L, n = 776, 4096
    q = np.float32((L * L) / (n * n))
    lo = np.nextafter(q, np.float32(0))
    hi = np.nextafter(q, np.float32(1))
    off = np.array([0, n, 2 * n, 3 * n], np.int64)
    u = np.array([lo, hi, q], np.float32)
    new, _ = ops.hstu_sl_lengths(off, 4096, 1.6, u)
    assert np.array_equal(new, SL.sl_lengths(off, 4096, 1.6, u))
    assert new[1] == n and new[2] - new[1] == L


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: each case fails validation first


def _sample(ops, off, new, keys=FAKE, src=FAKE, x=None, rb=0, ox=None, ts=None, ots=None, B=None):
    return ops.lib.hstu_sl_sample(len(off) - 1 if B is None else B, ops._i64p(off),
                                  ops._i64p(new) if new is not None else None, FAKE, FAKE, keys,
                                  src, x, rb, ox, ts, ots, None)


def test_sample_rejections(ops):
    off = np.array([0, 5, 12], np.int64)
    assert _sample(ops, off, np.array([0, 6, 8], np.int64)) == ops.HSTU_INVALID_ARGUMENT  # m > n
    assert _sample(ops, off, np.array([1, 3, 8], np.int64)) == ops.HSTU_INVALID_ARGUMENT  # new[0]
    assert _sample(ops, off, np.array([0, 5, 4], np.int64)) == ops.HSTU_INVALID_ARGUMENT  # decreasing
    assert _sample(ops, off, None) == ops.HSTU_INVALID_ARGUMENT
    assert _sample(ops, off, np.array([0, 3, 8], np.int64), keys=None) == ops.HSTU_INVALID_ARGUMENT
    assert _sample(ops, off, np.array([0, 3, 8], np.int64), src=None) == ops.HSTU_INVALID_ARGUMENT
    ok = np.array([0, 3, 8], np.int64)
    assert _sample(ops, off, ok, x=FAKE, rb=24, ox=FAKE) == ops.HSTU_INVALID_ARGUMENT  # rb % 16
    assert _sample(ops, off, ok, x=FAKE, rb=32, ox=None) == ops.HSTU_INVALID_ARGUMENT
    assert _sample(ops, off, ok, x=ctypes.c_void_p(0x10008), rb=32, ox=FAKE) == \
        ops.HSTU_INVALID_ARGUMENT                                                        # alignment
    assert _sample(ops, off, ok, ts=FAKE) == ops.HSTU_INVALID_ARGUMENT
    assert _sample(ops, np.array([0, 5, 3], np.int64), ok) == ops.HSTU_INVALID_ARGUMENT
    assert _sample(ops, off, ok, B=-1) == ops.HSTU_INVALID_ARGUMENT
    # nothing to do: whole sequences need no keys, empty output needs no buffers
    assert _sample(ops, np.array([0], np.int64), np.array([0], np.int64), keys=None, src=None,
                   B=0) == ops.HSTU_OK
    assert _sample(ops, off, np.array([0, 0, 0], np.int64), keys=None, src=None) == ops.HSTU_OK


def test_lengths_rejections(ops):
    off = np.array([0, 5], np.int64)
    u = np.zeros(1, np.float32)
    for N, a in ((0, 1.0), (10, -0.1), (10, 2.5), (10, float("nan"))):
        with pytest.raises(ops.HstuError) as e:
            ops.hstu_sl_lengths(off, N, a, u)
        assert e.value.status == ops.HSTU_INVALID_ARGUMENT
    with pytest.raises(ops.HstuError):
        ops.hstu_sl_lengths(np.array([1, 5], np.int64), 10, 1.0, u)
