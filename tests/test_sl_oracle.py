"""Pins of the Stochastic Length oracle (CPU): the page's worked number, closed
forms, a second route for the selection, and the sampling distribution."""
import math
from fractions import Fraction
from itertools import combinations

import numpy as np
import pytest

from oracle import stochastic_length as SL


def test_page_example_4096_becomes_776():
    # HSTU chapter, "Three more scaling components", Stochastic Length: alpha = 1.6
    # turns a length of 4,096 into 776
    assert SL.target_length(4096, 1.6) == 776


@pytest.mark.parametrize("N", [1, 2, 3, 4, 15, 16, 17, 100, 4096, 8192, 65536])
def test_target_length_closed_forms(N):
    assert SL.target_length(N, 1.0) == math.isqrt(N)  # floor(sqrt(N)) by integer square root
    assert SL.target_length(N, 2.0) == N
    assert SL.target_length(N, 0.0) == 1


def test_target_length_exact_powers_do_not_round_down():
    assert SL.target_length(4096, 1.5) == 512      # 4096 ** 0.75
    assert SL.target_length(65536, 1.5) == 4096    # 65536 ** 0.75
    assert SL.target_length(1024, 1.2) == 64       # 1024 ** 0.6


def test_keep_whole_rule():
    L = 776
    for n in (1, 500, 776):
        assert SL.keep_whole(n, L, 0.999)          # short sequences are never cut
    n = 4096
    q = Fraction(L * L, n * n)                     # keep probability, exact
    below = np.nextafter(np.float32(float(q)), np.float32(0))
    above = np.nextafter(np.float32(float(q)), np.float32(1))
    assert Fraction(float(below)) < q < Fraction(float(above))
    assert SL.keep_whole(n, L, float(below))
    assert not SL.keep_whole(n, L, float(above))
    assert not SL.keep_whole(n, L, 0.5)


def _select_by_sorting(keys, m):
    """The m smallest (key, position) pairs by plain Python sorting, positions in order."""
    n = len(keys)
    chosen = sorted(range(n), key=lambda p: (int(keys[p]), p))[:m]
    return sorted(chosen)


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_a_second_route(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 40, size=7)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    # small key range: many ties, broken by position
    keys = rng.integers(0, 6 if seed % 2 else 2**32, size=int(off[-1])).astype(np.uint32)
    new_len = [int(n) if rng.random() < 0.3 else int(rng.integers(0, n + 1)) for n in lens]
    new = np.concatenate([[0], np.cumsum(new_len)]).astype(np.int64)
    src = SL.sl_select(off, new, keys)
    for b in range(len(lens)):
        s, n, m = int(off[b]), int(lens[b]), new_len[b]
        got = list(src[new[b]:new[b + 1]] - s)
        want = list(range(n)) if m == n else _select_by_sorting(keys[s:s + n], m)
        assert got == want


def test_lengths_and_invariants():
    rng = np.random.default_rng(3)
    N, alpha = 300, 1.6
    L = SL.target_length(N, alpha)
    lens = np.array([0, 5, L, L + 1, 150, 299, 300, 64], np.int64)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    u = rng.random(len(lens)).astype(np.float32)
    new = SL.sl_lengths(off, N, alpha, u)
    for b, n in enumerate(lens):
        m = int(new[b + 1] - new[b])
        assert m == (n if SL.keep_whole(int(n), L, u[b]) else L)
        assert m in (n, L) and m <= max(n, 0)
    keys = rng.integers(0, 2**32, size=int(off[-1]), dtype=np.uint64).astype(np.uint32)
    src = SL.sl_select(off, new, keys)
    for b in range(len(lens)):
        part = src[new[b]:new[b + 1]]
        assert np.all(np.diff(part) > 0)                          # order kept, no repeats
        assert np.all((part >= off[b]) & (part < off[b + 1]))    # inside its own sequence
    x = rng.standard_normal((int(off[-1]), 3))
    ts = np.arange(int(off[-1]), dtype=np.int64) * 10
    gx, gts = SL.sl_gather(x, ts, src)
    assert np.array_equal(gx, x[src]) and np.array_equal(gts, ts[src])


def test_4096_becomes_776_most_of_the_time():
    """Under the keep-whole reading, a 4096-long history is cut to 776 with
    probability 1 - (776/4096)^2 = 0.964."""
    rng = np.random.default_rng(11)
    u = rng.random(20000).astype(np.float32)
    cut = np.mean([not SL.keep_whole(4096, 776, x) for x in u])
    p = 1 - (776 / 4096) ** 2
    assert abs(cut - p) < 4 * math.sqrt(p * (1 - p) / len(u))


def test_subsequence_is_uniform():
    """Every m-subset of positions is equally likely under uniform keys."""
    rng = np.random.default_rng(5)
    n, m, trials = 5, 2, 30000
    counts = {c: 0 for c in combinations(range(n), m)}
    off = np.array([0, n], np.int64)
    new = np.array([0, m], np.int64)
    for _ in range(trials):
        keys = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
        counts[tuple(SL.sl_select(off, new, keys))] += 1
    expect = trials / len(counts)
    chi2 = sum((v - expect) ** 2 / expect for v in counts.values())
    assert chi2 < 30  # 9 degrees of freedom; p ~ 4e-4 at 30
