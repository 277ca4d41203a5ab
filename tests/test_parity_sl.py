"""GPU parity of Stochastic Length sampling (hstu_sl_lengths + hstu_sl_sample)
against the oracle. Selection and gathers are integer and byte work, so they must
match bit for bit: the source index of every kept row, the gathered rows and the
gathered timestamps."""
import numpy as np
import pytest
import torch

from oracle import stochastic_length as SL
from hstu_jagged_pointwise_amd import synth
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu


def _keys_dev(keys):
    return dev(np.ascontiguousarray(keys, np.uint32).view(np.int32))


def _run(off, new, keys, x=None, ts=None, x_torch_dtype=None):
    from hstu_jagged_pointwise_amd import ops
    xd = None
    if x is not None:
        xd = dev(x, x_torch_dtype)
    src, ox, ots = ops.hstu_sl_sample(dev(off), dev(new), _keys_dev(keys), xd, dev(ts),
                                      offsets_host=off, new_offsets_host=new)
    torch.cuda.synchronize()
    return src.cpu().numpy(), ox, None if ots is None else ots.cpu().numpy()


def _offsets(lengths):
    return synth.offsets_from_lengths(np.asarray(lengths, np.int64))


def test_selection_edge_lengths():
    rng = np.random.default_rng(21)
    lens = [0, 1, 2, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 1000, 3, 7]
    off = _offsets(lens)
    keys = rng.integers(0, 2**32, size=int(off[-1]), dtype=np.uint64).astype(np.uint32)
    for case in ("whole", "empty", "one", "all_but_one", "random"):
        m = []
        for n in lens:
            m.append({"whole": n, "empty": 0, "one": min(1, n), "all_but_one": max(n - 1, 0),
                      "random": int(rng.integers(0, n + 1))}[case])
        new = _offsets(m)
        announce(f"sl select edge lengths, {case}")
        src, _, _ = _run(off, new, keys)
        assert np.array_equal(src, SL.sl_select(off, new, keys)), case


@pytest.mark.parametrize("kind", ["ties4", "all_zero", "all_max", "two_values"])
def test_selection_ties_broken_by_position(kind):
    rng = np.random.default_rng(22)
    lens = rng.integers(1, 700, size=12)
    off = _offsets(lens)
    T = int(off[-1])
    keys = {"ties4": rng.integers(0, 4, size=T),
            "all_zero": np.zeros(T),
            "all_max": np.full(T, 2**32 - 1),
            "two_values": np.where(rng.random(T) < 0.5, 7, 2**31 + 5)}[kind].astype(np.uint32)
    new = _offsets([int(rng.integers(0, n)) for n in lens])  # every sequence cut
    announce(f"sl select ties, {kind}")
    src, _, _ = _run(off, new, keys)
    assert np.array_equal(src, SL.sl_select(off, new, keys))


@pytest.mark.parametrize("n,m,key_range", [
    (200_000, 1000, 2**32), (200_000, 150_000, 2**32), (70_001, 70_000, 2**32),
    (8192, 100, 2**32), (8193, 5000, 2**32), (20_000, 7_000, 4), (8192, 3000, 3)])
def test_selection_one_long_sequence(n, m, key_range):
    """Sequences on both sides of the length up to which the keys are staged on chip,
    with and without heavy ties."""
    rng = np.random.default_rng(n + m)
    off = np.array([0, n], np.int64)
    new = np.array([0, m], np.int64)
    keys = rng.integers(0, key_range, size=n, dtype=np.uint64).astype(np.uint32)
    announce(f"sl select one sequence n={n} m={m} key_range={key_range}")
    src, _, _ = _run(off, new, keys)
    assert np.array_equal(src, SL.sl_select(off, new, keys))


def test_heavy_tail_batch_full_size():
    """The heavy-tailed training batch (32 users, lengths up to 4096, d_model 512, bf16)
    at N = 4096, alpha = 1.6: lengths, source rows, rows and timestamps, all exact."""
    from hstu_jagged_pointwise_amd import ops
    x = synth.workload_sl_heavy_tail()
    new, L = ops.hstu_sl_lengths(x.offsets, x.max_seq_len, x.alpha, x.u_keep)
    assert L == 776
    want_new = SL.sl_lengths(x.offsets, x.max_seq_len, x.alpha, x.u_keep)
    assert np.array_equal(new, want_new)
    announce("sl sample heavy-tail batch, bf16 rows + timestamps")
    src, ox, ots = _run(x.offsets, new, x.keys, x.x, x.ts, torch.bfloat16)
    want_src = SL.sl_select(x.offsets, want_new, x.keys)
    assert np.array_equal(src, want_src)
    want_x, want_ts = SL.sl_gather(synth.bf16_bits(x.x), x.ts, want_src)
    got_bits = ox.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_bits, want_x)
    assert np.array_equal(ots, want_ts)
    lens = np.diff(x.offsets)
    assert (lens > L).any() and (np.diff(new) == L).any()  # the batch exercises cutting


@pytest.mark.parametrize("what", ["f32_rows16", "bf16_rows16", "ts_only", "rows_only"])
def test_gather_variants(what):
    rng = np.random.default_rng(23)
    lens = [0, 40, 1, 300, 129]
    off = _offsets(lens)
    T = int(off[-1])
    keys = rng.integers(0, 2**32, size=T, dtype=np.uint64).astype(np.uint32)
    new = _offsets([0, 17, 1, 300, 64])
    ts = synth.timestamps(rng, lens)
    want_src = SL.sl_select(off, new, keys)
    announce(f"sl gather {what}")
    if what == "f32_rows16":
        x = rng.standard_normal((T, 4)).astype(np.float32)
        src, ox, ots = _run(off, new, keys, x, ts)
        assert np.array_equal(ox.cpu().numpy(), x[want_src]) and np.array_equal(ots, ts[want_src])
    elif what == "bf16_rows16":
        x = synth.round_bf16(rng.standard_normal((T, 8)).astype(np.float32))
        src, ox, ots = _run(off, new, keys, x, ts, torch.bfloat16)
        assert np.array_equal(ox.float().cpu().numpy(), x[want_src])
    elif what == "ts_only":
        src, ox, ots = _run(off, new, keys, None, ts)
        assert ox is None and np.array_equal(ots, ts[want_src])
    else:
        x = rng.standard_normal((T, 36)).astype(np.float32)
        src, ox, ots = _run(off, new, keys, x, None)
        assert ots is None and np.array_equal(ox.cpu().numpy(), x[want_src])
    assert np.array_equal(src, want_src)
