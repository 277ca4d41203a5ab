"""Bucket indices, bit-exact, on the GPU.

1. hstu_debug_buckets (the kernels' device functions) against the oracle's bucket
   functions, element for element, on crafted timestamps: power-of-two boundaries,
   spans beyond 2^31 s, unsorted values.
2. A decode test through the real attention kernels. With Q = 0 every score is the
   bias alone. With one-hot V the output row i holds SiLU(bias(i, j)) / N at
   column j. With table entries 20 + index, SiLU(x) equals x to within e^-20 and
   N = 128 is a power of two. The fp32 kernel reproduces 20 + bucket exactly. The
   bf16 MFMA kernel carries P as bf16(-log2(e) SiLU(x)) and divides -log2(e) out in
   its output scale, so P and the bf16 output are each rounded once (2^-9 relative
   each): the output times N lies within 83 * 2^-8 < 0.5 of 20 + bucket, and rounding
   it recovers the bucket index exactly. Hidden pairs read exactly 0 on both."""
import numpy as np
import pytest
import torch

from oracle import hstu_oracle as O
from hstu_jagged_pointwise_amd import synth
from gpu_util import announce, attn_on_gpu, dev

pytestmark = pytest.mark.gpu


def _crafted_timestamps():
    seqs = []
    # power-of-two boundaries of dt: 2^k - 2, 2^k - 1, 2^k for several k, from a base
    base = synth.T0
    pts = [0]
    for k in range(1, 31):
        pts += [(1 << k) - 2, (1 << k) - 1, 1 << k]
    seqs.append(base + np.array(sorted(set(pts)), np.int64))
    # a span beyond 2^31 and 2^32 seconds (64-bit path)
    seqs.append(base + np.array([0, 5, 2**31 - 3, 2**31 + 7, 2**32 + 1, 2**35, 2**40 + 3], np.int64))
    # unsorted
    rng = np.random.default_rng(1)
    seqs.append(base + rng.integers(0, 10**6, size=50).astype(np.int64))
    return seqs


def test_debug_buckets_match_oracle():
    from hstu_jagged_pointwise_amd import ops
    seqs = _crafted_timestamps()
    off = synth.offsets_from_lengths([len(s) for s in seqs])
    ts = np.concatenate(seqs)
    for P, T in [(64, 32), (128, 64), (8, 64)]:
        for b, s in enumerate(seqs):
            announce(f"debug buckets seq={b} P={P} T={T}")
            pb, tb = ops.hstu_debug_buckets(dev(off), dev(ts), b, max_seq_len=200,
                                            num_pos_buckets=P, num_time_buckets=T,
                                            seq_offsets_host=off)
            torch.cuda.synchronize()
            pb, tb = pb.cpu().numpy(), tb.cpu().numpy()
            n = len(s)
            i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
            vis = j <= i
            want_p = O.pos_bucket(i - j, P)
            want_t = O.time_bucket(s[:, None] - s[None, :], T)
            assert np.array_equal(pb[vis], want_p[vis])
            assert np.array_equal(tb[vis], want_t[vis])
            assert np.all(pb[~vis] == -1) and np.all(tb[~vis] == -1)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("which", ["pos", "time"])
def test_decode_buckets_through_attention_kernel(dt, d, which):
    n_max = min(d, 128)
    lens = [n_max, n_max // 2 + 3]
    seqs = _crafted_timestamps()
    x = synth.make_attn(3, lambda r: np.array(lens), 1, d, d, 64, 64, dt, max_seq_len=128)
    ts = x.ts.copy()
    ts[:lens[0]] = seqs[0][:lens[0]] if len(seqs[0]) >= lens[0] else ts[:lens[0]]
    ts[lens[0]:lens[0] + 7] = seqs[1]
    # one-hot values: v_j = e_j (position within its sequence); zero queries
    v = np.zeros_like(x.v)
    for b in range(2):
        s, e = x.offsets[b], x.offsets[b + 1]
        for jj in range(e - s):
            v[s + jj, 0, jj] = 1.0
    x.v = v
    q = np.zeros_like(x.q)
    table = (20.0 + np.arange(64, dtype=np.float32))[None, :]
    kw = dict(rab_pos=table, rab_time=None, ts=ts) if which == "pos" else \
        dict(rab_pos=None, rab_time=table, ts=ts)
    announce(f"decode {which} buckets {dt} d={d}")
    out = attn_on_gpu(x, q=q, **kw).float().cpu().numpy()[:, 0, :]
    for b in range(2):
        s, e = int(x.offsets[b]), int(x.offsets[b + 1])
        n = e - s
        blk = out[s:e, :n] * 128.0
        i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
        vis = j <= i
        if which == "pos":
            want = 20 + O.pos_bucket(i - j, 64)
        else:
            want = 20 + O.time_bucket(ts[s:e][:, None] - ts[s:e][None, :], 64)
        if dt == "f32":
            assert np.array_equal(blk[vis], want[vis].astype(np.float32)), f"{which} b={b}"
        else:
            err = np.abs(blk[vis] - want[vis])
            assert err.max() <= 83 * 2.0**-8, f"{which} b={b}: {err.max()}"
            assert np.array_equal(np.rint(blk[vis]), want[vis].astype(np.float32)), f"{which} b={b}"
        assert np.all(blk[~vis] == 0.0)
        assert np.all(out[s:e, n:] == 0.0)
