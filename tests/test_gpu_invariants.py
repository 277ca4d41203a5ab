"""Invariants of the GPU attention path, bit for bit (each output row has a fixed
reduction order, whatever the batch around it): jagged = each sequence alone,
future and other-sequence keys never leak, repeated runs agree, reordering the
sequences permutes the outputs."""
import numpy as np
import pytest
import torch

from hstu_jagged_pointwise_amd import synth
from gpu_util import announce, attn_on_gpu

pytestmark = pytest.mark.gpu


def _np(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_jagged_equals_each_sequence_alone(dt, d):
    x = synth.make_attn(40, lambda r: np.array([300, 0, 129, 64, 1]), 2, d, d, 64, 32, dt,
                        with_u=True, max_seq_len=300)
    announce(f"jagged vs alone {dt} d={d}")
    full = _np(attn_on_gpu(x))
    fullg = _np(attn_on_gpu(x, with_u=True))
    for b in range(5):
        s, e = int(x.offsets[b]), int(x.offsets[b + 1])
        if e == s:
            continue
        y = synth.AttnInputs(np.array([0, e - s]), x.ts[s:e], x.q[s:e], x.k[s:e], x.v[s:e],
                             x.u[s:e], x.rab_pos, x.rab_time, None, None, 2, d, d, 64, 32, 300, dt)
        assert np.array_equal(_np(attn_on_gpu(y)), full[s:e])
        assert np.array_equal(_np(attn_on_gpu(y, with_u=True)), fullg[s:e])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_future_keys_do_not_leak_and_runs_repeat(dt):
    x = synth.make_attn(41, lambda r: np.array([260, 100]), 2, 64, 64, 64, 32, dt)
    announce(f"leak/repeat {dt}")
    base = _np(attn_on_gpu(x))
    for _ in range(3):
        assert np.array_equal(_np(attn_on_gpu(x)), base)
    cut = 150
    x2 = synth.AttnInputs(**{**x.__dict__})
    x2.k = x.k.copy()
    x2.v = x.v.copy()
    ts2 = x.ts.copy()
    x2.k[cut:] = x2.k[cut:] * -3 + 1
    x2.v[cut:] = x2.v[cut:] * 5
    ts2[cut:260] += 123456789
    x2.ts = ts2
    assert np.array_equal(_np(attn_on_gpu(x2))[:cut], base[:cut])


def test_sequence_reorder_permutes_outputs():
    x = synth.make_attn(42, lambda r: np.array([70, 200, 5, 129]), 2, 64, 64, 64, 32, "bf16",
                        max_seq_len=200)
    announce("sequence reorder")
    base = _np(attn_on_gpu(x))
    perm = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(x.offsets[b], x.offsets[b + 1]) for b in perm])
    y = synth.AttnInputs(synth.offsets_from_lengths(x.lengths[perm]), x.ts[idx], x.q[idx],
                         x.k[idx], x.v[idx], None, x.rab_pos, x.rab_time, None, None, 2, 64, 64, 64,
                         32, 200, "bf16")
    assert np.array_equal(_np(attn_on_gpu(y)), base[idx])
