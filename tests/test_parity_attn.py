"""GPU parity of hstu_attn_fwd against the fp64 oracle.

Tolerances, per output row (infinity norm, relative): 1e-5 for fp32 inputs and
2e-2 for bf16 inputs with fp32 accumulation. A row that the oracle makes exactly
zero must be exactly zero on the GPU. Shapes span several 128-row tiles and
ragged tails, and include empty and length-1 sequences."""
import numpy as np
import pytest

from oracle import hstu_oracle as O
from hstu_jagged_pointwise_amd import synth
from gpu_util import announce, assert_rows_close, attn_on_gpu, to_np

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _oracle(x, with_u=False, **kw):
    rp = kw.get("rab_pos", x.rab_pos)
    rt = kw.get("rab_time", x.rab_time)
    ts = kw.get("ts", x.ts)
    q = kw.get("q", x.q)
    return O.hstu_attention(x.offsets, ts, q, x.k, x.v, rp, rt, x.max_seq_len,
                            u=x.u if with_u else None, gamma=x.gamma, beta=x.beta, eps=x.eps)


@pytest.mark.parametrize("with_u", [False, True])
def test_tiny_fp32_workload(with_u):
    x = synth.workload_tiny_attention(seed=0, with_u=True)
    announce(f"tiny fp32 attention, gated={with_u}, lens={x.lengths.tolist()}")
    g = to_np(attn_on_gpu(x, with_u))
    assert_rows_close(g, _oracle(x, with_u), TOL["f32"], "tiny fp32")


RAGGED = lambda r: np.array([0, 1, 127, 128, 129, 300, 5, 256])


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("H", [1, 3])
@pytest.mark.parametrize("with_u", [False, True])
def test_bf16_mfma_ragged(d, H, with_u):
    x = synth.make_attn(100 + d + H, RAGGED, H, d, d, 64, 32, "bf16", with_u=True,
                        with_ln_affine=True, rab_std=0.5)
    announce(f"bf16 MFMA attention d={d} H={H} gated={with_u}")
    g = to_np(attn_on_gpu(x, with_u))
    assert_rows_close(g, _oracle(x, with_u), TOL["bf16"], f"bf16 d={d} H={H}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("dqk,dv", [(64, 128), (128, 32), (32, 64)])
def test_mixed_head_widths(dt, dqk, dv):
    x = synth.make_attn(7, lambda r: np.array([70, 0, 33, 150]), 2, dqk, dv, 32, 32, dt,
                        with_u=True)
    announce(f"mixed widths {dt} d_qk={dqk} d_v={dv}")
    assert_rows_close(to_np(attn_on_gpu(x)), _oracle(x), TOL[dt], "mixed widths")
    assert_rows_close(to_np(attn_on_gpu(x, True)), _oracle(x, True), TOL[dt], "mixed gated")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_optional_bias_terms(dt):
    x = synth.make_attn(8, lambda r: np.array([200, 17, 64]), 2, 64, 64, 64, 32, dt, rab_std=0.5)
    for name, kw in [("no tables", dict(rab_pos=None, rab_time=None)),
                     ("no time table", dict(rab_time=None)),
                     ("no timestamps", dict(ts=None)),
                     ("no position table", dict(rab_pos=None))]:
        announce(f"{dt} {name}")
        g = to_np(attn_on_gpu(x, **kw))
        assert_rows_close(g, _oracle(x, **kw), TOL[dt], f"{dt} {name}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_wide_and_unsorted_timestamps(dt):
    """Elapsed times beyond 2^31 s take the 64-bit bucket path; unsorted timestamps give
    negative elapsed times, which clamp to bucket 0."""
    x = synth.make_attn(9, lambda r: np.array([190, 77]), 2, 64, 64, 64, 64, dt, rab_std=0.5)
    rng = np.random.default_rng(9)
    wide = x.ts.copy()
    wide[:190] = synth.T0 + np.cumsum(rng.integers(1, 3 * 10**8, size=190))  # spans ~3e10 s
    wide[190:] = rng.permutation(wide[190:])
    announce(f"{dt} wide/unsorted timestamps")
    g = to_np(attn_on_gpu(x, ts=wide))
    assert_rows_close(g, _oracle(x, ts=wide), TOL[dt], "wide timestamps")


@pytest.mark.parametrize("d", [64, 128])
def test_largest_tables_on_mfma_kernel(d):
    """P = 1024, the largest position table the MFMA kernel keeps in LDS, and T = 64 time
    buckets, with a sequence long enough (1,300) to reach position bucket 1023."""
    x = synth.make_attn(12, lambda r: np.array([1300, 5, 257]), 2, d, d, 1024, 64, "bf16",
                        rab_std=0.5)
    announce(f"bf16 P=1024 T=64 d={d}")
    assert_rows_close(to_np(attn_on_gpu(x)), _oracle(x), TOL["bf16"], f"P=1024 d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_key_block_groups(d):
    """The MFMA kernel decides the bias path of 64 key blocks (2,048 keys) at a time: rows
    that see exactly 2,048 keys, one more, and 4,160 (into a third group), beside a short
    sequence, with both bias tables."""
    x = synth.make_attn(13, lambda r: np.array([2048, 2049, 31, 4160]), 2, d, d, 128, 64, "bf16",
                        rab_std=0.5)
    announce(f"bf16 key-block groups d={d}")
    assert_rows_close(to_np(attn_on_gpu(x)), _oracle(x), TOL["bf16"], f"key-block groups d={d}")


def test_large_position_table_falls_back_to_vector_kernel():
    x = synth.make_attn(10, lambda r: np.array([1500, 40]), 2, 64, 64, 2048, 64, "bf16",
                        rab_std=0.5)
    announce("bf16 P=2048 (vector kernel)")
    assert_rows_close(to_np(attn_on_gpu(x)), _oracle(x), TOL["bf16"], "P=2048")


def test_long_sequence_workload_every_row():
    """The length-8192 workload (B=8, H=4, d=128, 46,858 rows) in the launch configuration
    the benchmark times: every row of every head within a flat 2e-2 of the fp64 oracle."""
    x = synth.workload_long_attention()
    announce(f"long attention, T_tot={int(x.offsets[-1])}")
    g = to_np(attn_on_gpu(x))
    d = x.d_v
    assert_rows_close(g.reshape(-1, d), _oracle(x).reshape(-1, d), TOL["bf16"],
                      "length 8192, every (row, head)")
