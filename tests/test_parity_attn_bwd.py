"""GPU parity of hstu_attn_bwd (gradients of the ungated attention) against the fp64
backward oracle: every row of dq, dk and dv and every bias-table row, within 1e-5
(fp32) or 2e-2 (bf16 inputs, fp32 accumulation) of the row's largest value.

At the full length-8192 workload the oracle computes sampled rows one at a time.
Three identities check the whole output, because each holds at any size:
  sum_i q_i.dq_i = sum_j k_j.dk_j  (both equal sum_ij dz_ij q_i.k_j, per head);
  sum_j v_j.dv_j = sum_i g_i.o_i   (o is the forward output);
  sum_p d_rab_pos[h][p] = sum_t d_rab_time[h][t]  (both sum every dz of head h)."""
import numpy as np
import pytest
import torch

from oracle import hstu_backward as BW
from hstu_jagged_pointwise_amd import synth
from gpu_util import announce, assert_rows_close, dev, act_dtype, attn_on_gpu

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 2e-2}


def _grad_out(x, seed=99):
    rng = np.random.default_rng(seed)
    return synth.normal(rng, x.v.shape, 1.0, x.dtype)


def bwd_gpu(x, g, rab_pos="x", rab_time="x", ts="x", rab_grads=True):
    from hstu_jagged_pointwise_amd import ops
    dt = act_dtype(x.dtype)
    rp = x.rab_pos if isinstance(rab_pos, str) else rab_pos
    rt = x.rab_time if isinstance(rab_time, str) else rab_time
    tsv = x.ts if isinstance(ts, str) else ts
    out = ops.hstu_attn_bwd(dev(x.offsets), dev(tsv), dev(x.q, dt), dev(x.k, dt), dev(x.v, dt),
                            dev(g, dt), dev(rp), dev(rt), max_seq_len=x.max_seq_len,
                            num_pos_buckets=x.num_pos_buckets, num_time_buckets=x.num_time_buckets,
                            rab_grads=rab_grads, seq_offsets_host=x.offsets)
    torch.cuda.synchronize()
    return out


def bwd_oracle(x, g, rab_pos="x", rab_time="x", ts="x"):
    rp = x.rab_pos if isinstance(rab_pos, str) else rab_pos
    rt = x.rab_time if isinstance(rab_time, str) else rab_time
    tsv = x.ts if isinstance(ts, str) else ts
    return BW.attention_backward(x.offsets, tsv, x.q, x.k, x.v, rp, rt, x.max_seq_len, g,
                                 P=x.num_pos_buckets, T=x.num_time_buckets)


def check_all(x, got, want, what, tables=True):
    tol = TOL[x.dtype]
    f = lambda t: t.float().cpu().numpy()
    for name, a, b in zip(("dq", "dk", "dv"), got[:3], want[:3]):
        assert_rows_close(f(a), b, tol, f"{what} {name}")
    if tables:
        assert_rows_close(f(got[3]), want[3], tol, f"{what} d_rab_pos")
        assert_rows_close(f(got[4]), want[4], tol, f"{what} d_rab_time")


def test_tiny_fp32():
    x = synth.workload_tiny_attention()
    g = _grad_out(x)
    announce("attn bwd tiny fp32")
    check_all(x, bwd_gpu(x, g), bwd_oracle(x, g), "tiny fp32")


@pytest.mark.parametrize("dtype,dqk,dv", [("f32", 32, 64), ("f32", 64, 32), ("f32", 128, 128),
                                          ("bf16", 32, 32), ("bf16", 64, 64), ("bf16", 128, 128),
                                          ("bf16", 64, 128)])
def test_ragged_tiles(dtype, dqk, dv):
    """Lengths across several 64-row tiles with ragged tails, an empty and a
    one-action sequence; 128 position and 64 time buckets (clamping occurs)."""
    x = synth.make_attn(11, lambda r: np.array([300, 1, 129, 0, 64, 65]), 2, dqk, dv, 128, 64,
                        dtype)
    g = _grad_out(x, 12)
    announce(f"attn bwd ragged {dtype} d_qk={dqk} d_v={dv}")
    check_all(x, bwd_gpu(x, g), bwd_oracle(x, g), f"ragged {dtype} {dqk}/{dv}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["no_timestamps", "no_tables", "no_table_grads", "pos_clamp"])
def test_bias_variants(variant, dtype):
    """P = 8 makes most blocks of the 600-long sequence take one position bucket."""
    P = 8 if variant == "pos_clamp" else 128
    x = synth.make_attn(13, lambda r: np.array([600, 37, 90]), 2, 64, 64, P, 64, dtype)
    g = _grad_out(x, 14)
    announce(f"attn bwd bias variant {variant} {dtype}")
    if variant == "no_timestamps":
        check_all(x, bwd_gpu(x, g, ts=None), bwd_oracle(x, g, ts=None), variant)
    elif variant == "no_tables":
        check_all(x, bwd_gpu(x, g, rab_pos=None, rab_time=None),
                  bwd_oracle(x, g, rab_pos=None, rab_time=None), variant)
    elif variant == "no_table_grads":
        got = bwd_gpu(x, g, rab_grads=False)
        assert got[3] is None and got[4] is None
        check_all(x, got, bwd_oracle(x, g), variant, tables=False)
    else:
        check_all(x, bwd_gpu(x, g), bwd_oracle(x, g), variant)


def test_empty_batches_write_zero_table_gradients():
    from hstu_jagged_pointwise_amd import ops
    for lens in ([], [0, 0, 0]):
        x = synth.make_attn(15, lambda r: np.array(lens, np.int64), 2, 32, 32, 16, 8, "f32")
        announce(f"attn bwd empty lengths={lens}")
        q = torch.zeros((0, 2, 32), device="cuda")
        off = dev(x.offsets)
        dq, dk, dv, drp, drt = ops.hstu_attn_bwd(off, None, q, q, q, q, max_seq_len=4,
                                                 num_pos_buckets=16, num_time_buckets=8,
                                                 seq_offsets_host=x.offsets)
        torch.cuda.synchronize()
        assert dq.numel() == 0
        assert torch.all(drp == 0) and torch.all(drt == 0)
        assert drp.shape == (2, 16) and drt.shape == (2, 8)


def test_repeatable_bit_for_bit():
    x = synth.make_attn(16, lambda r: np.array([257, 64, 3]), 2, 64, 64, 128, 64, "bf16")
    g = _grad_out(x, 17)
    announce("attn bwd repeatability")
    a = bwd_gpu(x, g)
    b = bwd_gpu(x, g)
    for name, s, t in zip(("dq", "dk", "dv"), a[:3], b[:3]):
        assert torch.equal(s, t), name
    # the table gradients are summed with LDS atomics: equal to rounding
    for s, t in zip(a[3:], b[3:]):
        assert torch.allclose(s, t, rtol=1e-5, atol=1e-6 * float(s.abs().max()))


def test_long_sequences_full_size():
    """The length-8192 workload: 8 sequences of 4096-8192 actions, 4 heads, d = 128, bf16."""
    x = synth.workload_long_attention()
    g = _grad_out(x, 18)
    announce("attn bwd full size (8 x 4096..8192, H=4, d=128, bf16)")
    dq, dk, dv, drp, drt = bwd_gpu(x, g)
    off = x.offsets
    rng = np.random.default_rng(19)
    rows = {int(off[0]), int(off[1]) - 1, int(off[1]) - 64, int(off[1]) - 65, int(off[3]),
            int(off[-1]) - 1}
    rows |= set(int(r) for r in rng.integers(0, int(off[-1]), size=10))
    rows = sorted(rows)
    wq, wk, wv = BW.attention_backward_rows(off, x.ts, x.q, x.k, x.v, x.rab_pos, x.rab_time,
                                            x.max_seq_len, g, rows)
    f = lambda t: t[rows].float().cpu().numpy()
    tol = TOL[x.dtype]
    assert_rows_close(f(dq), wq, tol, "full dq")
    assert_rows_close(f(dk), wk, tol, "full dk")
    assert_rows_close(f(dv), wv, tol, "full dv")
    # identities over the whole output, per head, in fp64 from the stored values
    q64 = x.q.astype(np.float64)
    k64 = x.k.astype(np.float64)
    v64 = x.v.astype(np.float64)
    g64 = g.astype(np.float64)
    dq64, dk64, dv64 = (t.double().cpu().numpy() for t in (dq, dk, dv))
    o = attn_on_gpu(x).double().cpu().numpy()
    for h in range(x.num_heads):
        lhs = np.einsum("rc,rc->r", q64[:, h], dq64[:, h])
        rhs = np.einsum("rc,rc->r", k64[:, h], dk64[:, h])
        scale = np.abs(lhs).sum() + np.abs(rhs).sum()
        assert abs(lhs.sum() - rhs.sum()) <= tol * scale, f"q.dq vs k.dk, head {h}"
        lhs = np.einsum("rc,rc->r", v64[:, h], dv64[:, h])
        rhs = np.einsum("rc,rc->r", g64[:, h], o[:, h])
        scale = np.abs(lhs).sum() + np.abs(rhs).sum()
        assert abs(lhs.sum() - rhs.sum()) <= tol * scale, f"v.dv vs g.o, head {h}"
        sp, st = drp[h].double().sum().item(), drt[h].double().sum().item()
        mag = drp[h].double().abs().sum().item() + drt[h].double().abs().sum().item()
        assert abs(sp - st) <= 1e-4 * mag, f"table sums, head {h}"


@pytest.mark.parametrize("gap", [700, 3])
def test_even_timestamps_two_bucket_blocks(gap):
    """Timestamps `gap` seconds apart with 8 position buckets: away from the diagonal most
    32x32 blocks have one position bucket and an elapsed-time range that covers one or
    two adjacent time buckets, so the constant and two-bucket block paths carry most of
    the work; the table gradients check their bucket sums."""
    x = synth.make_attn(21, lambda r: np.array([1024, 333]), 2, 64, 64, 8, 64, "bf16")
    x.ts = (np.concatenate([np.arange(1024), np.arange(333)]) * gap + 1_700_000_000).astype(np.int64)
    g = _grad_out(x, 22)
    announce(f"attn bwd even timestamps gap={gap}")
    check_all(x, bwd_gpu(x, g), bwd_oracle(x, g), f"even ts {gap}")
