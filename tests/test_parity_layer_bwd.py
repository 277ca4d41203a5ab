"""GPU parity of hstu_layer_bwd (gradients of a layer stack) against the fp64 oracle:
dL/dX per token row, each weight gradient per output row, the bias, gamma and beta
gradients as one row each, and the bias tables per head. Tolerances are per row,
relative to the row's largest value: 1e-5 for fp32. For bf16 inputs with fp32
accumulation the bound is 2e-2, or, where bf16 storage of the intermediates alone
moves a row by more, a multiple of that move (the oracle's storage="bf16" variant),
as in the forward layer tests; the median row must still meet 2e-2. The weight, bias and
bias-table gradients are sums over every token or pair: an entry may also differ by the
tolerance times the sum of the magnitudes of its terms (|A|^T |B| for A^T B; the oracle gives
it), the componentwise error bound of a sum, which matters only where the terms cancel."""
import numpy as np
import pytest
import torch

from oracle import hstu_backward as BW
from hstu_jagged_pointwise_amd import synth
from gpu_util import (announce, assert_rows_close, assert_rows_close_storage, assert_sums_close,
                      dev, act_dtype, layer_weights_on_gpu)

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 2e-2}
NAMES = {"dw1": "dw1", "db1": "db1", "d_rab_pos": "d_rab_pos", "d_rab_time": "d_rab_time",
         "d_ln_gamma": "dgamma", "d_ln_beta": "dbeta", "dw2": "dw2", "db2": "db2"}


def run_gpu(x, gy):
    from hstu_jagged_pointwise_amd import ops
    dt = act_dtype(x.dtype)
    dx, grads = ops.hstu_layer_bwd(dev(x.offsets), dev(x.ts), dev(x.x, dt),
                                   layer_weights_on_gpu(x.layers, x.dtype), dev(gy, dt),
                                   num_heads=x.num_heads, d_qk=x.d_qk, d_v=x.d_v,
                                   max_seq_len=x.max_seq_len, ln_eps=x.eps, residual=x.residual,
                                   seq_offsets_host=x.offsets)
    torch.cuda.synchronize()
    return dx, grads


def check(x, gy, what):
    dx, grads = run_gpu(x, gy)
    args = (x.offsets, x.ts, x.x, x.layers, x.num_heads, x.d_qk, x.d_v, x.max_seq_len, gy, x.eps,
            x.residual)
    want_dx, want = BW.layer_stack_backward(*args)
    tol = TOL[x.dtype]
    f = lambda t: t.float().cpu().numpy()
    if x.dtype == "f32":
        close = lambda got, ref, ref_s, name: assert_rows_close(got, ref, tol, name)
        sdx, swant = want_dx, want
    else:
        close = lambda got, ref, ref_s, name: assert_rows_close_storage(got, ref, ref_s, tol,
                                                                        what=name)
        sdx, swant = BW.layer_stack_backward(*args, storage="bf16")
    worst = {"dx": close(f(dx), want_dx, sdx, f"{what} dx")}
    for l, (g, w, ws) in enumerate(zip(grads, want, swant)):
        for k, name in NAMES.items():
            got, ref, ref_s = f(g[k]), np.asarray(getattr(w, name)), np.asarray(getattr(ws, name))
            if got.ndim == 1:
                got, ref, ref_s = got[None, :], ref[None, :], ref_s[None, :]
            terms = getattr(w, name + "_terms", None)
            if terms is not None:  # reductions over tokens or pairs
                terms = np.asarray(terms)
                if terms.ndim == 1:
                    terms = terms[None, :]
                worst[f"{k}[{l}]"] = assert_sums_close(got, ref, ref_s, terms, tol,
                                                       what=f"{what} {k}[{l}]")
            else:
                worst[f"{k}[{l}]"] = close(got, ref, ref_s, f"{what} {k}[{l}]")
    print(f"[{what}] worst row errors: " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()))


def _gy(x, seed):
    return synth.normal(np.random.default_rng(seed), x.x.shape, 1.0, x.dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("residual,num_layers", [(0, 1), (1, 1), (1, 2)])
def test_small_stacks(dtype, residual, num_layers):
    """Ragged lengths over several tiles, an empty and a one-action sequence; random
    biases and LayerNorm affine parameters; d_model 64, 2 heads of width 32."""
    x = synth.make_layer(31, lambda r: np.array([150, 1, 0, 70, 33]), 2, 32, 32, 64, 32, 16, dtype,
                         num_layers=num_layers, random_bias=True, with_ln_affine=True, w_std=0.1,
                         residual=residual)
    announce(f"layer bwd small {dtype} residual={residual} layers={num_layers}")
    check(x, _gy(x, 32), f"small {dtype} r{residual} L{num_layers}")


def test_short_history_batch_full_size():
    """The short-history jagged batch at full size: 256 users, lengths 20-200, d_model 128,
    2 heads of width 64, bf16, one layer."""
    x = synth.workload_short_history_layer()
    announce("layer bwd short-history batch (full size)")
    check(x, _gy(x, 33), "short-history")


def test_heavy_tail_stack_full_size():
    """The heavy-tailed training batch at full size, as the benchmark times it: 32 users,
    bounded power-law lengths on [64, 4096] (19,856 tokens), d_model 512, 8 heads of width
    64, 4 layers, bf16. Every gradient of every layer against the fp64 oracle."""
    x = synth.workload_heavy_tail_stack()
    announce("layer bwd heavy-tail 4-layer stack (full size)")
    check(x, _gy(x, 37), "heavy-tail x4")


def test_empty_batch_writes_zero_gradients():
    from hstu_jagged_pointwise_amd import ops
    x = synth.make_layer(34, lambda r: np.array([0, 0]), 2, 32, 32, 64, 32, 16, "bf16")
    announce("layer bwd empty batch")
    dt = act_dtype(x.dtype)
    xx = torch.zeros((0, 64), dtype=dt, device="cuda")
    dx, grads = ops.hstu_layer_bwd(dev(x.offsets), None, xx, layer_weights_on_gpu(x.layers, x.dtype),
                                   xx, num_heads=2, d_qk=32, d_v=32, max_seq_len=4,
                                   seq_offsets_host=x.offsets)
    torch.cuda.synchronize()
    assert dx.numel() == 0
    for g in grads:
        for k, t in g.items():
            assert torch.all(t == 0), k


def test_repeatable_bit_for_bit():
    x = synth.make_layer(35, lambda r: np.array([300, 64, 5]), 2, 64, 64, 128, 64, 32, "bf16",
                         random_bias=True, with_ln_affine=True)
    gy = _gy(x, 36)
    announce("layer bwd repeatability")
    a = run_gpu(x, gy)
    b = run_gpu(x, gy)
    assert torch.equal(a[0], b[0])
    for ga, gb in zip(a[1], b[1]):
        for k in ga:
            if k in ("d_rab_pos", "d_rab_time"):
                continue  # LDS atomics: equal to rounding only
            assert torch.equal(ga[k], gb[k]), k
