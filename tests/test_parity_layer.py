"""GPU parity of hstu_layer_fwd (eqs. 1-3, one layer or a stack) against the fp64 oracle.

fp32: every row within 1e-5 (infinity norm, relative). bf16 with fp32 accumulation:
every row within max(2e-2 |o|, 4 |o_s - o|), where o_s is the oracle with bf16
storage of U, V, Q, K, G and Y. Deep random-init stacks without a residual are
ill-conditioned: bf16 storage alone moves some rows by up to 100%. The median
row must still be within 2e-2."""
import numpy as np
import pytest
import torch

from oracle import hstu_oracle as O
from hstu_jagged_pointwise_amd import synth
from gpu_util import (announce, assert_rows_close, assert_rows_close_storage, dev, act_dtype,
                      layer_weights_on_gpu, to_np)

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 2e-2}


def layer_on_gpu(x):
    from hstu_jagged_pointwise_amd import ops
    dt = act_dtype(x.dtype)
    y = ops.hstu_layer_fwd(dev(x.offsets), dev(x.ts), dev(x.x, dt),
                           layer_weights_on_gpu(x.layers, x.dtype), num_heads=x.num_heads,
                           d_qk=x.d_qk, d_v=x.d_v, max_seq_len=x.max_seq_len, ln_eps=x.eps,
                           residual=x.residual, seq_offsets_host=x.offsets)
    torch.cuda.synchronize()
    return to_np(y)


def layer_oracle(x, storage=None):
    return O.hstu_layer_stack(x.offsets, x.ts, x.x, x.layers, x.num_heads, x.d_qk, x.d_v,
                              x.max_seq_len, x.eps, x.residual, storage)


def check_layer(x, what):
    g = layer_on_gpu(x)
    if x.dtype == "f32":
        return assert_rows_close(g, layer_oracle(x), TOL["f32"], what)
    return assert_rows_close_storage(g, layer_oracle(x), layer_oracle(x, "bf16"), TOL["bf16"],
                                     what=what)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("residual", [0, 1])
@pytest.mark.parametrize("num_layers", [1, 2, 3])
def test_small_layer_stack(dt, residual, num_layers):
    x = synth.make_layer(20 + num_layers, lambda r: np.array([0, 1, 130, 64, 257, 9]), 2, 64, 64,
                         96, 32, 16, dt, num_layers=num_layers, w_std=0.1, random_bias=True,
                         with_ln_affine=True, residual=residual)
    announce(f"layer stack {dt} L={num_layers} residual={residual}")
    check_layer(x, f"layer {dt} L={num_layers}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_layer_other_widths(dt):
    x = synth.make_layer(31, lambda r: np.array([50, 200, 3]), 3, 32, 128, 40, 64, 32, dt,
                         num_layers=2, w_std=0.1, random_bias=True, with_ln_affine=True)
    announce(f"layer {dt} d_qk=32 d_v=128 d_model=40")
    check_layer(x, "layer widths")


def test_short_history_workload_full():
    """B=256 short histories (lengths 20..200), H=2, d=64, d_model=128, bf16: every row."""
    x = synth.workload_short_history_layer()
    announce(f"short-history layer, T_tot={int(x.offsets[-1])}")
    check_layer(x, "short-history layer")


def test_heavy_tail_four_layer_stack_full():
    """B=32 power-law lengths (64..4096), d_model 512, H=8, d=64, 4 layers, bf16: every row."""
    x = synth.workload_heavy_tail_stack()
    announce(f"heavy-tail 4-layer stack, T_tot={int(x.offsets[-1])}")
    check_layer(x, "4-layer stack")
