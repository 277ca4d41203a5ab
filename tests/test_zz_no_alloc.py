"""GPU check of hstu_attn_fwd_noalloc, the allocation-free variant of hstu_attn_fwd (its
scratch is a device array inside the library). Through the C ABI, it must return what
hstu_attn_fwd returns, bit for bit, on two calls in a row, the second one smaller, so
that the second call reads nothing the first left behind."""
import numpy as np
import pytest
import torch

from hstu_jagged_pointwise_amd import synth
from gpu_util import act_dtype, announce, dev

pytestmark = pytest.mark.gpu


def _pair(x, with_u):
    from hstu_jagged_pointwise_amd import ops
    dt = act_dtype(x.dtype)
    args = (dev(x.offsets), dev(x.ts), dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.rab_pos),
            dev(x.rab_time))
    kw = dict(max_seq_len=x.max_seq_len, u=dev(x.u, dt) if with_u else None,
              ln_gamma=dev(x.gamma) if with_u else None, ln_beta=dev(x.beta) if with_u else None,
              ln_eps=x.eps, seq_offsets_host=x.offsets)
    ref = ops.hstu_attn_fwd(*args, **kw)
    got = ops.hstu_attn_fwd_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dt,d,with_u", [("bf16", 128, False), ("bf16", 64, True),
                                         ("bf16", 32, True), ("f32", 64, True)])
def test_noalloc_equals_workspace_call(dt, d, with_u):
    big = synth.make_attn(41 + d, lambda r: np.array([700, 1, 129, 0, 300, 2050]), 3, d, d, 128,
                          64, dt, with_u=True, with_ln_affine=True, rab_std=0.5)
    small = synth.make_attn(42 + d, lambda r: np.array([5, 140]), 3, d, d, 128, 64, dt,
                            with_u=True, with_ln_affine=True, rab_std=0.5)
    for name, x in (("first (larger)", big), ("second (smaller)", small)):
        announce(f"noalloc attention {dt} d={d} gated={with_u}: {name} call, "
                 f"T_tot={int(x.offsets[-1])}")
        ref, got = _pair(x, with_u)
        assert bool(torch.isfinite(ref.float()).all())
        assert torch.equal(got, ref), f"{name}: allocation-free output differs"
