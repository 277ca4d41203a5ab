"""Move seeded synthetic inputs (hstu_jagged_pointwise_amd.synth) to device tensors.

This is plumbing only: torch allocates device memory and copies the values.
bf16 inputs are already bf16-exact, so the cast is lossless.
"""
from __future__ import annotations

import numpy as np
import torch


def _dev(a, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def act_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def layer_weights(layers, dtype_name):
    from . import ops
    dt = act_dtype(dtype_name)
    return [ops.LayerWeights(w1=_dev(w.w1, dt), w2=_dev(w.w2, dt), b1=_dev(w.b1), b2=_dev(w.b2),
                             rab_pos=_dev(w.rab_pos), rab_time=_dev(w.rab_time),
                             ln_gamma=_dev(w.gamma), ln_beta=_dev(w.beta)) for w in layers]


def attn_to_device(x):
    dt = act_dtype(x.dtype)
    return dict(offsets=_dev(x.offsets), ts=_dev(x.ts), q=_dev(x.q, dt), k=_dev(x.k, dt),
                v=_dev(x.v, dt), u=_dev(x.u, dt), rab_pos=_dev(x.rab_pos), rab_time=_dev(x.rab_time),
                gamma=_dev(x.gamma), beta=_dev(x.beta))


def layer_to_device(x):
    return dict(offsets=_dev(x.offsets), ts=_dev(x.ts), x=_dev(x.x, act_dtype(x.dtype)),
                layers=layer_weights(x.layers, x.dtype))


def mfalcon_to_device(x):
    dt = act_dtype(x.dtype)
    return dict(hist_offsets=_dev(x.hist_offsets), hist_ts=_dev(x.hist_ts),
                hist_x=_dev(x.hist_x, dt), cand_offsets=_dev(x.cand_offsets),
                cand_ts=_dev(x.cand_ts), cand_x=_dev(x.cand_x, dt),
                layers=layer_weights(x.layers, x.dtype), w_head=_dev(x.w_head))
