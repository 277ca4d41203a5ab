"""Seeded synthetic inputs for the HSTU jagged pointwise-attention path.

This module only draws random inputs: sequence lengths, jagged offsets,
timestamps, activations, bias tables and weights. It contains none of the
method's arithmetic, so both the CPU oracle and the GPU path can take their
inputs from here.

Recipe (one ``numpy.random.default_rng(seed)`` per workload). Draws happen in
this order: lengths, timestamps, activations, tables, weights.

* Timestamps are int64 seconds. Each sequence starts at 1_700_000_000 and
  advances by ``max(1, rint(Exp(mean 3600)))`` per action, so it is strictly
  increasing. The HSTU pages (Yonas Stephen's course, "Problem 2") say the
  bias needs elapsed time as well as position.
* "N(0, s)" means standard deviation s.
* bf16 inputs are the round-to-nearest-even cast of the fp32 draw. Both sides
  receive exactly these values: the GPU gets the bf16 bits, the oracle gets the
  same numbers widened to fp64.

The workload shapes follow the five HSTU configurations: a tiny fp32 attention
case, a short-history jagged layer batch, long-sequence attention at length
8192, a heavy-tailed 4-layer stack and M-FALCON candidate scoring.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

T0 = 1_700_000_000
GAP_MEAN_S = 3600.0


# --------------------------------------------------------------------------
# bf16 rounding (storage format, not method arithmetic)
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even). Returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 array whose values are exactly representable in bf16 (RNE)."""
    return bf16_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------
# length samplers
# --------------------------------------------------------------------------
def lengths_uniform(rng, b, lo, hi):
    return rng.integers(lo, hi + 1, size=b).astype(np.int64)


def lengths_geometric_clipped(rng, b, mean, lo, hi):
    return np.clip(rng.geometric(1.0 / mean, size=b), lo, hi).astype(np.int64)


def lengths_power_law(rng, b, s, lo, hi):
    """Bounded power law: P(l) proportional to l**-s on the integers lo..hi."""
    support = np.arange(lo, hi + 1, dtype=np.float64)
    p = support ** (-s)
    p /= p.sum()
    return rng.choice(np.arange(lo, hi + 1), size=b, p=p).astype(np.int64)


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def timestamps(rng, lengths, t0=T0, gap_mean=GAP_MEAN_S) -> np.ndarray:
    out = []
    for n in lengths:
        gaps = np.maximum(1, np.rint(rng.exponential(gap_mean, size=int(n)))).astype(np.int64)
        gaps[:1] = 0  # first action sits at t0
        out.append(t0 + np.cumsum(gaps))
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def normal(rng, shape, std=1.0, dtype="bf16"):
    x = (rng.standard_normal(size=shape) * std).astype(np.float32)
    return round_bf16(x) if dtype == "bf16" else x


# --------------------------------------------------------------------------
# input bundles
# --------------------------------------------------------------------------
@dataclass
class AttnInputs:
    offsets: np.ndarray          # int64 [B+1]
    ts: Optional[np.ndarray]     # int64 [T_tot]
    q: np.ndarray                # f32 [T_tot, H, d_qk] (bf16-exact if dtype == "bf16")
    k: np.ndarray
    v: np.ndarray                # f32 [T_tot, H, d_v]
    u: Optional[np.ndarray]      # f32 [T_tot, H, d_v]
    rab_pos: Optional[np.ndarray]   # f32 [H, P]
    rab_time: Optional[np.ndarray]  # f32 [H, T]
    gamma: Optional[np.ndarray]  # f32 [H*d_v]
    beta: Optional[np.ndarray]
    num_heads: int
    d_qk: int
    d_v: int
    num_pos_buckets: int
    num_time_buckets: int
    max_seq_len: int             # N (the 1/N scale)
    dtype: str                   # "f32" or "bf16"
    eps: float = 1e-5

    @property
    def lengths(self):
        return np.diff(self.offsets)


@dataclass
class LayerWeights:
    w1: np.ndarray               # f32 [2H(d_v+d_qk), d_model], row blocks U|V|Q|K
    b1: Optional[np.ndarray]     # f32 [2H(d_v+d_qk)]
    rab_pos: Optional[np.ndarray]
    rab_time: Optional[np.ndarray]
    gamma: Optional[np.ndarray]  # f32 [H*d_v]
    beta: Optional[np.ndarray]
    w2: np.ndarray               # f32 [d_model, H*d_v]
    b2: Optional[np.ndarray]     # f32 [d_model]


@dataclass
class LayerInputs:
    offsets: np.ndarray
    ts: Optional[np.ndarray]
    x: np.ndarray                # f32 [T_tot, d_model]
    layers: list                 # list[LayerWeights]
    num_heads: int
    d_qk: int
    d_v: int
    d_model: int
    num_pos_buckets: int
    num_time_buckets: int
    max_seq_len: int
    dtype: str
    eps: float = 1e-5
    residual: int = 0

    @property
    def lengths(self):
        return np.diff(self.offsets)


@dataclass
class MfalconInputs:
    hist_offsets: np.ndarray
    hist_ts: Optional[np.ndarray]
    hist_x: np.ndarray
    cand_offsets: np.ndarray
    cand_ts: Optional[np.ndarray]
    cand_x: np.ndarray
    layers: list
    w_head: Optional[np.ndarray]
    num_heads: int
    d_qk: int
    d_v: int
    d_model: int
    num_pos_buckets: int
    num_time_buckets: int
    max_seq_len: int
    microbatch: int
    dtype: str
    eps: float = 1e-5
    residual: int = 0


def make_attn(seed, lengths_fn, H, d_qk, d_v, P, T, dtype, with_u=False, with_ln_affine=False,
              qkv_std=1.0, rab_std=0.02, with_time=True, with_pos=True, max_seq_len=None):
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths_fn(rng), dtype=np.int64)
    off = offsets_from_lengths(lengths)
    ts = timestamps(rng, lengths)
    n = int(off[-1])
    q = normal(rng, (n, H, d_qk), qkv_std, dtype)
    k = normal(rng, (n, H, d_qk), qkv_std, dtype)
    v = normal(rng, (n, H, d_v), qkv_std, dtype)
    u = normal(rng, (n, H, d_v), 1.0, dtype) if with_u else None
    rp = (rng.standard_normal((H, P)) * rab_std).astype(np.float32)
    rt = (rng.standard_normal((H, T)) * rab_std).astype(np.float32)
    g = b = None
    if with_ln_affine:
        g = (1.0 + 0.1 * rng.standard_normal(H * d_v)).astype(np.float32)
        b = (0.1 * rng.standard_normal(H * d_v)).astype(np.float32)
    N = int(max_seq_len) if max_seq_len is not None else int(max(1, lengths.max(initial=0)))
    return AttnInputs(off, ts if with_time else None, q, k, v, u, rp if with_pos else None,
                      rt if with_time else None, g, b, H, d_qk, d_v, P, T, N, dtype)


def make_layer_weights(rng, H, d_qk, d_v, d_model, P, T, dtype, w_std=0.02, random_bias=False,
                       with_ln_affine=False, rab_std=0.02):
    n1 = 2 * H * (d_v + d_qk)
    w1 = normal(rng, (n1, d_model), w_std, dtype)
    rp = (rng.standard_normal((H, P)) * rab_std).astype(np.float32)
    rt = (rng.standard_normal((H, T)) * rab_std).astype(np.float32)
    w2 = normal(rng, (d_model, H * d_v), w_std, dtype)
    if random_bias:
        b1 = (0.1 * rng.standard_normal(n1)).astype(np.float32)
        b2 = (0.1 * rng.standard_normal(d_model)).astype(np.float32)
    else:
        b1 = np.zeros(n1, np.float32)
        b2 = np.zeros(d_model, np.float32)
    g = be = None
    if with_ln_affine:
        g = (1.0 + 0.1 * rng.standard_normal(H * d_v)).astype(np.float32)
        be = (0.1 * rng.standard_normal(H * d_v)).astype(np.float32)
    return LayerWeights(w1, b1, rp, rt, g, be, w2, b2)


def make_layer(seed, lengths_fn, H, d_qk, d_v, d_model, P, T, dtype, num_layers=1, x_std=1.0,
               w_std=0.02, random_bias=False, with_ln_affine=False, residual=0, max_seq_len=None):
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths_fn(rng), dtype=np.int64)
    off = offsets_from_lengths(lengths)
    ts = timestamps(rng, lengths)
    x = normal(rng, (int(off[-1]), d_model), x_std, dtype)
    layers = [make_layer_weights(rng, H, d_qk, d_v, d_model, P, T, dtype, w_std, random_bias,
                                 with_ln_affine) for _ in range(num_layers)]
    N = int(max_seq_len) if max_seq_len is not None else int(max(1, lengths.max(initial=0)))
    return LayerInputs(off, ts, x, layers, H, d_qk, d_v, d_model, P, T, N, dtype, residual=residual)


def make_mfalcon(seed, hist_lengths, cand_counts, H, d_qk, d_v, d_model, P, T, dtype, num_layers=1,
                 microbatch=1024, shared_request_time=True, w_std=0.02, random_bias=False,
                 with_ln_affine=False, with_head=True, residual=0, max_seq_len=None):
    """Candidates of user b sit at position n_h(b) after its history. With
    ``shared_request_time`` every candidate of a user carries the request time
    t_req = (last history timestamp) + one more exponential gap; otherwise each
    candidate gets its own t_req + extra gap."""
    rng = np.random.default_rng(seed)
    hist_lengths = np.asarray(hist_lengths, dtype=np.int64)
    cand_counts = np.asarray(cand_counts, dtype=np.int64)
    hoff = offsets_from_lengths(hist_lengths)
    coff = offsets_from_lengths(cand_counts)
    hts = timestamps(rng, hist_lengths)
    cts = []
    for b in range(len(hist_lengths)):
        last = hts[hoff[b + 1] - 1] if hist_lengths[b] > 0 else T0
        t_req = last + max(1, int(np.rint(rng.exponential(GAP_MEAN_S))))
        c = int(cand_counts[b])
        if shared_request_time:
            cts.append(np.full(c, t_req, dtype=np.int64))
        else:
            cts.append(t_req + np.rint(rng.exponential(60.0, size=c)).astype(np.int64))
    cts = np.concatenate(cts) if cts else np.zeros(0, np.int64)
    hx = normal(rng, (int(hoff[-1]), d_model), 1.0, dtype)
    cx = normal(rng, (int(coff[-1]), d_model), 1.0, dtype)
    layers = [make_layer_weights(rng, H, d_qk, d_v, d_model, P, T, dtype, w_std, random_bias,
                                 with_ln_affine) for _ in range(num_layers)]
    w_head = (rng.standard_normal(d_model) * 0.02).astype(np.float32) if with_head else None
    N = int(max_seq_len) if max_seq_len is not None else int(hist_lengths.max(initial=0)) + 1
    return MfalconInputs(hoff, hts, hx, coff, cts, cx, layers, w_head, H, d_qk, d_v, d_model, P, T,
                         N, microbatch, dtype, residual=residual)


# --------------------------------------------------------------------------
# the five HSTU workloads
# --------------------------------------------------------------------------
def workload_tiny_attention(seed=0, with_u=False):
    """B=4, lengths uniform in [8,64], 2 heads, d=32, fp32, 64 pos / 32 time buckets."""
    return make_attn(seed, lambda r: lengths_uniform(r, 4, 8, 64), 2, 32, 32, 64, 32, "f32",
                     with_u=with_u)


def workload_short_history_layer(seed=1, num_layers=1):
    """B=256, lengths geometric(mean 120) clipped to [20,200], 2 heads, d=64, d_model 128, bf16."""
    return make_layer(seed, lambda r: lengths_geometric_clipped(r, 256, 120, 20, 200), 2, 64, 64,
                      128, 128, 64, "bf16", num_layers=num_layers)


def workload_long_attention(seed=2, batch=8):
    """B=8, lengths uniform in [4096,8192] with the first one exactly 8192, 4 heads, d=128, bf16."""
    def lens(r):
        x = lengths_uniform(r, batch, 4096, 8192)
        x[0] = 8192
        return x
    return make_attn(seed, lens, 4, 128, 128, 128, 64, "bf16")


def workload_heavy_tail_stack(seed=3, num_layers=4):
    """B=32, bounded power-law lengths (s=1.2) on [64,4096], d_model 512, 8 heads, d=64, 4 layers."""
    return make_layer(seed, lambda r: lengths_power_law(r, 32, 1.2, 64, 4096), 8, 64, 64, 512,
                      128, 64, "bf16", num_layers=num_layers)


def workload_mfalcon(seed=4, num_layers=1, num_candidates=16384, history=4096, microbatch=1024):
    """One user, history 4096, 16,384 candidates in microbatches of 1024, 8 heads, d=64, d_model 512."""
    return make_mfalcon(seed, [history], [num_candidates], 8, 64, 64, 512, 128, 64, "bf16",
                        num_layers=num_layers, microbatch=microbatch)


# --------------------------------------------------------------------------
# Stochastic Length sampling: the random draws it consumes
# --------------------------------------------------------------------------
@dataclass
class SlInputs:
    offsets: np.ndarray       # int64 [B+1]
    ts: np.ndarray            # int64 [T_tot]
    x: np.ndarray             # [T_tot, d_model] (fp32 values; bf16-exact when dtype is bf16)
    u_keep: np.ndarray        # float32 [B], uniform in [0, 1): the keep-whole draw per sequence
    keys: np.ndarray          # uint32 [T_tot], uniform: the per-action selection keys
    max_seq_len: int
    alpha: float
    dtype: str


def sl_draws(rng, batch, total):
    """(u_keep float32 [batch] uniform in [0,1), keys uint32 [total] uniform)."""
    u = rng.random(batch).astype(np.float32)
    u = np.minimum(u, np.float32(np.nextafter(np.float32(1), np.float32(0))))
    keys = rng.integers(0, 2**32, size=total, dtype=np.uint64).astype(np.uint32)
    return u, keys


def make_sl(seed, lengths_fn, d_model, N, alpha, dtype="bf16"):
    rng = np.random.default_rng(seed)
    lengths = lengths_fn(rng)
    off = offsets_from_lengths(lengths)
    ts = timestamps(rng, lengths)
    x = normal(rng, (int(off[-1]), d_model), 1.0, dtype)
    u, keys = sl_draws(rng, len(lengths), int(off[-1]))
    return SlInputs(off, ts, x, u, keys, N, alpha, dtype)


def workload_sl_heavy_tail(seed=5, batch=32):
    """The heavy-tailed training batch (bounded power-law lengths, s=1.2, on [64,4096],
    d_model 512, bf16) sampled with N = 4096, alpha = 1.6 (target length 776)."""
    return make_sl(seed, lambda r: lengths_power_law(r, batch, 1.2, 64, 4096), 512, 4096, 1.6)
