"""Helpers for the GPU parity tests: move the seeded inputs to the device, call the
C ABI through the ctypes binding, and compare with the oracle per output row."""
import sys

import numpy as np
import torch


def announce(msg: str):
    """Name the case before a GPU step (flushed), so a failing run says which case it was."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def act_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def row_errors(g, o):
    """Per output row: max|g - o| / max|o|. The rows are the first axis; the rest is flattened."""
    g = np.asarray(g, np.float64).reshape(len(g), -1)
    o = np.asarray(o, np.float64).reshape(len(o), -1)
    num = np.abs(g - o).max(axis=1) if g.size else np.zeros(0)
    den = np.abs(o).max(axis=1) if o.size else np.zeros(0)
    return num, den


def record(what, msg):
    """One line per checked output for the run's log: what was compared and how closely."""
    print(f"[parity] {what}: {msg}", flush=True)


def assert_rows_close(g, o, tol, what=""):
    """Relative error per row (infinity norm) <= tol on every row. Where the oracle row is
    exactly zero, the GPU row must be exactly zero too."""
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    num, den = row_errors(g, o)
    zero = den == 0
    assert np.all(num[zero] == 0), f"{what}: rows that must be zero are not"
    rel = num[~zero] / den[~zero]
    worst = float(rel.max()) if rel.size else 0.0
    p99 = float(np.quantile(rel, 0.99)) if rel.size else 0.0
    record(what, f"{len(num)} rows, flat tol {tol:.0e}: worst {worst:.3e}, p99 {p99:.3e}")
    assert worst <= tol, f"{what}: worst row error {worst:.3e} > {tol:.1e} (p99 {p99:.3e})"
    return worst


RANGE_FLOOR = 2.0 ** -100  # below this, a layer's fp32 products fall under fp32's normal range


def assert_rows_close_in_range(g, o, tol, what=""):
    """assert_rows_close on every row whose oracle values lie inside fp32's working range.
    A row whose largest oracle value is below RANGE_FLOOR (~7.9e-31) comes out of sums of
    products below 2^-126, which fp32 arithmetic flushes to zero or resolves only
    coarsely: such rows are counted and reported, and must be finite and no larger than
    RANGE_FLOOR on the GPU as well."""
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    g = np.asarray(g, np.float64).reshape(len(g), -1)
    o = np.asarray(o, np.float64).reshape(len(o), -1)
    tiny = np.abs(o).max(axis=1) < RANGE_FLOOR
    if tiny.any():
        record(what, f"{int(tiny.sum())} of {len(o)} rows below fp32 working range "
                     f"(oracle row max < 2^-100); GPU max there {np.abs(g[tiny]).max():.3e}")
        assert np.abs(g[tiny]).max() <= RANGE_FLOOR, f"{what}: out-of-range rows are not tiny"
    if (~tiny).any():
        return assert_rows_close(g[~tiny], o[~tiny], tol, what)
    return 0.0


def attn_on_gpu(x, with_u=False, out_dtype=None, rab_pos="x", rab_time="x", ts="x", q=None):
    dt = act_dtype(x.dtype)
    from hstu_jagged_pointwise_amd import ops
    rp = x.rab_pos if isinstance(rab_pos, str) else rab_pos
    rt = x.rab_time if isinstance(rab_time, str) else rab_time
    tsv = x.ts if isinstance(ts, str) else ts
    qv = x.q if q is None else q
    out = ops.hstu_attn_fwd(dev(x.offsets), dev(tsv), dev(qv, dt), dev(x.k, dt), dev(x.v, dt),
                            dev(rp), dev(rt), max_seq_len=x.max_seq_len,
                            num_pos_buckets=x.num_pos_buckets, num_time_buckets=x.num_time_buckets,
                            u=dev(x.u, dt) if with_u else None,
                            ln_gamma=dev(x.gamma) if with_u else None,
                            ln_beta=dev(x.beta) if with_u else None, ln_eps=x.eps,
                            seq_offsets_host=x.offsets)
    torch.cuda.synchronize()
    return out


def layer_weights_on_gpu(layers, dtype_name):
    from hstu_jagged_pointwise_amd import ops
    dt = act_dtype(dtype_name)
    return [ops.LayerWeights(w1=dev(w.w1, dt), w2=dev(w.w2, dt), b1=dev(w.b1), b2=dev(w.b2),
                             rab_pos=dev(w.rab_pos), rab_time=dev(w.rab_time),
                             ln_gamma=dev(w.gamma), ln_beta=dev(w.beta)) for w in layers]


FP32_TINY = 2.0 ** -126  # smallest normal fp32 value


def assert_sums_close(g, o, o_storage, terms, tol, k=4.0, what=""):
    """Gradients that are sums over many tokens or pairs (weight, bias and bias-table
    gradients). Per entry, |g - o| <= max(tol |o_row|_inf, k |o_s - o|_row_inf,
    tol * terms, FP32_TINY): besides the row bounds of assert_rows_close_storage, the error
    may reach tol times the sum of the magnitudes of the terms added up (terms, from the
    oracle), the standard error bound of a sum whose terms each carry a relative error.
    That matters where the terms cancel: a table entry of 1e-25 made of 1e7 terms of 1e-28
    has no meaningful relative error at the size of the result. Below the fp32 normal
    range (the device accumulates in fp32 and flushes denormals) differences are not
    resolved at all, hence the absolute floor."""
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    g = np.asarray(g, np.float64).reshape(len(g), -1)
    o = np.asarray(o, np.float64).reshape(len(o), -1)
    s = np.asarray(o_storage, np.float64).reshape(len(o), -1)
    t = np.asarray(terms, np.float64).reshape(len(o), -1)
    err = np.abs(g - o)
    row = np.maximum(tol * np.abs(o).max(axis=1), k * np.abs(s - o).max(axis=1))[:, None]
    bound = np.maximum(np.maximum(row, tol * t), FP32_TINY)
    bad = err > bound
    flat_ok = err <= tol * np.abs(o).max(axis=1)[:, None]
    record(what, f"{err.size} entries: {int((~flat_ok).sum())} above the flat row bound, decided "
                 f"by the storage, sum-of-terms or fp32-range terms")
    assert not bad.any(), f"{what}: {int(bad.sum())} entries outside the bound; worst excess " \
                          f"{float((err / np.maximum(bound, 1e-300)).max()):.3f}"
    return float((err / np.maximum(np.maximum(np.abs(o).max(axis=1)[:, None], t), 1e-300)).max())


def assert_rows_close_storage(g, o, o_storage, tol, k=4.0, what=""):
    """bf16 multi-step paths: per row, |g - o|_inf <= max(tol |o|_inf, k |o_s - o|_inf).
    Here o is the fp64 oracle and o_s is the oracle with bf16 storage of the tensors
    that the library stores between steps. In well-conditioned rows the first term
    applies. Where storage rounding alone moves a row by more than tol, the bound
    follows the size of that move. The median row must also meet tol."""
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    g = np.asarray(g, np.float64).reshape(len(g), -1)
    o = np.asarray(o, np.float64).reshape(len(o), -1)
    s = np.asarray(o_storage, np.float64).reshape(len(o), -1)
    num = np.abs(g - o).max(axis=1)
    den = np.abs(o).max(axis=1)
    sens = np.abs(s - o).max(axis=1)
    bound = np.maximum(tol * den, k * sens)
    bad = num > bound
    live = den > 0
    flat = num[live] / den[live]
    over = flat > tol  # rows that the flat tolerance alone would fail: decided by the storage term
    msg = f"{int(live.sum())} rows: flat worst {float(flat.max()) if flat.size else 0:.3e}, " \
          f"{int(over.sum())} rows above flat {tol:.0e}"
    if over.any():
        idx = np.flatnonzero(live)[over]
        msg += f" (rows {idx[:8].tolist()}{'...' if len(idx) > 8 else ''}), each within " \
               f"{k:g}x its storage-only deviation (which is >= " \
               f"{float((sens[live][over] / den[live][over]).min()):.3e} on those rows)"
    record(what, msg)
    assert not bad.any(), f"{what}: {int(bad.sum())} rows outside the bound; worst excess " \
                          f"{float((num / np.maximum(bound, 1e-300)).max()):.3f}"
    med = float(np.median(num[live] / den[live])) if live.any() else 0.0
    assert med <= tol, f"{what}: median row error {med:.3e} > {tol}"
    return float((num[live] / den[live]).max()) if live.any() else 0.0
