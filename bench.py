"""Benchmark of the HSTU jagged pointwise-attention hot path on one MI355X.

A step is one hstu_attn_fwd call on the long-sequence workload: B=8 jagged
sequences, lengths uniform in [4096, 8192] with one of exactly 8192, 4 heads,
d_qk = d_v = 128, bf16 in with fp32 accumulation, 128 position and 64 time
buckets, causal. That call plans the tiles on the device and runs the fused
attention kernel. `value` is attention TFLOP/s, counting useful pairs only:
H * sum_b n_b (n_b + 1) / 2 * 2 (d_qk + d_v) FLOPs per call. All inputs are
resident in HBM before the timed region. The same run also times:
  * M-FALCON: history 4096, 16,384 candidates in microbatches of 1024, H=8,
    d=64, d_model=512, 1 layer (candidates/s over the whole call, history pass
    included);
  * the short-history layer (B=256, lengths 20..200, d_model 128) and the
    heavy-tailed 4-layer stack (B=32, power-law lengths 64..4096, d_model 512);
  * the softmax ablation of the attention on the same length-8192 workload (same
    scores and bias), and the pointwise kernel's speedup over it;
  * the backward pass: attention gradients on the length-8192 workload and whole-layer
    gradients of both layer workloads;
  * Stochastic Length sampling of the heavy-tailed batch (N = 4096, alpha = 1.6);
  * the fp64 CPU oracle on a bounded sample of the attention workload.
One JSON line goes to stdout. Progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm-seconds S]
                    [--only attn,softmax,mfalcon,layers,backward,sl,cpu | copy]

Defaults: K = 200 timed calls of the attention (fewer for the slower legs), W = 20 warm-up
calls, and S = 2 s of untimed near-continuous load before the first timed call, so that the
clock has settled (the first ~100 calls of an idle device run up to 15% slower).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HSTU attn TFLOP/s + % bf16 MFMA peak at len 8192; M-FALCON candidates/sec"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_long_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the attention kernel sources; counter data is valid only for this hash."""
    h = hashlib.sha256()
    for f in ("attn_mfma.hip", "attn_common.h", "common.h", "plan.hip"):
        with open(os.path.join(ROOT, "hstu_jagged_pointwise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# Untimed near-continuous load before each later leg's timed calls (seconds; set from
# --warm-seconds): a leg's set-up idles the device, whose clock then ramps down again.
LEG_WARM_S = 0.0


def time_calls(fn, stream, steps, warmup, warm_s=None):
    """Per-call durations (ms) from HIP events recorded on the library's stream.

    After the `warmup` calls, further untimed calls run until `warm_s` seconds have
    passed: a device that was idle takes a second or so of load to reach its steady clock,
    and calls timed before that measure the ramp rather than the kernel. Anything that
    idles the device (here: the garbage collection and the event set-up) happens before the
    warm-up, so only the synchronize separates the last warm-up call from the first timed
    one.

    Python's cyclic garbage collector is run before the warm-up and paused until the timed
    calls are done, as timeit does: a full collection holds the host for tens of
    milliseconds, and one landing between a call's start event and its launches would be
    counted as GPU time of that call."""
    import gc
    import torch
    if warm_s is None:
        warm_s = LEG_WARM_S
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    gc.collect()
    gc_was_on = gc.isenabled()
    gc.disable()
    try:
        t_warm = time.perf_counter()
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        while time.perf_counter() - t_warm < warm_s:  # near-continuous load
            for _ in range(100):
                fn()
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        if gc_was_on:
            gc.enable()
    return np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]), wall


MALL_FLUSH_BYTES = 512 << 20  # twice the 256 MB last-level cache (MALL)


def time_calls_cold(fn, stream, steps):
    """Per-call durations (ms) with the last-level cache flushed before each call: a 512 MB
    buffer is written on the same stream between calls, outside the timed events, so that
    every call reads its inputs from HBM."""
    import torch
    flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    fn()
    torch.cuda.synchronize()
    for i in range(steps):
        flush.fill_(i & 0xff)
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])


def gate_f2_fused(x):
    """True when the library runs the LN gate and f2 as one kernel for this layer shape
    (bf16, gated width H*d_v of 64 or 128, model width 64, 128 or 256)."""
    return (x.dtype == "bf16" and x.num_heads * x.d_v in (64, 128)
            and x.d_model in (64, 128, 256))


def layer_bytes(x, split_qk=True):
    """Algorithmic HBM bytes of one layer as its steps run here, each step reading its
    inputs once and writing its outputs once (bf16 activations and weights, fp32 attention
    rows for the gate, int64 timestamps): f1 reads X and W1 and writes U|V|Q|K (plus the
    bf16 remainder of Q and K that the split-precision scores read); the attention reads
    Q, K, V (and the remainders) and the timestamps and writes fp32 O; the gate reads O
    and U and writes G; f2 reads G and W2 and writes Y. Where the gate and f2 are one
    kernel ("ln_gate_f2"), it reads O, U and W2 and writes Y: G never reaches HBM."""
    T, dm, H, dqk, dv = int(x.offsets[-1]), x.d_model, x.num_heads, x.d_qk, x.d_v
    f1c = 2 * H * (dqk + dv)
    lo = 2 * H * dqk if split_qk else 0
    f1 = T * dm * 2 + f1c * dm * 2 + T * (f1c + lo) * 2
    attn = T * (2 * H * dqk + lo + H * dv) * 2 + T * 8 + T * H * dv * 4
    if gate_f2_fused(x):
        g2 = T * H * dv * 4 + T * H * dv * 2 + dm * H * dv * 2 + T * dm * 2
        return {"f1": f1, "attention": attn, "ln_gate_f2": g2, "total": f1 + attn + g2}
    gate = T * H * dv * 4 + T * H * dv * 2 * 2
    f2 = T * H * dv * 2 + dm * H * dv * 2 + T * dm * 2
    return {"f1": f1, "attention": attn, "ln_gate": gate, "f2": f2,
            "total": f1 + attn + gate + f2}


def leg_attention(steps, warmup, warm_s=0.0):
    import torch
    from hstu_jagged_pointwise_amd import ops, synth
    from hstu_jagged_pointwise_amd.device import attn_to_device
    x = synth.workload_long_attention()
    d = attn_to_device(x)
    stream = torch.cuda.Stream()
    desc = ops.attn_desc(len(x.offsets) - 1, x.num_heads, x.d_qk, x.d_v, x.max_seq_len,
                         x.num_pos_buckets, x.num_time_buckets, ops.HSTU_BF16)
    ws_bytes = ops.hstu_attn_workspace_size(desc, x.offsets)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["v"])

    def call():
        ops.hstu_attn_fwd(d["offsets"], d["ts"], d["q"], d["k"], d["v"], d["rab_pos"],
                          d["rab_time"], max_seq_len=x.max_seq_len, out=out, workspace=ws,
                          seq_offsets_host=x.offsets, stream=stream)

    with torch.cuda.stream(stream):
        ms, wall = time_calls(call, stream, steps, warmup, warm_s)
    pairs = int(np.sum(x.lengths * (x.lengths + 1) // 2))
    flops = pairs * x.num_heads * 2 * (x.d_qk + x.d_v)
    mean = float(ms.mean())
    return dict(x=x, ms=ms, wall=wall, flops=flops, pairs=pairs, tflops=flops / (mean * 1e-3) / 1e12,
                out=out)


# Vector-ALU side of the attention's roofline. Every score goes through SiLU on the vector
# ALU. The instruction counts per score come from the committed hardware-counter record of
# the attention kernel (profiles/attn_long_counters.json: SQ_INSTS_VALU, SQ_INSTS_MFMA and
# SQ_INSTS_VALU_TRANS_F32 per dispatch, wave instructions of 64 lanes) when it was taken on
# the current kernel source; otherwise from the kernel's fast path as written (2
# transcendentals and 3.5 ordinary ops per score: the fma that scales the score and adds its
# block's constant bias, SiLU's add and multiply, half a pack). Rates
# from the chip's unit counts: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz ordinary lane-ops/s
# (packed fp32 disabled); transcendentals at half that (measured on the device: a wave64
# exp2 or reciprocal takes twice the cycles of an fp32 FMA).
VALU_PLAIN_PER_S = 256 * 4 * 16 * 2.4e9
VALU_TRANS_PER_S = VALU_PLAIN_PER_S / 2
FAST_PATH_OPS = {"transcendental": 2.0, "plain": 3.5}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_long_counters.json")


def counter_record():
    """The committed counter record, if it was taken on the current attention source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    rec = json.load(open(COUNTERS_FILE))
    return rec if rec.get("source_hash") == source_hash() else None


def valu_ceiling(attn):
    scores = attn["pairs"] * attn["x"].num_heads
    rec = counter_record()
    if rec:
        c = rec["counters_per_dispatch"]
        trans = c["SQ_INSTS_VALU_TRANS_F32"] * 64 / scores
        plain = (c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"] - c["SQ_INSTS_VALU_TRANS_F32"]) * 64 / scores
        ops = {"transcendental": round(trans, 3), "plain": round(plain, 3),
               "source": "hardware counters of this kernel source (profiles/attn_long_counters.json)"}
        cyc = c["SQ_CYCLES"] / rec["shader_engines"]  # per SIMD (the counter sums the engines)
        busy = {"mfma_busy": round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / rec["simds"] / cyc, 4),
                "valu_busy": round(4 * c["SQ_ACTIVE_INST_VALU"] / rec["simds"] / cyc, 4),
                "mfma_and_valu": round(c["SQ_VALU_MFMA_COEXEC_CYCLES"] / rec["simds"] / cyc, 4),
                "note": "fractions of each SIMD's cycles over the dispatch, from the counters"}
    else:
        ops = dict(FAST_PATH_OPS, source="the kernel's fast path as written (no counter record "
                                         "for this kernel source)")
        busy = None
    t_valu = scores * (ops["plain"] / VALU_PLAIN_PER_S + ops["transcendental"] / VALU_TRANS_PER_S)
    valu_tf = attn["flops"] / t_valu / 1e12
    both_tf = 1.0 / (1.0 / PEAK_BF16_TFLOPS + 1.0 / valu_tf)
    out = {"scores": int(scores), "ops_per_score": ops,
           "ceiling": round(valu_tf, 1), "mfma_plus_valu_ceiling": round(both_tf, 1),
           "unit": "TFLOP/s", "frac_of_mfma_plus_valu": round(attn["tflops"] / both_tf, 4),
           "note": "ceiling: the vector work alone at the vector-ALU rate; mfma_plus_valu: MFMA "
                   "at peak and the vector work at that rate, not overlapped"}
    if busy:
        out["busy"] = busy
    return out


def mfalcon_flops(x):
    """Algorithmic FLOPs of one mfalcon_score call: per layer, the candidates' f1 and f2 and
    their attention to n_h history keys plus themselves; the history's f1 (its keys and
    values) and, below the last layer, the history's whole layer."""
    C = int(x.cand_offsets[-1])
    n_h = int(x.hist_offsets[-1])
    H, dqk, dv, dm, L = x.num_heads, x.d_qk, x.d_v, x.d_model, len(x.layers)
    f1 = 2 * dm * 2 * H * (dqk + dv)
    f2 = 2 * H * dv * dm
    cand = C * (L * (f1 + f2) + L * (n_h + 1) * H * 2 * (dqk + dv))
    lens = np.diff(x.hist_offsets)
    hist_pairs = int(np.sum(lens * (lens + 1) // 2))
    hist = n_h * f1 * L + (L - 1) * (n_h * f2 + hist_pairs * H * 2 * (dqk + dv))
    return cand + hist


def leg_mfalcon(steps, warmup, num_layers=1):
    import torch
    from hstu_jagged_pointwise_amd import ops, synth
    from hstu_jagged_pointwise_amd.device import mfalcon_to_device
    x = synth.workload_mfalcon(num_layers=num_layers)
    d = mfalcon_to_device(x)
    stream = torch.cuda.Stream()
    ld = ops.layer_desc(d["layers"], 1, x.num_heads, x.d_qk, x.d_v, x.d_model, x.max_seq_len,
                        ops.HSTU_BF16)
    desc = ops.mfalcon_desc(ld, x.microbatch)
    ws = torch.empty(ops.mfalcon_workspace_size(desc, x.hist_offsets, x.cand_offsets),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["cand_x"])
    logit = torch.empty(out.shape[0], dtype=torch.float32, device="cuda")

    def call():
        ops.mfalcon_score(d["hist_offsets"], d["hist_ts"], d["hist_x"], d["cand_offsets"],
                          d["cand_ts"], d["cand_x"], d["layers"], num_heads=x.num_heads,
                          d_qk=x.d_qk, d_v=x.d_v, max_seq_len=x.max_seq_len,
                          microbatch=x.microbatch, w_head=d["w_head"], out=out, logit=logit,
                          workspace=ws, hist_offsets_host=x.hist_offsets,
                          cand_offsets_host=x.cand_offsets, stream=stream)

    with torch.cuda.stream(stream):
        ms, wall = time_calls(call, stream, max(3, steps // 2), max(1, warmup // 2))
    # the candidate pass alone, against a history cache built once (mfalcon_history)
    kw = dict(num_heads=x.num_heads, d_qk=x.d_qk, d_v=x.d_v, max_seq_len=x.max_seq_len,
              microbatch=x.microbatch, hist_offsets_host=x.hist_offsets, stream=stream)
    with torch.cuda.stream(stream):
        cache = ops.mfalcon_history(d["hist_offsets"], d["hist_ts"], d["hist_x"], d["layers"], **kw)
        cws = torch.empty(max(1, ops.mfalcon_cached_workspace_size(desc, x.hist_offsets,
                                                                   x.cand_offsets)),
                          dtype=torch.uint8, device="cuda")

        def cand_call():
            ops.mfalcon_score_cached(cache, d["hist_offsets"], d["hist_ts"], d["cand_offsets"],
                                     d["cand_ts"], d["cand_x"], d["layers"], w_head=d["w_head"],
                                     out=out, logit=logit, workspace=cws,
                                     cand_offsets_host=x.cand_offsets, **kw)

        cms, _ = time_calls(cand_call, stream, max(3, steps // 2), max(1, warmup // 2))
    C = int(x.cand_offsets[-1])
    mean = float(ms.mean())
    cmean = float(cms.mean())
    n_h = int(x.hist_offsets[-1])
    flops = mfalcon_flops(x)
    tf = flops / (mean * 1e-3) / 1e12
    return dict(candidates=C, ms=round(mean, 4), candidates_per_s=C / (mean * 1e-3),
                tflops=round(tf, 2),
                roofline={"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                          "flops_per_call": int(flops),
                          "note": "the whole call (history pass included); FLOPs of the "
                                  "projections and of the attention over useful pairs only"},
                candidates_only=dict(ms=round(cmean, 4), candidates_per_s=C / (cmean * 1e-3),
                                     note="mfalcon_score_cached against a history cache built "
                                          "once by mfalcon_history"),
                microbatch=x.microbatch, in_flight=16, history=n_h, layers=num_layers)


def leg_layers(steps, warmup):
    import torch
    from hstu_jagged_pointwise_amd import ops, synth
    from hstu_jagged_pointwise_amd.device import layer_to_device
    res = {}
    for name, x in (("short_history_layer", synth.workload_short_history_layer()),
                    ("heavy_tail_4_layer_stack", synth.workload_heavy_tail_stack())):
        d = layer_to_device(x)
        stream = torch.cuda.Stream()
        desc = ops.layer_desc(d["layers"], len(x.offsets) - 1, x.num_heads, x.d_qk, x.d_v,
                              x.d_model, x.max_seq_len, ops.HSTU_BF16)
        ws = torch.empty(ops.hstu_layer_workspace_size(desc, x.offsets), dtype=torch.uint8,
                         device="cuda")
        y = torch.empty_like(d["x"])

        def call():
            ops.hstu_layer_fwd(d["offsets"], d["ts"], d["x"], d["layers"], num_heads=x.num_heads,
                               d_qk=x.d_qk, d_v=x.d_v, max_seq_len=x.max_seq_len, out=y,
                               workspace=ws, seq_offsets_host=x.offsets, stream=stream)

        with torch.cuda.stream(stream):
            ms, _ = time_calls(call, stream, steps, warmup)
            cold = time_calls_cold(call, stream, max(10, steps // 4))
        L = len(x.layers)
        T = int(x.offsets[-1])
        pairs = int(np.sum(x.lengths * (x.lengths + 1) // 2))
        f1 = T * 2 * x.d_model * 2 * x.num_heads * (x.d_qk + x.d_v)
        f2 = T * 2 * x.num_heads * x.d_v * x.d_model
        at = pairs * x.num_heads * 2 * (x.d_qk + x.d_v)
        mean = float(ms.mean())
        cmean = float(cold.mean())
        tf = L * (f1 + f2 + at) / (mean * 1e-3) / 1e12
        by = layer_bytes(x)
        gbs = L * by["total"] / (mean * 1e-3) / 1e9
        cgbs = L * by["total"] / (cmean * 1e-3) / 1e9
        res[name] = dict(tokens=T, layers=L, ms_per_call=round(mean, 4),
                         us_per_layer=round(mean * 1e3 / L, 2), tflops=round(tf, 2),
                         mfma_frac=round(tf / PEAK_BF16_TFLOPS, 4),
                         bytes_per_layer=by, hbm_gbs=round(gbs, 1),
                         hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
                         cold=dict(ms_per_call=round(cmean, 4),
                                   us_per_layer=round(cmean * 1e3 / L, 2),
                                   hbm_gbs=round(cgbs, 1), hbm_frac=round(cgbs / PEAK_HBM_GBS, 4),
                                   note="512 MB written between calls (last-level cache "
                                        "flushed), outside the timed events"))
    return res


def leg_softmax(steps, warmup):
    """The softmax ablation on the length-8192 workload, same scores and bias tables."""
    import torch
    from hstu_jagged_pointwise_amd import ops, synth
    from hstu_jagged_pointwise_amd.device import attn_to_device
    x = synth.workload_long_attention()
    d = attn_to_device(x)
    stream = torch.cuda.Stream()
    desc = ops.attn_desc(len(x.offsets) - 1, x.num_heads, x.d_qk, x.d_v, x.max_seq_len,
                         x.num_pos_buckets, x.num_time_buckets, ops.HSTU_BF16)
    import ctypes
    n = ctypes.c_size_t(0)
    ops._check(ops.lib.hstu_softmax_attn_workspace_size(ctypes.byref(desc), ops._i64p(x.offsets),
                                                        ctypes.byref(n)))
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["v"])

    def call():
        ops.hstu_softmax_attn_fwd(d["offsets"], d["ts"], d["q"], d["k"], d["v"], d["rab_pos"],
                                  d["rab_time"], max_seq_len=x.max_seq_len, out=out, workspace=ws,
                                  seq_offsets_host=x.offsets, stream=stream)

    with torch.cuda.stream(stream):
        ms, _ = time_calls(call, stream, steps, warmup)
    pairs = int(np.sum(x.lengths * (x.lengths + 1) // 2))
    flops = pairs * x.num_heads * 2 * (x.d_qk + x.d_v)
    mean = float(ms.mean())
    tf = flops / (mean * 1e-3) / 1e12
    return dict(ms=round(mean, 4), tflops=round(tf, 2), roofline=mfma_roofline(tf))


def mfma_roofline(tflops, note=None):
    """A leg's rate against the bf16 MFMA peak."""
    r = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    if note:
        r["note"] = note
    return r


def layer_train_flops(x):
    """Algorithmic FLOPs of one layer's forward and backward (recomputation not counted):
    forward f1, attention over useful pairs and f2; backward two GEMMs per projection
    (activation and weight gradients) and four contractions per useful pair and head."""
    T, dm, H, dqk, dv = int(x.offsets[-1]), x.d_model, x.num_heads, x.d_qk, x.d_v
    f1c = 2 * H * (dqk + dv)
    n = np.diff(np.asarray(x.offsets, np.int64))
    attn = int(np.sum(n * (n + 1) // 2)) * H * 2 * (dqk + dv)
    gemm = 2 * T * dm * f1c + 2 * T * H * dv * dm
    return 3 * gemm + attn + 2 * attn


def leg_backward(steps, warmup):
    """Gradients: attention alone on the length-8192 workload, and whole layers."""
    import torch
    from hstu_jagged_pointwise_amd import ops, synth
    from hstu_jagged_pointwise_amd.device import attn_to_device, layer_to_device
    res = {}
    x = synth.workload_long_attention()
    d = attn_to_device(x)
    g = torch.from_numpy(synth.normal(np.random.default_rng(7), x.v.shape, 1.0, "bf16")).to(
        torch.bfloat16).cuda()
    stream = torch.cuda.Stream()
    desc = ops.attn_desc(len(x.offsets) - 1, x.num_heads, x.d_qk, x.d_v, x.max_seq_len,
                         x.num_pos_buckets, x.num_time_buckets, ops.HSTU_BF16)
    ws = torch.empty(max(1, ops.hstu_attn_bwd_workspace_size(desc, x.offsets)), dtype=torch.uint8,
                     device="cuda")

    def call():
        ops.hstu_attn_bwd(d["offsets"], d["ts"], d["q"], d["k"], d["v"], g, d["rab_pos"],
                          d["rab_time"], max_seq_len=x.max_seq_len, workspace=ws,
                          seq_offsets_host=x.offsets, stream=stream)

    with torch.cuda.stream(stream):
        ms, _ = time_calls(call, stream, max(5, steps // 5), max(2, warmup // 5))
    pairs = int(np.sum(x.lengths * (x.lengths + 1) // 2))
    # dV = A^T G, dP = G V^T, dQ = dZ K, dK = dZ^T Q: four contractions per pair and head
    flops = pairs * x.num_heads * 2 * (2 * x.d_v + 2 * x.d_qk)
    mean = float(ms.mean())
    tf = flops / (mean * 1e-3) / 1e12
    res["attention_length_8192"] = dict(ms=round(mean, 4), tflops=round(tf, 2),
                                        roofline=mfma_roofline(tf))
    for name, xl in (("short_history_layer", synth.workload_short_history_layer()),
                     ("heavy_tail_4_layer_stack", synth.workload_heavy_tail_stack())):
        dl = layer_to_device(xl)
        gy = torch.from_numpy(synth.normal(np.random.default_rng(8), xl.x.shape, 1.0, "bf16")).to(
            torch.bfloat16).cuda()
        ldesc = ops.layer_desc(dl["layers"], len(xl.offsets) - 1, xl.num_heads, xl.d_qk, xl.d_v,
                               xl.d_model, xl.max_seq_len, ops.HSTU_BF16)
        lws = torch.empty(max(1, ops.hstu_layer_bwd_workspace_size(ldesc, xl.offsets)),
                          dtype=torch.uint8, device="cuda")

        def lcall():
            ops.hstu_layer_bwd(dl["offsets"], dl["ts"], dl["x"], dl["layers"], gy,
                               num_heads=xl.num_heads, d_qk=xl.d_qk, d_v=xl.d_v,
                               max_seq_len=xl.max_seq_len, workspace=lws,
                               seq_offsets_host=xl.offsets, stream=stream)

        with torch.cuda.stream(stream):
            ms, _ = time_calls(lcall, stream, max(5, steps // 5), max(2, warmup // 5))
        lm = float(ms.mean())
        ltf = layer_train_flops(xl) * len(xl.layers) / (lm * 1e-3) / 1e12
        res[name] = dict(ms_per_call=round(lm, 4), layers=len(xl.layers),
                         note="forward recomputed inside the call",
                         roofline=mfma_roofline(ltf, "algorithmic FLOPs of forward and backward "
                                                     "(the recomputed forward not counted)"))
    return res


def leg_sl(steps, warmup):
    """Stochastic Length sampling of the heavy-tailed batch (rows, timestamps, indices)."""
    import torch
    from hstu_jagged_pointwise_amd import ops, synth
    x = synth.workload_sl_heavy_tail()
    new, L = ops.hstu_sl_lengths(x.offsets, x.max_seq_len, x.alpha, x.u_keep)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    off, nd, keys = dv(x.offsets), dv(new), dv(x.keys.view(np.int32))
    xx = dv(x.x).to(torch.bfloat16)
    ts = dv(x.ts)
    stream = torch.cuda.Stream()

    def call():
        ops.hstu_sl_sample(off, nd, keys, xx, ts, offsets_host=x.offsets, new_offsets_host=new,
                           stream=stream)

    with torch.cuda.stream(stream):
        ms, _ = time_calls(call, stream, steps, warmup)
    mean = float(ms.mean())
    # select: one 4-byte key per action; gather: each kept row and timestamp read and written
    rows_in, rows_out = int(x.offsets[-1]), int(new[-1])
    by = rows_in * 4 + rows_out * 2 * (x.x.shape[1] * 2 + 8)
    gbs = by / (mean * 1e-3) / 1e9
    return dict(ms=round(mean, 4), rows_in=rows_in, rows_out=rows_out, target_length=int(L),
                note="includes host validation and output allocation",
                roofline={"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                          "bytes_per_call": by})


def leg_copy():
    """A plain 1 GiB device copy: the calibration for the HBM byte counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return dict(bytes_read=n, bytes_written=n, launches=3)


def cpu_baseline(x, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the same workload: whole (sequence, head)
    pairs, longest sequence first, until about budget_s of host time has been spent."""
    from oracle import hstu_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    order = np.argsort(-x.lengths, kind="stable")
    done, flops, t_total, seqs = 0, 0, 0.0, set()
    for b in order:
        s, e = int(x.offsets[b]), int(x.offsets[b + 1])
        n = e - s
        for h in range(x.num_heads):
            t0 = time.perf_counter()
            O.hstu_attention(np.array([0, n]), x.ts[s:e], x.q[s:e, h:h + 1], x.k[s:e, h:h + 1],
                             x.v[s:e, h:h + 1], x.rab_pos[h:h + 1], x.rab_time[h:h + 1],
                             x.max_seq_len)
            t_total += time.perf_counter() - t0
            done += 1
            seqs.add(int(b))
            flops += n * (n + 1) // 2 * 2 * (x.d_qk + x.d_v)
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    try:
        cpu = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")][0]
    except Exception:  # noqa: BLE001
        cpu = "unknown"
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} (sequence, head) pairs of the workload ({len(seqs)} longest sequences), "
                      f"dense fp64 numpy, {flops:.3e} useful FLOPs in {t_total:.1f} s; host CPU {cpu}; "
                      f"{len(os.sched_getaffinity(0))} cores visible"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the clocks take a few dozen calls to settle; the timed calls start after them
    ap.add_argument("--warmup", type=int, default=20)
    # the first leg also keeps warming for this many seconds, so that an idle device has
    # reached its steady clock before the first timed call
    ap.add_argument("--warm-seconds", type=float, default=2.0)
    ap.add_argument("--only", default="attn,softmax,mfalcon,layers,backward,sl,cpu")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    legs = set(args.only.split(","))
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from hstu_jagged_pointwise_amd import ops  # noqa: F401  (fails loudly without libhstu.so)

    if legs == {"copy"}:
        log("copy calibration leg")
        print(json.dumps({"copy": leg_copy()}))
        return
    result = {}
    attn = None
    global LEG_WARM_S
    LEG_WARM_S = args.warm_seconds / 4  # the legs after the first
    if "attn" in legs:
        log("attention leg (length-8192 workload)")
        attn = leg_attention(args.steps, args.warmup, args.warm_seconds)
        log(f"attention: {attn['ms'].mean():.3f} ms/call, {attn['tflops']:.1f} TFLOP/s")
    if "mfalcon" in legs:
        log("M-FALCON leg")
        result["mfalcon"] = leg_mfalcon(args.steps, args.warmup)
        log(f"M-FALCON: {result['mfalcon']['candidates_per_s']:.3e} candidates/s")
        log("M-FALCON leg, 4 layers")
        result["mfalcon_4_layers"] = leg_mfalcon(max(10, args.steps // 4), args.warmup,
                                                 num_layers=4)
        log(f"M-FALCON 4 layers: {result['mfalcon_4_layers']['candidates_per_s']:.3e} "
            "candidates/s")
    if "layers" in legs:
        log("layer legs")
        result["layers"] = leg_layers(args.steps, args.warmup)
    if "softmax" in legs:
        log("softmax-variant leg")
        result["softmax_variant"] = leg_softmax(args.steps, args.warmup)
        if attn is not None:
            result["softmax_variant"]["pointwise_speedup"] = round(
                result["softmax_variant"]["ms"] / float(attn["ms"].mean()), 3)
    if "backward" in legs:
        log("backward legs")
        result["backward"] = leg_backward(args.steps, args.warmup)
    if "sl" in legs:
        log("Stochastic Length leg")
        result["stochastic_length"] = leg_sl(args.steps, args.warmup)
    if attn is None:
        print(json.dumps(result))
        return
    x = attn["x"]
    mean = float(attn["ms"].mean())
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("source_hash") == source_hash():
            traffic = rec.get("bytes_per_launch")
    line = {
        "metric": METRIC,
        "value": round(attn["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "long-sequence jagged HSTU attention: B=8, lengths uniform in [4096,8192] "
                        "with one of 8192, H=4, d_qk=d_v=128, bf16 in / fp32 accumulate, "
                        "128 position + 64 time buckets, causal, 1/N with N=8192",
            "batch": int(len(x.offsets) - 1), "tokens": int(x.offsets[-1]),
            "lengths": [int(v) for v in x.lengths], "heads": x.num_heads, "d_qk": x.d_qk,
            "d_v": x.d_v, "useful_pairs_per_head": attn["pairs"], "flops_per_call": attn["flops"],
        },
        "timing": {"ms_p10": round(float(np.quantile(attn["ms"], 0.1)), 4),
                   "ms_p50": round(float(np.median(attn["ms"])), 4),
                   "ms_p90": round(float(np.quantile(attn["ms"], 0.9)), 4),
                   "wall_s": round(attn["wall"], 4),
                   "warm_seconds": args.warm_seconds,
                   "note": "per-call HIP events on the library's stream; a call is the tile "
                           "planner plus the attention kernel"},
        "roofline": {"bound": "mfma", "achieved": round(attn["tflops"], 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "valu": valu_ceiling(attn),
    }
    line.update(result)
    if "cpu" in legs:
        log("CPU oracle baseline (bounded sample)")
        line["cpu_baseline"] = cpu_baseline(x, args.cpu_budget)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
