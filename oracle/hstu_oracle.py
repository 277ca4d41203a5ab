"""CPU oracle for the HSTU jagged pointwise-attention path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg use this module. The GPU library never imports it,
calls it or falls back to it.

This is a plain, slow, fp64 implementation of what an HSTU layer computes. It
runs dense per sequence and per head and has no tiling or fusion. It follows the
three HSTU layer equations as the chenhuiyu.github.io HSTU chapter states them
("What an HSTU layer changes", equations 1-3):

    U, V, Q, K = Split(phi1(f1(X)))                    (eq. 1)
    A(X) V     = phi2(Q K^T + rab^{p,t}) V             (eq. 2)
    Y          = f2(Norm(A(X) V) (.) U)                (eq. 3)

phi1 and phi2 are SiLU. rab^{p,t} is a relative attention bias over position
and elapsed time (same section; Yonas Stephen's course, "Problem 2"). Both pages
say there is no row softmax, which lets an attention row carry both relevance
and count ("No sequence-wise softmax"; course "Problem 1"). The pages do not fix
the 1/N scale, the bucket functions, the LayerNorm details or the layouts. This
module takes the following readings:

* scale: phi2(.) is multiplied by 1/N after SiLU. N is passed explicitly.
* no 1/sqrt(d): eq. 2 has none.
* position bucket: bp = min(i - j, P - 1), for query position i and key
  position j.
* time bucket: bt = min(floor(log2(max(dt, 0) + 1)), T - 1), where
  dt = t_query - t_key in integer seconds. floor(log2) is computed exactly on
  integers.
* bias = rab_pos[h, bp] + rab_time[h, bt]. A missing table (or missing
  timestamps, for the time table) adds 0.
* mask: key j is visible to query i iff j <= i. A hidden pair contributes an
  exact 0. It is a select, never an additive -inf, because SiLU(-inf) is NaN.
* Norm: LayerNorm over the whole concatenated row of H*d_v values, with the
  biased variance, eps as given, and gamma = 1, beta = 0 when not given.
* Split order: f1's output features are the row blocks [U | V | Q | K]. Inside
  each block, heads are contiguous chunks of d. phi1 applies to all four blocks,
  the gate U included.
* f1 and f2 are affine maps y = x W^T + b. W is stored [out, in].
* M-FALCON (HSTU chapter, "M-FALCON"; praveentn.live note, "What HSTU actually
  changed"; course, "Serving it: M-FALCON"): a candidate sits at position n_h,
  right after its user's n_h history actions, and carries its own timestamp.
  It attends to every history action and to itself, and to no other
  candidate. History rows never see candidates, so the history is computed
  once and reused for every candidate microbatch.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "silu", "round_storage", "floor_log2", "pos_bucket", "time_bucket", "bucket_indices",
    "bias_from_buckets", "bias_matrix", "attention_one_head",
    "hstu_attention", "hstu_attention_rows", "layer_norm_rows", "hstu_layer", "hstu_layer_stack", "mfalcon_score",
    "mfalcon_by_definition", "candidate_attention", "attention_pairs", "attention_flops",
]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def round_storage(x, storage):
    """Round to the storage format of a stored intermediate. storage=None keeps fp64.
    storage="bf16" rounds to the nearest bfloat16 value (ties to even): first to fp32
    (nearest), then keep the top 16 bits of the fp32 pattern, rounding half to even."""
    x = _f64(x)
    if storage is None:
        return x
    if storage != "bf16":
        raise ValueError(storage)
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    keep = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = (keep.astype(np.uint32) << 16).view(np.float32)
    out = np.where(np.isnan(f), np.float32(np.nan), out)
    return out.astype(np.float64)


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------
def silu(x):
    """SiLU(x) = x * sigmoid(x) = x / (1 + e^{-x}). The HSTU chapter uses it
    for both phi1 and phi2 (eqs. 1-2)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def floor_log2(x):
    """Exact floor(log2(x)) for integers x >= 1, by binary search on the bit length."""
    x = np.array(x, dtype=np.int64, copy=True)
    if np.any(x < 1):
        raise ValueError("floor_log2 needs x >= 1")
    r = np.zeros_like(x)
    for s in (32, 16, 8, 4, 2, 1):
        m = x >= (np.int64(1) << np.int64(s))
        r[m] += s
        x[m] >>= s
    return r


def pos_bucket(dpos, P):
    """Relative-position bucket, clamped linear: min(i - j, P - 1), for i - j >= 0."""
    dpos = np.asarray(dpos, dtype=np.int64)
    return np.minimum(np.maximum(dpos, 0), P - 1)


def time_bucket(dt, T):
    """Elapsed-time bucket: min(floor(log2(max(dt, 0) + 1)), T - 1), with dt in seconds."""
    dt = np.asarray(dt, dtype=np.int64)
    return np.minimum(floor_log2(np.maximum(dt, 0) + 1), T - 1)


def bucket_indices(qpos, kpos, qts, kts, rab_pos, rab_time):
    """The (position, time) bucket index matrices [nq, nk] of every query against every
    key. They do not depend on the head. An index matrix is None where its table (or,
    for time, the timestamps) is missing."""
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    bp = bt = None
    if rab_pos is not None:
        bp = pos_bucket(qpos[:, None] - kpos[None, :], rab_pos.shape[1])
    if rab_time is not None and qts is not None and kts is not None:
        bt = time_bucket(np.asarray(qts, np.int64)[:, None] - np.asarray(kts, np.int64)[None, :],
                         rab_time.shape[1])
    return bp, bt


def bias_from_buckets(h, shape, bp, bt, rab_pos, rab_time):
    """rab^{p,t} of head h: rab_pos[h][bp] + rab_time[h][bt], a missing term adding 0."""
    bias = np.zeros(shape, dtype=np.float64)
    if bp is not None:
        bias += _f64(rab_pos)[h][bp]
    if bt is not None:
        bias += _f64(rab_time)[h][bt]
    return bias


def bias_matrix(h, qpos, kpos, qts, kts, rab_pos, rab_time):
    """rab^{p,t}[i, j] for head h, over query positions and timestamps against key
    positions and timestamps. Missing tables or timestamps add 0."""
    bp, bt = bucket_indices(qpos, kpos, qts, kts, rab_pos, rab_time)
    return bias_from_buckets(h, (len(qpos), len(kpos)), bp, bt, rab_pos, rab_time)


# ---------------------------------------------------------------------------
# attention (eq. 2) over one sequence and head, then the jagged batch
# ---------------------------------------------------------------------------
def attention_one_head(q, k, v, visible, bias, N):
    """O = (SiLU(Q K^T + bias) / N, masked to 0 where not visible) V for one head.

    q [nq, d_qk], k [nk, d_qk], v [nk, d_v], visible bool [nq, nk], bias [nq, nk]."""
    s = _f64(q) @ _f64(k).T + bias
    a = np.where(visible, silu(s) / float(N), 0.0)
    return a @ _f64(v)


def hstu_attention(offsets, ts, q, k, v, rab_pos, rab_time, N, u=None, gamma=None, beta=None,
                   eps=1e-5):
    """Jagged causal HSTU attention (eq. 2), optionally followed by Norm(AV) (.) U (eq. 3).

    q, k: [T_tot, H, d_qk]; v, u: [T_tot, H, d_v]; offsets int64 [B+1].
    Returns fp64 [T_tot, H, d_v]. It holds AV without u, else LN(AV)*gamma+beta times U."""
    offsets = np.asarray(offsets, dtype=np.int64)
    q, k, v = _f64(q), _f64(k), _f64(v)
    Ttot, H, dv = v.shape
    out = np.zeros((Ttot, H, dv), dtype=np.float64)
    for b in range(len(offsets) - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        n = e - s
        if n == 0:
            continue
        pos = np.arange(n, dtype=np.int64)
        t = None if ts is None else np.asarray(ts, np.int64)[s:e]
        visible = pos[None, :] <= pos[:, None]
        bp, bt = bucket_indices(pos, pos, t, t, rab_pos, rab_time)  # the same for every head
        for h in range(H):
            bias = bias_from_buckets(h, (n, n), bp, bt, rab_pos, rab_time)
            out[s:e, h, :] = attention_one_head(q[s:e, h], k[s:e, h], v[s:e, h], visible, bias, N)
    if u is None:
        return out
    z = layer_norm_rows(out.reshape(Ttot, H * dv), gamma, beta, eps)
    return (z * _f64(u).reshape(Ttot, H * dv)).reshape(Ttot, H, dv)


def hstu_attention_rows(offsets, ts, q, k, v, rab_pos, rab_time, N, rows):
    """Selected rows of hstu_attention (without the gate), each computed on its own from
    its sequence prefix: row r at position i of sequence b attends keys 0..i of b.
    rows are global token indices. Returns fp64 [len(rows), H, d_v]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    H, dv = v.shape[1], v.shape[2]
    out = np.zeros((len(rows), H, dv), dtype=np.float64)
    for idx, r in enumerate(rows):
        r = int(r)
        b = int(np.searchsorted(offsets, r, side="right")) - 1
        s = int(offsets[b])
        i = r - s
        kpos = np.arange(i + 1, dtype=np.int64)
        qts = None if ts is None else np.asarray(ts, np.int64)[r:r + 1]
        kts = None if ts is None else np.asarray(ts, np.int64)[s:r + 1]
        vis = np.ones((1, i + 1), dtype=bool)
        for h in range(H):
            bias = bias_matrix(h, np.array([i]), kpos, qts, kts, rab_pos, rab_time)
            out[idx, h] = attention_one_head(_f64(q[r:r + 1, h]), _f64(k[s:r + 1, h]),
                                             _f64(v[s:r + 1, h]), vis, bias, N)[0]
    return out


def layer_norm_rows(z, gamma=None, beta=None, eps=1e-5):
    """LayerNorm of each row: (z - mean) / sqrt(var + eps) * gamma + beta, biased variance."""
    z = _f64(z)
    mu = z.mean(axis=1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=1, keepdims=True)
    y = (z - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * _f64(gamma)[None, :]
    if beta is not None:
        y = y + _f64(beta)[None, :]
    return y


# ---------------------------------------------------------------------------
# the HSTU layer (eqs. 1-3) and a stack of layers
# ---------------------------------------------------------------------------
def _affine(x, w, b):
    y = _f64(x) @ _f64(w).T
    if b is not None:
        y = y + _f64(b)[None, :]
    return y


def _split_uvqk(x, w, H, d_qk, d_v, storage=None):
    """eq. 1: SiLU(f1(X)), split into the row blocks [U | V | Q | K]."""
    z = round_storage(silu(_affine(x, w.w1, w.b1)), storage)
    n = z.shape[0]
    cu = H * d_v
    cq = H * d_qk
    U = z[:, 0:cu].reshape(n, H, d_v)
    V = z[:, cu:2 * cu].reshape(n, H, d_v)
    Q = z[:, 2 * cu:2 * cu + cq].reshape(n, H, d_qk)
    K = z[:, 2 * cu + cq:2 * cu + 2 * cq].reshape(n, H, d_qk)
    return U, V, Q, K


def hstu_layer(offsets, ts, x, w, H, d_qk, d_v, N, eps=1e-5, residual=0, storage=None):
    """One HSTU layer over a jagged batch: eq. 1, causal eq. 2, then eq. 3 with
    f2(G) = G W2^T + b2 (+ X when residual is set).

    storage=None computes in fp64 throughout. storage="bf16" rounds the tensors that a
    bf16 implementation stores between its steps (U, V, Q, K after eq. 1, the gated
    G, and Y) to bf16. The HSTU chapter sizes a layer's activation state in bfloat16
    ("Gating instead of a separate FFN"). This variant measures how much storage
    rounding alone moves each output row."""
    U, V, Q, K = _split_uvqk(x, w, H, d_qk, d_v, storage)
    g = hstu_attention(offsets, ts, Q, K, V, w.rab_pos, w.rab_time, N, u=U, gamma=w.gamma,
                       beta=w.beta, eps=eps)
    g = round_storage(g.reshape(g.shape[0], H * d_v), storage)
    y = _affine(g, w.w2, w.b2)
    if residual:
        y = y + _f64(x)
    return round_storage(y, storage)


def hstu_layer_stack(offsets, ts, x, layers, H, d_qk, d_v, N, eps=1e-5, residual=0,
                     storage=None):
    """X_{l+1} = layer_l(X_l) for each layer in order."""
    y = _f64(x)
    for w in layers:
        y = hstu_layer(offsets, ts, y, w, H, d_qk, d_v, N, eps, residual, storage)
    return y


# ---------------------------------------------------------------------------
# M-FALCON candidate scoring
# ---------------------------------------------------------------------------
def candidate_attention(Qc, Kc, Vc, Kh, Vh, cand_ts, hist_ts, rab_pos, rab_time, N):
    """eq. 2 for candidates under the M-FALCON mask. Each candidate sits at position
    n_h = len(Kh) and attends to all history keys j (relative position n_h - j,
    elapsed time t_c - t_j) and to its own key (relative position 0, elapsed time 0).

    Qc, Kc [nc, H, d_qk]; Vc [nc, H, d_v]; Kh [n_h, H, d_qk]; Vh [n_h, H, d_v].
    Returns fp64 [nc, H, d_v]."""
    Qc, Kc, Vc, Kh, Vh = _f64(Qc), _f64(Kc), _f64(Vc), _f64(Kh), _f64(Vh)
    nc, H, dv = Vc.shape
    nh = Kh.shape[0]
    o = np.zeros((nc, H, dv), dtype=np.float64)
    qpos = np.full(nc, nh, dtype=np.int64)
    kpos = np.arange(nh, dtype=np.int64)
    have_t = cand_ts is not None and hist_ts is not None
    zero = np.zeros(1, np.int64)
    bp, bt = bucket_indices(qpos, kpos, cand_ts if have_t else None, hist_ts if have_t else None,
                            rab_pos, rab_time)  # the same for every head
    for h in range(H):
        bias_h = bias_from_buckets(h, (nc, nh), bp, bt, rab_pos, rab_time)
        vis = np.ones((nc, nh), dtype=bool)
        o[:, h, :] = attention_one_head(Qc[:, h], Kh[:, h], Vh[:, h], vis, bias_h, N)
        self_bias = bias_matrix(h, zero, zero, zero if have_t else None,
                                zero if have_t else None, rab_pos, rab_time)[0, 0]
        s_self = np.sum(Qc[:, h] * Kc[:, h], axis=1) + self_bias
        o[:, h, :] += (silu(s_self) / float(N))[:, None] * Vc[:, h]
    return o


def mfalcon_score(hist_offsets, hist_ts, hist_x, cand_offsets, cand_ts, cand_x, layers, H, d_qk,
                  d_v, N, microbatch, w_head=None, eps=1e-5, residual=0, storage=None):
    """M-FALCON as the pages describe it: for each user, compute the history once
    per layer and keep that layer's history K and V. Then score the candidates in
    microbatches. Each candidate attends to all n_h cached history keys at
    relative positions n_h - j, and to itself at position offset 0 with
    elapsed time 0. No candidate sees another candidate.

    Returns (cand_out fp64 [C_tot, d_model], logits fp64 [C_tot] or None)."""
    hist_offsets = np.asarray(hist_offsets, np.int64)
    cand_offsets = np.asarray(cand_offsets, np.int64)
    d_model = hist_x.shape[1] if hist_x.size else cand_x.shape[1]
    out = np.zeros((int(cand_offsets[-1]), d_model), dtype=np.float64)
    for b in range(len(hist_offsets) - 1):
        hs, he = int(hist_offsets[b]), int(hist_offsets[b + 1])
        nh = he - hs
        h_off = np.array([0, nh], dtype=np.int64)
        hts = None if hist_ts is None else np.asarray(hist_ts, np.int64)[hs:he]
        # history pass, once: cache each layer's history K and V
        xh = _f64(hist_x[hs:he])
        cache = []
        for w in layers:
            U, V, Q, K = _split_uvqk(xh, w, H, d_qk, d_v, storage)
            cache.append((K, V))
            xh = hstu_layer(h_off, hts, xh, w, H, d_qk, d_v, N, eps, residual, storage)
        # candidate microbatches against the cache
        cs, ce = int(cand_offsets[b]), int(cand_offsets[b + 1])
        for m0 in range(cs, ce, max(1, int(microbatch))):
            m1 = min(ce, m0 + max(1, int(microbatch)))
            xc = _f64(cand_x[m0:m1])
            cts = None if cand_ts is None else np.asarray(cand_ts, np.int64)[m0:m1]
            nc = m1 - m0
            for w, (Kh, Vh) in zip(layers, cache):
                U, V, Q, K = _split_uvqk(xc, w, H, d_qk, d_v, storage)
                o = candidate_attention(Q, K, V, Kh, Vh, cts, hts, w.rab_pos, w.rab_time, N)
                z = layer_norm_rows(o.reshape(nc, H * d_v), w.gamma, w.beta, eps)
                g = round_storage(z * U.reshape(nc, H * d_v), storage)
                y = _affine(g, w.w2, w.b2)
                if residual:
                    y = y + xc
                xc = round_storage(y, storage)
            out[m0:m1] = xc
    logits = None if w_head is None else out @ _f64(w_head)
    return out, logits


def mfalcon_by_definition(hist_offsets, hist_ts, hist_x, cand_offsets, cand_ts, cand_x, layers, H,
                          d_qk, d_v, N, w_head=None, eps=1e-5, residual=0):
    """Candidate c's output is the last row of the causal layer stack run over
    the sequence (user history followed by c), with the same N. This is slow and
    only for small inputs; it pins mfalcon_score."""
    hist_offsets = np.asarray(hist_offsets, np.int64)
    cand_offsets = np.asarray(cand_offsets, np.int64)
    d_model = hist_x.shape[1] if hist_x.size else cand_x.shape[1]
    out = np.zeros((int(cand_offsets[-1]), d_model), dtype=np.float64)
    for b in range(len(hist_offsets) - 1):
        hs, he = int(hist_offsets[b]), int(hist_offsets[b + 1])
        for c in range(int(cand_offsets[b]), int(cand_offsets[b + 1])):
            xs = np.concatenate([_f64(hist_x[hs:he]), _f64(cand_x[c:c + 1])], axis=0)
            ts = None
            if hist_ts is not None and cand_ts is not None:
                ts = np.concatenate([np.asarray(hist_ts, np.int64)[hs:he],
                                     np.asarray(cand_ts, np.int64)[c:c + 1]])
            off = np.array([0, xs.shape[0]], dtype=np.int64)
            y = hstu_layer_stack(off, ts, xs, layers, H, d_qk, d_v, N, eps, residual)
            out[c] = y[-1]
    logits = None if w_head is None else out @ _f64(w_head)
    return out, logits


# ---------------------------------------------------------------------------
# work accounting (used by tests and the benchmark's CPU-baseline leg)
# ---------------------------------------------------------------------------
def attention_pairs(offsets):
    """Number of visible (query, key) pairs per head under the causal mask."""
    n = np.diff(np.asarray(offsets, np.int64))
    return int(np.sum(n * (n + 1) // 2))


def attention_flops(offsets, H, d_qk, d_v):
    """Algorithmic FLOPs of eq. 2: 2*(d_qk + d_v) per visible pair and head."""
    return attention_pairs(offsets) * H * 2 * (d_qk + d_v)
