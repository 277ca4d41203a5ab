"""CPU oracle for the gradients of the HSTU layer (the backward pass).

TEST INFRASTRUCTURE ONLY. Only the test suite uses this module. The GPU library
never imports it, calls it or falls back to it.

The HSTU chapter of chenhuiyu.github.io trains the model generatively ("What an
HSTU layer changes", equations 1-3; "Three more scaling components"), so every
forward step needs its gradient. These are the gradients of the forward oracle
(oracle/hstu_oracle.py, same readings: SiLU for phi1 and phi2, the 1/N scale
after SiLU, clamped position buckets, log2 time buckets, an exact 0 for hidden
pairs, LayerNorm over the whole H*d_v row), written out by the chain rule in
fp64, densely per sequence and head:

  attention, per head, visible pairs j <= i:
    z_ij  = q_i . k_j + bias_ij           a_ij = SiLU(z_ij) / N
    o_i   = sum_j a_ij v_j
  with g_i = dL/do_i:
    dv_j  = sum_i a_ij g_i
    da_ij = g_i . v_j
    dz_ij = da_ij SiLU'(z_ij) / N         (0 for hidden pairs)
    dq_i  = sum_j dz_ij k_j               dk_j = sum_i dz_ij q_i
    d rab_pos[h][p]  = sum of dz_ij over visible pairs with position bucket p
    d rab_time[h][t] = sum of dz_ij over visible pairs with time bucket t
  SiLU'(x) = s (1 + x (1 - s)), s = 1 / (1 + e^{-x}).

  gate (eq. 3), per row with y = LN(o) gamma + beta and out = y (.) u:
    du = g (.) y,   dy = g (.) u,   dgamma = sum_rows dy (.) xhat,   dbeta = sum_rows dy
    do = (dxhat - mean(dxhat) - xhat mean(dxhat (.) xhat)) / sqrt(var + eps),
    dxhat = dy (.) gamma

  layer: z1 = X W1^T + b1, [U|V|Q|K] = SiLU(z1); Y = G W2^T + b2 (+ X):
    dG = dY W2, dW2 = dY^T G, db2 = sum_rows dY
    dz1 = d[U|V|Q|K] (.) SiLU'(z1), dW1 = dz1^T X, db1 = sum_rows dz1
    dX = dz1 W1 (+ dY when residual)

Nothing here reuses the forward's code path for the gradient: the forward
oracle is called only to supply values (for the finite-difference pins in the
tests), and the backward formulas above are evaluated directly.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import hstu_oracle as F

__all__ = ["silu_grad", "attention_backward", "attention_backward_rows", "gate_backward",
           "layer_backward", "layer_stack_backward", "LayerGrads"]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def silu_grad(x):
    """d/dx SiLU(x) = s (1 + x (1 - s)) with s = sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def _buckets(n, t, P, T):
    """Position and time bucket matrices [n, n] of one sequence (query i, key j)."""
    pos = np.arange(n, dtype=np.int64)
    bp = F.pos_bucket(pos[:, None] - pos[None, :], P)
    bt = None
    if t is not None:
        bt = F.time_bucket(t[:, None] - t[None, :], T)
    return bp, bt


def attention_backward(offsets, ts, q, k, v, rab_pos, rab_time, N, d_out, P=None, T=None,
                       term_scale=None):
    """Gradients of causal jagged attention without the gate (eq. 2).

    q, k [T_tot, H, d_qk]; v, d_out [T_tot, H, d_v]. Returns
    (dq, dk, dv, d_rab_pos [H, P] or None, d_rab_time [H, T] or None), fp64.
    P and T give the table widths when a table is absent but its gradient is wanted: an
    absent table counts as zeros, and the time table's gradient needs timestamps (it is
    zero without them).
    term_scale, a dict, receives "d_rab_pos" and "d_rab_time": the same sums over |dz|, the
    size of the terms each table entry adds up (the scale of its rounding error)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(d_out)
    Ttot, H, dqk = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    P = rab_pos.shape[1] if rab_pos is not None else P
    T = rab_time.shape[1] if rab_time is not None else T
    have_ts = ts is not None
    use_time = rab_time is not None and have_ts
    drp = np.zeros((H, P)) if P else None
    drt = np.zeros((H, T)) if T else None  # stays zero without timestamps
    arp = np.zeros((H, P)) if P else None
    art = np.zeros((H, T)) if T else None
    for b in range(len(offsets) - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        n = e - s
        if n == 0:
            continue
        t = np.asarray(ts, np.int64)[s:e] if have_ts else None
        pos = np.arange(n, dtype=np.int64)
        vis = pos[None, :] <= pos[:, None]
        bp, bt = _buckets(n, t, P if P else 1, T if T else 1)
        for h in range(H):
            bias = F.bias_matrix(h, pos, pos, t, t, rab_pos, rab_time if use_time else None)
            z = q[s:e, h] @ k[s:e, h].T + bias
            a = np.where(vis, F.silu(z) / float(N), 0.0)
            dv[s:e, h] = a.T @ g[s:e, h]
            da = g[s:e, h] @ v[s:e, h].T
            dz = np.where(vis, da * silu_grad(z) / float(N), 0.0)
            dq[s:e, h] = dz @ k[s:e, h]
            dk[s:e, h] = dz.T @ q[s:e, h]
            if drp is not None:
                drp[h] += np.bincount(bp[vis], weights=dz[vis], minlength=P)
                arp[h] += np.bincount(bp[vis], weights=np.abs(dz[vis]), minlength=P)
            if drt is not None and have_ts:
                drt[h] += np.bincount(bt[vis], weights=dz[vis], minlength=T)
                art[h] += np.bincount(bt[vis], weights=np.abs(dz[vis]), minlength=T)
    if term_scale is not None:
        term_scale["d_rab_pos"], term_scale["d_rab_time"] = arp, art
    return dq, dk, dv, drp, drt


def attention_backward_rows(offsets, ts, q, k, v, rab_pos, rab_time, N, d_out, rows):
    """dq, dk and dv of selected global rows, each from its own definition: dq_i needs
    row i of dz (keys j <= i), dk_j and dv_j need column j of dz and a (queries i >= j).
    For checking long sequences one row at a time. Returns fp64 arrays [len(rows), H, d]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(d_out)
    H = q.shape[1]
    use_time = rab_time is not None and ts is not None
    tsa = np.asarray(ts, np.int64) if use_time else None
    dq = np.zeros((len(rows), H, q.shape[2]))
    dk = np.zeros((len(rows), H, k.shape[2]))
    dv = np.zeros((len(rows), H, v.shape[2]))
    for idx, r in enumerate(rows):
        r = int(r)
        b = int(np.searchsorted(offsets, r, side="right")) - 1
        s, e = int(offsets[b]), int(offsets[b + 1])
        p = r - s
        keys = np.arange(p + 1)           # keys seen by query p
        qrys = np.arange(p, e - s)        # queries that see key p
        for h in range(H):
            # row p of the pair matrices: query p against keys 0..p
            bias = F.bias_matrix(h, np.array([p]), keys, tsa[r:r + 1] if use_time else None,
                                 tsa[s:s + p + 1] if use_time else None, rab_pos,
                                 rab_time if use_time else None)[0]
            z = k[s:s + p + 1, h] @ q[r, h] + bias
            dz = (v[s:s + p + 1, h] @ g[r, h]) * silu_grad(z) / float(N)
            dq[idx, h] = dz @ k[s:s + p + 1, h]
            # column p: queries p..n-1 against key p
            bias = F.bias_matrix(h, qrys, np.array([p]), tsa[s + p:e] if use_time else None,
                                 tsa[r:r + 1] if use_time else None, rab_pos,
                                 rab_time if use_time else None)[:, 0]
            z = q[s + p:e, h] @ k[r, h] + bias
            a = F.silu(z) / float(N)
            dzc = (g[s + p:e, h] @ v[r, h]) * silu_grad(z) / float(N)
            dk[idx, h] = dzc @ q[s + p:e, h]
            dv[idx, h] = a @ g[s + p:e, h]
    return dq, dk, dv


def gate_backward(o, u, gamma, beta, eps, d_out):
    """Gradients of out = (LN(o) gamma + beta) (.) u over rows of width W = H*d_v.

    o, u, d_out [R, W]. Returns (do, du, dgamma [W], dbeta [W])."""
    o, u, g = _f64(o), _f64(u), _f64(d_out)
    W = o.shape[1]
    gam = np.ones(W) if gamma is None else _f64(gamma)
    bet = np.zeros(W) if beta is None else _f64(beta)
    mu = o.mean(axis=1, keepdims=True)
    var = ((o - mu) ** 2).mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (o - mu) * rstd
    y = xhat * gam[None, :] + bet[None, :]
    du = g * y
    dy = g * u
    dgamma = (dy * xhat).sum(axis=0)
    dbeta = dy.sum(axis=0)
    dxhat = dy * gam[None, :]
    do = rstd * (dxhat - dxhat.mean(axis=1, keepdims=True)
                 - xhat * (dxhat * xhat).mean(axis=1, keepdims=True))
    return do, du, dgamma, dbeta


@dataclass
class LayerGrads:
    dx: np.ndarray
    dw1: np.ndarray
    db1: np.ndarray
    dw2: np.ndarray
    db2: np.ndarray
    d_rab_pos: Optional[np.ndarray]
    d_rab_time: Optional[np.ndarray]
    dgamma: np.ndarray
    dbeta: np.ndarray
    # the size of the terms each reduction adds up: sums over |dz| for the two tables,
    # |A|^T |B| for a weight gradient A^T B, column sums of |A| for a bias gradient
    d_rab_pos_terms: Optional[np.ndarray] = None
    d_rab_time_terms: Optional[np.ndarray] = None
    dw1_terms: Optional[np.ndarray] = None
    db1_terms: Optional[np.ndarray] = None
    dw2_terms: Optional[np.ndarray] = None
    db2_terms: Optional[np.ndarray] = None


def layer_backward(offsets, ts, x, w, H, d_qk, d_v, N, d_y, eps=1e-5, residual=0, storage=None):
    """Gradients of one HSTU layer (eqs. 1-3) in fp64, given dL/dY.

    w has the fields of the forward oracle's layer weights (w1, b1, rab_pos, rab_time,
    gamma, beta, w2, b2). storage=None keeps fp64 throughout. storage="bf16" rounds
    the tensors that a bf16 implementation stores between its steps, the same reading
    as the forward oracle's storage variant (the HSTU chapter sizes a layer's
    activation state in bfloat16, "Gating instead of a separate FFN"):
    [U|V|Q|K], G, dG, dO, dU, dQ, dK, dV, dz1 and dX. It measures how much storage
    rounding alone moves each gradient row."""
    r = lambda a: F.round_storage(a, storage)
    x, gy = _f64(x), _f64(d_y)
    R = x.shape[0]
    z1 = x @ _f64(w.w1).T
    if w.b1 is not None:
        z1 = z1 + _f64(w.b1)[None, :]
    act = r(F.silu(z1))
    cu, cq = H * d_v, H * d_qk
    U = act[:, 0:cu]
    V = act[:, cu:2 * cu].reshape(R, H, d_v)
    Q = act[:, 2 * cu:2 * cu + cq].reshape(R, H, d_qk)
    K = act[:, 2 * cu + cq:2 * cu + 2 * cq].reshape(R, H, d_qk)
    o = F.hstu_attention(offsets, ts, Q, K, V, w.rab_pos, w.rab_time, N).reshape(R, cu)
    y = F.layer_norm_rows(o, w.gamma, w.beta, eps)
    G = r(y * U)
    # f2
    dG = r(gy @ _f64(w.w2))
    dw2 = gy.T @ G
    db2 = gy.sum(axis=0)
    # gate and norm
    do, dU, dgamma, dbeta = gate_backward(o, U, w.gamma, w.beta, eps, dG)
    do, dU = r(do), r(dU)
    # attention
    terms = {}
    dQ, dK, dV, drp, drt = attention_backward(offsets, ts, Q, K, V, w.rab_pos, w.rab_time, N,
                                              do.reshape(R, H, d_v), term_scale=terms)
    dact = np.concatenate([dU, r(dV).reshape(R, cu), r(dQ).reshape(R, cq), r(dK).reshape(R, cq)],
                          axis=1)
    dz1 = r(dact * silu_grad(z1))
    dw1 = dz1.T @ x
    db1 = dz1.sum(axis=0)
    dx = dz1 @ _f64(w.w1)
    if residual:
        dx = dx + gy
    dx = r(dx)
    return LayerGrads(dx, dw1, db1, dw2, db2, drp, drt, dgamma, dbeta, terms["d_rab_pos"],
                      terms["d_rab_time"], np.abs(dz1).T @ np.abs(x), np.abs(dz1).sum(axis=0),
                      np.abs(gy).T @ np.abs(G), np.abs(gy).sum(axis=0))


def layer_stack_backward(offsets, ts, x, layers, H, d_qk, d_v, N, d_y, eps=1e-5, residual=0,
                         storage=None):
    """Gradients of a stack of layers (X_{l+1} = layer_l(X_l)) given dL/dY of the last one.
    The inputs of each layer come from the forward oracle, then layer_backward runs from
    the last layer to the first, each layer's dX being the previous layer's dY.
    storage as in layer_backward (and the forward oracle, for the layer inputs).
    Returns (dL/dX of the stack input, [LayerGrads per layer])."""
    xs = [_f64(x)]
    for w in layers[:-1]:
        xs.append(F.hstu_layer(offsets, ts, xs[-1], w, H, d_qk, d_v, N, eps, residual, storage))
    grads = [None] * len(layers)
    g = _f64(d_y)
    for l in range(len(layers) - 1, -1, -1):
        grads[l] = layer_backward(offsets, ts, xs[l], layers[l], H, d_qk, d_v, N, g, eps, residual,
                                  storage)
        g = grads[l].dx
    return g, grads
