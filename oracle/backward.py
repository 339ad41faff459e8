"""Plain fp64 CPU oracle for the attention backward pass.

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the tests and the benchmark's
CPU-baseline leg, never by the HIP path, and sharing no code with it.

What is computed (page "FlashAttention/es", marovi.ai, section "Paso hacia atrás y
recomputación"): the backward pass of attention, i.e. the gradients dQ, dK, dV of a loss whose
gradient with respect to the output O is dO.  The page fixes what the fast kernel consumes (the
saved log-sum-exp L and dO, with S and P recomputed instead of stored) but not the formulas; the
result is the vector-Jacobian product of the forward definition (see attention.py), which this
oracle writes out with the whole score matrix materialised, one (batch, head) at a time:

  t = scale * Q K^T;  s_c = cap * tanh(t / cap) (soft-cap, else s_c = t);  s = s_c + bias (ALiBi);
  s = -inf where the mask disallows;  P = row softmax(s);  O = P V.
  dV = P^T dO
  dP = dO V^T
  dS = P * (dP - D),  D_i = sum_j P_ij dP_ij          (Jacobian of the row softmax)
  dT = dS * (1 - (s_c / cap)^2)                       (soft-cap; dT = dS without it)
  dQ = scale * dT K,  dK = scale * dT^T Q
The ALiBi bias and the mask do not depend on Q, K, V, so they only shape P.  A row with no allowed
key has O = 0 by convention (see attention.py) and contributes nothing.

All arithmetic is float64; inputs are float64 arrays (decode bf16 bit patterns with decode_bf16).
"""
from __future__ import annotations

import numpy as np

from .attention import allowed


def _head_forward(qh, kh, vh, scale, h, N, mask, window, softcap, slopes, off):
    """Materialised forward of one head: returns (P, s_c) with s_c the soft-capped scaled score."""
    rows = np.arange(N)
    t = float(scale) * (qh @ kh.T)
    if softcap:
        c = float(softcap)
        s_c = c * np.tanh(t / c)
    else:
        s_c = t
    s = s_c
    if slopes is not None:
        s = s - float(slopes[h]) * (rows[:, None] - rows[None, :]).astype(np.float64)
    ok = allowed(rows, rows, N, mask, window, off)
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    e = np.exp(s - np.where(empty, 0.0, m)[:, None])
    ell = e.sum(axis=1)
    p = e / np.where(empty, 1.0, ell)[:, None]
    p[empty] = 0.0
    return p, s_c


def attention_backward(q, k, v, do, scale, mask="none", window=0, softcap=0.0, slopes=None,
                       doc_offsets=None, heads=None):
    """Reference dQ, dK, dV [B, H, N, d] (float64).  Heads not in `heads` are left as NaN."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, d = q.shape
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        off = None if doc_offsets is None else np.asarray(doc_offsets)[b]
        p, s_c = _head_forward(q[b, h], k[b, h], v[b, h], scale, h, N, mask, window, softcap,
                               slopes, off)
        g = do[b, h]
        dv[b, h] = p.T @ g
        dp = g @ v[b, h].T
        dsum = (p * dp).sum(axis=1)
        ds = p * (dp - dsum[:, None])
        if softcap:
            ds = ds * (1.0 - (s_c / float(softcap)) ** 2)
        dq[b, h] = float(scale) * (ds @ k[b, h])
        dk[b, h] = float(scale) * (ds.T @ q[b, h])
    return dq, dk, dv


def backward_row_dot(o, do):
    """D_i = sum_c dO_ic O_ic: the row term of the softmax Jacobian written with the output
    (equal to sum_j P_ij dP_ij because O_i = sum_j P_ij V_j)."""
    return (np.asarray(o, dtype=np.float64) * np.asarray(do, dtype=np.float64)).sum(axis=-1)


def backward_magnitudes(q, k, v, do, scale, mask="none", window=0, softcap=0.0, slopes=None,
                        doc_offsets=None, heads=None):
    """Sums of absolute terms behind each gradient element (float64, [B, H, N, d] each):
         M_dV = |P|^T |dO|,   M_dK = scale |dT'|^T |Q|,   M_dQ = scale |dT'| |K|,
    with |dT'| = (|dS| + P * sum_c |dO_c O_c|) * |1 - (s_c/cap)^2|.  Rounding one operand of every
    product term to a relative precision u changes a gradient element by at most u times its M
    (the P * sum|dO O| part covers D_i = dO_i . O_i formed from an O rounded the same way).
    These are error scales for comparing a reduced-precision implementation, not gradients."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, d = q.shape
    mq = np.full(q.shape, np.nan)
    mk = np.full(k.shape, np.nan)
    mv = np.full(v.shape, np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        off = None if doc_offsets is None else np.asarray(doc_offsets)[b]
        p, s_c = _head_forward(q[b, h], k[b, h], v[b, h], scale, h, N, mask, window, softcap,
                               slopes, off)
        g = do[b, h]
        o = p @ v[b, h]
        dp = g @ v[b, h].T
        ds = p * (dp - (p * dp).sum(axis=1)[:, None])
        mds = np.abs(ds) + p * np.abs(g * o).sum(axis=1)[:, None]
        if softcap:
            mds = mds * np.abs(1.0 - (s_c / float(softcap)) ** 2)
        mv[b, h] = p.T @ np.abs(g)
        mk[b, h] = float(scale) * (mds.T @ np.abs(q[b, h]))
        mq[b, h] = float(scale) * (mds @ np.abs(k[b, h]))
    return mq, mk, mv
