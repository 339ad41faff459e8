"""Plain CPU oracle for attention with user-supplied score and mask modifications.

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the tests and the
benchmark's CPU-baseline leg, never by the HIP path, and sharing no code with it.

What is computed.  Page "El FlexAttention de PyTorch con FlashAttention-4 ..." (liora.io),
opening paragraph: FlexAttention lets the user express the score modification and the mask as
small functions that the attention kernel applies.  The page gives no signature; the reading
used here (and by the runtime-compiled kernels) is:
  * score_mod(s, b, h, i, j, p) maps the scaled score s = scale * q_i . k_j of query i, key j,
    batch entry b, head h to the score that enters the softmax (p: the caller's parameters);
  * mask_mod(b, i, j, p) says whether key j is allowed for query i (the same for every head).
The result is the definition (page "FlashAttention/es", section "Por qué la atención estándar es
lenta"): S is materialised per (b, h), the functions are applied element by element, disallowed
pairs get -inf, and the softmax is taken in two passes (row maximum, then the exponentials and
their sum; section "El truco del softmax en línea"), with L = m + ln l.  A row with no allowed
key gets O = 0 and L = -inf, the convention of oracle.attention.

Here the functions are numpy-vectorised Python callables: s is an [R, C] array and i, j are
broadcastable index arrays ([R, 1] and [1, C]); they return arrays of the broadcast shape.
"""
from __future__ import annotations

import numpy as np


def attention_mod(q, k, v, scale, score_mod=None, mask_mod=None, params=None, rows=None,
                  heads=None):
    """Reference O [B, H, R, d] and L [B, H, R] (float64).  q, k, v: float64 [B, H, N, d];
    rows: query indices (default all); heads: (b, h) pairs (default all; others stay NaN)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.full((B, H, rows.size, d), np.nan)
    L = np.full((B, H, rows.size), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    i = rows[:, None]
    j = np.arange(N)[None, :]
    for b, h in heads:
        s = float(scale) * (q[b, h, rows] @ k[b, h].T)
        if score_mod is not None:
            s = np.broadcast_to(np.asarray(score_mod(s, b, h, i, j, params), dtype=np.float64),
                                s.shape)
        if mask_mod is not None:
            ok = np.broadcast_to(np.asarray(mask_mod(b, i, j, params), dtype=bool), s.shape)
            s = np.where(ok, s, -np.inf)
        m = s.max(axis=1)                       # pass 1: the row maximum
        empty = ~np.isfinite(m)
        m_safe = np.where(empty, 0.0, m)
        e = np.exp(s - m_safe[:, None])         # pass 2: the exponentials and their sum
        ell = e.sum(axis=1)
        p = e / np.where(empty, 1.0, ell)[:, None]
        O[b, h] = p @ v[b, h]
        O[b, h][empty] = 0.0
        with np.errstate(divide="ignore"):
            L[b, h] = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, ell)))
    return O, L


def mod_tile_table(N: int, B: int, mask_mod, params=None, Br: int = 256, Bc: int = 64):
    """Block table of a mask function, pair by pair (the convention of oracle.tiles): per batch
    entry b and tile (qt, kt), class 0 if no in-range pair (i < N, j < N) is allowed, 2 if all
    Br * Bc pairs are in range and allowed, 1 otherwise; kv_cnt and the ascending kv_list.
    Returns (cls int8 [B, n_qt, n_kt], kv_cnt int32 [B, n_qt], kv_list int32 [B, n_qt, n_kt])."""
    n_qt = -(-N // Br)
    n_kt = -(-N // Bc)
    cls = np.zeros((B, n_qt, n_kt), dtype=np.int8)
    cnt = np.zeros((B, n_qt), dtype=np.int32)
    lst = np.zeros((B, n_qt, n_kt), dtype=np.int32)
    jj = np.arange(n_kt * Bc)[None, :]
    for b in range(B):
        for qt in range(n_qt):
            ii = np.arange(qt * Br, qt * Br + Br)[:, None]
            ok = (ii < N) & (jj < N) & np.broadcast_to(
                np.asarray(mask_mod(b, ii, jj, params), dtype=bool), (Br, n_kt * Bc))
            a = ok.reshape(Br, n_kt, Bc)
            c = np.where(a.all(axis=(0, 2)), 2, np.where(a.any(axis=(0, 2)), 1, 0))
            cls[b, qt] = c.astype(np.int8)
            nz = np.nonzero(c)[0]
            cnt[b, qt] = nz.size
            lst[b, qt, :nz.size] = nz
    return cls, cnt, lst
