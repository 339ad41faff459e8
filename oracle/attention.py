"""Plain fp64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  The HIP path never imports it, and it imports nothing from
the HIP path: it shares no kernels, headers, helpers or tables with it.  The only thing both
sides consume is the seeded input generator's output (numpy arrays), passed in by the caller.

What is computed (page "FlashAttention/es", marovi.ai):
  * section "Por qué la atención estándar es lenta": attention is softmax(Q K^T / sqrt(d)) V,
    formed naively by building the full score matrix S, taking a row-wise softmax P, and
    multiplying P by V.  FlashAttention is exact, so its result is this definition; the oracle is
    the definition written out, not the tiled algorithm.
  * section "El truco del softmax en línea": softmax(x)_i = e^{x_i - m} / l with m the maximum
    and l the sum of e^{x - m}.  The oracle takes the two passes literally: pass 1 the row maximum,
    pass 2 the exponentials and their sum.
  * section "El algoritmo FlashAttention", last step: the log-sum-exp L_i = m_i + log l_i is
    written beside O.  log is the natural logarithm (the same section writes softmax with e^x).

Score and mask variants (named on page "El FlexAttention de PyTorch con FlashAttention-4 ...",
liora.io, opening paragraph: ALiBi, sliding window, document masking, soft-capping).  The pages
name them but do not define them; the definitions used are those of the workloads:
  * causal: key j is allowed for query i iff j <= i;
  * sliding window W: iff i - W < j <= i;
  * document: iff doc(i) == doc(j) and j <= i, where doc(x) = r with off[r] <= x < off[r+1];
  * ALiBi: s_ij <- s_ij - slope_h * (i - j), applied to the already scaled score;
  * soft-capping with cap c: s_ij <- c * tanh(s_ij / c), applied to the scaled score.
Order of application (a reading; the pages are silent): scale -> soft-cap -> ALiBi -> mask.

Row convention for a row with no allowed key (unreachable for the workloads; a convention for
other variants): O = 0 and L = -inf.

All arithmetic is float64.  q, k, v are the exact bf16 input values widened to float64; scale,
slopes and cap are the float32 values handed to the HIP path, widened.
"""
from __future__ import annotations

import numpy as np

MASKS = ("none", "causal", "window", "document")


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def doc_index(x: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """doc(x) = r such that offsets[r] <= x < offsets[r+1] (offsets ascending, padded with N)."""
    return np.searchsorted(np.asarray(offsets), np.asarray(x), side="right") - 1


def allowed(rows, cols, N: int, mask: str, window: int = 0, offsets=None) -> np.ndarray:
    """Boolean matrix allowed[a, b] for query rows[a] and key cols[b]; out-of-range is False."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    ok = (i >= 0) & (i < N) & (j >= 0) & (j < N)
    if mask == "none":
        return ok
    if mask == "causal":
        return ok & (j <= i)
    if mask == "window":
        if window < 1:
            raise ValueError("window must be >= 1")
        return ok & (j <= i) & (j > i - window)
    if mask == "document":
        if offsets is None:
            raise ValueError("document mask needs offsets")
        di = doc_index(np.clip(i, 0, N - 1), offsets)
        dj = doc_index(np.clip(j, 0, N - 1), offsets)
        return ok & (j <= i) & (di == dj)
    raise ValueError(f"unknown mask {mask!r}")


def scores(q_rows, k_cols, scale, h, rows, cols, softcap=0.0, slopes=None):
    """Modified scores of query rows x key cols for head h: scale, soft-cap, ALiBi (no mask)."""
    s = float(scale) * (q_rows @ k_cols.T)
    if softcap:
        c = float(softcap)
        s = c * np.tanh(s / c)
    if slopes is not None:
        i = np.asarray(rows, dtype=np.float64)[:, None]
        j = np.asarray(cols, dtype=np.float64)[None, :]
        s = s - float(slopes[h]) * (i - j)
    return s


def attention(q, k, v, scale, mask="none", window=0, softcap=0.0, slopes=None,
              doc_offsets=None, rows=None, heads=None):
    """Reference O and L.

    q, k, v : float64 arrays [B, H, N, d] (use decode_bf16 on bit arrays first).
    rows    : optional 1-D array of query indices to evaluate (default: all N).
    heads   : optional list of (b, h) pairs to evaluate (default: all).
    doc_offsets : [B, max_docs + 1] integer array for the document mask.
    Returns (O [B, H, R, d], L [B, H, R]); heads not evaluated are left as NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.full((B, H, R, d), np.nan)
    L = np.full((B, H, R), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    cols = np.arange(N)
    for b, h in heads:
        off = None if doc_offsets is None else np.asarray(doc_offsets)[b]
        ok = allowed(rows, cols, N, mask, window, off)
        # A key that none of the evaluated rows may attend to gets s = -inf in every row, hence
        # weight e^{-inf} = 0 in every sum below: only keys some row allows are scored (at
        # least one, so that a row with no allowed key still goes through the same steps).
        live = np.flatnonzero(ok.any(axis=0))
        kc = cols[live] if live.size else cols[:1]
        ok = ok[:, kc]
        s = scores(q[b, h, rows], k[b, h, kc], scale, h, rows, kc, softcap, slopes)
        s = np.where(ok, s, -np.inf)
        # pass 1: row maximum
        m = s.max(axis=1)
        empty = ~np.isfinite(m)
        m_safe = np.where(empty, 0.0, m)
        # pass 2: exponentials and their sum
        e = np.exp(s - m_safe[:, None])
        ell = e.sum(axis=1)
        p = e / np.where(empty, 1.0, ell)[:, None]
        O[b, h] = p @ v[b, h, kc]
        with np.errstate(divide="ignore"):
            L[b, h] = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, ell)))
        O[b, h][empty] = 0.0
    return O, L


def attention_blocked(q, k, v, scale, Br, Bc, form="local_max", mask="none", window=0,
                      softcap=0.0, slopes=None, doc_offsets=None):
    """A tiled evaluation of the same softmax, used only to check the oracle (pin P3).

    Page "FlashAttention/es", section "El algoritmo FlashAttention", computes O and L block by
    block.  The mathematics behind it: for a set J of keys of one query row, the triple
    (m_J, l_J, o_J) = (max_{j in J} s_j, sum_j e^{s_j - m_J}, sum_j e^{s_j - m_J} v_j) merges with
    the triple of a disjoint set K into that of J u K by rescaling both to the larger maximum:
    m = max(m_J, m_K), l = e^{m_J - m} l_J + e^{m_K - m} l_K, o likewise.  The merge is
    associative, so folding the key blocks in order and dividing o by l at the end gives the
    two-pass result, with L = m + ln l.
    form="local_max" forms each block's triple with its own maximum and then merges it;
    form="running_max" exponentiates the block directly against the merged maximum (one
    exponential per score).  A block in which a row has no allowed key has m = -inf and
    contributes nothing.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if form not in ("local_max", "running_max"):
        raise ValueError(form)

    def rescale(m_from, m_to):
        # e^{m_from - m_to}, with a set that has seen no allowed key (m = -inf) weighing 0
        with np.errstate(invalid="ignore"):
            return np.where(np.isfinite(m_from), np.exp(m_from - np.where(np.isfinite(m_to),
                                                                          m_to, 0.0)), 0.0)

    def merge(x, y):
        # (m, l, o) of the union of two disjoint key sets
        m = np.maximum(x[0], y[0])
        ax, ay = rescale(x[0], m), rescale(y[0], m)
        return m, ax * x[1] + ay * y[1], ax[:, None] * x[2] + ay[:, None] * y[2]

    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        off = None if doc_offsets is None else np.asarray(doc_offsets)[b]
        for h in range(H):
            for r0 in range(0, N, Br):
                rows = np.arange(r0, min(r0 + Br, N))
                acc = (np.full(rows.size, -np.inf), np.zeros(rows.size), np.zeros((rows.size, d)))
                for c0 in range(0, N, Bc):
                    cols = np.arange(c0, min(c0 + Bc, N))
                    ok = allowed(rows, cols, N, mask, window, off)
                    s = np.where(ok, scores(q[b, h, rows], k[b, h, cols], scale, h, rows, cols,
                                            softcap, slopes), -np.inf)
                    m_blk = s.max(axis=1)
                    # the maximum the block's exponentials are taken against
                    ref = m_blk if form == "local_max" else np.maximum(acc[0], m_blk)
                    e = np.where(ok, np.exp(s - np.where(np.isfinite(ref), ref, 0.0)[:, None]), 0.0)
                    acc = merge(acc, (ref, e.sum(axis=1), e @ v[b, h, cols]))
                m, ell, o = acc
                empty = ell == 0
                O[b, h, rows] = np.where(empty[:, None], 0.0, o / np.where(empty, 1, ell)[:, None])
                with np.errstate(divide="ignore"):
                    L[b, h, rows] = np.where(empty, -np.inf, m + np.log(np.where(empty, 1, ell)))
    return O, L


def allowed_pair_count(N: int, mask: str, window: int = 0, offsets=None, chunk: int = 2048) -> int:
    """Number of allowed (i, j) pairs for one (batch, head), counted from allowed() itself."""
    total = 0
    cols = np.arange(N)
    for r0 in range(0, N, chunk):
        rows = np.arange(r0, min(r0 + chunk, N))
        total += int(allowed(rows, cols, N, mask, window, offsets).sum())
    return total
