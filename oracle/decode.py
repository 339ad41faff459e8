"""Plain fp64 CPU oracle for attention over a paged key/value cache (decoding).

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the tests and the
benchmark's CPU-baseline leg, never by the HIP path, and sharing no code with it.

What is computed.  Page "FlashAttention/es" (marovi.ai), section "Variantes y sucesores", names
PagedAttention: during inference the key/value cache is cut into pages, so that many sequences
of different lengths share one pool.  The pages define no arithmetic for it, so the result is the
attention of the definition (attention.py) over each sequence's keys and values laid out in
order: the pages listed in the sequence's row of the page table, concatenated, cut to the
sequence's length.  The Lq query rows of a sequence are its last Lq positions,
seq_len - Lq + i for i = 0 .. Lq-1 (the plain reading of a decoding step); with the causal mask
query i sees the keys at positions 0 .. seq_len - Lq + i, without it all seq_len keys.

Cache layout (the caller's): k_cache, v_cache [n_pages, H, page, d]; page_table [B, max_pages]
of page indices; seq_lens [B].  Position t of sequence b is slot t % page of page
page_table[b, t // page].

All arithmetic is float64 (decode bf16 bit arrays with decode_bf16 first).
"""
from __future__ import annotations

import numpy as np

from .attention import attention


def gather_sequence(cache, page_table_row, seq_len, page):
    """Keys (or values) of one sequence in position order: [H, seq_len, d]."""
    cache = np.asarray(cache)
    n_used = -(-int(seq_len) // int(page))
    pages = [cache[int(p)] for p in np.asarray(page_table_row)[:n_used]]  # each [H, page, d]
    return np.concatenate(pages, axis=1)[:, :int(seq_len)]


def decode_attention(q, k_cache, v_cache, page_table, seq_lens, scale, causal=True):
    """Reference O [B, H, Lq, d] and L [B, H, Lq] (natural log) for the last Lq positions."""
    q = np.asarray(q, dtype=np.float64)
    B, H, Lq, d = q.shape
    page = np.asarray(k_cache).shape[2]
    O = np.empty((B, H, Lq, d))
    L = np.empty((B, H, Lq))
    for b in range(B):
        n = int(seq_lens[b])
        k = gather_sequence(k_cache, page_table[b], n, page).astype(np.float64)
        v = gather_sequence(v_cache, page_table[b], n, page).astype(np.float64)
        # place the queries at their positions; the other rows are never evaluated
        qf = np.zeros((1, H, n, d))
        qf[0, :, n - Lq:] = q[b]
        rows = np.arange(n - Lq, n)
        o, lse = attention(qf, k[None], v[None], scale, mask="causal" if causal else "none",
                           rows=rows)
        O[b], L[b] = o[0], lse[0]
    return O, L
