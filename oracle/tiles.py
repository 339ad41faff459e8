"""Brute-force block-mask table for the tiled forward pass.

TEST INFRASTRUCTURE ONLY (same import rule as oracle.attention).

The tiled pass (page "FlashAttention/es", section "El algoritmo FlashAttention") walks, for each
block of Br query rows, over blocks of Bc keys.  Skipping blocks whose scores are all masked is
the block sparsity that page "El FlexAttention de PyTorch con FlashAttention-4 ..." (section
"Limitaciones actuales") names; the same page family notes that the method combines with sparse
or banded masks ("FlashAttention/es", section "Comparación con otros métodos de atención
rápida").  Neither page fixes a data structure, so the one used here is:

  tile (qt, kt) covers query rows [qt*Br, qt*Br + Br) and keys [kt*Bc, kt*Bc + Bc);
  class 0 (empty)   : no in-range (i < N, j < N) pair of the tile is allowed;
  class 2 (full)    : all Br*Bc pairs are in range and allowed;
  class 1 (partial) : otherwise.
  kv_cnt[qt]  = number of tiles of row qt with class != 0;
  kv_list[qt] = their kt in ascending order, padded to n_kt entries with 0.

Every class here is evaluated pair by pair from oracle.attention.allowed(): this is the
definition, with no closed form.  The table has one row block per batch entry for the document
mask (offsets differ per batch) and a single one otherwise.
"""
from __future__ import annotations

import numpy as np

from .attention import allowed


def tile_table(N: int, Br: int, Bc: int, mask: str, window: int = 0, doc_offsets=None):
    """Returns (cls int8 [Bm, n_qt, n_kt], kv_cnt int32 [Bm, n_qt], kv_list int32 [Bm, n_qt, n_kt])."""
    n_qt = -(-N // Br)
    n_kt = -(-N // Bc)
    if mask == "document":
        offs = [np.asarray(o) for o in np.asarray(doc_offsets)]
    else:
        offs = [None]
    Bm = len(offs)
    cls = np.zeros((Bm, n_qt, n_kt), dtype=np.int8)
    cnt = np.zeros((Bm, n_qt), dtype=np.int32)
    lst = np.zeros((Bm, n_qt, n_kt), dtype=np.int32)
    cols = np.arange(n_kt * Bc)
    for bm, off in enumerate(offs):
        for qt in range(n_qt):
            rows = np.arange(qt * Br, qt * Br + Br)
            a = allowed(rows, cols, N, mask, window, off).reshape(Br, n_kt, Bc)
            any_ = a.any(axis=(0, 2))
            all_ = a.all(axis=(0, 2))
            c = np.where(all_, 2, np.where(any_, 1, 0)).astype(np.int8)
            cls[bm, qt] = c
            nz = np.nonzero(c)[0]
            cnt[bm, qt] = nz.size
            lst[bm, qt, :nz.size] = nz
    return cls, cnt, lst


def tile_class_counts(cls: np.ndarray):
    """(empty, partial, full) tile counts of a class array."""
    return int((cls == 0).sum()), int((cls == 1).sum()), int((cls == 2).sum())
