"""Pins for the brute-force block-mask table (class / kv_cnt / kv_list).

The table is defined pair by pair (see oracle/tiles.py).  These tests check it against an
independent per-tile loop on tiny shapes and against counts that follow from the geometry of
each mask.
"""
import numpy as np
import pytest

import oracle
from exact_io_aware_21_amd import inputs


def _literal_table(N, Br, Bc, mask, window, off):
    n_qt, n_kt = -(-N // Br), -(-N // Bc)
    cls = np.zeros((n_qt, n_kt), dtype=np.int8)
    for qt in range(n_qt):
        for kt in range(n_kt):
            n_in, n_ok = 0, 0
            for i in range(qt * Br, qt * Br + Br):
                for j in range(kt * Bc, kt * Bc + Bc):
                    if i >= N or j >= N:
                        continue
                    n_in += 1
                    if mask == "none":
                        a = True
                    elif mask == "causal":
                        a = j <= i
                    elif mask == "window":
                        a = i - window < j <= i
                    else:
                        a = j <= i and not any(i >= o > j for o in off)  # no boundary between j and i
                    n_ok += a
            cls[qt, kt] = 2 if n_ok == Br * Bc else (1 if n_ok else 0)
    return cls


@pytest.mark.parametrize("N,Br,Bc", [(1, 4, 4), (17, 4, 8), (33, 8, 4), (40, 16, 8), (64, 16, 16)])
@pytest.mark.parametrize("mask", ["none", "causal", "window", "document"])
def test_table_matches_literal_loops(N, Br, Bc, mask):
    rng = np.random.default_rng(N * 7 + Br)
    for W in ([1, 3, 9, N + 2] if mask == "window" else [0]):
        offs = None
        if mask == "document":
            cuts = np.sort(rng.choice(np.arange(1, N), size=min(3, N - 1), replace=False)) if N > 1 \
                else np.array([], dtype=int)
            offs = np.concatenate([[0], cuts, [N]])[None]
        cls, cnt, lst = oracle.tile_table(N, Br, Bc, mask, W, offs)
        ref = _literal_table(N, Br, Bc, mask, W, None if offs is None else offs[0])
        assert np.array_equal(cls[0], ref)
        for qt in range(cls.shape[1]):
            nz = np.nonzero(ref[qt])[0]
            assert cnt[0, qt] == nz.size
            assert np.array_equal(lst[0, qt, :nz.size], nz)
            assert not lst[0, qt, nz.size:].any()


@pytest.mark.parametrize("n", [1, 2, 5, 16])
def test_causal_square_tiles_counts(n):
    # Br = Bc and N = n*Br: the diagonal tiles are partial, the strict lower triangle is full,
    # the strict upper triangle is empty.
    cls, cnt, _ = oracle.tile_table(n * 8, 8, 8, "causal")
    e, p, f = oracle.tile_class_counts(cls)
    assert (e, p, f) == (n * (n - 1) // 2, n, n * (n - 1) // 2)
    assert np.array_equal(cnt[0], np.arange(1, n + 1))


def test_long_causal_tile_counts():
    # N = 16384 with 128 x 64 tiles: q-tile t has 2t full tiles and 2 partial ones (kt = 2t, 2t+1).
    cls, cnt, lst = oracle.tile_table(16384, 128, 64, "causal")
    assert oracle.tile_class_counts(cls) == (16256, 256, 16256)
    assert np.array_equal(cnt[0], 2 * np.arange(128) + 2)
    assert np.array_equal(lst[0, 5, :12], np.arange(12))


def test_window_tile_counts():
    # window 1024, N = 8192, 128 x 64 tiles: q-tile t (rows 128t..128t+127) touches keys
    # 128t-1023 .. 128t+127; with 64-key tiles that is kt = 2t-16 .. 2t+1 (clipped at 0).
    cls, cnt, _ = oracle.tile_table(8192, 128, 64, "window", 1024)
    for t in range(64):
        lo = max(0, 2 * t - 16)
        nz = np.nonzero(cls[0, t])[0]
        assert np.array_equal(nz, np.arange(lo, 2 * t + 2))
        full = np.nonzero(cls[0, t] == 2)[0]
        # full iff keys [64kt, 64kt+63] within [r-1023, r] for every row r of the tile
        exp_full = [kt for kt in range(128) if 64 * kt + 63 <= 128 * t and 64 * kt >= 128 * t + 127 - 1023]
        assert list(full) == exp_full


def test_document_table_of_the_workload():
    w = inputs.WORKLOADS["doc_softcap30_h16_n16384_d64"]
    inp = inputs.make_inputs(w, with_qkv=False)
    off = inp["doc_offsets"]
    cls, cnt, lst = oracle.tile_table(w.N, 128, 64, "document", 0, off)
    # every allowed pair lies in some non-empty tile, so the non-empty tiles cover
    # at least the allowed-pair count, and no empty tile holds an allowed pair
    allowed_pairs = oracle.allowed_pair_count(w.N, "document", 0, off[0])
    n_nonempty = int((cls != 0).sum())
    assert n_nonempty * 128 * 64 >= allowed_pairs
    assert int((cls == 2).sum()) * 128 * 64 <= allowed_pairs
    assert np.array_equal(cnt[0], (cls[0] != 0).sum(axis=1))


def test_none_mask_tail_tiles_partial():
    cls, cnt, _ = oracle.tile_table(100, 32, 16, "none")
    assert (cls[0, :3, :6] == 2).all()
    assert (cls[0, 3, :] == 1).all() and (cls[0, :, 6] == 1).all()
    assert (cnt[0] == 7).all()
