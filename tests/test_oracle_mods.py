"""Pins for the modification oracle (oracle/mods.py): with functions that spell out the fixed
variants it must equal the fixed-variant oracle (itself pinned in test_oracle_pins.py), its
tile table must equal the fixed-variant table, and masks with a closed-form result must give
that result."""
import numpy as np
import pytest

import oracle
from oracle import mods


def qkv(B, H, N, d, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((B, H, N, d)) * sigma for _ in range(3))


def alibi(s, b, h, i, j, p):
    return s - p[h] * (i - j)


def causal(b, i, j, p):
    return j <= i


def test_alibi_causal_equals_fixed_variant():
    q, k, v = qkv(2, 3, 70, 16, 1)
    slopes = np.array([0.5, 0.25, 0.125])
    o1, l1 = mods.attention_mod(q, k, v, 0.3, alibi, causal, slopes)
    o2, l2 = oracle.attention(q, k, v, 0.3, mask="causal", slopes=slopes)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


@pytest.mark.parametrize("W", [1, 7, 64, 200])
def test_window_mask_equals_fixed_variant(W):
    q, k, v = qkv(1, 2, 90, 8, 2)
    o1, l1 = mods.attention_mod(q, k, v, 0.5, None, lambda b, i, j, p: (j <= i) & (j > i - p[0]),
                                np.array([W]))
    o2, l2 = oracle.attention(q, k, v, 0.5, mask="window", window=W)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


def test_softcap_score_equals_fixed_variant():
    q, k, v = qkv(1, 2, 50, 16, 3, sigma=3.0)
    o1, l1 = mods.attention_mod(q, k, v, 0.25, lambda s, b, h, i, j, p: p[0] * np.tanh(s / p[0]),
                                None, np.array([5.0]))
    o2, l2 = oracle.attention(q, k, v, 0.25, softcap=5.0)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


def test_document_mask_from_params_equals_fixed_variant():
    q, k, v = qkv(2, 1, 60, 8, 4)
    offs = np.array([[0, 13, 40, 60, 60], [0, 60, 60, 60, 60]])

    def doc(b, i, j, p):
        o = p[b]
        return (j <= i) & (np.searchsorted(o, i, side="right") == np.searchsorted(o, j, side="right"))
    o1, l1 = mods.attention_mod(q, k, v, 0.4, None, doc, offs)
    o2, l2 = oracle.attention(q, k, v, 0.4, mask="document", doc_offsets=offs)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


def test_diagonal_mask_returns_v_and_the_diagonal_score():
    q, k, v = qkv(1, 2, 33, 8, 5)
    o, l = mods.attention_mod(q, k, v, 0.7, None, lambda b, i, j, p: j == i)
    assert np.array_equal(o, v)
    assert np.allclose(l, 0.7 * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-12)


def test_head_dependent_score_mask_and_empty_rows():
    """-inf from the score function masks per head; a row with nothing allowed gets O = 0 and
    L = -inf; Q = 0 with a prefix-LM mask gives the mean of the allowed values, L = ln(count)."""
    B, H, N, d = 1, 2, 40, 4
    q, k, v = qkv(B, H, N, d, 6)
    o, l = mods.attention_mod(q, k, v, 1.0,
                              lambda s, b, h, i, j, p: np.where((h == 1) & (j > i), -np.inf, s))
    o0, l0 = oracle.attention(q, k, v, 1.0)
    o1, l1 = oracle.attention(q, k, v, 1.0, mask="causal")
    assert np.abs(o[:, 0] - o0[:, 0]).max() < 1e-12 and np.abs(o[:, 1] - o1[:, 1]).max() < 1e-12
    o, l = mods.attention_mod(q, k, v, 1.0, None, lambda b, i, j, p: (j < i - 100))
    assert np.all(o == 0) and np.all(np.isneginf(l))
    P = 7
    o, l = mods.attention_mod(np.zeros_like(q), k, v, 1.0, None,
                              lambda b, i, j, p: (j < p[0]) | (j <= i), np.array([P]))
    for i in range(N):
        n = max(P, i + 1)
        assert np.allclose(o[0, :, i], v[0, :, :n].mean(axis=1), atol=1e-12)
        assert np.allclose(l[0, :, i], np.log(n), atol=1e-12)


@pytest.mark.parametrize("N", [1, 63, 300, 1000])
def test_tile_table_equals_fixed_table(N):
    c1, n1, l1 = mods.mod_tile_table(N, 1, causal)
    c2, n2, l2 = oracle.tile_table(N, 256, 64, "causal")
    assert np.array_equal(c1, c2) and np.array_equal(n1, n2) and np.array_equal(l1, l2)
    W = 100
    c1, n1, l1 = mods.mod_tile_table(N, 1, lambda b, i, j, p: (j <= i) & (j > i - W))
    c2, n2, l2 = oracle.tile_table(N, 256, 64, "window", window=W)
    assert np.array_equal(c1, c2) and np.array_equal(n1, n2) and np.array_equal(l1, l2)


def test_tile_table_literal_loop_small():
    """A mask with no structure (a hash of i, j and b) against a literal loop over every pair."""
    N, B, Br, Bc = 45, 2, 8, 4

    def mask(b, i, j, p):
        return ((i * 7 + j * 13 + b * 5) % 5) != 0
    cls, cnt, lst = mods.mod_tile_table(N, B, mask, Br=Br, Bc=Bc)
    n_qt, n_kt = -(-N // Br), -(-N // Bc)
    for b in range(B):
        for qt in range(n_qt):
            got = []
            for kt in range(n_kt):
                pairs = [(i, j) for i in range(qt * Br, qt * Br + Br) for j in range(kt * Bc, kt * Bc + Bc)]
                ok = [i < N and j < N and ((i * 7 + j * 13 + b * 5) % 5) != 0 for i, j in pairs]
                c = 2 if all(ok) else (1 if any(ok) else 0)
                assert cls[b, qt, kt] == c
                if c:
                    got.append(kt)
            assert cnt[b, qt] == len(got) and list(lst[b, qt, :len(got)]) == got
            assert not lst[b, qt, len(got):].any()
