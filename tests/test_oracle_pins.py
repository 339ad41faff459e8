"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics, not by the oracle itself.

Each test names the passage or the mathematical fact it rests on.  Every one is chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a transposed operand, the
wrong order of scale and soft-cap, a base-2 instead of natural log) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _variant_kwargs(mask, N, H, B=1, seed=0, alibi=False, softcap=0.0, window=5):
    kw = {"mask": mask, "softcap": softcap}
    if mask == "window":
        kw["window"] = window
    if mask == "document":
        rng = np.random.default_rng(seed + 100)
        offs = []
        for _ in range(B):
            cuts = np.sort(rng.choice(np.arange(1, N), size=min(3, N - 1), replace=False))
            offs.append(np.concatenate([[0], cuts, [N]]))
        kw["doc_offsets"] = np.array(offs)
    if alibi:
        kw["slopes"] = np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)])
    return kw


VARIANTS = [
    ("none", False, 0.0), ("causal", False, 0.0), ("window", False, 0.0),
    ("document", False, 0.0), ("causal", True, 0.0), ("window", True, 0.0),
    ("document", False, 30.0), ("causal", True, 5.0), ("none", True, 2.0),
]


# --- P1: rows of P sum to 1 ("FlashAttention/es", "El truco del softmax en línea") ----------
@pytest.mark.parametrize("mask,alibi,cap", VARIANTS)
def test_rows_of_P_sum_to_one(mask, alibi, cap):
    # With V = identity (d = N) the output row O_i is the probability row P_i itself.
    N, H = 24, 2
    q = rnd((1, H, N, N), 1, 2.0)
    k = rnd((1, H, N, N), 2, 2.0)
    v = np.broadcast_to(np.eye(N), (1, H, N, N)).copy()
    kw = _variant_kwargs(mask, N, H, alibi=alibi, softcap=cap)
    O, L = oracle.attention(q, k, v, 0.3, **kw)
    ok = oracle.allowed(np.arange(N), np.arange(N), N, mask, kw.get("window", 0),
                        kw.get("doc_offsets", [None])[0])
    assert np.all(np.abs(O.sum(axis=-1) - 1.0) <= 1e-12)
    assert np.all(O >= 0)
    assert np.all(O[..., ~ok] == 0.0)  # masked pairs get exactly zero weight
    # ... and the weights are the normalised exponentials of the scores (definition of softmax)
    for h in range(H):
        s = oracle.scores(q[0, h], k[0, h], 0.3, h, np.arange(N), np.arange(N), cap,
                          kw.get("slopes"))
        for i in range(N):
            cols = np.nonzero(ok[i])[0]
            w = np.exp(s[i, cols] - s[i, cols].max())
            np.testing.assert_allclose(O[0, h, i, cols], w / w.sum(), rtol=1e-12, atol=1e-15)


# --- P2: constant V gives O = V (convex combination) ---------------------------------------
@pytest.mark.parametrize("mask,alibi,cap", VARIANTS)
def test_constant_v_gives_v(mask, alibi, cap):
    B, H, N, d = 2, 3, 33, 8
    q, k = rnd((B, H, N, d), 3), rnd((B, H, N, d), 4)
    c = rnd((B, H, 1, d), 5)
    v = np.broadcast_to(c, (B, H, N, d)).copy()
    O, _ = oracle.attention(q, k, v, 0.35, **_variant_kwargs(mask, N, H, B, alibi=alibi,
                                                              softcap=cap))
    assert np.max(np.abs(O - c)) <= 1e-12


# --- P3: the tiled online recurrence equals the two-pass softmax ----------------------------
@pytest.mark.parametrize("form", ["local_max", "running_max"])
@pytest.mark.parametrize("mask,alibi,cap", VARIANTS)
def test_blocked_recurrence_matches_two_pass(form, mask, alibi, cap):
    B, H, N, d = 2, 2, 37, 5
    q, k, v = rnd((B, H, N, d), 6, 1.5), rnd((B, H, N, d), 7, 1.5), rnd((B, H, N, d), 8)
    kw = _variant_kwargs(mask, N, H, B, seed=1, alibi=alibi, softcap=cap, window=4)
    O, L = oracle.attention(q, k, v, 0.4, **kw)
    for Br, Bc in [(1, 1), (4, 6), (7, 5), (16, 16), (37, 37), (64, 3)]:
        Ob, Lb = oracle.attention_blocked(q, k, v, 0.4, Br, Bc, form=form, **kw)
        assert np.max(np.abs(Ob - O)) <= 1e-12, (Br, Bc)
        assert np.max(np.abs(Lb - L)) <= 1e-12, (Br, Bc)


# --- P4: the vectorised mask equals a literal double loop over the definitions --------------
def _literal_allowed(N, mask, window, offsets):
    out = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for j in range(N):
            if mask == "none":
                a = True
            elif mask == "causal":
                a = j <= i
            elif mask == "window":
                a = (i - window < j) and (j <= i)
            else:  # document: walk the offsets to find each token's document
                di = dj = None
                for r in range(len(offsets) - 1):
                    if offsets[r] <= i < offsets[r + 1]:
                        di = r
                    if offsets[r] <= j < offsets[r + 1]:
                        dj = r
                a = (di == dj) and (j <= i)
            out[i, j] = a
    return out


@pytest.mark.parametrize("N", [1, 2, 7, 33, 64])
def test_mask_matches_literal_loops(N):
    idx = np.arange(N)
    for mask in ("none", "causal"):
        assert np.array_equal(oracle.allowed(idx, idx, N, mask), _literal_allowed(N, mask, 0, None))
    for W in (1, 3, N, N + 5):
        assert np.array_equal(oracle.allowed(idx, idx, N, "window", W),
                              _literal_allowed(N, "window", W, None))
    rng = np.random.default_rng(N)
    docs = [np.array([0, N])]  # one document
    if N > 1:
        docs.append(np.arange(N + 1))  # every token its own document (length 1)
        cuts = np.sort(rng.choice(np.arange(1, N), size=min(4, N - 1), replace=False))
        docs.append(np.concatenate([[0], cuts, [N], [N, N]]))  # padded with N
    for off in docs:
        assert np.array_equal(oracle.allowed(idx, idx, N, "document", 0, off),
                              _literal_allowed(N, "document", 0, off))
    # keys or queries beyond N are never allowed
    big = np.arange(N + 3)
    a = oracle.allowed(big, big, N, "none")
    assert not a[N:, :].any() and not a[:, N:].any()


def test_allowed_pair_counts_closed_form():
    N = 300
    assert oracle.allowed_pair_count(N, "none") == N * N
    assert oracle.allowed_pair_count(N, "causal") == N * (N + 1) // 2
    for W in (1, 17, 299, 300, 1000):
        assert oracle.allowed_pair_count(N, "window", W) == sum(min(i + 1, W) for i in range(N))
    lens = [5, 128, 1, 166]
    off = np.concatenate([[0], np.cumsum(lens)])
    assert oracle.allowed_pair_count(N, "document", 0, off) == sum(n * (n + 1) // 2 for n in lens)


# --- P5: closed forms with Q = 0 ----------------------------------------------------------
def _n_allowed(i, mask, W, off):
    if mask == "none":
        return None
    if mask == "causal":
        return i + 1
    if mask == "window":
        return min(i + 1, W)
    start = max(o for o in off if o <= i)
    return i - start + 1


@pytest.mark.parametrize("mask", ["none", "causal", "window", "document"])
def test_zero_q_closed_form(mask):
    # Every score is 0, so the softmax is uniform over the allowed keys:
    # L_i = ln(n_i) and O_i = mean of the allowed v_j.
    B, H, N, d, W = 1, 2, 40, 6, 7
    q = np.zeros((B, H, N, d))
    k, v = rnd((B, H, N, d), 9), rnd((B, H, N, d), 10)
    off = np.array([0, 1, 9, 30, N])
    O, L = oracle.attention(q, k, v, 0.5, mask=mask, window=W, doc_offsets=off[None])
    for i in range(N):
        n = _n_allowed(i, mask, W, off) or N
        lo = i - n + 1 if mask != "none" else 0
        hi = i + 1 if mask != "none" else N
        assert abs(L[0, 0, i] - math.log(n)) <= 1e-12
        np.testing.assert_allclose(O[0, :, i], v[0, :, lo:hi].mean(axis=1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask", ["causal", "window"])
def test_zero_q_alibi_geometric_series(mask):
    # Scores are -slope*(i-j) for the allowed j = i, i-1, ..., i-n+1; the maximum is 0 (j = i),
    # so L_i = ln sum_{t<n} e^{-slope t} = ln((1 - e^{-slope n}) / (1 - e^{-slope})) and the
    # weights are e^{-slope t} / that sum.
    B, H, N, d, W = 1, 4, 50, 3, 9
    slopes = np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)])
    q = np.zeros((B, H, N, d))
    k, v = rnd((B, H, N, d), 11), rnd((B, H, N, d), 12)
    O, L = oracle.attention(q, k, v, 0.5, mask=mask, window=W, slopes=slopes)
    for h in range(H):
        a = slopes[h]
        for i in range(N):
            n = i + 1 if mask == "causal" else min(i + 1, W)
            Z = (1 - math.exp(-a * n)) / (1 - math.exp(-a))
            assert abs(L[0, h, i] - math.log(Z)) <= 1e-12
            w = np.array([math.exp(-a * t) for t in range(n)]) / Z
            ref = sum(w[t] * v[0, h, i - t] for t in range(n))
            np.testing.assert_allclose(O[0, h, i], ref, rtol=0, atol=1e-12)


def test_softcap_zero_q_and_large_cap():
    B, H, N, d = 1, 2, 30, 4
    k, v = rnd((B, H, N, d), 13), rnd((B, H, N, d), 14)
    q0 = np.zeros((B, H, N, d))
    O1, L1 = oracle.attention(q0, k, v, 0.5, mask="causal", softcap=30.0)
    O2, L2 = oracle.attention(q0, k, v, 0.5, mask="causal")
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)  # tanh(0) = 0
    q = rnd((B, H, N, d), 15, 3.0)
    O3, L3 = oracle.attention(q, k, v, 0.5, mask="causal", softcap=1e9)
    O4, L4 = oracle.attention(q, k, v, 0.5, mask="causal")
    assert np.max(np.abs(O3 - O4)) <= 1e-12 and np.max(np.abs(L3 - L4)) <= 1e-12


def test_softcap_values_and_order():
    # Two keys with raw dot products +6 and -2000, scale 0.5, cap 30.  The scaled scores are
    # 3 and -1000; capped (after scaling) they are 30*tanh(0.1) and ~ -30.  Softcap applied
    # before the scale would give 0.5*30*tanh(0.2) instead.
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[6.0, 0.0], [-2000.0, 0.0]]]])
    q2 = np.broadcast_to(q, (1, 1, 2, 2)).copy()
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    O, L = oracle.attention(q2, k, v, 0.5, softcap=30.0)
    s0, s1 = 30.0 * math.tanh(0.1), 30.0 * math.tanh(-1000.0 / 30.0)
    assert abs(s1 + 30.0) < 1e-12
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert abs(O[0, 0, 0, 0] - w0) <= 1e-15 and abs(O[0, 0, 0, 1] - (1 - w0)) <= 1e-15
    assert abs(L[0, 0, 0] - (s0 + math.log1p(math.exp(s1 - s0)))) <= 1e-12
    assert abs(s0 - 2.9900398387486744) < 1e-12  # 30 tanh(0.1) = 30 * 0.0996679946249558...


# --- P6: library cross-check (torch SDPA in float64 on the CPU, scipy logsumexp) ------------
@pytest.mark.parametrize("mask,alibi", [("none", False), ("causal", False), ("window", False),
                                        ("document", False), ("causal", True),
                                        ("window", True), ("none", True)])
def test_matches_torch_sdpa_fp64(mask, alibi):
    B, H, N, d = 2, 3, 70, 16
    q, k, v = rnd((B, H, N, d), 16, 1.7), rnd((B, H, N, d), 17, 1.7), rnd((B, H, N, d), 18)
    scale = 1.0 / math.sqrt(d)
    kw = _variant_kwargs(mask, N, H, B, seed=3, alibi=alibi, window=11)
    O, L = oracle.attention(q, k, v, scale, **kw)
    idx = np.arange(N)
    for b in range(B):
        off = kw["doc_offsets"][b] if mask == "document" else None
        ok = oracle.allowed(idx, idx, N, mask, kw.get("window", 0), off)
        bias = np.where(ok, 0.0, -np.inf)[None].repeat(H, 0)
        if alibi:
            bias = bias - kw["slopes"][:, None, None] * (idx[:, None] - idx[None, :])[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b]), torch.from_numpy(k[b]), torch.from_numpy(v[b]),
            attn_mask=torch.from_numpy(bias), scale=scale).numpy()
        np.testing.assert_allclose(O[b], ref, rtol=0, atol=1e-12)
        s = np.einsum("hnd,hmd->hnm", q[b], k[b]) * scale + bias
        np.testing.assert_allclose(L[b], scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-12)


# --- golden fixtures (hand-derived exact values) ------------------------------------------
def test_golden_fixtures():
    with open(os.path.join(GOLDEN, "tiny_cases.json")) as f:
        cases = json.load(f)["cases"]
    assert cases
    for c in cases:
        q, k, v = (np.array(c[x], dtype=np.float64)[None, None] for x in ("q", "k", "v"))
        O, L = oracle.attention(q, k, v, c["scale"], mask=c["mask"], window=c.get("window", 0),
                                softcap=c.get("softcap", 0.0),
                                slopes=np.array(c["slopes"]) if "slopes" in c else None,
                                doc_offsets=np.array([c["doc_offsets"]]) if "doc_offsets" in c
                                else None)
        np.testing.assert_allclose(O[0, 0], np.array(c["O"]), rtol=0, atol=1e-12, err_msg=c["name"])
        Lref = np.array([eval(x, {"ln": math.log, "__builtins__": {}}) if isinstance(x, str) else x
                         for x in c["L"]])
        np.testing.assert_allclose(L[0, 0], Lref, rtol=0, atol=1e-12, err_msg=c["name"])


def test_decode_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    expect = [1.0, -1.0, 3.140625, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41]
    got = oracle.decode_bf16(bits)
    assert list(got) == expect
