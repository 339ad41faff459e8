"""Pins for the fp64 decoding oracle (oracle/decode.py), which reads keys and values through the
page table and places the Lq queries at the last Lq positions.  Its arithmetic is the pinned
forward oracle; what these tests pin is the paging and the positions, with checks that do not
go through its gather:
  * D1  moving the physical pages around (and the table with them) changes nothing;
  * D2  closed form: Q = 0 gives O = the mean of the allowed value rows and L = ln(count),
        which fixes how many positions each query sees (causal offset, length cut);
  * D3  a single dominant key at a chosen position t: O equals that position's value row, read
        by its page and slot directly, which fixes which cache slot holds position t;
  * D4  torch's fp64 scaled_dot_product_attention on keys and values gathered by torch indexing.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_21_amd import inputs


def small(B=3, H=2, Lq=2, d=16, page=8, lo=2, hi=45, causal=True, seed=21):
    w = inputs.DecodeWorkload("t", B=B, H=H, Lq=Lq, d=d, page=page, len_lo=lo, len_hi=hi,
                              causal=causal, seed=seed)
    x = inputs.make_paged_inputs(w)
    return w, x, [oracle.decode_bf16(x[n]) for n in ("q", "k_cache", "v_cache")]


@pytest.mark.parametrize("causal", [True, False])
def test_d1_page_permutation_invariance(causal):
    w, x, (q, kc, vc) = small(causal=causal)
    o1, l1 = oracle.decode_attention(q, kc, vc, x["page_table"], x["seq_lens"], 0.3, causal)
    perm = np.random.default_rng(5).permutation(kc.shape[0])  # new slot of each old page
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    o2, l2 = oracle.decode_attention(q, kc2, vc2, perm[x["page_table"]], x["seq_lens"], 0.3,
                                     causal)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [True, False])
def test_d2_zero_queries(causal):
    w, x, (q, kc, vc) = small(causal=causal, Lq=3)
    q = np.zeros_like(q)
    o, lse = oracle.decode_attention(q, kc, vc, x["page_table"], x["seq_lens"], 0.5, causal)
    for b in range(w.B):
        n = int(x["seq_lens"][b])
        for i in range(w.Lq):
            cnt = n - w.Lq + i + 1 if causal else n
            rows = []
            for t in range(cnt):
                rows.append(vc[x["page_table"][b, t // w.page], :, t % w.page])
            mean = np.mean(np.stack(rows), axis=0)  # [H, d]
            assert np.abs(o[b, :, i] - mean).max() <= 1e-12
            assert np.abs(lse[b, :, i] - np.log(cnt)).max() <= 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_d3_dominant_key(causal):
    w, x, (q, kc, vc) = small(causal=causal, Lq=2, d=8, page=4, lo=9, hi=30)
    kc = np.zeros_like(kc)
    rng = np.random.default_rng(3)
    for b in range(w.B):
        n = int(x["seq_lens"][b])
        t = int(rng.integers(0, n - w.Lq + 1))  # seen by every query row
        page, slot = x["page_table"][b, t // w.page], t % w.page
        kc[page, :, slot, 0] = 10.0
        qb = np.zeros((1, w.H, w.Lq, w.d))
        qb[..., 0] = 10.0
        o, _ = oracle.decode_attention(qb, kc, vc, x["page_table"][b:b + 1],
                                       x["seq_lens"][b:b + 1], 1.0, causal)
        for i in range(w.Lq):
            assert np.abs(o[0, :, i] - vc[page, :, slot]).max() <= 1e-30 * n + 1e-40
        kc[page, :, slot, 0] = 0.0


@pytest.mark.parametrize("causal", [True, False])
def test_d4_torch_sdpa(causal):
    w, x, (q, kc, vc) = small(causal=causal, B=2, H=3, Lq=4, d=16, page=8, lo=4, hi=60)
    o, lse = oracle.decode_attention(q, kc, vc, x["page_table"], x["seq_lens"], 0.25, causal)
    tk, tv = torch.tensor(kc), torch.tensor(vc)
    for b in range(w.B):
        n = int(x["seq_lens"][b])
        pages = torch.tensor(x["page_table"][b])
        k = tk[pages].permute(1, 0, 2, 3).reshape(w.H, -1, w.d)[:, :n]
        v = tv[pages].permute(1, 0, 2, 3).reshape(w.H, -1, w.d)[:, :n]
        pos = torch.arange(n - w.Lq, n)[:, None]
        mask = (torch.arange(n)[None, :] <= pos) if causal else torch.ones(w.Lq, n, dtype=bool)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[b]), k, v, attn_mask=mask, scale=0.25)
        assert np.abs(o[b] - ref.numpy()).max() <= 1e-12
        s = 0.25 * torch.tensor(q[b]) @ k.transpose(1, 2)
        s = s.masked_fill(~mask, float("-inf"))
        assert np.abs(lse[b] - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12
