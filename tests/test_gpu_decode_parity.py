"""GPU parity of paged decoding (attn_decode, through the C ABI) against the fp64 oracle.

Tolerance: the forward pass's, max|O - O_ref| <= 1e-2 and max|L - L_ref| <= 1e-3, checked on
the fp32-output run (the kernels' arithmetic); the bf16-output run must equal the fp32 run
rounded to bf16 (round to nearest even) bit for bit, since the two differ only in the store.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_21_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_TOL, L_TOL = 1e-2, 1e-3


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def run(w, x, out_f32):
    q, kc, vc = (dev_bf16(x[n]) for n in ("q", "k_cache", "v_cache"))
    table = torch.from_numpy(x["page_table"]).to(DEV)
    lens = torch.from_numpy(x["seq_lens"]).to(DEV)
    o = torch.full((w.B, w.H, w.Lq, w.d), float("nan"), device=DEV,
                   dtype=torch.float32 if out_f32 else torch.bfloat16)
    lse = torch.full((w.B, w.H, w.Lq), float("nan"), device=DEV)
    print(f"[gpu-decode] {w.name} B={w.B} H={w.H} Lq={w.Lq} d={w.d} page={w.page} "
          f"lens={x['seq_lens'].tolist()[:8]} causal={w.causal} out_f32={out_f32}", flush=True)
    attn.attn_decode(q, kc, vc, table, lens, o, lse, float(x["scale"]), causal=w.causal)
    torch.cuda.synchronize()
    return o, lse


def check(w, x):
    q, kc, vc = (oracle.decode_bf16(x[n]) for n in ("q", "k_cache", "v_cache"))
    o_ref, l_ref = oracle.decode_attention(q, kc, vc, x["page_table"], x["seq_lens"],
                                           float(x["scale"]), w.causal)
    o32, l32 = run(w, x, True)
    o16, l16 = run(w, x, False)
    o32n, l32n = o32.cpu().numpy(), l32.cpu().numpy()
    assert np.all(np.isfinite(o32n)) and np.all(np.isfinite(l32n))
    eo, el = np.abs(o32n - o_ref).max(), np.abs(l32n - l_ref).max()
    print(f"[parity-decode] {w.name}: max|O-O_ref|={eo:.3e} max|L-L_ref|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= L_TOL
    assert torch.equal(o16.cpu(), o32.cpu().to(torch.bfloat16))
    assert torch.equal(l16.cpu(), l32.cpu())


CASES = [
    # name, B, H, Lq, d, page, len_lo, len_hi, causal
    ("dec_len1_d128_p16", 2, 2, 1, 128, 16, 1, 1, True),
    ("dec_short_d128_p16", 4, 3, 1, 128, 16, 1, 40, True),
    ("dec_ragged_d128_p64", 5, 2, 1, 128, 64, 60, 1100, True),
    ("dec_lq4_d64_p32", 3, 2, 4, 64, 32, 4, 300, True),
    ("dec_lq3_none_d64_p32", 3, 2, 3, 64, 32, 3, 500, False),
    ("dec_lq8_d128_p128", 2, 4, 8, 128, 128, 8, 2000, True),
    ("dec_lq2_none_d128_p256", 2, 2, 2, 128, 256, 300, 5000, False),
    ("dec_long_d128_p64", 2, 2, 1, 128, 64, 30000, 40000, True),
    # 64 splits per sequence-head (B*H = 128, 16k table): the single-wave merge at its largest,
    # four chunks of 16 splits, with several query rows and one column per lane (d = 64)
    ("dec_ns64_lq4_d64_p32", 8, 16, 4, 64, 32, 8000, 16384, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_shapes(case):
    name, B, H, Lq, d, page, lo, hi, causal = case
    w = inputs.DecodeWorkload(name, B=B, H=H, Lq=Lq, d=d, page=page, len_lo=lo, len_hi=hi,
                              causal=causal, seed=300 + CASES.index(case))
    check(w, inputs.make_paged_inputs(w))


def test_decode_workload_full():
    """The benchmark's decoding workload at full size, every sequence and head."""
    w = inputs.DECODE_WORKLOADS["decode_b8h32_len2k_14k_d128_p64"]
    check(w, inputs.make_paged_inputs(w))


def test_decode_deterministic():
    w = inputs.DecodeWorkload("det", B=3, H=2, Lq=2, d=128, page=32, len_lo=100, len_hi=3000,
                              seed=399)
    x = inputs.make_paged_inputs(w)
    a, la = run(w, x, True)
    b, lb = run(w, x, True)
    assert torch.equal(a, b) and torch.equal(la, lb)
