"""Head dimension 256 (page "FlashAttention/es", section "Limitaciones": the method's sweet spot
reaches head dimensions of about 256), GPU against the fp64 oracle through the C ABI.

At d = 256 each workgroup forms the scores over all of d and accumulates one half of O (two
workgroups per q-tile), with three LDS buffers in the copy ring; the tolerances are the forward
pass's: max|O32 - O_ref| <= 1e-2, max|L - L_ref| <= 1e-3, bf16 O = RNE(O32) bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_21_amd import attn, inputs
from test_gpu_parity import check, run_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

D256 = [
    # (name, B, H, N, d, mask, window, alibi, softcap, sigma)
    ("d256_n1_none", 1, 2, 1, 256, "none", 0, False, 0.0, 1.0),
    ("d256_n300_none", 2, 2, 300, 256, "none", 0, False, 0.0, 1.0),
    ("d256_n1000_causal", 1, 3, 1000, 256, "causal", 0, False, 0.0, 1.0),
    ("d256_n700_window_alibi", 2, 4, 700, 256, "window", 100, True, 0.0, 1.0),
    ("d256_n900_doc_softcap", 2, 2, 900, 256, "document", 0, False, 30.0, 2.0),
    ("d256_n333_causal_softcap_sig3", 1, 2, 333, 256, "causal", 0, False, 5.0, 3.0),
    ("d256_n2048_causal_place", 2, 8, 2048, 256, "causal", 0, False, 0.0, 1.0),
]


@pytest.mark.parametrize("case", D256, ids=[c[0] for c in D256])
def test_d256_shapes(case):
    name, B, H, N, d, mask, window, alibi, softcap, sigma = case
    extra = {"doc_len_range": (1, 300)} if mask == "document" else {}
    w = inputs.Workload(name, B=B, H=H, N=N, d=d, sigma=sigma, mask=mask, window=window,
                        alibi=alibi, softcap=softcap, seed=3000 + D256.index(case), **extra)
    inp = inputs.make_inputs(w)
    o32, l32 = run_gpu(inp, w, out_f32=True)
    o16, l16 = run_gpu(inp, w, out_f32=False)
    check(w, inp, o32, l32, o16, l16)


def test_d256_scale_negative():
    w = inputs.Workload("d256_scaleneg", B=1, H=2, N=500, d=256, mask="causal", seed=3010,
                        scale=-0.0625)
    inp = inputs.make_inputs(w)
    o32, l32 = run_gpu(inp, w, out_f32=True)
    o16, l16 = run_gpu(inp, w, out_f32=False)
    check(w, inp, o32, l32, o16, l16)


def test_d256_runtime_modification():
    """A runtime-compiled ALiBi score plus prefix-LM mask at d = 256 against the oracle."""
    B, H, N, d = 1, 4, 600, 256
    src = ("__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p)"
           " { return s - p[h] * (float)(i - j); }\n"
           "__device__ bool attn_mask_mod(int b, int i, int j, const float *p)"
           " { return j <= i || j < 64; }\n")
    m = attn.AttnMod(src, attn.ATTN_MODF_SCORE | attn.ATTN_MODF_MASK, d)
    w = inputs.Workload("d256_mod", B=B, H=H, N=N, d=d, seed=3011)
    inp = inputs.make_inputs(w)
    slopes = inputs.alibi_slopes(H)
    t = {x: torch.from_numpy(inp[x].view(np.int16)).view(torch.bfloat16).to(DEV)
         for x in ("q", "k", "v")}
    o = torch.full((B, H, N, d), float("nan"), device=DEV)
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    print("[gpu] d256 runtime modification", flush=True)
    m.fwd(t["q"], t["k"], t["v"], o, lse, inp["scale"], torch.from_numpy(slopes).to(DEV))
    torch.cuda.synchronize()
    q, k, v = (oracle.decode_bf16(inp[x]) for x in ("q", "k", "v"))
    O, L = oracle.attention_mod(
        q, k, v, float(inp["scale"]),
        score_mod=lambda s, b, h, i, j, p: s - float(p[h]) * (i - j),
        mask_mod=lambda b, i, j, p: (j <= i) | (j < 64), params=slopes.astype(np.float64))
    eo = np.abs(o.cpu().numpy() - O).max()
    el = np.abs(lse.cpu().numpy() - L).max()
    print(f"[parity] d256_mod: max|O-Oref|={eo:.3e} max|L-Lref|={el:.3e}", flush=True)
    assert eo <= 1e-2 and el <= 1e-3
    m.close()


def test_d256_noalloc_and_table():
    """The allocation-free entry point at d = 256 equals attn_fwd bit for bit."""
    w = inputs.Workload("d256_noalloc", B=1, H=4, N=1500, d=256, mask="causal", seed=3012)
    inp = inputs.make_inputs(w)
    t = {x: torch.from_numpy(inp[x].view(np.int16)).view(torch.bfloat16).to(DEV)
         for x in ("q", "k", "v")}
    o1 = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty_like(o1)
    l1 = torch.empty((w.B, w.H, w.N), device=DEV)
    l2 = torch.empty_like(l1)
    print("[gpu] d256 noalloc", flush=True)
    attn.attn_fwd(t["q"], t["k"], t["v"], o1, l1, inp["scale"], attn.ATTN_MASK_CAUSAL)
    attn.attn_fwd_noalloc(t["q"], t["k"], t["v"], o2, l2, inp["scale"], attn.ATTN_MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
