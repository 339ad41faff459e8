"""GPU parity of the FP8 forward pass (attn_fwd with ATTN_PREC_FP8, and attn_quantize_fp8)
against the fp64 oracle (oracle/fp8.py), through the C ABI.

* Block quantization is integer work decided in float32 on both sides (amax, a correctly
  rounded x / s, round-to-nearest-even to E4M3), so codes and scales must match bit for bit.
* The forward pass is compared with the attention of the dequantized Q and K blocks (Q blocks
  of Br = 256 rows, K blocks of Bc = 64 rows) and the unquantized V, at the forward pass's
  tolerances: max|O - O_ref| <= 1e-2 on the fp32-output run, max|L - L_ref| <= 1e-3, and the
  bf16-output run equal to the fp32 run rounded to bf16 bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_21_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O, TOL_L = 1e-2, 1e-3
BR, BC = 256, 64


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


# --- block quantization: bit-exact -----------------------------------------------------------
QUANT = [
    # name, B, H, N, d, rows, sigma
    ("q_n1_d64_r64", 1, 1, 1, 64, 64, 1.0),
    ("q_n100_d128_r64", 1, 2, 100, 128, 64, 1.0),
    ("q_n1000_d128_r256", 2, 2, 1000, 128, 256, 3.0),
    ("q_n333_d64_r256", 1, 3, 333, 64, 256, 0.01),
    ("q_n4096_d128_r64", 1, 4, 4096, 128, 64, 1.0),
    ("q_n50_d128_r7", 1, 1, 50, 128, 7, 100.0),
]


def quant_case(case):
    name, B, H, N, d, rows, sigma = case
    rng = np.random.default_rng(700 + QUANT.index(case))
    x = (rng.standard_normal((B, H, N, d)) * sigma).astype(np.float32)
    x[0, 0, :min(N, rows)] = 0.0             # an all-zero block (scale 1, codes 0)
    if N > 3 * rows:
        x[0, -1, 2 * rows + 1, 5] = 1e4      # one block with a far larger maximum
        x[0, -1, 2 * rows + 2, 7] = -0.05    # a value in its E4M3 subnormal range
        x[0, -1, 2 * rows + 3, 9] = -2e-6    # and one that rounds to -0
    return x, inputs.f32_to_bf16_bits(x)


@pytest.mark.parametrize("case", QUANT, ids=[c[0] for c in QUANT])
def test_quantize_bit_exact(case):
    name, B, H, N, d, rows, _ = case
    x, bits = quant_case(case)
    ref_codes, ref_scales = oracle.quantize_blocks(inputs.bf16_bits_to_f32(bits), rows)
    nb = -(-N // rows)
    codes = torch.full((B, H, N, d), 0xAA, dtype=torch.uint8, device=DEV)
    scales = torch.full((B, H, nb), float("nan"), device=DEV)
    print(f"[gpu-fp8] quantize {name} B={B} H={H} N={N} d={d} rows={rows}", flush=True)
    attn.attn_quantize_fp8(dev_bf16(bits), codes, scales, rows)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(s.view(np.uint32), ref_scales.view(np.uint32)), name
    bad = np.argwhere(c != ref_codes)
    assert bad.size == 0, f"{name}: {len(bad)} codes differ, first at {bad[0].tolist()}"


# --- the forward pass ------------------------------------------------------------------------
def run_fp8(w, inp, out_f32):
    B, H, N, d = w.B, w.H, w.N, w.d
    o = torch.full((B, H, N, d), float("nan"), device=DEV,
                   dtype=torch.float32 if out_f32 else torch.bfloat16)
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    offs = None if inp["doc_offsets"] is None else torch.from_numpy(inp["doc_offsets"]).to(DEV)
    var = attn.variant_bits(w.mask, fp8=True)
    print(f"[gpu-fp8] {w.name} B={B} H={H} N={N} d={d} var={var} out_f32={out_f32}", flush=True)
    attn.attn_fwd(dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]), o, lse,
                  inp["scale"], var, window=w.window, doc_offsets=offs)
    torch.cuda.synchronize()
    return o, lse


def oracle_fp8(w, inp, rows=None, heads=None):
    """O, L of the oracle for the given rows of the given (b, h) heads (all when None).
    Quantization is per (b, h), so a head can be evaluated on its own slice."""
    q, k, v = (inputs.bf16_bits_to_f32(inp[n]) for n in ("q", "k", "v"))
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    out = {}
    for b, h in heads:
        offs = None if inp["doc_offsets"] is None else inp["doc_offsets"][b:b + 1]
        o, l = oracle.attention_fp8(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                    v[b:b + 1, h:h + 1], float(inp["scale"]), br=BR, bc=BC,
                                    mask=w.mask, window=w.window, doc_offsets=offs, rows=rows)
        out[(b, h)] = (o[0, 0], l[0, 0])
    return out


def check(w, inp, rows=None, heads=None):
    o32, l32 = run_fp8(w, inp, True)
    o16, l16 = run_fp8(w, inp, False)
    assert torch.equal(o16.cpu(), o32.cpu().to(torch.bfloat16))
    assert torch.equal(l16.cpu(), l32.cpu())
    o32n, l32n = o32.cpu().numpy(), l32.cpu().numpy()
    sel = np.arange(w.N) if rows is None else np.asarray(rows)
    worst = [0.0, 0.0]
    for (b, h), (o_ref, l_ref) in oracle_fp8(w, inp, rows, heads).items():
        assert np.all(np.isfinite(o32n[b, h, sel])) and np.all(np.isfinite(l32n[b, h, sel]))
        eo = np.abs(o32n[b, h, sel] - o_ref).max()
        el = np.abs(l32n[b, h, sel] - l_ref).max()
        assert eo <= TOL_O, f"{w.name} b={b} h={h}: max|O-O_ref|={eo:.3e}"
        assert el <= TOL_L, f"{w.name} b={b} h={h}: max|L-L_ref|={el:.3e}"
        worst = [max(worst[0], eo), max(worst[1], el)]
    print(f"[parity-fp8] {w.name}: max|O-O_ref|={worst[0]:.3e} max|L-L_ref|={worst[1]:.3e}",
          flush=True)


SMALL = [
    # name, B, H, N, d, mask, window, sigma
    ("f8_n1_none_d64", 1, 2, 1, 64, "none", 0, 1.0),
    ("f8_n100_causal_d128", 1, 3, 100, 128, "causal", 0, 1.0),
    ("f8_n255_none_d64", 2, 2, 255, 64, "none", 0, 1.0),
    ("f8_n300_causal_d128_sig2", 1, 2, 300, 128, "causal", 0, 2.0),
    ("f8_n1000_causal_d128", 1, 2, 1000, 128, "causal", 0, 1.0),
    ("f8_n1000_causal_d64_sig3", 1, 1, 1000, 64, "causal", 0, 3.0),
    ("f8_w65_d128", 1, 2, 700, 128, "window", 65, 1.0),
    ("f8_w1_d64", 1, 2, 200, 64, "window", 1, 1.0),
    ("f8_doc_d128", 2, 1, 900, 128, "document", 0, 1.0),
    ("f8_n2048_none_d128_sig01", 1, 1, 2048, 128, "none", 0, 0.1),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fp8_small_shapes(case):
    name, B, H, N, d, mask, window, sigma = case
    kw = {"doc_len_range": (1, 300)} if mask == "document" else {}
    w = inputs.Workload(name, B=B, H=H, N=N, d=d, sigma=sigma, mask=mask, window=window,
                        seed=1500 + SMALL.index(case), **kw)
    check(w, inputs.make_inputs(w))


def test_fp8_workload_full_size():
    """The causal B=1 H=32 N=16384 d=128 workload at full size, sampled rows of three heads."""
    w = inputs.WORKLOADS["causal_h32_n16384_d128"]
    inp = inputs.make_inputs(w)
    rng = np.random.default_rng(15)
    N = w.N
    rows = sorted({0, 1, 63, 64, 255, 256, 257, N // 2, N - 257, N - 256, N - 1}
                  | {int(x) for x in rng.integers(0, N, 20)})
    check(w, inp, rows=rows, heads=[(0, 0), (0, 17), (0, 31)])


def test_fp8_zero_q_and_zero_k_tiles():
    """Q = 0 (scale 1, all codes 0): every score is 0, so O is the mean of the allowed V rows and
    L = ln(count); a K tile of zeros likewise contributes scores of exactly 0."""
    w = inputs.Workload("f8_zero", B=1, H=2, N=500, d=128, mask="causal", seed=1600)
    inp = dict(inputs.make_inputs(w))
    inp["q"] = np.zeros_like(inp["q"])
    o32, l32 = run_fp8(w, inp, True)
    v = inputs.bf16_bits_to_f32(inp["v"]).astype(np.float64)
    n = np.arange(1, w.N + 1)
    mean = np.cumsum(v, axis=2) / n[None, None, :, None]
    assert np.abs(o32.cpu().numpy() - mean).max() <= TOL_O
    assert np.abs(l32.cpu().numpy() - np.log(n)[None, None]).max() <= TOL_L
    inp = dict(inputs.make_inputs(w))
    k = inp["k"].copy()
    k[:, :, 64:128] = 0
    inp["k"] = k
    check(w, inp)


def test_fp8_deterministic():
    w = inputs.Workload("f8_det", B=1, H=2, N=777, d=128, mask="causal", seed=1601)
    inp = inputs.make_inputs(w)
    a, la = run_fp8(w, inp, True)
    b, lb = run_fp8(w, inp, True)
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("scale", [0.0, -0.125, -1.0 / 128 ** 0.5])
def test_fp8_scale_not_positive(scale):
    """scale = 0 and scale < 0 select the FP8 instance that scales every score before its
    maximum is taken."""
    for mask, d in (("causal", 128), ("none", 64)):
        w = inputs.Workload(f"f8_scale{scale:+.3f}_{mask}", B=1, H=2, N=333, d=d, mask=mask,
                            seed=1610, scale=scale)
        check(w, inputs.make_inputs(w))
