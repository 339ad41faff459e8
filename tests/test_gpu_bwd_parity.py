"""GPU parity of the HIP backward pass (attn_bwd, through the C ABI) against the fp64 oracle.

No tolerance is stated for the gradients, so it is derived from the arithmetic: every product of
the backward pass has one operand rounded to bf16 (P and dS; D from an O rounded the same way),
i.e. a relative perturbation of at most u = 2^-8 (bf16 has 8 significant bits; round to nearest)
per product term, so each gradient element is off by at most u times the sum of the absolute
values of its terms (oracle.backward_magnitudes, M).  The test allows 2 u M (a factor for fp32
accumulation, the exp approximation and the forward's own L and O errors) plus 1e-6 of the
largest M, element by element; with bf16 outputs, plus u |ref| for the store.
The forward output and log-sum-exp fed to attn_bwd come from attn_fwd.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_21_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -8
FACTOR = 2.0


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def run_fwd_bwd(inp, w, dout_bits, out_f32, reps=1):
    B, H, N, d = w.B, w.H, w.N, w.d
    dt = torch.float32 if out_f32 else torch.bfloat16
    q, k, v, g = (dev_bf16(x) for x in (inp["q"], inp["k"], inp["v"], dout_bits))
    o = torch.empty((B, H, N, d), device=DEV, dtype=dt)
    lse = torch.empty((B, H, N), device=DEV, dtype=torch.float32)
    slopes = None if inp["slopes"] is None else torch.from_numpy(inp["slopes"]).to(DEV)
    offs = None if inp["doc_offsets"] is None else torch.from_numpy(inp["doc_offsets"]).to(DEV)
    var = attn.variant_bits(w.mask, w.alibi, w.softcap > 0)
    print(f"[gpu-bwd] {w.name} B={B} H={H} N={N} d={d} var={var} out_f32={out_f32}", flush=True)
    attn.attn_fwd(q, k, v, o, lse, inp["scale"], var, window=w.window, softcap=w.softcap,
                  alibi_slopes=slopes, doc_offsets=offs)
    outs = []
    for _ in range(reps):
        dq, dk, dv = (torch.full((B, H, N, d), float("nan"), device=DEV, dtype=dt)
                      for _ in range(3))
        attn.attn_bwd(q, k, v, o, lse, g, dq, dk, dv, inp["scale"], var, window=w.window,
                      softcap=w.softcap, alibi_slopes=slopes, doc_offsets=offs)
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    return outs


def check_bwd(w, inp, dout_bits, grads, out_f32, heads=None):
    qd, kd, vd, gd = (oracle.decode_bf16(x) for x in (inp["q"], inp["k"], inp["v"], dout_bits))
    kw = dict(mask=w.mask, window=w.window, softcap=float(w.softcap), slopes=inp["slopes"],
              doc_offsets=inp["doc_offsets"], heads=heads)
    ref = oracle.attention_backward(qd, kd, vd, gd, float(inp["scale"]), **kw)
    mag = oracle.backward_magnitudes(qd, kd, vd, gd, float(inp["scale"]), **kw)
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    worst = {}
    for name, x, r, m in zip(("dQ", "dK", "dV"), grads, ref, mag):
        x = x.float().cpu().numpy()
        for b, h in heads:
            xb, rb, mb = x[b, h], r[b, h], m[b, h]
            assert np.all(np.isfinite(xb)), f"{w.name} {name} b={b} h={h}: non-finite"
            err = np.abs(xb - rb)
            bound = FACTOR * U * mb + 1e-6 * mb.max() + 1e-30
            if not out_f32:
                bound = bound + U * np.abs(rb)
            ratio = err / (U * mb + 1e-6 * mb.max() + 1e-30)
            assert np.all(err <= bound), (
                f"{w.name} {name} b={b} h={h}: max|err|={err.max():.3e}, "
                f"max err/(u M)={ratio.max():.2f}")
            prev = worst.get(name, (0.0, 0.0, 0.0))
            worst[name] = (max(prev[0], err.max()), max(prev[1], ratio.max()),
                           max(prev[2], np.abs(rb).max()))
    print(f"[parity-bwd] {w.name} out_f32={out_f32}: " + "  ".join(
        f"{n} max|err|={e:.2e} (max|ref|={a:.2e}, max err/(u M)={q:.2f})"
        for n, (e, q, a) in worst.items()), flush=True)


CASES = [
    # (name, B, H, N, d, mask, window, alibi, softcap, sigma)
    ("b_n1_none_d64", 1, 2, 1, 64, "none", 0, False, 0.0, 1.0),
    ("b_n17_none_d128", 1, 2, 17, 128, "none", 0, False, 0.0, 1.0),
    ("b_n100_causal_d64", 1, 2, 100, 64, "causal", 0, False, 0.0, 1.0),
    ("b_n255_causal_d128", 2, 1, 255, 128, "causal", 0, False, 0.0, 1.0),
    ("b_n300_none_d128", 1, 2, 300, 128, "none", 0, False, 0.0, 1.0),
    ("b_n600_causal_d128", 1, 2, 600, 128, "causal", 0, False, 0.0, 1.0),
    ("b_w65_alibi_d128", 1, 2, 300, 128, "window", 65, True, 0.0, 1.0),
    ("b_w1_d64", 1, 2, 200, 64, "window", 1, False, 0.0, 1.0),
    ("b_causal_alibi_d64", 1, 4, 400, 64, "causal", 0, True, 0.0, 1.0),
    ("b_causal_softcap_d128", 1, 2, 333, 128, "causal", 0, False, 5.0, 3.0),
    ("b_none_softcap_alibi_d64", 1, 2, 150, 64, "none", 0, True, 2.0, 2.0),
    ("b_doc_softcap_d64", 2, 2, 500, 64, "document", 0, False, 30.0, 2.0),
    ("b_doc_d128", 2, 1, 400, 128, "document", 0, False, 0.0, 1.0),
    # block placement of both kernels: shares of 2 whole heads walked position-major, and
    # shares that are not whole heads with a tail past the last multiple of 8 blocks
    ("b_place_grp2_causal_d64", 2, 8, 512, 64, "causal", 0, False, 0.0, 1.0),
    ("b_place_tail_causal_d128", 3, 5, 700, 128, "causal", 0, False, 0.0, 1.0),
    # the d = 128 dK/dV kernel walks 32-query steps in whole triples (three LDS stages) and
    # then one or two more: 2 steps (no triple), 3 (one triple, no tail), and up to 5 steps
    # per key block under the causal mask (a triple and two more)
    ("b_n64_none_d128", 1, 2, 64, 128, "none", 0, False, 0.0, 1.0),
    ("b_n96_none_alibi_d128", 1, 2, 96, 128, "none", 0, True, 0.0, 1.0),
    ("b_n160_causal_d128", 2, 2, 160, 128, "causal", 0, False, 0.0, 1.0),
]


def case_inputs(name, B, H, N, d, mask, window, alibi, softcap, sigma, seed):
    extra = {"doc_len_range": (1, 130)} if mask == "document" else {}
    w = inputs.Workload(name, B=B, H=H, N=N, d=d, sigma=sigma, mask=mask, window=window,
                        alibi=alibi, softcap=softcap, seed=seed, **extra)
    inp = inputs.make_inputs(w)
    return w, inp, inputs.draw_dout(B, H, N, d, seed)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_small_shapes(case):
    w, inp, g = case_inputs(*case, seed=2000 + CASES.index(case))
    (grads32,) = run_fwd_bwd(inp, w, g, out_f32=True)
    check_bwd(w, inp, g, grads32, out_f32=True)
    (grads16,) = run_fwd_bwd(inp, w, g, out_f32=False)
    check_bwd(w, inp, g, grads16, out_f32=False)


def test_bwd_deterministic():
    """No atomics: two calls give bit-identical gradients."""
    w, inp, g = case_inputs("b_det", 1, 2, 700, 128, "causal", 0, False, 0.0, 1.0, seed=2100)
    (a, b) = run_fwd_bwd(inp, w, g, out_f32=True, reps=2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_workload_causal_b4h16_n2048_d128():
    """The causal N=2048 workload at full size; two heads compared element by element."""
    w = inputs.WORKLOADS["causal_b4h16_n2048_d128"]
    inp = inputs.make_inputs(w)
    g = inputs.draw_dout(w.B, w.H, w.N, w.d, w.seed)
    (grads,) = run_fwd_bwd(inp, w, g, out_f32=True)
    check_bwd(w, inp, g, grads, out_f32=True, heads=[(0, 0), (3, 15)])
