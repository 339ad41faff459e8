"""GPU parity of runtime-compiled score / mask modifications (attn_mod_create + attn_fwd_mod,
through the C ABI) against the fp64 modification oracle (oracle/mods.py).

Each modification is written twice, as the HIP C++ the library compiles and as the numpy
function the oracle applies.  Tolerances are the forward pass's: max|O - O_ref| <= 1e-2 on the
fp32-output run, max|L - L_ref| <= 1e-3, and the bf16-output run equal to the fp32 run rounded to
bf16.  The mask's block table (classes, counts, lists in the workspace) must equal the oracle's
bit for bit.
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

SCORE = attn.ATTN_MODF_SCORE
MASK = attn.ATTN_MODF_MASK
MAX_FIRST = attn.ATTN_MODF_MAX_FIRST  # ascending key walk, tile maximum first (a hint only)

# name: (flags, HIP source, numpy score_mod, numpy mask_mod, params(H) -> np.float32 array)
MODS = {
    "alibi_causal": (
        SCORE | MASK,
        """__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) {
             return s - p[h] * (float)(i - j); }
           __device__ bool attn_mask_mod(int b, int i, int j, const float *p) { return j <= i; }""",
        lambda s, b, h, i, j, p: s - p[h] * (i - j),
        lambda b, i, j, p: j <= i,
        lambda H: inputs.alibi_slopes(H)),
    "softcap_per_head": (
        SCORE,
        """__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) {
             return p[h] * tanhf(s / p[h]); }""",
        lambda s, b, h, i, j, p: p[h] * np.tanh(s / p[h]),
        None,
        lambda H: np.array([2.0 + 3.0 * h for h in range(H)], dtype=np.float32)),
    "softcap_per_head_max_first": (
        SCORE | MAX_FIRST,
        """__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) {
             return p[h] * tanhf(s / p[h]); }""",
        lambda s, b, h, i, j, p: p[h] * np.tanh(s / p[h]),
        None,
        lambda H: np.array([2.0 + 3.0 * h for h in range(H)], dtype=np.float32)),
    "alibi_causal_max_first": (
        SCORE | MASK | MAX_FIRST,
        """__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) {
             return s - p[h] * (float)(i - j); }
           __device__ bool attn_mask_mod(int b, int i, int j, const float *p) { return j <= i; }""",
        lambda s, b, h, i, j, p: s - p[h] * (i - j),
        lambda b, i, j, p: j <= i,
        lambda H: inputs.alibi_slopes(H)),
    "prefix_lm": (
        MASK,
        """__device__ bool attn_mask_mod(int b, int i, int j, const float *p) {
             return j < (int)p[0] || j <= i; }""",
        None,
        lambda b, i, j, p: (j < int(p[0])) | (j <= i),
        lambda H: np.array([300.0], dtype=np.float32)),
    "relbias_window": (
        SCORE | MASK,
        """__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) {
             const int r = min(i - j, 63);
             return s + p[r < 0 ? 0 : r]; }
           __device__ bool attn_mask_mod(int b, int i, int j, const float *p) {
             return j <= i && i - j < 200; }""",
        lambda s, b, h, i, j, p: s + p[np.clip(i - j, 0, 63)],
        lambda b, i, j, p: (j <= i) & (i - j < 200),
        lambda H: (np.cos(np.arange(64)) * 0.5).astype(np.float32)),
    "causal_odd_heads_by_score": (
        SCORE,
        """__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) {
             return ((h & 1) && j > i) ? -INFINITY : s; }""",
        lambda s, b, h, i, j, p: np.where((h % 2 == 1) & (j > i), -np.inf, s),
        None,
        lambda H: np.zeros(1, dtype=np.float32)),
    "dilated_causal": (
        MASK,
        """__device__ bool attn_mask_mod(int b, int i, int j, const float *p) {
             return j <= i && ((i - j) % 4 == 0 || b == 1); }""",
        None,
        lambda b, i, j, p: (j <= i) & (((i - j) % 4 == 0) | (b == 1)),
        lambda H: np.zeros(1, dtype=np.float32)),
    "alibi_window1024": (
        SCORE | MASK,
        """__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) {
             return s - p[h] * (float)(i - j); }
           __device__ bool attn_mask_mod(int b, int i, int j, const float *p) {
             return j <= i && i - j < 1024; }""",
        lambda s, b, h, i, j, p: s - p[h] * (i - j),
        lambda b, i, j, p: (j <= i) & (i - j < 1024),
        lambda H: inputs.alibi_slopes(H)),
}

_compiled = {}


def compiled(name, d):
    key = (name, d)
    if key not in _compiled:
        flags, src = MODS[name][:2]
        _compiled[key] = attn.AttnMod(src, flags, d)
    return _compiled[key]


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def run(name, w, inp, params, out_f32, workspace=None, cached=False):
    m = compiled(name, w.d)
    o = torch.full((w.B, w.H, w.N, w.d), float("nan"), device=DEV,
                   dtype=torch.float32 if out_f32 else torch.bfloat16)
    lse = torch.full((w.B, w.H, w.N), float("nan"), device=DEV)
    p = torch.from_numpy(params).to(DEV)
    print(f"[gpu-mod] {name} B={w.B} H={w.H} N={w.N} d={w.d} out_f32={out_f32} cached={cached}",
          flush=True)
    m.fwd(dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]), o, lse, inp["scale"], p,
          workspace=workspace, cached_table=cached)
    torch.cuda.synchronize()
    return o, lse


def table_of(ws, w):
    """(cls, cnt, lst, wfull) of the block table in a modification's workspace: after the
    key-transposed V, 256-byte aligned regions cls int8 [B][n_qt][n_kt], cnt int32 [B][n_qt],
    lst int32 [B][n_qt][n_kt], wfull uint8 [B][n_qt][n_kt]."""
    n_qt, n_kt = -(-w.N // BR), -(-w.N // BC)
    al = lambda x: (x + 255) // 256 * 256
    off = al(w.B * w.H * w.d * n_kt * BC * 2)
    rows_t = w.B * n_qt
    raw = ws.cpu().numpy()
    cls = raw[off:off + rows_t * n_kt].view(np.int8).reshape(w.B, n_qt, n_kt)
    off = al(off + rows_t * n_kt)
    cnt = raw[off:off + rows_t * 4].view(np.int32).reshape(w.B, n_qt)
    off = al(off + rows_t * 4)
    lst = raw[off:off + rows_t * n_kt * 4].view(np.int32).reshape(w.B, n_qt, n_kt)
    off = al(off + rows_t * n_kt * 4)
    wfull = raw[off:off + rows_t * n_kt].reshape(w.B, n_qt, n_kt)
    return cls, cnt, lst, wfull


def check(name, w, inp, rows=None, heads=None):
    flags, _, smod, mmod, pfun = MODS[name]
    params = pfun(w.H)
    ws = compiled(name, w.d).alloc_workspace(w.B, w.H, w.N, DEV)
    o32, l32 = run(name, w, inp, params, True, ws)
    if flags & MASK:  # the block table the call left in its workspace
        cls, cnt, lst, wfull = table_of(ws, w)
        n_qt, n_kt = cls.shape[1:]
        c2, n2, l2 = oracle.mod_tile_table(w.N, w.B, mmod, params.astype(np.float64))
        assert np.array_equal(cls, c2) and np.array_equal(cnt, n2) and np.array_equal(lst, l2)
        # bit w of a tile's byte: its rows 32w .. 32w + 31 all in range and allowed (32-row
        # blocks of the same pair-by-pair evaluation)
        c32, _, _ = oracle.mod_tile_table(w.N, w.B, mmod, params.astype(np.float64), Br=32, Bc=BC)
        full = np.zeros((w.B, n_qt * 8, n_kt), dtype=bool)
        full[:, :c32.shape[1]] = c32 == 2
        ref = (full.reshape(w.B, n_qt, 8, n_kt) * (1 << np.arange(8))[None, None, :, None]).sum(axis=2)
        assert np.array_equal(wfull, ref.astype(np.uint8))
    o16, l16 = run(name, w, inp, params, False)
    assert torch.equal(o16.cpu(), o32.cpu().to(torch.bfloat16))
    assert torch.equal(l16.cpu(), l32.cpu())
    q, k, v = (oracle.decode_bf16(inp[n]) for n in ("q", "k", "v"))
    o_ref, l_ref = oracle.attention_mod(q, k, v, float(inp["scale"]), smod, mmod,
                                        params.astype(np.float64), rows=rows, heads=heads)
    sel = np.arange(w.N) if rows is None else np.asarray(rows)
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    o32n, l32n = o32.cpu().numpy(), l32.cpu().numpy()
    eo = el = 0.0
    for b, h in heads:
        ref_l = l_ref[b, h]
        got_l = l32n[b, h, sel]
        assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
        fin = np.isfinite(ref_l)
        assert np.all(np.isfinite(o32n[b, h, sel]))
        eo = max(eo, np.abs(o32n[b, h, sel] - o_ref[b, h]).max())
        if fin.any():
            el = max(el, np.abs(got_l[fin] - ref_l[fin]).max())
    print(f"[parity-mod] {name} {w.name}: max|O-O_ref|={eo:.3e} max|L-L_ref|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_L


CASES = [
    # mod, B, H, N, d, sigma
    ("alibi_causal", 1, 4, 1000, 128, 1.0),
    ("alibi_causal", 2, 2, 333, 64, 1.0),
    ("softcap_per_head", 1, 3, 700, 128, 3.0),
    ("softcap_per_head_max_first", 1, 3, 700, 128, 3.0),
    ("alibi_causal_max_first", 1, 4, 1000, 128, 1.0),
    ("prefix_lm", 2, 2, 900, 128, 1.0),
    ("prefix_lm", 1, 2, 1, 64, 1.0),
    ("relbias_window", 1, 2, 1300, 128, 1.0),
    ("causal_odd_heads_by_score", 1, 4, 500, 64, 1.0),
    ("dilated_causal", 2, 2, 600, 128, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}_n{c[3]}_d{c[4]}" for c in CASES])
def test_mod_shapes(case):
    name, B, H, N, d, sigma = case
    w = inputs.Workload(f"{name}_n{N}", B=B, H=H, N=N, d=d, sigma=sigma,
                        seed=2000 + CASES.index(case))
    check(name, w, inputs.make_inputs(w))


def test_mod_alibi_window_workload_full_size():
    """The sliding-window + ALiBi workload (B=2, H=32, N=8192, d=128, window 1024) written as a
    runtime-compiled modification, on sampled rows of three heads against the oracle and on
    every row against the built-in window + ALiBi variant."""
    name = "alibi_window1024"
    w = inputs.WORKLOADS["window1024_alibi_b2h32_n8192_d128"]
    inp = inputs.make_inputs(w)
    rng = np.random.default_rng(21)
    rows = sorted({0, 1, 255, 256, 1023, 1024, 1025, w.N - 1} | {int(x) for x in rng.integers(0, w.N, 16)})
    check(name, w, inp, rows=rows, heads=[(0, 0), (1, 17), (1, 31)])
    o_mod, l_mod = run(name, w, inp, MODS[name][4](w.H), True)
    o = torch.empty_like(o_mod)
    lse = torch.empty_like(l_mod)
    attn.attn_fwd(dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]), o, lse, inp["scale"],
                  attn.variant_bits("window", alibi=True), window=w.window,
                  alibi_slopes=torch.from_numpy(inp["slopes"]).to(DEV))
    torch.cuda.synchronize()
    # every row, against the built-in variant (each within the tolerance of the oracle, so the
    # two within twice it)
    assert (o - o_mod).abs().max().item() <= 2 * TOL_O
    assert (lse - l_mod).abs().max().item() <= 2 * TOL_L


def test_mod_deterministic():
    w = inputs.Workload("mod_det", B=1, H=2, N=777, d=128, seed=2100)
    inp = inputs.make_inputs(w)
    params = MODS["alibi_causal"][4](w.H)
    a, la = run("alibi_causal", w, inp, params, True)
    b, lb = run("alibi_causal", w, inp, params, True)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_mod_cached_table_reuse():
    """attn_fwd_mod_cached on new inputs with the table an earlier attn_fwd_mod call left in the
    workspace: the same O and L, bit for bit, as a call that builds its own table (and within
    the oracle's tolerance), and the table untouched by the cached call."""
    name = "prefix_lm"
    w = inputs.Workload("mod_cache", B=2, H=2, N=900, d=128, seed=2200)
    params = MODS[name][4](w.H)
    ws = compiled(name, w.d).alloc_workspace(w.B, w.H, w.N, DEV)
    run(name, w, inputs.make_inputs(w), params, True, ws)           # builds the table
    before = [t.copy() for t in table_of(ws, w)]
    w2 = inputs.Workload("mod_cache2", B=2, H=2, N=900, d=128, seed=2201, sigma=2.0)
    inp2 = inputs.make_inputs(w2)
    for out_f32 in (True, False):
        oc, lc = run(name, w2, inp2, params, out_f32, ws, cached=True)
        ob, lb = run(name, w2, inp2, params, out_f32)                # builds its own
        assert torch.equal(oc, ob) and torch.equal(lc, lb)
    # other parameter values: the cached call neither reads nor rewrites the table from them
    run(name, w2, inp2, np.array([0.0], dtype=np.float32), True, ws, cached=True)
    assert all(np.array_equal(a, b) for a, b in zip(before, table_of(ws, w)))
    check(name, w2, inp2)
