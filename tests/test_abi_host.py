"""CPU-side checks of the C ABI: the library loads, exports every declared symbol, validates its
arguments before any HIP call, and its host-compiled tile predicates reproduce the oracle's
brute-force block table bit for bit.  No compute call reaches a GPU here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from exact_io_aware_21_amd import attn, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = attn.lib()
    names = declared_functions()
    assert set(names) == set(attn.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_strerror_and_tile_shape():
    L = attn.lib()
    assert L.attn_strerror(0) == b"ok"
    for code in (-1, -2, -3, -4):
        assert L.attn_strerror(code) != b"unknown error code"
    assert attn.attn_tile_shape(128, attn.ATTN_MASK_CAUSAL) == (256, 64)
    assert attn.attn_tile_shape(64, attn.ATTN_MASK_DOCUMENT | attn.ATTN_MOD_SOFTCAP) == (256, 64)
    with pytest.raises(attn.AttnError):
        attn.attn_tile_shape(96, 0)
    with pytest.raises(attn.AttnError):
        attn.attn_tile_shape(64, 1 << 7)


def test_workspace_size():
    # V^T (B*H*d*Npad bf16) plus, for masked kinds, the table; each part 256-byte aligned.
    al = lambda x: (x + 255) // 256 * 256
    assert attn.attn_workspace_size(1, 1, 256, 64, 0) == al(1 * 64 * 256 * 2)
    B, H, N, d = 2, 3, 1000, 128
    npad = 16 * 64
    rows = 4  # ceil(1000/256)
    exp = al(B * H * d * npad * 2) + al(rows * 16) + al(rows * 4) + al(rows * 16 * 4)
    assert attn.attn_workspace_size(B, H, N, d, attn.ATTN_MASK_CAUSAL) == exp
    rows_doc = B * rows
    exp_doc = al(B * H * d * npad * 2) + al(rows_doc * 16) + al(rows_doc * 4) + al(rows_doc * 64)
    assert attn.attn_workspace_size(B, H, N, d, attn.ATTN_MASK_DOCUMENT) == exp_doc
    assert attn.attn_workspace_size(1, 1, 0, 64, 0) == 0
    assert attn.attn_workspace_size(1, 1, 16, 80, 0) == 0
    # FP8: plus the E4M3 codes of K (B*H*N*d bytes) and one fp32 scale per 64-key tile
    assert attn.attn_workspace_size(B, H, N, d, attn.ATTN_MASK_CAUSAL | attn.ATTN_PREC_FP8) == \
        exp + al(B * H * N * d) + al(B * H * 16 * 4)
    assert attn.attn_workspace_size(B, H, N, d, attn.ATTN_PREC_FP8 | attn.ATTN_MOD_ALIBI) == 0
    assert attn.attn_tile_shape(128, attn.ATTN_PREC_FP8) == (256, 64)


def _call_fwd(q=16, k=16, v=16, o=16, lse=None, B=1, H=1, N=64, d=64, scale=0.125, variant=0,
              params="default"):
    L = attn.lib()
    p = attn.attn_params()
    p.workspace = 256
    p.workspace_bytes = 1 << 40
    p.window = 4
    p.softcap = 30.0
    p.alibi_slopes = 4096
    p.doc_offsets = 4096
    p.max_docs = 2
    pp = ctypes.byref(p) if params == "default" else params
    return L.attn_fwd(q, k, v, o, lse, B, H, N, d, scale, variant, pp, None)


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, attn.ATTN_ERR_INVALID_ARG),
    ({"o": None}, attn.ATTN_ERR_INVALID_ARG),
    ({"k": 8}, attn.ATTN_ERR_INVALID_ARG),  # misaligned
    ({"lse": 2}, attn.ATTN_ERR_INVALID_ARG),
    ({"N": 0}, attn.ATTN_ERR_INVALID_ARG),
    ({"B": -1}, attn.ATTN_ERR_INVALID_ARG),
    ({"N": (1 << 24) + 1}, attn.ATTN_ERR_INVALID_ARG),
    ({"N": (1 << 23) + 1, "d": 128}, attn.ATTN_ERR_INVALID_ARG),  # 32-bit V^T tile offsets
    ({"N": (1 << 23) + 1, "d": 256}, attn.ATTN_ERR_INVALID_ARG),
    ({"d": 32}, attn.ATTN_ERR_INVALID_ARG),
    ({"scale": float("inf")}, attn.ATTN_ERR_INVALID_ARG),
    ({"scale": float("nan")}, attn.ATTN_ERR_INVALID_ARG),
    ({"variant": 4}, attn.ATTN_ERR_INVALID_ARG),
    ({"variant": 1 << 8}, attn.ATTN_ERR_INVALID_ARG),
    ({"params": None}, attn.ATTN_ERR_INVALID_ARG),
    ({"B": 40000, "H": 40000, "N": 1000}, attn.ATTN_ERR_INVALID_ARG),
    ({"variant": (1 << 6) | (1 << 4)}, attn.ATTN_ERR_INVALID_ARG),  # FP8 with ALiBi
    ({"variant": (1 << 6) | (1 << 5)}, attn.ATTN_ERR_INVALID_ARG),  # FP8 with soft-capping
    ({"variant": 1 << 6, "B": 300, "H": 300}, attn.ATTN_ERR_INVALID_ARG),  # FP8, B*H > 65535
])
def test_fwd_rejects_invalid_arguments(kw, code):
    assert _call_fwd(**kw) == code
    assert attn.lib().attn_last_error() != b""


def test_fwd_rejects_bad_params():
    L = attn.lib()

    def call(variant, **fields):
        p = attn.attn_params()
        p.workspace, p.workspace_bytes = 256, 1 << 40
        p.window, p.softcap, p.alibi_slopes, p.doc_offsets, p.max_docs = 4, 30.0, 4096, 4096, 2
        for f, val in fields.items():
            setattr(p, f, val)
        return L.attn_fwd(16, 16, 16, 16, None, 1, 1, 64, 64, 0.125, variant, ctypes.byref(p), None)

    E, W = attn.ATTN_ERR_INVALID_ARG, attn.ATTN_ERR_WORKSPACE
    assert call(attn.ATTN_MASK_SLIDING_WINDOW, window=0) == E
    assert call(attn.ATTN_MASK_DOCUMENT, doc_offsets=None) == E
    assert call(attn.ATTN_MASK_DOCUMENT, max_docs=0) == E
    assert call(attn.ATTN_MOD_SOFTCAP, softcap=0.0) == E
    assert call(attn.ATTN_MOD_SOFTCAP, softcap=float("inf")) == E
    assert call(attn.ATTN_MOD_ALIBI, alibi_slopes=None) == E
    assert call(0, o_dtype=2) == E
    assert call(0, workspace=None) == W
    assert call(0, workspace=128) == W  # not 256-byte aligned
    assert call(0, workspace_bytes=100) == W


def test_block_table_rejects_invalid_arguments():
    L = attn.lib()
    assert L.attn_block_table(1, 1, 64, 64, 1, None, None, 16, 16, None) == attn.ATTN_ERR_INVALID_ARG
    assert L.attn_block_table(1, 1, 64, 64, 3, None, 16, 16, 16, None) == attn.ATTN_ERR_INVALID_ARG
    assert L.attn_block_table(1, 1, 64, 64, 1, None, 16, 18, 16, None) == attn.ATTN_ERR_INVALID_ARG


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="only meaningful on a host without a GPU")
def test_valid_call_without_gpu_reports_unsupported_device():
    # All arguments valid: validation passes, then the device check fails (no GPU here).
    assert _call_fwd() == attn.ATTN_ERR_UNSUPPORTED_DEVICE


# --- host-compiled closed-form table vs the oracle's brute force ----------------------------
TABLE_CASES = [
    (1, 64, "none", 0), (17, 64, "none", 0), (300, 128, "none", 0),
    (1, 64, "causal", 0), (100, 64, "causal", 0), (255, 128, "causal", 0), (1000, 64, "causal", 0),
    (2048, 128, "causal", 0),
    (1, 64, "window", 1), (200, 64, "window", 1), (300, 64, "window", 63), (300, 64, "window", 64),
    (300, 64, "window", 65), (1000, 128, "window", 128), (1000, 128, "window", 5000),
    (8192, 128, "window", 1024),
]


@pytest.mark.parametrize("N,d,mask,W", TABLE_CASES)
def test_host_table_matches_oracle(N, d, mask, W):
    v = attn.variant_bits(mask)
    Br, Bc = attn.attn_tile_shape(d, v)
    ours = attn.attn_block_table_host(1, 1, N, d, v, window=W)
    ref = oracle.tile_table(N, Br, Bc, mask, W)
    for a, b in zip(ours, ref):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("seed", range(6))
def test_host_table_document_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    B = 3
    N = int(rng.integers(1, 700))
    lens = []
    for b in range(B):
        lo, hi = [(1, 1), (1, 40), (100, 300)][(seed + b) % 3]
        lens.append(inputs.draw_doc_lengths(N, lo, hi, (seed, b)))
    off = inputs.doc_offsets(lens, N)
    v = attn.variant_bits("document")
    Br, Bc = attn.attn_tile_shape(64, v)
    ours = attn.attn_block_table_host(B, 2, N, 64, v, doc_offsets=off)
    ref = oracle.tile_table(N, Br, Bc, "document", 0, off)
    for a, b in zip(ours, ref):
        assert np.array_equal(a, b)


def test_host_table_document_workload():
    w = inputs.WORKLOADS["doc_softcap30_h16_n16384_d64"]
    off = inputs.make_inputs(w, with_qkv=False)["doc_offsets"]
    v = attn.variant_bits("document", softcap=True)
    Br, Bc = attn.attn_tile_shape(w.d, v)
    ours = attn.attn_block_table_host(w.B, w.H, w.N, w.d, v, doc_offsets=off)
    ref = oracle.tile_table(w.N, Br, Bc, "document", 0, off)
    for a, b in zip(ours, ref):
        assert np.array_equal(a, b)


# --- backward entry point ---------------------------------------------------------------------
def test_bwd_workspace_size():
    # D (fp32 B*H*N), then the table for masked kinds.
    al = lambda x: (x + 255) // 256 * 256
    B, H, N, d = 2, 3, 1000, 128
    base = al(B * H * N * 4)
    assert attn.attn_bwd_workspace_size(B, H, N, d, attn.ATTN_MASK_NONE) == base
    rows = 4
    assert attn.attn_bwd_workspace_size(B, H, N, d, attn.ATTN_MASK_CAUSAL) == \
        base + al(rows * 16) + al(rows * 4) + al(rows * 16 * 4)
    assert attn.attn_bwd_workspace_size(1, 1, 16, 80, 0) == 0
    assert attn.attn_bwd_workspace_size(B, H, N, d, attn.ATTN_PREC_FP8) == 0  # forward only


def _call_bwd(ptrs=None, B=1, H=1, N=64, d=64, scale=0.125, variant=0, params="default"):
    L = attn.lib()
    p = attn.attn_params()
    p.workspace = 256
    p.workspace_bytes = 1 << 40
    pp = ctypes.byref(p) if params == "default" else params
    args = {"q": 16, "k": 16, "v": 16, "o": 16, "lse": 16, "dout": 16, "dq": 16, "dk": 16,
            "dv": 16}
    args.update(ptrs or {})
    return L.attn_bwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["dout"],
                      args["dq"], args["dk"], args["dv"], B, H, N, d, scale, variant, pp, None)


@pytest.mark.parametrize("kw,code", [
    ({"ptrs": {"lse": None}}, attn.ATTN_ERR_INVALID_ARG),
    ({"ptrs": {"dout": None}}, attn.ATTN_ERR_INVALID_ARG),
    ({"ptrs": {"dk": 8}}, attn.ATTN_ERR_INVALID_ARG),
    ({"ptrs": {"lse": 2}}, attn.ATTN_ERR_INVALID_ARG),
    ({"N": 0}, attn.ATTN_ERR_INVALID_ARG),
    ({"d": 96}, attn.ATTN_ERR_INVALID_ARG),
    ({"B": 300, "H": 300}, attn.ATTN_ERR_INVALID_ARG),
    ({"scale": float("nan")}, attn.ATTN_ERR_INVALID_ARG),
    ({"params": None}, attn.ATTN_ERR_INVALID_ARG),
    ({"variant": 1 << 6}, attn.ATTN_ERR_INVALID_ARG),  # FP8 is forward only
])
def test_bwd_rejects_invalid_arguments(kw, code):
    assert _call_bwd(**kw) == code
    assert attn.lib().attn_last_error() != b""


def test_bwd_rejects_small_workspace():
    p = attn.attn_params()
    p.workspace, p.workspace_bytes = 256, 100
    assert _call_bwd(params=ctypes.byref(p)) == attn.ATTN_ERR_WORKSPACE


@pytest.mark.skipif(_gpu_present(), reason="only meaningful on a host without a GPU")
def test_bwd_valid_call_without_gpu_reports_unsupported_device():
    assert _call_bwd() == attn.ATTN_ERR_UNSUPPORTED_DEVICE


# --- paged decoding entry point ---------------------------------------------------------------
def test_decode_workspace_size():
    # fp32 partials [B*H][n_split][Lq padded to 1/2/4/8] x d, then m and l; about 8192
    # workgroups over all (sequence, head) pairs, no split shorter than 256 positions.
    al = lambda x: (x + 255) // 256 * 256
    for (B, H, Lq, d, page, max_pages) in [(16, 32, 1, 128, 64, 256), (1, 1, 3, 64, 32, 4),
                                           (2, 8, 8, 128, 16, 1000)]:
        rows = 256 // (d // 8)
        max_len = max_pages * page
        ns = min(-(-8192 // (B * H)), -(-max_len // 256))
        kps = -(-(-(-max_len // ns)) // rows) * rows
        nsplit = -(-max_len // kps)
        lqp = 1 if Lq <= 1 else 2 if Lq <= 2 else 4 if Lq <= 4 else 8
        parts = B * H * nsplit * lqp
        want = al(parts * d * 4) + 2 * al(parts * 4)
        assert attn.attn_decode_workspace_size(B, H, Lq, d, page, max_pages) == want


@pytest.mark.parametrize("args", [
    (0, 1, 1, 128, 64, 4), (1, 1, 0, 128, 64, 4), (1, 1, 9, 128, 64, 4), (1, 1, 1, 96, 64, 4),
    (1, 1, 1, 128, 8, 4), (1, 1, 1, 64, 16, 4), (1, 1, 1, 128, 48, 4), (1, 1, 1, 128, 8192, 4),
    (1, 1, 1, 128, 64, 0), (300, 300, 1, 128, 64, 4), (1, 1, 1, 128, 4096, 1 << 13),
])
def test_decode_workspace_size_rejects(args):
    assert attn.attn_decode_workspace_size(*args) == 0


def _call_decode(ptrs=None, B=1, H=1, Lq=1, d=128, page=64, max_pages=4, n_pages=4, scale=0.1,
                 variant=1, params="default"):
    L = attn.lib()
    p = attn.attn_params()
    p.workspace = 256
    p.workspace_bytes = 1 << 40
    pp = ctypes.byref(p) if params == "default" else params
    args = {"q": 16, "k": 16, "v": 16, "table": 16, "lens": 16, "o": 16, "lse": 16}
    args.update(ptrs or {})
    return L.attn_decode(args["q"], args["k"], args["v"], args["table"], args["lens"], args["o"],
                         args["lse"], B, H, Lq, d, page, max_pages, n_pages, scale, variant, pp,
                         None)


@pytest.mark.parametrize("kw,code", [
    ({"ptrs": {"q": None}}, attn.ATTN_ERR_INVALID_ARG),
    ({"ptrs": {"table": None}}, attn.ATTN_ERR_INVALID_ARG),
    ({"ptrs": {"lens": None}}, attn.ATTN_ERR_INVALID_ARG),
    ({"ptrs": {"k": 8}}, attn.ATTN_ERR_INVALID_ARG),
    ({"ptrs": {"table": 2}}, attn.ATTN_ERR_INVALID_ARG),
    ({"ptrs": {"lse": 6}}, attn.ATTN_ERR_INVALID_ARG),
    ({"Lq": 9}, attn.ATTN_ERR_INVALID_ARG),
    ({"page": 24}, attn.ATTN_ERR_INVALID_ARG),
    ({"n_pages": 0}, attn.ATTN_ERR_INVALID_ARG),
    ({"variant": attn.ATTN_MASK_SLIDING_WINDOW}, attn.ATTN_ERR_INVALID_ARG),
    ({"variant": attn.ATTN_MASK_CAUSAL | attn.ATTN_MOD_ALIBI}, attn.ATTN_ERR_INVALID_ARG),
    ({"scale": float("inf")}, attn.ATTN_ERR_INVALID_ARG),
    ({"params": None}, attn.ATTN_ERR_INVALID_ARG),
])
def test_decode_rejects_invalid_arguments(kw, code):
    assert _call_decode(**kw) == code
    assert attn.lib().attn_last_error() != b""


def test_decode_rejects_small_workspace():
    p = attn.attn_params()
    p.workspace, p.workspace_bytes = 256, 100
    assert _call_decode(params=ctypes.byref(p)) == attn.ATTN_ERR_WORKSPACE
    p.workspace, p.workspace_bytes = 16, 1 << 40
    assert _call_decode(params=ctypes.byref(p)) == attn.ATTN_ERR_WORKSPACE


@pytest.mark.skipif(_gpu_present(), reason="only meaningful on a host without a GPU")
def test_decode_valid_call_without_gpu_reports_unsupported_device():
    assert _call_decode() == attn.ATTN_ERR_UNSUPPORTED_DEVICE
    assert _call_decode(variant=attn.ATTN_MASK_NONE, ptrs={"lse": None}) == \
        attn.ATTN_ERR_UNSUPPORTED_DEVICE


# --- FP8 block quantization entry point -------------------------------------------------------
@pytest.mark.parametrize("args,code", [
    ((16, 16, 16, 1, 1, 64, 128, 256), attn.ATTN_ERR_UNSUPPORTED_DEVICE),
    ((None, 16, 16, 1, 1, 64, 128, 256), attn.ATTN_ERR_INVALID_ARG),
    ((8, 16, 16, 1, 1, 64, 128, 256), attn.ATTN_ERR_INVALID_ARG),
    ((16, 16, 2, 1, 1, 64, 128, 256), attn.ATTN_ERR_INVALID_ARG),
    ((16, 16, 16, 1, 1, 0, 128, 256), attn.ATTN_ERR_INVALID_ARG),
    ((16, 16, 16, 1, 1, 64, 96, 256), attn.ATTN_ERR_INVALID_ARG),
    ((16, 16, 16, 1, 1, 64, 128, 0), attn.ATTN_ERR_INVALID_ARG),
    ((16, 16, 16, 1, 1, 64, 128, 5000), attn.ATTN_ERR_INVALID_ARG),
])
def test_quantize_fp8_argument_checks(args, code):
    if code == attn.ATTN_ERR_UNSUPPORTED_DEVICE and _gpu_present():
        pytest.skip("only meaningful on a host without a GPU")
    assert attn.lib().attn_quantize_fp8(*args, None) == code


# --- runtime-compiled modifications -----------------------------------------------------------
MOD_SRC = """__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) {
  return s - p[h] * (float)(i - j); }
__device__ bool attn_mask_mod(int b, int i, int j, const float *p) { return j <= i; }"""


@pytest.fixture(scope="module")
def alibi_causal_mod():
    m = attn.AttnMod(MOD_SRC, attn.ATTN_MODF_SCORE | attn.ATTN_MODF_MASK, 128)
    yield m
    m.close()


def test_mod_compiles_without_gpu_and_sizes_its_workspace(alibi_causal_mod):
    m = alibi_causal_mod
    al = lambda x: (x + 255) // 256 * 256
    B, H, N, d = 2, 3, 1000, 128
    n_qt, n_kt = 4, 16
    rows = B * n_qt
    assert m.workspace_size(B, H, N) == al(B * H * d * n_kt * 64 * 2) + al(rows * n_kt) + \
        al(rows * 4) + al(rows * n_kt * 4) + al(rows * n_kt)
    assert m.workspace_size(1, 1, 0) == 0
    assert m.workspace_size(300, 1, 1 << 16) == 0  # B * ceil(N/Br) > 65535 with a mask
    score_only = attn.AttnMod(MOD_SRC.split("__device__ bool")[0], attn.ATTN_MODF_SCORE, 64)
    assert score_only.workspace_size(B, H, N) == al(B * H * 64 * n_kt * 64 * 2)
    score_only.close()
    # the max-first hint compiles the same functions, with the same workspace
    hinted = attn.AttnMod(MOD_SRC, attn.ATTN_MODF_SCORE | attn.ATTN_MODF_MASK |
                          attn.ATTN_MODF_MAX_FIRST, 128)
    assert hinted.workspace_size(B, H, N) == m.workspace_size(B, H, N)
    hinted.close()


@pytest.mark.parametrize("src,flags,d", [
    (MOD_SRC, 0, 128), (MOD_SRC, 4, 128), (MOD_SRC, 8 | 3, 128), (MOD_SRC, 3, 96), (None, 3, 128)])
def test_mod_create_rejects_invalid_arguments(src, flags, d):
    h = ctypes.c_void_p()
    rc = attn.lib().attn_mod_create(None if src is None else src.encode(), flags, d,
                                    ctypes.byref(h), None, 0)
    assert rc == attn.ATTN_ERR_INVALID_ARG and not h.value


@pytest.mark.parametrize("src,flags", [
    ("__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) { return s + ; }", 1),
    # the declared signature is not defined: the link step fails
    ("__device__ float attn_score_mod(float s) { return s; }", 1),
    ("__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p) { return s; }", 2),
])
def test_mod_compile_errors_are_reported(src, flags):
    with pytest.raises(attn.AttnError) as e:
        attn.AttnMod(src, flags, 64)
    assert e.value.code == attn.ATTN_ERR_COMPILE and "error" in str(e.value)


def _call_fwd_mod(m, q=16, k=16, v=16, o=16, lse=None, B=1, H=1, N=64, scale=0.125, mp=None,
                  params="default", cached=False):
    p = attn.attn_params()
    p.workspace = 256
    p.workspace_bytes = 1 << 40
    pp = ctypes.byref(p) if params == "default" else params
    fn = attn.lib().attn_fwd_mod_cached if cached else attn.lib().attn_fwd_mod
    return fn(m, q, k, v, o, lse, B, H, N, scale, mp, pp, None)


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, attn.ATTN_ERR_INVALID_ARG),
    ({"k": 8}, attn.ATTN_ERR_INVALID_ARG),
    ({"lse": 2}, attn.ATTN_ERR_INVALID_ARG),
    ({"mp": 2}, attn.ATTN_ERR_INVALID_ARG),
    ({"N": 0}, attn.ATTN_ERR_INVALID_ARG),
    ({"scale": float("inf")}, attn.ATTN_ERR_INVALID_ARG),
    ({"params": None}, attn.ATTN_ERR_INVALID_ARG),
    ({"B": 300, "N": 1 << 16}, attn.ATTN_ERR_INVALID_ARG),
])
@pytest.mark.parametrize("cached", [False, True], ids=["build", "cached"])
def test_fwd_mod_rejects_invalid_arguments(alibi_causal_mod, kw, code, cached):
    assert _call_fwd_mod(alibi_causal_mod._h, cached=cached, **kw) == code
    assert attn.lib().attn_last_error() != b""


@pytest.mark.parametrize("cached", [False, True], ids=["build", "cached"])
def test_fwd_mod_rejects_null_mod_and_small_workspace(alibi_causal_mod, cached):
    assert _call_fwd_mod(None, cached=cached) == attn.ATTN_ERR_INVALID_ARG
    p = attn.attn_params()
    p.workspace, p.workspace_bytes = 256, 100
    assert _call_fwd_mod(alibi_causal_mod._h, params=ctypes.byref(p),
                         cached=cached) == attn.ATTN_ERR_WORKSPACE


@pytest.mark.skipif(_gpu_present(), reason="only meaningful on a host without a GPU")
@pytest.mark.parametrize("cached", [False, True], ids=["build", "cached"])
def test_fwd_mod_valid_call_without_gpu_reports_unsupported_device(alibi_causal_mod, cached):
    assert _call_fwd_mod(alibi_causal_mod._h, cached=cached) == attn.ATTN_ERR_UNSUPPORTED_DEVICE


def test_fwd_mod_cached_binding_needs_a_workspace(alibi_causal_mod):
    import torch
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        alibi_causal_mod.fwd(x, x, x, x.clone(), None, 0.125, cached_table=True)


def test_fwd_noalloc_validates_before_any_hip_call():
    """attn_fwd_noalloc refuses, with no HIP call, a shape whose workspace exceeds the static
    scratch (ATTN_ERR_WORKSPACE) and the argument errors attn_fwd refuses."""
    L = attn.lib()
    p = attn.attn_params()
    big = (1, 32, 16384, 128)  # V^T alone is 128 MiB
    assert attn.attn_workspace_size(*big, attn.ATTN_MASK_CAUSAL) > attn.ATTN_NOALLOC_SCRATCH_BYTES
    rc = L.attn_fwd_noalloc(16, 16, 16, 16, None, *big, 0.1, attn.ATTN_MASK_CAUSAL,
                            ctypes.byref(p), None)
    assert rc == attn.ATTN_ERR_WORKSPACE
    assert b"static scratch" in L.attn_last_error()
    assert L.attn_fwd_noalloc(16, 16, 16, 16, None, 1, 1, 256, 64, 0.1, 0, None, None) == \
        attn.ATTN_ERR_INVALID_ARG
    assert L.attn_fwd_noalloc(16, 16, 16, 16, None, 1, 1, 256, 96, 0.1, 0, ctypes.byref(p),
                              None) == attn.ATTN_ERR_INVALID_ARG
    assert L.attn_fwd_noalloc(0, 16, 16, 16, None, 1, 1, 256, 64, 0.1, 0, ctypes.byref(p),
                              None) == attn.ATTN_ERR_INVALID_ARG


def test_head_dim_256_contract():
    """d = 256 is accepted by the forward pass, its tables and runtime-compiled modifications on
    the same 256 x 64 tiles; the backward pass and the FP8 variant refuse it."""
    assert attn.attn_tile_shape(256, attn.ATTN_MASK_CAUSAL) == (256, 64)
    with pytest.raises(attn.AttnError):
        attn.attn_tile_shape(256, attn.ATTN_PREC_FP8)
    al = lambda x: (x + 255) // 256 * 256
    assert attn.attn_workspace_size(1, 2, 300, 256, 0) == al(2 * 256 * 320 * 2)
    assert attn.attn_workspace_size(1, 2, 300, 256, attn.ATTN_PREC_FP8) == 0
    assert attn.attn_bwd_workspace_size(1, 2, 300, 256, 0) == 0
    L = attn.lib()
    p = attn.attn_params()
    p.workspace, p.workspace_bytes = 4096, 1 << 30
    z = [16] * 9
    assert L.attn_bwd(*z, 1, 1, 64, 256, 0.1, 0, ctypes.byref(p), None) == \
        attn.ATTN_ERR_INVALID_ARG
    assert L.attn_fwd(16, 16, 16, 16, None, 1, 1, 64, 256, 0.1, attn.ATTN_PREC_FP8,
                      ctypes.byref(p), None) == attn.ATTN_ERR_INVALID_ARG
    # the host block table is defined on the same tiles for d = 256
    ref = oracle.tile_table(1000, 256, 64, "causal")
    got = attn.attn_block_table_host(1, 1, 1000, 256, attn.ATTN_MASK_CAUSAL)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


def test_mod_compiles_for_head_dim_256():
    m = attn.AttnMod("__device__ bool attn_mask_mod(int b, int i, int j, const float *p)"
                     " { return j <= i; }", attn.ATTN_MODF_MASK, 256)
    assert m.workspace_size(1, 2, 300) > 0
    m.close()
