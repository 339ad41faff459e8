"""The Python binding's own guards (CPU): the C ABI receives raw addresses and cannot tell host
memory, another GPU's memory or a mistyped array from valid input, so the binding must reject
them with ValueError before it calls into the library at all."""
import pytest
import torch

from exact_io_aware_21_amd import attn


@pytest.fixture
def no_library(monkeypatch):
    """Any call into the library (or its loader) fails the test."""
    def boom(*a, **k):
        raise AssertionError("the library was called")
    monkeypatch.setattr(attn, "lib", boom)
    monkeypatch.setattr(attn, "alloc_workspace", boom)
    monkeypatch.setattr(attn, "alloc_bwd_workspace", boom)
    monkeypatch.setattr(attn, "alloc_decode_workspace", boom)


def bf16(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_host_tensors_rejected(no_library):
    q = bf16(1, 2, 64, 64)
    o = torch.zeros(1, 2, 64, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_fwd(q, q, q, o, None, 0.125, attn.ATTN_MASK_CAUSAL)
    lse = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_bwd(q, q, q, o, lse, q, o, o, o, 0.125, attn.ATTN_MASK_CAUSAL)
    x8 = torch.zeros(1, 2, 64, 64, dtype=torch.uint8)
    sc = torch.zeros(1, 2, 1)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_quantize_fp8(q, x8, sc, 64)
    qd = bf16(1, 2, 1, 64)
    kc = bf16(4, 2, 32, 64)
    pt = torch.zeros(1, 4, dtype=torch.int32)
    sl = torch.zeros(1, dtype=torch.int32)
    od = torch.zeros(1, 2, 1, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_decode(qd, kc, kc, pt, sl, od, None, 0.125)


@pytest.fixture
def host_as_device(monkeypatch, no_library):
    """Treats host tensors as if they were on the GPU, to reach the dtype and shape checks that
    follow the device check."""
    monkeypatch.setattr(attn, "_on_device", lambda dev, **t: None)


@pytest.mark.parametrize("bad", ["f64_slopes", "short_slopes", "strided_slopes", "missing_slopes"])
def test_alibi_slopes_checked(host_as_device, bad):
    B, H, N, d = 1, 4, 64, 64
    q, o = bf16(B, H, N, d), bf16(B, H, N, d)
    slopes = {"f64_slopes": torch.zeros(H, dtype=torch.float64),
              "short_slopes": torch.zeros(H - 1),
              "strided_slopes": torch.zeros(2 * H)[::2],
              "missing_slopes": None}[bad]
    with pytest.raises(ValueError, match="alibi_slopes"):
        attn.attn_fwd(q, q, q, o, None, 0.125, attn.ATTN_MASK_CAUSAL | attn.ATTN_MOD_ALIBI,
                      alibi_slopes=slopes)


@pytest.mark.parametrize("bad", ["int64", "one_dim_batch2", "wrong_batch", "missing"])
def test_doc_offsets_checked(host_as_device, bad):
    B, H, N, d = 2, 1, 64, 64
    q, o = bf16(B, H, N, d), bf16(B, H, N, d)
    offs = {"int64": torch.tensor([[0, 32, 64], [0, 10, 64]], dtype=torch.int64),
            "one_dim_batch2": torch.tensor([0, 32, 64], dtype=torch.int32),
            "wrong_batch": torch.tensor([[0, 32, 64]], dtype=torch.int32),
            "missing": None}[bad]
    with pytest.raises(ValueError, match="doc_offsets"):
        attn.attn_fwd(q, q, q, o, None, 0.125, attn.ATTN_MASK_DOCUMENT, doc_offsets=offs)
    lse = torch.zeros(B, H, N)
    with pytest.raises(ValueError, match="doc_offsets"):
        attn.attn_bwd(q, q, q, o, lse, q, o, o, o, 0.125, attn.ATTN_MASK_DOCUMENT,
                      doc_offsets=offs)


def test_valid_arguments_reach_the_library(host_as_device):
    """The guards accept well-formed input: the call gets as far as the library (stubbed)."""
    B, H, N, d = 2, 4, 64, 64
    q, o = bf16(B, H, N, d), bf16(B, H, N, d)
    with pytest.raises(AssertionError, match="library was called"):
        attn.attn_fwd(q, q, q, o, None, 0.125,
                      attn.ATTN_MASK_DOCUMENT | attn.ATTN_MOD_ALIBI,
                      alibi_slopes=torch.zeros(H),
                      doc_offsets=torch.tensor([[0, 32, 64], [0, 10, 64]], dtype=torch.int32))
