"""attn_fwd_noalloc (GPU, through the C ABI): the forward pass with the library's static scratch
as its workspace, for callers that cannot allocate.  It must give exactly attn_fwd's results
(the same kernels on the same inputs: O and L bit for bit), on two calls in a row whose second
input is smaller (the scratch keeps the first call's contents), allocate no device memory, and
refuse shapes that do not fit the scratch before launching anything."""
import numpy as np
import pytest
import torch

from exact_io_aware_21_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def warm():
    """One tiny call: the first call on a device resolves the scratch array's address, and the
    runtime may load the code object that holds it then (a one-time set-up, not per call)."""
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    attn.attn_fwd_noalloc(q, q, q, o, None, 0.125, attn.ATTN_MASK_NONE)
    torch.cuda.synchronize()


def both(w, out_f32):
    inp = inputs.make_inputs(w)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    dt = torch.float32 if out_f32 else torch.bfloat16
    sl = None if inp["slopes"] is None else torch.from_numpy(inp["slopes"]).to(DEV)
    of = None if inp["doc_offsets"] is None else torch.from_numpy(inp["doc_offsets"]).to(DEV)
    var = attn.variant_bits(w.mask, w.alibi, w.softcap > 0)
    kw = dict(window=w.window, softcap=w.softcap, alibi_slopes=sl, doc_offsets=of)
    o_ref = torch.full((w.B, w.H, w.N, w.d), float("nan"), dtype=dt, device=DEV)
    l_ref = torch.full((w.B, w.H, w.N), float("nan"), device=DEV)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    warm()
    print(f"[gpu] {w.name} B={w.B} H={w.H} N={w.N} d={w.d} var={var} out_f32={out_f32}",
          flush=True)
    attn.attn_fwd(q, k, v, o_ref, l_ref, inp["scale"], var, **kw)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    attn.attn_fwd_noalloc(q, k, v, o, lse, inp["scale"], var, **kw)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return o, lse, o_ref, l_ref, free0, free1


def test_noalloc_equals_attn_fwd_on_two_calls_second_smaller():
    first = inputs.Workload("noalloc_big", B=2, H=8, N=3000, d=128, mask="causal", seed=2100)
    second = inputs.Workload("noalloc_small", B=1, H=3, N=777, d=64, mask="window", window=130,
                             alibi=True, seed=2101)
    for w in (first, second):
        o, lse, o_ref, l_ref, free0, free1 = both(w, out_f32=False)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), w.name
        assert torch.equal(lse, l_ref), w.name
        assert free0 == free1, f"{w.name}: device memory changed by {free0 - free1} bytes"


@pytest.mark.parametrize("case", [
    ("noalloc_doc_softcap", dict(B=2, H=2, N=1500, d=64, mask="document", softcap=30.0,
                                 sigma=2.0, doc_len_range=(50, 700))),
    ("noalloc_none_f32", dict(B=1, H=2, N=257, d=128, mask="none")),
])
def test_noalloc_variants_fp32_out(case):
    name, kw = case
    w = inputs.Workload(name, seed=2102, **kw)
    o, lse, o_ref, l_ref, free0, free1 = both(w, out_f32=True)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), name
    assert free0 == free1


def test_noalloc_refuses_shapes_beyond_the_scratch():
    B, H, N, d = 1, 32, 16384, 128
    assert attn.attn_workspace_size(B, H, N, d, attn.ATTN_MASK_CAUSAL) > \
        attn.ATTN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=DEV)
    o = torch.full_like(q, float("nan"))
    with pytest.raises(attn.AttnError) as e:
        attn.attn_fwd_noalloc(q, q, q, o, None, 0.088, attn.ATTN_MASK_CAUSAL)
    assert e.value.code == attn.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all()
