"""Graph capture of the forward entry points (GPU).  Page "FlashAttention-3 y torch.compile ...",
section 6, item 2: graph-captured execution forbids allocation during the recorded run.  attn_fwd
(with a workspace allocated beforehand) and attn_fwd_noalloc allocate nothing and issue no
memset, so a HIP graph of a call can be replayed.  Each graph is replayed several times, with
new inputs copied in by eager work and a synchronisation between replays, and every replay is
checked bit for bit against an eager call on the same inputs.  FwdPlan's calls are captured
the same way (the plan takes the capturing stream as the current one)."""
import numpy as np
import pytest
import torch

from exact_io_aware_21_amd import attn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


CASES = [
    inputs.Workload("graph_causal", B=2, H=4, N=1000, d=128, mask="causal", seed=2200),
    inputs.Workload("graph_window_alibi", B=1, H=4, N=777, d=64, mask="window", window=100,
                    alibi=True, seed=2201),
    inputs.Workload("graph_doc_softcap", B=2, H=2, N=900, d=64, mask="document", softcap=30.0,
                    sigma=2.0, seed=2202, doc_len_range=(50, 400)),
    # a short sequence: the single-launch kernel
    inputs.Workload("graph_short_causal_alibi", B=1, H=2, N=200, d=128, mask="causal",
                    alibi=True, seed=2203),
]


@pytest.mark.parametrize("how", ["attn_fwd", "attn_fwd_noalloc", "plan"])
@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_graph_replays_match_eager(w, how):
    noalloc = how == "attn_fwd_noalloc"
    var = attn.variant_bits(w.mask, w.alibi, w.softcap > 0)
    sets = [inputs.make_inputs(inputs.Workload(w.name, B=w.B, H=w.H, N=w.N, d=w.d,
                                               sigma=w.sigma, mask=w.mask, window=w.window,
                                               alibi=w.alibi, softcap=w.softcap,
                                               seed=w.seed + 10 * r,
                                               doc_len_range=w.doc_len_range))
            for r in range(3)]
    first = sets[0]
    q, k, v = (dev_bf16(first[x]) for x in ("q", "k", "v"))
    sl = None if first["slopes"] is None else torch.from_numpy(first["slopes"]).to(DEV)
    of = None if first["doc_offsets"] is None else torch.from_numpy(first["doc_offsets"]).to(DEV)
    o = torch.zeros(w.B, w.H, w.N, w.d, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(w.B, w.H, w.N, device=DEV)
    kw = dict(window=w.window, softcap=w.softcap, alibi_slopes=sl, doc_offsets=of)
    ws = None if noalloc else attn.alloc_workspace(w.B, w.H, w.N, w.d, var)
    scale = first["scale"]

    plan = attn.FwdPlan(q, k, v, o, lse, scale, var, workspace=ws, **kw) if how == "plan" \
        else None

    def call(out, l):
        if plan is not None and out is o:
            plan()
        elif noalloc:
            attn.attn_fwd_noalloc(q, k, v, out, l, scale, var, **kw)
        else:
            attn.attn_fwd(q, k, v, out, l, scale, var, workspace=ws, **kw)

    call(o, lse)  # first call outside the capture (resolves the static scratch on the device)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print(f"[gpu] capture {w.name} {how}", flush=True)
    with torch.cuda.graph(g):
        call(o, lse)
    o_ref = torch.empty_like(o)
    l_ref = torch.empty_like(lse)
    for r, inp in enumerate(sets):
        # eager work between replays: new inputs in the captured buffers (document offsets and
        # slopes stay those of the capture, as the graph holds their addresses)
        q.copy_(dev_bf16(inp["q"]))
        k.copy_(dev_bf16(inp["k"]))
        v.copy_(dev_bf16(inp["v"]))
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(o_ref, l_ref)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), (w.name, r)
        assert torch.equal(lse, l_ref), (w.name, r)
