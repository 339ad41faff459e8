"""Race detection for the forward kernel's copy ring (GPU).

The forward kernel stages K and V^T tiles with buffer-to-LDS copies into a ring of four LDS
buffers, two iterations ahead, waited with hand-counted vmcnt values before bare barriers.  A
miscounted wait, or a copy landing in a buffer another wave still reads, would perturb the
output by far less than the parity tolerances.  So the race-check build of the library
(libattn_racecheck.so: LDS tiles poisoned with NaN before the first copy, every ring wait
draining all memory operations, full barriers) runs the five workloads in a child process, and
its O and L must equal the production build's bit for bit.  Page "FlashAttention/es", section
"Limitaciones": the result is exact up to the order of the reductions, which both builds share.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from exact_io_aware_21_amd import attn, inputs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RACE_LIB = os.path.join(ROOT, "exact_io_aware_21_amd", "libattn_racecheck.so")

CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from exact_io_aware_21_amd import attn, inputs
out = sys.argv[2]
for name in inputs.WORKLOAD_ORDER:
    w = inputs.WORKLOADS[name]
    inp = inputs.make_inputs(w)
    dev = "cuda:0"
    t = {x: torch.from_numpy(inp[x].view(np.int16)).view(torch.bfloat16).to(dev)
         for x in ("q", "k", "v")}
    o = torch.full((w.B, w.H, w.N, w.d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((w.B, w.H, w.N), float("nan"), device=dev)
    sl = None if inp["slopes"] is None else torch.from_numpy(inp["slopes"]).to(dev)
    of = None if inp["doc_offsets"] is None else torch.from_numpy(inp["doc_offsets"]).to(dev)
    print("[race-check child]", name, flush=True)
    attn.attn_fwd(t["q"], t["k"], t["v"], o, lse, inp["scale"],
                  attn.variant_bits(w.mask, w.alibi, w.softcap > 0), window=w.window,
                  softcap=w.softcap, alibi_slopes=sl, doc_offsets=of)
    torch.cuda.synchronize()
    np.save(f"{out}/{name}_o.npy", o.view(torch.int16).cpu().numpy())
    np.save(f"{out}/{name}_l.npy", lse.cpu().numpy())
print("done", attn.LIB_PATH, flush=True)
"""


def test_race_check_build_equals_pipelined_build(tmp_path):
    if not os.path.exists(RACE_LIB):
        pytest.fail(f"{RACE_LIB} is not built (make -C exact_io_aware_21_amd/csrc)")
    env = dict(os.environ, ATTN_LIB_PATH=RACE_LIB)
    print("[gpu] race-check build in a child process", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", CHILD, ROOT, str(tmp_path)], env=env,
                       capture_output=True, text=True, timeout=600)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0 and "libattn_racecheck.so" in r.stdout
    for name in inputs.WORKLOAD_ORDER:
        w = inputs.WORKLOADS[name]
        inp = inputs.make_inputs(w)
        dev = "cuda:0"
        t = {x: torch.from_numpy(inp[x].view(np.int16)).view(torch.bfloat16).to(dev)
             for x in ("q", "k", "v")}
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H, w.N), device=dev)
        sl = None if inp["slopes"] is None else torch.from_numpy(inp["slopes"]).to(dev)
        of = None if inp["doc_offsets"] is None else torch.from_numpy(inp["doc_offsets"]).to(dev)
        print(f"[gpu] pipelined build {name}", flush=True)
        attn.attn_fwd(t["q"], t["k"], t["v"], o, lse, inp["scale"],
                      attn.variant_bits(w.mask, w.alibi, w.softcap > 0), window=w.window,
                      softcap=w.softcap, alibi_slopes=sl, doc_offsets=of)
        torch.cuda.synchronize()
        ro = np.load(tmp_path / f"{name}_o.npy")
        rl = np.load(tmp_path / f"{name}_l.npy")
        assert not np.isnan(rl).any(), f"{name}: NaN in the race-check build's L"
        go = o.view(torch.int16).cpu().numpy()
        diff = np.count_nonzero(go != ro)
        assert diff == 0, f"{name}: {diff} O elements differ between the builds"
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), rl.view(np.uint32)), name
        print(f"[race-check] {name}: O and L bit-identical", flush=True)
