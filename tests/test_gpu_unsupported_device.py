"""The capability check on a device that is present (page "FlashAttention-3 y torch.compile ...",
section 6, item 3: check the device's capability instead of crashing).  A child process sets
ATTN_TEST_ARCH_OVERRIDE, so the library sees a GPU that reports another architecture: every
entry point that launches work must return ATTN_ERR_UNSUPPORTED_DEVICE with a message and leave
its outputs untouched, and calls that need no device keep working."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import torch
sys.path.insert(0, sys.argv[1])
from exact_io_aware_21_amd import attn
dev = "cuda:0"
B, H, N, d = 1, 2, 300, 128
q = torch.randn(B, H, N, d, device=dev).to(torch.bfloat16)
o = torch.full((B, H, N, d), float("nan"), device=dev)
lse = torch.full((B, H, N), float("nan"), device=dev)
seen = []

def expect_unsupported(fn, name):
    try:
        fn()
    except attn.AttnError as e:
        assert e.code == attn.ATTN_ERR_UNSUPPORTED_DEVICE, (name, e.code)
        assert "gfx942" in str(e), (name, str(e))
        seen.append(name)
        return
    raise AssertionError(name + " did not fail")

expect_unsupported(lambda: attn.attn_fwd(q, q, q, o, lse, 0.088, attn.ATTN_MASK_CAUSAL), "fwd")
expect_unsupported(lambda: attn.attn_fwd(q, q, q, o, lse, 0.088,
                                         attn.ATTN_MASK_CAUSAL | attn.ATTN_PREC_FP8), "fwd_fp8")
g = torch.zeros(B, H, N, d, device=dev)
expect_unsupported(lambda: attn.attn_bwd(q, q, q, g, lse, q, g.clone(), g.clone(), g.clone(),
                                         0.088, attn.ATTN_MASK_CAUSAL), "bwd")
c8 = torch.zeros(B, H, N, d, dtype=torch.uint8, device=dev)
sc = torch.zeros(B, H, -(-N // 64), device=dev)
expect_unsupported(lambda: attn.attn_quantize_fp8(q, c8, sc, 64), "quantize")
kc = torch.zeros(4, H, 16, d, dtype=torch.bfloat16, device=dev)
pt = torch.zeros(B, 4, dtype=torch.int32, device=dev)
sl = torch.full((B,), 10, dtype=torch.int32, device=dev)
od = torch.full((B, H, 1, d), float("nan"), device=dev)
expect_unsupported(lambda: attn.attn_decode(q[:, :, :1].contiguous(), kc, kc, pt, sl, od, None,
                                            0.088), "decode")
Br, Bc = attn.attn_tile_shape(d, attn.ATTN_MASK_CAUSAL)
cls = torch.zeros(1, -(-N // Br), -(-N // Bc), dtype=torch.int8, device=dev)
cnt = torch.zeros(1, -(-N // Br), dtype=torch.int32, device=dev)
lst = torch.zeros(1, -(-N // Br), -(-N // Bc), dtype=torch.int32, device=dev)
expect_unsupported(lambda: attn.attn_block_table(B, H, N, d, attn.ATTN_MASK_CAUSAL, cls, cnt, lst),
                   "block_table")
m = attn.AttnMod("__device__ bool attn_mask_mod(int b, int i, int j, const float *p)"
                 " { return j <= i; }", attn.ATTN_MODF_MASK, d)
expect_unsupported(lambda: m.fwd(q, q, q, o, lse, 0.088), "fwd_mod")
torch.cuda.synchronize()
assert torch.isnan(o).all() and torch.isnan(lse).all() and torch.isnan(od).all()
# host-only calls are unaffected
assert attn.attn_workspace_size(B, H, N, d, attn.ATTN_MASK_CAUSAL) > 0
attn.attn_block_table_host(B, H, N, d, attn.ATTN_MASK_CAUSAL)
print("OK", " ".join(seen), flush=True)
"""


def test_reported_other_architecture_is_refused():
    env = dict(os.environ, ATTN_TEST_ARCH_OVERRIDE="gfx942")
    print("[gpu] child process with ATTN_TEST_ARCH_OVERRIDE=gfx942", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    assert r.stdout.strip().splitlines()[-1].startswith("OK fwd fwd_fp8 bwd quantize decode")
