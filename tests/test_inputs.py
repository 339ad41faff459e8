"""The seeded input generator: determinism, bf16 rounding, document offsets, ALiBi slopes."""
import numpy as np
import torch

from exact_io_aware_21_amd import inputs


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        # exact ties: bf16 value plus half an ulp, both parities
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                  1.5 + 2 ** -8, 0.0, -0.0, 1e-40], dtype=np.float32)])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(inputs.bf16_bits_to_f32(ours),
                          torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_draws_are_deterministic():
    a = inputs.draw_qkv(1, 2, 16, 8, 2.0, 7)
    b = inputs.draw_qkv(1, 2, 16, 8, 2.0, 7)
    c = inputs.draw_qkv(1, 2, 16, 8, 2.0, 8)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], c[0])
    assert a[0].shape == (1, 2, 16, 8) and a[0].dtype == np.uint16
    vals = inputs.bf16_bits_to_f32(inputs.draw_qkv(1, 1, 4096, 64, 2.0, 3)[0])
    assert abs(vals.std() - 2.0) < 0.02


def test_doc_offsets_valid():
    for seed in range(5):
        lens = inputs.draw_doc_lengths(16384, 128, 4096, (seed, 1))
        assert sum(lens) == 16384
        assert all(128 <= n <= 4096 for n in lens[:-1]) and 1 <= lens[-1] <= 4096
    off = inputs.doc_offsets([[3, 5], [1, 1, 6]], 8)
    assert off.tolist() == [[0, 3, 8, 8], [0, 1, 2, 8]]


def test_alibi_slopes():
    s = inputs.alibi_slopes(32)
    assert s.dtype == np.float32
    assert s[0] == np.float32(2 ** -0.25) and s[31] == np.float32(2 ** -8)
    assert np.all(np.diff(s) < 0)


def test_workloads_shapes():
    w = inputs.WORKLOADS
    assert [x.N for x in w.values()] == [256, 2048, 8192, 16384, 16384]
    inp = inputs.make_inputs(w["doc_softcap30_h16_n16384_d64"], with_qkv=False)
    assert inp["doc_offsets"][0, 0] == 0 and inp["doc_offsets"][0, -1] == 16384
    assert inp["scale"] == np.float32(0.125)
