"""Pins for the FP8 oracle (oracle/fp8.py): the E4M3 format, its rounding, the block quantizer,
and the attention on dequantized blocks.  The format anchors are those of the E4M3 layout
(1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities; S.1111.111 is NaN)."""
import numpy as np
import pytest

import oracle
from oracle import fp8


def test_e4m3_anchor_values():
    dec = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert dec[0x00] == 0.0 and dec[0x80] == 0.0 and np.signbit(dec[0x80])
    assert dec[0x01] == 2.0 ** -9          # smallest subnormal
    assert dec[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert dec[0x08] == 2.0 ** -6          # smallest normal
    assert dec[0x38] == 1.0
    assert dec[0x39] == 1.125
    assert dec[0x7E] == 448.0              # largest finite
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert np.array_equal(dec[0x80:0xFF], -dec[0x00:0x7F])
    assert np.all(np.diff(dec[0x00:0x7F]) > 0)  # monotonic over the finite positive codes


def test_e4m3_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(fp8.e4m3_encode(vals), codes)


def test_e4m3_round_to_nearest_even():
    pos = fp8.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2  # exact in float32 for this format
    c_mid = fp8.e4m3_encode(mid.astype(np.float32))
    even = np.where(np.arange(0x00, 0x7E) % 2 == 0, np.arange(0x00, 0x7E), np.arange(0x01, 0x7F))
    assert np.array_equal(c_mid, even.astype(np.uint8))
    below = np.nextafter(mid.astype(np.float32), np.float32(0))
    above = np.nextafter(mid.astype(np.float32), np.float32(1e9))
    assert np.array_equal(fp8.e4m3_encode(below), np.arange(0x00, 0x7E, dtype=np.uint8))
    assert np.array_equal(fp8.e4m3_encode(above), np.arange(0x01, 0x7F, dtype=np.uint8))
    # negative values mirror the positive ones
    assert np.array_equal(fp8.e4m3_encode(-mid.astype(np.float32)), even.astype(np.uint8) | 0x80)


def test_e4m3_overflow():
    assert fp8.e4m3_encode(np.float32(464.0)) == 0x7E  # tie between 448 and 480 -> even
    assert fp8.e4m3_encode(np.float32(465.0)) == 0x7F  # rounds past 448 -> NaN code
    assert fp8.e4m3_encode(np.float32(-1e6)) == 0xFF
    assert fp8.e4m3_encode(np.float32(np.nan)) & 0x7F == 0x7F


def test_quantize_blocks_properties():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((2, 3, 100, 16)) * 3).astype(np.float32)
    x[1, 2, 64:] = 0.0  # an all-zero block (rows 64..99 with 32-row blocks: rows 64..95, 96..99)
    codes, scales = fp8.quantize_blocks(x, 32)
    assert scales.shape == (2, 3, 4)
    assert scales[1, 2, 2] == 1.0 and scales[1, 2, 3] == 1.0
    assert not codes[1, 2, 64:].any()
    deq = fp8.dequantize_blocks(codes, scales, 32)
    for b in range(2):
        for h in range(3):
            for t in range(4):
                blk = x[b, h, 32 * t:32 * (t + 1)]
                if not blk.any():
                    continue
                i = np.unravel_index(np.abs(blk).argmax(), blk.shape)
                # the block maximum maps to +-448
                assert codes[b, h, 32 * t + i[0], i[1]] & 0x7F == 0x7E
                # every element within half a grid step of its value (relative 2^-4 for
                # normals, absolute 2^-10 * scale for subnormals), plus float32 division error
                d = np.abs(deq[b, h, 32 * t:32 * (t + 1)] - blk)
                bound = np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * scales[b, h, t])
                assert np.all(d <= bound * (1 + 1e-6))


def test_attention_fp8_exact_on_grid():
    """Values already on the block grid quantize exactly, so the FP8 pass equals the plain
    attention on them."""
    rng = np.random.default_rng(6)
    B, H, N, d = 1, 2, 70, 16

    def on_grid(rows, scale):
        c = rng.integers(0, 0x7E, size=(B, H, N, d), endpoint=True).astype(np.uint8)
        c |= rng.integers(0, 2, size=c.shape).astype(np.uint8) << 7
        x = fp8.e4m3_decode(c)
        for t in range(-(-N // rows)):
            x[:, :, t * rows, 0] = 448.0  # each block's maximum is 448 * its scale
            x[:, :, t * rows:(t + 1) * rows] *= scale * 2.0 ** (t % 3)  # scales differ by block
        return x.astype(np.float32)

    q, k = on_grid(32, 2.0 ** -8), on_grid(16, 2.0 ** -7)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    o1, l1 = fp8.attention_fp8(q, k, v, 0.25, br=32, bc=16, mask="causal")
    o2, l2 = oracle.attention(q.astype(np.float64), k.astype(np.float64), v, 0.25, mask="causal")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
