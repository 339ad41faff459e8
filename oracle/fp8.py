"""Plain CPU oracle for the FP8 forward pass: block quantization of Q and K, then attention.

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the tests and the
benchmark's CPU-baseline leg, never by the HIP path, and sharing no code with it.

What is computed.  Page "FlashAttention/es" (marovi.ai), section "Variantes y sucesores": the
third version supports FP8 with a smaller quantization error thanks to per-block scaling; page
"FlashAttention-3 y torch.compile ..." (thecalata.com), section "FlashAttention-3: Asincronía
y Explotación del Silicio Hopper": block normalisation with a scale estimated from the data at
run time.  The pages fix no block size, format or rounding, so the readings are:
  * format: FP8 E4M3 without infinities (the OCP "e4m3fn" layout: 1 sign, 4 exponent bits with
    bias 7, 3 mantissa bits; largest finite 448; subnormals down to 2^-9; S.1111.111 is NaN),
    the FP8 layout the gfx950 matrix cores take;
  * blocks: Q per (batch, head, 256-row query tile) and K per (batch, head, 64-row key tile),
    the tiles of the forward kernel; V is not quantized (P V stays as in the bf16 pass);
  * scale of a block: s = amax / 448 in float32 (s = 1 for an all-zero block), amax the largest
    |x| over the block;
  * code of x: x / s in float32 (correctly rounded), then to E4M3 by round-to-nearest-even; a
    value that would round past 448 becomes NaN (cannot happen here: |x / s| <= 448 up to one
    float32 rounding, which rounds back to 448);
  * the attention is then the definition (attention.py) on the dequantized values code * s
    (exact in float64) for Q and K, and the original V.
"""
from __future__ import annotations

import numpy as np

from .attention import attention

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e4m3_encode(x) -> np.ndarray:
    """float32 values -> E4M3 codes, round to nearest even; past 448 (or NaN) -> NaN code."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    bad = ~np.isfinite(a)
    a = np.where(bad, 0.0, a)
    # grid spacing at a's binade: 2^(e-3) for normals (e >= -6), 2^-9 for subnormals
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.exp2(np.clip(e, -6, 8) - 3)
    q = a / step
    r = np.floor(q)
    half = q - r
    r = np.where((half > 0.5) | ((half == 0.5) & (np.mod(r, 2) == 1)), r + 1, r)
    val = r * step  # the rounded magnitude, exact in float64
    with np.errstate(divide="ignore"):
        ev = np.floor(np.log2(np.where(val > 0, val, 1.0)))
    sub = val < 2.0 ** -6
    code_sub = np.rint(val / 2.0 ** -9)
    code_norm = (ev + 7) * 8 + np.rint((val / np.exp2(ev) - 1.0) * 8)
    code = np.where(sub, code_sub, code_norm).astype(np.int64)
    code = np.where((val > E4M3_MAX) | bad, 0x7F, code)
    return (code | sign).astype(np.uint8)


def quantize_blocks(x, rows):
    """x: float32-representable values [B, H, N, d]; blocks of `rows` rows per (b, h).
    Returns (codes uint8 [B, H, N, d], scales float32 [B, H, ceil(N / rows)])."""
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nb = -(-N // rows)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for t in range(nb):
        blk = x[:, :, t * rows:(t + 1) * rows]
        amax = np.abs(blk).max(axis=(2, 3))
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[:, :, t] = s
        codes[:, :, t * rows:(t + 1) * rows] = e4m3_encode(
            (blk / s[:, :, None, None]).astype(np.float32))
    return codes, scales


def dequantize_blocks(codes, scales, rows):
    """codes [B, H, N, d], scales [B, H, nb] -> float64 values code * scale."""
    v = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), rows, axis=2)[:, :, :v.shape[2]]
    return v * s[..., None]


def attention_fp8(q, k, v, scale, br=256, bc=64, **kw):
    """Reference O, L of the FP8 pass: q, k, v float32-representable [B, H, N, d] (decode bf16
    bits first); Q blocks of br rows and K blocks of bc rows are quantized, V is not."""
    qc, qs = quantize_blocks(q, br)
    kc, ks = quantize_blocks(k, bc)
    return attention(dequantize_blocks(qc, qs, br), dequantize_blocks(kc, ks, bc),
                     np.asarray(v, dtype=np.float64), scale, **kw)
