"""Seeded synthetic inputs for the attention forward pass.

This module draws Q, K, V, document lengths and ALiBi slopes.  It holds none of the
attention arithmetic: both the HIP path (through the tests and the benchmark) and the CPU
oracle receive what it returns, so the two sides see exactly the same input values.

Recipe (numpy PCG64):
  * ``default_rng(seed)`` draws Q, then K, then V, each ``standard_normal([B,H,N,d], float32)``
    times sigma, then rounds each value to bfloat16 with round-to-nearest-even.
  * Document lengths for batch b come from ``default_rng((seed, 1 + b))``: integers uniform on
    [lo, hi] inclusive, drawn until their sum reaches N; the last one is cut so the sum is N.
  * ALiBi slopes are float32 ``2 ** (-8 * (h + 1) / H)`` for head index h = 0 .. H-1.

Nothing here depends on a GPU; the arrays are plain numpy.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One attention-forward workload: shapes, value distribution and the score/mask variant."""

    name: str
    B: int
    H: int
    N: int
    d: int
    sigma: float = 1.0
    mask: str = "none"  # 'none' | 'causal' | 'window' | 'document'
    window: int = 0  # sliding window W: key j allowed iff i - W < j <= i
    alibi: bool = False
    softcap: float = 0.0  # 0 = off
    seed: int = 0
    doc_len_range: tuple = (128, 4096)
    scale: float = field(default=None)  # None -> 1/sqrt(d)

    def scale_f32(self) -> np.float32:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)
        return np.float32(s)


# The five workloads the measurements and parity tests are quoted on.
WORKLOADS = {
    "plain_n256_d64": Workload("plain_n256_d64", B=1, H=1, N=256, d=64, seed=1),
    "causal_b4h16_n2048_d128": Workload(
        "causal_b4h16_n2048_d128", B=4, H=16, N=2048, d=128, mask="causal", seed=2),
    "window1024_alibi_b2h32_n8192_d128": Workload(
        "window1024_alibi_b2h32_n8192_d128", B=2, H=32, N=8192, d=128, mask="window",
        window=1024, alibi=True, seed=3),
    "doc_softcap30_h16_n16384_d64": Workload(
        "doc_softcap30_h16_n16384_d64", B=1, H=16, N=16384, d=64, sigma=2.0, mask="document",
        softcap=30.0, seed=4),
    "causal_h32_n16384_d128": Workload(
        "causal_h32_n16384_d128", B=1, H=32, N=16384, d=128, mask="causal", seed=5),
}
WORKLOAD_ORDER = list(WORKLOADS)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Inputs here are finite Gaussian draws, so the NaN case of the rounding is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat, fo = x.reshape(-1).view(np.uint32), out.reshape(-1)
    step = min(flat.size, 1 << 20)
    ubuf, lbuf = np.empty(step, np.uint32), np.empty(step, np.uint32)
    for a in range(0, flat.size, step):  # in pieces, through two reused buffers
        n = min(step, flat.size - a)
        u, lsb = ubuf[:n], lbuf[:n]
        np.copyto(u, flat[a:a + n])
        np.right_shift(u, np.uint32(16), out=lsb)
        np.bitwise_and(lsb, np.uint32(1), out=lsb)
        # no wrap-around: the largest finite or infinite pattern plus 0x8000 stays below 2^32
        u += np.uint32(0x7FFF)
        u += lsb
        u >>= np.uint32(16)
        fo[a:a + n] = u
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_qkv(B: int, H: int, N: int, d: int, sigma: float, seed: int):
    """Q, K, V as bfloat16 bit arrays of shape [B, H, N, d] (d contiguous)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out.append(f32_to_bf16_bits(x))
    return tuple(out)


def draw_dout(B: int, H: int, N: int, d: int, seed: int) -> np.ndarray:
    """The output gradient dO of a backward call: i.i.d. N(0, 1) rounded to bfloat16 bits
    [B, H, N, d], from its own stream (seed, 99) so that Q, K, V are unchanged."""
    rng = np.random.default_rng((seed, 99))
    return f32_to_bf16_bits(rng.standard_normal((B, H, N, d), dtype=np.float32))


def draw_doc_lengths(N: int, lo: int, hi: int, seed) -> list:
    """Document lengths, uniform integers on [lo, hi], drawn until they cover N tokens."""
    rng = np.random.default_rng(seed)
    lengths, total = [], 0
    while total < N:
        n = int(rng.integers(lo, hi, endpoint=True))
        n = min(n, N - total)
        lengths.append(n)
        total += n
    return lengths


def doc_offsets(lengths_per_batch: list, N: int) -> np.ndarray:
    """[B, max_docs + 1] int32: 0 = off[0] < off[1] < ... < off[n] = N, then padded with N."""
    max_docs = max(len(L) for L in lengths_per_batch)
    off = np.full((len(lengths_per_batch), max_docs + 1), N, dtype=np.int32)
    for b, L in enumerate(lengths_per_batch):
        off[b, 0] = 0
        off[b, 1:len(L) + 1] = np.cumsum(L)
    return off


def alibi_slopes(H: int) -> np.ndarray:
    """float32 slopes 2^(-8(h+1)/H), h = 0 .. H-1."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def make_inputs(w: Workload, with_qkv: bool = True) -> dict:
    """Everything one call needs, as numpy arrays: q/k/v bf16 bits, slopes, offsets, scalars."""
    inp = {"workload": w, "scale": w.scale_f32(), "window": int(w.window),
           "softcap": np.float32(w.softcap), "slopes": None, "doc_offsets": None}
    if with_qkv:
        inp["q"], inp["k"], inp["v"] = draw_qkv(w.B, w.H, w.N, w.d, w.sigma, w.seed)
    if w.alibi:
        inp["slopes"] = alibi_slopes(w.H)
    if w.mask == "document":
        lo, hi = w.doc_len_range
        lens = [draw_doc_lengths(w.N, lo, hi, (w.seed, 1 + b)) for b in range(w.B)]
        inp["doc_lengths"] = lens
        inp["doc_offsets"] = doc_offsets(lens, w.N)
    return inp


# ---------------------------------------------------------------------------------------------
# Paged key/value cache for decoding.
#
# Recipe (numpy PCG64, default_rng((seed, 7))): sequence lengths uniform integers on
# [len_lo, len_hi] (at least Lq); each sequence gets ceil(len / page) pages, and the pool holds
# those plus `spare` extra pages; the physical page of every logical page is a random
# permutation of the pool (so a sequence's pages are scattered, as in a shared cache);
# unused table entries point at page 0.  Then K cache, V cache ([n_pages, H, page, d]) and Q
# ([B, H, Lq, d]) are standard_normal * sigma rounded to bfloat16, in that order.

@dataclass(frozen=True)
class DecodeWorkload:
    """One decoding workload: B sequences of H heads, Lq query rows each, over a paged cache."""

    name: str
    B: int
    H: int
    Lq: int
    d: int
    page: int
    len_lo: int
    len_hi: int
    causal: bool = True
    sigma: float = 1.0
    seed: int = 11
    spare: int = 3
    max_pages: int = field(default=None)  # None -> ceil(len_hi / page)

    def scale_f32(self) -> np.float32:
        return np.float32(1.0 / math.sqrt(self.d))


DECODE_WORKLOADS = {
    # one new token per sequence against 2k-14k cached tokens: 1.07 GB of K and V per step
    "decode_b8h32_len2k_14k_d128_p64": DecodeWorkload(
        "decode_b8h32_len2k_14k_d128_p64", B=8, H=32, Lq=1, d=128, page=64, len_lo=2048,
        len_hi=14336, seed=12),
}


def make_paged_inputs(w: DecodeWorkload) -> dict:
    """q, k_cache, v_cache (bf16 bits), page_table, seq_lens (int32) and scalars."""
    rng = np.random.default_rng((w.seed, 7))
    lens = rng.integers(max(w.len_lo, w.Lq), w.len_hi, size=w.B, endpoint=True).astype(np.int32)
    max_pages = w.max_pages or -(-w.len_hi // w.page)
    need = [-(-int(n) // w.page) for n in lens]
    n_pages = int(sum(need)) + w.spare
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.zeros((w.B, max_pages), dtype=np.int32)
    at = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[at:at + k]
        at += k
    out = {"workload": w, "scale": w.scale_f32(), "seq_lens": lens, "page_table": table,
           "n_pages": n_pages}
    for name, shape in (("k_cache", (n_pages, w.H, w.page, w.d)),
                        ("v_cache", (n_pages, w.H, w.page, w.d)), ("q", (w.B, w.H, w.Lq, w.d))):
        x = rng.standard_normal(shape, dtype=np.float32)
        if w.sigma != 1.0:
            x *= np.float32(w.sigma)
        out[name] = f32_to_bf16_bits(x)
    return out
