// Device helpers shared by the kernels: operand types of the gfx950 32x32x16 and 32x32x64
// MFMAs, FP8 E4M3 packing, the register-layout permutations that let MFMA results feed the
// next MFMA directly, and lane-pair reductions.
#pragma once

#include "hipdefs.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef __attribute__((address_space(4))) const float const_f32;

constexpr float kLn2 = 0.69314718055994531f;
// s_getreg operand for HW_ID.SIMD_ID: register 4, bit offset 4, 2 bits.
constexpr int kHwRegSimdId = (4) | (4 << 6) | ((2 - 1) << 11);
constexpr float kTau = 8.0f;
constexpr float kPmax = 256.0f;  // 2^kTau: the largest probability the lazy rescale allows
// Word 3 of a raw (unformatted, stride 0) buffer resource on gfx9-family parts: 32-bit data
// format, no swizzle.  Loads past the resource's byte size return zero.
constexpr int kBufferWord3 = 0x00020000;

// A compile-time integer passed to generic lambdas (scheduling masks must be constants).
template <int V>
struct IntC {
  static constexpr int value = V;
};

// Key permutation inside a 64-key tile: swap bits 2 and 3 (an involution).
__device__ __forceinline__ int pi_key(int x) {
  return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Output-column permutation inside a 32-block of d: accumulator row i = 8a + 4h + b of the
// 32x32 MFMA result (a = i>>3, h = (i>>2)&1, b = i&3) holds column 16h + 4a + b.
__host__ __device__ constexpr int sigma_d(int i) {
  return (((i >> 2) & 1) << 4) | ((i >> 3) << 2) | (i & 3);
}

// LDS row pitch (elements) for a row of `len` 2-byte elements: 16 bytes of padding.  With a
// 256-, 128- or 144-byte row (len 128 or 64), rows r = 0..15 start at 16 distinct 16-byte bank
// slots modulo 256 bytes (and r = 0..7 at 8 distinct slots modulo 128 bytes).
constexpr int pitch(int len) { return len + 8; }

// Marks a wave-uniform branch body as having a side effect so the compiler keeps the branch
// instead of speculating the body into straight-line selects (the element mask and the output
// rescale are rare and must cost nothing when skipped).
__device__ __forceinline__ void keep_branch() { __asm__ volatile("" ::); }

// max / sum of x over the lane pair (l, l ^ 32) that holds the two halves of one query's keys,
// with v_permlane32_swap (no LDS round trip).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 32x32x64 product on FP8 E4M3 operands (cbsz = blgp = 0) with unit block scales (E8M0 code
// 127 = 2^0).  Lane l holds row (A) or column (B) l % 32 and the 32 consecutive k values
// 32 * (l / 32) .. +31, one byte each, lowest k in the lowest byte; the result has the layout of
// the 32x32x16 products.
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four float32 values -> four E4M3 codes, value i in byte i: round to nearest even, no
// saturation (past 448 gives the NaN code).
__device__ __forceinline__ uint32_t pack_e4m3x4(float x0, float x1, float x2, float x3) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false) & 0xFFFFu;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, 0, false) & 0xFFFFu;
  return lo | (hi << 16);
}

// 16 bytes at byte offset voff + soff (voff per lane, soff wave-uniform) of a buffer of `bytes`
// bytes at base (zero past its end).  A free function: buffer built-ins inside a kernel's
// lambdas break its host-side stub.
__device__ __forceinline__ u32x4 buffer_load16(const void *base, uint32_t bytes, int voff,
                                               int soff) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, kBufferWord3);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// One buffer-to-LDS copy instruction: the 64 lanes move 16 bytes each, from byte offset voff
// (per lane) of a buffer of `bytes` bytes at base, into the 1 KB at lds (wave-uniform), lane l to
// bytes 16 l .. 16 l + 15.  Offsets past `bytes` read as zero (bytes = 0: the instruction reads
// nothing and writes zeros).  Completion is counted by vmcnt, like a vector load.
__device__ __forceinline__ void copy16_to_lds(const void *base, uint32_t bytes, int voff,
                                              uint16_t *lds) {
  typedef __attribute__((address_space(3))) void lds_void;
  const auto r = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, 0, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of this wave are
// outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Placement of block w of a grid of nblk blocks over (position, head) pairs, n_pos positions per
// head.  Blocks are dispatched round-robin over the 8 XCDs in order (XCD x receives blocks
// x, x + 8, ...) and a freed compute unit takes the next one.  Each XCD gets a contiguous range
// of heads, whose data then shares its L2.  With lpt (positions of very different work, longest
// at position 0), when the range is whole heads it is walked in groups of g heads: inside a
// group position-major (every head's position p before any head's p + 1), so that long blocks
// start before short ones while only g heads' data is in flight per XCD; g is the largest
// divisor of the range's head count whose heads' bytes (head_bytes each) stay within 16 MiB,
// at least 1.  Otherwise position-major within one head at a time (the natural order).
__device__ __forceinline__ void place_block(int w, int nblk, int n_pos, bool lpt, size_t head_bytes,
                                            int &pos, int &bh) {
  const int n8 = nblk & ~7, per = n8 >> 3;
  if (w < n8 && per % n_pos == 0) {
    const int hc = per / n_pos, i = w >> 3;
    int g = 1;
    if (lpt)
      for (int c = hc; c >= 1; --c)
        if (hc % c == 0 && (size_t)c * head_bytes <= (size_t)16 << 20) {
          g = c;
          break;
        }
    const int gi = i / (g * n_pos), r = i - gi * (g * n_pos);
    bh = (w & 7) * hc + gi * g + r % g;
    pos = r / g;
  } else {
    const int lb = (w < n8) ? (w & 7) * per + (w >> 3) : w;
    bh = lb / n_pos;
    pos = lb - bh * n_pos;
  }
}

// bf16 bits -> fp16 bits; exact for |x| in [2^-14, 65504], saturating beyond (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_to_f16_bits(uint32_t b) {
  float f = __uint_as_float(b << 16);
  if (fabsf(f) > 65504.f) f = copysignf(65504.f, f);
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace
}  // namespace attn
