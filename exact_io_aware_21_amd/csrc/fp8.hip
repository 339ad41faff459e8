// gfx950 kernel of the FP8 forward pass's block quantization.
//
// Page "FlashAttention/es" (marovi.ai), section "Variantes y sucesores": FP8 with a smaller
// quantization error thanks to per-block scaling; page "FlashAttention-3 y torch.compile ..."
// (thecalata.com), section "FlashAttention-3: Asincronía y Explotación del Silicio Hopper": the
// scale is estimated from the data at run time.  Per block of `rows` rows of one (batch, head):
//   scale = amax / 448 (float32; 1 for an all-zero block),  code = E4M3(x / scale),
// with x / scale a correctly rounded float32 division and the E4M3 conversion the hardware's
// round-to-nearest-even (v_cvt_pk_fp8_f32).  One workgroup per block: a max-reduction pass,
// then a conversion pass over the same rows (still in L2).
#include "kcommon.h"
#include "launch.h"

namespace attn {
namespace {

template <int D>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t *__restrict__ x,
                                                        uint8_t *__restrict__ codes,
                                                        float *__restrict__ scales, int N,
                                                        int rows, int nblk) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  __shared__ float wmax[4];
  const int blk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int r0 = blk * rows, r1 = min(N, r0 + rows);
  const uint16_t *src = x + ((size_t)bh * N + r0) * D;
  uint8_t *dst = codes + ((size_t)bh * N + r0) * D;
  const int nchunk = (r1 - r0) * CPR;

  float m = 0.f;
  for (int ci = tid; ci < nchunk; ci += 256) {
    const u32x4 v = *(const u32x4 *)(src + (size_t)ci * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      m = fmaxf(m, fabsf(__uint_as_float(v[w] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(v[w] & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  if (tid == 0) scales[(size_t)bh * nblk + blk] = s;

  for (int ci = tid; ci < nchunk; ci += 256) {
    const u32x4 v = *(const u32x4 *)(src + (size_t)ci * 8);
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w0 = v[2 * h], w1 = v[2 * h + 1];
      out[h] = pack_e4m3x4(__uint_as_float(w0 << 16) / s, __uint_as_float(w0 & 0xFFFF0000u) / s,
                           __uint_as_float(w1 << 16) / s, __uint_as_float(w1 & 0xFFFF0000u) / s);
    }
    *(uint2 *)(dst + (size_t)ci * 8) = make_uint2(out[0], out[1]);
  }
}

}  // namespace

hipError_t launch_quant_fp8(const uint16_t *x, uint8_t *codes, float *scales, int BH, int N,
                            int d, int rows, hipStream_t stream) {
  const int nblk = (N + rows - 1) / rows;
  dim3 grid((unsigned)nblk, (unsigned)BH);
  if (d == 128)
    quant_fp8_kernel<128><<<grid, 256, 0, stream>>>(x, codes, scales, N, rows, nblk);
  else
    quant_fp8_kernel<64><<<grid, 256, 0, stream>>>(x, codes, scales, N, rows, nblk);
  return hipGetLastError();
}

}  // namespace attn
