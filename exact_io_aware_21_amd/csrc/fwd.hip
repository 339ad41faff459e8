// gfx950 kernels of the FlashAttention forward pass: the V transpose-pack kernel, the block-table
// kernel and the instances of the forward kernel (whose body is in fwd_kernel.h), with their
// launch functions.
#include "fwd_kernel.h"

namespace attn {
namespace {

// ---------------------------------------------------------------------------------------------
// V [BH][N][D] bf16 -> V^T [BH][D][Npad] fp16: keys contiguous, zero beyond N, d rows permuted
// by sigma_d.
template <int D>
__device__ __forceinline__ void vt_pack_body(const uint16_t *__restrict__ v,
                                             uint16_t *__restrict__ vt, int N, int Npad, int kt,
                                             int bh) {
  constexpr int RS = D + 2;  // padded LDS row, in elements
  __shared__ uint16_t t[64 * RS];
  const int tid = threadIdx.x;
  const uint16_t *src = v + (size_t)bh * N * D;
  for (int c = tid; c < 64 * D / 8; c += 256) {
    const int key = c / (D / 8), ch = c % (D / 8);
    const int j = kt * 64 + key;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (j < N) x = *(const u32x4 *)(src + (size_t)j * D + ch * 8);
    uint32_t *dst = (uint32_t *)(t + key * RS + ch * 8);
    dst[0] = x[0];
    dst[1] = x[1];
    dst[2] = x[2];
    dst[3] = x[3];
  }
  __syncthreads();
  uint16_t *out = vt + (size_t)bh * D * Npad + (size_t)kt * 64;
  for (int c = tid; c < D * 8; c += 256) {
    const int p = c >> 3, e = c & 7;
    const int dcol = (p & ~31) | sigma_d(p & 31);
    u32x4 x;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t b0 = t[(e * 8 + 2 * w) * RS + dcol], b1 = t[(e * 8 + 2 * w + 1) * RS + dcol];
      const uint32_t lo = bf16_to_f16_bits(b0);
      const uint32_t hi = bf16_to_f16_bits(b1);
      x[w] = lo | (hi << 16);
    }
    *(u32x4 *)(out + (size_t)p * Npad + e * 8) = x;
  }
}

template <int D>
__global__ __launch_bounds__(256) void vt_pack_kernel(const uint16_t *__restrict__ v,
                                                      uint16_t *__restrict__ vt, int N, int Npad) {
  vt_pack_body<D>(v, vt, N, Npad, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------------------------
// One workgroup per table row (bm, qt): 256 tiles are classified at a time and the non-empty
// ones compacted in ascending kt with a wave ballot plus a 4-entry LDS prefix.
__device__ __forceinline__ void block_table_body(const MaskDesc &m, const int32_t *offs_all,
                                                 int n_qt, int n_kt, int8_t *cls, int32_t *cnt,
                                                 int32_t *list, int row) {
  __shared__ int wave_tot[4];
  const int bm = row / n_qt, qt = row - bm * n_qt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  MaskDesc mm = m;
  if (offs_all) mm.offs = offs_all + (size_t)bm * (m.max_docs + 1);
  int8_t *crow = cls + (size_t)row * n_kt;
  int32_t *lrow = list + (size_t)row * n_kt;
  int base = 0;
  for (int c0 = 0; c0 < n_kt; c0 += 256) {
    const int kt = c0 + tid;
    const int k = kt < n_kt ? tile_class(mm, qt, kt, kBr, kBc) : 0;
    if (kt < n_kt) crow[kt] = (int8_t)k;
    const uint64_t bal = __ballot(k != 0);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(bal);
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      woff += w < wave ? wave_tot[w] : 0;
      tot += wave_tot[w];
    }
    if (k) lrow[base + woff + pre] = kt;
    base += tot;
    __syncthreads();
  }
  for (int kt = base + tid; kt < n_kt; kt += 256) lrow[kt] = 0;
  if (tid == 0) cnt[row] = base;
}

__global__ __launch_bounds__(256) void block_table_kernel(MaskDesc m, const int32_t *offs_all,
                                                          int n_qt, int n_kt, int8_t *cls,
                                                          int32_t *cnt, int32_t *list) {
  block_table_body(m, offs_all, n_qt, n_kt, cls, cnt, list, blockIdx.x);
}

// The two preparation steps of a forward call in one launch: workgroups [0, n_rows) build the
// block table (one row each, when the kind has one), the rest pack V^T (one 64-key tile of one
// head each).  Saves a launch and its gap, which is a few percent of the short workloads' step.
template <int D>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t *__restrict__ v,
                                                   uint16_t *__restrict__ vt, int N, int Npad,
                                                   MaskDesc m, const int32_t *offs_all, int n_rows,
                                                   int n_qt, int n_kt, int8_t *cls, int32_t *cnt,
                                                   int32_t *list) {
  const int w = blockIdx.x;
  if (w < n_rows) {
    block_table_body(m, offs_all, n_qt, n_kt, cls, cnt, list, w);
  } else {
    const int p = w - n_rows, tiles = Npad / 64;
    vt_pack_body<D>(v, vt, N, Npad, p % tiles, p / tiles);
  }
}

template <int D, bool ALIBI, bool SOFTCAP, bool POS, bool OUTF32, bool FP8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(
    FwdArgs a) {
  fwd_body<D, ALIBI, SOFTCAP, POS, OUTF32, FP8, 0>(a);
}

template <int D, bool ALIBI, bool SOFTCAP, bool POS, bool FP8 = false>
hipError_t launch_out(bool out_f32, const FwdArgs &a, dim3 grid, hipStream_t s) {
  if (out_f32)
    fwd_kernel<D, ALIBI, SOFTCAP, POS, true, FP8><<<grid, 512, 0, s>>>(a);
  else
    fwd_kernel<D, ALIBI, SOFTCAP, POS, false, FP8><<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdInstance &in, const FwdArgs &a, dim3 grid, hipStream_t s) {
  if constexpr (D > 128) {
    // two workgroups per (q-tile, head): one for each half of the columns of O
    grid.y = 2;
    if (in.fp8) return hipErrorInvalidValue;
  } else if (in.fp8) {
    if (in.alibi || in.softcap) return hipErrorInvalidValue;
    if (in.pos_scale) return launch_out<D, false, false, true, true>(in.out_f32, a, grid, s);
    return launch_out<D, false, false, false, true>(in.out_f32, a, grid, s);
  }
  if (in.alibi && in.softcap) return launch_out<D, true, true, false>(in.out_f32, a, grid, s);
  // (d = 256 reaches this point only without FP8)
  if (in.alibi) return launch_out<D, true, false, false>(in.out_f32, a, grid, s);
  if (in.softcap) return launch_out<D, false, true, false>(in.out_f32, a, grid, s);
  if (in.pos_scale) return launch_out<D, false, false, true>(in.out_f32, a, grid, s);
  return launch_out<D, false, false, false>(in.out_f32, a, grid, s);
}

}  // namespace

hipError_t launch_vt_pack(const uint16_t *v, uint16_t *vt, int BH, int N, int Npad, int d,
                          hipStream_t stream) {
  dim3 grid(Npad / 64, BH);
  if (d == 256)
    vt_pack_kernel<256><<<grid, 256, 0, stream>>>(v, vt, N, Npad);
  else if (d == 128)
    vt_pack_kernel<128><<<grid, 256, 0, stream>>>(v, vt, N, Npad);
  else
    vt_pack_kernel<64><<<grid, 256, 0, stream>>>(v, vt, N, Npad);
  return hipGetLastError();
}

hipError_t launch_prep(const uint16_t *v, uint16_t *vt, int BH, int N, int Npad, int d,
                       const MaskDesc &m, const int32_t *offs_all, int Bm, int n_qt, int n_kt,
                       int8_t *cls, int32_t *cnt, int32_t *list, hipStream_t stream) {
  const int n_rows = cls ? Bm * n_qt : 0;
  const dim3 grid((unsigned)(n_rows + (Npad / 64) * BH));
  if (d == 256)
    prep_kernel<256><<<grid, 256, 0, stream>>>(v, vt, N, Npad, m, offs_all, n_rows, n_qt, n_kt,
                                               cls, cnt, list);
  else if (d == 128)
    prep_kernel<128><<<grid, 256, 0, stream>>>(v, vt, N, Npad, m, offs_all, n_rows, n_qt, n_kt,
                                               cls, cnt, list);
  else
    prep_kernel<64><<<grid, 256, 0, stream>>>(v, vt, N, Npad, m, offs_all, n_rows, n_qt, n_kt,
                                              cls, cnt, list);
  return hipGetLastError();
}

hipError_t launch_block_table(MaskDesc m, const int32_t *offs_all, int Bm, int n_qt, int n_kt,
                              int8_t *cls, int32_t *cnt, int32_t *list, hipStream_t stream) {
  block_table_kernel<<<Bm * n_qt, 256, 0, stream>>>(m, offs_all, n_qt, n_kt, cls, cnt, list);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdInstance &in, const FwdArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)a.n_qt * (unsigned)(a.B * a.H));
  if (in.d == 256) return launch_d<256>(in, a, grid, stream);
  if (in.d == 128) return launch_d<128>(in, a, grid, stream);
  return launch_d<64>(in, a, grid, stream);
}

}  // namespace attn
