// Forward pass for short sequences (N <= 256 keys) in a single launch.
//
// The tiled kernel (fwd.hip) needs a V^T pack and a block table before it runs, and walks the
// key tiles of one 256-row query tile serially in one workgroup.  For a short sequence those
// steps are pure latency: on B = H = 1, N = 256 the two launches cost more than the
// arithmetic.  Here every workgroup takes 64 query rows (4 waves x 16) against all N keys at
// once, so the softmax is the plain one of page "FlashAttention/es" (marovi.ai), sections "Por
// qué la atención estándar es lenta" and "El truco del softmax en línea" (one maximum m and one
// sum l per row over all keys), without the block-by-block merge of its section "El algoritmo
// FlashAttention", which only pays when the keys do not fit on chip:
//   * K is staged in LDS once per workgroup (coalesced loads; the four waves then read their A
//     operands from LDS instead of each fetching all of K through the vector cache);
//   * S^T = K Q^T on 16x16x32 bf16 MFMAs, with the rows of the A operand permuted so that a
//     lane's 8 results per 32-key chunk are 8 consecutive keys of its own query: they are then
//     the B operand of the P V product as they stand;
//   * V is transposed into LDS as fp16 (saturating, the conversion of the tiled path) by the
//     four waves together, after the scores are computed;
//   * O^T = V^T P^T on 16x16x32 fp16 MFMAs, P = exp2(t - m) in [0, 1] with the exact row max.
// Score modifications (ALiBi, soft-cap) and masks follow the tiled kernel's definitions: base-2
// scores t = scale log2(e) q.k, or cap log2(e) tanh(scale q.k / cap), plus slope log2(e) (j - i);
// key j is allowed for row i iff lo(i) <= j <= hi(i) (tiles.h).
#include "kcommon.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kSRows = 64;  // query rows per workgroup: 4 waves x 16

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// NC: 32-key chunks covering N (2, 4 or 8).  Every load of the kernel is unconditional, with
// row indexes clamped to N - 1 and out-of-range values replaced afterwards, and every loop has a
// compile-time trip count, so all loads are in flight together: the kernel's time is a few
// memory latencies, not one per chunk.
template <int D, int NC, bool ALIBI, bool SOFTCAP, bool OUTF32>
__global__ __launch_bounds__(256) void fwd_short_kernel(FwdArgs a) {
  constexpr int VP = NC * 32 + 8;              // V^T row pitch in LDS (fp16 elements)
  constexpr int KP = D + 8;                    // K row pitch in LDS (bf16 elements)
  __shared__ __align__(16) uint16_t vt[D * VP];
  __shared__ __align__(16) uint16_t kl[NC * 32 * KP];
  constexpr int NKS = D / 32;                  // k-steps of the score product
  constexpr int NKI = NC * 32 * (D / 8) / 256; // K items (16-byte chunks) per thread
  constexpr int NPAIR = NC * 16;               // key pairs
  constexpr int NIT = NPAIR * (D / 8) / 256;   // V items per thread
  static_assert(NPAIR * (D / 8) % 256 == 0, "V items must divide evenly");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
  const int N = a.N;
  const int q = blockIdx.x * kSRows + wave * 16 + c16;  // this lane's query row
  const bool q_ok = q < N;
  const int qc = q_ok ? q : N - 1;
  const uint16_t *qp = a.q + (size_t)bh * N * D;
  const uint16_t *kp = a.k + (size_t)bh * N * D;
  const uint16_t *vp = a.v + (size_t)bh * N * D;

  // Q^T fragments (B operand): lane holds Q[qc][32 ks + 8 g .. + 7].
  bf16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = *(const bf16x8 *)(qp + (size_t)qc * D + 32 * ks + 8 * g);

  // K rows for LDS: item = (row, 8-column chunk), consecutive threads along a row; rows past
  // N are clamped to N - 1 (their scores are masked).
  u32x4 kx[NKI];
#pragma unroll
  for (int it = 0; it < NKI; ++it) {
    const int idx = tid + 256 * it, row = idx / (D / 8), ch = idx % (D / 8);
    kx[it] = *(const u32x4 *)(kp + (size_t)min(row, N - 1) * D + 8 * ch);
  }
  // V rows for the transpose: item = (key pair, 8-column chunk), keys 2 kp and 2 kp + 1.
  u32x4 vx[NIT][2];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = tid + 256 * it, kpair = idx % NPAIR, ch = idx / NPAIR;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int key = min(2 * kpair + r, N - 1);
      vx[it][r] = *(const u32x4 *)(vp + (size_t)key * D + 8 * ch);
    }
  }
#pragma unroll
  for (int it = 0; it < NKI; ++it) {
    const int idx = tid + 256 * it, row = idx / (D / 8), ch = idx % (D / 8);
    *(u32x4 *)(kl + row * KP + 8 * ch) = kx[it];
  }
  __syncthreads();  // K complete

  // Scores: chunk c, half hf: A row r (lane c16 supplies row r = c16) is key
  // 32 c + 8 (r / 4) + 4 hf + r % 4, so result register i of lane (g, q) is key 32 c + 8 g + 4 hf + i.
  f32x4 s[NC][2];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int key = 32 * c + 8 * (c16 >> 2) + 4 * hf + (c16 & 3);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        acc = mfma16(*(const bf16x8 *)(kl + key * KP + 32 * ks + 8 * g), qf[ks], acc);
      s[c][hf] = acc;
    }
  }

  // V -> V^T (fp16, saturating) in LDS; keys past N are zero.
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = tid + 256 * it, kpair = idx % NPAIR, ch = idx / NPAIR;
    const bool ok0 = 2 * kpair < N, ok1 = 2 * kpair + 1 < N;
    uint32_t *dst = (uint32_t *)vt + (size_t)(8 * ch) * (VP / 2) + kpair;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w0 = ok0 ? (vx[it][0][i >> 1] >> (16 * (i & 1))) & 0xFFFFu : 0u;
      const uint32_t w1 = ok1 ? (vx[it][1][i >> 1] >> (16 * (i & 1))) & 0xFFFFu : 0u;
      dst[i * (VP / 2)] = bf16_to_f16_bits(w0) | (bf16_to_f16_bits(w1) << 16);
    }
  }

  // Base-2 modified scores, masked to -inf outside [lo, hi] (hi <= N - 1).
  const MaskDesc md{a.kind, N, a.window,
                    a.offs ? a.offs + (size_t)b * (a.max_docs + 1) : nullptr, a.max_docs};
  const int lo = row_lo(md, qc), hi = row_hi(md, qc);
  const uint32_t span = (uint32_t)(hi - lo);
  const float slopeL = ALIBI ? a.slopes[h] * 1.4426950408889634f : 0.f;
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 32 * c + 8 * g + e;
      const float x = s[c][e >> 2][e & 3];
      float t;
      if constexpr (SOFTCAP) {
        const float u = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * a.cap_c1));
        t = fmaf(-2.f * a.capL, u, a.capL);
      } else {
        t = x * a.c;
      }
      if constexpr (ALIBI) t = fmaf(slopeL, (float)(j - qc), t);
      if ((uint32_t)(j - lo) > span) t = -INFINITY;
      s[c][e >> 2][e & 3] = t;
      m = fmaxf(m, t);
    }
  }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  const float mu = m == -INFINITY ? 0.f : m;
  float l = 0.f;
  f16x8 pf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(s[c][e >> 2][e & 3] - mu);
      l += p;
      pf[c][e] = (_Float16)p;
    }
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  __syncthreads();  // V^T complete

  // O^T = V^T P^T per 16-column block db: A row = column 16 db + c16, keys 32 c + 8 g .. + 7.
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t *vrow = vt + (size_t)(16 * db + c16) * VP + 8 * g;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = mfma16(*(const f16x8 *)(vrow + 32 * c), pf[c], acc);
    // lane holds O[q][16 db + 4 g + i], i = 0..3
    if (q_ok) {
      const size_t o0 = ((size_t)bh * N + q) * D + 16 * db + 4 * g;
      const f32x4 y = acc * inv;
      if constexpr (OUTF32) {
        *(f32x4 *)((float *)a.o + o0) = y;
      } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        *(bf16x4 *)((uint16_t *)a.o + o0) = __builtin_convertvector(y, bf16x4);
      }
    }
  }
  if (a.lse && q_ok && g == 0)
    a.lse[(size_t)bh * N + q] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

template <int D, bool ALIBI, bool SOFTCAP, bool OUTF32>
hipError_t launch_short_n(const FwdArgs &a, dim3 grid, hipStream_t st) {
  if (a.N <= 64)
    fwd_short_kernel<D, 2, ALIBI, SOFTCAP, OUTF32><<<grid, 256, 0, st>>>(a);
  else if (a.N <= 128)
    fwd_short_kernel<D, 4, ALIBI, SOFTCAP, OUTF32><<<grid, 256, 0, st>>>(a);
  else
    fwd_short_kernel<D, 8, ALIBI, SOFTCAP, OUTF32><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, bool ALIBI, bool SOFTCAP>
hipError_t launch_short_o(bool out_f32, const FwdArgs &a, dim3 grid, hipStream_t st) {
  return out_f32 ? launch_short_n<D, ALIBI, SOFTCAP, true>(a, grid, st)
                 : launch_short_n<D, ALIBI, SOFTCAP, false>(a, grid, st);
}

template <int D>
hipError_t launch_short_d(const FwdInstance &in, const FwdArgs &a, dim3 grid, hipStream_t st) {
  if (in.alibi)
    return in.softcap ? launch_short_o<D, true, true>(in.out_f32, a, grid, st)
                      : launch_short_o<D, true, false>(in.out_f32, a, grid, st);
  return in.softcap ? launch_short_o<D, false, true>(in.out_f32, a, grid, st)
                    : launch_short_o<D, false, false>(in.out_f32, a, grid, st);
}

}  // namespace

hipError_t launch_fwd_short(const FwdInstance &in, const FwdArgs &a, hipStream_t stream) {
  if (a.N < 1 || a.N > kShortMaxN || in.fp8 || (in.d != 64 && in.d != 128))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.N + kSRows - 1) / kSRows), (unsigned)(a.B * a.H));
  if (in.d == 128) return launch_short_d<128>(in, a, grid, stream);
  return launch_short_d<64>(in, a, grid, stream);
}

}  // namespace attn
