// gfx950 kernels of attention over a paged key/value cache (decoding).
//
// Page "FlashAttention/es" (marovi.ai), section "Variantes y sucesores", names PagedAttention:
// at inference the key/value cache is cut into pages so that many sequences of different
// lengths share one pool.  The result is the attention of each sequence's last Lq positions over
// its keys and values in order (the pages listed in its page-table row, cut to its length);
// causally, query i (position seq_len - Lq + i) sees positions 0 .. seq_len - Lq + i.
//
// Work split (split-KV): one workgroup per (key range of one sequence and head).  Each forms a
// partial result over its range with the online softmax of section "El truco del softmax en
// línea" (running maximum m, normaliser l, output rescaled by e^{m_old - m_new}); a second
// kernel merges the partials of a (sequence, head) with the same identity.  The work is a
// stream of K and V rows from HBM with a few FLOPs per byte, so the kernels are organised for
// bandwidth, not for the matrix cores:
//  * 256 threads = G groups of D/8 lanes; a group owns one key row per chunk of G consecutive
//    positions, each lane 8 of its d columns (one 16-byte load of K and one of V per row);
//  * a chunk lies inside one page (pages are a power of two >= G rows), so its page id is one
//    scalar load and its rows one buffer resource; rows past the sequence lie beyond that
//    resource's size and read as zero;
//  * q . k is an 8-term FMA per lane and a butterfly over the group's lanes; the softmax is
//    online per group with a lazy rescale (the running maximum only moves when a score exceeds
//    it by more than 8 in base 2), and the groups' partials are combined through LDS.
#include "kcommon.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kDecWord3 = 0x00020000;  // raw buffer resource word 3: 32-bit format, no swizzle

// One 16-byte buffer load at byte offset voff of a resource of `bytes` bytes at base; zero
// past the end.  Every cached K and V row is read exactly once per call, so the loads carry the
// non-temporal hint (cache policy bit nt): the streamed rows then do not displace other lines
// from the caches, and the benchmark workload moves 6.0 TB/s instead of 5.1.  (A free device
// function: buffer builtins must not sit in a lambda, which the host compilation pass also
// instantiates.)
constexpr int kLoadNonTemporal = 2;  // aux operand of the buffer load: nt
__device__ __forceinline__ u32x4 load16(const uint16_t *base, int bytes, int voff) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, kDecWord3);
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kLoadNonTemporal);
}

template <int D, int LQ>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int LPR = D / 8;     // lanes per key row
  constexpr int G = 256 / LPR;   // groups = rows per chunk
  __shared__ float sm[G][LQ], sl[G][LQ];
  __shared__ __attribute__((aligned(16))) float so[G][LQ][D];

  // Consecutive workgroups are the heads of one sequence (same positions, pages 16 KB apart),
  // so the traffic in flight spreads over the whole address range of each page.
  const int bh = blockIdx.x, split = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
  const int tid = threadIdx.x, g = tid / LPR, c = tid % LPR;
  const int max_len = a.max_pages * a.page;
  int seq = ((const_i32 *)a.seq_lens)[b];
  seq = seq < 0 ? 0 : (seq > max_len ? max_len : seq);
  const int t_begin = split * a.keys_per_split;
  const int t_end = min(seq, t_begin + a.keys_per_split);

  // This lane's 8 columns of each query row (fp32), and the running state of its group.
  float qv[LQ][8];
#pragma unroll
  for (int i = 0; i < LQ; ++i) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (i < a.Lq) x = *(const u32x4 *)(a.q + ((size_t)bh * a.Lq + i) * D + 8 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      qv[i][2 * w] = __uint_as_float(x[w] << 16);
      qv[i][2 * w + 1] = __uint_as_float(x[w] & 0xFFFF0000u);
    }
  }
  float m[LQ], l[LQ], o[LQ][8];
#pragma unroll
  for (int i = 0; i < LQ; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
  }

  const_i32 *ptab = (const_i32 *)a.page_table + (size_t)b * a.max_pages;
  const int voff = (g * D + 8 * c) * 2;
  // Rounds of U chunks, software-pipelined: the loads of round r + 1 are issued before round r
  // is computed, so each lane keeps 2 U 16-byte loads in flight while it computes.
  constexpr int U = 4;
  auto load_round = [&](int t0, u32x4 (&kx)[U], u32x4 (&vx)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tu = t0 + u * G;
      kx[u] = vx[u] = u32x4{0u, 0u, 0u, 0u};
      if (tu < t_end) {  // uniform
        int pid = ptab[tu / a.page];
        pid = pid < 0 ? 0 : (pid >= a.n_pages ? a.n_pages - 1 : pid);
        const size_t rbase = ((size_t)pid * a.H + h) * a.page + (tu & (a.page - 1));
        const int bytes = min(G, t_end - tu) * D * 2;
        kx[u] = load16(a.k_cache + rbase * D, bytes, voff);
        vx[u] = load16(a.v_cache + rbase * D, bytes, voff);
      }
    }
  };
  auto compute_round = [&](int t0, const u32x4 (&kx)[U], const u32x4 (&vx)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * G + g;
      float kf[8], vf[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        kf[2 * w] = __uint_as_float(kx[u][w] << 16);
        kf[2 * w + 1] = __uint_as_float(kx[u][w] & 0xFFFF0000u);
        vf[2 * w] = __uint_as_float(vx[u][w] << 16);
        vf[2 * w + 1] = __uint_as_float(vx[u][w] & 0xFFFF0000u);
      }
#pragma unroll
      for (int i = 0; i < LQ; ++i) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(qv[i][e], kf[e], s);
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, LPR);
        const int pos = seq - a.Lq + i;  // position of query i
        const bool ok = t < t_end && (!a.causal || t <= pos);
        s = ok ? s * a.c : -INFINITY;
        if (s > m[i] + kTau) {  // the group's lanes agree (same s, same m)
          const float alpha = m[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[i] - s);
          l[i] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[i][e] *= alpha;
          m[i] = s;
        }
        const float p = ok ? __builtin_amdgcn_exp2f(s - m[i]) : 0.f;
        l[i] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] = fmaf(p, vf[e], o[i][e]);
      }
    }
  };
  u32x4 ka[U], va[U], kb[U], vb[U];
  if (t_begin < t_end) load_round(t_begin, ka, va);
  for (int t0 = t_begin; t0 < t_end; t0 += 2 * U * G) {
    if (t0 + U * G < t_end) load_round(t0 + U * G, kb, vb);
    compute_round(t0, ka, va);
    if (t0 + U * G >= t_end) break;
    if (t0 + 2 * U * G < t_end) load_round(t0 + 2 * U * G, ka, va);
    compute_round(t0 + U * G, kb, vb);
  }

  // Combine the G groups' partials (each relative to its own maximum) through LDS.
#pragma unroll
  for (int i = 0; i < LQ; ++i) {
    if (c == 0) {
      sm[g][i] = m[i];
      sl[g][i] = l[i];
    }
    *(f32x4 *)&so[g][i][8 * c] = f32x4{o[i][0], o[i][1], o[i][2], o[i][3]};
    *(f32x4 *)&so[g][i][8 * c + 4] = f32x4{o[i][4], o[i][5], o[i][6], o[i][7]};
  }
  __syncthreads();
  const size_t pbase = (size_t)bh * a.nsplit + split;  // partial index
  for (int x = tid; x < LQ * D; x += 256) {
    const int i = x / D, col = x % D;
    float M = -INFINITY;
#pragma unroll 4
    for (int gg = 0; gg < G; ++gg) M = fmaxf(M, sm[gg][i]);
    float acc = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll 4
      for (int gg = 0; gg < G; ++gg) {
        const float w = __builtin_amdgcn_exp2f(sm[gg][i] - M);  // 0 for an empty group
        acc = fmaf(w, so[gg][i][col], acc);
        lsum = fmaf(w, sl[gg][i], lsum);
      }
    }
    a.part_o[(pbase * LQ + i) * D + col] = acc;
    if (col == 0) {
      a.part_m[pbase * LQ + i] = M;
      a.part_l[pbase * LQ + i] = lsum;
    }
  }
}

// Merge of the splits of one (sequence, head): O = sum_s w_s o_s / sum_s w_s l_s with
// w_s = 2^{m_s - M}, L = (M + log2 l) ln 2.  One workgroup per (sequence, head).
template <int D, int LQ, bool OUTF32>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  // Per query row: the maximum over splits, each split's weight and the normaliser, in LDS
  // (splits in chunks of 256), then every output column sums its weighted partials.
  __shared__ float sw[256], red[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const size_t pbase = (size_t)bh * a.nsplit;
  for (int i = 0; i < a.Lq; ++i) {
    float M = -INFINITY;
    for (int s0 = tid; s0 < a.nsplit; s0 += 256) M = fmaxf(M, a.part_m[(pbase + s0) * LQ + i]);
    red[tid] = M;
    __syncthreads();
    for (int st = 128; st >= 1; st >>= 1) {
      if (tid < st) red[tid] = fmaxf(red[tid], red[tid + st]);
      __syncthreads();
    }
    M = red[0];
    __syncthreads();
    float lsum = 0.f;
    float acc[D / 64 > 0 ? (D + 255) / 256 : 1] = {};
    for (int s0 = 0; s0 < a.nsplit; s0 += 256) {
      const int s = s0 + tid;
      float w = 0.f;
      if (s < a.nsplit && M != -INFINITY) {
        const size_t ps = (pbase + s) * LQ + i;
        w = __builtin_amdgcn_exp2f(a.part_m[ps] - M);
        lsum = fmaf(w, a.part_l[ps], lsum);
      }
      sw[tid] = w;
      __syncthreads();
      const int n = min(256, a.nsplit - s0);
      for (int col = tid, k = 0; col < D; col += 256, ++k) {
        // independent loads, eight at a time
        float x[8] = {};
        int ss = 0;
        for (; ss + 8 <= n; ss += 8)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            x[u] = fmaf(sw[ss + u], a.part_o[((pbase + s0 + ss + u) * LQ + i) * D + col], x[u]);
        for (; ss < n; ++ss) x[0] = fmaf(sw[ss], a.part_o[((pbase + s0 + ss) * LQ + i) * D + col], x[0]);
        acc[k] += ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
      }
      __syncthreads();
    }
    red[tid] = lsum;
    __syncthreads();
    for (int st = 128; st >= 1; st >>= 1) {
      if (tid < st) red[tid] += red[tid + st];
      __syncthreads();
    }
    const float L = red[0];
    __syncthreads();
    for (int col = tid, k = 0; col < D; col += 256, ++k) {
      const float val = L > 0.f ? acc[k] / L : 0.f;
      const size_t oi = ((size_t)bh * a.Lq + i) * D + col;
      if constexpr (OUTF32)
        ((float *)a.o)[oi] = val;
      else
        ((__bf16 *)a.o)[oi] = (__bf16)val;
    }
    if (tid == 0 && a.lse) a.lse[(size_t)bh * a.Lq + i] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
}

// The same merge for at most 64 splits, with one wave per (sequence, head, query row) and no
// LDS: lane s holds split s's (m, l), the maximum and the normaliser are wave reductions, and
// each lane sums its D / 64 columns over the splits with the weights broadcast from their lanes.
// The partial outputs are loaded in chunks of 16 splits, each chunk's loads issued together; the
// first chunk is loaded with (m, l), before the maximum is known.
template <int D, int LQ, bool OUTF32>
__global__ __launch_bounds__(64) void decode_merge_small_kernel(DecodeArgs a) {
  constexpr int CPL = D / 64;  // columns per lane
  constexpr int CH = 16;       // splits per chunk
  const int bh = blockIdx.x, i = blockIdx.y, lane = threadIdx.x;
  const int ns = a.nsplit;  // <= 64
  const size_t pbase = (size_t)bh * ns;
  const float *po = a.part_o + (pbase * LQ + i) * D + lane;
  const size_t sstride = (size_t)LQ * D;  // between the partials of consecutive splits
  float v[CH][CPL];
  auto load_chunk = [&](int s0) {
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) v[u][c] = s0 + u < ns ? po[(s0 + u) * sstride + 64 * c] : 0.f;
  };
  load_chunk(0);
  float m = -INFINITY, l = 0.f;
  if (lane < ns) {
    m = a.part_m[(pbase + lane) * LQ + i];
    l = a.part_l[(pbase + lane) * LQ + i];
  }
  float M = m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float w = (lane < ns && M != -INFINITY) ? __builtin_amdgcn_exp2f(m - M) : 0.f;
  float L = w * l;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
  float acc[CPL][2] = {};
  for (int s0 = 0; s0 < ns; s0 += CH) {
    if (s0 > 0) load_chunk(s0);
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      // weight of split s0 + u (0 past ns: lanes >= ns hold w = 0)
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(s0 + u, 63)));
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c][u & 1] = fmaf(ws, v[u][c], acc[c][u & 1]);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const float val = L > 0.f ? (acc[c][0] + acc[c][1]) / L : 0.f;
    const size_t oi = ((size_t)bh * a.Lq + i) * D + 64 * c + lane;
    if constexpr (OUTF32)
      ((float *)a.o)[oi] = val;
    else
      ((__bf16 *)a.o)[oi] = (__bf16)val;
  }
  if (lane == 0 && a.lse) a.lse[(size_t)bh * a.Lq + i] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int D, int LQ>
hipError_t launch_decode_lq(const DecodeArgs &a, bool out_f32, hipStream_t s) {
  decode_split_kernel<D, LQ><<<dim3((unsigned)(a.B * a.H), (unsigned)a.nsplit), 256, 0, s>>>(a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (a.nsplit <= 64) {
    const dim3 grid((unsigned)(a.B * a.H), (unsigned)a.Lq);
    if (out_f32)
      decode_merge_small_kernel<D, LQ, true><<<grid, 64, 0, s>>>(a);
    else
      decode_merge_small_kernel<D, LQ, false><<<grid, 64, 0, s>>>(a);
  } else if (out_f32) {
    decode_merge_kernel<D, LQ, true><<<(unsigned)(a.B * a.H), 256, 0, s>>>(a);
  } else {
    decode_merge_kernel<D, LQ, false><<<(unsigned)(a.B * a.H), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs &a, bool out_f32, hipStream_t s) {
  if (a.lq_pad == 1) return launch_decode_lq<D, 1>(a, out_f32, s);
  if (a.lq_pad == 2) return launch_decode_lq<D, 2>(a, out_f32, s);
  if (a.lq_pad == 4) return launch_decode_lq<D, 4>(a, out_f32, s);
  return launch_decode_lq<D, 8>(a, out_f32, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int d, bool out_f32, hipStream_t stream) {
  if (d == 128) return launch_decode_d<128>(a, out_f32, stream);
  return launch_decode_d<64>(a, out_f32, stream);
}

}  // namespace attn
