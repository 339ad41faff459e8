// The gfx950 forward kernel of the FlashAttention forward pass (body template).
//
// The tiled forward pass with the online softmax follows page "FlashAttention/es" (marovi.ai),
// section "El algoritmo FlashAttention": Q is split into blocks of Br rows that stay on chip,
// K and V are streamed block by block (Bc keys) through on-chip memory, each score block is
// formed and reduced while the running maximum m and normaliser l are carried along, the output
// is rescaled by e^{m_old - m_new} when the maximum moves, and at the end O is divided by l and
// L = m + ln(l) is written.  The loop order (outer over query blocks, one workgroup each; inner
// over key blocks) is the one the section "Variantes y sucesores" credits to the second version.
// The N x N score matrix never leaves registers.
//
// gfx950 mapping (one workgroup = 8 wave64s = Br = 256 query rows, 32 per wave; the two waves
// on each SIMD alternate between matrix-core and vector phases, see fwd_body):
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K is the A operand
//    read from LDS, Q^T the B operand held in VGPRs for the whole kernel.  In the 32x32 result
//    each lane owns one query (lane % 32) and 16 keys, so a row maximum is an in-lane max plus a
//    single exchange with lane ^ 32, and the running m, l live in one VGPR per lane.
//  * K rows are stored in LDS with key bits 2 and 3 swapped.  After that permutation the 16
//    score registers of a lane hold keys {16*(r/8) + 8*(lane/32) + r%8}, i.e. two runs of 8
//    consecutive keys, which is exactly the B-operand layout of the P V product: P^T feeds
//    O^T = V^T P^T straight from registers, with no LDS round trip.
//  * V^T (d rows, keys contiguous) is the A operand of that product.  The call's preparation
//    launch (prep_kernel, which also builds the block table) writes V^T into the workspace,
//    with the d rows of each 32-block permuted so that each lane's 16 accumulator registers
//    hold 16 consecutive output columns.
//  * The P V product runs on fp16 operands (v_mfma_f32_32x32x16_f16, the same rate as bf16):
//    bf16 V converts to fp16 exactly inside the pack kernel, and P <= 2^8 (see below) keeps
//    11 significant bits instead of bf16's 8.  With bf16 P the rounding of a dominant
//    probability alone moves O by up to 2^-9 |v|, which exceeds 1e-2 for |v| near 8.
//    Q K^T stays on bf16 operands, which are the exact input values.
//  * K and V^T tiles go through a ring of four LDS buffers (three for d = 256), filled by
//    buffer-to-LDS copies (buffer_load ... lds: no staging registers, no ds_write) that each
//    wave issues, for the tile pair three (d = 256: two) iterations ahead, between the MFMAs
//    of its own matrix-core phase: spread out, not a burst of every wave's loads at a barrier.
//    Each LDS row is padded by 16 bytes, so the 8 (or 16) lanes of one ds_read_b128 phase,
//    which read the same column of 8 (16) consecutive rows, hit distinct banks, while every
//    operand address stays lane base + compile-time offset.
//  * Scores are kept in base-2 units (scale * log2 e folded in), so each probability costs one
//    v_exp_f32; L is converted back to natural log in the epilogue.
//  * The running maximum is only moved when a tile's scores exceed it by more than 8 (base 2):
//    the output and l are then rescaled, otherwise probabilities are formed against the older
//    maximum and stay below 2^8.  Both are exact rewritings of the same sums.  Except under the
//    built-in soft-cap the test is made on the probabilities' sum, so the common tile skips its
//    row maximum altogether.
//  * Fully masked tiles never reach the kernel: it walks the per-q-tile list of non-empty tiles
//    from the block table, and evaluates the element mask only on partial tiles.
//
// This header is compiled twice: into the library (fwd.hip instantiates the fixed variants) and
// at run time by hipRTC together with a user's score / mask modification (MOD != 0), for which
// the two functions below are declared here and defined by the user's source:
//   attn_score_mod(s, b, h, i, j, p): the modified score of query i and key j from the scaled
//     score s = scale * q_i . k_j (natural units), p the caller's parameter array;
//   attn_mask_mod(b, i, j, p): whether key j is allowed for query i of batch entry b.
#pragma once

#include "kcommon.h"
#include "launch.h"

__device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p);
__device__ bool attn_mask_mod(int b, int i, int j, const float *p);

// Race-check build (ATTN_RACE_CHECK=1, a debug library only): every LDS tile word starts as a
// pattern that is NaN as bf16, as fp16 and as each of its two E4M3 bytes, so a read of a slot no
// copy has filled poisons the output; every wait of the copy ring drains all outstanding memory
// operations and every barrier in the loop is a full workgroup barrier with a memory fence, so
// no copy is in flight across a barrier.  Its outputs must equal the pipelined build's bit for
// bit: a miscounted wait, or a copy landing in a buffer still being read, shows up as a
// difference (or a NaN) there.
#ifndef ATTN_RACE_CHECK
#define ATTN_RACE_CHECK 0
#endif

namespace attn {
namespace {

// Waits until at most the copies the immediate allows are outstanding (all of them in the
// race-check build).
template <int IMM>
__device__ __forceinline__ void ring_wait() {
  if constexpr (ATTN_RACE_CHECK)
    __builtin_amdgcn_s_waitcnt(0);
  else
    __builtin_amdgcn_s_waitcnt(IMM);
}

// The barriers of the loop: bare (copies stay in flight across them), or full in the
// race-check build.
__device__ __forceinline__ void ring_barrier() {
  if constexpr (ATTN_RACE_CHECK)
    __syncthreads();
  else
    __builtin_amdgcn_s_barrier();
}

constexpr int kModScore = 1;     // MOD bit: attn_score_mod replaces the scaled score
constexpr int kModMask = 2;      // MOD bit: attn_mask_mod decides the element mask
constexpr int kModMaxFirst = 4;  // MOD bit: the score modification moves row maxima often

// The forward kernel body.  One workgroup = 8 wave64s over Br = 256 query rows (32 rows per wave).
// Waves w and w + 4 run on the same SIMD; they form two groups (w < 4 and w >= 4) that work one
// phase apart:
//   M-phase of tile t : O^T += V_{t-1}^T P_{t-1}^T, then S_t^T = K_t Q^T   (MFMA + LDS reads)
//   V-phase of tile t : mask, row max, lazy rescale, P_t = exp2(S_t - m)   (VALU)
// Slot s (between two barriers) runs the M-phase of group (s & 1) and the V-phase of the other,
// so on every SIMD one wave keeps the matrix core busy while the other does the softmax.
// K_t and V_{t-1} are the LDS tiles read in slots 2t and 2t+1; each wave stages its share of
// the next tiles between the MFMAs of its own M-phase (see the loop below).
//
// FP8 instances (FP8 = true) form the scores from E4M3 codes with v_mfma_scale_f32_32x32x64_f8f6f4:
// the workgroup quantizes its own 256 Q rows (one scale s_q for the tile) and reads K as codes
// with one scale s_k per 64-key tile (quantized by quant_fp8_kernel beforehand), so the score
// block is s_q s_k (Q8 K8^T); the factor s_q s_k is folded into the base-2 scale of the V-phase.
// K8 rows take D + 16 bytes in LDS (the same bank spread as the bf16 rows); P V is unchanged.
template <int D, bool ALIBI, bool SOFTCAP, bool POS, bool OUTF32, bool FP8, int MOD>
__device__ __forceinline__ void fwd_body(const FwdArgs &a) {
  constexpr int NT = 512;                // threads per workgroup
  // Head dimension 256: the scores need all of d, but 256 columns of O do not fit the register
  // file beside Q^T at two waves per SIMD, so each workgroup forms the scores over all of d and
  // accumulates one half of O, DV = 128 columns (blockIdx.y picks the half); the tiles then take
  // three LDS buffers instead of four.
  constexpr int DV = D > 128 ? 128 : D;  // columns of O (rows of V^T) of this workgroup
  constexpr int NB = D > 128 ? 3 : 4;    // LDS buffers of the copy ring
  constexpr int VCH = kBc / 8;           // 16-byte chunks per V^T row
  constexpr int NKS = D / 16;            // k-steps of the score product
  constexpr int NDB = DV / 32;           // 32-column blocks of O
  constexpr int KP = pitch(D);           // LDS pitch of a K row (keys x D)
  constexpr int VP = pitch(kBc);         // LDS pitch of a V^T row (D x keys)
  constexpr int KP8 = D + 16;            // LDS pitch of an FP8 K row, bytes
  constexpr int NKS8 = D / 64;           // k-steps of the FP8 score product
  static_assert(kBr == 256 && kBc == 64, "kernel is written for 256 x 64 tiles");
  static_assert(!FP8 || (!ALIBI && !SOFTCAP), "FP8 instances take no score modification");
  static_assert(MOD == 0 || (POS && !ALIBI && !SOFTCAP && !FP8),
                "modification instances take natural-units scores on the POS path");
  // LDS tiles: four buffers, each an array of its own holding a K tile, then a V^T tile, then
  // a spare 1 KB row, so that every access of the bf16 instances names its buffer statically
  // (the compiler then tracks the buffer-to-LDS copies in flight per buffer and waits only
  // where a read needs one).  The spare row takes the copy instructions a wave issues beyond
  // the tiles' share, which read nothing and write zeros.  FP8 K rows are KP8 bytes.
  constexpr int SPK = FP8 ? KP8 / 16 : KP / 8, SPV = VP / 8;  // 16-byte slots per LDS row
  constexpr int NJK = kBc * SPK / 64, NJV = DV * SPV / 64;  // copy instructions per tile
  constexpr int NJ = NJK + NJV;
  static_assert(kBc * SPK % 64 == 0 && DV * SPV % 64 == 0, "tiles must fill whole copy rows");
  static_assert(!FP8 || D <= 128, "FP8 instances are built for d <= 128");
  __shared__ __attribute__((aligned(16))) uint16_t sB0[(NJ + 1) * 512];
  __shared__ __attribute__((aligned(16))) uint16_t sB1[(NJ + 1) * 512];
  __shared__ __attribute__((aligned(16))) uint16_t sB2[(NJ + 1) * 512];
  __shared__ __attribute__((aligned(16))) uint16_t sB3[NB > 3 ? (NJ + 1) * 512 : 8];
  auto buf = [&](auto bc) -> uint16_t * {
    constexpr int Bi = decltype(bc)::value;
    if constexpr (Bi == 0) return sB0;
    if constexpr (Bi == 1) return sB1;
    if constexpr (Bi == 2) return sB2;
    if constexpr (Bi == 3) return sB3;
    return nullptr;
  };

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  // Phase group: of the two waves the dispatcher placed on a SIMD, the lower-numbered one is
  // group 0 and the other group 1 (SIMD id from the HW_ID register).  Correctness does not
  // depend on this choice, only the overlap of matrix-core and vector work does.
  __shared__ int simd_of[8];
  __shared__ float qmax[8];
  if (lane == 0) simd_of[wave] = __builtin_amdgcn_s_getreg(kHwRegSimdId) & 3;
  __syncthreads();
  int grp = 0;
  for (int w2 = 0; w2 < wave; ++w2) grp += simd_of[w2] == simd_of[wave];
  grp = __builtin_amdgcn_readfirstlane(grp > 1 ? 1 : grp);  // wave-uniform: scalar branches

  // Each XCD works on a contiguous range of heads (their q-tiles share K and V in its L2).
  // Causal and document masks give q-tiles key lists of very different lengths: their blocks
  // are placed longest first across small groups of heads (see place_block; a head's K and V^T
  // take 4 N d bytes).  Other kinds keep one head at a time, whose concurrently running q-tiles
  // share most of their keys (a sliding window ran 5 % slower interleaved).
  const bool lpt = MOD == 0 && (a.kind == kMaskCausal || a.kind == kMaskDocument);
  int qx, bh;
  place_block(blockIdx.x, gridDim.x, a.n_qt, lpt, (size_t)2 * a.N * (D + DV), qx, bh);
  const int vcol0 = D > 128 ? (int)blockIdx.y * DV : 0;  // first column of O of this workgroup
  // Masked kinds have longer key lists for later q-tiles: start those first.
  const int qt = (a.kind != kMaskNone || (MOD & kModMask)) ? a.n_qt - 1 - qx : qx;
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N;

  const int qrow = qt * kBr + wave * 32 + l32;
  const bool q_ok = qrow < N;
  const MaskDesc md{a.kind, N, a.window, a.offs ? a.offs + (size_t)b * (a.max_docs + 1) : nullptr,
                    a.max_docs};
  int lo = N + kBc, hi = N + kBc;  // rows beyond N: a single key past every tile (all masked)
  if (q_ok) {
    lo = row_lo(md, qrow);
    hi = row_hi(md, qrow);
  }

  // Q^T fragments (B operand): lane holds Q[qrow][16*ks + 8*hf .. +7]; FP8: lane holds the
  // codes of Q[qrow][64*ks + 32*hf .. +31].
  bf16x8 qf[FP8 ? 1 : NKS];
  i32x8 q8f[FP8 ? NKS8 : 1];
  float cq = a.c;  // base-2 score scale; FP8: times s_q
  if constexpr (FP8) {
    u32x4 xq[NKS8][4];
    const uint16_t *qp = a.q + ((size_t)bh * N + (q_ok ? qrow : 0)) * D + hf * 32;
#pragma unroll
    for (int ks = 0; ks < NKS8; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (q_ok) x = *(const u32x4 *)(qp + ks * 64 + u * 8);
        xq[ks][u] = x;
      }
    // s_q = amax / 448 over the workgroup's rows (rows beyond N hold zeros).
    float mx = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS8; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mx = fmaxf(mx, fabsf(__uint_as_float(xq[ks][u][e] << 16)));
          mx = fmaxf(mx, fabsf(__uint_as_float(xq[ks][u][e] & 0xFFFF0000u)));
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if (lane == 0) qmax[wave] = mx;
    __syncthreads();
    float amax = qmax[0];
#pragma unroll
    for (int w2 = 1; w2 < 8; ++w2) amax = fmaxf(amax, qmax[w2]);
    const float sq = amax > 0.f ? amax / 448.0f : 1.0f;
    // code = E4M3(x / s_q), a correctly rounded division then round-to-nearest-even.
#pragma unroll
    for (int ks = 0; ks < NKS8; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const uint32_t w0 = xq[ks][u][2 * h2], w1 = xq[ks][u][2 * h2 + 1];
          q8f[ks][2 * u + h2] = (int32_t)pack_e4m3x4(
              __uint_as_float(w0 << 16) / sq, __uint_as_float(w0 & 0xFFFF0000u) / sq,
              __uint_as_float(w1 << 16) / sq, __uint_as_float(w1 & 0xFFFF0000u) / sq);
        }
    cq = a.c * sq;
  } else {
    const uint16_t *qp = a.q + ((size_t)bh * N + (q_ok ? qrow : 0)) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (q_ok) x = *(const u32x4 *)(qp + ks * 16);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
    // Settle the Q loads here, once, so no memory wait is charged to the first MFMA of every
    // loop iteration.
    __builtin_amdgcn_s_waitcnt(0);
  }

  // The key-tile list of this q-tile (written by the table kernel before this launch, so it is
  // read-only here): read through the constant address space, i.e. with scalar loads.
  int T;
  const_i32 *lst = nullptr;
  if (a.list) {
    const int bm = (a.kind == kMaskDocument || (MOD & kModMask)) ? b : 0;
    const size_t row = (size_t)bm * a.n_qt + qt;
    T = ((const_i32 *)a.cnt)[row];
    lst = (const_i32 *)a.list + row * a.n_kt;
    // A modification's table may have been left by an earlier call (the caller vouches for it):
    // clamp what is read from it so that any contents stay in bounds.
    if constexpr ((MOD & kModMask) != 0) T = min(max(T, 0), a.n_kt);
  } else {
    T = a.n_kt;
  }
  // ALiBi instances walk the key tiles from the last one back to the first.  The bias
  // -slope (i - j) grows towards larger keys, by slope * 64 per tile, so in ascending order the
  // running maximum of a steep head moves on nearly every tile (each move rescales O); the
  // first tile of the descending walk holds the largest biases, and the maximum then rarely
  // moves.  Instances with a user score modification walk the same way (unless created with
  // the max-first flag): the position biases such functions usually add (ALiBi,
  // relative-position terms) favour the nearest keys too.  The order of the tiles does not
  // change the sums (the online softmax is a merge of per-tile partial results), only their
  // rounding order.
  constexpr bool REV = (ALIBI && MOD == 0) || ((MOD & kModScore) != 0 && (MOD & kModMaxFirst) == 0);
  auto kt_of = [&](int t) -> int {
    if constexpr (REV) t = T - 1 - t;
    if (!lst) return t;
    if constexpr ((MOD & kModMask) != 0) return min(max(lst[t], 0), a.n_kt - 1);
    return lst[t];
  };

  constexpr int KROW = FP8 ? D : 2 * D;  // bytes per K row in memory
  constexpr int KCHR = KROW / 16;        // 16-byte chunks per K row
  const char *kbytes = FP8 ? (const char *)(a.k8 + (size_t)bh * N * D)
                           : (const char *)(a.k + (size_t)bh * N * D);
  const uint16_t *vbase = a.vt + ((size_t)bh * D + vcol0) * a.Npad;

  const float slopeL = ALIBI ? a.slopes[h] * 1.4426950408889634f : 0.f;
  // Soft-cap without ALiBi keeps u = 1 / (1 + e^{2 s / cap}) per score instead of the capped
  // score t = cap (1 - 2 u) (base 2: capL - 2 capL u): the probability is then one FMA and one
  // exponential, exp2(capL - m - 2 capL u), and the tile maximum of t is taken as the minimum
  // of u.  A masked score is u = +inf.  (An odd polynomial for tanh on the FMA pipe, taking
  // two transcendentals per score off, ran 10 % slower: these kernels are bound by vector
  // issue, not by the transcendental unit.)
  constexpr bool UCAP = SOFTCAP && !ALIBI && !POS && MOD == 0;
  constexpr float kMasked = UCAP ? INFINITY : -INFINITY;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  f32x16 s[2];
  f16x8 pb[4];

  // One M-phase as a single software-pipelined sequence of MFMA steps: the P V steps
  // (key group kk, d block db) and then the score steps (k-step ks, key block blk), ordered so
  // that consecutive MFMAs write different accumulators.  The A
  // fragment of step i + kDepth is read from LDS while step i runs, so LDS latency stays hidden
  // behind the matrix core.
  // Staging item j (`item(j)`: one buffer-to-LDS copy instruction of a later tile pair) goes
  // after MFMA step 1 + j * NST / NI.  The first kDepth fragments are read before the phase:
  // the wave's previous V-phase issues them into win_pre (see prefetch).
  constexpr int kDepth = 4;
  u32x4 win_pre[kDepth];
  // Both M-phases start with P V steps, so the window holds V^T fragments (kDepth <= 4 NDB).
  static_assert(kDepth <= 4 * NDB, "the first fragments must be V^T fragments");
  auto prefetch = [&](const uint16_t *buf) {
    const uint16_t *vl = buf + NJK * 512 + l32 * VP + hf * 8;
#pragma unroll
    for (int i = 0; i < kDepth; ++i)
      win_pre[i] = *(const u32x4 *)(vl + (i % NDB) * 32 * VP + (i / NDB) * 16);
  };
  auto mphase_bf16 = [&](const uint16_t *kl, const uint16_t *vl, auto item, auto nitc) {
    constexpr int NPV = 4 * NDB;
    constexpr int NST = NPV + 2 * NKS;
    constexpr int NI = decltype(nitc)::value;
    const uint16_t *vbuf = vl + l32 * VP + hf * 8;
    const uint16_t *kbuf = kl + l32 * KP + hf * 8;
    auto frag = [&](int i) -> u32x4 {
      if (i < NPV) {
        const int kk = i / NDB, db = i % NDB;
        return *(const u32x4 *)(vbuf + db * 32 * VP + kk * 16);
      }
      const int j = i - NPV, ks = j >> 1, blk = j & 1;
      return *(const u32x4 *)(kbuf + blk * 32 * KP + ks * 16);
    };
    u32x4 win[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) win[i] = win_pre[i];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const u32x4 cur = win[i % kDepth];
      if (i + kDepth < NST) win[i % kDepth] = frag(i + kDepth);
      if (i < NPV) {
        const int kk = i / NDB, db = i % NDB;
        oacc[db] = mfma32(__builtin_bit_cast(f16x8, cur), pb[kk], oacc[db]);
      } else {
        const int j = i - NPV, ks = j >> 1, blk = j & 1;
        s[blk] = mfma32(__builtin_bit_cast(bf16x8, cur), qf[ks], ks == 0 ? f32x16{} : s[blk]);
      }
#pragma unroll
      for (int j = 0; j < NI; ++j)
        if (i == 1 + j * NST / NI) item(j);
    }
    // Pin that order for the scheduler: MFMA / LDS read pairs, with the copy items in between.
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        if (i == 1 + j * NST / NI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (i + kDepth < NST) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  // The FP8 M-phase: the same P V steps, then 2 * D / 64 score steps (k-step ks, key block blk),
  // each fed by two 16-byte LDS reads of K8 (bytes 64*ks + 32*hf .. +31 of the lane's key row).
  // The LDS reads form one stream, kDepth reads ahead of the MFMA that consumes them.
  auto mphase_fp8 = [&](const uint16_t *kl, const uint16_t *vl, auto item, auto nitc) {
    constexpr int NPV = 4 * NDB;
    constexpr int NSS = 2 * NKS8;      // score MFMAs
    constexpr int NST = NPV + NSS;     // MFMAs
    constexpr int NR = NPV + 2 * NSS;  // LDS reads
    constexpr int NI = decltype(nitc)::value;
    const uint16_t *vbuf = vl + l32 * VP + hf * 8;
    const uint8_t *kbuf = (const uint8_t *)kl + l32 * KP8 + hf * 32;
    auto frag = [&](int r) -> u32x4 {
      if (r < NPV) {
        const int kk = r / NDB, db = r % NDB;
        return *(const u32x4 *)(vbuf + db * 32 * VP + kk * 16);
      }
      const int j = r - NPV, st = j >> 1, half = j & 1, ks = st >> 1, blk = st & 1;
      return *(const u32x4 *)(kbuf + blk * 32 * KP8 + ks * 64 + half * 16);
    };
    u32x4 win[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) win[i] = win_pre[i];
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const u32x4 cur = win[i % kDepth];
      if (i + kDepth < NR) win[i % kDepth] = frag(i + kDepth);
      const int kk = i / NDB, db = i % NDB;
      oacc[db] = mfma32(__builtin_bit_cast(f16x8, cur), pb[kk], oacc[db]);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        if (i == 1 + j * NST / NI) item(j);
    }
#pragma unroll
    for (int st = 0; st < NSS; ++st) {
      const int r0 = NPV + 2 * st, ks = st >> 1, blk = st & 1;
      const u32x4 a0 = win[r0 % kDepth];
      if (r0 + kDepth < NR) win[r0 % kDepth] = frag(r0 + kDepth);
      const u32x4 a1 = win[(r0 + 1) % kDepth];
      if (r0 + 1 + kDepth < NR) win[(r0 + 1) % kDepth] = frag(r0 + 1 + kDepth);
      const i32x8 kf = {(int32_t)a0[0], (int32_t)a0[1], (int32_t)a0[2], (int32_t)a0[3],
                        (int32_t)a1[0], (int32_t)a1[1], (int32_t)a1[2], (int32_t)a1[3]};
      s[blk] = mfma32_fp8(kf, q8f[ks], ks == 0 ? f32x16{} : s[blk]);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        if (NPV + st == 1 + j * NST / NI) item(j);
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        if (i == 1 + j * NST / NI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (i + kDepth < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int st = 0; st < NSS; ++st) {
      const int r0 = NPV + 2 * st;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        if (NPV + st == 1 + j * NST / NI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (r0 + kDepth < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (r0 + 1 + kDepth < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto mphase = [&](auto body) {
    // The matrix-core wave issues first: without this the older wave of each SIMD pair wins
    // issue arbitration in both slots, and the younger one's M-phase ran ~25 % longer than the
    // older one's (in-kernel timestamps; with the priority both take the same time).
    __builtin_amdgcn_s_setprio(3);
    body();
    // Keep the score MFMAs in this slot: without a use here the compiler sinks the last ones
    // past the barrier into the (conditional) V-phase that reads them.
    const f32x16 s0 = s[0], s1 = s[1];
    __asm__ volatile("" ::"v"(s0), "v"(s1));
    __builtin_amdgcn_s_setprio(0);
  };

  // P = 0 for the first M-phase (its P V step then adds exactly 0 against a zero V^T tile).
#pragma unroll
  for (int g = 0; g < 4; ++g) pb[g] = f16x8{};

  // V-phase of tile t: score modifications, mask, online softmax, P_t in fp16.
  // ALiBi without soft-cap forms its scores relative to the running maximum m (folded into the
  // per-tile bias base), so its probabilities need no subtraction: exp2(s) directly.
  constexpr bool REL = ALIBI && !SOFTCAP && MOD == 0;
  auto vphase = [&](int kt, float skt) {
    // Base-2 score scale of this tile; FP8: times s_k of the key tile (skt, loaded ahead).
    const float c = FP8 ? cq * skt : cq;
    // Register r of block blk is key kt*Bc + 32*blk + 16*(r/8) + 8*hf + r%8.
    const int kb = kt * kBc + 8 * hf;
    // The reference the scores of this tile are taken against (REL): m, or 0 before the row
    // has seen a finite score.
    const float m_ref = REL ? (m_run == -INFINITY ? 0.f : m_run) : 0.f;
    if constexpr (MOD != 0) {
      // Natural-units scores, modified by the user's function; these instances run with
      // POS = true and c = log2(e), so the conversion to base 2 rides on the exponent's FMA.
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = s[blk][r] * a.scale;
          if constexpr ((MOD & kModScore) != 0) {
            const int j = kb + 32 * blk + 16 * (r >> 3) + (r & 7);
            s[blk][r] = attn_score_mod(x, b, h, qrow, j, a.mod_params);
          } else {
            s[blk][r] = x;
          }
        }
      }
    } else if constexpr (!POS) {
      const float abase = ALIBI ? slopeL * (float)(kb - qrow) - m_ref : 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = s[blk][r];
          float tt;
          if constexpr (SOFTCAP) {
            const float e = __builtin_amdgcn_exp2f(x * a.cap_c1);
            const float u = __builtin_amdgcn_rcpf(1.f + e);
            tt = UCAP ? u : fmaf(-2.f * a.capL, u, a.capL);
          } else {
            tt = x * c;
          }
          if constexpr (ALIBI)
            tt += fmaf(slopeL, (float)(32 * blk + 16 * (r >> 3) + (r & 7)), abase);
          s[blk][r] = tt;
        }
      }
    }
    if constexpr ((MOD & kModMask) != 0) {
      // The user's mask on every element, unless the table marks this wave's 32 rows of the
      // tile fully allowed (bit `wave` of its row-block byte).
      const size_t ci = ((size_t)b * a.n_qt + qt) * a.n_kt + kt;
      const int wf = (((const_i32 *)a.wfull)[ci >> 2] >> (8 * (int)(ci & 3))) & 0xFF;
      if (!((wf >> wave) & 1)) {
        keep_branch();
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kb + 32 * blk + 16 * (r >> 3) + (r & 7);
            if (!q_ok || j >= N || !attn_mask_mod(b, qrow, j, a.mod_params))
              s[blk][r] = kMasked;
          }
        }
      }
    } else if (__builtin_amdgcn_ballot_w64(!(lo <= kt * kBc && hi >= kt * kBc + kBc - 1))) {
      // Element mask only when some row of this wave does not allow all 64 keys of the tile
      // (hi <= N - 1 always, so a fully allowed row also has the tile in range).  Key j = kb + o
      // is allowed iff lo <= j <= hi, i.e. iff (unsigned)(o - (lo - kb)) <= (unsigned)(hi - lo):
      // one subtraction, one compare and one select per score.
      keep_branch();
      const int a0 = lo - kb;
      const uint32_t span = (uint32_t)(hi - lo);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 32 * blk + 16 * (r >> 3) + (r & 7);
          if ((uint32_t)(o - a0) > span) s[blk][r] = kMasked;
        }
      }
    }
    // Probabilities against the running maximum m (base 2), which must keep every P <= 2^8
    // (the range and precision of the fp16 P V operands): the lazy rescale with threshold 8.
    // Unmodified scores (POS instances without a modification) and ALiBi scores walked in
    // descending key order skip the tile maximum in the common case: a lane's sum of its 32
    // probabilities bounds each of them, so while every sum is <= 2^8 the running m stands.
    // Otherwise, or for a row with no maximum yet that sees a finite score, the tile maximum is
    // taken, m moves and the output is rescaled, and the probabilities are formed again.  User
    // modifications (natural-units scores, POS) take the same path, walked in descending key
    // order when they modify scores.  The built-in soft-cap moves the maximum often, so those
    // instances take the tile maximum first, every tile, and so do modifications created with
    // the max-first flag.
    auto probs = [&](float m_use) -> float {
      float psum[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x8 pv;
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = s[g >> 1][8 * (g & 1) + e];
          const float p = POS    ? __builtin_amdgcn_exp2f(fmaf(x, c, -m_use))
                          : UCAP ? __builtin_amdgcn_exp2f(fmaf(-2.f * a.capL, x, a.capL - m_use))
                                 : __builtin_amdgcn_exp2f(x - m_use);
          pv[e] = p;
          acc += p;
        }
        psum[g] = acc;
        pb[g] = __builtin_convertvector(pv, f16x8);
      }
      return (psum[0] + psum[1]) + (psum[2] + psum[3]);
    };
    auto lane_max = [&]() -> float {
      if constexpr (UCAP) {
        float mn = INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) mn = fminf(mn, s[blk][r]);
        return fmaf(-2.f * a.capL, mn, a.capL);  // -inf when every score is masked
      }
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
      return mx;
    };
    auto rescale_to = [&](float m_new) {
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
      m_run = m_new;
    };
    // Without the built-in soft-cap the maximum moves rarely (ALiBi and score modifications
    // walked in descending key order), and the probabilities are formed against the running
    // maximum first (see below).
    if constexpr (!(POS || (ALIBI && !SOFTCAP)) || (MOD & kModMaxFirst) != 0) {
      const float mx = pair_max(lane_max());
      const float m_tile = POS ? mx * c : mx;
      if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kTau)) {
        keep_branch();
        rescale_to(fmaxf(m_run, m_tile));
      }
      l_run += probs(m_run == -INFINITY ? 0.f : m_run);
      return;
    }
    // A wave with a row that has no maximum yet (the first tiles of its rows) takes the tile
    // maximum first: probabilities formed against no maximum would only be formed again.
    const bool fresh = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    float lsum = 0.f;
    if (!fresh) lsum = probs(REL ? 0.f : m_run);
    if (fresh || __builtin_amdgcn_ballot_w64(!(lsum <= kPmax))) {
      keep_branch();
      // Tile row maximum: in-lane over 32 keys, then with the lane that shares the query.
      const float mx = pair_max(lane_max());
      rescale_to(fmaxf(m_run, REL ? m_ref + mx : POS ? mx * c : mx));
      lsum = probs(m_run == -INFINITY ? 0.f : REL ? m_run - m_ref : m_run);
    }
    l_run += lsum;
  };
  // kt of tiles k - 1 .. k + 3 are kept in scalars; tile k + 4's is read one iteration ahead.
  // Past the last tile they are 0 (a valid tile: its data is staged but never used).
  int kt_prev = 0, kt_cur = T > 0 ? kt_of(0) : 0, kt_next = T > 1 ? kt_of(1) : 0;
  int kt_n2 = T > 2 ? kt_of(2) : 0, kt_n3 = T > 3 ? kt_of(3) : 0;
  // FP8: the K scales of tiles k - 1 .. k + 1, each read (scalar load) an iteration before use.
  auto sk_of = [&](int kt) -> float {
    return FP8 ? ((const_f32 *)a.sk)[(size_t)bh * a.n_kt + kt] : 1.f;
  };
  float sk_prev = 1.f, sk_cur = sk_of(kt_cur), sk_next = sk_of(kt_next);
  auto advance = [&](int k) {
    const int kt_n4 = k + 4 < T ? kt_of(k + 4) : 0;
    const float sk_n2 = sk_of(kt_n2);
    kt_prev = kt_cur;
    kt_cur = kt_next;
    kt_next = kt_n2;
    kt_n2 = kt_n3;
    kt_n3 = kt_n4;
    sk_prev = sk_cur;
    sk_cur = sk_next;
    sk_next = sk_n2;
  };
  {
    // Buffer-to-LDS copies through NB LDS buffers (four; three for d = 256): buffer t mod NB
    // holds the pair (K_t, V^T_{t-1}), which is what the M-phase of iteration t reads.  In
    // iteration k every wave issues, between the MFMAs of its own M-phase, its share of the
    // copies of pair k + NB - 1 (K_{k+NB-1}, V^T_{k+NB-2}) into the buffer last read in
    // iteration k - 1.  Before the barrier in the middle of iteration k each wave waits for its
    // copies of pair k + 1 (issued in iteration k + 2 - NB; vmcnt counts the copies in issue
    // order), so after that barrier pair k + 1 is whole and the wave whose next M-phase reads
    // it issues that phase's first fragment reads at the end of its V-phase, across the next
    // barrier.  With four buffers the copies are in flight for more than an iteration; with
    // three, for about one.  Nothing else waits for them: the barriers inside the loop are bare
    // s_barrier instructions (a workgroup fence would wait for every copy).
    //
    // A tile row is SPK (K) or SPV (V^T) 16-byte slots, the last one padding; copy instruction
    // g of a pair fills slots 64 g .. 64 g + 63 of its buffer (K tile first).  Wave w issues
    // instructions w, w + 8, ...; one past the pair's count reads nothing and writes zeros to
    // the spare row.  Padding slots read the row's last chunk again (the same cache line as
    // their neighbour).
    constexpr int NDMA = (NJ + 7) / 8;
    const int wv = __builtin_amdgcn_readfirstlane(wave) & 7;  // the range lets most items resolve
    int dvo[NDMA];
#pragma unroll
    for (int r = 0; r < NDMA; ++r) {
      const int g = min(wv + 8 * r, NJ - 1);
      if (g < NJK) {
        const int sl = g * 64 + lane, row = sl / SPK, ch = sl % SPK;
        // LDS row `row` holds key pi(row) (pi is an involution)
        dvo[r] = pi_key(row) * KROW + min(ch, KCHR - 1) * 16;
      } else {
        const int sl = (g - NJK) * 64 + lane, row = sl / SPV, ch = sl % SPV;
        // < 2^31: row < DV, Npad <= 2^24 for DV = 64 and <= 2^23 for DV = 128 (attn_fwd's limits)
        dvo[r] = row * a.Npad * 2 + min(ch, VCH - 1) * 16;
      }
    }
    // Copy item r of pair (K tile ktk, V^T tile ktv) into buffer buf; vzero: write zeros in
    // place of the V^T tile.
    auto copy_item = [&](int r, uint16_t *buf, int ktk, int ktv, bool vzero) {
      const int g = wv + 8 * r;
      const int rows = min(kBc, N - ktk * kBc);
      const size_t left = ((size_t)(D - vcol0) * a.Npad - (size_t)ktv * kBc) * 2;
      const uint32_t vbytes = (uint32_t)(left < 0xFFFFFFFFull ? left : 0xFFFFFFFFull);
      const bool isk = g < NJK;
      const char *base = isk ? kbytes + (size_t)ktk * kBc * KROW
                             : (const char *)(vbase + (size_t)ktv * kBc);
      const uint32_t bytes = isk ? (uint32_t)(rows * KROW) : (g < NJ && !vzero) ? vbytes : 0u;
      copy16_to_lds(base, bytes, dvo[r], buf + min(g, NJ) * 512);
    };
    if constexpr (ATTN_RACE_CHECK) {
      constexpr int NW = (NJ + 1) * 512 / 2;  // 32-bit words per buffer
      for (int i = tid; i < NW; i += NT) {
        ((uint32_t *)sB0)[i] = 0x7FFF7FFFu;
        ((uint32_t *)sB1)[i] = 0x7FFF7FFFu;
        ((uint32_t *)sB2)[i] = 0x7FFF7FFFu;
        if constexpr (NB > 3) ((uint32_t *)sB3)[i] = 0x7FFF7FFFu;
      }
      __syncthreads();
    }
    // Pairs 0 (K_0 and a zero V^T_{-1}: P = 0 in the first M-phase) .. NB - 2.
#pragma unroll
    for (int r = 0; r < NDMA; ++r) copy_item(r, sB0, kt_cur, kt_cur, true);
#pragma unroll
    for (int r = 0; r < NDMA; ++r) copy_item(r, sB1, kt_next, kt_cur, false);
    if constexpr (NB > 3) {
#pragma unroll
      for (int r = 0; r < NDMA; ++r) copy_item(r, sB2, kt_n2, kt_next, false);
    }
    // Only pair 0 has to be whole before the loop (both groups' first M-phase and group 0's
    // first fragment reads use it); the loop's own waits cover pairs 1 and 2.  When every
    // workgroup starts at once, waiting for all three pairs would put the whole burst of
    // first loads in front of the first MFMA.  The copies are the only vector-memory
    // operations in flight here (the Q loads have been waited for).
    ring_wait<waitcnt_vm((NB - 2) * NDMA)>();
    ring_barrier();
    if (grp == 0) prefetch(sB0);

    // Iteration k with B = k mod NB and phase group G, every buffer named statically.
    auto iteration = [&](int k, auto bc, auto gc) {
      constexpr int B = decltype(bc)::value, G = decltype(gc)::value;
      uint16_t *rb = buf(IntC<B>{});                 // pair k
      uint16_t *nb = buf(IntC<(B + 1) % NB>{});      // pair k + 1
      uint16_t *wb = buf(IntC<(B + NB - 1) % NB>{});  // pair k + NB - 1
      auto item = [&](int r) {
        if constexpr (NB == 4)
          copy_item(r, wb, kt_n3, kt_n2, false);
        else
          copy_item(r, wb, kt_n2, kt_next, false);
      };
      auto mp = [&] {
        if constexpr (FP8)
          mphase_fp8(rb, rb + NJK * 512, item, IntC<NDMA>{});
        else
          mphase_bf16(rb, rb + NJK * 512, item, IntC<NDMA>{});
      };
      // Pair k + 1 was issued in iteration k + 2 - NB; the copies of the younger iterations
      // (and, in group 0, of this one) may stay in flight.
      if constexpr (G == 0) {
        mphase(mp);
        ring_wait<waitcnt_vm((NB - 2) * NDMA)>();
        ring_barrier();
        if (k < T) vphase(kt_cur, sk_cur);
        advance(k);
        prefetch(nb);
      } else {
        if (k >= 1) vphase(kt_prev, sk_prev);
        prefetch(rb);
        ring_wait<waitcnt_vm((NB - 3) * NDMA)>();
        ring_barrier();
        mphase(mp);
        advance(k);
      }
      ring_barrier();
    };
    auto run = [&](auto gc) {
      for (int k = 0;; k += NB) {
        iteration(k, IntC<0>{}, gc);
        if (k >= T) break;
        iteration(k + 1, IntC<1>{}, gc);
        if (k + 1 >= T) break;
        iteration(k + 2, IntC<2 % NB>{}, gc);
        if (k + 2 >= T) break;
        if constexpr (NB > 3) {
          iteration(k + 3, IntC<3 % NB>{}, gc);
          if (k + 3 >= T) break;
        }
      }
    };
    if (grp == 0)
      run(IntC<0>{});
    else
      run(IntC<1>{});
  }

  // Epilogue: O = O / l, L = (m + log2 l) * ln 2.
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    const size_t obase = ((size_t)bh * N + qrow) * D + vcol0 + 16 * hf;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x16 o = oacc[db] * inv;
      if constexpr (OUTF32) {
        float *op = (float *)a.o + obase + 32 * db;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(f32x4 *)(op + 4 * i) = f32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
      } else {
        uint16_t *op = (uint16_t *)a.o + obase + 32 * db;
        const f32x8 o0 = {o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]};
        const f32x8 o1 = {o[8], o[9], o[10], o[11], o[12], o[13], o[14], o[15]};
        *(bf16x8 *)op = __builtin_convertvector(o0, bf16x8);
        *(bf16x8 *)(op + 8) = __builtin_convertvector(o1, bf16x8);
      }
    }
    if (a.lse && hf == 0 && vcol0 == 0)
      a.lse[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------------
// Block table of a user mask (MOD & kModMask): the classes of the kernel's tiles, from the mask
// evaluated on every pair, and per tile a byte whose bit w says that rows 32w .. 32w + 31 of the
// tile are all in range and allowed against all its keys (the forward kernel's wave w then
// skips the element mask).  One workgroup of 256 threads per tile (kt, row = b * n_qt + qt);
// thread t tests query row qt * Br + t against the tile's 64 keys.  Class 0: no allowed
// in-range pair; 2: all Br * Bc pairs in range and allowed; 1: otherwise (the convention of the
// built-in table).
__device__ __forceinline__ void mod_class_body(const ModTableArgs &t) {
  __shared__ int flags[4][2];
  __shared__ int wfull[4];
  const int kt = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = row / t.n_qt, qt = row - b * t.n_qt;
  const int i = qt * kBr + tid;
  bool any = false, all = i < t.N;
  for (int jj = 0; jj < kBc; ++jj) {
    const int j = kt * kBc + jj;
    const bool ok = i < t.N && j < t.N && attn_mask_mod(b, i, j, t.params);
    any = any || ok;
    all = all && ok;
  }
  const uint64_t bany = __builtin_amdgcn_ballot_w64(any), bnot = __builtin_amdgcn_ballot_w64(!all);
  if (lane == 0) {
    flags[wave][0] = bany != 0;
    flags[wave][1] = bnot == 0;
    // the forward kernel's waves hold 32 rows: this wave's rows are its waves 2w and 2w + 1
    wfull[wave] = ((uint32_t)bnot == 0u ? 1 : 0) | ((bnot >> 32) == 0u ? 2 : 0);
  }
  __syncthreads();
  if (tid == 0) {
    const bool A = flags[0][0] | flags[1][0] | flags[2][0] | flags[3][0];
    const bool F = flags[0][1] & flags[1][1] & flags[2][1] & flags[3][1];
    t.cls[(size_t)row * t.n_kt + kt] = (int8_t)(A ? (F ? 2 : 1) : 0);
    t.wfull[(size_t)row * t.n_kt + kt] =
        (uint8_t)(wfull[0] | (wfull[1] << 2) | (wfull[2] << 4) | (wfull[3] << 6));
  }
}

// The per-row list of non-empty tiles (ascending kt, then zeros) and its count, from the
// classes: one workgroup of 256 threads per row, 256 tiles at a time, a ballot prefix per wave.
__device__ __forceinline__ void mod_list_body(const ModTableArgs &t) {
  __shared__ int wave_tot[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int8_t *crow = t.cls + (size_t)row * t.n_kt;
  int32_t *lrow = t.list + (size_t)row * t.n_kt;
  int base = 0;
  for (int c0 = 0; c0 < t.n_kt; c0 += 256) {
    const int kt = c0 + tid;
    const bool nz = kt < t.n_kt && crow[kt] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(nz);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(bal);
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      woff += w < wave ? wave_tot[w] : 0;
      tot += wave_tot[w];
    }
    if (nz) lrow[base + woff + pre] = kt;
    base += tot;
    __syncthreads();
  }
  for (int kt = base + tid; kt < t.n_kt; kt += 256) lrow[kt] = 0;
  if (tid == 0) t.cnt[row] = base;
}

}  // namespace
}  // namespace attn
