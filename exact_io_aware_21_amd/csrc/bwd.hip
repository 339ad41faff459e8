// gfx950 kernels of the attention backward pass.
//
// Page "FlashAttention/es" (marovi.ai), section "Paso hacia atrás y recomputación": the backward
// pass does not read a stored attention matrix; it recomputes S and P tile by tile from the saved
// log-sum-exp L and the output gradient dO.  With P_ij = exp(s_ij - L_i) recomputed:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D) with D_i = dO_i . O_i,
//   dT = dS * (1 - tanh^2) under the soft-cap,  dQ = scale * dT K,  dK = scale * dT^T Q.
// Two kernels, both deterministic (no atomics; every output element is written by one lane):
//  * bwd_dkdv_kernel owns keys: 4 waves x 32 keys per workgroup; it walks the query steps
//    (32 rows) that the mask allows for its keys and accumulates dK^T and dV^T in registers.
//  * bwd_dq_kernel owns queries: 8 waves x 32 rows = one forward q-tile; it walks that q-tile's
//    non-empty key tiles from the forward block table and accumulates dQ^T in registers.
// Both recompute S and dP, so the score and dP products run twice; in exchange no partial dQ is
// ever summed across workgroups.
//
// gfx950 mapping (same devices as the forward kernel, see fwd.hip):
//  * Every product is a v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Q, K, V, dO are the
//    exact bf16 inputs; P (<= 1) and dS are rounded to bf16 as MFMA operands.
//  * The recomputed tile is built so that its lane owns one row of the output being accumulated:
//    in bwd_dkdv_kernel S = Q K^T (A = Q rows from LDS, B = K^T of the wave's keys in VGPRs), so
//    lane % 32 is a key; in bwd_dq_kernel S^T = K Q^T, so lane % 32 is a query.
//  * The rows of the LDS tiles are stored with index bits 2 and 3 swapped (pi_key), which makes
//    the 16 accumulator registers of a lane two runs of 8 consecutive rows: P and dS then feed the
//    next product as its B operand straight from registers.  Within each block of 16, the tile
//    rows are placed in LDS by lds_row, which keeps the transposing reads free of bank conflicts.
//  * The other operand of those products (Q^T, dO^T for dK, dV; K^T for dQ) is read from the
//    same row tiles with the transposing LDS read ds_read_b64_tr_b16, with its columns in the
//    sigma_d order, so each lane's accumulator registers are 16 consecutive output columns and
//    the epilogue stores 16-byte vectors.  No transposed copy of any input is made.
//  * The row tiles are copied straight from global memory into LDS (buffer loads with the LDS
//    destination), double-buffered one step or tile ahead, with no VGPR staging; rows past N lie
//    outside the buffer resource and read as zero.
#include "kcommon.h"
#include "launch.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// D_i = sum_c dO_ic O_ic (fp32).  One group of D/8 lanes per row, 16-byte loads.
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row
  constexpr int RPB = 256 / LPR;
  const size_t rows = (size_t)a.B * a.H * a.N;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int ch = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 g = *(const u32x4 *)(a.dout + row * D + ch * 8);
    float of[8];
    if (a.o_f32) {
      const f32x4 o0 = *(const f32x4 *)((const float *)a.o + row * D + ch * 8);
      const f32x4 o1 = *(const f32x4 *)((const float *)a.o + row * D + ch * 8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        of[e] = o0[e];
        of[4 + e] = o1[e];
      }
    } else {
      const u32x4 ob = *(const u32x4 *)((const uint16_t *)a.o + row * D + ch * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        of[2 * w] = __uint_as_float(ob[w] << 16);
        of[2 * w + 1] = __uint_as_float(ob[w] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(__uint_as_float(g[w] << 16), of[2 * w], acc);
      acc = fmaf(__uint_as_float(g[w] & 0xFFFF0000u), of[2 * w + 1], acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && ch == 0) a.dvec[row] = acc;
}

// Stores one lane's 16 consecutive fp32 output columns (bf16 or fp32 output).
template <bool OUTF32>
__device__ __forceinline__ void store16(void *out, size_t off, const f32x16 &o) {
  if constexpr (OUTF32) {
    float *op = (float *)out + off;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(f32x4 *)(op + 4 * i) = f32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  } else {
    uint16_t *op = (uint16_t *)out + off;
    const f32x8 o0 = {o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]};
    const f32x8 o1 = {o[8], o[9], o[10], o[11], o[12], o[13], o[14], o[15]};
    *(bf16x8 *)op = __builtin_convertvector(o0, bf16x8);
    *(bf16x8 *)(op + 8) = __builtin_convertvector(o1, bf16x8);
  }
}

// Score of one (query i, key j) pair from its raw dot product x, in base-2 units, and the factor
// d s / d t of the soft-cap (1 - tanh^2; 1 without it).  The ALiBi distance j - i comes as a
// float (exact: |j - i| < 2^24), which callers form as a per-tile base plus a compile-time
// offset.
template <bool ALIBI, bool SOFTCAP>
__device__ __forceinline__ float score2f(const BwdArgs &a, float x, float slopeL, float dji,
                                         float &dcap) {
  float t;
  if constexpr (SOFTCAP) {
    const float e = __builtin_amdgcn_exp2f(x * a.cap_c1);
    t = fmaf(-2.f * a.capL, __builtin_amdgcn_rcpf(1.f + e), a.capL);
    const float th = t / a.capL;
    dcap = 1.f - th * th;
  } else {
    t = x * a.c;
    dcap = 1.f;
  }
  if constexpr (ALIBI) t = fmaf(slopeL, dji, t);
  return t;
}

// ---------------------------------------------------------------------------------------------
// Buffer-to-LDS copy of two equally laid-out tiles (byte size `bytes` each, from x and y) into
// dst: wave instruction j (j = wave + NW r < NJ) fills the 64 16-byte slots j * 64 .. j * 64 + 63
// of the first tile and the same slots of the second, which starts NJ * 64 slots later, from
// per-lane byte offsets voff[r].  Loads past `bytes` read as zero.  (A free device function: the
// copy builtin must not sit in a lambda, which the host compilation pass also instantiates.)
template <int NR, int NJ, int NW>
__device__ __forceinline__ void copy_tiles_to_lds(const void *x, const void *y, int bytes,
                                                  uint16_t *dst, int wave, const int *voff) {
  typedef __attribute__((address_space(3))) void lds_void;
  const auto rx = __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, bytes, kBufferWord3);
  const auto ry = __builtin_amdgcn_make_buffer_rsrc((void *)y, 0, bytes, kBufferWord3);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int j = r * NW + wave;
    if (j < NJ) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)&dst[j * 64 * 8], 16, voff[r], 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (lds_void *)&dst[(NJ + j) * 64 * 8], 16,
                                               voff[r], 0, 0, 0);
    }
  }
}

// Buffer-to-LDS copy of two 4-byte-per-lane rows (bytes each, from x and y) into dst and
// dst + 128 elements (64 floats each); loads past `bytes` read as zero.
__device__ __forceinline__ void copy_rows4_to_lds(const float *x, const float *y, int bytes,
                                                  uint16_t *dst, int voff) {
  typedef __attribute__((address_space(3))) void lds_void;
  const auto rx = __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, bytes, kBufferWord3);
  const auto ry = __builtin_amdgcn_make_buffer_rsrc((void *)y, 0, bytes, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)dst, 4, voff, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (lds_void *)&dst[128], 4, voff, 0, 0, 0);
}

// Where tile row rho sits in LDS: bits 0-1 and bits 2-3 of the row index swapped (an involution
// that keeps every aligned block of 16 rows in place).  A transposing read of 32 lanes covers
// the same 64-byte column span of four rows whose indices differ in bits 0-1; with a pitch of
// 272 bytes (d = 128) or 144 bytes (d = 64), rows 4 apart start 16 banks apart modulo the 64
// banks, so stored 4 apart the four spans take all 64 banks once (stored adjacent they overlapped
// 4-fold at d = 128, 2-fold at d = 64).  The 16 rows a ds_read_b128 phase reads stay the 16 rows
// of one block, which start at 16 distinct 4-bank groups, as before.
__device__ __forceinline__ int lds_row(int rho) {
  return (rho & ~15) | ((rho & 3) << 2) | ((rho >> 2) & 3);
}

// Per-lane byte offset of 16-byte slot `slot` of a tile of pi-permuted rows (pitch P elements,
// P / 8 slots a row) of a row-major [rows][D] bf16 source: tile row rho, stored at LDS row
// lds_row(rho), holds source row pi_key(rho); a pad slot repeats the row's last chunk; slots
// past the tile read row 0.
template <int D, int P, int ROWS>
__device__ __forceinline__ int tile_slot_offset(int slot) {
  constexpr int SPR = P / 8;
  static_assert(ROWS % 16 == 0, "lds_row permutes whole blocks of 16 rows");
  if (slot >= ROWS * SPR) return 0;
  const int row = lds_row(slot / SPR), ch = slot % SPR;
  return (pi_key(row) * D + (ch < D / 8 ? ch : D / 8 - 1) * 8) * 2;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposed A fragment of a 32x32x16 MFMA from an LDS tile of pi-permuted rows (pitch P):
// lane l gets, for output row dd = l % 32 (column 32 d0 + sigma_d(dd) of the tile) and
// k = 8 (l / 32) + t, t = 0..7, the element of tile row 16 kg + 8 (l / 32) + t (before the
// permutation).  ds_read_b64_tr_b16 hands lane 16 g + 4 q + e, for m = 0..3, element e of the
// 8 bytes addressed by lane 16 g + q + 4 m, so the addressing lane s = 16 g + q + 4 m points at
// row 16 kg + 8 (g / 2) + m (+ 4 for t = 4..7) and column 32 d0 + 16 (q & 1) + 8 (g & 1) +
// 4 (q >> 1).  tr_base() is the lane's part; kg and d0 add the immediate 16 kg P + 32 d0
// (lds_row moves rows only within their block of 16).
template <int P>
__device__ __forceinline__ void tr_base(int lane, int off[2]) {
  const int q = lane & 3, m = (lane >> 2) & 3, g = lane >> 4;
  const int col = 16 * (q & 1) + 8 * (g & 1) + 4 * (q >> 1);
#pragma unroll
  for (int u = 0; u < 2; ++u) off[u] = lds_row(pi_key(8 * (g >> 1) + m + 4 * u)) * P + col;
}

__device__ __forceinline__ u32x4 tr_frag(const uint16_t *tile, const int off[2], int imm) {
  const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)&tile[off[0] + imm]);
  const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)&tile[off[1] + imm]);
  return __builtin_bit_cast(u32x4, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------------------------
// Block placement of a (position, head) grid, gridDim = (n_pos, B*H): for causal and document
// masks longest position first across small groups of heads (see place_block; head_bytes are
// the two row arrays one head's blocks stream, 4 N d bytes), otherwise the natural order.
__device__ __forceinline__ void block_place(int kind, int N, int d, int &pos, int &bh) {
  if (kind == kMaskCausal || kind == kMaskDocument) {
    const int nx = gridDim.x;
    place_block(blockIdx.y * nx + blockIdx.x, nx * gridDim.y, nx, true, (size_t)4 * N * d, pos,
                bh);
  } else {
    bh = blockIdx.y;
    pos = blockIdx.x;
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV for d = 64: one workgroup = 4 waves x 32 keys of one (batch, head); query steps of 32
// rows.
//
// Each query step's Q and dO rows (32 pi-permuted rows of pitch RP each) and its L and D are
// copied straight into LDS (buffer-to-LDS loads) one step ahead, double-buffered, one copy for
// the workgroup (21 KB); the transposed operands Q^T and dO^T of the dK and dV products are read
// from the same row tiles with ds_read_b64_tr_b16.  Two workgroups fit a CU (two waves per SIMD),
// whose interleaving hides the wait at the barrier that ends every step.
template <int D, bool ALIBI, bool SOFTCAP, bool OUTF32>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NT = 256, NW = 4, QS = 32, KPW = 32;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int RP = pitch(D);                    // LDS pitch of a Q / dO row
  constexpr int RSLOT = QS * (RP / 8);            // 16-byte slots of a row tile
  constexpr int NJR = (RSLOT + 63) / 64;          // wave instructions per row tile
  constexpr int TILE = NJR * 64 * 8;              // elements per row tile (with the spill-over)
  constexpr int STAGE = 2 * TILE + 2 * 64 * 2;    // Q, dO, then L and D (64 floats each)
  constexpr int NRR = (NJR + NW - 1) / NW;        // copy instructions per wave and tile
  static_assert(D == 64, "d = 128 runs bwd_dkdv2_kernel");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: LDS copy targets
  int kx, bh;
  block_place(a.kind, a.N, D, kx, bh);  // key blocks: the first ones see the most queries
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N;
  const int key0 = kx * (NW * KPW);
  const int j = key0 + wave * KPW + l32;  // this lane's key
  const bool j_ok = j < N;
  const MaskDesc md{a.kind, N, a.window, a.offs ? a.offs + (size_t)b * (a.max_docs + 1) : nullptr,
                    a.max_docs};
  int qlo = 1, qhi = 0;  // queries allowed to attend to key j (empty past N)
  if (j_ok) {
    qlo = col_lo(md, j);
    qhi = col_hi(md, j);
  }
  // Query steps the workgroup visits: the union over its keys (both bounds grow with j).
  // (wave-uniform: read into scalars, so the loop below is a scalar loop)
  const int jl = min(key0 + NW * KPW, N) - 1;
  const int qs_begin = __builtin_amdgcn_readfirstlane(col_lo(md, key0) / QS);
  const int qs_end = __builtin_amdgcn_readfirstlane(col_hi(md, jl) / QS + 1);

  const size_t hbase = (size_t)bh * N * D;
  const float slopeL = ALIBI ? a.slopes[h] * kLog2e : 0.f;
  bf16x8 kf[NKS], vf[NKS];  // B operands: K^T and V^T of this lane's key
  {
    const size_t off = hbase + (size_t)(j_ok ? j : 0) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (j_ok) {
        x = *(const u32x4 *)(a.k + off + ks * 16);
        y = *(const u32x4 *)(a.v + off + ks * 16);
      }
      kf[ks] = __builtin_bit_cast(bf16x8, x);
      vf[ks] = __builtin_bit_cast(bf16x8, y);
    }
  }
  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dkt[i] = dvt[i] = f32x16{};

  // Zero every stage once, so that no LDS byte is ever read unwritten.
  for (int i = tid; i < (int)(sizeof(lds) / 16); i += NT) *(u32x4 *)&lds[i * 8] = u32x4{0u, 0u, 0u, 0u};
  uint16_t *const stages = lds;
  int voff[NRR];  // copy instruction r of a tile: r * NW + wave
#pragma unroll
  for (int r = 0; r < NRR; ++r) voff[r] = tile_slot_offset<D, RP, QS>(64 * (r * NW + wave) + lane);
  auto fill = [&](int qs, int stage) {
    const int q0 = qs * QS;
    // rows of this step (0 past the last step: the copies read nothing), so that the tiles'
    // byte count stays far below 2^31 for every N
    const int rows_left = min(max(N - q0, 0), QS);
    uint16_t *dst = &stages[stage * STAGE];
    copy_tiles_to_lds<NRR, NJR, NW>(a.q + hbase + (size_t)q0 * D, a.dout + hbase + (size_t)q0 * D,
                                    rows_left * D * 2, dst, wave, voff);
    // L and D of the 32 queries: one 4-byte-per-lane copy each (lanes 32..63 land in the unused
    // upper half of the 64-float slot).
    if (wave == 0)
      copy_rows4_to_lds(a.lse + (size_t)bh * N + q0, a.dvec + (size_t)bh * N + q0, max(N - q0, 0) * 4,
                        &dst[2 * TILE], lane * 4);
  };
  int tro[2];
  tr_base<RP>(lane, tro);
  // A step's LDS operands: the A fragments of the score products S = Q K^T (k-step i, i < NKS)
  // and dP = dO V^T (k-step i - NKS), the transposed A fragments of dV^T += dO^T P and
  // dK^T += Q^T dS (16-query half kk, d block d0; dK when odd), and L and D.  They are read at
  // the end of the step before, while its dK products run, so every MFMA of a step finds its
  // operands in registers.
  constexpr int NA = 2 * NKS, NB = 4 * NDB;
  u32x4 fb[NB], fa[NA];
  f32x4 l2v[4], dv4[4];
  auto load_ops = [&](int stage) {
    const uint16_t *sQ = &stages[stage * STAGE];
    const uint16_t *sDO = sQ + TILE;
    const float *sL = (const float *)(sQ + 2 * TILE);
    const float *sDv = sL + 64;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      fa[i] = *(const u32x4 *)&(i < NKS ? sQ : sDO)[lds_row(l32) * RP + hf * 8 + (i % NKS) * 16];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int kk = i / (2 * NDB), d0 = (i >> 1) % NDB;
      fb[i] = tr_frag((i & 1) ? sQ : sDO, tro, 16 * kk * RP + 32 * d0);
    }
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const int base = 16 * (aa >> 1) + 8 * hf + 4 * (aa & 1);
      l2v[aa] = *(const f32x4 *)&sL[base];
      dv4[aa] = *(const f32x4 *)&sDv[base];
    }
  };
  // Settle the loads above and the zero fill before the first copy lands.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (qs_begin < qs_end) fill(qs_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  load_ops(0);

  for (int qs = qs_begin; qs < qs_end; ++qs) {
    const int q0 = qs * QS, stage = (qs - qs_begin) & 1;
    // One wave runs per SIMD, so the step is ordered for the wave to overlap its own vector
    // work with its own MFMAs: all of S first (while the copies of the next step are issued),
    // then the dP products while the probabilities (which need only S) are formed; then the dV
    // products (which need only P) while dS is formed, then the dK products while the next
    // step's operands are read.  sched_group_barrier pins that interleave.  The copies of the
    // next step are issued between the score MFMAs (past the last step they read nothing and
    // fill the unused stage with zeros).
    fill(qs + 1, stage ^ 1);
    // S and dP: accumulator register r (row 8(r/4) + 4 hf + r%4 of the pi-permuted tile) is
    // query q0 + 16(r/8) + 8 hf + r%8, column = key j.
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i < NKS)
        s = mfma32(__builtin_bit_cast(bf16x8, fa[i]), kf[i], s);
      else
        dp = mfma32(__builtin_bit_cast(bf16x8, fa[i]), vf[i - NKS], dp);
    }
    float p[16], ds[16], dc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int aa = r >> 2, bb = r & 3;
      // key - query distance: the step's base plus this register's offset, exact in float
      const float dji = (float)(j - q0 - 8 * hf) - (float)(16 * (aa >> 1) + 4 * (aa & 1) + bb);
      const float t = score2f<ALIBI, SOFTCAP>(a, s[r], slopeL, dji, dc[r]);
      p[r] = __builtin_amdgcn_exp2f(fmaf(-kLog2e, l2v[aa][bb], t));  // L is natural-log
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i < NKS) __builtin_amdgcn_sched_group_barrier(0x020, 3, 0);  // copy instructions
      if (i >= NKS) __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // vector ALU
    }
    // Element mask only when some key of this wave does not take all 32 queries of the step.
    if (__builtin_amdgcn_ballot_w64(!(qlo <= q0 && qhi >= q0 + QS - 1))) {
      keep_branch();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int aa = r >> 2, bb = r & 3;
        const int i = q0 + 16 * (aa >> 1) + 8 * hf + 4 * (aa & 1) + bb;
        if (i < qlo || i > qhi) p[r] = 0.f;
      }
    }
    bf16x8 pb[2], db[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p[8 * kk + e];
      pb[kk] = __builtin_convertvector(x, bf16x8);
    }
    // dV^T += dO^T P over the 32 queries (two 16-row halves), while dS is formed.
#pragma unroll
    for (int i = 0; i < NB; i += 2) {
      const int kk = i / (2 * NDB), d0 = (i >> 1) % NDB;
      dvt[d0] = mfma32(__builtin_bit_cast(bf16x8, fb[i]), pb[kk], dvt[d0]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = p[r] * (dp[r] - dv4[r >> 2][r & 3]) * dc[r];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f32x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = ds[8 * kk + e];
      db[kk] = __builtin_convertvector(y, bf16x8);
    }
    // dK^T += Q^T dS.
#pragma unroll
    for (int i = 1; i < NB; i += 2) {
      const int kk = i / (2 * NDB), d0 = (i >> 1) % NDB;
      dkt[d0] = mfma32(__builtin_bit_cast(bf16x8, fb[i]), db[kk], dkt[d0]);
    }
    // The next step's operands: its copies (issued at the top of this step) have landed; after
    // the barrier every wave's have, and every wave is done reading this stage (which the
    // copies at the top of the next step overwrite).  After the last step the reads fetch unused
    // data from the other stage.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    load_ops(stage ^ 1);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // the P conversions
#pragma unroll
    for (int i = 0; i < NB / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
#pragma unroll
    for (int i = 0; i < NB / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, (NA + NB + 8) / (NB / 2) + 1, 0);
    }
  }

  if (j_ok) {
    const size_t off = hbase + (size_t)j * D + 16 * hf;
#pragma unroll
    for (int d0 = 0; d0 < NDB; ++d0) {
      store16<OUTF32>(a.dk, off + 32 * d0, dkt[d0] * a.scale);
      store16<OUTF32>(a.dv, off + 32 * d0, dvt[d0]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV for d = 128 with two waves per SIMD: one workgroup = 8 waves = 4 pairs x 32 keys of one
// (batch, head).  Waves w and w + 4 (pair w % 4) share the keys; per 32-query step, role 0 forms
// S = Q K^T, P and dV^T += dO^T P, role 1 forms dP = dO V^T, dS and dK^T += Q^T dS: 16 MFMAs each.
// P (with the soft-cap factor) goes from role 0 to role 1 through LDS.  In the single-wave form
// (bwd_dkdv_kernel, d = 64) one wave issues all 32 MFMAs of a step and every vector and LDS
// instruction itself; here two waves share a SIMD, so one issues while the other waits, and role
// 0's exponentials run beside its own dV products of the step before and beside role 1's
// products.  The products, and the order in which each accumulator sums them, are those of the
// single-wave form.
// The workgroup shares the steps' Q, dO, L, D tiles in three LDS stages (one array each, so the
// compiler tracks the copies into each separately; one copy of each tile per workgroup, where
// private stages per wave took four), filled two steps ahead; each stage also holds the P of its
// step.  Each role runs its own loop with one barrier per step: role 0 after writing P, role 1
// after its dP products, both after waiting for their own copies.  Barrier s therefore orders:
// P of step s written before it is read; step s + 1's tiles landed before they are read; the last
// reads of step s - 1's stage (the dV operands of role 0 and the dK operands of role 1, both
// before barrier s) before the copies of step s + 2 (issued after barrier s) overwrite it.
template <int D, bool ALIBI, bool SOFTCAP, bool OUTF32>
__global__ __launch_bounds__(512) void bwd_dkdv2_kernel(BwdArgs a) {
  constexpr int NT = 512, NPAIR = 4, QS = 32, KPW = 32;
  constexpr int NKS = D / 16, NDB = D / 32;     // k-steps of the score products; d blocks
  constexpr int RP = pitch(D);                  // LDS pitch of a Q / dO row
  constexpr int RSLOT = QS * (RP / 8);          // 16-byte slots of a row tile
  constexpr int NJR = (RSLOT + 63) / 64;        // wave instructions per row tile
  constexpr int TILE = NJR * 64 * 8;            // elements per row tile (with the spill-over)
  constexpr int NRR = (NJR + 7) / 8;            // copy instructions per wave and tile (at most)
  constexpr int XF = SOFTCAP ? 2 : 1;           // vectors role 0 sends: P, the soft-cap factor
  constexpr int XOFF = 2 * TILE + 2 * 64 * 2;   // Q, dO, then L and D (64 floats each), then P
  constexpr int STAGE = XOFF + NPAIR * XF * 1024 * 2;  // P: [pair][vector][4 groups][64 lanes][4]
  static_assert(D == 128, "the paired kernel is written for d = 128");
  __shared__ __attribute__((aligned(16))) uint16_t st0[STAGE], st1[STAGE], st2[STAGE];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: LDS copy targets
  const int pair = wave & 3, role = wave >> 2;
  int kx, bh;
  block_place(a.kind, a.N, D, kx, bh);  // key blocks: the first ones see the most queries
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N;
  const int key0 = kx * (NPAIR * KPW);
  const int j = key0 + pair * KPW + l32;  // this lane's key
  const bool j_ok = j < N;
  const MaskDesc md{a.kind, N, a.window, a.offs ? a.offs + (size_t)b * (a.max_docs + 1) : nullptr,
                    a.max_docs};
  int qlo = 1, qhi = 0;  // queries allowed to attend to key j (empty past N)
  if (j_ok) {
    qlo = col_lo(md, j);
    qhi = col_hi(md, j);
  }
  const int jl = min(key0 + NPAIR * KPW, N) - 1;
  const int qs_begin = __builtin_amdgcn_readfirstlane(col_lo(md, key0) / QS);
  const int qs_end = __builtin_amdgcn_readfirstlane(col_hi(md, jl) / QS + 1);

  const size_t hbase = (size_t)bh * N * D;
  const float slopeL = ALIBI ? a.slopes[h] * kLog2e : 0.f;
  bf16x8 bop[NKS];  // B operand: K^T (role 0) or V^T (role 1) of this lane's key
  {
    const uint16_t *src = (role ? a.v : a.k) + hbase + (size_t)(j_ok ? j : 0) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j_ok) x = *(const u32x4 *)(src + ks * 16);
      bop[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  f32x16 acc4[NDB];  // dV^T (role 0) or dK^T (role 1), column block d0
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc4[i] = f32x16{};

  // Zero the stages once, so that no LDS byte is ever read unwritten.
  for (int i = tid; i < STAGE / 8; i += NT) {
    *(u32x4 *)&st0[i * 8] = u32x4{0u, 0u, 0u, 0u};
    *(u32x4 *)&st1[i * 8] = u32x4{0u, 0u, 0u, 0u};
    *(u32x4 *)&st2[i * 8] = u32x4{0u, 0u, 0u, 0u};
  }
  int voff[NRR];
#pragma unroll
  for (int r = 0; r < NRR; ++r) voff[r] = tile_slot_offset<D, RP, QS>(64 * (r * 8 + wave) + lane);
  auto fill = [&](int qs, uint16_t *dst) __attribute__((always_inline)) {
    const int q0 = qs * QS;
    // rows of this step, so that the tiles' byte count stays far below 2^31 for every N
    // (read into scalars: the buffer descriptors they enter must be wave-uniform)
    const int rows = __builtin_amdgcn_readfirstlane(min(max(N - q0, 0), QS));
    const int left = __builtin_amdgcn_readfirstlane(max(N - q0, 0));
    copy_tiles_to_lds<NRR, NJR, 8>(a.q + hbase + (size_t)q0 * D, a.dout + hbase + (size_t)q0 * D,
                                   rows * D * 2, dst, wave, voff);
    // L and D of the 32 queries (lanes 32..63 land in the unused upper half of each slot)
    if (wave == 0)
      copy_rows4_to_lds(a.lse + (size_t)bh * N + q0, a.dvec + (size_t)bh * N + q0, left * 4,
                        &dst[2 * TILE], lane * 4);
  };
  int tro[2];
  tr_base<RP>(lane, tro);
  auto stage = [&](auto sc) __attribute__((always_inline)) -> uint16_t * {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return st0;
    else if constexpr (S == 1) return st1;
    else return st2;
  };
  // This lane's slot of vector v of the pair's P block (conflict-free 16-byte writes and reads).
  auto xslot = [&](uint16_t *st, int v, int g) __attribute__((always_inline)) -> float * {
    return (float *)&st[XOFF] + ((pair * XF + v) * 4 + g) * 256 + lane * 4;
  };
  // The score-product operand rows (Q for role 0, dO for role 1) of a stage, k-step ks:
  // accumulator register r (row 8(r/4) + 4 hf + r%4 of the pi-permuted tile) is query
  // q0 + 16(r/8) + 8 hf + r%8, column = key j.
  auto scores = [&](const uint16_t *rows) __attribute__((always_inline)) -> f32x16 {
    const uint16_t *ra = rows + lds_row(l32) * RP + hf * 8;
    u32x4 fa[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) fa[ks] = *(const u32x4 *)(ra + ks * 16);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = mfma32(__builtin_bit_cast(bf16x8, fa[ks]), bop[ks], acc);
    return acc;
  };
  // acc4[d0] += X^T F over the 32 queries (two 16-row halves kk), X = dO (role 0) or Q (role 1).
  auto accumulate = [&](const uint16_t *x, const bf16x8 (&f)[2]) __attribute__((always_inline)) {
    u32x4 fb[2][NDB];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int d0 = 0; d0 < NDB; ++d0) fb[kk][d0] = tr_frag(x, tro, 16 * kk * RP + 32 * d0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int d0 = 0; d0 < NDB; ++d0)
        acc4[d0] = mfma32(__builtin_bit_cast(bf16x8, fb[kk][d0]), f[kk], acc4[d0]);
  };
  auto to_bf16 = [&](const float (&v)[16], bf16x8 (&o)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = v[8 * kk + e];
      o[kk] = __builtin_convertvector(x, bf16x8);
    }
  };
  // Each wave's copies landed, then the barrier (with the workgroup fence: the P writes before
  // it, the P reads after it); then the copies of step qs + 2.
  auto sync_and_fill = [&](int qs, uint16_t *next) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (qs + 2 < qs_end) fill(qs + 2, next);
  };

  // Role 0, step qs from stage S: S, then dV of step qs - 1 (its stage, the one before S, is
  // overwritten only by the copies after this step's barrier) while P is formed and written to
  // the stage's P block.  pbp holds the previous step's P in bf16; before the first step it is
  // zero and the stage before is the zero-filled st2, so that first product adds exact zeros.
  bf16x8 pbp[2] = {};
  auto step0 = [&](int qs, auto sc) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    uint16_t *st = stage(IntC<S>{});
    const float *sL = (const float *)(st + 2 * TILE);
    const int q0 = qs * QS;
    const f32x16 acc = scores(st);
    accumulate(stage(IntC<(S + 2) % 3>{}) + TILE, pbp);  // dV^T += dO^T P, step qs - 1
    f32x4 l2v[4];
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) l2v[aa] = *(const f32x4 *)&sL[16 * (aa >> 1) + 8 * hf + 4 * (aa & 1)];
    float p[16], dc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int aa = r >> 2, bb = r & 3;
      // key - query distance: the step's base plus this register's offset, exact in float
      const float dji = (float)(j - q0 - 8 * hf) - (float)(16 * (aa >> 1) + 4 * (aa & 1) + bb);
      const float t = score2f<ALIBI, SOFTCAP>(a, acc[r], slopeL, dji, dc[r]);
      p[r] = __builtin_amdgcn_exp2f(fmaf(-kLog2e, l2v[aa][bb], t));  // L is natural-log
    }
    // Element mask only when some key of this wave does not take all 32 queries of the step.
    if (__builtin_amdgcn_ballot_w64(!(qlo <= q0 && qhi >= q0 + QS - 1))) {
      keep_branch();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int aa = r >> 2, bb = r & 3;
        const int i = q0 + 16 * (aa >> 1) + 8 * hf + 4 * (aa & 1) + bb;
        if (i < qlo || i > qhi) p[r] = 0.f;
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      *(f32x4 *)xslot(st, 0, g) = f32x4{p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
      if constexpr (SOFTCAP)
        *(f32x4 *)xslot(st, XF - 1, g) = f32x4{dc[4 * g], dc[4 * g + 1], dc[4 * g + 2], dc[4 * g + 3]};
    }
    to_bf16(p, pbp);
    sync_and_fill(qs, stage(IntC<(S + 2) % 3>{}));
  };
  // Role 1, step qs from stage S: dP, the barrier, then dS (with the P role 0 wrote) and dK.
  auto step1 = [&](int qs, auto sc) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    uint16_t *st = stage(IntC<S>{});
    const float *sDv = (const float *)(st + 2 * TILE) + 64;
    const f32x16 dp = scores(st + TILE);
    sync_and_fill(qs, stage(IntC<(S + 2) % 3>{}));
    float ds[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 pv = *(const f32x4 *)xslot(st, 0, g);
      const f32x4 dv4 = *(const f32x4 *)&sDv[16 * (g >> 1) + 8 * hf + 4 * (g & 1)];
      f32x4 dc = {1.f, 1.f, 1.f, 1.f};
      if constexpr (SOFTCAP) dc = *(const f32x4 *)xslot(st, XF - 1, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[4 * g + e] = pv[e] * (dp[4 * g + e] - dv4[e]) * dc[e];
    }
    bf16x8 db[2];
    to_bf16(ds, db);
    accumulate(st, db);  // dK^T += Q^T dS
  };

  // Settle the loads above and the zero fill before the first copies land.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (qs_begin < qs_end) fill(qs_begin, st0);
  if (qs_begin + 1 < qs_end) fill(qs_begin + 1, st1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Whole triples of steps in the loop (one exit, so the accumulators stay in place), then the
  // last one or two steps.
  int qs = qs_begin;
  if (role == 0) {
    for (; qs + 3 <= qs_end; qs += 3) {
      step0(qs, IntC<0>{});
      step0(qs + 1, IntC<1>{});
      step0(qs + 2, IntC<2>{});
    }
    // dV of the last step, from its stage (no copies follow it)
    if (qs + 1 < qs_end) {
      step0(qs, IntC<0>{});
      step0(qs + 1, IntC<1>{});
      accumulate(st1 + TILE, pbp);
    } else if (qs < qs_end) {
      step0(qs, IntC<0>{});
      accumulate(st0 + TILE, pbp);
    } else if (qs_begin < qs_end) {
      accumulate(st2 + TILE, pbp);
    }
  } else {
    for (; qs + 3 <= qs_end; qs += 3) {
      step1(qs, IntC<0>{});
      step1(qs + 1, IntC<1>{});
      step1(qs + 2, IntC<2>{});
    }
    if (qs < qs_end) step1(qs, IntC<0>{});
    if (qs + 1 < qs_end) step1(qs + 1, IntC<1>{});
  }

  if (j_ok) {
    const size_t off = hbase + (size_t)j * D + 16 * hf;
#pragma unroll
    for (int d0 = 0; d0 < NDB; ++d0) {
      if (role)
        store16<OUTF32>(a.dk, off + 32 * d0, acc4[d0] * a.scale);
      else
        store16<OUTF32>(a.dv, off + 32 * d0, acc4[d0]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dQ: one workgroup = 8 waves x 32 queries = one forward q-tile; it walks the q-tile's list of
// non-empty 64-key tiles (the forward block table).
//
// The K and V tiles are double-buffered in LDS and filled by buffer-to-LDS loads
// (buffer_load_dwordx4 ... lds): no VGPR staging, and the loads of tile t + 1 are in flight
// while tile t is computed.  One LDS stage holds the K tile then the V tile, each 64
// pi-permuted key rows of pitch KP placed by lds_row, as 16-byte slots; a wave instruction fills 64 consecutive
// slots, and a wave fills slot group j of both tiles (same offsets).  A pad slot repeats a real
// chunk of its row; keys past N lie beyond the K and V resources and read as zero.
// K^T, the A operand of dQ^T += K^T dS^T, is read from the same K tile with the transposing
// LDS read ds_read_b64_tr_b16.
template <int D, bool ALIBI, bool SOFTCAP, bool OUTF32>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NT = 512;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int KP = pitch(D);          // LDS pitch of a K / V row
  constexpr int KSPR = KP / 8;          // 16-byte slots per LDS row
  constexpr int KSLOT = kBc * KSPR;     // slots of one tile
  constexpr int NJK = KSLOT / 64;       // wave instructions per tile
  constexpr int NRK = (NJK + 7) / 8;    // slot groups per wave (at most)
  constexpr int STAGE = 2 * KSLOT * 8;  // elements per LDS stage
  static_assert(kBr == 256 && kBc == 64, "kernel is written for 256 x 64 tiles");
  static_assert(KSLOT % 64 == 0, "tiles must be whole wave instructions");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  // wave-uniform by construction; readfirstlane tells the compiler, so the LDS destinations of
  // the buffer-to-LDS copies (M0) are scalars
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int qx, bh;
  block_place(a.kind, a.N, D, qx, bh);
  const int b = bh / a.H, h = bh - b * a.H;
  // q-tiles: the last ones see the most keys
  const int qt = (a.kind == kMaskCausal || a.kind == kMaskDocument) ? a.n_qt - 1 - qx : qx;
  const int N = a.N;
  const int qrow = qt * kBr + wave * 32 + l32;
  const bool q_ok = qrow < N;
  const MaskDesc md{a.kind, N, a.window, a.offs ? a.offs + (size_t)b * (a.max_docs + 1) : nullptr,
                    a.max_docs};
  int lo = 1, hi = 0;  // empty interval for rows past N
  if (q_ok) {
    lo = row_lo(md, qrow);
    hi = row_hi(md, qrow);
  }
  const size_t hbase = (size_t)bh * N * D;
  bf16x8 qf[NKS], df[NKS];  // B operands: Q^T and dO^T of this lane's query
  {
    const size_t off = hbase + (size_t)(q_ok ? qrow : 0) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (q_ok) {
        x = *(const u32x4 *)(a.q + off + ks * 16);
        y = *(const u32x4 *)(a.dout + off + ks * 16);
      }
      qf[ks] = __builtin_bit_cast(bf16x8, x);
      df[ks] = __builtin_bit_cast(bf16x8, y);
    }
  }
  const float l2 = q_ok ? a.lse[(size_t)bh * N + qrow] * kLog2e : 0.f;
  const float dq_row = q_ok ? a.dvec[(size_t)bh * N + qrow] : 0.f;
  const float slopeL = ALIBI ? a.slopes[h] * kLog2e : 0.f;

  // The key-tile list (written by the table kernel before this launch): read through the
  // constant address space, i.e. with scalar loads, so the loop below is wave-uniform.
  int T;
  const_i32 *lst = nullptr;
  if (a.list) {
    const int bm = (a.kind == kMaskDocument) ? b : 0;
    const size_t row = (size_t)bm * a.n_qt + qt;
    T = ((const_i32 *)a.cnt)[row];
    lst = (const_i32 *)a.list + row * a.n_kt;
  } else {
    T = a.n_kt;
  }
  auto kt_of = [&](int t) -> int { return lst ? lst[t] : t; };

  // Zero both stages once, so that no LDS byte is ever read unwritten (keys past N may read as
  // stale finite data or zero; their probabilities are masked to 0 either way).
  for (int i = tid; i < 2 * STAGE / 8; i += NT) *(u32x4 *)&lds[i * 8] = u32x4{0u, 0u, 0u, 0u};

  // Per-lane byte offsets of this wave's slot groups j = wave + 8 r (the same in K and V).
  int voff[NRK];
#pragma unroll
  for (int r = 0; r < NRK; ++r) {
    const int slot = 64 * (r * 8 + wave) + lane;
    const int row = lds_row(slot / KSPR), ch = slot % KSPR;
    voff[r] = (pi_key(row) * D + (ch < D / 8 ? ch : D / 8 - 1) * 8) * 2;
  }
  auto fill = [&](int kt, int stage) {
    const int keys_left = min(N - kt * kBc, kBc);  // keys of this tile, >= 1
    const size_t off = hbase + (size_t)kt * kBc * D;
    copy_tiles_to_lds<NRK, NJK, 8>(a.k + off, a.v + off, keys_left * D * 2, &lds[stage * STAGE],
                                wave, voff);
  };

  // Transposing-read addresses for the K^T fragments.  ds_read_b64_tr_b16 hands lane
  // 16 g + 4 q + e, for m = 0..3, element e of the 8 bytes addressed by lane 16 g + q + 4 m.  So
  // for the A fragment (row = d block row dd = lane % 32, whose output column is
  // 32 d0 + sigma_d(dd); k = key 16 kg + 8 (lane / 32) + t, t = 0..7) the addressing lane
  // s = 16 g + q + 4 m points at key 16 kg + 8 (g / 2) + m (+ 4 for t = 4..7) and at column
  // 32 d0 + 16 (q & 1) + 8 (g & 1) + 4 (q >> 1); kg and d0 are immediate offsets.
  int tr_off[2];
  {
    const int q = lane & 3, m = (lane >> 2) & 3, g = lane >> 4;
    const int col = 16 * (q & 1) + 8 * (g & 1) + 4 * (q >> 1);
#pragma unroll
    for (int u = 0; u < 2; ++u) tr_off[u] = lds_row(pi_key(8 * (g >> 1) + m + 4 * u)) * KP + col;
  }
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

  f32x16 dqt[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqt[i] = f32x16{};

  __syncthreads();  // the zero fill is complete before any copy lands
  if (T > 0) fill(kt_of(0), 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const int kt = kt_of(t), stage = t & 1;
    if (t + 1 < T) fill(kt_of(t + 1), stage ^ 1);  // in flight during this tile's compute
    const uint16_t *sK = &lds[stage * STAGE];
    const uint16_t *sV = sK + KSLOT * 8;

    // S^T = K Q^T and dP^T = V dO^T: register r of key block blk is key
    // kt*Bc + 32*blk + 16*(r/8) + 8*hf + r%8, column = query qrow.
    f32x16 s[2] = {}, dp[2] = {};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint16_t *ka = &sK[(32 * blk + lds_row(l32)) * KP + hf * 8];
      const uint16_t *va = &sV[(32 * blk + lds_row(l32)) * KP + hf * 8];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        s[blk] = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4 *)(ka + ks * 16)), qf[ks], s[blk]);
        dp[blk] =
            mfma32(__builtin_bit_cast(bf16x8, *(const u32x4 *)(va + ks * 16)), df[ks], dp[blk]);
      }
    }
    // P^T overwrites S^T in place.
    float dc[2][16];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // key - query distance: the tile's base plus this register's offset, exact in float
        const float dji = (float)(kt * kBc + 8 * hf - qrow) + (float)(32 * blk + 16 * (r >> 3) + (r & 7));
        const float tt = score2f<ALIBI, SOFTCAP>(a, s[blk][r], slopeL, dji, dc[blk][r]);
        s[blk][r] = __builtin_amdgcn_exp2f(tt - l2);
      }
    // Element mask only when some row of this wave does not allow all 64 keys of the tile.
    if (__builtin_amdgcn_ballot_w64(!(lo <= kt * kBc && hi >= kt * kBc + kBc - 1))) {
      keep_branch();
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = kt * kBc + 32 * blk + 16 * (r >> 3) + 8 * hf + (r & 7);
          if (jj < lo || jj > hi) s[blk][r] = 0.f;
        }
    }
    bf16x8 db[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int blk = g >> 1, r = 8 * (g & 1) + e;
        y[e] = s[blk][r] * (dp[blk][r] - dq_row) * dc[blk][r];
      }
      db[g] = __builtin_convertvector(y, bf16x8);
    }
    // dQ^T += K^T dS^T over the 64 keys (four 16-key steps); K^T fragments by transposing
    // reads of the K tile.
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int d0 = 0; d0 < NDB; ++d0) {
        const int imm = 16 * g * KP + 32 * d0;
        const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)&sK[tr_off[0] + imm]);
        const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)&sK[tr_off[1] + imm]);
        const v8i16 x = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        dqt[d0] = mfma32(__builtin_bit_cast(bf16x8, x), db[g], dqt[d0]);
      }
    // This wave's copies of tile t + 1 have landed; after the barrier every wave's have, and
    // every wave is done reading this stage (the next iteration's copies overwrite it).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (q_ok) {
    const size_t off = hbase + (size_t)qrow * D + 16 * hf;
#pragma unroll
    for (int d0 = 0; d0 < NDB; ++d0) store16<OUTF32>(a.dq, off + 32 * d0, dqt[d0] * a.scale);
  }
}

template <int D, bool ALIBI, bool SOFTCAP, bool OUTF32>
hipError_t launch_bwd_inst(const BwdArgs &a, hipStream_t s) {
  const unsigned BH = (unsigned)(a.B * a.H);
  if constexpr (D == 128)
    bwd_dkdv2_kernel<D, ALIBI, SOFTCAP, OUTF32>
        <<<dim3((unsigned)((a.N + 127) / 128), BH), 512, 0, s>>>(a);
  else
    bwd_dkdv_kernel<D, ALIBI, SOFTCAP, OUTF32>
        <<<dim3((unsigned)((a.N + 127) / 128), BH), 256, 0, s>>>(a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  bwd_dq_kernel<D, ALIBI, SOFTCAP, OUTF32><<<dim3((unsigned)a.n_qt, BH), 512, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, bool ALIBI, bool SOFTCAP>
hipError_t launch_bwd_out(const BwdArgs &a, hipStream_t s) {
  return a.out_f32 ? launch_bwd_inst<D, ALIBI, SOFTCAP, true>(a, s)
                   : launch_bwd_inst<D, ALIBI, SOFTCAP, false>(a, s);
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs &a, bool alibi, bool softcap, hipStream_t s) {
  if (alibi && softcap) return launch_bwd_out<D, true, true>(a, s);
  if (alibi) return launch_bwd_out<D, true, false>(a, s);
  if (softcap) return launch_bwd_out<D, false, true>(a, s);
  return launch_bwd_out<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_bwd_dot(const BwdArgs &a, int d, hipStream_t stream) {
  const size_t rows = (size_t)a.B * a.H * a.N;
  const int rpb = 256 / (d / 8);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (d == 128)
    bwd_dot_kernel<128><<<grid, 256, 0, stream>>>(a);
  else
    bwd_dot_kernel<64><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs &a, int d, bool alibi, bool softcap, hipStream_t stream) {
  if (d == 128) return launch_bwd_d<128>(a, alibi, softcap, stream);
  return launch_bwd_d<64>(a, alibi, softcap, stream);
}

}  // namespace attn
