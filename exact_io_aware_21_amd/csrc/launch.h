// Internal launch interface between the C-ABI layer (api.cpp) and the kernels (fwd.hip).
#pragma once

#include "hipdefs.h"

#include "tiles.h"

namespace attn {

struct FwdArgs {
  const uint16_t *q;   // bf16 [BH][N][D]
  const uint16_t *k;   // bf16 [BH][N][D]
  const uint16_t *vt;  // bf16 [BH][D][Npad], key-contiguous, d rows permuted (see fwd.hip)
  const uint16_t *v;   // bf16 [BH][N][D]: read directly by the short-sequence kernel
  void *o;             // bf16 or fp32 [BH][N][D]
  float *lse;          // fp32 [BH][N] or null
  int B, H, N, Npad, n_qt, n_kt;
  float c;       // scale * log2(e): scores are kept in base-2 units
  float cap_c1;  // soft-cap: 2 * scale * log2(e) / cap
  float capL;    // soft-cap: cap * log2(e)
  const float *slopes;  // ALiBi slopes [H] or null
  int kind, window, max_docs;
  const int32_t *offs;   // [B][max_docs + 1] or null
  const int8_t *cls;     // block table (null for the unmasked kind)
  const int32_t *cnt;
  const int32_t *list;
  const uint8_t *k8;  // FP8 instances: K as E4M3 codes [BH][N][D]
  const float *sk;    // FP8 instances: K scales [BH][n_kt], one per 64-key tile
  float scale;               // runtime-compiled modifications: the natural-units score scale
  const float *mod_params;   // runtime-compiled modifications: the caller's parameters
  const uint8_t *wfull;      // runtime-compiled masks: per tile, the fully allowed 32-row blocks
};

// Block table of a runtime-compiled mask: cls [B][n_qt][n_kt], cnt [B][n_qt], list [B][n_qt][n_kt],
// wfull [B][n_qt][n_kt].
struct ModTableArgs {
  int N, n_qt, n_kt;
  const float *params;
  int8_t *cls;
  int32_t *cnt;
  int32_t *list;
  uint8_t *wfull;  // [B][n_qt][n_kt]
};

// Variant switches that select a kernel instance.
struct FwdInstance {
  int d;         // 64 or 128
  bool alibi;
  bool softcap;
  bool pos_scale;  // scale > 0 and no score modification: max is taken on raw scores
  bool out_f32;
  bool fp8;        // scores from E4M3 codes of Q (quantized in the kernel) and K (a.k8, a.sk)
};

// Backward pass (bwd.hip).
struct BwdArgs {
  const uint16_t *q, *k, *v, *dout;  // bf16 [BH][N][D]
  const void *o;                     // bf16 or fp32 [BH][N][D] (o_f32)
  const float *lse;                  // fp32 [BH][N], natural log
  float *dvec;                       // fp32 [BH][N]: D_i = dO_i . O_i
  void *dq, *dk, *dv;                // bf16 or fp32 [BH][N][D] (out_f32)
  int B, H, N, Npad, n_qt, n_kt;
  float scale;   // dQ = scale * dS K, dK = scale * dS^T Q
  float c;       // scale * log2(e)
  float cap_c1;  // soft-cap: 2 * scale * log2(e) / cap
  float capL;    // soft-cap: cap * log2(e)
  const float *slopes;
  int kind, window, max_docs;
  const int32_t *offs;
  const int32_t *cnt, *list;  // forward block table (null for the unmasked kind)
  bool o_f32, out_f32;
};

hipError_t launch_bwd_dot(const BwdArgs &a, int d, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs &a, int d, bool alibi, bool softcap, hipStream_t stream);

// Paged-cache decoding (decode.hip).
struct DecodeArgs {
  const uint16_t *q;                 // bf16 [B][H][Lq][D]
  const uint16_t *k_cache, *v_cache; // bf16 [n_pages][H][page][D]
  const int32_t *page_table;         // [B][max_pages]
  const int32_t *seq_lens;           // [B]
  void *o;                           // bf16 or fp32 [B][H][Lq][D]
  float *lse;                        // fp32 [B][H][Lq] or null
  float *part_o, *part_m, *part_l;   // split partials [B*H][nsplit][lq_pad]([D])
  int B, H, Lq, lq_pad, page, max_pages, n_pages, keys_per_split, nsplit, causal;
  float c;  // scale * log2(e)
};

hipError_t launch_decode(const DecodeArgs &a, int d, bool out_f32, hipStream_t stream);

// FP8 block quantization (fp8.hip): codes [BH][N][d] E4M3, scales [BH][ceil(N / rows)].
hipError_t launch_quant_fp8(const uint16_t *x, uint8_t *codes, float *scales, int BH, int N,
                            int d, int rows, hipStream_t stream);

// V [BH][N][d] bf16 -> V^T [BH][d][Npad] fp16 (saturating), keys contiguous, zero beyond N,
// d rows permuted within 32-blocks (sigma_d).
hipError_t launch_vt_pack(const uint16_t *v, uint16_t *vt, int BH, int N, int Npad, int d,
                          hipStream_t stream);
hipError_t launch_block_table(MaskDesc m, const int32_t *offs_all, int Bm, int n_qt, int n_kt,
                              int8_t *cls, int32_t *cnt, int32_t *list, hipStream_t stream);
hipError_t launch_fwd(const FwdInstance &inst, const FwdArgs &a, hipStream_t stream);
// Short sequences (short.hip): N <= kShortMaxN, d 64 or 128, bf16 operands; one launch, reads
// V directly (no V^T pack, no block table).
constexpr int kShortMaxN = 256;
hipError_t launch_fwd_short(const FwdInstance &inst, const FwdArgs &a, hipStream_t stream);
// The V^T pack and, when cls is not null, the block table (Bm * n_qt rows), in one launch.
hipError_t launch_prep(const uint16_t *v, uint16_t *vt, int BH, int N, int Npad, int d,
                       const MaskDesc &m, const int32_t *offs_all, int Bm, int n_qt, int n_kt,
                       int8_t *cls, int32_t *cnt, int32_t *list, hipStream_t stream);

}  // namespace attn
