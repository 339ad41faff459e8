/*
 * attn.h -- C ABI of the MI355X (gfx950) FlashAttention library (libattn.so): the forward pass
 * (bf16, or FP8 scores with per-block scales), its backward pass, decoding over a paged
 * key/value cache, and forward passes with runtime-compiled score and mask modifications.
 *
 * What it computes.  For every batch entry b and head h, with Q, K, V in R^{N x d}:
 *     O = softmax(S) V,   S_ij = modified score of query i and key j,
 *     L_i = m_i + ln(l_i) (natural log), m_i = max_j S_ij, l_i = sum_j e^{S_ij - m_i},
 * exactly as the plain definition (page "FlashAttention/es", sections "Por qué la atención
 * estándar es lenta" and "El truco del softmax en línea"), evaluated by the tiled forward pass
 * with the online softmax (same page, section "El algoritmo FlashAttention"): Q is walked in
 * blocks of Br rows, K and V in blocks of Bc rows, the running maximum and normaliser stay in
 * registers, and no N x N matrix is ever written to device memory.  L is the log-sum-exp the
 * same section writes beside O.
 *
 * Score modifications and masks (named on page "El FlexAttention de PyTorch con
 * FlashAttention-4 ...", opening paragraph), applied in this order to s = scale * q_i . k_j:
 *     ATTN_MOD_SOFTCAP : s <- cap * tanh(s / cap)
 *     ATTN_MOD_ALIBI   : s <- s - slope[h] * (i - j)
 *     mask             : disallowed pairs get s = -inf
 * with the mask kind (low 4 bits of `variant`):
 *     ATTN_MASK_NONE            every key
 *     ATTN_MASK_CAUSAL          j <= i
 *     ATTN_MASK_SLIDING_WINDOW  i - window < j <= i
 *     ATTN_MASK_DOCUMENT        j <= i and doc(i) == doc(j), doc(x) = r with off[r] <= x < off[r+1]
 * Tiles of Br x Bc scores with no allowed pair are skipped entirely (block sparsity, page
 * "El FlexAttention ...", section "Limitaciones actuales"): a per-tile class table is built on
 * the device from the variant (see attn_block_table) and the kernel walks only non-empty tiles.
 *
 * Memory.  Every pointer is caller-owned device memory unless stated otherwise.  The library
 * allocates nothing on any call and keeps no per-call state; the only state it keeps is a
 * per-device cache of the architecture check.  The exceptions are the modification objects:
 * attn_mod_create allocates the compiled code in host memory, and the first attn_fwd_mod call
 * on a device loads it there; attn_mod_destroy releases both.  All launches are asynchronous on `stream`
 * (a hipStream_t, NULL = the default stream); a kernel fault surfaces at the caller's next
 * synchronisation.  Entry points are reentrant; calls that share a workspace must not overlap.
 *
 * Errors.  Every entry point returns an int (ATTN_OK or a negative code) and never throws.
 * All arguments are validated before any HIP call.  attn_strerror(code) names a code;
 * attn_last_error() returns a thread-local message naming the offending argument.
 * A device that is not gfx950 gives ATTN_ERR_UNSUPPORTED_DEVICE: there is no fallback path.
 * For tests, the environment variable ATTN_TEST_ARCH_OVERRIDE, if set when the library first
 * checks a device in a process, replaces the architecture name that device reports.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* variant bits */
enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_CAUSAL = 1,
  ATTN_MASK_SLIDING_WINDOW = 2,
  ATTN_MASK_DOCUMENT = 3, /* mask kind: bits 0-3 */
  ATTN_MOD_ALIBI = 1u << 4,
  ATTN_MOD_SOFTCAP = 1u << 5,
  ATTN_PREC_FP8 = 1u << 6 /* attn_fwd only: scores from FP8 E4M3 codes of Q and K, see attn_fwd */
};

/* return codes */
enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,        /* a pointer, size, alignment or variant field is invalid */
  ATTN_ERR_UNSUPPORTED_DEVICE = -2, /* no HIP device, or the current device is not gfx950 */
  ATTN_ERR_LAUNCH = -3,             /* a kernel launch was rejected by the runtime */
  ATTN_ERR_WORKSPACE = -4,          /* workspace missing, misaligned or smaller than needed */
  ATTN_ERR_COMPILE = -5             /* attn_mod_create: the modification did not compile */
};

/* output dtype of O */
enum { ATTN_O_BF16 = 0, ATTN_O_F32 = 1 };

typedef struct {
  int32_t window;              /* SLIDING_WINDOW: W >= 1; key j allowed iff i - W < j <= i */
  float softcap;               /* SOFTCAP: cap, finite and > 0 */
  const float *alibi_slopes;   /* ALIBI: device, H floats, finite; slope of head h */
  const int32_t *doc_offsets;  /* DOCUMENT: device, [B][max_docs + 1] int32, per batch entry
                                  0 = off[0] < off[1] < ... < off[n] = N, then padded with N.
                                  Contents are not validated: invalid offsets give unspecified
                                  values in O and L but no out-of-bounds access. */
  int32_t max_docs;            /* DOCUMENT: >= 1, row length of doc_offsets minus one */
  int32_t o_dtype;             /* ATTN_O_BF16 (default) or ATTN_O_F32 */
  void *workspace;             /* device, 256-byte aligned, >= attn_workspace_size() bytes */
  size_t workspace_bytes;
  void *const *timing_events;  /* optional instrumentation: NULL, or two caller-created
                                  hipEvent_t recorded on `stream` right before and right after
                                  the main forward kernel (not the transpose or table kernels) */
} attn_params;

/*
 * attn_fwd -- the forward pass.
 *   q, k, v : device, bf16, [B][H][N][d] row-major (d contiguous), 16-byte aligned.
 *   o       : device, [B][H][N][d], bf16 or fp32 per params->o_dtype, 16-byte aligned.
 *   lse     : device, fp32 [B][H][N], the natural-log L; NULL skips it.
 *   B, H, N : >= 1, N <= 2^24 (2^23 for d 128 and 256), B*H*ceil(N/Br) < 2^31.
 *   d       : 64, 128 or 256 (ATTN_PREC_FP8: 64 or 128).
 *   scale   : finite (1/sqrt(d) for the standard scaling).
 *   variant : one mask kind, optionally OR-ed with ATTN_MOD_ALIBI and/or ATTN_MOD_SOFTCAP, or
 *             with ATTN_PREC_FP8 (no score modification; B*H <= 65535).
 *   params  : required (it carries the workspace).
 * A query row with no allowed key (impossible for the masks above with valid arguments) gets
 * O = 0 and L = -inf.
 * Precision: Q K^T is formed from the bf16 inputs with fp32 accumulation; probabilities and V
 * enter the P V product as fp16 (V converted exactly for |v| in [2^-14, 65504]; larger
 * magnitudes saturate to +-65504), accumulated in fp32; l is summed from fp32 probabilities.
 * With ATTN_PREC_FP8 (page "FlashAttention/es", section "Variantes y sucesores": FP8 with
 * per-block scaling), Q and K are first block-quantized as attn_quantize_fp8 does, Q with
 * rows = Br (inside the forward kernel) and K with rows = Bc (into the workspace), and
 * S = scale * (s_q Q8)(s_k K8)^T is formed from the E4M3 codes with fp32 accumulation; V and
 * the P V product are as above.  Inputs must be finite.
 * Kernels: sequences of N <= 256 keys (d 64 or 128, bf16 operands) run, while the grid is
 * small, on a single-launch kernel that holds all keys of a head on chip and takes the exact
 * row maximum (the workspace is then unused); other shapes run the tiled kernel (V^T pack and
 * block table into the workspace, then the online softmax over key tiles).  Both are within
 * the precision above; they are not bit-identical to each other.  The environment variable
 * ATTN_FWD_PATH = "tiled" or "short", read at each call, forces one of them (for tests and
 * measurements); "short" on a shape that kernel does not take, or any other non-empty value,
 * gives ATTN_ERR_INVALID_ARG.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
             int d, float scale, uint32_t variant, const attn_params *params, void *stream);

/*
 * attn_fwd_noalloc -- attn_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same forward pass,
 * kernels and results, with the workspace taken from a static device array of
 * ATTN_NOALLOC_SCRATCH_BYTES bytes inside the library instead of params->workspace.
 *   Arguments, outputs and errors as attn_fwd; params is required, but its workspace and
 *   workspace_bytes fields are ignored.  A shape whose attn_workspace_size exceeds
 *   ATTN_NOALLOC_SCRATCH_BYTES is rejected with ATTN_ERR_WORKSPACE before any HIP call.
 *   The call allocates nothing: each device holds its own copy of the array from the library's
 *   load on it until the process ends, and its address is resolved once, on the device's first
 *   call.  Every call on a device uses that device's one array and nothing is carried between
 *   calls, so calls that can overlap on one device (other streams, other threads) race and must
 *   be serialised by the caller.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int attn_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                     int H, int N, int d, float scale, uint32_t variant,
                     const attn_params *params, void *stream);

/*
 * attn_workspace_size -- bytes of device workspace attn_fwd needs for this shape and variant
 * (0 on invalid arguments; no HIP call).  The caller allocates it once and passes it in
 * params->workspace, so that no call allocates: page "FlashAttention-3 y torch.compile ...",
 * section 6, item 2, explains that graph-captured execution forbids memory allocation during
 * the recorded run and that intermediate buffers must be allocated beforehand.  The workspace
 * holds a key-transposed fp16 copy of V ([B][H][d][ceil(N/Bc)*Bc]), the block table and, with
 * ATTN_PREC_FP8, the E4M3 codes of K ([B][H][N][d] bytes) and their scales (fp32
 * [B][H][ceil(N/Bc)]).  Its contents are scratch: rewritten by every call, never read across
 * calls.
 */
size_t attn_workspace_size(int B, int H, int N, int d, uint32_t variant);

/*
 * attn_tile_shape -- the tile shape (*Br query rows x *Bc keys) of the forward kernel for
 * (d, variant).  Page "FlashAttention/es", section "El algoritmo FlashAttention", cuts Q into
 * blocks of Br rows and K, V into blocks of Bc rows; page "El FlexAttention de PyTorch con
 * FlashAttention-4 ...", section "Limitaciones actuales", skips the blocks the mask empties.
 * The block table (attn_block_table) classifies exactly these tiles, so its contents are only
 * defined together with this shape.  d as for attn_fwd; Br, Bc are host pointers.
 * Returns ATTN_OK, or ATTN_ERR_INVALID_ARG (unsupported d, unknown variant bits, NULL output);
 * no HIP call.
 */
int attn_tile_shape(int d, uint32_t variant, int *Br, int *Bc);

/*
 * attn_block_table -- the per-tile class table attn_fwd builds and walks, written to caller
 * buffers (device).  With (Br, Bc) = attn_tile_shape(d, variant), n_qt = ceil(N/Br),
 * n_kt = ceil(N/Bc), Bm = B for ATTN_MASK_DOCUMENT and 1 otherwise:
 *   cls[Bm][n_qt][n_kt]     int8 : 0 no allowed in-range pair, 2 all Br*Bc pairs in range and
 *                                  allowed, 1 otherwise;
 *   kv_cnt[Bm][n_qt]        int32: number of tiles with class != 0 in the row;
 *   kv_list[Bm][n_qt][n_kt] int32: their kt in ascending order, then zeros.
 * H is unused (the mask does not depend on the head) but validated like attn_fwd's.
 * params may be NULL for NONE/CAUSAL; its workspace fields are ignored.
 */
int attn_block_table(int B, int H, int N, int d, uint32_t variant, const attn_params *params,
                     int8_t *cls, int32_t *kv_cnt, int32_t *kv_list, void *stream);

/* attn_block_table_host -- the same block table (page "El FlexAttention ...", section
   "Limitaciones actuales": tiles the mask empties are skipped) computed on the host by the same
   closed-form tile predicates the device uses, for checking without a GPU.  Arguments as
   attn_block_table, but params->doc_offsets and the three outputs are HOST pointers (caller
   owned, sized as there).  Returns ATTN_OK or ATTN_ERR_INVALID_ARG; no HIP call is made. */
int attn_block_table_host(int B, int H, int N, int d, uint32_t variant, const attn_params *params,
                          int8_t *cls, int32_t *kv_cnt, int32_t *kv_list);

/*
 * attn_bwd -- the backward pass (page "FlashAttention/es", section "Paso hacia atrás y
 * recomputación"): the gradients dQ, dK, dV of a loss whose gradient with respect to the
 * forward output O is dout, for the same (scale, variant, params) as the forward call.  S and P
 * are recomputed tile by tile from q, k and the saved log-sum-exp; no N x N matrix is stored.
 *   q, k, v : device, bf16, [B][H][N][d], 16-byte aligned (the forward inputs).
 *   o       : device, [B][H][N][d], the forward output, bf16 or fp32 per params->o_dtype.
 *   lse     : device, fp32 [B][H][N], the forward's natural-log L (required).
 *   dout    : device, bf16, [B][H][N][d], 16-byte aligned.
 *   dq, dk, dv : device outputs, [B][H][N][d], bf16 or fp32 per params->o_dtype, 16-byte
 *             aligned; every element is written (deterministically: no atomics).
 *   B, H, N, d, scale, variant : as for attn_fwd; additionally B*H <= 65535 and no
 *             ATTN_PREC_FP8 (the backward pass is bf16 only).
 *   params  : required; workspace of >= attn_bwd_workspace_size() bytes, 256-byte aligned.
 *             timing_events, if set, bracket the two main backward kernels.
 * Precision: all products are bf16 MFMAs with fp32 accumulation; P (<= 1) and dS are rounded
 * to bf16 as operands, D_i = dO_i . O_i is formed in fp32 from the given o.
 * Returns ATTN_OK or an error code; no HIP call is made for invalid arguments.
 */
int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dout, void *dq, void *dk, void *dv, int B, int H, int N, int d,
             float scale, uint32_t variant, const attn_params *params, void *stream);

/* Bytes of workspace attn_bwd needs (0 on invalid arguments): D (fp32 [B][H][N]) and, for the
   masked kinds, the block table. */
size_t attn_bwd_workspace_size(int B, int H, int N, int d, uint32_t variant);

/*
 * attn_quantize_fp8 -- the block quantization of the FP8 forward pass (page "FlashAttention/es",
 * section "Variantes y sucesores": FP8 with per-block scaling; page "FlashAttention-3 y
 * torch.compile ...", section "FlashAttention-3: Asincronía y Explotación del Silicio Hopper":
 * a scale estimated from the data at run time).  For each (b, h) and block of `rows` rows:
 *     scale = amax / 448 (float32; 1 for an all-zero block),  code = E4M3(x / scale)
 * with a correctly rounded float32 division and round-to-nearest-even to E4M3 (no infinities,
 * largest finite 448).
 *   x      : device, bf16 [B][H][N][d], 16-byte aligned.
 *   codes  : device, uint8 [B][H][N][d] E4M3, 16-byte aligned.
 *   scales : device, fp32 [B][H][ceil(N / rows)].
 *   B*H <= 65535, 1 <= N <= 2^24, d 64 or 128, rows 1..4096.
 * attn_fwd with ATTN_PREC_FP8 applies the same quantization to Q (rows = Br, inside the forward
 * kernel) and to K (rows = Bc, into its workspace).
 */
int attn_quantize_fp8(const void *x, uint8_t *codes, float *scales, int B, int H, int N, int d,
                      int rows, void *stream);

/*
 * attn_decode -- attention of the last Lq positions of each sequence over a paged key/value
 * cache (decoding).  Page "FlashAttention/es", section "Variantes y sucesores", names
 * PagedAttention: at inference the cache is cut into pages shared by many sequences.  The
 * result is the plain attention of the definition above over each sequence's keys and values
 * in position order, computed by split-KV: each workgroup forms a partial (m, l, O) over a range
 * of positions with the online softmax (section "El truco del softmax en línea"), and a second
 * kernel merges the partials of a (sequence, head) with the same identity.
 *   q          : device, bf16 [B][H][Lq][d], 16-byte aligned; row i of sequence b is position
 *                seq_lens[b] - Lq + i.
 *   k_cache, v_cache : device, bf16 [n_pages][H][page_size][d], 16-byte aligned.  Position t
 *                of sequence b is slot t % page_size of page page_table[b][t / page_size].
 *   page_table : device, int32 [B][max_pages], page indices in [0, n_pages).
 *   seq_lens   : device, int32 [B], lengths in [Lq, max_pages * page_size].
 *   o          : device, [B][H][Lq][d], bf16 or fp32 per params->o_dtype, 16-byte aligned.
 *   lse        : device, fp32 [B][H][Lq], natural-log L; NULL skips it.
 *   B, H       : >= 1, B*H <= 65535.   Lq : 1..8.   d : 64 or 128.
 *   page_size  : a power of two in [256 / (d / 8), 4096] (16 for d = 128, 32 for d = 64).
 *   max_pages  : >= 1, max_pages * page_size <= 2^24.   n_pages : >= 1.
 *   scale      : finite.
 *   variant    : ATTN_MASK_CAUSAL (query i sees positions <= seq_lens[b] - Lq + i) or
 *                ATTN_MASK_NONE (every position < seq_lens[b]); no score modifications.
 *   params     : required; workspace of >= attn_decode_workspace_size() bytes, 256-byte
 *                aligned; o_dtype; timing_events, if set, bracket the two decode kernels.
 * Device data is not validated: page indices outside [0, n_pages) are clamped into it and
 * lengths into [0, max_pages * page_size] (wrong values, no out-of-bounds access); a query row
 * with no allowed position gets O = 0 and L = -inf.
 * Precision: fp32 scores and accumulation from the bf16 inputs; O rounded once at the end.
 * Returns ATTN_OK or an error code; no HIP call is made for invalid arguments.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *page_table, const int32_t *seq_lens, void *o, float *lse, int B,
                int H, int Lq, int d, int page_size, int max_pages, int n_pages, float scale,
                uint32_t variant, const attn_params *params, void *stream);

/* Bytes of workspace attn_decode needs (0 on invalid arguments): the split partials, fp32
   [B*H][n_split][Lq rounded up to 1, 2, 4 or 8] x (d + 2). */
size_t attn_decode_workspace_size(int B, int H, int Lq, int d, int page_size, int max_pages);

/*
 * attn_strerror -- a static, NUL-terminated English name of a return code ("unknown error code"
 * for values not listed above); never NULL, never freed by the caller.
 * attn_last_error -- a thread-local, NUL-terminated message naming the argument or condition
 * behind the last error this thread received ("" if none); valid until the thread's next call.
 * Errors are reported and never hidden behind another code path: page "Hugging Face Reduce el
 * Exceso de Atención ..." warns that an attention dispatcher which silently falls back to an
 * unfused path for an unsupported head size or dtype is only found with a profiler, and page
 * "FlashAttention-3 y torch.compile ...", section 6, item 3, asks for a capability check on the
 * device instead of a crash.  So an unsupported shape is ATTN_ERR_INVALID_ARG and a device that
 * is not gfx950 is ATTN_ERR_UNSUPPORTED_DEVICE, each with its message, before any launch.
 */
const char *attn_strerror(int code);
const char *attn_last_error(void);

/*
 * Runtime-compiled score and mask modifications.  Page "El FlexAttention de PyTorch con
 * FlashAttention-4 ..." (opening paragraph): FlexAttention lets the user write the score
 * modification and the mask as small functions that are compiled into the attention kernel.
 * Here they are HIP C++ device functions, compiled with hipRTC into the same forward kernel the
 * fixed variants use (its tiles, block-sparse skip and online softmax):
 *     __device__ float attn_score_mod(float s, int b, int h, int i, int j, const float *p);
 *         the score of query i and key j of batch entry b, head h, from the scaled score
 *         s = scale * q_i . k_j (natural units); p = the caller's mod_params;
 *     __device__ bool attn_mask_mod(int b, int i, int j, const float *p);
 *         whether key j is allowed for query i (the same for every head; a head-dependent
 *         mask can return -INFINITY from attn_score_mod instead, without tile skipping).
 * The source defines the ones named by `flags` and may hold other device code.
 */
typedef struct attn_mod_s attn_mod;
enum { ATTN_MODF_SCORE = 1, ATTN_MODF_MASK = 2, ATTN_MODF_MAX_FIRST = 4 };
/*
 * ATTN_MODF_MAX_FIRST is a performance hint, not a change of the result: by default a kernel
 * with a score modification walks each query tile's key tiles from the last to the first and
 * forms the probabilities against the running row maximum, taking a tile's maximum only when
 * a probability sum shows that the maximum moved (cheap when the modification adds a bias that
 * favours near keys, as ALiBi does).  With the flag it walks them in ascending order and takes
 * every tile's maximum first, which is cheaper when the modification moves the maximum often
 * (a soft-cap, say).  Both orders give the same attention up to the rounding order.
 */

/*
 * attn_mod_create -- compiles `source` (NUL-terminated) for head dimension d (64, 128 or 256)
 * and the functions named by flags (ATTN_MODF_SCORE and/or ATTN_MODF_MASK, optionally with
 * ATTN_MODF_MAX_FIRST) into a gfx950 code
 * object held by *out (host memory; each device loads it on first use).  Needs no GPU.
 * log (optional, log_size bytes) receives the compiler's messages, NUL-terminated.
 * Returns ATTN_OK, ATTN_ERR_INVALID_ARG or ATTN_ERR_COMPILE (*out = NULL).
 */
int attn_mod_create(const char *source, uint32_t flags, int d, attn_mod **out, char *log,
                    size_t log_size);

/* Releases a modification and its loaded code (NULL is ignored).  Not while a call using it
   is being enqueued; kernels already launched keep running. */
void attn_mod_destroy(attn_mod *m);

/* Bytes of workspace attn_fwd_mod needs (0 on invalid arguments): the key-transposed V and,
   with a mask, the block table ([B][ceil(N/Br)] rows of ceil(N/Bc) tiles). */
size_t attn_mod_workspace_size(const attn_mod *m, int B, int H, int N);

/*
 * attn_fwd_mod -- the forward pass with a runtime-compiled modification: O = softmax(S) V and
 * L as for attn_fwd, with S_ij = attn_score_mod(scale * q_i . k_j, b, h, i, j, p) (or the scaled
 * score without ATTN_MODF_SCORE) and S_ij = -inf where attn_mask_mod(b, i, j, p) is false.
 *   q, k, v, o, lse, B, H, N, scale : as for attn_fwd, d = the mod's d; with a mask
 *             additionally B * ceil(N/Br) <= 65535.
 *   mod_params : device pointer (4-byte aligned) passed to the functions as p; may be NULL if
 *             they do not read it.  Not validated.
 *   params  : required: workspace (>= attn_mod_workspace_size bytes, 256-byte aligned),
 *             o_dtype, timing_events (bracket the forward kernel); other fields are ignored.
 * With a mask, the call first evaluates attn_mask_mod on every (i, j) to classify the tiles
 * (the attn_block_table classes, per batch entry) and skips the empty ones; on partial tiles it
 * evaluates the mask per element.  A row with no allowed key gets O = 0, L = -inf.
 * Precision as attn_fwd (the score function runs in fp32).
 */
int attn_fwd_mod(const attn_mod *m, const void *q, const void *k, const void *v, void *o,
                 float *lse, int B, int H, int N, float scale, const float *mod_params,
                 const attn_params *params, void *stream);

/*
 * attn_fwd_mod_cached -- attn_fwd_mod without the tile classification: it walks the block table
 * an earlier attn_fwd_mod call left in the same workspace.  The table depends only on the mask,
 * B, N and the values mod_params held when it was built (not on q, k, v, H or the score
 * function), so a caller that repeats a masked forward pass with new inputs (every layer of a
 * model, every training step) classifies once.  Arguments and errors as attn_fwd_mod; the
 * caller guarantees that the last attn_fwd_mod call on this workspace used this mod, this B
 * and N, and mod_params of the same values, and that nothing has written the workspace's table
 * since.  Otherwise the table is stale: O and L follow that table (allowed tiles it classes
 * empty are skipped, tiles it classes full are not masked), with no out-of-bounds access as
 * long as B and N are those of the build.  Without a mask it is attn_fwd_mod.
 */
int attn_fwd_mod_cached(const attn_mod *m, const void *q, const void *k, const void *v, void *o,
                        float *lse, int B, int H, int N, float scale, const float *mod_params,
                        const attn_params *params, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
