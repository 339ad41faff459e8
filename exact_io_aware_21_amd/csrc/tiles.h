// Closed-form block-mask predicates, compiled for both host and gfx950.
//
// Every mask kind here allows, for query row i, exactly the keys of one interval
// [lo(i), hi(i)] (intersected with [0, N)), and both ends are non-decreasing in i:
//   none     lo = 0                 hi = N - 1
//   causal   lo = 0                 hi = i
//   window   lo = max(0, i - W + 1) hi = i
//   document lo = start of doc(i)   hi = i
// That monotone-interval shape gives each tile's class from two rows only, instead of
// Br * Bc pair tests: a tile of rows R = [r0, rl] and keys C = [c0, cl] is
//   empty  iff no i in R has [lo(i), hi(i)] meeting C; for hi(i) = i the best candidate is
//          i* = max(r0, c0), so empty iff i* > rl or lo(i*) > cl;
//   full   iff the tile is wholly in range and lo(rl) <= c0 and hi(r0) >= cl.
// The block sparsity this feeds is the one named on page "El FlexAttention de PyTorch con
// FlashAttention-4 ..." (section "Limitaciones actuales").
#pragma once

#include "hipdefs.h"

namespace attn {

enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2, kMaskDocument = 3 };

// Tile shape of the forward kernel: Br query rows (8 waves x 32) and Bc keys per step.
constexpr int kBr = 256;
constexpr int kBc = 64;

struct MaskDesc {
  int kind;
  int N;
  int window;
  const int32_t *offs;  // this batch entry's offsets row (document mask only)
  int max_docs;
};

// offs[r] of the largest r in [0, max_docs] with offs[r] <= i (offs[0] = 0 for valid input).
// Reads only offs[0 .. max_docs].
__host__ __device__ inline int doc_start(const int32_t *offs, int max_docs, int i) {
  int lo = 0, hi = max_docs;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= i)
      lo = mid;
    else
      hi = mid - 1;
  }
  return offs[lo];
}

// offs[r + 1] for the same r as doc_start: the first index of the next document.
__host__ __device__ inline int doc_end(const int32_t *offs, int max_docs, int i) {
  int lo = 0, hi = max_docs;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= i)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo < max_docs ? offs[lo + 1] : offs[max_docs];
}

// The same interval seen from a key j: the queries that may attend to it are [col_lo, col_hi]
// (used by the backward pass, whose key-major kernel owns keys).
__host__ __device__ inline int col_lo(const MaskDesc &m, int j) {
  return m.kind == kMaskNone ? 0 : j;
}

__host__ __device__ inline int col_hi(const MaskDesc &m, int j) {
  switch (m.kind) {
    case kMaskWindow: {
      const long long x = (long long)j + m.window - 1;
      return x < m.N - 1 ? (int)x : m.N - 1;
    }
    case kMaskDocument: {
      const int e = doc_end(m.offs, m.max_docs, j);
      return (e < m.N ? e : m.N) - 1;
    }
    default:
      return m.N - 1;
  }
}

__host__ __device__ inline int row_lo(const MaskDesc &m, int i) {
  switch (m.kind) {
    case kMaskWindow: {
      long long x = (long long)i - m.window + 1;
      return x > 0 ? (int)x : 0;
    }
    case kMaskDocument:
      return doc_start(m.offs, m.max_docs, i);
    default:
      return 0;
  }
}

__host__ __device__ inline int row_hi(const MaskDesc &m, int i) {
  return m.kind == kMaskNone ? m.N - 1 : i;
}

// 0 empty, 1 partial, 2 full, for the tile of q-tile qt and k-tile kt.
__host__ __device__ inline int tile_class(const MaskDesc &m, int qt, int kt, int Br, int Bc) {
  const int N = m.N;
  const int r0 = qt * Br, c0 = kt * Bc;
  const int rl = (r0 + Br < N ? r0 + Br : N) - 1;
  const int cl = (c0 + Bc < N ? c0 + Bc : N) - 1;
  const bool in_full = (r0 + Br <= N) && (c0 + Bc <= N);
  if (m.kind == kMaskNone) return in_full ? 2 : 1;
  const int istar = r0 > c0 ? r0 : c0;
  if (istar > rl || row_lo(m, istar) > cl) return 0;
  if (in_full && row_lo(m, rl) <= c0 && row_hi(m, r0) >= cl) return 2;
  return 1;
}

// Fills one q-tile row of the table: cls[n_kt], list[n_kt] (ascending non-empty kt, then 0);
// returns the count.
__host__ __device__ inline int tile_row(const MaskDesc &m, int qt, int n_kt, int Br, int Bc,
                                        int8_t *cls, int32_t *list) {
  int c = 0;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k = tile_class(m, qt, kt, Br, Bc);
    cls[kt] = (int8_t)k;
    if (k) list[c++] = kt;
  }
  for (int kt = c; kt < n_kt; ++kt) list[kt] = 0;
  return c;
}

}  // namespace attn
