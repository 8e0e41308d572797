// qi_common.h - internal definitions shared by the host helpers and the device kernels.
//
// The Block-Causal mask ("Qwen-Image-2.1" course overview, card 3C and the learning goals)
// has a per-row structure that the whole library relies on: because segments are contiguous
// and ordered (text, references, target last), a query q sees exactly the keys k <= lim(q),
// where lim(q) = q for a causal text token and lim(q) = (end of q's segment) - 1 for an image
// token or a bidirectional text token.  lim is non-decreasing in q, so for a tile of queries
// [q0, q1] and keys [k0, k1]: no pair is visible iff k0 > lim(q1), and every pair is visible
// iff k1 <= lim(q0).  Host tile maps and device tile skipping both use these two tests.
#pragma once

#include <stdint.h>

#include "qi.h"

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define QI_HD __host__ __device__ __forceinline__
#else
#define QI_HD inline
#endif

namespace qi {

// Segment table passed by value to the kernels (fits the kernel-argument segment).
struct SegTable {
  int32_t n;
  int32_t end[QI_MAX_SEG];        // exclusive end token of each segment
  uint8_t causal[QI_MAX_SEG];     // 1 = causal text segment
};

// Last visible key of query row q (global sequence index).
QI_HD int64_t row_limit(const SegTable& t, int64_t q) {
  int32_t start = 0;
  for (int s = 0; s < t.n; ++s) {
    if (q < t.end[s]) return t.causal[s] ? q : (int64_t)t.end[s] - 1;
    start = t.end[s];
  }
  (void)start;
  return q;  // past the layout: only itself (never reached for in-range rows)
}

// Tile class from the limits of the first and last query row of the tile and the key range
// [k0, k1) (k1 exclusive, already clamped to the number of keys): 0 skip, 1 full, 2 partial.
QI_HD int tile_class(int64_t lim_first, int64_t lim_last, int64_t k0, int64_t k1) {
  if (k0 > lim_last) return 0;
  if (k1 - 1 <= lim_first) return 1;
  return 2;
}

// Host-side analysis of a qi_layout.
struct LayoutInfo {
  int64_t S = 0, P = 0, T = 0;
  SegTable tab{};
};

// Validates a layout and fills `info`.  Returns QI_OK or a negative qi_status.
int analyse_layout(const qi_layout* L, LayoutInfo* info);

}  // namespace qi
