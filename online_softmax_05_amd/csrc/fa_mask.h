// Position masks of the general kernels: causal alignment and sliding
// windows ([GS] "How Does FlashAttention Preserve Global Softmax Across
// Tiles?", section 6: zero-based positions, bottom-right or top-left
// alignment, and the same alignment rule for sliding windows).
//
// Query row i sits at key position pos = i + off, where off = Nk - Nq when
// the ENDS of the two sequences line up (bottom-right) and off = 0 when
// their starts do (top-left).  Row i may see key j iff
//     j < klen,   j >= pos - wl  (if wl >= 0),   j <= pos + wr  (if wr >= 0).
// A causal mask is the right width wr = 0 (intersected with any wider right
// window), so the kernels carry one (off, wl, wr) triple.  Both ends of the
// visible range [key_lo(i), key_end(i)) are non-decreasing in i, which is what
// lets a block of consecutive rows skip whole key tiles at both ends.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct KeyRange {
  int off;  // pos - i
  int wl;   // left width, < 0: unbounded
  int wr;   // right width, < 0: unbounded (0 for causal)
};

// first visible key of row i (may exceed klen: then the row is empty)
__device__ __forceinline__ int key_lo(const KeyRange& m, int i) {
  if (m.wl < 0) return 0;
  const long long x = (long long)i + m.off - m.wl;
  return x < 0 ? 0 : (int)x;
}

// one past the last visible key of row i, in [0, klen]
__device__ __forceinline__ int key_end(const KeyRange& m, int i, int klen) {
  if (m.wr < 0) return klen;
  const long long x = (long long)i + m.off + m.wr + 1;
  return x <= 0 ? 0 : (x < klen ? (int)x : klen);
}

}  // namespace fa
