// Key range of a decode query, shared by the decode kernels.
#pragma once

#include "launch.h"

namespace hswa {

// Key range of sequence b: `len` keys, key t is cache row `row0 + t`.
// Returns false for a position the caller's contract rules out.
__device__ __forceinline__ bool key_range(const AttnArgs& a, int layout, int b, long long* p_out,
                                          long long* row0, long long* len) {
  const long long p = a.pos[b];
  *p_out = p;
  if (p < 0 || p > a.max_pos) return false;
  if (layout == 0) {  // ring: slots 0 .. min(p, W-1) hold tokens
    *row0 = (long long)b * a.window;
    *len = (p + 1 < a.window) ? p + 1 : a.window;
    return true;
  }
  const long long off = a.seq_offsets[b];
  const long long rows = a.seq_offsets[b + 1] - off;
  if (p >= rows) return false;
  const long long lo = (a.window > 0 && p - a.window + 1 > 0) ? p - a.window + 1 : 0;
  *row0 = off + lo;
  *len = p - lo + 1;
  return true;
}

}  // namespace hswa
