// host_common.hpp -- argument checks shared by the C-ABI entry points.  They
// run on the host before any HIP call, so a rejected call has no effect.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nvfp4kv.h"

namespace nvfp4 {

struct Range {
  uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};

inline Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (p ? bytes : 0)};
}

inline bool overlaps(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// True when any output range overlaps an input range or another output.
inline bool any_alias(const Range* in, int nin, const Range* out, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(out[i], in[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(out[i], out[j])) return true;
  }
  return false;
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int launch_status() { return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace nvfp4
