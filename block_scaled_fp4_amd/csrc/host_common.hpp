// Host-side argument checks shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4mi.h"

namespace fp4mi {

inline bool is_aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Byte ranges [a, a+na) and [b, b+nb) intersect.
inline bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

inline int dtype_size(int dtype) {
  return dtype == FP4_DTYPE_F32 ? 4 : (dtype == FP4_DTYPE_BF16 ? 2 : 0);
}

// rows*cols without overflow; element counts above 2^46 are refused.
inline bool checked_count(int64_t rows, int64_t cols, int64_t* n) {
  if (rows < 0 || cols < 0) return false;
  if (rows == 0 || cols == 0) { *n = 0; return true; }
  if (cols > (int64_t(1) << 46) / rows) return false;
  *n = rows * cols;
  return true;
}

// hipGetLastError() both reads and resets the calling thread's last error.
// An entry point calls this once its arguments are valid and before its
// first HIP call, so that launch_status() afterwards reports only errors
// raised by that entry point's own launches, not one left by an earlier,
// unrelated HIP call on the same thread.
inline void clear_stale_error() { (void)hipGetLastError(); }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP4_OK : FP4_EHIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace fp4mi
