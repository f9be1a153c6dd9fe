// Host-side helpers of the C ABI: argument checks and launch-error mapping.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg.h"

#define DG_REQUIRE(cond, code) \
  do {                         \
    if (!(cond)) return (code); \
  } while (0)

#define DG_ARG(cond) DG_REQUIRE(cond, DG_E_ARG)
#define DG_UNSUP(cond) DG_REQUIRE(cond, DG_E_UNSUPPORTED)

#define DG_LAUNCHED()                                      \
  do {                                                     \
    if (hipGetLastError() != hipSuccess) return DG_E_HIP; \
  } while (0)

namespace dg {

inline hipStream_t as_stream(dg_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

}  // namespace dg
