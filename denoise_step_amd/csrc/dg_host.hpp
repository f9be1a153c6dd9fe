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

// Operand written by dg_lmhead_denoise_sample (dg_lmhead_operand_bytes) and read by
// dg_selfcond_embed_lm: the self-conditioning operand of the sampling pass (w [Kp / 32][Mp][32]
// fp16, then ref [rows][nrun] f32, one run per 16384 ids, the refs integers here), then each
// row's argmax id [rows] i32.
struct LmOperandLayout {
  int64_t Mp, Kp;
  int32_t nrun;
  size_t off_ref, off_top, bytes;
};

inline LmOperandLayout lm_operand_layout(int32_t rows, int32_t V) {
  LmOperandLayout L{};
  L.Mp = cdiv(rows, 256) * 256;
  L.Kp = cdiv(V, 128) * 128;
  L.nrun = static_cast<int32_t>(cdiv(V, 16384));
  L.off_ref = round_up(static_cast<size_t>(L.Mp) * L.Kp * 2, 256);
  L.off_top = round_up(L.off_ref + static_cast<size_t>(rows) * L.nrun * 4, 256);
  L.bytes = round_up(L.off_top + static_cast<size_t>(rows) * 4, 256);
  return L;
}

}  // namespace dg
