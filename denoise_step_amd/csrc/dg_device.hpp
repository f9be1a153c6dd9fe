// Device-side helpers shared by the gfx950 kernels: bf16 / fp16 conversion,
// Philox4x32-10, wave64 reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg.h"

#define DG_DEV __device__ __forceinline__

namespace dg {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 / f16
DG_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
DG_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
DG_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// round to nearest even (inputs are finite)
DG_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw (SC'11): 10 rounds of the Philox-4x32 bijection.
struct u32x4 {
  uint32_t x, y, z, w;
};

DG_DEV u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    c = u32x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// token = (w * V) >> 32
DG_DEV int32_t token_from_word(uint32_t w, int32_t V) {
  return static_cast<int32_t>((static_cast<uint64_t>(w) * static_cast<uint32_t>(V)) >> 32);
}

// One random token for (seed, pos, step, stream): word 0 of Philox(key, (0, pos, step, stream)).
DG_DEV int32_t philox_token(uint64_t seed, int32_t pos, int32_t step, uint32_t stream, int32_t V) {
  u32x4 r = philox4x32_10(u32x4{0u, static_cast<uint32_t>(pos), static_cast<uint32_t>(step), stream},
                          static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  return token_from_word(r.x, V);
}

// ---------------------------------------------------------------- reductions
DG_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
DG_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
DG_DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// (value, index) max with lowest-index tie-break
DG_DEV void argmax_merge(float& v, int32_t& i, float v2, int32_t i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}
DG_DEV void wave_argmax(float& v, int32_t& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v2 = __shfl_xor(v, o, kWave);
    int32_t i2 = __shfl_xor(i, o, kWave);
    argmax_merge(v, i, v2, i2);
  }
}

// s_waitcnt immediate that waits for vmcnt <= n only (vmcnt in bits 3:0 and 15:14; expcnt 6:4 and
// lgkmcnt 11:8 left at their maxima).  Used where direct global -> LDS copies issued from inline
// asm must have landed: the compiler does not count those instructions.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

}  // namespace dg
