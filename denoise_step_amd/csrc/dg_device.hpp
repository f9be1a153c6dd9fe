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

// ---------------------------------------------------------------- DPP wave reductions
// Reductions over the 64 lanes by DPP moves (no LDS traffic): inside each row of 16 lanes by
// quad permutations and mirrors, then across rows by row broadcasts into lane 63, whose value is
// returned to every lane.  The order of the operations is fixed, so sums are deterministic.
namespace dpp {
constexpr int kXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7 - i inside each 8
constexpr int kMirror = 0x140;      // lane i <-> 15 - i inside each 16
constexpr int kBcast15 = 0x142;     // lane 15 of row r -> row r + 1 (applied to rows 1 and 3)
constexpr int kBcast31 = 0x143;     // lane 31 -> rows 2 and 3 (applied to rows 2 and 3)
}  // namespace dpp

// value of the DPP source lane; lanes the move does not write get `fill`
template <int CTRL, int ROW_MASK>
DG_DEV float dpp_f(float v, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK>
DG_DEV int32_t dpp_i(int32_t v, int32_t fill) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, ROW_MASK, 0xF, false);
}
DG_DEV float lane63_f(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63)); }

DG_DEV float dpp_wave_max(float v) {
  v = fmaxf(v, dpp_f<dpp::kXor1, 0xF>(v, -INFINITY));
  v = fmaxf(v, dpp_f<dpp::kXor2, 0xF>(v, -INFINITY));
  v = fmaxf(v, dpp_f<dpp::kHalfMirror, 0xF>(v, -INFINITY));
  v = fmaxf(v, dpp_f<dpp::kMirror, 0xF>(v, -INFINITY));
  v = fmaxf(v, dpp_f<dpp::kBcast15, 0xA>(v, -INFINITY));
  v = fmaxf(v, dpp_f<dpp::kBcast31, 0xC>(v, -INFINITY));
  return lane63_f(v);
}

DG_DEV float dpp_wave_sum(float v) {
  v += dpp_f<dpp::kXor1, 0xF>(v, 0.f);
  v += dpp_f<dpp::kXor2, 0xF>(v, 0.f);
  v += dpp_f<dpp::kHalfMirror, 0xF>(v, 0.f);
  v += dpp_f<dpp::kMirror, 0xF>(v, 0.f);
  v += dpp_f<dpp::kBcast15, 0xA>(v, 0.f);
  v += dpp_f<dpp::kBcast31, 0xC>(v, 0.f);
  return lane63_f(v);
}

// (value, index) maximum with lowest-index tie-break; the result is returned to every lane
template <int CTRL, int ROW_MASK>
DG_DEV void dpp_argmax_step(float& v, int32_t& i) {
  const float v2 = dpp_f<CTRL, ROW_MASK>(v, -INFINITY);
  const int32_t i2 = dpp_i<CTRL, ROW_MASK>(i, 0x7FFFFFFF);
  const bool better = v2 > v || (v2 == v && i2 < i);
  v = better ? v2 : v;
  i = better ? i2 : i;
}
DG_DEV void dpp_wave_argmax(float& v, int32_t& i) {
  dpp_argmax_step<dpp::kXor1, 0xF>(v, i);
  dpp_argmax_step<dpp::kXor2, 0xF>(v, i);
  dpp_argmax_step<dpp::kHalfMirror, 0xF>(v, i);
  dpp_argmax_step<dpp::kMirror, 0xF>(v, i);
  dpp_argmax_step<dpp::kBcast15, 0xA>(v, i);
  dpp_argmax_step<dpp::kBcast31, 0xC>(v, i);
  v = lane63_f(v);
  i = __builtin_amdgcn_readlane(i, 63);
}

// ---------------------------------------------------------------- softmax state and Gumbel keys
// Online softmax state in base 2 relative to a reference m (the running maximum in a streaming
// pass): Z = sum 2^(x2 - m), S = sum 2^(x2 - m) (x2 - m), x2 = x log2(e).
struct SoftState {
  float m, Z, S;
};

DG_DEV float exp2f_fast(float d) { return __builtin_amdgcn_exp2f(d); }

// merge b into a (each relative to its own reference); Z == 0 marks an empty state
DG_DEV void soft_merge(SoftState& a, SoftState b) {
  if (b.Z == 0.f) return;
  if (a.Z == 0.f) {
    a = b;
    return;
  }
  const float m = fmaxf(a.m, b.m);
  const float da = a.m - m, db = b.m - m;
  const float fa = exp2f_fast(da), fb = exp2f_fast(db);
  a.S = fa * (a.S + da * a.Z) + fb * (b.S + db * b.Z);
  a.Z = fa * a.Z + fb * b.Z;
  a.m = m;
}

// Softmax state of the whole wave: every lane's (Z, S) rescaled to the wave's largest reference, then summed.
DG_DEV SoftState dpp_wave_soft(SoftState s) {
  const float M = dpp_wave_max(s.m);
  float Z = 0.f, S = 0.f;
  if (s.Z != 0.f) {
    const float d = s.m - M;
    const float f = exp2f_fast(d);
    Z = f * s.Z;
    S = f * (s.S + d * s.Z);
  }
  return SoftState{M, dpp_wave_sum(Z), dpp_wave_sum(S)};
}

// Gumbel-max key in log2 units.  With u = (2a + 1) 2^-24 (a = w >> 9, exact in fp32),
// g = -ln(-ln u) and x2 = x log2(e):
//   (x + g) log2(e) = x2 - log2(-log2 u) - log2(ln 2),
// so argmax (x + g) = argmax (x2 - log2(-log2 u)) (a positive rescale and a shift).
// Both logs are the hardware base-2 logarithm on normal inputs (u >= 2^-24, -log2 u >= 2^-24 / ln 2).
DG_DEV float gumbel_key2(float x2, uint32_t w) {
  const float u = fmaf(static_cast<float>(w >> 9), 0x1.0p-23f, 0x1.0p-24f);
  const float L = -__builtin_amdgcn_logf(u);
  return x2 - __builtin_amdgcn_logf(L);
}

// ---------------------------------------------------------------- OCP E4M3 (FP8) codes
// Conversions by gfx950's instructions; exact, since every E4M3 value is an fp16 (and fp32) value.
// Byte b of a word holds element b.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

DG_DEV half8 e4m3x8_to_half8(uint32_t lo, uint32_t hi) {
  const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  half8 h;
  h[0] = a[0]; h[1] = a[1]; h[2] = b[0]; h[3] = b[1];
  h[4] = c[0]; h[5] = c[1]; h[6] = d[0]; h[7] = d[1];
  return h;
}

DG_DEV float4 e4m3x4_to_float4(uint32_t w) {
  const float2v a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const float2v b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return make_float4(a[0], a[1], b[0], b[1]);
}

// Direct global -> LDS copies (global_load_lds_dwordx4): each lane fetches 16 bytes and lane i's bytes
// land at LDS address lds + 16 i.  lds must be wave-uniform; it is passed in M0 through a register
// constraint, so the compiler sets M0 itself and knows it is in use.  Issued from inline asm, the
// copies are tracked only by the explicit vmcnt waits of the code that issues them.
DG_DEV void lds_copy16(uint32_t lds, const void* src) {  // per-lane 64-bit source address
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}

// the same with a wave-uniform base and a per-lane 32-bit byte offset; NT marks the load non-temporal
template <bool NT>
DG_DEV void lds_copy16(uint32_t lds, const void* base, uint32_t lane_off) {
  if constexpr (NT)
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(lane_off), "s"(base), "{m0}"(lds) : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(lane_off), "s"(base), "{m0}"(lds) : "memory");
}

// s_waitcnt immediate that waits for vmcnt <= n only (vmcnt in bits 3:0 and 15:14; expcnt 6:4 and
// lgkmcnt 11:8 left at their maxima).  Used where direct global -> LDS copies issued from inline
// asm must have landed: the compiler does not count those instructions.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt operand that waits for LDS / scalar-memory counts <= n only (vmcnt and expcnt at their maxima)
constexpr int lgkmcnt_only(int n) { return 15 | (3 << 14) | (7 << 4) | ((n & 15) << 8); }

}  // namespace dg
