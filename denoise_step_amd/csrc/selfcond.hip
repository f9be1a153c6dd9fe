// dg_selfcond_prepare / dg_selfcond_embed: self-conditioning of the next
// denoise pass.
//
// Method: DiffusionGemma/vLLM page, section "Self-conditioning" (the previous
// step's full softmax becomes a probability-weighted mean of the token
// embeddings, goes through a small gated MLP and is added to the canvas
// embedding; zero for encoder passes) and section "DiffusionGemmaModelState
// and DiffusionSampler" (prepare_inputs embeds the canvas and applies it).
//
// bf16 path (gfx950):
//   1. probs:   w[r][i] = fp16(exp(x_i - m_r) * 2^15), zero-padded to Kp = roundup(V, 128).
//               The 2^15 scale keeps every weight above exp(-20) in fp16's normal range
//               (a plain fp16 or bf16 probability would lose 11+ bits on diffuse rows).
//   2. P.E:     split-K fp16 MFMA GEMM against E^T (fp16, prepared once; bf16 values
//               convert exactly except below 2^-14, where the absolute error is < 2^-25).
//   3. reduce:  s = sum(partials) * 2^-15 * exp(-ln Z) -> s (fp32, optional output) and an
//               fp16 copy scaled per row by a power of two (largest |s| in (2^13, 2^14]).
//   4. MLP:     [gate | up] = s [W_gate | W_up] (one GEMM), h = gelu_tanh(gate) * up, stored in
//               fp16 with its own per-row power-of-two scale (at the weights' N(0, 0.02^2) scale
//               h is ~1e-5, below fp16's normal range unscaled), y = h W_down (second GEMM).
//   5. embed:   x_out = bf16(E[canvas] + (sc_on ? y : 0)).
// fp32 path: the same steps with fp32 kernels (used by the tiny closed loop).
#include "dg_device.hpp"
#include "dg_host.hpp"
#include "gemm_f16.hpp"

#include <algorithm>

namespace dg {
namespace {

constexpr float kProbScale = 32768.0f;  // 2^15

int64_t pad128(int64_t v) { return (v + 127) / 128 * 128; }

// P.E against an E4M3 embedding table (N a multiple of 256): the E stream is one byte per element.
__global__ __launch_bounds__(kGemmThreads) void gemm_f16_e4m3_splitk_kernel(GemmArgs g) {
  gemm_splitk_body<256, true, true>(g);
}

// ---------------------------------------------------------------- prepare
// dst = fp16(src^T) placed at rows row_off .. row_off + N - 1 of a K-blocked operand with R rows:
// element (row_off + n, k) = src[k][n] for k < K (rows of src), zero for K <= k < Kp.
__global__ __launch_bounds__(256) void transpose_bf16_to_f16_kernel(const uint16_t* __restrict__ src, int32_t K,
                                                                    int32_t N, int64_t Kp, int32_t row_off,
                                                                    int32_t R, _Float16* __restrict__ dst) {
  __shared__ float tile[64][65];
  const int k0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int k = k0 + i, n = n0 + tx;
    tile[i][tx] = (k < K && n < N) ? bf16_to_f32(src[static_cast<int64_t>(k) * N + n]) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int n = n0 + i, k = k0 + tx;
    if (n < N && k < Kp) dst[kblk_index(row_off + n, k, R)] = static_cast<_Float16>(tile[tx][i]);
  }
}

// E4M3 codes src [K][N] -> dst, the K-blocked byte operand with N rows and Kp columns: element
// (n, k) = src[k][n] for k < K, code 0 (+0.0) for K <= k < Kp.
__global__ __launch_bounds__(256) void transpose_e4m3_kernel(const uint8_t* __restrict__ src, int32_t K, int32_t N,
                                                             int64_t Kp, uint8_t* __restrict__ dst) {
  __shared__ uint8_t tile[64][65];
  const int k0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int k = k0 + i, n = n0 + tx;
    tile[i][tx] = (k < K && n < N) ? src[static_cast<int64_t>(k) * N + n] : uint8_t{0};
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int n = n0 + i, k = k0 + tx;
    if (n < N && k < Kp) dst[kblk_index(n, k, N)] = tile[tx][i];
  }
}

// ---------------------------------------------------------------- bf16 path kernels
// w is written in the K-blocked layout with Mp rows (the GEMM's left operand).  A workgroup covers
// 8 rows x 256 columns: each row is read as 512 contiguous bytes and, for each of the 8 K slices of
// 32, the 8 rows are written as 512 contiguous bytes.
template <bool BF16>
__global__ __launch_bounds__(256) void probs_f16_kernel(const void* __restrict__ logits, int64_t ld, int32_t V,
                                                        int64_t Kp, int64_t Mp, int32_t rows, float inv_t,
                                                        const float* __restrict__ row_max, _Float16* __restrict__ w) {
  const int r = blockIdx.y * 8 + (threadIdx.x >> 5);
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 + (threadIdx.x & 31) * 8;
  if (r >= rows || i0 >= Kp) return;
  const float m = row_max[r];
  float l[8];
  if constexpr (BF16) {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(logits) + r * ld;
    if (i0 + 8 <= V) {
      const uint4 q = *reinterpret_cast<const uint4*>(row + i0);
      l[0] = bf16_lo(q.x); l[1] = bf16_hi(q.x); l[2] = bf16_lo(q.y); l[3] = bf16_hi(q.y);
      l[4] = bf16_lo(q.z); l[5] = bf16_hi(q.z); l[6] = bf16_lo(q.w); l[7] = bf16_hi(q.w);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) l[j] = (i0 + j < V) ? bf16_to_f32(row[i0 + j]) : -INFINITY;
    }
  } else {
    const float* row = reinterpret_cast<const float*>(logits) + r * ld;
#pragma unroll
    for (int j = 0; j < 8; ++j) l[j] = (i0 + j < V) ? row[i0 + j] : -INFINITY;
  }
  half8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = static_cast<_Float16>(__expf(l[j] * inv_t - m) * kProbScale);
  *reinterpret_cast<half8*>(w + kblk_index(r, i0, Mp)) = o;
}

// Power-of-two scale that brings a row's largest magnitude to (2^13, 2^14]: applied before a
// row is stored in fp16 so that small activations stay in fp16's normal range (exact, undone
// by multiplying the GEMM result by the reciprocal).
DG_DEV float row_pow2_scale(float amax) {
  if (!(amax > 0.f) || !(amax < INFINITY)) return 1.f;
  int e;
  frexpf(amax, &e);  // amax in [2^(e-1), 2^e)
  return ldexpf(1.f, 14 - e);
}

// Largest value over the NT threads of the workgroup (DPP inside each wave, the waves via LDS).
template <int NT>
DG_DEV float block_max(float v, float* red) {
  v = dpp_wave_max(v);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) m = fmaxf(m, red[w]);
  return m;
}

DG_DEV float4 f4_add(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
DG_DEV float f4_amax(float4 a) { return fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))); }

// four consecutive columns n .. n + 3 (n % 4 == 0) of row r stored as fp16 in the K-blocked layout
// (they are contiguous there: one 8-byte store)
DG_DEV void store4_f16(_Float16* dst, int r, int n, int64_t Mp, float4 v, float sc) {
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  half4 h;
  h[0] = static_cast<_Float16>(v.x * sc);
  h[1] = static_cast<_Float16>(v.y * sc);
  h[2] = static_cast<_Float16>(v.z * sc);
  h[3] = static_cast<_Float16>(v.w * sc);
  *reinterpret_cast<half4*>(dst + kblk_index(r, n, Mp)) = h;
}

// Split-K reduce of the P.E partials, one workgroup of 1024 threads per row, each thread C groups of
// 4 columns: s = sum_split part * 2^-15 / Z (-> s_out when requested), then s16 = fp16(s * scale_r)
// in the K-blocked layout with scale_r the power of two that brings the row's largest |s| into
// (2^13, 2^14], and s_inv[r] = 1 / scale_r.  The split loads are issued eight splits at a time, so
// a workgroup has up to 128 KB of the row in flight.
constexpr int kReduceThreads = 1024;
// With sc_ref (the operand written by the sampling pass), split k's probabilities are relative to
// 2^ref[r][k] instead of the row max, so its partial is weighted by 2^(ref[r][k] - row_max log2 e).
// Operand of the fused LM head (lm.w != nullptr): its values were written relative to an integer
// power of two per 256-id tile and rescaled exactly to the run's integer reference, so a row's
// largest probability carries up to 2^-11 relative rounding, where the sampling pass's operand
// holds it exactly (2^15); the term of the argmax id i* is replaced by its exact value:
// s += (2^15 - g w~) E[i*] in operand units, with w~ the stored value and g its split's weight.
struct LmTop {
  const _Float16* w;  // operand [Kp / 32][Mp][32]
  const int32_t* top; // [rows]
  const uint16_t* E;  // [V][N] bf16
  int32_t V;
};

template <int C>
__global__ __launch_bounds__(kReduceThreads) void pe_reduce_kernel(const float* __restrict__ part, int32_t splits, int32_t M,
                                                        int32_t N, int64_t Mp, const float* __restrict__ row_max,
                                                        const float* __restrict__ row_lnz,
                                                        const float* __restrict__ sc_ref, int32_t nchunk,
                                                        float e_scale, float* __restrict__ s_out,
                                                        _Float16* __restrict__ s16, float* __restrict__ s_inv,
                                                        LmTop lm) {
  __shared__ float red[kReduceThreads / kWave];
  const int r = blockIdx.x;
  const float f = (e_scale / kProbScale) * __expf(-row_lnz[r]);
  const float m2 = sc_ref != nullptr ? row_max[r] * 1.4426950408889634f : 0.f;
  float4 acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (lm.w != nullptr && lm.top[r] >= 0 && lm.top[r] < lm.V) {  // out of range only for non-finite logits
    const int64_t i = lm.top[r];
    const float wt = static_cast<float>(lm.w[((i >> 5) * Mp + r) * 32 + (i & 31)]);
    const float g = exp2f(sc_ref[static_cast<int64_t>(r) * nchunk + (i >> 14)] - m2);
    const float coef = kProbScale - g * wt;
    const uint16_t* er = lm.E + i * N;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int n = 4 * (threadIdx.x + kReduceThreads * c);
      if (n < N) {
        const uint2 e = *reinterpret_cast<const uint2*>(er + n);
        acc[c] = make_float4(coef * bf16_lo(e.x), coef * bf16_hi(e.x), coef * bf16_lo(e.y), coef * bf16_hi(e.y));
      }
    }
  }
#pragma unroll 8
  for (int k = 0; k < splits; ++k) {
    const float* p = part + (static_cast<int64_t>(k) * M + r) * N;
    const float g = sc_ref != nullptr ? exp2f(sc_ref[static_cast<int64_t>(r) * nchunk + k] - m2) : 1.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int n = 4 * (threadIdx.x + kReduceThreads * c);
      if (n < N) {
        const float4 v = *reinterpret_cast<const float4*>(p + n);
        acc[c] = make_float4(fmaf(v.x, g, acc[c].x), fmaf(v.y, g, acc[c].y), fmaf(v.z, g, acc[c].z),
                             fmaf(v.w, g, acc[c].w));
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    acc[c] = make_float4(acc[c].x * f, acc[c].y * f, acc[c].z * f, acc[c].w * f);
    const int n = 4 * (threadIdx.x + kReduceThreads * c);
    if (n < N) {
      amax = fmaxf(amax, f4_amax(acc[c]));
      if (s_out != nullptr) *reinterpret_cast<float4*>(s_out + static_cast<int64_t>(r) * N + n) = acc[c];
    }
  }
  const float sc = row_pow2_scale(block_max<kReduceThreads>(amax, red));
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int n = 4 * (threadIdx.x + kReduceThreads * c);
    if (n < N) store4_f16(s16, r, n, Mp, acc[c], sc);
  }
  if (threadIdx.x == 0) s_inv[r] = 1.f / sc;
}

DG_DEV float gelu_tanh(float z) {
  const float c = 0.7978845608028654f;  // sqrt(2 / pi)
  return 0.5f * z * (1.f + tanhf(c * (z + 0.044715f * z * z * z)));
}

// One workgroup per row: h = gelu_tanh(gate) * up from the partials of the [gate | up] GEMM (whose
// input row was scaled by 1 / s_inv[r]), then h16 = fp16(h * scale_r) in the K-blocked layout,
// h_inv[r] = 1 / scale_r.  Each thread owns C groups of 4 hidden units.
template <int C>
__global__ __launch_bounds__(256) void glu_reduce_kernel(const float* __restrict__ part, int32_t splits, int32_t M,
                                                         int32_t H, int64_t Mp, const float* __restrict__ s_inv,
                                                         _Float16* __restrict__ h16, float* __restrict__ h_inv) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int64_t N2 = 2 * static_cast<int64_t>(H);
  float4 g[C], u[C];
#pragma unroll
  for (int c = 0; c < C; ++c) g[c] = u[c] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int k = 0; k < splits; ++k) {
    const float* p = part + (static_cast<int64_t>(k) * M + r) * N2;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = 4 * (threadIdx.x + 256 * c);
      if (j < H) {
        g[c] = f4_add(g[c], *reinterpret_cast<const float4*>(p + j));
        u[c] = f4_add(u[c], *reinterpret_cast<const float4*>(p + H + j));
      }
    }
  }
  const float si = s_inv[r];
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    g[c] = make_float4(gelu_tanh(g[c].x * si) * (u[c].x * si), gelu_tanh(g[c].y * si) * (u[c].y * si),
                       gelu_tanh(g[c].z * si) * (u[c].z * si), gelu_tanh(g[c].w * si) * (u[c].w * si));
    if (4 * static_cast<int>(threadIdx.x + 256 * c) < H) amax = fmaxf(amax, f4_amax(g[c]));
  }
  const float sc = row_pow2_scale(block_max<256>(amax, red));
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = 4 * (threadIdx.x + 256 * c);
    if (j < H) store4_f16(h16, r, j, Mp, g[c], sc);
  }
  if (threadIdx.x == 0) h_inv[r] = 1.f / sc;
}

// x_out = bf16(E[canvas] + (sc_on ? y : 0)), y from the partials of the down GEMM; one thread per
// 4 consecutive values of a row.  E8: E is E4M3 codes, each value times e_scale.
template <bool E8>
__global__ __launch_bounds__(256) void embed_reduce_kernel(const float* __restrict__ part, int32_t splits, int32_t M,
                                                           int32_t d, int32_t V, int32_t C,
                                                           const void* __restrict__ E, float e_scale,
                                                           const int32_t* __restrict__ canvas,
                                                           const uint8_t* __restrict__ sc_on,
                                                           const float* __restrict__ h_inv,
                                                           uint16_t* __restrict__ x_out, float* __restrict__ y_out) {
  const int64_t idx = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
  if (idx >= static_cast<int64_t>(M) * d) return;
  const int r = static_cast<int>(idx / d), c = static_cast<int>(idx - static_cast<int64_t>(r) * d);
  const int64_t tok = min(max(canvas[r], 0), V - 1);
  float4 x;
  if constexpr (E8) {
    x = e4m3x4_to_float4(*reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(E) + tok * d + c));
    x = make_float4(x.x * e_scale, x.y * e_scale, x.z * e_scale, x.w * e_scale);
  } else {
    const uint2 e = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(E) + tok * d + c);
    x = make_float4(bf16_lo(e.x), bf16_hi(e.x), bf16_lo(e.y), bf16_hi(e.y));
  }
  const bool on = sc_on[r / C] != 0;
  if (on || y_out != nullptr) {
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int k = 0; k < splits; ++k) y = f4_add(y, *reinterpret_cast<const float4*>(part + static_cast<int64_t>(k) * M * d + idx));
    const float hi = h_inv[r];
    y = make_float4(y.x * hi, y.y * hi, y.z * hi, y.w * hi);
    if (on) x = f4_add(x, y);
    if (y_out != nullptr) *reinterpret_cast<float4*>(y_out + idx) = y;
  }
  const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
  const uint32_t hi2 = static_cast<uint32_t>(f32_to_bf16(x.z)) | (static_cast<uint32_t>(f32_to_bf16(x.w)) << 16);
  *reinterpret_cast<uint2*>(x_out + idx) = make_uint2(lo, hi2);
}

// ---------------------------------------------------------------- fp32 path kernels
__global__ __launch_bounds__(256) void probs_f32_kernel(const float* __restrict__ logits, int64_t ld, int32_t V,
                                                        float inv_t, const float* __restrict__ row_max,
                                                        const float* __restrict__ row_lnz, float* __restrict__ P) {
  const int r = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= V) return;
  P[r * static_cast<int64_t>(V) + i] = expf(logits[r * ld + i] * inv_t - row_max[r] - row_lnz[r]);
}

__global__ __launch_bounds__(256) void glu_f32_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                      int64_t n, float* __restrict__ h) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) h[i] = gelu_tanh(g[i]) * u[i];
}

__global__ __launch_bounds__(256) void embed_f32_kernel(const float* __restrict__ y, int32_t M, int32_t d, int32_t V,
                                                        int32_t C, const float* __restrict__ E,
                                                        const int32_t* __restrict__ canvas,
                                                        const uint8_t* __restrict__ sc_on, float* __restrict__ x_out,
                                                        float* __restrict__ y_out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(M) * d) return;
  const int r = static_cast<int>(idx / d), c = static_cast<int>(idx - static_cast<int64_t>(r) * d);
  const int64_t tok = min(max(canvas[r], 0), V - 1);
  x_out[idx] = E[tok * d + c] + (sc_on[r / C] ? y[idx] : 0.f);
  if (y_out != nullptr) y_out[idx] = y[idx];
}

// ---------------------------------------------------------------- workspace plans
struct PreparedLayout {
  int64_t Kp;
  size_t off_et, off_wgu, off_wd, bytes;
};

PreparedLayout prepared_layout(int32_t V, int32_t d, int32_t hidden) {
  PreparedLayout p{};
  p.Kp = pad128(V);
  p.off_et = 0;
  p.off_wgu = round_up(p.off_et + static_cast<size_t>(d) * p.Kp * 2, 256);
  p.off_wd = round_up(p.off_wgu + static_cast<size_t>(2) * hidden * d * 2, 256);
  p.bytes = round_up(p.off_wd + static_cast<size_t>(d) * hidden * 2, 256);
  return p;
}

// E4M3 table: E^T as bytes (d rows, Kp columns), then the same fp16 MLP operands
PreparedLayout prepared_layout_e4m3(int32_t V, int32_t d, int32_t hidden) {
  PreparedLayout p{};
  p.Kp = pad128(V);
  p.off_et = 0;
  p.off_wgu = round_up(p.off_et + static_cast<size_t>(d) * p.Kp, 256);
  p.off_wd = round_up(p.off_wgu + static_cast<size_t>(2) * hidden * d * 2, 256);
  p.bytes = round_up(p.off_wd + static_cast<size_t>(d) * hidden * 2, 256);
  return p;
}

struct Bf16Plan {
  int64_t Kp, Mp;
  GemmPlan pe, g1, g2;
  size_t off_w, off_part, off_s16, off_h16, off_sinv, off_hinv, bytes;
};

// sc: the probability operand comes from the sampling pass (dg_denoise_sample_sc), in runs of
// kScChunk vocabulary ids with their own reference, so each P.E split covers exactly one run and the
// workspace holds no operand of its own.
constexpr int32_t kScChunk = 16384;

Bf16Plan bf16_plan(int32_t rows, int32_t V, int32_t d, int32_t hidden, bool sc = false) {
  Bf16Plan p{};
  // GEMM left operands are allocated with whole 256-row tiles (the tail rows are read, never stored)
  const int64_t rows_p = (static_cast<int64_t>(rows) + kGemmTM - 1) / kGemmTM * kGemmTM;
  p.Mp = rows_p;
  p.Kp = pad128(V);
  // Every split of K is fixed by K alone (batch invariance: a row's sums run in the same order
  // whatever the number of rows).  P.E: one split per 16384 vocabulary ids (the operand's runs).
  // The MLP GEMMs (M = rows, K = d or hidden) use 128-wide N tiles with 8 splits of d and 4 of
  // hidden, which at 256 rows is about 128 workgroups and halves the split-K partials against one
  // 256-wide tile per CU (measured 30 -> 24 us for 4096 -> 2 x 1024 -> 4096 at 256 rows).
  p.pe = plan_gemm_kchunk(rows, d, static_cast<int32_t>(p.Kp), kScChunk);
  const auto kchunk = [](int32_t K, int32_t parts) {
    const int32_t r = kGemmStages * kGemmTK;
    const int32_t c = (K + parts - 1) / parts;
    return std::max(r, (c + r - 1) / r * r);
  };
  p.g1 = plan_gemm_kchunk(rows, 2 * hidden, d, kchunk(d, 8), true);
  p.g2 = plan_gemm_kchunk(rows, d, hidden, kchunk(hidden, 4), true);
  size_t part = 0;
  part = std::max(part, static_cast<size_t>(p.pe.splits) * rows * d * 4);
  part = std::max(part, static_cast<size_t>(p.g1.splits) * rows * 2 * hidden * 4);
  part = std::max(part, static_cast<size_t>(p.g2.splits) * rows * d * 4);
  p.off_w = 0;
  p.off_part = round_up(p.off_w + (sc ? 0 : static_cast<size_t>(rows_p) * p.Kp * 2), 256);
  p.off_s16 = round_up(p.off_part + part, 256);
  p.off_h16 = round_up(p.off_s16 + static_cast<size_t>(rows_p) * d * 2, 256);
  p.off_sinv = round_up(p.off_h16 + static_cast<size_t>(rows_p) * hidden * 2, 256);
  p.off_hinv = round_up(p.off_sinv + static_cast<size_t>(rows) * 4, 256);
  p.bytes = round_up(p.off_hinv + static_cast<size_t>(rows) * 4, 256);
  return p;
}

struct F32Plan {
  size_t off_P, off_s, off_g, off_u, off_h, off_y, bytes;
};

F32Plan f32_plan(int32_t rows, int32_t V, int32_t d, int32_t hidden) {
  F32Plan p{};
  p.off_P = 0;
  p.off_s = round_up(p.off_P + static_cast<size_t>(rows) * V * 4, 256);
  p.off_g = round_up(p.off_s + static_cast<size_t>(rows) * d * 4, 256);
  p.off_u = round_up(p.off_g + static_cast<size_t>(rows) * hidden * 4, 256);
  p.off_h = round_up(p.off_u + static_cast<size_t>(rows) * hidden * 4, 256);
  p.off_y = round_up(p.off_h + static_cast<size_t>(rows) * hidden * 4, 256);
  p.bytes = round_up(p.off_y + static_cast<size_t>(rows) * d * 4, 256);
  return p;
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

// One M tile (a canvas of <= 256 rows): the right operand streams non-temporally; several M tiles
// (a batch of canvases) re-read each of its chunks, which then stay in L2.
template <int ROLE>
void launch_gemm(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  if (p.mtiles == 1) {
    if (p.tn == 256)
      gemm_f16_splitk_kernel<ROLE, 256><<<p.grid, kGemmThreads, 0, s>>>(a);
    else
      gemm_f16_splitk_kernel<ROLE, 128><<<p.grid, kGemmThreads, 0, s>>>(a);
  } else {
    if (p.tn == 256)
      gemm_f16_splitk_kernel<ROLE, 256, false><<<p.grid, kGemmThreads, 0, s>>>(a);
    else
      gemm_f16_splitk_kernel<ROLE, 128, false><<<p.grid, kGemmThreads, 0, s>>>(a);
  }
}

// P.E (from the operand w), its reduce, the gated MLP and the embedding: the bf16 path after the
// probability operand exists.  sc_ref != nullptr: w comes from the sampling pass (per-run references).
// et8 != nullptr: the table is E4M3 (E holds the codes, values times e_scale) and et8 is its
// K-blocked transpose; et is then unused.
dg_status selfcond_bf16_tail(const Bf16Plan& p, const _Float16* w, const float* sc_ref, int32_t nchunk,
                             const float* row_max, const float* row_lnz, const uint8_t* sc_on, const int32_t* canvas,
                             int32_t rows, int32_t C, const void* E, const _Float16* et, const _Float16* wgu,
                             const _Float16* wd, int32_t V, int32_t d, int32_t hidden, void* x_out, float* s_out,
                             float* y_out, char* wsb, void* pe_start, void* pe_stop, hipStream_t s,
                             const uint8_t* et8 = nullptr, float e_scale = 1.f, const int32_t* lm_top = nullptr) {
  const int64_t rows64 = rows;
  auto* part = reinterpret_cast<float*>(wsb + p.off_part);
  auto* s16 = reinterpret_cast<_Float16*>(wsb + p.off_s16);
  auto* h16 = reinterpret_cast<_Float16*>(wsb + p.off_h16);
  auto* s_inv = reinterpret_cast<float*>(wsb + p.off_sinv);
  auto* h_inv = reinterpret_cast<float*>(wsb + p.off_hinv);
  if (pe_start != nullptr) DG_REQUIRE(hipEventRecord(reinterpret_cast<hipEvent_t>(pe_start), s) == hipSuccess, DG_E_HIP);
  if (et8 != nullptr)
    gemm_f16_e4m3_splitk_kernel<<<p.pe.grid, kGemmThreads, 0, s>>>(
        gemm_args(w, p.Mp, nullptr, d, part, rows, d, static_cast<int32_t>(p.Kp), p.pe, et8));
  else
    launch_gemm<0>(p.pe, gemm_args(w, p.Mp, et, d, part, rows, d, static_cast<int32_t>(p.Kp), p.pe), s);
  DG_LAUNCHED();
  if (pe_stop != nullptr) DG_REQUIRE(hipEventRecord(reinterpret_cast<hipEvent_t>(pe_stop), s) == hipSuccess, DG_E_HIP);
  const int rc = static_cast<int>(cdiv(d, 4 * kReduceThreads)), hc = static_cast<int>(cdiv(hidden, 1024));
  const LmTop lm = lm_top != nullptr ? LmTop{w, lm_top, reinterpret_cast<const uint16_t*>(E), V}
                                      : LmTop{nullptr, nullptr, nullptr, 0};
  if (rc == 1)
    pe_reduce_kernel<1><<<rows, kReduceThreads, 0, s>>>(part, p.pe.splits, rows, d, p.Mp, row_max, row_lnz, sc_ref,
                                                        nchunk, e_scale, s_out, s16, s_inv, lm);
  else
    pe_reduce_kernel<2><<<rows, kReduceThreads, 0, s>>>(part, p.pe.splits, rows, d, p.Mp, row_max, row_lnz, sc_ref,
                                                        nchunk, e_scale, s_out, s16, s_inv, lm);
  DG_LAUNCHED();
  launch_gemm<1>(p.g1, gemm_args(s16, p.Mp, wgu, 2 * hidden, part, rows, 2 * hidden, d, p.g1), s);
  DG_LAUNCHED();
  if (hc == 1)
    glu_reduce_kernel<1><<<rows, 256, 0, s>>>(part, p.g1.splits, rows, hidden, p.Mp, s_inv, h16, h_inv);
  else if (hc == 2)
    glu_reduce_kernel<2><<<rows, 256, 0, s>>>(part, p.g1.splits, rows, hidden, p.Mp, s_inv, h16, h_inv);
  else if (hc <= 4)
    glu_reduce_kernel<4><<<rows, 256, 0, s>>>(part, p.g1.splits, rows, hidden, p.Mp, s_inv, h16, h_inv);
  else
    glu_reduce_kernel<8><<<rows, 256, 0, s>>>(part, p.g1.splits, rows, hidden, p.Mp, s_inv, h16, h_inv);
  DG_LAUNCHED();
  launch_gemm<1>(p.g2, gemm_args(h16, p.Mp, wd, d, part, rows, d, hidden, p.g2), s);
  DG_LAUNCHED();
  if (et8 != nullptr)
    embed_reduce_kernel<true><<<blocks_for(rows64 * d / 4), 256, 0, s>>>(
        part, p.g2.splits, rows, d, V, C, E, e_scale, canvas, sc_on, h_inv, reinterpret_cast<uint16_t*>(x_out), y_out);
  else
    embed_reduce_kernel<false><<<blocks_for(rows64 * d / 4), 256, 0, s>>>(
        part, p.g2.splits, rows, d, V, C, E, 1.f, canvas, sc_on, h_inv, reinterpret_cast<uint16_t*>(x_out), y_out);
  DG_LAUNCHED();
  return DG_OK;
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" size_t dg_selfcond_prepared_bytes(int32_t V, int32_t d, int32_t hidden, int32_t dtype) {
  if (dtype != DG_BF16 || V <= 0 || d <= 0 || hidden <= 0) return 0;
  return prepared_layout(V, d, hidden).bytes;
}

extern "C" dg_status dg_selfcond_prepare(const void* E, const void* w_gate, const void* w_up, const void* w_down,
                                         int32_t V, int32_t d, int32_t hidden, int32_t dtype, void* prepared,
                                         size_t prepared_bytes, dg_stream_t stream) {
  DG_ARG(V > 0 && d > 0 && hidden > 0);
  DG_UNSUP(dtype == DG_BF16 || dtype == DG_F32);
  if (dtype == DG_F32) return DG_OK;  // the fp32 path reads the tables as given
  DG_ARG(E && w_gate && w_up && w_down && prepared);
  DG_UNSUP(d % 128 == 0 && hidden % 128 == 0);
  const PreparedLayout L = prepared_layout(V, d, hidden);
  DG_REQUIRE(prepared_bytes >= L.bytes, DG_E_WORKSPACE);
  hipStream_t s = as_stream(stream);
  char* base = reinterpret_cast<char*>(prepared);
  auto* et = reinterpret_cast<_Float16*>(base + L.off_et);
  auto* wgu = reinterpret_cast<_Float16*>(base + L.off_wgu);
  auto* wd = reinterpret_cast<_Float16*>(base + L.off_wd);
  const auto* Eb = reinterpret_cast<const uint16_t*>(E);
  // E [V][d] -> E^T (d rows, Kp columns)
  transpose_bf16_to_f16_kernel<<<dim3(static_cast<unsigned>(cdiv(L.Kp, 64)), static_cast<unsigned>(cdiv(d, 64))), 256,
                                 0, s>>>(Eb, V, d, L.Kp, 0, d, et);
  DG_LAUNCHED();
  // W_gate, W_up [d][hidden] -> rows [0, hidden) and [hidden, 2 hidden) of one operand (2 hidden rows, d columns)
  transpose_bf16_to_f16_kernel<<<dim3(static_cast<unsigned>(cdiv(d, 64)), static_cast<unsigned>(cdiv(hidden, 64))),
                                 256, 0, s>>>(reinterpret_cast<const uint16_t*>(w_gate), d, hidden, d, 0, 2 * hidden,
                                              wgu);
  transpose_bf16_to_f16_kernel<<<dim3(static_cast<unsigned>(cdiv(d, 64)), static_cast<unsigned>(cdiv(hidden, 64))),
                                 256, 0, s>>>(reinterpret_cast<const uint16_t*>(w_up), d, hidden, d, hidden,
                                              2 * hidden, wgu);
  // W_down [hidden][d] -> d rows, hidden columns
  transpose_bf16_to_f16_kernel<<<dim3(static_cast<unsigned>(cdiv(hidden, 64)), static_cast<unsigned>(cdiv(d, 64))),
                                 256, 0, s>>>(reinterpret_cast<const uint16_t*>(w_down), hidden, d, hidden, 0, d, wd);
  DG_LAUNCHED();
  return DG_OK;
}

extern "C" size_t dg_selfcond_ws_bytes(int32_t rows, int32_t V, int32_t d, int32_t hidden, int32_t dtype) {
  if (rows <= 0 || V <= 0 || d <= 0 || hidden <= 0) return 0;
  if (dtype == DG_BF16) {
    if (d % 128 != 0 || hidden % 128 != 0) return 0;
    return bf16_plan(rows, V, d, hidden).bytes;
  }
  return f32_plan(rows, V, d, hidden).bytes;
}

extern "C" dg_status dg_selfcond_embed_traced(const void* logits, int64_t ld, int32_t dtype, float temperature,
                                              const float* row_max, const float* row_lnz, const uint8_t* sc_on,
                                              const int32_t* canvas, int32_t B, int32_t C, const void* E,
                                              const void* w_gate, const void* w_up, const void* w_down,
                                              const void* prepared, int32_t V, int32_t d, int32_t hidden, void* x_out,
                                              float* s_out, float* y_out, void* ws, size_t ws_bytes, void* pe_start,
                                              void* pe_stop, dg_stream_t stream) {
  DG_ARG(logits && row_max && row_lnz && sc_on && canvas && E && x_out);
  DG_ARG(B > 0 && C > 0 && V > 0 && d > 0 && hidden > 0 && ld >= V);
  DG_ARG(temperature > 0.f && temperature < INFINITY);
  DG_UNSUP(dtype == DG_BF16 || dtype == DG_F32);
  const int64_t rows64 = static_cast<int64_t>(B) * C;
  DG_ARG(rows64 <= 65535);
  const int32_t rows = static_cast<int32_t>(rows64);
  hipStream_t s = as_stream(stream);
  const float inv_t = 1.0f / temperature;
  char* wsb = reinterpret_cast<char*>(ws);

  if (dtype == DG_F32) {
    DG_ARG(w_gate && w_up && w_down);
    const F32Plan p = f32_plan(rows, V, d, hidden);
    DG_REQUIRE(ws != nullptr && ws_bytes >= p.bytes, DG_E_WORKSPACE);
    float* P = reinterpret_cast<float*>(wsb + p.off_P);
    float* sv = reinterpret_cast<float*>(wsb + p.off_s);
    float* g = reinterpret_cast<float*>(wsb + p.off_g);
    float* u = reinterpret_cast<float*>(wsb + p.off_u);
    float* h = reinterpret_cast<float*>(wsb + p.off_h);
    float* y = reinterpret_cast<float*>(wsb + p.off_y);
    const float* Ef = reinterpret_cast<const float*>(E);
    probs_f32_kernel<<<dim3(blocks_for(V), rows), 256, 0, s>>>(reinterpret_cast<const float*>(logits), ld, V, inv_t,
                                                               row_max, row_lnz, P);
    DG_LAUNCHED();
    dg_status st;
    if ((st = dg_linear(P, Ef, nullptr, sv, rows, d, V, 0, 1.f, stream)) != DG_OK) return st;
    if ((st = dg_linear(sv, reinterpret_cast<const float*>(w_gate), nullptr, g, rows, hidden, d, 0, 1.f, stream)) !=
        DG_OK)
      return st;
    if ((st = dg_linear(sv, reinterpret_cast<const float*>(w_up), nullptr, u, rows, hidden, d, 0, 1.f, stream)) !=
        DG_OK)
      return st;
    glu_f32_kernel<<<blocks_for(rows64 * hidden), 256, 0, s>>>(g, u, rows64 * hidden, h);
    DG_LAUNCHED();
    if ((st = dg_linear(h, reinterpret_cast<const float*>(w_down), nullptr, y, rows, d, hidden, 0, 1.f, stream)) !=
        DG_OK)
      return st;
    embed_f32_kernel<<<blocks_for(rows64 * d), 256, 0, s>>>(y, rows, d, V, C, Ef, canvas, sc_on,
                                                            reinterpret_cast<float*>(x_out), y_out);
    DG_LAUNCHED();
    if (s_out != nullptr) {
      DG_REQUIRE(hipMemcpyAsync(s_out, sv, static_cast<size_t>(rows) * d * 4, hipMemcpyDeviceToDevice, s) ==
                     hipSuccess,
                 DG_E_HIP);
    }
    return DG_OK;
  }

  // bf16 path
  DG_ARG(prepared != nullptr);
  DG_UNSUP(d % 128 == 0 && hidden % 128 == 0 && d <= 8192 && hidden <= 8192);
  DG_UNSUP(ld % 8 == 0 && aligned16(logits));
  const Bf16Plan p = bf16_plan(rows, V, d, hidden);
  DG_REQUIRE(ws != nullptr && ws_bytes >= p.bytes, DG_E_WORKSPACE);
  const PreparedLayout L = prepared_layout(V, d, hidden);
  const char* pb = reinterpret_cast<const char*>(prepared);
  const auto* et = reinterpret_cast<const _Float16*>(pb + L.off_et);
  const auto* wgu = reinterpret_cast<const _Float16*>(pb + L.off_wgu);
  const auto* wd = reinterpret_cast<const _Float16*>(pb + L.off_wd);
  auto* w = reinterpret_cast<_Float16*>(wsb + p.off_w);

  probs_f16_kernel<true><<<dim3(static_cast<unsigned>(cdiv(p.Kp, 256)), static_cast<unsigned>(cdiv(rows, 8))), 256, 0,
                          s>>>(logits, ld, V, p.Kp, p.Mp, rows, inv_t, row_max, w);
  DG_LAUNCHED();
  return selfcond_bf16_tail(p, w, nullptr, 0, row_max, row_lnz, sc_on, canvas, rows, C, E, et, wgu, wd, V, d, hidden,
                            x_out, s_out, y_out, wsb, pe_start, pe_stop, s);
}

extern "C" dg_status dg_selfcond_embed(const void* logits, int64_t ld, int32_t dtype, float temperature,
                                       const float* row_max, const float* row_lnz, const uint8_t* sc_on,
                                       const int32_t* canvas, int32_t B, int32_t C, const void* E,
                                       const void* w_gate, const void* w_up, const void* w_down, const void* prepared,
                                       int32_t V, int32_t d, int32_t hidden, void* x_out, float* s_out, float* y_out,
                                       void* ws, size_t ws_bytes, dg_stream_t stream) {
  return dg_selfcond_embed_traced(logits, ld, dtype, temperature, row_max, row_lnz, sc_on, canvas, B, C, E, w_gate,
                                  w_up, w_down, prepared, V, d, hidden, x_out, s_out, y_out, ws, ws_bytes, nullptr,
                                  nullptr, stream);
}

extern "C" size_t dg_selfcond_ws_bytes_sc(int32_t rows, int32_t V, int32_t d, int32_t hidden) {
  if (rows <= 0 || V <= 0 || d <= 0 || hidden <= 0 || d % 128 != 0 || hidden % 128 != 0) return 0;
  return bf16_plan(rows, V, d, hidden, true).bytes;
}

extern "C" dg_status dg_selfcond_embed_sc(const void* sc_operand, const float* row_max, const float* row_lnz,
                                          const uint8_t* sc_on, const int32_t* canvas, int32_t B, int32_t C,
                                          const void* E, const void* prepared, int32_t V, int32_t d, int32_t hidden,
                                          void* x_out, float* s_out, float* y_out, void* ws, size_t ws_bytes,
                                          void* pe_start, void* pe_stop, dg_stream_t stream) {
  DG_ARG(sc_operand && row_max && row_lnz && sc_on && canvas && E && prepared && x_out);
  DG_ARG(B > 0 && C > 0 && V > 0 && d > 0 && hidden > 0);
  DG_UNSUP(d % 128 == 0 && hidden % 128 == 0 && d <= 8192 && hidden <= 8192);
  const int64_t rows64 = static_cast<int64_t>(B) * C;
  DG_ARG(rows64 <= 65535);
  const int32_t rows = static_cast<int32_t>(rows64);
  const Bf16Plan p = bf16_plan(rows, V, d, hidden, true);
  DG_REQUIRE(ws != nullptr && ws_bytes >= p.bytes, DG_E_WORKSPACE);
  const PreparedLayout L = prepared_layout(V, d, hidden);
  const char* pb = reinterpret_cast<const char*>(prepared);
  const auto* et = reinterpret_cast<const _Float16*>(pb + L.off_et);
  const auto* wgu = reinterpret_cast<const _Float16*>(pb + L.off_wgu);
  const auto* wd = reinterpret_cast<const _Float16*>(pb + L.off_wd);
  // operand layout of dg_selfcond_operand_bytes: w [Kp / 32][Mp][32] fp16, then ref [rows][nchunk] f32
  const char* ob = reinterpret_cast<const char*>(sc_operand);
  const auto* w = reinterpret_cast<const _Float16*>(ob);
  const auto* ref = reinterpret_cast<const float*>(ob + round_up(static_cast<size_t>(p.Mp) * p.Kp * 2, 256));
  const int32_t nchunk = static_cast<int32_t>(cdiv(V, kScChunk));
  return selfcond_bf16_tail(p, w, ref, nchunk, row_max, row_lnz, sc_on, canvas, rows, C, E, et, wgu, wd, V, d, hidden,
                            x_out, s_out, y_out, reinterpret_cast<char*>(ws), pe_start, pe_stop, as_stream(stream));
}

extern "C" dg_status dg_selfcond_embed_lm(const void* lm_operand, const float* row_max, const float* row_lnz,
                                          const uint8_t* sc_on, const int32_t* canvas, int32_t B, int32_t C,
                                          const void* E, const void* prepared, int32_t V, int32_t d, int32_t hidden,
                                          void* x_out, float* s_out, float* y_out, void* ws, size_t ws_bytes,
                                          void* pe_start, void* pe_stop, dg_stream_t stream) {
  DG_ARG(lm_operand && row_max && row_lnz && sc_on && canvas && E && prepared && x_out);
  DG_ARG(B > 0 && C > 0 && V > 0 && d > 0 && hidden > 0);
  DG_UNSUP(V % 16 == 0 && d % 128 == 0 && hidden % 128 == 0 && d <= 8192 && hidden <= 8192);
  const int64_t rows64 = static_cast<int64_t>(B) * C;
  DG_ARG(rows64 <= 65535);
  const int32_t rows = static_cast<int32_t>(rows64);
  const Bf16Plan p = bf16_plan(rows, V, d, hidden, true);
  DG_REQUIRE(ws != nullptr && ws_bytes >= p.bytes, DG_E_WORKSPACE);
  const PreparedLayout L = prepared_layout(V, d, hidden);
  const char* pb = reinterpret_cast<const char*>(prepared);
  const auto* et = reinterpret_cast<const _Float16*>(pb + L.off_et);
  const auto* wgu = reinterpret_cast<const _Float16*>(pb + L.off_wgu);
  const auto* wd = reinterpret_cast<const _Float16*>(pb + L.off_wd);
  const LmOperandLayout O = lm_operand_layout(rows, V);
  const char* ob = reinterpret_cast<const char*>(lm_operand);
  return selfcond_bf16_tail(p, reinterpret_cast<const _Float16*>(ob), reinterpret_cast<const float*>(ob + O.off_ref),
                            O.nrun, row_max, row_lnz, sc_on, canvas, rows, C, E, et, wgu, wd, V, d, hidden, x_out,
                            s_out, y_out, reinterpret_cast<char*>(ws), pe_start, pe_stop, as_stream(stream), nullptr,
                            1.f, reinterpret_cast<const int32_t*>(ob + O.off_top));
}

extern "C" size_t dg_selfcond_prepared_bytes_e4m3(int32_t V, int32_t d, int32_t hidden) {
  if (V <= 0 || d <= 0 || hidden <= 0) return 0;
  return prepared_layout_e4m3(V, d, hidden).bytes;
}

extern "C" dg_status dg_selfcond_prepare_e4m3(const uint8_t* E8, const void* w_gate, const void* w_up,
                                              const void* w_down, int32_t V, int32_t d, int32_t hidden,
                                              void* prepared, size_t prepared_bytes, dg_stream_t stream) {
  DG_ARG(E8 && w_gate && w_up && w_down && prepared && V > 0 && d > 0 && hidden > 0);
  DG_UNSUP(d % 256 == 0 && hidden % 128 == 0 && d <= 8192 && hidden <= 8192);
  const PreparedLayout L = prepared_layout_e4m3(V, d, hidden);
  DG_REQUIRE(prepared_bytes >= L.bytes, DG_E_WORKSPACE);
  hipStream_t s = as_stream(stream);
  char* base = reinterpret_cast<char*>(prepared);
  auto* et8 = reinterpret_cast<uint8_t*>(base + L.off_et);
  auto* wgu = reinterpret_cast<_Float16*>(base + L.off_wgu);
  auto* wd = reinterpret_cast<_Float16*>(base + L.off_wd);
  // E8 [V][d] -> E8^T (d rows, Kp columns)
  transpose_e4m3_kernel<<<dim3(static_cast<unsigned>(cdiv(L.Kp, 64)), static_cast<unsigned>(cdiv(d, 64))), 256, 0,
                          s>>>(E8, V, d, L.Kp, et8);
  DG_LAUNCHED();
  transpose_bf16_to_f16_kernel<<<dim3(static_cast<unsigned>(cdiv(d, 64)), static_cast<unsigned>(cdiv(hidden, 64))),
                                 256, 0, s>>>(reinterpret_cast<const uint16_t*>(w_gate), d, hidden, d, 0, 2 * hidden,
                                              wgu);
  transpose_bf16_to_f16_kernel<<<dim3(static_cast<unsigned>(cdiv(d, 64)), static_cast<unsigned>(cdiv(hidden, 64))),
                                 256, 0, s>>>(reinterpret_cast<const uint16_t*>(w_up), d, hidden, d, hidden,
                                              2 * hidden, wgu);
  transpose_bf16_to_f16_kernel<<<dim3(static_cast<unsigned>(cdiv(hidden, 64)), static_cast<unsigned>(cdiv(d, 64))),
                                 256, 0, s>>>(reinterpret_cast<const uint16_t*>(w_down), hidden, d, hidden, 0, d, wd);
  DG_LAUNCHED();
  return DG_OK;
}

extern "C" dg_status dg_selfcond_embed_sc_e4m3(const void* sc_operand, const float* row_max, const float* row_lnz,
                                               const uint8_t* sc_on, const int32_t* canvas, int32_t B, int32_t C,
                                               const uint8_t* E8, float e_scale, const void* prepared, int32_t V,
                                               int32_t d, int32_t hidden, void* x_out, float* s_out, float* y_out,
                                               void* ws, size_t ws_bytes, void* pe_start, void* pe_stop,
                                               dg_stream_t stream) {
  DG_ARG(sc_operand && row_max && row_lnz && sc_on && canvas && E8 && prepared && x_out);
  DG_ARG(B > 0 && C > 0 && V > 0 && d > 0 && hidden > 0 && e_scale > 0.f && e_scale < INFINITY);
  DG_UNSUP(d % 256 == 0 && hidden % 128 == 0 && d <= 8192 && hidden <= 8192);
  const int64_t rows64 = static_cast<int64_t>(B) * C;
  DG_ARG(rows64 <= 65535);
  const int32_t rows = static_cast<int32_t>(rows64);
  const Bf16Plan p = bf16_plan(rows, V, d, hidden, true);
  DG_REQUIRE(ws != nullptr && ws_bytes >= p.bytes, DG_E_WORKSPACE);
  const PreparedLayout L = prepared_layout_e4m3(V, d, hidden);
  const char* pb = reinterpret_cast<const char*>(prepared);
  const auto* et8 = reinterpret_cast<const uint8_t*>(pb + L.off_et);
  const auto* wgu = reinterpret_cast<const _Float16*>(pb + L.off_wgu);
  const auto* wd = reinterpret_cast<const _Float16*>(pb + L.off_wd);
  const char* ob = reinterpret_cast<const char*>(sc_operand);
  const auto* w = reinterpret_cast<const _Float16*>(ob);
  const auto* ref = reinterpret_cast<const float*>(ob + round_up(static_cast<size_t>(p.Mp) * p.Kp * 2, 256));
  const int32_t nchunk = static_cast<int32_t>(cdiv(V, kScChunk));
  return selfcond_bf16_tail(p, w, ref, nchunk, row_max, row_lnz, sc_on, canvas, rows, C, E8, nullptr, wgu, wd, V, d,
                            hidden, x_out, s_out, y_out, reinterpret_cast<char*>(ws), pe_start, pe_stop,
                            as_stream(stream), et8, e_scale);
}
