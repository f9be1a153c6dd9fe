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

// ---------------------------------------------------------------- bf16 path kernels
// w is written in the K-blocked layout with Mp rows (the GEMM's left operand).  A workgroup covers
// 8 rows x 256 columns: each row is read as 512 contiguous bytes and, for each of the 8 K slices of
// 32, the 8 rows are written as 512 contiguous bytes.
template <bool BF16>
__global__ __launch_bounds__(256) void probs_f16_kernel(const void* __restrict__ logits, int64_t ld, int32_t V,
                                                        int64_t Kp, int64_t Mp, int32_t rows, float inv_t,
                                                        const float* __restrict__ row_max, _Float16* __restrict__ w,
                                                        uint32_t* __restrict__ row_amax) {
  const int r = blockIdx.y * 8 + (threadIdx.x >> 5);
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 + (threadIdx.x & 31) * 8;
  if (r >= rows || i0 >= Kp) return;
  if (i0 == 0) row_amax[r] = 0u;  // consumed by the P.E reduce, which runs after the GEMM
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

DG_DEV float block_max_256(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

// Split-K reduce of the P.E partials: one thread per (row, column), 256 columns per workgroup:
// s = sum_split part * 2^-15 / Z -> s32 (and s_out); the row's largest |s| is folded into
// row_amax[r] with an atomic max on the (non-negative) fp32 bit pattern.
__global__ __launch_bounds__(256) void pe_reduce_kernel(const float* __restrict__ part, int32_t splits, int32_t M,
                                                        int32_t N, const float* __restrict__ row_lnz,
                                                        float* __restrict__ s32, float* __restrict__ s_out,
                                                        uint32_t* __restrict__ row_amax) {
  __shared__ float red[4];
  const int r = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const float f = (1.0f / kProbScale) * __expf(-row_lnz[r]);
  const int64_t idx = static_cast<int64_t>(r) * N + n;
  float v = 0.f;
  if (n < N) {
    float acc = 0.f;
    for (int k = 0; k < splits; ++k) acc += part[static_cast<int64_t>(k) * M * N + idx];
    v = acc * f;
    s32[idx] = v;
    if (s_out != nullptr) s_out[idx] = v;
  }
  const float amax = block_max_256(fabsf(v), red);
  if (threadIdx.x == 0) atomicMax(row_amax + r, __float_as_uint(amax));
}

// s16 = fp16(s * scale_r) in the K-blocked layout, scale_r the power of two that brings the row's
// largest |s| into (2^13, 2^14]; inv_scale[r] = 1 / scale_r.
__global__ __launch_bounds__(256) void pe_to_f16_kernel(const float* __restrict__ s32, int32_t N, int64_t Mp,
                                                        const uint32_t* __restrict__ row_amax,
                                                        _Float16* __restrict__ s16, float* __restrict__ inv_scale) {
  const int r = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const float sc = row_pow2_scale(__uint_as_float(row_amax[r]));
  if (n < N) s16[kblk_index(r, n, Mp)] = static_cast<_Float16>(s32[static_cast<int64_t>(r) * N + n] * sc);
  if (n == 0) inv_scale[r] = 1.f / sc;
}

DG_DEV float gelu_tanh(float z) {
  const float c = 0.7978845608028654f;  // sqrt(2 / pi)
  return 0.5f * z * (1.f + tanhf(c * (z + 0.044715f * z * z * z)));
}

// One workgroup per row: h = gelu_tanh(gate) * up from the partials of the [gate | up] GEMM (whose
// input row was scaled by 1 / s_inv[r]), then h16 = fp16(h * scale_r), h_inv[r] = 1 / scale_r.
__global__ __launch_bounds__(256) void glu_reduce_kernel(const float* __restrict__ part, int32_t splits, int32_t M,
                                                         int32_t H, int64_t Mp, const float* __restrict__ s_inv,
                                                         float* __restrict__ h32, _Float16* __restrict__ h16,
                                                         float* __restrict__ h_inv) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int64_t N2 = 2 * static_cast<int64_t>(H);
  const float si = s_inv[r];
  const int64_t base = static_cast<int64_t>(r) * H;
  float amax = 0.f;
  for (int j = threadIdx.x; j < H; j += 256) {
    float gsum = 0.f, usum = 0.f;
    for (int k = 0; k < splits; ++k) {
      const float* p = part + static_cast<int64_t>(k) * M * N2 + r * N2;
      gsum += p[j];
      usum += p[H + j];
    }
    const float h = gelu_tanh(gsum * si) * (usum * si);
    h32[base + j] = h;
    amax = fmaxf(amax, fabsf(h));
  }
  const float sc = row_pow2_scale(block_max_256(amax, red));
  for (int j = threadIdx.x; j < H; j += 256) h16[kblk_index(r, j, Mp)] = static_cast<_Float16>(h32[base + j] * sc);
  if (threadIdx.x == 0) h_inv[r] = 1.f / sc;
}

// x_out = bf16(E[canvas] + (sc_on ? y : 0)), y from the partials of the down GEMM
__global__ __launch_bounds__(256) void embed_reduce_kernel(const float* __restrict__ part, int32_t splits, int32_t M,
                                                           int32_t d, int32_t V, int32_t C,
                                                           const uint16_t* __restrict__ E,
                                                           const int32_t* __restrict__ canvas,
                                                           const uint8_t* __restrict__ sc_on,
                                                           const float* __restrict__ h_inv,
                                                           uint16_t* __restrict__ x_out, float* __restrict__ y_out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(M) * d) return;
  const int r = static_cast<int>(idx / d), c = static_cast<int>(idx - static_cast<int64_t>(r) * d);
  const int64_t tok = min(max(canvas[r], 0), V - 1);
  float x = bf16_to_f32(E[tok * d + c]);
  const bool on = sc_on[r / C] != 0;
  if (on || y_out != nullptr) {
    float y = 0.f;
    for (int k = 0; k < splits; ++k) y += part[static_cast<int64_t>(k) * M * d + idx];
    y *= h_inv[r];
    if (on) x += y;
    if (y_out != nullptr) y_out[idx] = y;
  }
  x_out[idx] = f32_to_bf16(x);
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

struct Bf16Plan {
  int64_t Kp, Mp;
  GemmPlan pe, g1, g2;
  size_t off_w, off_part, off_s16, off_h16, off_s32, off_h32, off_sinv, off_hinv, off_amax, bytes;
};

Bf16Plan bf16_plan(int32_t rows, int32_t V, int32_t d, int32_t hidden) {
  Bf16Plan p{};
  // GEMM left operands are allocated with whole 256-row tiles (the tail rows are read, never stored)
  const int64_t rows_p = (static_cast<int64_t>(rows) + kGemmTM - 1) / kGemmTM * kGemmTM;
  p.Mp = rows_p;
  p.Kp = pad128(V);
  p.pe = plan_gemm(rows, d, static_cast<int32_t>(p.Kp));
  p.g1 = plan_gemm(rows, 2 * hidden, d);
  p.g2 = plan_gemm(rows, d, hidden);
  size_t part = 0;
  part = std::max(part, static_cast<size_t>(p.pe.splits) * rows * d * 4);
  part = std::max(part, static_cast<size_t>(p.g1.splits) * rows * 2 * hidden * 4);
  part = std::max(part, static_cast<size_t>(p.g2.splits) * rows * d * 4);
  p.off_w = 0;
  p.off_part = round_up(p.off_w + static_cast<size_t>(rows_p) * p.Kp * 2, 256);
  p.off_s16 = round_up(p.off_part + part, 256);
  p.off_h16 = round_up(p.off_s16 + static_cast<size_t>(rows_p) * d * 2, 256);
  p.off_s32 = round_up(p.off_h16 + static_cast<size_t>(rows_p) * hidden * 2, 256);
  p.off_h32 = round_up(p.off_s32 + static_cast<size_t>(rows) * d * 4, 256);
  p.off_sinv = round_up(p.off_h32 + static_cast<size_t>(rows) * hidden * 4, 256);
  p.off_hinv = round_up(p.off_sinv + static_cast<size_t>(rows) * 4, 256);
  p.off_amax = round_up(p.off_hinv + static_cast<size_t>(rows) * 4, 256);
  p.bytes = round_up(p.off_amax + static_cast<size_t>(rows) * 4, 256);
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

template <int ROLE>
void launch_gemm(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  if (p.tn == 256)
    gemm_f16_splitk_kernel<ROLE, 256><<<p.grid, kGemmThreads, 0, s>>>(a);
  else
    gemm_f16_splitk_kernel<ROLE, 128><<<p.grid, kGemmThreads, 0, s>>>(a);
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
  DG_UNSUP(d % 128 == 0 && hidden % 128 == 0);
  DG_UNSUP(ld % 8 == 0 && aligned16(logits));
  const Bf16Plan p = bf16_plan(rows, V, d, hidden);
  DG_REQUIRE(ws != nullptr && ws_bytes >= p.bytes, DG_E_WORKSPACE);
  const PreparedLayout L = prepared_layout(V, d, hidden);
  const char* pb = reinterpret_cast<const char*>(prepared);
  const auto* et = reinterpret_cast<const _Float16*>(pb + L.off_et);
  const auto* wgu = reinterpret_cast<const _Float16*>(pb + L.off_wgu);
  const auto* wd = reinterpret_cast<const _Float16*>(pb + L.off_wd);
  auto* w = reinterpret_cast<_Float16*>(wsb + p.off_w);
  auto* part = reinterpret_cast<float*>(wsb + p.off_part);
  auto* s16 = reinterpret_cast<_Float16*>(wsb + p.off_s16);
  auto* h16 = reinterpret_cast<_Float16*>(wsb + p.off_h16);
  auto* s32 = reinterpret_cast<float*>(wsb + p.off_s32);
  auto* h32 = reinterpret_cast<float*>(wsb + p.off_h32);
  auto* s_inv = reinterpret_cast<float*>(wsb + p.off_sinv);
  auto* h_inv = reinterpret_cast<float*>(wsb + p.off_hinv);
  auto* row_amax = reinterpret_cast<uint32_t*>(wsb + p.off_amax);

  probs_f16_kernel<true><<<dim3(static_cast<unsigned>(cdiv(p.Kp, 256)), static_cast<unsigned>(cdiv(rows, 8))), 256, 0,
                          s>>>(logits, ld, V, p.Kp, p.Mp, rows, inv_t, row_max, w, row_amax);
  DG_LAUNCHED();
  if (pe_start != nullptr) DG_REQUIRE(hipEventRecord(reinterpret_cast<hipEvent_t>(pe_start), s) == hipSuccess, DG_E_HIP);
  launch_gemm<0>(p.pe, gemm_args(w, p.Mp, et, d, part, rows, d, static_cast<int32_t>(p.Kp), p.pe), s);
  DG_LAUNCHED();
  if (pe_stop != nullptr) DG_REQUIRE(hipEventRecord(reinterpret_cast<hipEvent_t>(pe_stop), s) == hipSuccess, DG_E_HIP);
  const dim3 rgrid(static_cast<unsigned>(cdiv(d, 256)), rows);
  pe_reduce_kernel<<<rgrid, 256, 0, s>>>(part, p.pe.splits, rows, d, row_lnz, s32, s_out, row_amax);
  DG_LAUNCHED();
  pe_to_f16_kernel<<<rgrid, 256, 0, s>>>(s32, d, p.Mp, row_amax, s16, s_inv);
  DG_LAUNCHED();
  launch_gemm<1>(p.g1, gemm_args(s16, p.Mp, wgu, 2 * hidden, part, rows, 2 * hidden, d, p.g1), s);
  DG_LAUNCHED();
  glu_reduce_kernel<<<rows, 256, 0, s>>>(part, p.g1.splits, rows, hidden, p.Mp, s_inv, h32, h16, h_inv);
  DG_LAUNCHED();
  launch_gemm<1>(p.g2, gemm_args(h16, p.Mp, wd, d, part, rows, d, hidden, p.g2), s);
  DG_LAUNCHED();
  embed_reduce_kernel<<<blocks_for(rows64 * d), 256, 0, s>>>(part, p.g2.splits, rows, d, V, C,
                                                             reinterpret_cast<const uint16_t*>(E), canvas, sc_on,
                                                             h_inv, reinterpret_cast<uint16_t*>(x_out), y_out);
  DG_LAUNCHED();
  return DG_OK;
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
