// Small entry points: version / status strings, device Philox, greedy block
// verification, allowed-choice readout, row gather and the fp32 linear layer
// of the tiny backbone.
#include "dg_device.hpp"
#include "dg_host.hpp"

namespace dg {
namespace {

__global__ void philox_kernel(const uint32_t* __restrict__ ctr, const uint32_t* __restrict__ key, int64_t n,
                              uint32_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const u32x4 r = philox4x32_10(u32x4{ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]}, key[2 * i],
                                key[2 * i + 1]);
  out[4 * i] = r.x;
  out[4 * i + 1] = r.y;
  out[4 * i + 2] = r.z;
  out[4 * i + 3] = r.w;
}

// Greedy verification (DFlash page, "What DFlash does differently", verification step):
// accepted length = first mismatch index, or L.  One wave per request.
__global__ __launch_bounds__(kWave) void verify_kernel(const int32_t* __restrict__ draft,
                                                       const int32_t* __restrict__ target, int32_t L,
                                                       int32_t* __restrict__ accepted) {
  const int b = blockIdx.x;
  int first = L;
  for (int j = threadIdx.x; j < L; j += kWave)
    if (draft[static_cast<int64_t>(b) * L + j] != target[static_cast<int64_t>(b) * L + j]) {
      first = min(first, j);
      break;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o, kWave));
  if (threadIdx.x == 0) accepted[b] = first;
}

// Structured-read readout (single-pass-reads page, answer slots): one wave per slot,
// one allowed id per lane (<= 64 ids).
template <bool BF16>
__global__ __launch_bounds__(kWave) void allowed_probs_kernel(const void* __restrict__ logits, int64_t ld,
                                                              int32_t n_rows, int32_t V,
                                                              const int32_t* __restrict__ slot_row,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ ids, float inv_t,
                                                              float* __restrict__ q, int32_t* __restrict__ answer) {
  const int s = blockIdx.x;
  const int t = threadIdx.x;
  const int32_t o0 = offsets[s], n = min(offsets[s + 1] - o0, kWave);
  const int64_t row = min(max(slot_row[s], 0), n_rows - 1);
  float x = -INFINITY;
  int32_t id = 0x7FFFFFFF;
  if (t < n) {
    id = min(max(ids[o0 + t], 0), V - 1);
    x = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(logits)[row * ld + id])
             : reinterpret_cast<const float*>(logits)[row * ld + id];
    x *= inv_t;
  }
  // argmax over list order: lowest list position wins ties
  float bv = x;
  int32_t bi = (t < n) ? t : 0x7FFFFFFF;
  wave_argmax(bv, bi);
  const float e = (t < n) ? __expf(x - bv) : 0.f;
  const float z = wave_sum(e);
  if (t < n) q[o0 + t] = e / z;
  if (t == 0) answer[s] = (n > 0) ? min(max(ids[o0 + bi], 0), V - 1) : -1;
}

template <bool BF16>
__global__ void gather_rows_kernel(const void* __restrict__ table, int32_t n_table, int32_t d,
                                   const int32_t* __restrict__ idx, void* __restrict__ out) {
  const int i = blockIdx.x;  // one workgroup per index: the grid is the index count
  const int64_t src = min(max(idx[i], 0), n_table - 1);
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    if constexpr (BF16)
      reinterpret_cast<uint16_t*>(out)[static_cast<int64_t>(i) * d + c] =
          reinterpret_cast<const uint16_t*>(table)[src * d + c];
    else
      reinterpret_cast<float*>(out)[static_cast<int64_t>(i) * d + c] =
          reinterpret_cast<const float*>(table)[src * d + c];
  }
}

// fp32 C = alpha * A op(B) (+ residual): 16x16 output tile per 256-lane workgroup, K staged
// through LDS in 16-wide slabs.  Only used at the tiny backbone's sizes.
template <bool TRANS_B>
__global__ __launch_bounds__(256) void linear_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                         const float* __restrict__ R, float* __restrict__ Cm,
                                                         int32_t M, int32_t N, int32_t K, float alpha) {
  __shared__ float As[16][17];
  __shared__ float Bs[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m = blockIdx.y * 16 + ty, n = blockIdx.x * 16 + tx;
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int am = blockIdx.y * 16 + ty, ak = k0 + tx;
    As[ty][tx] = (am < M && ak < K) ? A[static_cast<int64_t>(am) * K + ak] : 0.f;
    const int bk = k0 + ty, bn = blockIdx.x * 16 + tx;
    float bv = 0.f;
    if (bk < K && bn < N) bv = TRANS_B ? B[static_cast<int64_t>(bn) * K + bk] : B[static_cast<int64_t>(bk) * N + bn];
    Bs[ty][tx] = bv;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(As[ty][kk], Bs[kk][tx], acc);
    __syncthreads();
  }
  if (m < M && n < N) {
    float v = alpha * acc;
    if (R != nullptr) v += R[static_cast<int64_t>(m) * N + n];
    Cm[static_cast<int64_t>(m) * N + n] = v;
  }
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" int32_t dg_version(void) { return 100; }

extern "C" const char* dg_status_str(dg_status s) {
  switch (s) {
    case DG_OK: return "ok";
    case DG_E_ARG: return "invalid argument";
    case DG_E_UNSUPPORTED: return "unsupported dtype, size or alignment";
    case DG_E_WORKSPACE: return "workspace missing or too small";
    case DG_E_HIP: return "HIP launch error";
    case DG_E_SCRATCH: return "input larger than the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

extern "C" dg_status dg_philox4x32_10(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out,
                                      dg_stream_t stream) {
  DG_ARG(ctr && key && out && n > 0 && n < (int64_t(1) << 40));
  philox_kernel<<<static_cast<unsigned>(cdiv(n, 256)), 256, 0, as_stream(stream)>>>(ctr, key, n, out);
  DG_LAUNCHED();
  return DG_OK;
}

namespace dg {
namespace {
// 8 codes per thread through both conversions the kernels use (fp32 for the embedding rows, fp16
// for the GEMM operand)
__global__ void e4m3_decode_kernel(const uint8_t* __restrict__ codes, int64_t n8, float scale,
                                   float* __restrict__ out32, _Float16* __restrict__ out16) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint2 q = *reinterpret_cast<const uint2*>(codes + 8 * i);
  const float4 a = e4m3x4_to_float4(q.x), b = e4m3x4_to_float4(q.y);
  *reinterpret_cast<float4*>(out32 + 8 * i) = make_float4(a.x * scale, a.y * scale, a.z * scale, a.w * scale);
  *reinterpret_cast<float4*>(out32 + 8 * i + 4) = make_float4(b.x * scale, b.y * scale, b.z * scale, b.w * scale);
  if (out16 != nullptr) *reinterpret_cast<half8*>(out16 + 8 * i) = e4m3x8_to_half8(q.x, q.y);
}
}  // namespace
}  // namespace dg

extern "C" dg_status dg_e4m3_decode(const uint8_t* codes, int64_t n, float scale, float* out32, void* out16,
                                    dg_stream_t stream) {
  DG_ARG(codes && out32 && n > 0 && n % 8 == 0 && n < (int64_t(1) << 40));
  DG_UNSUP(aligned16(codes) && aligned16(out32) && (out16 == nullptr || aligned16(out16)));
  e4m3_decode_kernel<<<static_cast<unsigned>(cdiv(n / 8, 256)), 256, 0, as_stream(stream)>>>(
      codes, n / 8, scale, out32, reinterpret_cast<_Float16*>(out16));
  DG_LAUNCHED();
  return DG_OK;
}

extern "C" dg_status dg_verify_prefix(const int32_t* draft, const int32_t* target, int32_t B, int32_t L,
                                      int32_t* accepted, dg_stream_t stream) {
  DG_ARG(draft && target && accepted && B > 0 && L > 0);
  verify_kernel<<<B, kWave, 0, as_stream(stream)>>>(draft, target, L, accepted);
  DG_LAUNCHED();
  return DG_OK;
}

extern "C" dg_status dg_allowed_probs(const void* logits, int64_t ld, int32_t dtype, int32_t n_rows,
                                      int32_t n_slots, int32_t V, const int32_t* slot_row, const int32_t* offsets,
                                      const int32_t* ids, float temperature, float* q, int32_t* answer,
                                      dg_stream_t stream) {
  DG_ARG(logits && slot_row && offsets && ids && q && answer);
  DG_ARG(n_rows > 0 && n_slots > 0 && V > 0 && ld >= V && temperature > 0.f);
  DG_UNSUP(dtype == DG_BF16 || dtype == DG_F32);
  const float inv_t = 1.0f / temperature;
  if (dtype == DG_BF16)
    allowed_probs_kernel<true><<<n_slots, kWave, 0, as_stream(stream)>>>(logits, ld, n_rows, V, slot_row, offsets,
                                                                         ids, inv_t, q, answer);
  else
    allowed_probs_kernel<false><<<n_slots, kWave, 0, as_stream(stream)>>>(logits, ld, n_rows, V, slot_row, offsets,
                                                                          ids, inv_t, q, answer);
  DG_LAUNCHED();
  return DG_OK;
}

extern "C" dg_status dg_gather_rows(const void* table, int32_t n_table, int32_t d, int32_t dtype, const int32_t* idx,
                                    int32_t n, void* out, dg_stream_t stream) {
  DG_ARG(table && idx && out && n_table > 0 && d > 0 && n > 0);
  DG_UNSUP(dtype == DG_BF16 || dtype == DG_F32);
  if (dtype == DG_BF16)
    gather_rows_kernel<true><<<n, 256, 0, as_stream(stream)>>>(table, n_table, d, idx, out);
  else
    gather_rows_kernel<false><<<n, 256, 0, as_stream(stream)>>>(table, n_table, d, idx, out);
  DG_LAUNCHED();
  return DG_OK;
}

extern "C" dg_status dg_linear(const float* A, const float* B, const float* residual, float* C, int32_t M, int32_t N,
                               int32_t K, int32_t trans_b, float alpha, dg_stream_t stream) {
  DG_ARG(A && B && C && M > 0 && N > 0 && K > 0);
  const dim3 grid(static_cast<unsigned>(cdiv(N, 16)), static_cast<unsigned>(cdiv(M, 16)));
  if (trans_b)
    linear_f32_kernel<true><<<grid, 256, 0, as_stream(stream)>>>(A, B, residual, C, M, N, K, alpha);
  else
    linear_f32_kernel<false><<<grid, 256, 0, as_stream(stream)>>>(A, B, residual, C, M, N, K, alpha);
  DG_LAUNCHED();
  return DG_OK;
}
