// dg_entropy_accept: per canvas, order positions by (entropy, position),
// accept the longest prefix whose running entropy total stays within the
// budget, keep the Gumbel candidate there and renoise everything else.
//
// Method: DiffusionGemma/vLLM page, section "Entropy-based denoising"
// (acceptance from the most to the least confident position until the
// cumulative entropy would exceed the budget; the rest are replaced by random
// tokens) and section "DiffusionGemmaModelState and DiffusionSampler"
// (denoise case).
//
// gfx950 design: one workgroup per canvas (C <= 1024 = one LDS-resident
// problem).  Keys (order-preserving fp32 bits << 32 | position) are sorted by
// a bitonic network in LDS; the running total is an fp64 Hillis-Steele scan
// in LDS (fixed order -> deterministic); the accept count is a block vote.
#include "dg_device.hpp"
#include "dg_host.hpp"

namespace dg {
namespace {

// order-preserving map of fp32 bits to uint32 (negative values flipped, -0 -> +0)
DG_DEV uint32_t float_order_bits(float h) {
  const uint32_t u = __float_as_uint(h + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int N>
__global__ __launch_bounds__(N) void accept_kernel(const float* __restrict__ entropy, const int32_t* __restrict__ sample,
                                                   int32_t C, int32_t V, double budget,
                                                   const uint64_t* __restrict__ seed, const int32_t* __restrict__ step,
                                                   const uint8_t* __restrict__ active, int32_t* __restrict__ canvas,
                                                   uint8_t* __restrict__ accept, int32_t* __restrict__ n_accept) {
  __shared__ uint64_t key[N];
  __shared__ double scan[2][N];
  const int b = blockIdx.x;
  if (active != nullptr && active[b] == 0) return;
  const int t = threadIdx.x;
  const int64_t off = static_cast<int64_t>(b) * C;
  key[t] = (t < C) ? ((static_cast<uint64_t>(float_order_bits(entropy[off + t])) << 32) | static_cast<uint32_t>(t))
                   : ~0ull;
  __syncthreads();
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int p = t ^ j;
      if (p > t) {
        const uint64_t a = key[t], c = key[p];
        const bool up = (t & k) == 0;
        if ((a > c) == up) {
          key[t] = c;
          key[p] = a;
        }
      }
      __syncthreads();
    }
  }
  const int pos = static_cast<int>(key[t] & 0xFFFFFFFFu);
  scan[0][t] = (t < C) ? static_cast<double>(entropy[off + pos]) : 0.0;
  __syncthreads();
  int cur = 0;
  for (int d = 1; d < N; d <<= 1) {
    const double v = scan[cur][t] + ((t >= d) ? scan[cur][t - d] : 0.0);
    scan[cur ^ 1][t] = v;
    cur ^= 1;
    __syncthreads();
  }
  const int n = __syncthreads_count(t < C && scan[cur][t] <= budget);
  if (t < C) {
    const bool acc = t < n;
    const int32_t tok = acc ? sample[off + pos]
                            : philox_token(seed[b], pos, step[b], DG_STREAM_RENOISE, V);
    canvas[off + pos] = tok;
    if (accept != nullptr) accept[off + pos] = acc ? 1 : 0;
  }
  if (t == 0 && n_accept != nullptr) n_accept[b] = n;
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" dg_status dg_entropy_accept(const float* entropy, const int32_t* sample, int32_t B, int32_t C, int32_t V,
                                       double budget, const uint64_t* seed, const int32_t* step,
                                       const uint8_t* active, int32_t* canvas, uint8_t* accept, int32_t* n_accept,
                                       dg_stream_t stream) {
  DG_ARG(entropy && sample && seed && step && canvas);
  DG_ARG(B > 0 && C > 0 && C <= 1024 && V > 0);
  DG_ARG(budget == budget);  // not NaN
  hipStream_t s = as_stream(stream);
#define DG_ACCEPT_LAUNCH(N)                                                                                      \
  accept_kernel<N><<<B, N, 0, s>>>(entropy, sample, C, V, budget, seed, step, active, canvas, accept, n_accept)
  if (C <= 64)
    DG_ACCEPT_LAUNCH(64);
  else if (C <= 128)
    DG_ACCEPT_LAUNCH(128);
  else if (C <= 256)
    DG_ACCEPT_LAUNCH(256);
  else if (C <= 512)
    DG_ACCEPT_LAUNCH(512);
  else
    DG_ACCEPT_LAUNCH(1024);
#undef DG_ACCEPT_LAUNCH
  DG_LAUNCHED();
  return DG_OK;
}
