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
// gfx950 design: one workgroup per canvas (C <= 1024).  Keys (order-preserving
// fp32 bits << 32 | position) are unique and sorted by a bitonic network held in
// registers, one key per lane: exchanges between lanes of one wave64 are lane
// shuffles, only partners 64 or more apart go through LDS (3 barriers for
// C = 256).  The running total is an fp64 scan in a fixed order (shuffles in
// the wave, then the wave totals in wave order), so it is deterministic; the
// accept count is a block vote.
#include "dg_device.hpp"
#include "dg_host.hpp"

namespace dg {
namespace {

// order-preserving map of fp32 bits to uint32 (negative values flipped, -0 -> +0)
DG_DEV uint32_t float_order_bits(float h) {
  const uint32_t u = __float_as_uint(h + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

DG_DEV uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, kWave);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, kWave);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

DG_DEV double shfl_up_f64(double v, int d) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = __shfl_up(static_cast<uint32_t>(u), d, kWave);
  const uint32_t hi = __shfl_up(static_cast<uint32_t>(u >> 32), d, kWave);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

template <int N>
__global__ __launch_bounds__(N) void accept_kernel(const float* __restrict__ entropy, const int32_t* __restrict__ sample,
                                                   int32_t C, int32_t V, double budget,
                                                   const uint64_t* __restrict__ seed, const int32_t* __restrict__ step,
                                                   const uint8_t* __restrict__ active, int32_t* __restrict__ canvas,
                                                   uint8_t* __restrict__ accept, int32_t* __restrict__ n_accept) {
  constexpr int kWaves = N / kWave;
  __shared__ uint64_t xkey[2][N];  // cross-wave exchanges, alternating buffers
  __shared__ double wsum[kWaves];
  const int b = blockIdx.x;
  if (active != nullptr && active[b] == 0) return;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wave = t / kWave;
  const int64_t off = static_cast<int64_t>(b) * C;
  uint64_t kv = (t < C) ? ((static_cast<uint64_t>(float_order_bits(entropy[off + t])) << 32) | static_cast<uint32_t>(t))
                        : ~0ull;
  // bitonic network: after stage (k, j) lane t holds the key of position t; the lower lane of a
  // pair keeps the smaller key in ascending runs (t & k == 0) and the larger in descending runs
  int buf = 0;
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint64_t other;
      if (j >= kWave) {
        xkey[buf][t] = kv;
        __syncthreads();
        other = xkey[buf][t ^ j];
        buf ^= 1;  // the next cross-wave stage writes the other buffer, so no second barrier
      } else {
        other = shfl_xor_u64(kv, j);
      }
      const bool keep_min = ((t & j) == 0) == ((t & k) == 0);
      kv = keep_min ? (other < kv ? other : kv) : (other > kv ? other : kv);
    }
  }
  const int pos = static_cast<int>(kv & 0xFFFFFFFFu);
  // inclusive fp64 running total in sorted order: within the wave, then the earlier waves' totals
  double v = (t < C) ? static_cast<double>(entropy[off + pos]) : 0.0;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double u = shfl_up_f64(v, d);
    if (lane >= d) v += u;
  }
  if (lane == kWave - 1) wsum[wave] = v;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  v += before;
  const int n = __syncthreads_count(t < C && v <= budget);
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
