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
#include "canvas_update.hpp"
#include "dg_host.hpp"

namespace dg {
namespace {

template <int N>
__global__ __launch_bounds__(N) void accept_kernel(const float* __restrict__ entropy, const int32_t* __restrict__ sample,
                                                   int32_t C, int32_t V, double budget,
                                                   const uint64_t* __restrict__ seed, const int32_t* __restrict__ step,
                                                   const uint8_t* __restrict__ active, int32_t* __restrict__ canvas,
                                                   uint8_t* __restrict__ accept, int32_t* __restrict__ n_accept) {
  const int b = blockIdx.x;
  if (active != nullptr && active[b] == 0) return;
  accept_canvas<N>(b, entropy, sample, C, V, budget, seed, step, canvas, accept, n_accept);
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
