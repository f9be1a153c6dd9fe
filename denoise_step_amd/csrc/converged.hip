// dg_converged: per-request convergence test, commit of the argmax canvas and
// block restart (plus the prefill case that draws the first random canvas).
//
// Method: DiffusionGemma/vLLM page, section "Entropy-based denoising" (a
// canvas has converged when its argmax has not changed for several steps and
// its mean entropy is below a threshold; a step cap stops it otherwise; the
// clean argmax canvas is what is committed) and section
// "DiffusionGemmaModelState and DiffusionSampler" (prefill / denoise / commit
// cases, zero sampled tokens on denoise steps, C on a commit, state reset).
//
// gfx950 design: one workgroup per request; the whole-canvas equality is a
// block vote, the mean entropy an fp64 block sum in a fixed order.
#include "canvas_update.hpp"
#include "dg_host.hpp"

namespace dg {
namespace {

template <int N>
__global__ __launch_bounds__(N) void converged_kernel(
    const int32_t* __restrict__ argmax, const float* __restrict__ entropy, int32_t C, int32_t V, int32_t k, double tau,
    int32_t max_steps, const uint64_t* __restrict__ seed, const uint8_t* __restrict__ active,
    int32_t* __restrict__ prev_argmax, int32_t* __restrict__ unchanged, int32_t* __restrict__ step_in_block,
    int32_t* __restrict__ step_global, int32_t* __restrict__ canvas, uint8_t* __restrict__ sc_on,
    uint8_t* __restrict__ committed, int32_t* __restrict__ out_tokens, int32_t* __restrict__ steps_used,
    int32_t* __restrict__ num_sampled) {
  const int b = blockIdx.x;
  if (active != nullptr && active[b] == 0) return;
  converged_canvas<N>(b, argmax, entropy, C, V, k, tau, max_steps, seed, prev_argmax, unchanged, step_in_block,
                      step_global, canvas, sc_on, committed, out_tokens, steps_used, num_sampled);
}

// dg_accept_converged: a request in its prefill case (step_in_block < 0) gets only dg_converged's
// prefill; every other active request gets dg_entropy_accept (renoise at its current global step)
// and then dg_converged, in one workgroup, with a barrier between the two.
template <int N>
__global__ __launch_bounds__(N) void accept_converged_kernel(
    const float* __restrict__ entropy, const int32_t* __restrict__ sample, const int32_t* __restrict__ argmax,
    int32_t C, int32_t V, double budget, int32_t k, double tau, int32_t max_steps, const uint64_t* __restrict__ seed,
    const uint8_t* __restrict__ active, int32_t* __restrict__ prev_argmax, int32_t* __restrict__ unchanged,
    int32_t* __restrict__ step_in_block, int32_t* __restrict__ step_global, int32_t* __restrict__ canvas,
    uint8_t* __restrict__ sc_on, uint8_t* __restrict__ committed, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ steps_used, int32_t* __restrict__ num_sampled, uint8_t* __restrict__ accept,
    int32_t* __restrict__ n_accept) {
  const int b = blockIdx.x;
  if (active != nullptr && active[b] == 0) return;
  if (step_in_block[b] >= 0) {
    accept_canvas<N>(b, entropy, sample, C, V, budget, seed, step_global, canvas, accept, n_accept);
    __syncthreads();  // the accepted canvas is complete before a commit overwrites it
  }
  converged_canvas<N>(b, argmax, entropy, C, V, k, tau, max_steps, seed, prev_argmax, unchanged, step_in_block,
                      step_global, canvas, sc_on, committed, out_tokens, steps_used, num_sampled);
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" dg_status dg_converged(const int32_t* argmax, const float* entropy, int32_t B, int32_t C, int32_t V,
                                  int32_t k, double tau, int32_t max_steps, const uint64_t* seed,
                                  const uint8_t* active, int32_t* prev_argmax, int32_t* unchanged,
                                  int32_t* step_in_block, int32_t* step_global, int32_t* canvas, uint8_t* sc_on,
                                  uint8_t* committed, int32_t* out_tokens, int32_t* steps_used, int32_t* num_sampled,
                                  dg_stream_t stream) {
  DG_ARG(argmax && entropy && seed && prev_argmax && unchanged && step_in_block && step_global && canvas && sc_on &&
         committed && out_tokens && steps_used && num_sampled);
  DG_ARG(B > 0 && C > 0 && C <= 1024 && V > 0 && k >= 0 && max_steps > 0 && tau == tau);
  hipStream_t s = as_stream(stream);
#define DG_CONV_LAUNCH(N)                                                                                    \
  converged_kernel<N><<<B, N, 0, s>>>(argmax, entropy, C, V, k, tau, max_steps, seed, active, prev_argmax, \
                                      unchanged, step_in_block, step_global, canvas, sc_on, committed,      \
                                      out_tokens, steps_used, num_sampled)
  if (C <= 64)
    DG_CONV_LAUNCH(64);
  else if (C <= 256)
    DG_CONV_LAUNCH(256);
  else
    DG_CONV_LAUNCH(1024);
#undef DG_CONV_LAUNCH
  DG_LAUNCHED();
  return DG_OK;
}

extern "C" dg_status dg_accept_converged(const float* entropy, const int32_t* sample, const int32_t* argmax, int32_t B,
                                         int32_t C, int32_t V, double budget, int32_t k, double tau, int32_t max_steps,
                                         const uint64_t* seed, const uint8_t* active, int32_t* prev_argmax,
                                         int32_t* unchanged, int32_t* step_in_block, int32_t* step_global,
                                         int32_t* canvas, uint8_t* sc_on, uint8_t* committed, int32_t* out_tokens,
                                         int32_t* steps_used, int32_t* num_sampled, uint8_t* accept,
                                         int32_t* n_accept, dg_stream_t stream) {
  DG_ARG(entropy && sample && argmax && seed && prev_argmax && unchanged && step_in_block && step_global && canvas &&
         sc_on && committed && out_tokens && steps_used && num_sampled);
  DG_ARG(B > 0 && C > 0 && C <= 1024 && V > 0 && k >= 0 && max_steps > 0 && tau == tau && budget == budget);
  hipStream_t s = as_stream(stream);
#define DG_AC_LAUNCH(N)                                                                                        \
  accept_converged_kernel<N><<<B, N, 0, s>>>(entropy, sample, argmax, C, V, budget, k, tau, max_steps, seed,   \
                                             active, prev_argmax, unchanged, step_in_block, step_global, canvas, \
                                             sc_on, committed, out_tokens, steps_used, num_sampled, accept,    \
                                             n_accept)
  if (C <= 64)
    DG_AC_LAUNCH(64);
  else if (C <= 128)
    DG_AC_LAUNCH(128);
  else if (C <= 256)
    DG_AC_LAUNCH(256);
  else if (C <= 512)
    DG_AC_LAUNCH(512);
  else
    DG_AC_LAUNCH(1024);
#undef DG_AC_LAUNCH
  DG_LAUNCHED();
  return DG_OK;
}
