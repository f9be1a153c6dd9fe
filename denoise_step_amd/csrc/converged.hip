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
#include "dg_device.hpp"
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
  constexpr int kWaves = N / kWave;
  __shared__ double wsum[kWaves];
  const int b = blockIdx.x;
  if (active != nullptr && active[b] == 0) return;
  const int t = threadIdx.x;
  const int64_t off = static_cast<int64_t>(b) * C;
  const int32_t sib = step_in_block[b];
  const int32_t g = step_global[b];
  const uint64_t sd = seed[b];

  if (sib < 0) {  // prefill case
    for (int p = t; p < C; p += N) canvas[off + p] = philox_token(sd, p, g, DG_STREAM_INIT, V);
    if (t == 0) {
      step_in_block[b] = 0;
      unchanged[b] = 0;
      sc_on[b] = 0;
      committed[b] = 0;
      num_sampled[b] = 0;
      step_global[b] = g + 1;
    }
    return;
  }

  int diff = 0;
  double hs = 0.0;
  for (int p = t; p < C; p += N) {
    diff |= argmax[off + p] != prev_argmax[off + p];
    hs += static_cast<double>(entropy[off + p]);
  }
  const int any_diff = __syncthreads_or(diff);
  hs = wave_sum_d(hs);
  if ((t & (kWave - 1)) == 0) wsum[t / kWave] = hs;
  __syncthreads();
  double total = 0.0;
  for (int w = 0; w < kWaves; ++w) total += wsum[w];
  const bool same = sib > 0 && !any_diff;
  const int32_t u = same ? unchanged[b] + 1 : 0;
  const double mean = total / static_cast<double>(C);
  const bool conv = u >= k && mean < tau;
  const bool commit = conv || (sib + 1 >= max_steps);
  __syncthreads();  // every lane has read unchanged[b] before lane 0 rewrites it
  for (int p = t; p < C; p += N) {
    const int32_t a = argmax[off + p];
    prev_argmax[off + p] = a;
    if (commit) {
      out_tokens[off + p] = a;
      canvas[off + p] = philox_token(sd, p, g, DG_STREAM_INIT, V);
    }
  }
  if (t == 0) {
    committed[b] = commit ? 1 : 0;
    num_sampled[b] = commit ? C : 0;
    if (commit) {
      steps_used[b] = sib + 1;
      unchanged[b] = 0;
      step_in_block[b] = 0;
      sc_on[b] = 0;
    } else {
      unchanged[b] = u;
      step_in_block[b] = sib + 1;
      sc_on[b] = 1;
    }
    step_global[b] = g + 1;
  }
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
