// Per-canvas bodies of dg_entropy_accept and dg_converged (one workgroup of N threads per canvas),
// shared by their own kernels and by the fused dg_accept_converged.
#pragma once
#include "dg_device.hpp"

namespace dg {

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

// dg_entropy_accept on canvas b (N >= C, a power of two): see accept.hip.
template <int N>
DG_DEV void accept_canvas(int b, const float* __restrict__ entropy, const int32_t* __restrict__ sample, int32_t C,
                          int32_t V, double budget, const uint64_t* __restrict__ seed, const int32_t* __restrict__ step,
                          int32_t* __restrict__ canvas, uint8_t* __restrict__ accept, int32_t* __restrict__ n_accept) {
  constexpr int kWaves = N / kWave;
  __shared__ uint64_t xkey[2][N];  // cross-wave exchanges, alternating buffers
  __shared__ double wsum[kWaves];
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

// dg_converged on canvas b: see converged.hip.
template <int N>
DG_DEV void converged_canvas(int b, const int32_t* __restrict__ argmax, const float* __restrict__ entropy, int32_t C,
                             int32_t V, int32_t k, double tau, int32_t max_steps, const uint64_t* __restrict__ seed,
                             int32_t* __restrict__ prev_argmax, int32_t* __restrict__ unchanged,
                             int32_t* __restrict__ step_in_block, int32_t* __restrict__ step_global,
                             int32_t* __restrict__ canvas, uint8_t* __restrict__ sc_on, uint8_t* __restrict__ committed,
                             int32_t* __restrict__ out_tokens, int32_t* __restrict__ steps_used,
                             int32_t* __restrict__ num_sampled) {
  constexpr int kWaves = N / kWave;
  __shared__ double wsum[kWaves];
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

}  // namespace dg
