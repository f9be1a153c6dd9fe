// dg_denoise_sample: one streaming pass over each logit row computing the
// softmax statistics (max, sum exp, sum exp * shifted logit), the entropy
// H = ln Z - S / Z, the argmax and the Gumbel-max candidate argmax(x + g).
//
// Method: DiffusionGemma/vLLM page, section "Entropy-based denoising" (entropy
// of every position's predicted distribution) and section
// "DiffusionGemmaModelState and DiffusionSampler", denoise case (temperature
// scaling, Gumbel-max candidate, argmax canvas).
//
// gfx950 design.  A row of V bf16 logits is split into `nsplit` chunks so that
// a launch has >= ~2048 workgroups of 256 lanes; each lane streams 16-byte
// loads (8 logits) with consecutive lanes on consecutive addresses.  Each
// lane keeps an online (m, Z, S) state, a (value, index) argmax and a
// (key, index) Gumbel candidate; the workgroup merges them with wave64
// shuffles and LDS, and a second small kernel merges the chunks of a row (the
// merge is associative, with lowest-index tie-breaks at every level).
//
// The Gumbel noise of element i is word i & 3 of Philox4x32-10 at counter
// (i >> 2, pos, step, 0): one Philox call per 4 logits.  Everything runs in
// base 2 (x2 = x log2 e): the softmax sums use the hardware exp2, and the
// Gumbel key is compared as x2 - log2(-log2 u), which orders elements exactly
// as x + g does; two hardware log2 per element, no branches.  The sampler is
// bound by this ALU work (Philox plus two transcendentals per logit), not by
// the logit bytes.
#include "dg_device.hpp"
#include "dg_host.hpp"

namespace dg {
namespace {

constexpr int kSampleThreads = 256;
constexpr int kGroup = 8;  // logits per lane per iteration (one 16-byte bf16 load)

struct Partial {
  float m, Z, S, amax_v;
  int32_t amax_i;
  float key_v;
  int32_t key_i;
  int32_t pad;
};
static_assert(sizeof(Partial) == 32, "partial layout");

// Online softmax state in base 2: m = max x2, Z = sum 2^(x2 - m), S = sum 2^(x2 - m) (x2 - m).
struct SoftState {
  float m, Z, S;
};

DG_DEV float exp2f_fast(float d) { return __builtin_amdgcn_exp2f(d); }

// merge b into a (both relative to their own max); Z == 0 marks an empty state
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

DG_DEV void wave_soft_merge(SoftState& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    SoftState t{__shfl_xor(s.m, o, kWave), __shfl_xor(s.Z, o, kWave), __shfl_xor(s.S, o, kWave)};
    soft_merge(s, t);
  }
}

// Gumbel-max key in log2 units.  With u = (2a + 1) 2^-24 (a = w >> 9, exact in fp32),
// g = -ln(-ln u) and x2 = x log2(e):
//   (x + g) log2(e) = x2 - log2(-log2 u) - log2(ln 2),
// so argmax_i (x_i + g_i) = argmax_i (x2_i - log2(-log2 u_i)) (a positive rescale and a shift).
// Both logs are the hardware base-2 logarithm on normal inputs (u >= 2^-24, -log2 u >= 2^-24 / ln 2).
DG_DEV float gumbel_key2(float x2, uint32_t w) {
  const float u = fmaf(static_cast<float>(w >> 9), 0x1.0p-23f, 0x1.0p-24f);
  const float L = -__builtin_amdgcn_logf(u);
  return x2 - __builtin_amdgcn_logf(L);
}

template <bool BF16>
DG_DEV void load8(const void* row, int64_t idx, float (&l)[kGroup]) {
  if constexpr (BF16) {
    const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(row) + idx);
    l[0] = bf16_lo(q.x); l[1] = bf16_hi(q.x);
    l[2] = bf16_lo(q.y); l[3] = bf16_hi(q.y);
    l[4] = bf16_lo(q.z); l[5] = bf16_hi(q.z);
    l[6] = bf16_lo(q.w); l[7] = bf16_hi(q.w);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(row) + idx);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(row) + idx + 4);
    l[0] = a.x; l[1] = a.y; l[2] = a.z; l[3] = a.w;
    l[4] = b.x; l[5] = b.y; l[6] = b.z; l[7] = b.w;
  }
}

template <bool BF16, bool ARGMAX_ONLY>
__global__ __launch_bounds__(kSampleThreads) void sample_partial_kernel(
    const void* __restrict__ logits, int64_t ld, int32_t V, int32_t rows_per_req, const uint64_t* __restrict__ seed,
    const int32_t* __restrict__ step, const uint8_t* __restrict__ active, float inv_t2, int32_t chunk,
    int32_t nsplit, Partial* __restrict__ part) {
  const int r = blockIdx.y;
  const int split = blockIdx.x;
  const int req = r / rows_per_req;
  if (active != nullptr && active[req] == 0) return;
  const int pos = r - req * rows_per_req;
  const int64_t c0 = static_cast<int64_t>(split) * chunk;
  const int64_t c1 = min<int64_t>(V, c0 + chunk);
  const char* row = reinterpret_cast<const char*>(logits) + r * ld * (BF16 ? 2 : 4);

  uint32_t k0 = 0, k1 = 0, st = 0;
  if constexpr (!ARGMAX_ONLY) {
    const uint64_t s = seed[req];
    k0 = static_cast<uint32_t>(s);
    k1 = static_cast<uint32_t>(s >> 32);
    st = static_cast<uint32_t>(step[req]);
  }

  float av = -INFINITY;
  int32_t ai = 0x7FFFFFFF;
  SoftState ss{-INFINITY, 0.f, 0.f};
  float kv = -INFINITY;
  int32_t ki = 0x7FFFFFFF;

  for (int64_t base = c0 + threadIdx.x * kGroup; base < c1; base += kSampleThreads * kGroup) {
    float l[kGroup];
    load8<BF16>(row, base, l);
    const bool full = base + kGroup <= c1;
    if (!full) {
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (base + j >= c1) l[j] = -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (l[j] > av) {
        av = l[j];
        ai = static_cast<int32_t>(base + j);
      }
    }
    if constexpr (!ARGMAX_ONLY) {
      // x2 = l * log2(e) / T: softmax statistics and keys in base 2 (S is rescaled by ln 2 at the end)
      float x[kGroup];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        x[j] = l[j] * inv_t2;
        mx = fmaxf(mx, x[j]);
      }
      if (mx > ss.m) {
        if (ss.Z != 0.f) {
          const float d = ss.m - mx;
          const float f = exp2f_fast(d);
          ss.S = f * (ss.S + d * ss.Z);
          ss.Z *= f;
        }
        ss.m = mx;
      }
      if (full) {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          const float d = x[j] - ss.m;
          const float e = exp2f_fast(d);
          ss.Z += e;
          ss.S = fmaf(e, d, ss.S);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          const float d = x[j] - ss.m;
          const float e = exp2f_fast(d);  // d = -inf -> 0
          ss.Z += e;
          ss.S = (e != 0.f) ? fmaf(e, d, ss.S) : ss.S;
        }
      }
      // Gumbel candidates: two Philox calls cover the 8 logits (base is a multiple of 8)
      const uint32_t c = static_cast<uint32_t>(base >> 2);
      const u32x4 wa = philox4x32_10(u32x4{c, static_cast<uint32_t>(pos), st, 0u}, k0, k1);
      const u32x4 wb = philox4x32_10(u32x4{c + 1u, static_cast<uint32_t>(pos), st, 0u}, k0, k1);
      const uint32_t w[kGroup] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const float key = gumbel_key2(x[j], w[j]);
        if (key > kv) {
          kv = key;
          ki = static_cast<int32_t>(base + j);
        }
      }
    }
  }

  // workgroup reduction: wave shuffles, then 4 waves through LDS
  wave_argmax(av, ai);
  if constexpr (!ARGMAX_ONLY) {
    wave_soft_merge(ss);
    wave_argmax(kv, ki);
  }
  __shared__ Partial red[kSampleThreads / kWave];
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wid] = Partial{ss.m, ss.Z, ss.S, av, ai, kv, ki, 0};
  __syncthreads();
  if (threadIdx.x == 0) {
    Partial p = red[0];
    SoftState a{p.m, p.Z, p.S};
    for (int w2 = 1; w2 < kSampleThreads / kWave; ++w2) {
      const Partial q = red[w2];
      argmax_merge(p.amax_v, p.amax_i, q.amax_v, q.amax_i);
      if constexpr (!ARGMAX_ONLY) {
        soft_merge(a, SoftState{q.m, q.Z, q.S});
        argmax_merge(p.key_v, p.key_i, q.key_v, q.key_i);
      }
    }
    p.m = a.m;
    p.Z = a.Z;
    p.S = a.S;
    part[static_cast<int64_t>(r) * nsplit + split] = p;
  }
}

template <bool ARGMAX_ONLY>
__global__ __launch_bounds__(kWave) void sample_merge_kernel(const Partial* __restrict__ part, int32_t nsplit,
                                                              int32_t rows_per_req,
                                                              const uint8_t* __restrict__ active,
                                                              float* __restrict__ entropy, int32_t* __restrict__ argmax,
                                                              int32_t* __restrict__ sample, float* __restrict__ row_max,
                                                              float* __restrict__ row_lnz) {
  const int r = blockIdx.x;
  if (active != nullptr && active[r / rows_per_req] == 0) return;
  float av = -INFINITY, kv = -INFINITY;
  int32_t ai = 0x7FFFFFFF, ki = 0x7FFFFFFF;
  SoftState ss{-INFINITY, 0.f, 0.f};
  for (int s = threadIdx.x; s < nsplit; s += kWave) {
    const Partial p = part[static_cast<int64_t>(r) * nsplit + s];
    argmax_merge(av, ai, p.amax_v, p.amax_i);
    if constexpr (!ARGMAX_ONLY) {
      soft_merge(ss, SoftState{p.m, p.Z, p.S});
      argmax_merge(kv, ki, p.key_v, p.key_i);
    }
  }
  wave_argmax(av, ai);
  if constexpr (!ARGMAX_ONLY) {
    wave_soft_merge(ss);
    wave_argmax(kv, ki);
  }
  if (threadIdx.x == 0) {
    argmax[r] = ai;
    if constexpr (!ARGMAX_ONLY) {
      // back to natural units: x = x2 ln 2, ln Z = log2(Z) ln 2, S_nat = S ln 2
      constexpr float kLn2 = 0.69314718055994531f;
      const float lnz = logf(ss.Z);
      entropy[r] = fmaxf(0.f, lnz - kLn2 * ss.S / ss.Z);
      sample[r] = ki;
      row_max[r] = ss.m * kLn2;
      row_lnz[r] = lnz;
    }
  }
}

struct SamplePlan {
  int32_t nsplit, chunk;
};

SamplePlan plan_sample(int32_t rows, int32_t V) {
  const int32_t per_iter = kSampleThreads * kGroup;  // 2048 logits per workgroup iteration
  const int32_t max_split = static_cast<int32_t>(cdiv(V, 4 * per_iter));
  int32_t nsplit = static_cast<int32_t>(cdiv(2048, rows));
  nsplit = max(1, min(nsplit, max_split));
  const int32_t chunk = static_cast<int32_t>(round_up(cdiv(V, nsplit), per_iter));
  nsplit = static_cast<int32_t>(cdiv(V, chunk));
  return {nsplit, chunk};
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" size_t dg_denoise_sample_ws_bytes(int32_t rows, int32_t V) {
  if (rows <= 0 || V <= 0) return 0;
  const SamplePlan p = plan_sample(rows, V);
  return static_cast<size_t>(rows) * p.nsplit * sizeof(Partial);
}

extern "C" dg_status dg_denoise_sample(const void* logits, int64_t ld, int32_t dtype, int32_t rows, int32_t V,
                                       int32_t rows_per_req, const uint64_t* seed, const int32_t* step,
                                       const uint8_t* active, float temperature, uint32_t flags, float* entropy,
                                       int32_t* argmax, int32_t* sample, float* row_max, float* row_lnz, void* ws,
                                       size_t ws_bytes, dg_stream_t stream) {
  const bool amax_only = (flags & DG_SAMPLE_ARGMAX_ONLY) != 0;
  DG_ARG(logits != nullptr && argmax != nullptr);
  DG_ARG(rows > 0 && V > 0 && rows_per_req > 0 && rows % rows_per_req == 0 && rows <= 65535);
  DG_ARG(ld >= V && (flags & ~static_cast<uint32_t>(DG_SAMPLE_ARGMAX_ONLY)) == 0);
  DG_UNSUP(dtype == DG_BF16 || dtype == DG_F32);
  DG_UNSUP(ld % 8 == 0 && aligned16(logits));
  if (!amax_only) {
    DG_ARG(entropy && sample && row_max && row_lnz && seed && step);
    DG_ARG(temperature > 0.f && temperature < INFINITY);
  }
  const size_t need = dg_denoise_sample_ws_bytes(rows, V);
  DG_REQUIRE(ws != nullptr && ws_bytes >= need, DG_E_WORKSPACE);
  const SamplePlan p = plan_sample(rows, V);
  hipStream_t s = as_stream(stream);
  Partial* part = reinterpret_cast<Partial*>(ws);
  const dim3 grid(p.nsplit, rows);
  const float inv_t = 1.4426950408889634f / temperature;  // log2(e) / T
  if (dtype == DG_BF16) {
    if (amax_only)
      sample_partial_kernel<true, true><<<grid, kSampleThreads, 0, s>>>(logits, ld, V, rows_per_req, seed, step,
                                                                         active, inv_t, p.chunk, p.nsplit, part);
    else
      sample_partial_kernel<true, false><<<grid, kSampleThreads, 0, s>>>(logits, ld, V, rows_per_req, seed, step,
                                                                          active, inv_t, p.chunk, p.nsplit, part);
  } else {
    if (amax_only)
      sample_partial_kernel<false, true><<<grid, kSampleThreads, 0, s>>>(logits, ld, V, rows_per_req, seed, step,
                                                                          active, inv_t, p.chunk, p.nsplit, part);
    else
      sample_partial_kernel<false, false><<<grid, kSampleThreads, 0, s>>>(logits, ld, V, rows_per_req, seed, step,
                                                                           active, inv_t, p.chunk, p.nsplit, part);
  }
  DG_LAUNCHED();
  if (amax_only)
    sample_merge_kernel<true><<<rows, kWave, 0, s>>>(part, p.nsplit, rows_per_req, active, entropy, argmax, sample,
                                                     row_max, row_lnz);
  else
    sample_merge_kernel<false><<<rows, kWave, 0, s>>>(part, p.nsplit, rows_per_req, active, entropy, argmax, sample,
                                                      row_max, row_lnz);
  DG_LAUNCHED();
  return DG_OK;
}
