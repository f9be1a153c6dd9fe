// dg_denoise_sample: one streaming pass over each logit row computing the
// softmax statistics (max, sum exp, sum exp * shifted logit), the entropy
// H = ln Z - S / Z, the argmax and a Gumbel-max candidate.
//
// Method: DiffusionGemma/vLLM page, section "Entropy-based denoising" (entropy
// of every position's predicted distribution) and section
// "DiffusionGemmaModelState and DiffusionSampler", denoise case (temperature
// scaling, Gumbel-max candidate, argmax canvas).
//
// The candidate is drawn in two levels over blocks of 16 consecutive ids: the
// winning block is argmax_b (L_b + G_b) with L_b = ln sum_{i in b} e^{x_i} and
// one Gumbel value G_b per block (Philox stream 0, block b -> word (b >> 7) & 3
// of counter 128 (b >> 9) + (b & 127)); inside it, argmax_i (x_i + g_i) with
// per-element noise (stream 3, word i & 3 of counter i >> 2).  The maximum of
// Gumbel-perturbed values over a set is Gumbel with the set's log-mass as its
// location and an independent argmax, so the candidate follows softmax(x)
// exactly, with one Philox word per 16 logits on the streaming pass.
//
// gfx950 design.  A workgroup (256 lanes) covers 16384 logits per iteration as
// eight rounds of 16-byte loads with consecutive lanes on consecutive
// addresses; the two lanes of a pair hold one 16-id block per round.  Each
// lane keeps an online base-2 softmax state (m, Z, S) whose reference m is
// shared with its pair partner (one DPP swap), so the pair's half-sums of a
// block add up directly; lane h of the pair scores the blocks of rounds
// 4h .. 4h + 3, which the block map puts under one Philox counter (one
// Philox call per lane per iteration).  The argmax is tracked per 8-logit
// group and resolved to its first index at the end.  The workgroup merges its
// lanes with wave64 shuffles and LDS; a second small kernel merges the chunks
// of a row (associative, lowest-index tie-breaks at every level) and draws
// the element inside the winning block.
#include <mutex>

#include "dg_device.hpp"
#include "dg_host.hpp"

namespace dg {
namespace {

constexpr int kSampleThreads = 256;
constexpr int kGroup = 8;                                        // logits per 16-byte bf16 load
constexpr int kRounds = 8;                                       // loads per lane per iteration
constexpr int kIterElems = kSampleThreads * kRounds * kGroup;    // 16384 logits per workgroup iteration
constexpr int kBlock = 16;                                       // ids per block of the first level

struct Partial {
  float m, Z, S, amax_v;
  int32_t amax_i;
  float key_v;
  int32_t key_b;  // block of the best first-level key
  int32_t pad;
};
static_assert(sizeof(Partial) == 32, "partial layout");

// value of the neighbouring lane (lane ^ 1), one DPP move
DG_DEV float pair_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));

// 8 logits from a 16-byte aligned index; the streaming loads are non-temporal (each logit is read once)
template <bool BF16>
DG_DEV void load8(const void* row, int64_t idx, float (&l)[kGroup]) {
  if constexpr (BF16) {
    const u32v4 q = __builtin_nontemporal_load(reinterpret_cast<const u32v4*>(reinterpret_cast<const uint16_t*>(row) + idx));
    l[0] = bf16_lo(q.x); l[1] = bf16_hi(q.x);
    l[2] = bf16_lo(q.y); l[3] = bf16_hi(q.y);
    l[4] = bf16_lo(q.z); l[5] = bf16_hi(q.z);
    l[6] = bf16_lo(q.w); l[7] = bf16_hi(q.w);
  } else {
    const u32v4 a = __builtin_nontemporal_load(reinterpret_cast<const u32v4*>(reinterpret_cast<const float*>(row) + idx));
    const u32v4 b = __builtin_nontemporal_load(reinterpret_cast<const u32v4*>(reinterpret_cast<const float*>(row) + idx + 4));
    l[0] = __uint_as_float(a.x); l[1] = __uint_as_float(a.y); l[2] = __uint_as_float(a.z); l[3] = __uint_as_float(a.w);
    l[4] = __uint_as_float(b.x); l[5] = __uint_as_float(b.y); l[6] = __uint_as_float(b.z); l[7] = __uint_as_float(b.w);
  }
}

template <bool BF16>
DG_DEV float load1(const void* row, int64_t idx) {
  if constexpr (BF16)
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[idx]);
  else
    return reinterpret_cast<const float*>(row)[idx];
}

// Per-lane state of the streaming pass.
struct LaneState {
  float av;     // largest logit seen
  int32_t ag;   // first index of the 8-logit group holding it (-1: none; a row index fits in int32)
  SoftState ss;
  float kv;     // best first-level key (log2 units)
  int32_t kb;   // its block
};

// Self-conditioning operand written by the pass (dg_denoise_sample_sc): w[r][k] = fp16(2^15 2^(x2_k -
// ref_{r,j})) in the K-blocked layout with Mp rows, k < Kp (zero past V), where ref_{r,j} is the
// largest x2 of the row's j-th run of 16384 logits; ref [rows][nchunk].
struct ScOut {
  _Float16* w;
  int64_t Mp, Kp;
  float* ref;
  int32_t nchunk;
  int32_t row;
};

// One iteration of a workgroup: logits E .. E + 16384 of the row.  FULL: all of them are < V.
// SC: the exponentials of the iteration use the workgroup's largest logit of the iteration as their
// reference (one block-wide max through `red`), are written as the self-conditioning operand and are
// folded into the lane's running softmax state.
template <bool BF16, bool ARGMAX_ONLY, bool FULL, bool SC>
DG_DEV void sample_iteration(const char* row, int64_t E, int32_t V, float c, uint32_t pos, uint32_t st, uint32_t k0,
                             uint32_t k1, LaneState& ls, const ScOut& so, float* red) {
  const int t = threadIdx.x, h = t & 1, pr = t >> 1;
  float l[kRounds][kGroup];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int64_t e0 = E + q * (kSampleThreads * kGroup) + kGroup * t;
    if (FULL) {
      load8<BF16>(row, e0, l[q]);
    } else if (e0 < V) {  // the 8-aligned group ends within ld: in bounds
      load8<BF16>(row, e0, l[q]);
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (e0 + j >= V) l[q][j] = -INFINITY;
    } else {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) l[q][j] = -INFINITY;
    }
  }
  float gm[kRounds];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    float v = l[q][0];
#pragma unroll
    for (int j = 1; j < kGroup; ++j) v = __builtin_elementwise_maximum(v, l[q][j]);  // v_maximum3_f32 chains
    gm[q] = v;
    const bool better = v > ls.av;
    ls.av = better ? v : ls.av;
    ls.ag = better ? static_cast<int32_t>(E) + q * (kSampleThreads * kGroup) + kGroup * t : ls.ag;
  }
  if constexpr (!ARGMAX_ONLY) {
    float mx = gm[0];
#pragma unroll
    for (int q = 1; q < kRounds; ++q) mx = __builtin_elementwise_maximum(mx, gm[q]);
    // reference of this iteration's exponentials: shared by the lane pair (the pair's running max in
    // base 2), or by the whole workgroup (the iteration's max) when the operand is written
    float m;
    if constexpr (SC) {
      const float mw = dpp_wave_max(mx * c);
      if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = mw;
      __syncthreads();
      m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      __syncthreads();  // red is reused by the next iteration
    } else {
      float mn = fmaxf(ls.ss.m, mx * c);
      mn = fmaxf(mn, pair_swap(mn));
      if (mn > ls.ss.m) {
        if (ls.ss.Z != 0.f) {
          const float d = ls.ss.m - mn;
          const float f = exp2f_fast(d);
          ls.ss.S = f * (ls.ss.S + d * ls.ss.Z);
          ls.ss.Z *= f;
        }
        ls.ss.m = mn;
      }
      m = ls.ss.m;
    }
    float hs[kRounds];  // this lane's half of each round's block, relative to m
    float S = SC ? 0.f : ls.ss.S, Z = SC ? 0.f : ls.ss.Z;
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      float bs = 0.f;
      float ev[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const float d = fmaf(l[q][j], c, -m);
        if (FULL) {
          const float e = exp2f_fast(d);
          ev[j] = e;
          bs += e;
          S = fmaf(e, d, S);
        } else {
          const bool ok = l[q][j] != -INFINITY;
          const float e = ok ? exp2f_fast(d) : 0.f;
          ev[j] = e;
          bs += e;
          S = ok ? fmaf(e, d, S) : S;
        }
      }
      hs[q] = bs;
      Z += bs;
      if constexpr (SC) {
        const int64_t e0 = E + q * (kSampleThreads * kGroup) + kGroup * t;
        if (FULL || e0 < so.Kp) {
          half8 hw;
#pragma unroll
          for (int j = 0; j < kGroup; ++j) hw[j] = static_cast<_Float16>(ev[j] * 32768.f);
          *reinterpret_cast<half8*>(so.w + ((e0 >> 5) * so.Mp + so.row) * 32 + (e0 & 31)) = hw;
        }
      }
    }
    if constexpr (SC) {
      soft_merge(ls.ss, SoftState{m, Z, S});
      if (threadIdx.x == 0) so.ref[static_cast<int64_t>(so.row) * so.nchunk + E / kIterElems] = m;
    } else {
      ls.ss.S = S;
      ls.ss.Z = Z;
    }
    // lane h of the pair scores the blocks of rounds 4h .. 4h + 3: blocks
    // b = E / 16 + 128 (4h + j) + pr, which share counter 128 (E / 8192 + h) + pr (word j)
    float own[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float mine = h ? hs[4 + j] : hs[j];
      const float give = h ? hs[j] : hs[4 + j];
      own[j] = mine + pair_swap(give);
    }
    const uint32_t ctr = 128u * static_cast<uint32_t>(E / 8192 + h) + static_cast<uint32_t>(pr);
    const u32x4 w = philox4x32_10(u32x4{ctr, pos, st, static_cast<uint32_t>(DG_STREAM_GUMBEL)}, k0, k1);
    const uint32_t wj[4] = {w.x, w.y, w.z, w.w};
    const int32_t b0 = static_cast<int32_t>(E / kBlock) + 128 * 4 * h + pr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float key = gumbel_key2(m + __builtin_amdgcn_logf(own[j]), wj[j]);  // log2(0) = -inf
      const bool better = key > ls.kv;
      ls.kv = better ? key : ls.kv;
      ls.kb = better ? b0 + 128 * j : ls.kb;
    }
  }
}

// One workgroup per (row, chunk of `iters` iterations).  Logits must be finite.
template <bool BF16, bool ARGMAX_ONLY, bool SC>
__global__ __launch_bounds__(kSampleThreads) void sample_partial_kernel(
    const void* __restrict__ logits, int64_t ld, int32_t V, int32_t rows_per_req, const uint64_t* __restrict__ seed,
    const int32_t* __restrict__ step, const uint8_t* __restrict__ active, float c, int32_t iters, int32_t nsplit,
    Partial* __restrict__ part, ScOut so) {
  __shared__ float red_sc[kSampleThreads / kWave];
  const int r = blockIdx.y;
  const int split = blockIdx.x;
  const int req = r / rows_per_req;
  if (active != nullptr && active[req] == 0) return;
  const uint32_t pos = static_cast<uint32_t>(r - req * rows_per_req);
  const char* row = reinterpret_cast<const char*>(logits) + r * ld * (BF16 ? 2 : 4);

  uint32_t k0 = 0, k1 = 0, st = 0;
  if constexpr (!ARGMAX_ONLY) {
    const uint64_t sd = seed[req];
    k0 = static_cast<uint32_t>(sd);
    k1 = static_cast<uint32_t>(sd >> 32);
    st = static_cast<uint32_t>(step[req]);
  }
  LaneState ls{-INFINITY, -1, SoftState{-INFINITY, 0.f, 0.f}, -INFINITY, 0x7FFFFFFF};
  const int64_t E0 = static_cast<int64_t>(split) * iters * kIterElems;
  const int64_t full_end = min(static_cast<int64_t>(iters), (V - E0) / kIterElems);  // iterations entirely < V
  so.row = r;
  int64_t it = 0;
  for (; it < full_end; ++it)
    sample_iteration<BF16, ARGMAX_ONLY, true, SC>(row, E0 + it * kIterElems, V, c, pos, st, k0, k1, ls, so, red_sc);
  if (it < iters && E0 + it * kIterElems < V)
    sample_iteration<BF16, ARGMAX_ONLY, false, SC>(row, E0 + it * kIterElems, V, c, pos, st, k0, k1, ls, so, red_sc);

  // the argmax travels as (value, first index of its 8-logit group); the merge resolves the index
  float av = ls.av;
  int32_t ai = ls.ag >= 0 ? ls.ag : 0x7FFFFFFF;
  SoftState ss = ls.ss;
  float kv = ls.kv;
  int32_t kb = ls.kb;

  // workgroup reduction: DPP inside each wave, then the 4 waves through LDS
  dpp_wave_argmax(av, ai);
  if constexpr (!ARGMAX_ONLY) {
    ss = dpp_wave_soft(ss);
    dpp_wave_argmax(kv, kb);
  }
  __shared__ Partial red[kSampleThreads / kWave];
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wid] = Partial{ss.m, ss.Z, ss.S, av, ai, kv, kb, 0};
  __syncthreads();
  if (threadIdx.x == 0) {
    Partial pa = red[0];
    SoftState a{pa.m, pa.Z, pa.S};
    for (int w2 = 1; w2 < kSampleThreads / kWave; ++w2) {
      const Partial q = red[w2];
      argmax_merge(pa.amax_v, pa.amax_i, q.amax_v, q.amax_i);
      if constexpr (!ARGMAX_ONLY) {
        soft_merge(a, SoftState{q.m, q.Z, q.S});
        argmax_merge(pa.key_v, pa.key_b, q.key_v, q.key_b);
      }
    }
    pa.m = a.m;
    pa.Z = a.Z;
    pa.S = a.S;
    part[static_cast<int64_t>(r) * nsplit + split] = pa;
  }
}

// One wave per row: merge the chunks, then draw the element inside the winning block.
template <bool BF16, bool ARGMAX_ONLY>
__global__ __launch_bounds__(kWave) void sample_merge_kernel(const Partial* __restrict__ part, int32_t nsplit,
                                                              const void* __restrict__ logits, int64_t ld, int32_t V,
                                                              int32_t rows_per_req, const uint64_t* __restrict__ seed,
                                                              const int32_t* __restrict__ step,
                                                              const uint8_t* __restrict__ active, float c,
                                                              float* __restrict__ entropy, int32_t* __restrict__ argmax,
                                                              int32_t* __restrict__ sample, float* __restrict__ row_max,
                                                              float* __restrict__ row_lnz) {
  const int r = blockIdx.x;
  const int req = r / rows_per_req;
  if (active != nullptr && active[req] == 0) return;
  float av = -INFINITY, kv = -INFINITY;
  int32_t ag = 0x7FFFFFFF, kb = 0x7FFFFFFF;
  SoftState ss{-INFINITY, 0.f, 0.f};
  for (int s = threadIdx.x; s < nsplit; s += kWave) {
    const Partial p = part[static_cast<int64_t>(r) * nsplit + s];
    argmax_merge(av, ag, p.amax_v, p.amax_i);
    if constexpr (!ARGMAX_ONLY) {
      soft_merge(ss, SoftState{p.m, p.Z, p.S});
      argmax_merge(kv, kb, p.key_v, p.key_b);
    }
  }
  dpp_wave_argmax(av, ag);
  const char* row = reinterpret_cast<const char*>(logits) + r * ld * (BF16 ? 2 : 4);
  const int lane = threadIdx.x;
  // argmax: the first id of the winning 8-logit group (the earliest group holding the maximum)
  // whose logit equals the maximum
  const int64_t ga = static_cast<int64_t>(min(max(ag, 0), V - 1)) + lane;
  const bool hit = lane < kGroup && ga < V && load1<BF16>(row, ga) == av;
  const uint64_t hits = __ballot(hit);
  const int32_t amax = hits ? static_cast<int32_t>(ga - lane) + __ffsll(static_cast<unsigned long long>(hits)) - 1
                            : min(max(ag, 0), V - 1);
  if constexpr (!ARGMAX_ONLY) {
    ss = dpp_wave_soft(ss);
    dpp_wave_argmax(kv, kb);
    // second level: lanes 0..15 score the ids of block kb with per-element noise
    const int64_t i = static_cast<int64_t>(min(max(kb, 0), (V - 1) / kBlock)) * kBlock + lane;
    float key = -INFINITY;
    int32_t si = 0x7FFFFFFF;
    if (lane < kBlock && i < V) {
      const uint64_t sd = seed[req];
      const u32x4 w = philox4x32_10(u32x4{static_cast<uint32_t>(i >> 2), static_cast<uint32_t>(r - req * rows_per_req),
                                          static_cast<uint32_t>(step[req]), static_cast<uint32_t>(DG_STREAM_GUMBEL_INNER)},
                                    static_cast<uint32_t>(sd), static_cast<uint32_t>(sd >> 32));
      const uint32_t wi = (i & 3) == 0 ? w.x : ((i & 3) == 1 ? w.y : ((i & 3) == 2 ? w.z : w.w));
      key = gumbel_key2(load1<BF16>(row, i) * c, wi);
      si = static_cast<int32_t>(i);
    }
    dpp_wave_argmax(key, si);
    if (threadIdx.x == 0) {
      // back to natural units: x = x2 ln 2, ln Z = log2(Z) ln 2, S_nat = S ln 2
      constexpr float kLn2 = 0.69314718055994531f;
      const float lnz = logf(ss.Z);
      entropy[r] = fmaxf(0.f, lnz - kLn2 * ss.S / ss.Z);
      sample[r] = si;
      row_max[r] = ss.m * kLn2;
      row_lnz[r] = lnz;
    }
  }
  if (threadIdx.x == 0) argmax[r] = amax;
}

struct SamplePlan {
  int32_t nsplit, iters;
};

// A row is cut into chunks of kChunkIters iterations (65536 logits) whatever the launch holds, so a
// row's statistics are summed in the same order in every batch it can be part of (batch-invariant
// per request); only the number of workgroups grows with the rows.  Four iterations per workgroup:
// on the 256 x 262144 step, 1024 workgroups of 4 iterations beat 4096 of 1 by 15 % (the
// per-workgroup reductions are amortised over more logits).
constexpr int32_t kChunkIters = 4;

SamplePlan plan_sample(int32_t V) {
  const int32_t row_iters = static_cast<int32_t>(cdiv(V, kIterElems));
  const int32_t iters = min(row_iters, kChunkIters);
  return {static_cast<int32_t>(cdiv(row_iters, iters)), iters};
}

// Shared by dg_denoise_sample and dg_denoise_sample_sc (so.w != nullptr: also writes the operand).
dg_status denoise_sample_impl(const void* logits, int64_t ld, int32_t dtype, int32_t rows, int32_t V,
                              int32_t rows_per_req, const uint64_t* seed, const int32_t* step, const uint8_t* active,
                              float temperature, uint32_t flags, float* entropy, int32_t* argmax, int32_t* sample,
                              float* row_max, float* row_lnz, void* ws, size_t ws_bytes, ScOut so,
                              dg_stream_t stream) {
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
  const SamplePlan p = plan_sample(V);
  hipStream_t s = as_stream(stream);
  Partial* part = reinterpret_cast<Partial*>(ws);
  const dim3 grid(p.nsplit, rows);
  const float c = 1.4426950408889634f / (amax_only ? 1.f : temperature);  // log2(e) / T
#define DG_SAMPLE_LAUNCH(BF, AO, SC)                                                                                  \
  sample_partial_kernel<BF, AO, SC><<<grid, kSampleThreads, 0, s>>>(logits, ld, V, rows_per_req, seed, step, active,  \
                                                                     c, p.iters, p.nsplit, part, so);                 \
  DG_LAUNCHED();                                                                                                      \
  sample_merge_kernel<BF, AO><<<rows, kWave, 0, s>>>(part, p.nsplit, logits, ld, V, rows_per_req, seed, step,         \
                                                      active, c, entropy, argmax, sample, row_max, row_lnz);
  if (so.w != nullptr) {
    DG_UNSUP(dtype == DG_BF16 && !amax_only);
    DG_SAMPLE_LAUNCH(true, false, true)
  } else if (dtype == DG_BF16) {
    if (amax_only) {
      DG_SAMPLE_LAUNCH(true, true, false)
    } else {
      DG_SAMPLE_LAUNCH(true, false, false)
    }
  } else {
    if (amax_only) {
      DG_SAMPLE_LAUNCH(false, true, false)
    } else {
      DG_SAMPLE_LAUNCH(false, false, false)
    }
  }
#undef DG_SAMPLE_LAUNCH
  DG_LAUNCHED();
  return DG_OK;
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" size_t dg_denoise_sample_ws_bytes(int32_t rows, int32_t V) {
  if (rows <= 0 || V <= 0) return 0;
  const SamplePlan p = plan_sample(V);
  return static_cast<size_t>(rows) * p.nsplit * sizeof(Partial);
}

extern "C" dg_status dg_denoise_sample(const void* logits, int64_t ld, int32_t dtype, int32_t rows, int32_t V,
                                       int32_t rows_per_req, const uint64_t* seed, const int32_t* step,
                                       const uint8_t* active, float temperature, uint32_t flags, float* entropy,
                                       int32_t* argmax, int32_t* sample, float* row_max, float* row_lnz, void* ws,
                                       size_t ws_bytes, dg_stream_t stream) {
  return denoise_sample_impl(logits, ld, dtype, rows, V, rows_per_req, seed, step, active, temperature, flags, entropy,
                             argmax, sample, row_max, row_lnz, ws, ws_bytes, ScOut{nullptr, 0, 0, nullptr, 0, 0},
                             stream);
}

extern "C" size_t dg_selfcond_operand_bytes(int32_t rows, int32_t V) {
  if (rows <= 0 || V <= 0) return 0;
  const int64_t Mp = (static_cast<int64_t>(rows) + 255) / 256 * 256, Kp = (static_cast<int64_t>(V) + 127) / 128 * 128;
  const int64_t nchunk = cdiv(V, kIterElems);
  return static_cast<size_t>(round_up(Mp * Kp * 2, 256) + rows * nchunk * 4);
}

extern "C" dg_status dg_denoise_sample_sc(const void* logits, int64_t ld, int32_t dtype, int32_t rows, int32_t V,
                                          int32_t rows_per_req, const uint64_t* seed, const int32_t* step,
                                          const uint8_t* active, float temperature, float* entropy, int32_t* argmax,
                                          int32_t* sample, float* row_max, float* row_lnz, void* ws, size_t ws_bytes,
                                          void* sc_operand, size_t sc_operand_bytes, dg_stream_t stream) {
  DG_ARG(sc_operand != nullptr && rows > 0 && V > 0);
  DG_UNSUP(dtype == DG_BF16);
  DG_REQUIRE(sc_operand_bytes >= dg_selfcond_operand_bytes(rows, V), DG_E_WORKSPACE);
  const int64_t Mp = (static_cast<int64_t>(rows) + 255) / 256 * 256, Kp = (static_cast<int64_t>(V) + 127) / 128 * 128;
  char* base = reinterpret_cast<char*>(sc_operand);
  const ScOut so{reinterpret_cast<_Float16*>(base), Mp, Kp, reinterpret_cast<float*>(base + round_up(Mp * Kp * 2, 256)),
                 static_cast<int32_t>(cdiv(V, kIterElems)), 0};
  return denoise_sample_impl(logits, ld, dtype, rows, V, rows_per_req, seed, step, active, temperature, 0, entropy,
                             argmax, sample, row_max, row_lnz, ws, ws_bytes, so, stream);
}

// ---------------------------------------------------------------- allocation-free variant
// dg_denoise_sample with its chunk partials in a fixed device array instead of a caller workspace,
// for callers that cannot allocate.  Each GPU holds its own copy of the array (a static __device__
// symbol); its address on the current device is looked up once per device with
// hipGetSymbolAddress and passed to the kernels like a workspace.  The partials are written in
// full before they are read, so nothing needs clearing between calls.
namespace dg {
namespace {
constexpr size_t kScratchPartials = 262144;  // 8 MiB: rows * chunks per row (V = 262144: 4 chunks, 65536 rows)
constexpr int kScratchDevices = 64;
__device__ __align__(256) Partial scratch[kScratchPartials];
void* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
std::once_flag g_scratch_once[kScratchDevices];
}  // namespace
}  // namespace dg

extern "C" size_t dg_denoise_sample_noalloc_max_bytes(void) { return sizeof(Partial) * kScratchPartials; }

extern "C" dg_status dg_denoise_sample_noalloc(const void* logits, int64_t ld, int32_t dtype, int32_t rows, int32_t V,
                                               int32_t rows_per_req, const uint64_t* seed, const int32_t* step,
                                               const uint8_t* active, float temperature, uint32_t flags,
                                               float* entropy, int32_t* argmax, int32_t* sample, float* row_max,
                                               float* row_lnz, dg_stream_t stream) {
  DG_ARG(rows > 0 && V > 0);
  DG_REQUIRE(dg_denoise_sample_ws_bytes(rows, V) <= sizeof(Partial) * kScratchPartials, DG_E_SCRATCH);
  int dev = -1;
  DG_REQUIRE(hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kScratchDevices, DG_E_HIP);
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = ptr;
  });
  DG_REQUIRE(g_scratch_err[dev] == hipSuccess && g_scratch_ptr[dev] != nullptr, DG_E_HIP);
  return denoise_sample_impl(logits, ld, dtype, rows, V, rows_per_req, seed, step, active, temperature, flags, entropy,
                             argmax, sample, row_max, row_lnz, g_scratch_ptr[dev], sizeof(Partial) * kScratchPartials,
                             ScOut{nullptr, 0, 0, nullptr, 0, 0}, stream);
}
