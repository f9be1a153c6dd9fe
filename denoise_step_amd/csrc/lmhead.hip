// dg_lmhead_denoise_sample: the LM head (logits = scale h E^T with the embedding table E as the
// output projection) fused with the denoise sampler and the writing of the self-conditioning
// operand; the [rows, V] logits exist only in registers and LDS.
//
// Method: DiffusionGemma/vLLM page, section "Entropy-based denoising" (entropy of every position's
// distribution), section "DiffusionGemmaModelState and DiffusionSampler", denoise case (temperature,
// Gumbel-max candidate, argmax) and section "Self-conditioning" (this step's full softmax is the left
// operand of P.E).  The sampler's two-level Gumbel draw is the one of dg_denoise_sample: block
// b of 16 ids gets word (b >> 7) & 3 of Philox counter 128 (b >> 9) + (b & 127) (stream 0), the
// ids inside the winning block words i & 3 of counter i >> 2 (stream 3).
//
// gfx950 design.  One workgroup per (256 rows, 256 ids) tile, the whole d contraction on
// v_mfma_f32_32x32x16_bf16 with the pipeline and ping-pong schedule of the P.E GEMM.  Both operands
// are bf16 in the K-blocked layout (h copied per call, E prepared once by dg_lmhead_prepare), so
// each 16-id group of a stage is one contiguous kilobyte (the table as stored, [V][d], would give
// 64-byte pieces 8 KB apart, which all workgroups fetch from the same few HBM channels at once).
// A tile's 256 ids are four runs of 64 ids spaced 2048 apart inside a group of 8192 ids: the 16
// Gumbel blocks of a row then share four Philox counters (one call per lane).  After the main loop
// the tile's logits go through LDS, 128 rows at a time; four lanes per row then compute the tile's
// partial softmax state (relative to ref = ceil of the tile's largest base-2 logit), argmax, best
// Gumbel block and the draw inside that block, and write the fp16 operand w = 2^15 2^(x2 - ref).
// A merge kernel combines a row's tiles and derives, per 16384-id run of P.E, the run's reference
// R (the largest tile ref) and each tile's exponent ref - R; a streaming pass then multiplies every
// tile's operand values by 2^(ref - R) (exact), which leaves the operand of the sampling pass
// (values relative to one reference per run) for the P.E GEMM.
#include "dg_device.hpp"
#include "dg_host.hpp"
#include "gemm_f16.hpp"

namespace dg {
namespace {

constexpr int kLmTS = 260;                    // row stride (floats) of the logits tile in LDS
constexpr int kLmSmem = 128 * kLmTS * 4;       // 133120 bytes: the tile's 128-row half (>= 4 stages)
static_assert(kLmSmem >= kGemmStages * 2 * kGemmTM * kGemmTK * 2, "epilogue tile covers the stages");

struct LmPartial {
  float mt;     // largest x2 = scale log2(e) / T * (h . E_v) of the tile row
  float Z, S;   // sum 2^(x2 - ref), sum 2^(x2 - ref) (x2 - ref), ref = ceil(mt)
  float av;     // largest h . E_v
  int32_t ai;   // its lowest id
  float kv;     // best first-level Gumbel key (log2 units)
  int32_t kb;   // its block
  int32_t inner;  // the id drawn inside block kb
};
static_assert(sizeof(LmPartial) == 32, "partial layout");

struct LmArgs {
  const _Float16* hk;  // h as bf16 bit patterns, K-blocked with Mp rows
  int64_t Mp;
  const _Float16* Ek;  // E as bf16 bit patterns, K-blocked with V rows
  int32_t rows, V, d;
  int64_t Kp;
  int32_t mtiles, ntiles;
  float c2;            // scale log2(e) / T
  int32_t rows_per_req;
  const uint64_t* seed;
  const int32_t* step;
  _Float16* w;         // operand [Kp / 32][Mp][32]
  LmPartial* part;     // [rows][ntiles]
};

// h [rows][ldh] bf16 -> hk, K-blocked with Mp rows (rows past `rows` zero); 8 elements per thread.
__global__ __launch_bounds__(256) void lm_h_kblk_kernel(const uint16_t* __restrict__ h, int64_t ldh, int32_t rows,
                                                        int32_t d, int64_t Mp, uint16_t* __restrict__ hk) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= Mp * d) return;
  const int64_t r = i / d;
  const int32_t k = static_cast<int32_t>(i - r * d);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (r < rows) v = *reinterpret_cast<const uint4*>(h + r * ldh + k);
  *reinterpret_cast<uint4*>(hk + kblk_index(r, k, Mp)) = v;
}

// Operand source of the LM-head main loop: A = hk, B = the tile's 256 rows of Ek (both K-blocked).
// 16-id group q of the tile holds ids id_base + 2048 (q / 4) + 16 (q % 4) + [0, 16), one contiguous
// kilobyte per stage; groups past V read ids 0..15 instead (their logits are discarded).
struct LmSrc {
  const LmArgs& a;
  int m0;
  int64_t id_base;
  uint32_t off;
  int wave;
  DG_DEV void issue(int s, _Float16* as, _Float16* bs) const {
    const int k0 = s * kGemmTK;
#pragma unroll
    for (int i = 0; i < kGemmTM / 16 / kGemmWaves; ++i)
      gemm_dma<false>(a.hk, a.Mp, m0, k0, off, as, wave + kGemmWaves * i);
#pragma unroll
    for (int i = 0; i < 256 / 16 / kGemmWaves; ++i) {
      const int q = wave + kGemmWaves * i;
      const int64_t id0 = id_base + 2048 * (q >> 2) + 16 * (q & 3);
      gemm_dma<true>(a.Ek, a.V, static_cast<int>(id0 < a.V ? id0 : 0), k0, off, bs + q * kWave * 8, 0);
    }
  }
  DG_DEV void fix(GemmFrag<256>&, int) const {}
};

// reductions over the four lanes of a quad (all four active or none)
DG_DEV float quad_sum(float v) {
  v += dpp_f<dpp::kXor1, 0xF>(v, 0.f);
  return v + dpp_f<dpp::kXor2, 0xF>(v, 0.f);
}
DG_DEV void quad_argmax(float& v, int32_t& i) {
  dpp_argmax_step<dpp::kXor1, 0xF>(v, i);
  dpp_argmax_step<dpp::kXor2, 0xF>(v, i);
}

// One lane's quarter of a tile row: ids id_base + 2048 j + 16 qi + [0, 16), j = 0..3 (four Gumbel
// blocks under one Philox counter).  trow: the row's logits (h . E_v) in LDS, column 64 j + c for
// id id_base + 2048 j + c.  The segments are read twice (maximum, then exponentials) so that only
// 16 logits are live next to the accumulators that the other half of the waves still holds.
DG_DEV void lm_row_quarter(const LmArgs& a, const float* trow, int row, int qi, int64_t id_base, int nt) {
  int64_t idj[4];
  bool ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    idj[j] = id_base + 2048 * j + 16 * qi;
    ok[j] = idj[j] < a.V;  // V % 16 == 0: a 16-id segment is all in or all out
  }
  // argmax of h . E_v, lowest id on ties (ids grow with j, then u)
  float av = -INFINITY;
  int32_t ai = 0x7FFFFFFF;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!ok[j]) continue;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 v = *reinterpret_cast<const float4*>(trow + 64 * j + 16 * qi + 4 * k);
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (vv[u] > av) {
          av = vv[u];
          ai = static_cast<int32_t>(idj[j]) + 4 * k + u;
        }
    }
  }
  quad_argmax(av, ai);
  const float mt = av * a.c2;  // the row's largest x2 in the tile (the product rounds monotonically)
  const float ref = ceilf(mt);
  float Z = 0.f, S = 0.f, bs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float b = 0.f;
    half8 hw[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 v = *reinterpret_cast<const float4*>(trow + 64 * j + 16 * qi + 4 * k);
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float dd = fmaf(vv[u], a.c2, -ref);
        const float e = ok[j] ? __builtin_amdgcn_exp2f(dd) : 0.f;
        b += e;
        S = ok[j] ? fmaf(e, dd, S) : S;
        hw[k >> 1][4 * (k & 1) + u] = static_cast<_Float16>(e * 32768.f);
      }
    }
    bs[j] = b;
    Z += b;
    if (idj[j] < a.Kp) {  // ids in [V, Kp) get zeros; the operand ends at Kp
      _Float16* dst = a.w + ((idj[j] >> 5) * a.Mp + row) * 32 + (idj[j] & 31);
      *reinterpret_cast<half8*>(dst) = hw[0];
      *reinterpret_cast<half8*>(dst + 8) = hw[1];
    }
  }
  Z = quad_sum(Z);
  S = quad_sum(S);

  const int req = row / a.rows_per_req;
  const uint32_t pos = static_cast<uint32_t>(row - req * a.rows_per_req);
  const uint64_t sd = a.seed[req];
  const uint32_t k0 = static_cast<uint32_t>(sd), k1 = static_cast<uint32_t>(sd >> 32);
  const uint32_t st = static_cast<uint32_t>(a.step[req]);
  // block b = idj / 16 = 512 g + 128 j + 4 sub + qi: counter 128 g + 4 sub + qi, word j
  const uint32_t ctr = static_cast<uint32_t>(128 * (nt >> 5) + 4 * (nt & 31) + qi);
  const u32x4 w = philox4x32_10(u32x4{ctr, pos, st, static_cast<uint32_t>(DG_STREAM_GUMBEL)}, k0, k1);
  const uint32_t wj[4] = {w.x, w.y, w.z, w.w};
  float kv = -INFINITY;
  int32_t kb = 0x7FFFFFFF;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!ok[j]) continue;
    const float key = gumbel_key2(ref + __builtin_amdgcn_logf(bs[j]), wj[j]);
    argmax_merge(kv, kb, key, static_cast<int32_t>(idj[j] >> 4));
  }
  quad_argmax(kv, kb);
  // the draw inside the row's best block of the tile: lane qi scores its ids 4 qi .. 4 qi + 3
  float ik = -INFINITY;
  int32_t ii = 0x7FFFFFFF;
  if (kb != 0x7FFFFFFF) {
    const int64_t lo = static_cast<int64_t>(kb) * 16;
    const int64_t off = lo - id_base;  // 2048 j + 16 i of the block
    const float4 v = *reinterpret_cast<const float4*>(trow + 64 * (off >> 11) + (off & 2047) + 4 * qi);
    const int64_t i0 = lo + 4 * qi;
    const u32x4 wi = philox4x32_10(
        u32x4{static_cast<uint32_t>(i0 >> 2), pos, st, static_cast<uint32_t>(DG_STREAM_GUMBEL_INNER)}, k0, k1);
    const int32_t i32 = static_cast<int32_t>(i0);
    argmax_merge(ik, ii, gumbel_key2(v.x * a.c2, wi.x), i32);
    argmax_merge(ik, ii, gumbel_key2(v.y * a.c2, wi.y), i32 + 1);
    argmax_merge(ik, ii, gumbel_key2(v.z * a.c2, wi.z), i32 + 2);
    argmax_merge(ik, ii, gumbel_key2(v.w * a.c2, wi.w), i32 + 3);
  }
  quad_argmax(ik, ii);
  if (qi == 0) a.part[static_cast<int64_t>(row) * a.ntiles + nt] = LmPartial{mt, Z, S, av, ai, kv, kb, ii};
}

// A wave's 128 x 64 accumulator block into the LDS tile (row stride kLmTS): element e of lane l of
// block (i, j) is row 32 i + 8 (e / 4) + 4 (l / 32) + e % 4, column wn + 32 j + l % 32.
DG_DEV void lm_store_acc(const floatx16 (&acc)[4][2], float* T, int wn, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        T[(32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * kLmTS + wn + 32 * j + (lane & 31)] = acc[i][j][e];
}

__global__ __launch_bounds__(kGemmThreads) void lmhead_sample_kernel(LmArgs a) {
  __shared__ __attribute__((aligned(16))) float smem[kLmSmem / 4];
  _Float16* As = reinterpret_cast<_Float16*>(smem);
  _Float16* Bs = As + kGemmStages * kGemmTM * kGemmTK;
  // XCD-aware order as in the GEMM: t = ntile * mtiles + mtile, consecutive t on one XCD
  const int total = a.mtiles * a.ntiles;
  const int per_xcd = (total + kGemmXcds - 1) / kGemmXcds;
  const int t = (blockIdx.x % kGemmXcds) * per_xcd + blockIdx.x / kGemmXcds;
  if (t >= total) return;
  const int mt = t % a.mtiles, nt = t / a.mtiles;
  const int64_t id_base = static_cast<int64_t>(nt >> 5) * 8192 + 64 * (nt & 31);
  if (id_base >= a.Kp) return;  // no id of the operand in this tile
  const int m0 = mt * kGemmTM;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int group = wave >> 2;
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 64;

  floatx16 acc[4][2];
  gemm_main<256, false, true, true>(LmSrc{a, m0, id_base, gemm_lane_offset(), wave}, a.d / kGemmTK, As, Bs, wm, wn,
                                    lane, group, acc);

  // Epilogue: the tile's logits through LDS in two halves of 128 rows.  The even waves hold rows
  // 0..127 (wm = 0): they store them and, four lanes per row, process them while the odd waves
  // keep rows 128..255 in registers; then the odd waves store theirs and all waves process them.
  // The two branches keep the accumulators of a wave dead wherever it runs the row code.
  __syncthreads();  // every wave is past its last LDS read of the main loop
  if ((wave & 1) == 0) {
    lm_store_acc(acc, smem, wn, lane);
    __syncthreads();  // rows 0..127 in LDS
    const int t4 = (wave >> 1) * kWave + lane;  // 0..255 over the even waves; t4 % 4 == lane % 4
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rr = 64 * h + (t4 >> 2);
      if (m0 + rr < a.rows) lm_row_quarter(a, smem + rr * kLmTS, m0 + rr, lane & 3, id_base, nt);
    }
    __syncthreads();  // rows 0..127 consumed
    __syncthreads();  // rows 128..255 in LDS
  } else {
    __syncthreads();
    __syncthreads();
    lm_store_acc(acc, smem, wn, lane);
    __syncthreads();
  }
  const int r = threadIdx.x >> 2;
  if (m0 + 128 + r < a.rows) lm_row_quarter(a, smem + r * kLmTS, m0 + 128 + r, threadIdx.x & 3, id_base, nt);
}

// One wave per row: the row's tiles (those with an id < V) merged into the sampler outputs; per
// 16384-id run k of P.E the reference R_k = the largest ceil(mt) of its 64 tiles (ref_out) and each
// tile's exponent ceil(mt) - R_k (exps [64 nrun][Mp], 0 for tiles without ids < V), and the
// argmax (top, for every row).  Lane l merges tile 64 k + l of every run k.
__global__ __launch_bounds__(kWave) void lmhead_merge_kernel(const LmPartial* __restrict__ part, int32_t ntiles,
                                                             int32_t nrun, int32_t V, int64_t Mp, int32_t rows_per_req,
                                                             const uint8_t* __restrict__ active, float* __restrict__ entropy,
                                                             int32_t* __restrict__ argmax, int32_t* __restrict__ sample,
                                                             float* __restrict__ row_max, float* __restrict__ row_lnz,
                                                             float* __restrict__ ref_out, int8_t* __restrict__ exps,
                                                             int32_t* __restrict__ top) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const LmPartial* pr = part + static_cast<int64_t>(r) * ntiles;
  SoftState ss{-INFINITY, 0.f, 0.f};
  float mx = -INFINITY, av = -INFINITY, kv = -INFINITY;
  int32_t ai = 0x7FFFFFFF, kb = 0x7FFFFFFF;
  for (int k = 0; k < nrun; ++k) {
    const int t = 64 * k + lane;
    const int64_t first = static_cast<int64_t>(t >> 5) * 8192 + 64 * (t & 31);
    float rt = -INFINITY;
    if (t < ntiles && first < V) {
      const LmPartial p = pr[t];
      rt = ceilf(p.mt);
      soft_merge(ss, SoftState{rt, p.Z, p.S});
      mx = fmaxf(mx, p.mt);
      argmax_merge(av, ai, p.av, p.ai);
      argmax_merge(kv, kb, p.kv, p.kb);
    }
    const float R = dpp_wave_max(rt);  // finite: tile 64 k starts at 16384 k < V
    exps[static_cast<int64_t>(t) * Mp + r] = rt > -INFINITY ? static_cast<int8_t>(fmaxf(rt - R, -128.f)) : int8_t{0};
    if (lane == 0) ref_out[static_cast<int64_t>(r) * nrun + k] = R;
  }
  dpp_wave_argmax(av, ai);
  if (lane == 0) top[r] = ai;
  if (active != nullptr && active[r / rows_per_req] == 0) return;
  dpp_wave_argmax(kv, kb);
  mx = dpp_wave_max(mx);
  ss = dpp_wave_soft(ss);
  if (lane == 0) {
    constexpr float kLn2 = 0.69314718055994531f;
    const int tb = 32 * (kb >> 9) + ((kb & 127) >> 2);  // the tile holding block kb
    const float lnz = logf(ss.Z);  // relative to ss.m (base 2)
    entropy[r] = fmaxf(0.f, lnz - kLn2 * ss.S / ss.Z);
    argmax[r] = ai;
    sample[r] = (kb >= 0 && tb < ntiles) ? pr[tb].inner : -1;  // -1 only when no key is finite (non-finite h)
    row_max[r] = mx * kLn2;
    row_lnz[r] = lnz + kLn2 * (ss.m - mx);
  }
}

// w *= 2^e per (row, LM-head tile), e = exps[tile][row] <= 0 (exact for powers of two, except that
// values below fp16's normal range round), so that every value is relative to its run's reference.
// Thread g covers 16 ids (32 bytes) of one row: K block g / (2 Mp), row (g / 2) % Mp, half g % 2, so
// consecutive threads cover consecutive memory.  Tiles with e == 0 (the largest of each run) are
// left as they are.
__global__ __launch_bounds__(256) void lm_rescale_kernel(_Float16* __restrict__ w, int64_t Mp, int64_t Kp, int32_t rows,
                                                         const int8_t* __restrict__ exps) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= Kp / 16 * Mp) return;
  const int64_t kb = g / (2 * Mp);
  const int64_t r = (g >> 1) % Mp;
  if (r >= rows) return;
  const int64_t id = kb * 32 + 16 * (g & 1);
  const int e = exps[(32 * (id >> 13) + ((id & 2047) >> 6)) * Mp + r];
  if (e == 0) return;
  half8* p = reinterpret_cast<half8*>(w + (kb * Mp + r) * 32 + 16 * (g & 1));
  const float sc = ldexpf(1.f, e);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    half8 v = p[k];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = static_cast<_Float16>(static_cast<float>(v[j]) * sc);
    p[k] = v;
  }
}

// E [V][d] bf16 -> Ek, K-blocked with V rows; 8 elements per thread.
__global__ __launch_bounds__(256) void lm_prepare_kernel(const uint16_t* __restrict__ E, int32_t V, int32_t d,
                                                         uint16_t* __restrict__ Ek) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= static_cast<int64_t>(V) * d) return;
  const int64_t v = i / d;
  const int32_t k = static_cast<int32_t>(i - v * d);
  *reinterpret_cast<uint4*>(Ek + kblk_index(v, k, V)) = *reinterpret_cast<const uint4*>(E + i);
}

struct LmPlan {
  int64_t Mp, Kp;
  int32_t mtiles, ntiles;
  size_t off_hk, off_part, off_exp, bytes;
};

LmPlan lm_plan(int32_t rows, int32_t V, int32_t d) {
  LmPlan p{};
  p.Mp = cdiv(rows, kGemmTM) * kGemmTM;
  p.Kp = cdiv(V, 128) * 128;
  p.mtiles = static_cast<int32_t>(p.Mp / kGemmTM);
  p.ntiles = static_cast<int32_t>(32 * cdiv(V, 8192));
  p.off_hk = 0;
  p.off_part = round_up(static_cast<size_t>(p.Mp) * d * 2, 256);
  p.off_exp = round_up(p.off_part + static_cast<size_t>(rows) * p.ntiles * sizeof(LmPartial), 256);
  // exponents of 64 tiles per run (the last run may hold fewer LM-head tiles)
  p.bytes = round_up(p.off_exp + static_cast<size_t>(64) * cdiv(V, 16384) * p.Mp, 256);
  return p;
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" size_t dg_lmhead_prepared_bytes(int32_t V, int32_t d) {
  if (V <= 0 || d <= 0) return 0;
  return static_cast<size_t>(V) * d * 2;
}

extern "C" dg_status dg_lmhead_prepare(const void* E, int32_t V, int32_t d, void* prepared, size_t prepared_bytes,
                                       dg_stream_t stream) {
  DG_ARG(E && prepared && V > 0 && d > 0);
  DG_UNSUP(V % 16 == 0 && d % 128 == 0 && aligned16(E) && aligned16(prepared));
  DG_REQUIRE(prepared_bytes >= dg_lmhead_prepared_bytes(V, d), DG_E_WORKSPACE);
  lm_prepare_kernel<<<static_cast<unsigned>(cdiv(static_cast<int64_t>(V) * d / 8, 256)), 256, 0, as_stream(stream)>>>(
      reinterpret_cast<const uint16_t*>(E), V, d, reinterpret_cast<uint16_t*>(prepared));
  DG_LAUNCHED();
  return DG_OK;
}

extern "C" size_t dg_lmhead_ws_bytes(int32_t rows, int32_t V, int32_t d) {
  if (rows <= 0 || V <= 0 || d <= 0) return 0;
  return lm_plan(rows, V, d).bytes;
}

extern "C" size_t dg_lmhead_operand_bytes(int32_t rows, int32_t V) {
  if (rows <= 0 || V <= 0) return 0;
  return lm_operand_layout(rows, V).bytes;
}

extern "C" dg_status dg_lmhead_denoise_sample_traced(const void* h, int64_t ldh, const void* prepared, int32_t rows,
                                                     int32_t V, int32_t d, float scale, int32_t rows_per_req,
                                                     const uint64_t* seed, const int32_t* step, const uint8_t* active,
                                                     float temperature, float* entropy, int32_t* argmax,
                                                     int32_t* sample, float* row_max, float* row_lnz, void* ws,
                                                     size_t ws_bytes, void* operand, size_t operand_bytes,
                                                     void* k_start, void* k_stop, dg_stream_t stream) {
  DG_ARG(h && prepared && seed && step && entropy && argmax && sample && row_max && row_lnz && operand);
  DG_ARG(rows > 0 && V > 0 && d > 0 && rows_per_req > 0 && rows % rows_per_req == 0 && rows <= 65535 && ldh >= d);
  DG_ARG(scale > 0.f && scale < INFINITY && temperature > 0.f && temperature < INFINITY);
  DG_UNSUP(V % 16 == 0 && V <= (1 << 30) && d % 128 == 0 && d <= 16384);
  DG_UNSUP(ldh % 8 == 0 && aligned16(h) && aligned16(prepared));
  const LmPlan p = lm_plan(rows, V, d);
  const LmOperandLayout L = lm_operand_layout(rows, V);
  DG_REQUIRE(ws != nullptr && ws_bytes >= p.bytes, DG_E_WORKSPACE);
  DG_REQUIRE(operand_bytes >= L.bytes, DG_E_WORKSPACE);
  hipStream_t s = as_stream(stream);
  char* wsb = reinterpret_cast<char*>(ws);
  char* ob = reinterpret_cast<char*>(operand);
  auto* hk = reinterpret_cast<uint16_t*>(wsb + p.off_hk);
  auto* part = reinterpret_cast<LmPartial*>(wsb + p.off_part);
  auto* exps = reinterpret_cast<int8_t*>(wsb + p.off_exp);
  auto* w = reinterpret_cast<_Float16*>(ob);
  lm_h_kblk_kernel<<<static_cast<unsigned>(cdiv(p.Mp * d / 8, 256)), 256, 0, s>>>(
      reinterpret_cast<const uint16_t*>(h), ldh, rows, d, p.Mp, hk);
  DG_LAUNCHED();
  const LmArgs a{reinterpret_cast<const _Float16*>(hk), p.Mp, reinterpret_cast<const _Float16*>(prepared), rows, V, d,
                 p.Kp, p.mtiles, p.ntiles, scale * 1.4426950408889634f / temperature, rows_per_req, seed, step, w,
                 part};
  const int64_t total = static_cast<int64_t>(p.mtiles) * p.ntiles;
  if (k_start != nullptr) DG_REQUIRE(hipEventRecord(reinterpret_cast<hipEvent_t>(k_start), s) == hipSuccess, DG_E_HIP);
  lmhead_sample_kernel<<<static_cast<unsigned>(cdiv(total, kGemmXcds) * kGemmXcds), kGemmThreads, 0, s>>>(a);
  DG_LAUNCHED();
  if (k_stop != nullptr) DG_REQUIRE(hipEventRecord(reinterpret_cast<hipEvent_t>(k_stop), s) == hipSuccess, DG_E_HIP);
  lmhead_merge_kernel<<<rows, kWave, 0, s>>>(part, p.ntiles, L.nrun, V, p.Mp, rows_per_req, active, entropy, argmax,
                                             sample, row_max, row_lnz, reinterpret_cast<float*>(ob + L.off_ref), exps,
                                             reinterpret_cast<int32_t*>(ob + L.off_top));
  DG_LAUNCHED();
  lm_rescale_kernel<<<static_cast<unsigned>(cdiv(p.Kp / 16 * p.Mp, 256)), 256, 0, s>>>(w, p.Mp, p.Kp, rows, exps);
  DG_LAUNCHED();
  return DG_OK;
}

extern "C" dg_status dg_lmhead_denoise_sample(const void* h, int64_t ldh, const void* prepared, int32_t rows, int32_t V,
                                              int32_t d, float scale, int32_t rows_per_req, const uint64_t* seed,
                                              const int32_t* step, const uint8_t* active, float temperature,
                                              float* entropy, int32_t* argmax, int32_t* sample, float* row_max,
                                              float* row_lnz, void* ws, size_t ws_bytes, void* operand,
                                              size_t operand_bytes, dg_stream_t stream) {
  return dg_lmhead_denoise_sample_traced(h, ldh, prepared, rows, V, d, scale, rows_per_req, seed, step, active,
                                         temperature, entropy, argmax, sample, row_max, row_lnz, ws, ws_bytes, operand,
                                         operand_bytes, nullptr, nullptr, stream);
}
