// Split-K fp16 MFMA GEMM for gfx950 with fp32 partial outputs:
//   part[split][m][n] = sum_{k in split} A[m][k] * Bt[n][k]
// Both operands are fp16 in the K-blocked layout of kblk_index(): element
// (row, k) of an R-row operand lives at ((k / 32) R + row) 32 + k % 32, so the
// 32-wide K slice of any run of rows is one contiguous block of memory.  Bt is
// the transposed right operand (prepared once for the constant tables); A is
// written in this layout by the kernel that produces it.
//
// Shaped for the self-conditioning contraction P.E, where M (canvas rows) is
// small, K (the vocabulary) is huge and the right operand E must stream from
// HBM exactly once:
//   * workgroup tile 256 x 256 (256 x 128 when N is not a multiple of 256)
//     with eight wave64s (2 x 4), each wave 128 x 64 as 4 x 2
//     v_mfma_f32_32x32x16_f16 accumulators; a canvas of 256 rows is one M
//     tile, so every E element is fetched by exactly one workgroup;
//   * ping-pong schedule for the long-K P.E launches (the short-K MLP GEMMs
//     keep one barrier per stage): waves w and w + 4 share a SIMD; waves 0-3 run one
//     half-step ahead of waves 4-7, and at every workgroup barrier the two
//     groups swap roles, so in each half-step one wave per SIMD issues its
//     MFMAs while the other reads its next fragments from LDS and issues the
//     copies of a later stage;
//   * K advances 32 per stage through four LDS stages filled by direct
//     global -> LDS copies (no staging registers) issued three stages ahead,
//     about 96 KB per CU in flight against HBM latency;
//   * an XOR swizzle of the 16-byte chunks keeps the MFMA operand reads free
//     of LDS bank conflicts;
//   * XCD-aware order: hardware deals workgroup L to XCD L % 8; tiles are
//     numbered so the workgroups on one XCD share their A chunk (the same
//     probability rows) or their B chunk, which then comes from that XCD's L2.
#pragma once
#include "dg_device.hpp"

namespace dg {

constexpr int kGemmTM = 256;
constexpr int kGemmTK = 32;          // K per LDS stage
constexpr int kGemmStages = 4;       // LDS stages (loads run kGemmStages - 1 ahead)
constexpr int kGemmThreads = 512;      // eight wave64s: 2 (M) x 4 (N)
constexpr int kGemmWaves = kGemmThreads / 64;
constexpr int kGemmXcds = 8;

// index of element (row, k) of an operand with R rows in the K-blocked layout
DG_DEV int64_t kblk_index(int64_t row, int64_t k, int64_t R) { return ((k >> 5) * R + row) * 32 + (k & 31); }

struct GemmArgs {
  const _Float16* A;
  int64_t lda;        // rows of the A operand's blocked layout (M rounded up to 256)
  const _Float16* Bt;
  int64_t ldb;        // rows of Bt (N)
  const uint8_t* Bt8; // E4M3 right operand (gemm_f16_e4m3_splitk_kernel), same blocked layout in bytes
  float* part;  // [splits][M][N]
  int32_t M, N, K;
  int32_t kchunk;  // K per split (multiple of kGemmStages * kGemmTK)
  int32_t mtiles, ntiles, splits;
};

// LDS layout of one stage: rows of 32 halves = four 16-byte chunks, chunk c of row r stored at
// slot 4 r + (c ^ f(r)), f(r) = ((r >> 1) & 7) + ((r >> 3) & 1) (mod 4).  A 16-byte LDS read serves
// the lanes in groups that ask for one chunk of 8 or 16 consecutive rows; f is a bijection on every
// set of rows that would share a bank in either grouping (same parity within 8 rows, same residue
// mod 4 within 16 rows), so the reads are conflict-free.  f depends on r mod 16 only, which the
// copy below relies on.
DG_DEV int gemm_swz(int row) { return (((row >> 1) & 7) + ((row >> 3) & 1)) & 3; }
DG_DEV int gemm_slot(int row, int c) { return row * 4 + (c ^ gemm_swz(row)); }

// Direct global -> LDS copy: one instruction fills 64 consecutive slots (1 KB) starting at `lds`;
// lane i writes slot i.  For instruction q, slot 64 q + i holds row 16 q + i / 4 and, by the
// swizzle, chunk (i & 3) ^ f(i / 4) -- independent of q (f only sees the row mod 16).  In the
// K-blocked layout rows 16 q .. 16 q + 15 of one K slice are 1 KB of contiguous memory, so each
// lane keeps one byte offset inside that kilobyte and the instruction adds a wave-uniform base.
DG_DEV uint32_t gemm_lane_offset() {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = (lane & 3) ^ gemm_swz(lane >> 2);
  return static_cast<uint32_t>(((lane >> 2) * 32 + 8 * c) * 2);
}

// The copy (lds_copy16: scalar base + per-lane 32-bit offset) is tracked only by the explicit vmcnt
// waits of the pipeline below; the main loop issues no other vector-memory instruction, so those
// counts are exact.
// NT marks the load non-temporal: used for the right operand when there is one M tile (E^T is then
// read by exactly one tile per K range), so it does not evict the left operand that the workgroups
// of the other N tiles re-read from L2 (BNT); with several M tiles every B chunk is re-read by each
// of them and is loaded normally.
template <bool NT>
DG_DEV void gemm_dma(const _Float16* __restrict__ base, int64_t rows, int row0, int k0, uint32_t lane_off,
                     _Float16* lds, int q) {
  const char* ub = reinterpret_cast<const char*>(base) + kblk_index(row0 + 16 * q, k0, rows) * 2;
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds + q * kWave * 8));
  lds_copy16<NT>(lds_addr, ub, lane_off);
}

// E4M3 right operand: a K slice of one row is 32 bytes, two 16-byte chunks; chunk c of row r is
// stored at LDS chunk c ^ f8(r), f8(r) = ((r >> 2) ^ (r >> 3)) & 1.  A B-fragment read has 32 lanes
// ask for the same 8-byte quarter of 32 consecutive rows; with the flip, every run of 4 rows that
// would share banks (same r mod 4, or same r mod 8 on a 64-bank array) is split evenly between the
// two halves of the row, so the read runs at the array's full width.  f8 depends on r mod 16 only.
DG_DEV int gemm_swz8(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

// One copy instruction moves 1 KB = 32 rows x 32 bytes of one K slice; lane i writes LDS chunk i,
// i.e. row i / 2, chunk i & 1, and fetches source chunk (i & 1) ^ f8(i / 2) of that row.
DG_DEV uint32_t gemm_lane_offset8() {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane >> 1;
  return static_cast<uint32_t>(r * 32 + 16 * ((lane & 1) ^ gemm_swz8(r)));
}

DG_DEV void gemm_dma8(const uint8_t* __restrict__ base, int64_t rows, int row0, int k0, uint32_t lane_off,
                      uint8_t* lds, int q) {
  const uint8_t* ub = base + kblk_index(row0 + 32 * q, k0, rows);
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds + q * 1024));
  lds_copy16<true>(lds_addr, ub, lane_off);
}

// Issue one stage: A (256 rows) and B (TN rows) as 1-KB instructions shared round-robin by the waves.
// A has mtiles * 256 rows in its layout (rows past M are read but never stored); Bt has N rows.
template <int TN, bool BF8, bool BNT = true>
DG_DEV void gemm_issue(const GemmArgs& g, int m0, int n0, int k0, uint32_t off, uint32_t off8, int wave,
                       _Float16* as, _Float16* bs) {
#pragma unroll
  for (int i = 0; i < kGemmTM / 16 / kGemmWaves; ++i) gemm_dma<false>(g.A, g.lda, m0, k0, off, as, wave + kGemmWaves * i);
  if constexpr (BF8) {
#pragma unroll
    for (int i = 0; i < TN / 32 / kGemmWaves; ++i)
      gemm_dma8(g.Bt8, g.ldb, n0, k0, off8, reinterpret_cast<uint8_t*>(bs), wave + kGemmWaves * i);
  } else {
#pragma unroll
    for (int i = 0; i < TN / 16 / kGemmWaves; ++i) gemm_dma<BNT>(g.Bt, g.ldb, n0, k0, off, bs, wave + kGemmWaves * i);
  }
}

// Operand fragments of one stage for one wave: both 16-K steps of its 4 A blocks and TN / 128 B
// blocks of 32 rows.
template <int TN>
struct GemmFrag {
  half8 a[2][4], b[2][TN / 128];
};

// Read half-step: every fragment of the stage from LDS (E4M3 B fragments converted to fp16 here,
// so the MFMA half-step issues nothing but MFMAs).
template <int TN, bool BF8>
DG_DEV void gemm_read(const _Float16* __restrict__ as, const _Float16* __restrict__ bs, int wm, int wn, int lane,
                      GemmFrag<TN>& f) {
  constexpr int NJ = TN / 128;
  uint2 b8[2][NJ];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c = 2 * ks + (lane >> 5);  // 8-K chunk of this lane
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[ks][i] = *reinterpret_cast<const half8*>(as + 8 * gemm_slot(wm + i * 32 + (lane & 31), c));
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int row = wn + j * 32 + (lane & 31);
      if constexpr (BF8)
        b8[ks][j] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(bs) + row * 32 +
                                                    16 * ((c >> 1) ^ gemm_swz8(row)) + 8 * (c & 1));
      else
        f.b[ks][j] = *reinterpret_cast<const half8*>(bs + 8 * gemm_slot(row, c));
    }
  }
  if constexpr (BF8) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < NJ; ++j) f.b[ks][j] = e4m3x8_to_half8(b8[ks][j].x, b8[ks][j].y);
  }
}

typedef __bf16 bf16x8_g __attribute__((ext_vector_type(8)));

// MFMA half-step: the wave's 128 x (TN / 4) block, 4 x (TN / 128) accumulators of 32 x 32, both 16-K steps.
// BF16: the fragments hold bf16 bit patterns (v_mfma_f32_32x32x16_bf16), else fp16.
template <int TN, bool BF16 = false>
DG_DEV void gemm_mfma(const GemmFrag<TN>& f, floatx16 (&acc)[4][TN / 128]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TN / 128; ++j) {
        if constexpr (BF16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_g, f.a[ks][i]),
                                                              __builtin_bit_cast(bf16x8_g, f.b[ks][j]), acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[ks][i], f.b[ks][j], acc[i][j], 0, 0, 0);
      }
}

// vector-memory instructions a wave issues per stage
template <int TN, bool BF8>
constexpr int gemm_dma_per_stage() {
  return (kGemmTM / 16 + (BF8 ? TN / 32 : TN / 16)) / kGemmWaves;
}

// Wait until at most `pending` (0..3) later stages of this wave's copies are still in flight.
template <int TN, bool BF8>
DG_DEV void gemm_vmwait(int pending) {
  constexpr int n = gemm_dma_per_stage<TN, BF8>();
  if (pending >= 3)
    __builtin_amdgcn_s_waitcnt(vmcnt_only(3 * n));
  else if (pending == 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * n));
  else if (pending == 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_only(n));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
}

// A bare s_barrier is used instead of __syncthreads(): the latter's release fence would wait for
// every outstanding copy, including the prefetched stages.  The empty asm statements and scheduling
// barriers keep the compiler from moving LDS accesses or MFMAs across it.
DG_DEV void gemm_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Operand source of the main loop for the K-blocked operands of GemmArgs: issue(s, as, bs) starts
// the copies of stage s (K offset s * kGemmTK of the workgroup's range) into the given LDS buffers;
// fix(f, s) adjusts the fragments of stage s after their LDS read (nothing here).
template <int TN, bool BF8, bool BNT = true>
struct GemmSrc {
  const GemmArgs& g;
  int m0, n0, k_begin;
  uint32_t off, off8;
  int wave;
  DG_DEV void issue(int s, _Float16* as, _Float16* bs) const {
    gemm_issue<TN, BF8, BNT>(g, m0, n0, k_begin + s * kGemmTK, off, off8, wave, as, bs);
  }
  DG_DEV void fix(GemmFrag<TN>&, int) const {}
};

// The main loop over nstage stages of K into acc (zeroed here).
// PP: ping-pong schedule (long K loops); otherwise all eight waves read and multiply each stage
// together between one barrier per stage (short K loops, where the ping-pong's extra barriers and
// its staggered start cost more than they hide).
// PRIO (ping-pong only): the group in its MFMA half-step runs at raised wave priority, so the other
// group's LDS reads and copies do not delay its MFMA issue.  Measured 4 % faster on launches with
// many M tiles (8192 rows) and 0.5-1 % slower with one M tile, where it stays off.
template <int TN, bool BF8, bool PP, bool BF16, bool PRIO = false, class Src>
DG_DEV void gemm_main(const Src& src, int nstage, _Float16* As, _Float16* Bs, int wm, int wn, int lane, int group,
                      floatx16 (&acc)[4][TN / 128]) {
  constexpr int NJ = TN / 128;
  constexpr int kAs = kGemmTM * kGemmTK;                     // halves per A stage
  constexpr int kBs = BF8 ? TN * kGemmTK / 2 : TN * kGemmTK;  // halves per B stage
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  GemmFrag<TN> f;

  if constexpr (!PP) {
    // iteration s: wait for stage s, barrier (stage s visible; every wave is past MFMA(s - 1), so
    // that stage's buffer may be refilled), issue stage s + 3, read and multiply stage s
    const int pro = min(kGemmStages - 1, nstage);
    for (int s = 0; s < pro; ++s) src.issue(s, As + s * kAs, Bs + s * kBs);
    for (int s = 0; s < nstage; ++s) {
      gemm_vmwait<TN, BF8>(min(kGemmStages - 2, nstage - 1 - s));
      gemm_barrier();
      if (s + kGemmStages - 1 < nstage) {
        const int nb = (s + kGemmStages - 1) & (kGemmStages - 1);
        src.issue(s + kGemmStages - 1, As + nb * kAs, Bs + nb * kBs);
      }
      const int buf = s & (kGemmStages - 1);
      gemm_read<TN, BF8>(As + buf * kAs, Bs + buf * kBs, wm, wn, lane, f);
      src.fix(f, s);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead (the scheduler would sink them to their uses)
      gemm_mfma<TN, BF16>(f, acc);
    }
  } else {
    const int pro = min(kGemmStages, nstage);
    for (int s = 0; s < pro; ++s) src.issue(s, As + s * kAs, Bs + s * kBs);
    gemm_vmwait<TN, BF8>(pro - 1);
    gemm_barrier();
    // Every wave runs read(s) | barrier | MFMA(s) | barrier; group 1 starts one barrier late (and
    // group 0 ends one barrier late), so between two barriers one group reads while the other
    // multiplies.  Stage s + 3 refills the buffer of stage s - 1, which both groups have read (and
    // waited for) before the barrier that precedes this half-step.  Before its barrier each wave
    // waits for its own copies of stage s + 1, which the next read half-step needs.
    if (group == 1) gemm_barrier();
    for (int s = 0; s < nstage; ++s) {
      const int buf = s & (kGemmStages - 1);
      gemm_read<TN, BF8>(As + buf * kAs, Bs + buf * kBs, wm, wn, lane, f);
      src.fix(f, s);
      if (s >= 1 && s + kGemmStages - 1 < nstage) {
        const int nb = (s + kGemmStages - 1) & (kGemmStages - 1);
        src.issue(s + kGemmStages - 1, As + nb * kAs, Bs + nb * kBs);
      }
      __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
      gemm_vmwait<TN, BF8>(min(kGemmStages - 2, max(0, nstage - 2 - s)));
      gemm_barrier();
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
      gemm_mfma<TN, BF16>(f, acc);
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
      gemm_barrier();
    }
    if (group == 0) gemm_barrier();
  }
}

// The split-K GEMM; BF8: the right operand is E4M3 (g.Bt8), converted to fp16 fragment by fragment;
// BNT: the fp16 right operand is loaded non-temporally (launches with one M tile).
template <int TN, bool BF8, bool PP, bool BNT = true>
DG_DEV void gemm_splitk_body(const GemmArgs& g) {
  constexpr int NJ = TN / 128;
  constexpr int kAs = kGemmTM * kGemmTK;                     // halves per A stage
  constexpr int kBs = BF8 ? TN * kGemmTK / 2 : TN * kGemmTK;  // halves per B stage
  __shared__ __attribute__((aligned(16))) _Float16 As[kGemmStages * kAs];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[kGemmStages * kBs];
  // XCD-aware tile order: XCD x owns the contiguous range [x per_xcd, (x + 1) per_xcd) of linear
  // tiles and its 32 CUs run 32 consecutive ones at a time.  One M tile (the single canvas): t =
  // (split * ntiles + ntile) * mtiles + mtile, so the 32 concurrent tiles are N tiles of one split and
  // share their A chunk.  Several M tiles (a batch of canvases, B loaded normally): within a split t
  // walks blocks of 4 M tiles x 8 N tiles, one block per 32 consecutive tiles, so the concurrent
  // workgroups share 4 A and 8 B chunks through the XCD's L2 instead of reading 32 A chunks.
  const int total = g.mtiles * g.ntiles * g.splits;
  const int per_xcd = (total + kGemmXcds - 1) / kGemmXcds;
  const int t = (blockIdx.x % kGemmXcds) * per_xcd + blockIdx.x / kGemmXcds;
  if (t >= total) return;
  int mt, nt, split;
  if (!BNT && g.mtiles % 4 == 0 && g.ntiles % 8 == 0 && per_xcd % 32 == 0) {
    const int per_split = g.mtiles * g.ntiles;  // a multiple of 32
    split = t / per_split;
    const int loc = t - split * per_split, blk = loc / 32, l = loc % 32, nbn = g.ntiles / 8;
    mt = (blk / nbn) * 4 + l / 8;
    nt = (blk % nbn) * 8 + l % 8;
  } else {
    mt = t % g.mtiles;
    nt = (t / g.mtiles) % g.ntiles;
    split = t / (g.mtiles * g.ntiles);
  }
  const int m0 = mt * kGemmTM, n0 = nt * TN;
  const int k_begin = split * g.kchunk;
  const int k_end = min(g.K, k_begin + g.kchunk);
  const int nstage = (k_end - k_begin) / kGemmTK;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int group = wave >> 2;  // one wave of each group per SIMD
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * (TN / 4);

  floatx16 acc[4][NJ];
  gemm_main<TN, BF8, PP, false, !BNT>(GemmSrc<TN, BF8, BNT>{g, m0, n0, k_begin, gemm_lane_offset(),
                                                       BF8 ? gemm_lane_offset8() : 0u, wave},
                                nstage, As, Bs, wm, wn, lane, group, acc);
  // accumulator element e of lane l: row 8 * (e / 4) + 4 * (l / 32) + e % 4, column l % 32
  float* out = g.part + static_cast<int64_t>(split) * g.M * g.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int n = n0 + wn + j * 32 + (lane & 31);
        if (m < g.M) out[static_cast<int64_t>(m) * g.N + n] = acc[i][j][e];
      }
}

// ROLE names the instantiation (0: P.E contraction, ping-pong schedule; 1: MLP GEMMs, one barrier per
// stage), so that profilers also report the dominant P.E launch under its own symbol.  TN is the N tile (256, or 128 when N is not a multiple
// of 256).
template <int ROLE, int TN, bool BNT = true>
__global__ __launch_bounds__(kGemmThreads) void gemm_f16_splitk_kernel(GemmArgs g) {
  gemm_splitk_body<TN, false, ROLE == 0, BNT>(g);
}


struct GemmPlan {
  int32_t splits, kchunk, mtiles, ntiles, tn;
  dim3 grid;
};

// N % 128 == 0 and K % 128 == 0 are required (every split runs a whole number of 4-stage rounds);
// M may be ragged.  The N tile is 256 when N allows it and `narrow` is false, else 128.
// About `target_wgs` workgroups (one per CU by default; each holds up to ~144 KB of LDS); splits
// are added only to reach that.
inline GemmPlan plan_gemm(int32_t M, int32_t N, int32_t K, int32_t target_wgs = 256, bool narrow = false) {
  const int32_t tn = (N % 256 == 0 && !narrow) ? 256 : 128;
  const int32_t mtiles = (M + kGemmTM - 1) / kGemmTM, ntiles = N / tn;
  const int32_t tiles = mtiles * ntiles;
  int32_t splits = (target_wgs + tiles - 1) / tiles;
  const int32_t max_splits = (K + 255) / 256;
  splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
  int32_t kchunk = (K + splits - 1) / splits;
  constexpr int32_t round = kGemmStages * kGemmTK;
  kchunk = (kchunk + round - 1) / round * round;
  splits = (K + kchunk - 1) / kchunk;
  const int32_t total = tiles * splits;
  const int32_t launched = (total + kGemmXcds - 1) / kGemmXcds * kGemmXcds;
  return {splits, kchunk, mtiles, ntiles, tn, dim3(launched)};
}

// The same tiling with a given K per split (a multiple of kGemmStages * kGemmTK), so that the split
// of K -- and with it the order of every output's partial sums -- does not depend on M.
inline GemmPlan plan_gemm_kchunk(int32_t M, int32_t N, int32_t K, int32_t kchunk, bool narrow = false) {
  const int32_t tn = (N % 256 == 0 && !narrow) ? 256 : 128;
  const int32_t mtiles = (M + kGemmTM - 1) / kGemmTM, ntiles = N / tn;
  const int32_t splits = (K + kchunk - 1) / kchunk;
  const int32_t total = mtiles * ntiles * splits;
  const int32_t launched = (total + kGemmXcds - 1) / kGemmXcds * kGemmXcds;
  return {splits, kchunk, mtiles, ntiles, tn, dim3(launched)};
}

inline GemmArgs gemm_args(const _Float16* A, int64_t lda, const _Float16* Bt, int64_t ldb, float* part, int32_t M,
                          int32_t N, int32_t K, const GemmPlan& p, const uint8_t* Bt8 = nullptr) {
  return GemmArgs{A, lda, Bt, ldb, Bt8, part, M, N, K, p.kchunk, p.mtiles, p.ntiles, p.splits};
}

}  // namespace dg
