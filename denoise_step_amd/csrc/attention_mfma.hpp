// bf16 MFMA flash attention for dg_canvas_attention (head_dim 128 / 256).
//
// Work item: (request, KV head, tile of 128 packed query rows, KV split).  A
// packed query row is m = j * G + g (row j of the request, query head
// hk * G + g of the KV group), so the G query heads that share a KV head share
// every K/V tile.  Four wave64s own 32 packed rows each.
//
// Per 64-key block the wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (A = K from LDS, B = Q preloaded in registers): each lane then holds 16
// scores of ONE query row, so the online softmax is in-lane plus one xor-32
// shuffle.  The probabilities stay in registers as the B operand of
// O^T = V^T P^T (A = V^T read from a transposed LDS copy of the V block); the
// key order inside each 16-key MFMA step is permuted consistently on both
// operands to match the accumulator layout.  O^T accumulates in fp32 (each
// lane again owns one row, so the rescale is in-lane).
//
// Visibility (per request): key index kk (cache positions first, then canvas
// rows) is visible to causal row j iff kk <= cached + j, to a canvas row
// always.  Blocks past the last visible key of the tile are never loaded
// (tiles holding only masked entries are skipped).  With several KV splits each
// split writes unnormalised partials (O, running max, running sum) and a merge
// kernel combines them with log-sum-exp weights.
#pragma once
#include "dg_device.hpp"

namespace dg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kAttRows = 128;   // packed query rows per workgroup
constexpr int kAttKeys = 64;    // keys per block
constexpr int kAttThreads = 256;
constexpr int kAttMaxPages = 1024;  // page ids of one split staged in LDS (16K keys)
constexpr float kLog2e = 1.4426950408889634f;

struct AttArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int32_t n_pages;
  const int32_t* page_table;
  int32_t page_table_len;
  const dg_split* splits;
  int32_t rows, Hq, Hkv, G, page_size;
  float scale_log2;     // scale * log2(e)
  int32_t nsplit;       // KV splits
  int32_t split_keys;   // keys per split (multiple of kAttKeys)
  uint16_t* out;        // [rows][Hq][D] bf16 (nsplit == 1)
  float* o_part;        // [nsplit][rows][Hq][D] (nsplit > 1)
  float2* ml_part;      // [nsplit][rows][Hq]    (nsplit > 1)
};

template <int D>
struct AttSmem {
  static constexpr int kPitch = D + 8;          // bf16 per K row in LDS
  static constexpr int vPitch = kAttKeys + 4;   // bf16 per transposed V row in LDS
  uint16_t K[2][kAttKeys * kPitch];
  uint16_t Vt[2][D * vPitch];
  int32_t pages[kAttMaxPages];
};

// Registers holding one key block between its global loads and its LDS stores.
template <int D>
struct AttStage {
  static constexpr int kChunks = D / 8;
  static constexpr int kK = kAttKeys * kChunks / kAttThreads;        // 16-byte K chunks per lane
  static constexpr int kV = (kAttKeys / 2) * kChunks / kAttThreads;  // V key-pair chunks per lane
  uint4 k[kK];
  uint4 v0[kV], v1[kV];
};

// Key kk of a request: cache positions come from the staged page ids (index and id clamped, so a
// stale entry can only give a wrong key, never an out-of-range address), canvas keys from k / v.
template <int D>
DG_DEV const uint16_t* att_row(const AttArgs& a, const dg_split& sp, const int32_t* pages, int32_t page_lo, int hk,
                               int kk, int n_cache, bool is_v) {
  if (kk < n_cache) {
    const int slot = min(max(kk / 16 - page_lo, 0), kAttMaxPages - 1);
    const int64_t page = min(max(pages[slot], 0), a.n_pages - 1);
    return (is_v ? a.v_cache : a.k_cache) + ((page * a.Hkv + hk) * 16 + (kk & 15)) * D;
  }
  const int64_t row = sp.row0 + sp.n_causal + (kk - n_cache);
  return (is_v ? a.v : a.k) + (row * a.Hkv + hk) * D;
}

// Keys at or past k_end (the split's last visible key + 1) are masked for every row of the tile;
// they are filled with zeros and never loaded (their pages are not staged).
template <int D>
DG_DEV void att_load(const AttArgs& a, const dg_split& sp, const int32_t* pages, int32_t page_lo, int hk, int kb,
                     int n_cache, int k_end, AttStage<D>& st) {
  constexpr int kChunks = D / 8;
#pragma unroll
  for (int i = 0; i < AttStage<D>::kK; ++i) {
    const int u = threadIdx.x + i * kAttThreads;
    const int kk = kb + u / kChunks, c = u % kChunks;
    st.k[i] = (kk < k_end) ? *reinterpret_cast<const uint4*>(att_row<D>(a, sp, pages, page_lo, hk, kk, n_cache, false) + 8 * c)
                             : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < AttStage<D>::kV; ++i) {
    const int u = threadIdx.x + i * kAttThreads;
    const int pair = u % (kAttKeys / 2), c = u / (kAttKeys / 2);
    const int kk = kb + 2 * pair;
    st.v0[i] = (kk < k_end) ? *reinterpret_cast<const uint4*>(att_row<D>(a, sp, pages, page_lo, hk, kk, n_cache, true) + 8 * c)
                              : make_uint4(0, 0, 0, 0);
    st.v1[i] = (kk + 1 < k_end)
                   ? *reinterpret_cast<const uint4*>(att_row<D>(a, sp, pages, page_lo, hk, kk + 1, n_cache, true) + 8 * c)
                   : make_uint4(0, 0, 0, 0);
  }
}

template <int D>
DG_DEV void att_store(AttSmem<D>& sm, int buf, const AttStage<D>& st) {
  constexpr int kChunks = D / 8;
#pragma unroll
  for (int i = 0; i < AttStage<D>::kK; ++i) {
    const int u = threadIdx.x + i * kAttThreads;
    *reinterpret_cast<uint4*>(&sm.K[buf][(u / kChunks) * AttSmem<D>::kPitch + 8 * (u % kChunks)]) = st.k[i];
  }
#pragma unroll
  for (int i = 0; i < AttStage<D>::kV; ++i) {
    const int u = threadIdx.x + i * kAttThreads;
    const int pair = u % (kAttKeys / 2), c = u / (kAttKeys / 2);
    const uint32_t w0[4] = {st.v0[i].x, st.v0[i].y, st.v0[i].z, st.v0[i].w};
    const uint32_t w1[4] = {st.v1[i].x, st.v1[i].y, st.v1[i].z, st.v1[i].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // d = 8c + 2t (low halves) and 8c + 2t + 1 (high halves); keys 2 pair, 2 pair + 1
      const uint32_t lo = (w0[t] & 0xFFFFu) | (w1[t] << 16);
      const uint32_t hi = (w0[t] >> 16) | (w1[t] & 0xFFFF0000u);
      *reinterpret_cast<uint32_t*>(&sm.Vt[buf][(8 * c + 2 * t) * AttSmem<D>::vPitch + 2 * pair]) = lo;
      *reinterpret_cast<uint32_t*>(&sm.Vt[buf][(8 * c + 2 * t + 1) * AttSmem<D>::vPitch + 2 * pair]) = hi;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kAttThreads) void attend_mfma_kernel(AttArgs a) {
  constexpr int kDSteps = D / 16;                // MFMA k-steps over D
  constexpr int kDTiles = D / 32;                // 32-wide output tiles over D
  __shared__ __attribute__((aligned(16))) AttSmem<D> sm;

  const dg_split sp = a.splits[blockIdx.z];
  const int hk = blockIdx.y % a.Hkv;
  const int split = blockIdx.y / a.Hkv;
  const int nr = sp.n_causal + sp.n_canvas;
  const int m_tile0 = blockIdx.x * kAttRows;
  if (m_tile0 >= nr * a.G) return;
  const int n_cache = sp.cached + sp.n_causal;
  const int n_total = n_cache + sp.n_canvas;
  // last visible key + 1 over the tile's rows (rows are ordered causal then canvas)
  const int j_last = min(nr - 1, (m_tile0 + kAttRows - 1) / a.G);
  const int tile_lim = (j_last < sp.n_causal) ? sp.cached + j_last + 1 : n_total;
  const int k_begin = split * a.split_keys;
  const int k_end = min(tile_lim, k_begin + a.split_keys);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int half = lane >> 5;
  const int m = m_tile0 + wave * 32 + (lane & 31);
  const bool row_ok = m < nr * a.G;
  const int j = row_ok ? m / a.G : 0;
  const int h = hk * a.G + (row_ok ? m % a.G : 0);
  const int row = sp.row0 + j;
  const int lim = !row_ok ? 0 : (j < sp.n_causal ? sp.cached + j + 1 : n_total);

  // stage the physical page ids of the split's cache positions (clamped into range)
  const int page_lo = k_begin / 16;
  const int page_hi = min((min(k_end, n_cache) + 15) / 16, page_lo + kAttMaxPages);
  for (int p = page_lo + tid; p < page_hi; p += kAttThreads) {
    const int ti = min(max(sp.page0 + p, 0), a.page_table_len - 1);
    sm.pages[p - page_lo] = min(max(a.page_table[ti], 0), a.n_pages - 1);
  }

  // Q fragment (B operand of S^T = K Q^T): 8 consecutive d per MFMA step
  bf16x8 qf[kDSteps];
  {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(row_ok ? row : sp.row0) * a.Hq + h) * D;
#pragma unroll
    for (int s = 0; s < kDSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * half);
  }

  floatx16 o[kDTiles];
#pragma unroll
  for (int t = 0; t < kDTiles; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  AttStage<D> st;
  __syncthreads();  // page ids visible
  if (k_begin < k_end) {
    att_load<D>(a, sp, sm.pages, page_lo, hk, k_begin, n_cache, k_end, st);
    att_store<D>(sm, 0, st);
  }
  __syncthreads();
  int buf = 0;
  for (int kb = k_begin; kb < k_end; kb += kAttKeys) {
    const bool more = kb + kAttKeys < k_end;
    if (more) att_load<D>(a, sp, sm.pages, page_lo, hk, kb + kAttKeys, n_cache, k_end, st);
    const uint16_t* Kb = sm.K[buf];
    const uint16_t* Vb = sm.Vt[buf];
    // ---- S^T = K Q^T : two 32-key sub-blocks x 32 rows
    floatx16 sc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[b][e] = 0.f;
#pragma unroll
      for (int s = 0; s < kDSteps; ++s) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&Kb[(32 * b + (lane & 31)) * AttSmem<D>::kPitch + 16 * s + 8 * half]);
        sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sc[b], 0, 0, 0);
      }
    }
    // ---- online softmax; element e of sub-block b holds key 32 b + 8 (e / 4) + 4 half + e % 4 of this lane's row
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb + 32 * b + 8 * (e >> 2) + 4 * half + (e & 3);
        sc[b][e] = (key < lim) ? sc[b][e] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[b][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = (sc[b][e] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[b][e] - m_new);
        psum += p;
        pf[2 * b + (e >> 3)][e & 7] = static_cast<__bf16>(p);
      }
    psum += __shfl_xor(psum, 32, kWave);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {  // the running max moved for some row of the wave
#pragma unroll
      for (int t = 0; t < kDTiles; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[t][e] *= alpha;
    }
    // ---- O^T += V^T P^T over four 16-key chunks; key slots follow the accumulator layout
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int t = 0; t < kDTiles; ++t) {
        const uint16_t* vrow = &Vb[(32 * t + (lane & 31)) * AttSmem<D>::vPitch + 16 * c + 4 * half];
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], o[t], 0, 0, 0);
      }
    }
    if (more) att_store<D>(sm, buf ^ 1, st);
    __syncthreads();
    buf ^= 1;
  }

  if (!row_ok) return;
  // O^T element e of tile t: d = 32 t + 8 (e / 4) + 4 half + e % 4, row = this lane's row
  if (a.nsplit == 1) {
    const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
    uint16_t* orow = a.out + (static_cast<int64_t>(row) * a.Hq + h) * D;
#pragma unroll
    for (int t = 0; t < kDTiles; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * t + 8 * g4 + 4 * half;
        uint2 w;
        w.x = static_cast<uint32_t>(f32_to_bf16(o[t][4 * g4] * inv)) |
              (static_cast<uint32_t>(f32_to_bf16(o[t][4 * g4 + 1] * inv)) << 16);
        w.y = static_cast<uint32_t>(f32_to_bf16(o[t][4 * g4 + 2] * inv)) |
              (static_cast<uint32_t>(f32_to_bf16(o[t][4 * g4 + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
  } else {
    const int64_t ridx = static_cast<int64_t>(split) * a.rows * a.Hq + static_cast<int64_t>(row) * a.Hq + h;
    float* orow = a.o_part + ridx * D;
#pragma unroll
    for (int t = 0; t < kDTiles; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * t + 8 * g4 + 4 * half;
        *reinterpret_cast<float4*>(orow + d) =
            make_float4(o[t][4 * g4], o[t][4 * g4 + 1], o[t][4 * g4 + 2], o[t][4 * g4 + 3]);
      }
    if (half == 0) a.ml_part[ridx] = make_float2(m_run, l_run);
  }
}

// Combine KV splits: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.  One workgroup per (row, head).
template <int D>
__global__ __launch_bounds__(D) void attend_merge_kernel(const float* __restrict__ o_part,
                                                         const float2* __restrict__ ml_part, int32_t nsplit,
                                                         int32_t rows, int32_t Hq, const dg_split* __restrict__ splits,
                                                         int32_t n_req, uint16_t* __restrict__ out) {
  const int64_t rh = blockIdx.x;  // row * Hq + h
  const int row = static_cast<int>(rh / Hq);
  // rows outside every request's range were never written: skip them
  bool owned = false;
  for (int r = 0; r < n_req && !owned; ++r) {
    const dg_split sp = splits[r];
    owned = row >= sp.row0 && row < sp.row0 + sp.n_causal + sp.n_canvas;
  }
  if (!owned) return;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml_part[s * static_cast<int64_t>(rows) * Hq + rh].x);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float2 ml = ml_part[s * static_cast<int64_t>(rows) * Hq + rh];
    if (ml.x == -INFINITY) continue;
    const float w = exp2f(ml.x - M);
    L += w * ml.y;
    acc += w * o_part[(s * static_cast<int64_t>(rows) * Hq + rh) * D + threadIdx.x];
  }
  out[rh * D + threadIdx.x] = f32_to_bf16(L > 0.f ? acc / L : 0.f);
}

}  // namespace dg
