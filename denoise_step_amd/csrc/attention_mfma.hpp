// bf16 MFMA flash attention for dg_canvas_attention (head_dim 128 / 256).
//
// Work item: (request, KV head, tile of 128 packed query rows, KV split).  A
// packed query row is m = j * G + g (row j of the request, query head
// hk * G + g of the KV group), so the G query heads that share a KV head share
// every K/V tile.  Four wave64s own 32 packed rows each.
//
// Per 32-key block the wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
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
constexpr int kAttKeys = 32;    // keys per block
constexpr int kAttThreads = 256;
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
  uint16_t K[kAttKeys * kPitch];
  uint16_t Vt[D * vPitch];
};

DG_DEV const uint16_t* att_key_row(const AttArgs& a, const dg_split& sp, int32_t hk, int32_t kk, int32_t n_cache,
                                   bool is_v, int D) {
  if (kk < n_cache) {
    const int32_t ti = min(max(sp.page0 + kk / a.page_size, 0), a.page_table_len - 1);
    const int64_t page = min(max(a.page_table[ti], 0), a.n_pages - 1);
    const int64_t off = ((page * a.Hkv + hk) * a.page_size + kk % a.page_size) * D;
    return (is_v ? a.v_cache : a.k_cache) + off;
  }
  const int64_t row = sp.row0 + sp.n_causal + (kk - n_cache);
  return (is_v ? a.v : a.k) + (row * a.Hkv + hk) * D;
}

template <int D>
__global__ __launch_bounds__(kAttThreads) void attend_mfma_kernel(AttArgs a) {
  constexpr int kChunks = D / 8;                 // 16-byte chunks per key row
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

  for (int kb = k_begin; kb < k_end; kb += kAttKeys) {
    __syncthreads();  // previous block's LDS reads are done
    // ---- stage K (row-major) and V (transposed) for keys kb .. kb+31
    for (int u = tid; u < kAttKeys * kChunks; u += kAttThreads) {
      const int key = u / kChunks, c = u % kChunks;
      const int kk = kb + key;
      uint4 kv = make_uint4(0, 0, 0, 0);
      if (kk < n_total) kv = *reinterpret_cast<const uint4*>(att_key_row(a, sp, hk, kk, n_cache, false, D) + 8 * c);
      *reinterpret_cast<uint4*>(&sm.K[key * AttSmem<D>::kPitch + 8 * c]) = kv;
    }
    for (int u = tid; u < (kAttKeys / 2) * kChunks; u += kAttThreads) {
      const int pair = u % (kAttKeys / 2), c = u / (kAttKeys / 2);
      const int kk = kb + 2 * pair;
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
      if (kk < n_total) v0 = *reinterpret_cast<const uint4*>(att_key_row(a, sp, hk, kk, n_cache, true, D) + 8 * c);
      if (kk + 1 < n_total)
        v1 = *reinterpret_cast<const uint4*>(att_key_row(a, sp, hk, kk + 1, n_cache, true, D) + 8 * c);
      const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
      const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // d = 8c + 2t (low halves) and 8c + 2t + 1 (high halves)
        const uint32_t lo = (w0[t] & 0xFFFFu) | (w1[t] << 16);
        const uint32_t hi = (w0[t] >> 16) | (w1[t] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(&sm.Vt[(8 * c + 2 * t) * AttSmem<D>::vPitch + 2 * pair]) = lo;
        *reinterpret_cast<uint32_t*>(&sm.Vt[(8 * c + 2 * t + 1) * AttSmem<D>::vPitch + 2 * pair]) = hi;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T : 32 keys x 32 rows
    floatx16 st;
#pragma unroll
    for (int e = 0; e < 16; ++e) st[e] = 0.f;
#pragma unroll
    for (int s = 0; s < kDSteps; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sm.K[(lane & 31) * AttSmem<D>::kPitch + 16 * s + 8 * half]);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st, 0, 0, 0);
    }
    // ---- online softmax; element e holds key 8 * (e / 4) + 4 * half + e % 4 of this lane's row
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kb + 8 * (e >> 2) + 4 * half + (e & 3);
      st[e] = (key < lim) ? st[e] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, st[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = (st[e] == -INFINITY) ? 0.f : exp2f(st[e] - m_new);
      psum += p;
      pf[e >> 3][e & 7] = static_cast<__bf16>(p);
    }
    psum += __shfl_xor(psum, 32, kWave);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < kDTiles; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] *= alpha;

    // ---- O^T += V^T P^T over two 16-key chunks; key slots follow the accumulator layout
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int t = 0; t < kDTiles; ++t) {
        const uint16_t* vrow = &sm.Vt[(32 * t + (lane & 31)) * AttSmem<D>::vPitch + 16 * c + 4 * half];
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], o[t], 0, 0, 0);
      }
    }
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
