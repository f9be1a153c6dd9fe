// dg_canvas_attention: mixed-mask attention over a paged KV prefix.
//
// Method: DiffusionGemma/vLLM page, section "Two modes, one set of weights"
// (encoder rows are causal and write K/V; decoder/canvas rows are
// bidirectional and only read K/V) and section "Dynamic per-sequence causal
// attention" (causality per request inside one batch; tiles holding only
// masked entries are skipped); single-pass-reads page, section on keeping
// each row's visibility (a request split into causal input rows and canvas
// rows that share its KV block table; the p0 p1 c0 c1 example); section on
// symmetric sliding-window attention (a window W keeps causal rows' keys
// within W before the row and canvas rows' within W on both sides).
//
// bf16, head_dim 128 / 256: one MFMA kernel reads prefix keys from the pages
// and causal / canvas keys from the k/v inputs, and appends the causal rows'
// K/V to the pages itself (then a merge kernel if the keys were split).
// Other shapes: (1) the causal rows' K/V are appended to the request's pages
// at positions cached + j; (2) one wave per (row, head) reads every prefix and
// causal key from the pages and the canvas keys from the k/v inputs.
#include "attention_mfma.hpp"
#include "dg_device.hpp"
#include "dg_host.hpp"

#include <algorithm>
#include <cmath>

namespace dg {
namespace {

template <bool BF16>
DG_DEV float ld_elem(const void* p, int64_t i) {
  if constexpr (BF16)
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else
    return reinterpret_cast<const float*>(p)[i];
}

DG_DEV int32_t clamp_page(int32_t p, int32_t n_pages) { return min(max(p, 0), n_pages - 1); }

DG_DEV int32_t page_of(const int32_t* page_table, int32_t page_table_len, int32_t n_pages, const dg_split& sp,
                       int32_t pos, int32_t page_size) {
  const int32_t idx = min(max(sp.page0 + pos / page_size, 0), page_table_len - 1);
  return clamp_page(page_table[idx], n_pages);
}

// (1) append: one workgroup per (request, causal row); element-wise copy of Hkv * D values.
template <bool BF16>
__global__ void append_kv_kernel(const void* __restrict__ k, const void* __restrict__ v, void* __restrict__ k_cache,
                                 void* __restrict__ v_cache, int32_t n_pages, const int32_t* __restrict__ page_table,
                                 int32_t page_table_len, const dg_split* __restrict__ splits, int32_t rows,
                                 int32_t Hkv, int32_t D, int32_t page_size) {
  const dg_split sp = splits[blockIdx.y];
  const int j = blockIdx.x;
  if (j >= sp.n_causal) return;
  const int32_t row = sp.row0 + j;
  if (row < 0 || row >= rows) return;
  const int32_t pos = sp.cached + j;
  const int64_t page = page_of(page_table, page_table_len, n_pages, sp, pos, page_size);
  const int32_t slot = pos % page_size;
  const int n = Hkv * D;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int h = e / D, d = e - h * D;
    const int64_t src = (static_cast<int64_t>(row) * Hkv + h) * D + d;
    const int64_t dst = ((page * Hkv + h) * page_size + slot) * D + d;
    if constexpr (BF16) {
      reinterpret_cast<uint16_t*>(k_cache)[dst] = reinterpret_cast<const uint16_t*>(k)[src];
      reinterpret_cast<uint16_t*>(v_cache)[dst] = reinterpret_cast<const uint16_t*>(v)[src];
    } else {
      reinterpret_cast<float*>(k_cache)[dst] = reinterpret_cast<const float*>(k)[src];
      reinterpret_cast<float*>(v_cache)[dst] = reinterpret_cast<const float*>(v)[src];
    }
  }
}

// (2) one wave per (query row, query head): keys in blocks of 64, one key per lane for the
// score, online softmax across blocks, each lane owning D / 64 output columns.
template <bool BF16, int D>
__global__ __launch_bounds__(kWave) void attend_wave_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ k_cache, const void* __restrict__ v_cache, int32_t n_pages,
    const int32_t* __restrict__ page_table, int32_t page_table_len, const dg_split* __restrict__ splits,
    int32_t rows, int32_t Hq, int32_t Hkv, int32_t page_size, float scale, void* __restrict__ out) {
  constexpr int kCols = (D + kWave - 1) / kWave;
  __shared__ float qs[D];
  const dg_split sp = splits[blockIdx.z];
  const int j = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  if (j >= sp.n_causal + sp.n_canvas) return;
  const int32_t row = sp.row0 + j;
  if (row < 0 || row >= rows) return;
  const int hk = h / (Hq / Hkv);
  const int32_t n_cache = sp.cached + sp.n_causal;
  const int2 rk = att_row_keys(sp, j);  // visible keys [rk.x, rk.y)
  const int32_t k_lo = rk.x, n_vis = rk.y;
  for (int d = lane; d < D; d += kWave) qs[d] = ld_elem<BF16>(q, (static_cast<int64_t>(row) * Hq + h) * D + d) * scale;
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) acc[c] = 0.f;

  for (int kb = k_lo; kb < n_vis; kb += kWave) {
    const int kk = kb + lane;
    int64_t kbase = -1;  // element offset of this lane's key row (K and V share the layout)
    const void* ksrc = nullptr;
    const void* vsrc = nullptr;
    float s = -INFINITY;
    if (kk < n_vis) {
      if (kk < n_cache) {
        const int64_t page = page_of(page_table, page_table_len, n_pages, sp, kk, page_size);
        kbase = ((page * Hkv + hk) * page_size + kk % page_size) * D;
        ksrc = k_cache;
        vsrc = v_cache;
      } else {
        const int64_t crow = min(max(sp.row0 + sp.n_causal + (kk - n_cache), 0), rows - 1);  // clamped
        kbase = (crow * Hkv + hk) * D;
        ksrc = k;
        vsrc = v;
      }
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], ld_elem<BF16>(ksrc, kbase + d), dot);
      s = dot;
    }
    const float bm = wave_max(s);
    const float mn = fmaxf(m, bm);
    const float f = (m == -INFINITY) ? 0.f : __expf(m - mn);
    const float p = (kk < n_vis) ? __expf(s - mn) : 0.f;
    l = l * f + wave_sum(p);
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[c] *= f;
    m = mn;
    const int nb = min(kWave, n_vis - kb);
    for (int i = 0; i < nb; ++i) {
      const float pi = __shfl(p, i, kWave);
      const int64_t vb = __shfl(kbase, i, kWave);
      const bool from_cache = (kb + i) < n_cache;
      const void* vs = from_cache ? v_cache : v;
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        const int d = lane + c * kWave;
        if (d < D) acc[c] = fmaf(pi, ld_elem<BF16>(vs, vb + d), acc[c]);
      }
    }
    (void)vsrc;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    const int d = lane + c * kWave;
    if (d < D) {
      const int64_t o = (static_cast<int64_t>(row) * Hq + h) * D + d;
      if constexpr (BF16)
        reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16(acc[c] * inv);
      else
        reinterpret_cast<float*>(out)[o] = acc[c] * inv;
    }
  }
}

template <bool BF16, int D>
void launch_attend_wave(const void* q, const void* k, const void* v, const void* kc, const void* vc, int32_t n_pages,
                        const int32_t* pt, int32_t ptl, const dg_split* splits, int32_t n_req, int32_t rows,
                        int32_t max_rows, int32_t Hq, int32_t Hkv, int32_t ps, float scale, void* out, hipStream_t s) {
  const dim3 grid(max_rows, Hq, n_req);
  attend_wave_kernel<BF16, D><<<grid, kWave, 0, s>>>(q, k, v, kc, vc, n_pages, pt, ptl, splits, rows, Hq, Hkv, ps,
                                                     scale, out);
}

// Host bounds of the MFMA path.  A request's splits depend on its own descriptor (att_nsplit), which
// the host does not see; from the launch bounds it sizes the grid (work items) and the split
// partials so that every set of descriptors within them fits:
//   a request has at most ns_hi = att_nsplit(1, nb_max) splits (the rule grows with the keys and
//   shrinks with the rows), and a split request at most T / (Hkv qt) + 1 splits plus the ones its
//   key span forces (T = att_target_items(tr), tr = att_tile_rows(D) packed rows per tile), so over
//   the launch
//     items      <= n_req T + Hkv extra (ceil(rows G / tr) + n_req)
//     split rows <= n_req ceil(tr T / Hq) + extra rows
//   with extra = 1 + ceil(nb_max / kAttMaxSplitBlocks); each bound also <= the plain product.
// The grid holds at most kAttMaxGrid workgroups (a few per CU); each walks its items in turn.
constexpr int64_t kAttMaxGrid = 4096;

struct AttPlan {
  bool mfma;
  int64_t item_cap, part_cap, grid;
  bool fits;  // items are numbered in 32 bits inside a request
  size_t off_ml, off_np, bytes;
};

AttPlan plan_attention(int32_t n_req, int32_t rows, int32_t max_rows, int32_t max_keys, int32_t Hq, int32_t Hkv,
                       int32_t D, int32_t dtype) {
  AttPlan p{};
  p.mfma = dtype == DG_BF16 && (D == 128 || D == 256);
  if (!p.mfma) return p;
  const int64_t G = Hq / Hkv;
  const int64_t tr = att_tile_rows(D), target = att_target_items(att_tile_rows(D));
  const int64_t qt_max = cdiv(static_cast<int64_t>(max_rows) * G, tr);
  const int64_t nb_max = cdiv(max_keys, kAttKeys);
  const int64_t ns_hi = att_nsplit<int64_t>(1, nb_max, Hkv, target);
  const int64_t extra = 1 + cdiv(nb_max, kAttMaxSplitBlocks);
  p.item_cap = std::min<int64_t>(static_cast<int64_t>(n_req) * ns_hi * Hkv * qt_max,
                                 static_cast<int64_t>(n_req) * target +
                                     Hkv * extra * (cdiv(static_cast<int64_t>(rows) * G, tr) + n_req));
  p.grid = round_up(static_cast<size_t>(std::min<int64_t>(p.item_cap, kAttMaxGrid)), 8);
  p.fits = p.item_cap < (int64_t{1} << 31);
  p.part_cap = ns_hi < 2 ? 0
                         : std::min<int64_t>(ns_hi * rows, static_cast<int64_t>(n_req) *
                                                                   cdiv(tr * target, Hq) +
                                                               extra * rows);
  if (p.part_cap > 0) {
    const size_t n = static_cast<size_t>(p.part_cap) * Hq;
    p.off_ml = round_up(n * D * sizeof(uint16_t), 256);
    p.off_np = round_up(p.off_ml + n * sizeof(float2), 256);
    p.bytes = p.off_np + 256;
  }
  return p;
}

// Both MFMA entry points: fill the arguments shared by the bf16 and E4M3 caches, launch the kernel
// and, with several key splits, the merge.
template <bool E8>
dg_status launch_mfma(AttArgs& a, const AttPlan& plan, const void* q, const void* k, const void* v, int32_t n_pages,
                      const int32_t* page_table, int32_t page_table_len, const dg_split* splits, int32_t n_req,
                      int32_t rows, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, float scale, void* out,
                      void* ws, hipStream_t s) {
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.n_pages = n_pages;
  a.page_table = page_table;
  a.page_table_len = page_table_len;
  a.splits = splits;
  a.rows = rows;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.page_size = page_size;
  a.scale_log2 = scale * kLog2e;
  a.tile_rows = att_tile_rows(D);
  a.n_req = n_req;
  a.item_cap = plan.item_cap;
  a.part_cap = plan.part_cap;
  a.out = reinterpret_cast<uint16_t*>(out);
  a.o_part = reinterpret_cast<uint16_t*>(ws);
  a.ml_part = reinterpret_cast<float2*>(reinterpret_cast<char*>(ws) + plan.off_ml);
  a.n_part = plan.part_cap > 0 ? reinterpret_cast<int64_t*>(reinterpret_cast<char*>(ws) + plan.off_np) : nullptr;
  const dim3 grid(static_cast<unsigned>(plan.grid));
  if (D == 256)
    attend_mfma16_kernel<256, E8><<<grid, att_threads(256), 0, s>>>(a);
  else
    attend_mfma16_kernel<128, E8><<<grid, att_threads(128), 0, s>>>(a);
  DG_LAUNCHED();
  if (plan.part_cap > 0) {
    const dim3 mgrid(static_cast<unsigned>(std::min<int64_t>(rows, 2048)),
                     static_cast<unsigned>(cdiv(static_cast<int64_t>(Hq) * D, 1024)));
    if (D == 256)
      attend_merge_kernel<256><<<mgrid, 256, 0, s>>>(a);
    else
      attend_merge_kernel<128><<<mgrid, 256, 0, s>>>(a);
    DG_LAUNCHED();
  }
  return DG_OK;
}

bool power_of_two(float x) {
  if (!(x > 0.f) || !(x < INFINITY)) return false;
  int e;
  return std::frexp(x, &e) == 0.5f;
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" size_t dg_canvas_attention_ws_bytes(int32_t n_req, int32_t rows, int32_t max_rows_per_req,
                                               int32_t max_keys_per_req, int32_t Hq, int32_t Hkv, int32_t D,
                                               int32_t dtype) {
  if (n_req <= 0 || rows <= 0 || max_rows_per_req <= 0 || max_keys_per_req <= 0 || Hq <= 0 || Hkv <= 0 ||
      Hq % Hkv != 0)
    return 0;
  return plan_attention(n_req, rows, max_rows_per_req, max_keys_per_req, Hq, Hkv, D, dtype).bytes;
}

extern "C" dg_status dg_canvas_attention(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                                         int32_t n_pages, const int32_t* page_table, int32_t page_table_len,
                                         const dg_split* splits, int32_t n_req, int32_t rows,
                                         int32_t max_rows_per_req, int32_t max_keys_per_req, int32_t Hq,
                                         int32_t Hkv, int32_t D, int32_t page_size, float scale, int32_t dtype,
                                         void* out, void* ws, size_t ws_bytes, dg_stream_t stream) {
  DG_ARG(q && k && v && k_cache && v_cache && page_table && splits && out);
  DG_ARG(n_pages > 0 && page_table_len > 0 && n_req > 0 && rows > 0 && max_rows_per_req > 0 &&
         max_keys_per_req > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0);
  DG_ARG(n_req <= 65535 && max_rows_per_req <= (1 << 20) && Hq <= 65535);
  DG_UNSUP(dtype == DG_BF16 || dtype == DG_F32);
  DG_UNSUP(page_size == 16);
  DG_UNSUP(D == 32 || D == 64 || D == 128 || D == 256);
  const AttPlan plan = plan_attention(n_req, rows, max_rows_per_req, max_keys_per_req, Hq, Hkv, D, dtype);
  // a request's splits (at most kMergeSplits, each with its keys plus one alignment block) must fit
  // the staged page list
  DG_UNSUP(!plan.mfma || (plan.fits && cdiv(max_keys_per_req, kAttKeys) <=
                                             static_cast<int64_t>(kMergeSplits) * kAttMaxSplitBlocks));
  DG_REQUIRE(plan.bytes == 0 || (ws != nullptr && ws_bytes >= plan.bytes), DG_E_WORKSPACE);
  hipStream_t s = as_stream(stream);
  const bool bf = dtype == DG_BF16;
  if (!plan.mfma) {
    const dim3 grid(max_rows_per_req, n_req);
    if (bf)
      append_kv_kernel<true><<<grid, 256, 0, s>>>(k, v, k_cache, v_cache, n_pages, page_table, page_table_len,
                                                  splits, rows, Hkv, D, page_size);
    else
      append_kv_kernel<false><<<grid, 256, 0, s>>>(k, v, k_cache, v_cache, n_pages, page_table, page_table_len,
                                                   splits, rows, Hkv, D, page_size);
    DG_LAUNCHED();
  }
  if (plan.mfma) {
    AttArgs a{};
    a.k_cache = reinterpret_cast<const uint16_t*>(k_cache);
    a.v_cache = reinterpret_cast<const uint16_t*>(v_cache);
    a.k_cache_w = reinterpret_cast<uint16_t*>(k_cache);
    a.v_cache_w = reinterpret_cast<uint16_t*>(v_cache);
    return launch_mfma<false>(a, plan, q, k, v, n_pages, page_table, page_table_len, splits, n_req, rows, Hq, Hkv, D,
                              page_size, scale, out, ws, s);
  }
#define DG_ATT(BF, DD)                                                                                        \
  launch_attend_wave<BF, DD>(q, k, v, k_cache, v_cache, n_pages, page_table, page_table_len, splits, n_req, rows, \
                             max_rows_per_req, Hq, Hkv, page_size, scale, out, s)
  if (bf) {
    switch (D) {
      case 32: DG_ATT(true, 32); break;
      case 64: DG_ATT(true, 64); break;
      case 128: DG_ATT(true, 128); break;
      default: DG_ATT(true, 256); break;
    }
  } else {
    switch (D) {
      case 32: DG_ATT(false, 32); break;
      case 64: DG_ATT(false, 64); break;
      case 128: DG_ATT(false, 128); break;
      default: DG_ATT(false, 256); break;
    }
  }
#undef DG_ATT
  DG_LAUNCHED();
  (void)max_keys_per_req;
  return DG_OK;
}

extern "C" dg_status dg_canvas_attention_e4m3(const void* q, const void* k, const void* v, uint8_t* k_cache8,
                                              uint8_t* v_cache8, float k_scale, float v_scale, int32_t n_pages,
                                              const int32_t* page_table, int32_t page_table_len,
                                              const dg_split* splits, int32_t n_req, int32_t rows,
                                              int32_t max_rows_per_req, int32_t max_keys_per_req, int32_t Hq,
                                              int32_t Hkv, int32_t D, int32_t page_size, float scale, void* out,
                                              void* ws, size_t ws_bytes, dg_stream_t stream) {
  DG_ARG(q && k && v && k_cache8 && v_cache8 && page_table && splits && out);
  DG_ARG(n_pages > 0 && page_table_len > 0 && n_req > 0 && rows > 0 && max_rows_per_req > 0 &&
         max_keys_per_req > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0);
  DG_ARG(n_req <= 65535 && max_rows_per_req <= (1 << 20) && Hq <= 65535);
  DG_UNSUP(power_of_two(k_scale) && power_of_two(v_scale));
  DG_UNSUP(page_size == 16);
  DG_UNSUP(D == 128 || D == 256);
  const AttPlan plan = plan_attention(n_req, rows, max_rows_per_req, max_keys_per_req, Hq, Hkv, D, DG_BF16);
  DG_UNSUP(plan.fits && cdiv(max_keys_per_req, kAttKeys) <= static_cast<int64_t>(kMergeSplits) * kAttMaxSplitBlocks);
  DG_REQUIRE(plan.bytes == 0 || (ws != nullptr && ws_bytes >= plan.bytes), DG_E_WORKSPACE);
  AttArgs a{};
  a.k_cache8 = k_cache8;
  a.v_cache8 = v_cache8;
  a.k_cache8_w = k_cache8;
  a.v_cache8_w = v_cache8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return launch_mfma<true>(a, plan, q, k, v, n_pages, page_table, page_table_len, splits, n_req, rows, Hq, Hkv, D,
                           page_size, scale, out, ws, as_stream(stream));
}
