// bf16 MFMA flash attention for dg_canvas_attention (head_dim 128 / 256).
//
// Work item: (request, KV head, tile of 128 packed query rows, KV split).  A
// packed query row is m = j * G + g (row j of the request, query head
// hk * G + g of the KV group), so the G query heads that share a KV head share
// every K/V tile.  Eight wave64s own 16 packed rows each (two waves per SIMD).
//
// K and V blocks go global -> LDS by direct copies (global_load_lds_dwordx4, one 16-byte chunk per
// lane, no staging registers; each copy reads whole key rows) into the same XOR-swizzled row-major
// layout, prefetched one block ahead by waves 0 - 3 (one 16-key page each, a scalar base per page
// when the page is whole).  The V operand of the PV product needs several keys at one d per lane:
// it is read with gfx950's transposing LDS load (ds_read_b64_tr_b16), which gives each lane of a
// 16-lane group one column of the 4 rows x 16 columns its lanes address.  Every operand read address
// is a per-lane base XORed with a constant plus an immediate offset.  The reads run ahead of their MFMAs in hand-pipelined
// rings (at D = 256: K two steps, V four fragments), since the kernel is bound by LDS latency, not
// by MFMA or LDS bandwidth.
//
// Per 64-key block a wave computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16
// (A = K from LDS, B = Q preloaded in registers): each lane holds 16 scores of
// one query row and the row's other 48 scores sit in the three lanes 16, 32 and
// 48 away, so the online softmax is in-lane plus two lane-group swaps.  The
// probabilities stay in registers as the B operand of O^T = V^T P^T; the key
// order inside each 32-key MFMA step is permuted consistently on both operands
// to match the accumulator layout.  O^T accumulates in fp32 (the lanes of a row
// share its softmax state, so the rescale is in-lane).  The softmax reference
// (running max) moves only when a block's maximum exceeds it by more than 2^8,
// so the rescale of O is rare; probabilities are then at most 2^8, which bf16
// and the fp32 sums hold as well as values below 1.  The final division uses
// the same reference, so the result is the same softmax.
//
// Visibility (per request): key index kk (prefix positions first, then causal
// rows, then canvas rows) is visible to causal row j iff kk <= cached + j, to a
// canvas row always, both cut to the window when the split has one.  Keys at or
// past `cached` are read from the k / v inputs (the causal rows' K/V are exactly
// the values this launch appends to the pages), so the append has no ordering
// constraint and the same kernel does it: the split-0 workgroup of each row
// tile writes its causal rows' K/V for its KV head.  Blocks outside the tile's
// key range are never loaded (tiles holding only masked entries are skipped);
// only blocks that are not fully visible to every row of a wave evaluate the
// mask.  With several KV splits each split writes its output normalised by its
// own sum (bf16) with (reference max, sum), and a merge kernel combines them
// with log-sum-exp weights.
//
// Batch invariance: how a request's keys are cut into splits depends on that
// request's own descriptor only (its rows, cached keys and window), never on
// the other requests of the launch, so a request's output is bitwise the same
// alone or in any batch.  Work items are numbered request by request; each
// workgroup recomputes the per-request item counts of the launch (a wave-wide
// prefix sum over the descriptors) to find its item, so the grid holds no
// empty items beyond a rounding to the XCD count.
#pragma once
#include "dg_device.hpp"

namespace dg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Packed query rows per workgroup (16 per wave): 128 at head_dim 256; 64 at head_dim 128, where the
// blocks of a 64-row tile (68 KB of LDS) let two workgroups share a CU and a request with 64 packed
// rows per KV head (16 rows x 4 query heads of a group) fills its tiles instead of half of them.
// Fixed by the head size, so a request's tiling depends on its own shape only.
__host__ __device__ constexpr int att_tile_rows(int D) { return D > 128 ? 128 : 64; }
constexpr int kAttKeys = 64;    // keys per block
constexpr int kAttMaxPages = 1024;  // page ids of one split staged in LDS (16K keys)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMergeSplits = 16;     // the most splits of one request
// work items a request alone is split into at most: one per CU for 128-row tiles, two for 64-row tiles
__host__ __device__ constexpr int att_target_items(int tile_rows) { return 256 * 128 / tile_rows; }
constexpr int kAttMaxSplitBlocks = kAttMaxPages / 4 - 1;  // a split's pages plus one block fit the staged list

// Keys a request's rows see together: the whole request, or at most its rows plus two windows.
__host__ __device__ inline int64_t att_span(int64_t cached, int64_t nr, int64_t window) {
  const int64_t n_total = cached + nr;
  return window > 0 ? (n_total < nr + 2 * window ? n_total : nr + 2 * window) : n_total;
}

// KV splits of a request with qt row tiles per KV head and nb 64-key blocks (its own shape only):
// enough splits that the request alone gives about `target` work items, at least 4 blocks per
// split, at most kMergeSplits, and few enough blocks per split for the staged page list.
template <typename I>
__host__ __device__ inline I att_nsplit(I qt, I nb, I Hkv, I target) {
  // ceil(target / (Hkv qt)), without forming a product that could overflow
  const I want = (qt >= target || Hkv >= target || Hkv * qt >= target) ? I(1) : (target + Hkv * qt - 1) / (Hkv * qt);
  I n = nb / 4;
  n = n < want ? n : want;
  n = n < kMergeSplits ? n : I(kMergeSplits);
  const I need = (nb + kAttMaxSplitBlocks - 1) / kAttMaxSplitBlocks;
  n = n > need ? n : need;
  n = n < 1 ? I(1) : n;
  return n < kMergeSplits ? n : I(kMergeSplits);
}

struct AttArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  uint16_t* k_cache_w;  // the same pages, written by the append of the causal rows
  uint16_t* v_cache_w;
  int32_t n_pages;
  const int32_t* page_table;
  int32_t page_table_len;
  const dg_split* splits;
  int32_t n_req, rows, Hq, Hkv, G, page_size;
  int32_t tile_rows;    // packed query rows per work item: att_tile_rows(D)
  float scale_log2;     // scale * log2(e)
  int64_t item_cap;     // work items the grid holds (the host bound)
  int64_t part_cap;     // split rows the workspace holds
  uint16_t* out;        // [rows][Hq][D] bf16 (requests with one split write here directly)
  uint16_t* o_part;     // [split rows][Hq][D] bf16: split s of a split request, its row j at part_off + s nr + j,
                        // the split's output normalised by its own l
  float2* ml_part;      // [split rows][Hq] (reference max in log2 units, l)
  int64_t* n_part;      // split rows of the launch, written by the attention kernel for the merge (with ml_part)
  // E4M3 cache (attend_mfma16_kernel<D, true>): codes in place of k_cache / v_cache, values scale * code
  const uint8_t* k_cache8;
  const uint8_t* v_cache8;
  uint8_t* k_cache8_w;
  uint8_t* v_cache8_w;
  float k_scale, v_scale;  // powers of two
};

template <int D, bool E8>
struct AttSmem;
// every K / V block buffer starts at a multiple of 1024 bytes of the struct (operand read addressing)
static_assert(kAttKeys * 128 * 2 % 1024 == 0, "block buffers 1024-aligned");
template <int D>
struct AttSmem<D, false> {
  uint16_t K[2][kAttKeys * D];
  uint16_t V[2][kAttKeys * D];
  int32_t pages[kAttMaxPages];
};
// E4M3 cache: the codes of a block's cached keys land in S (K codes, then V codes, D bytes per key)
// and are converted into the bf16 block; page ids are read from the table (no room to stage them).
template <int D>
struct AttSmem<D, true> {
  uint16_t K[2][kAttKeys * D];
  uint16_t V[2][kAttKeys * D];
  uint8_t S[2 * kAttKeys * D];
};

// K and V in LDS: chunk c (8 bf16) of key r of the block sits in 16-byte slot r * (D / 8) + (c ^ sw(r)),
// sw(r) = r mod 16.  A K operand read has 16 consecutive keys ask for one chunk per 16-lane group, and
// a transposing V read has 4 consecutive keys ask for 32 bytes each: the XOR puts them in distinct
// slots of a 256-byte bank row.  (The bank-conflict counter reads a third of the LDS cycles for this
// kernel with this swizzle and with two others that spread the reads further; the time does not
// change with it either.)
DG_DEV int att_sw(int r) { return r & 15; }
template <int D>
DG_DEV int att_kslot(int r, int c) {
  return r * (D / 8) + (c ^ att_sw(r));
}

// Keys [x, y) visible to row j of a request (key positions: the cache, then the canvas rows; row j
// sits at position cached + j).  Causal rows see up to themselves, canvas rows every key of the
// request; a window W > 0 keeps positions within W before the row, and for a canvas row also
// within W after it (DiffusionGemma/vLLM page, section on symmetric sliding-window attention).
DG_DEV int2 att_row_keys(const dg_split& sp, int j) {
  const int n_total = sp.cached + sp.n_causal + sp.n_canvas;
  const int p = sp.cached + j;
  const bool causal = j < sp.n_causal;
  const int w = sp.window;
  int lo = 0, hi = causal ? p + 1 : n_total;
  if (w > 0) {
    lo = max(0, p - w);
    if (!causal) hi = min(hi, p + w + 1);
  }
  return make_int2(lo, hi);
}

// ---------------------------------------------------------------- per-request plan and work items
// A request's plan from its own descriptor: rows nr (clamped to the launch), row tiles qt of
// a.tile_rows packed rows per KV head, splits ns and keys per split sk (a multiple of kAttKeys).  A
// request without rows, or whose key span is beyond what kMergeSplits staged splits hold, has no
// work (ns = 0): a bad descriptor yields a wrong result, never an out-of-range access.
struct AttReqPlan {
  int32_t nr, qt, ns, sk;
};

DG_DEV AttReqPlan att_req_plan(const AttArgs& a, const dg_split& sp) {
  AttReqPlan p{0, 0, 0, kAttKeys};
  const int32_t nr = min(static_cast<int32_t>(min(static_cast<int64_t>(max(sp.n_causal, 0)) + max(sp.n_canvas, 0),
                                                  static_cast<int64_t>(a.rows))), a.rows);
  const int64_t nb64 = (att_span(max(sp.cached, 0), nr, sp.window) + kAttKeys - 1) / kAttKeys;
  const int64_t qt64 = (static_cast<int64_t>(nr) * a.G + a.tile_rows - 1) / a.tile_rows;
  if (nr == 0 || nb64 > kMergeSplits * kAttMaxSplitBlocks || qt64 > (1 << 24)) return p;
  const int32_t nb = static_cast<int32_t>(nb64);
  p.nr = nr;
  p.qt = static_cast<int32_t>(qt64);
  const int32_t ns = att_nsplit<int32_t>(p.qt, nb, a.Hkv, att_target_items(a.tile_rows));
  p.sk = (nb + ns - 1) / ns * kAttKeys;
  p.ns = (nb * kAttKeys + p.sk - 1) / p.sk;
  return p;
}

DG_DEV int64_t wave_incl_scan(int64_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// Work items of request r: its splits x KV heads x row tiles, item (s Hkv + hk) qt + qtile; split
// rows (partials) of a split request: ns nr.  Both numbered request by request.
DG_DEV void att_req_counts(const AttArgs& a, int r, AttReqPlan& p, int64_t& items, int64_t& part) {
  items = part = 0;
  p = AttReqPlan{0, 0, 0, kAttKeys};
  if (r < a.n_req) {
    p = att_req_plan(a, a.splits[r]);
    items = static_cast<int64_t>(p.ns) * a.Hkv * p.qt;
    part = p.ns > 1 ? static_cast<int64_t>(p.ns) * p.nr : 0;
  }
}

struct AttItem {
  int32_t req, split, hk, qtile;
  AttReqPlan p;
  int64_t part_off;  // first split row of the request (split requests)
};

// Launch totals (every lane of the calling wave gets them); false when they exceed what the grid
// or the workspace holds (descriptors inconsistent with the host bounds: nothing is done).
DG_DEV bool att_totals(const AttArgs& a, int64_t& n_items, int64_t& np) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t ni = 0;
  np = 0;
  for (int r0 = 0; r0 < a.n_req; r0 += kWave) {
    AttReqPlan p;
    int64_t items, part;
    att_req_counts(a, r0 + lane, p, items, part);
    ni += __shfl(wave_incl_scan(items), kWave - 1, kWave);
    np += __shfl(wave_incl_scan(part), kWave - 1, kWave);
  }
  n_items = ni;
  return ni <= a.item_cap && np <= a.part_cap;
}

// The request of item t among the 64 requests from r0 (per lane: its request's plan p, its items and
// the exclusive scans of items and parts), or false when none of them holds it.
DG_DEV bool att_pick(const AttArgs& a, int64_t t, int r0, const AttReqPlan& p, int64_t items, int64_t first,
                     int64_t part_first, AttItem& it) {
  const uint64_t own = __ballot(items > 0 && t >= first && t < first + items);
  if (!own) return false;
  const int src = __ffsll(static_cast<unsigned long long>(own)) - 1;
  it.req = r0 + src;
  it.p = AttReqPlan{__shfl(p.nr, src, kWave), __shfl(p.qt, src, kWave), __shfl(p.ns, src, kWave),
                    __shfl(p.sk, src, kWave)};
  it.part_off = __shfl(part_first, src, kWave);
  // local < the request's items <= item_cap < 2^31
  const int32_t local = static_cast<int32_t>(t - __shfl(first, src, kWave));
  it.qtile = local % it.p.qt;
  const int32_t rest = local / it.p.qt;
  it.hk = rest % a.Hkv;
  it.split = rest / a.Hkv;
  return true;
}

// Item t (< the launch's item total) -> its request, split, KV head and row tile.
DG_DEV AttItem att_find(const AttArgs& a, int64_t t) {
  const int lane = threadIdx.x & (kWave - 1);
  AttItem it{0, 0, 0, 0, AttReqPlan{0, 0, 0, kAttKeys}, 0};
  int64_t base_i = 0, base_p = 0;
  for (int r0 = 0; r0 < a.n_req; r0 += kWave) {
    AttReqPlan p;
    int64_t items, part;
    att_req_counts(a, r0 + lane, p, items, part);
    const int64_t inc_i = wave_incl_scan(items), inc_p = wave_incl_scan(part);
    if (att_pick(a, t, r0, p, items, base_i + inc_i - items, base_p + inc_p - part, it)) return it;
    base_i += __shfl(inc_i, kWave - 1, kWave);
    base_p += __shfl(inc_p, kWave - 1, kWave);
  }
  return it;
}

// Key kk (kb <= kk < kb + 64) of a request: prefix positions (kk < cached) live in the page of
// their 16-key group, whose id is one of the block's four staged ids `pq`; the causal and canvas
// keys are rows row0 + kk - cached of k / v.  Both candidates are formed and one is selected, so
// the address math has no branches and no memory access.
template <int D>
DG_DEV const uint16_t* att_row(const AttArgs& a, const dg_split& sp, int4 pq, int kb, int hk, int kk, bool is_v) {
  const int g = (kk - kb) >> 4;
  int page = g == 0 ? pq.x : (g == 1 ? pq.y : (g == 2 ? pq.z : pq.w));
  page = min(max(page, 0), a.n_pages - 1);
  const int64_t cache_off = ((static_cast<int64_t>(page) * a.Hkv + hk) * 16 + (kk & 15)) * D;
  const int64_t row = min(max(sp.row0 + max(kk - sp.cached, 0), 0), a.rows - 1);  // clamped: cannot fault
  const int64_t new_off = (row * a.Hkv + hk) * D;
  const uint16_t* cache = is_v ? a.v_cache : a.k_cache;
  const uint16_t* fresh = is_v ? a.v : a.k;
  return kk < sp.cached ? cache + cache_off : fresh + new_off;
}

// Keys at or past k_end (the split's last visible key + 1) are masked for every row of the tile:
// they re-read the last visible key (whose page is staged), so their K and V are finite and their
// probability is 0.
//
// Copy q fills slots 64 q .. 64 q + 63, i.e. the 64 / (D / 8) keys q * 64 / (D / 8) ...; lane l
// fetches chunk (l % (D / 8)) ^ sw(r) of its key r, so each copy reads whole key rows.
// Copies of the bf16 blocks are issued by waves 0 - 3 only: wave w fills keys 16 w .. 16 w + 15 of a
// block, one whole page of the cache.
constexpr int kAttCopyWaves = 4;

// One tensor (K or V) of the block at kb into dst, issued by copying wave w (0 - 3); pq holds the
// physical ids of the block's four 16-key pages (in range; only used for keys below `cached`).  When
// its page holds only cached keys below k_end, or only fresh rows inside the launch's rows, the
// copies take a scalar base and the precomputed per-lane offsets.
template <int D>
DG_DEV void att_load(const AttArgs& a, const dg_split& sp, int4 pq, int hk, int kb, int k_end, bool is_v,
                     uint16_t* dst) {
  constexpr int kChunks = D / 8;
  constexpr int kKeysPerCopy = kWave / kChunks;
  constexpr int kPerWave = kChunks / kAttCopyWaves;  // copies per wave of one tensor and block
  static_assert(kAttKeys / kAttCopyWaves == 16, "a copying wave fills one 16-key page");
  const int lane = threadIdx.x & (kWave - 1);
  // copy i of the wave: key lk = i keys-per-copy + lane / chunks of its page, swizzled chunk c; its
  // lane offset lk D 2 + 16 c bytes from the page's head
  auto lane_off = [&](int i) {
    const int lk = i * kKeysPerCopy + lane / kChunks;
    return static_cast<uint32_t>(lk * D * 2 + 16 * ((lane % kChunks) ^ att_sw(lk)));
  };
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform: M0 is scalar
  {
    const int k0 = __builtin_amdgcn_readfirstlane(kb) + 16 * wave;
    const int cached = __builtin_amdgcn_readfirstlane(sp.cached);
    const int kend = __builtin_amdgcn_readfirstlane(k_end);
    const int hks = __builtin_amdgcn_readfirstlane(hk);
    if (k0 + 15 < min(cached, kend)) {
      const int64_t pid = __builtin_amdgcn_readfirstlane(wave == 0 ? pq.x : (wave == 1 ? pq.y : (wave == 2 ? pq.z : pq.w)));
      const int64_t head = (pid * a.Hkv + hks) * 16 * D * 2;
      const char* base = reinterpret_cast<const char*>(is_v ? a.v_cache : a.k_cache) + head;
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int q = wave * kPerWave + i;
        lds_copy16<false>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst + kWave * 8 * q)), base, lane_off(i));
      }
      return;
    }
    const int64_t rb = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(sp.row0)) + (k0 - cached);
    if (k0 >= cached && k0 + 15 < kend && rb >= 0 && rb + 15 < a.rows) {
      // key lk of the page is row rb + lk: its lk D 2 bytes of the page offset become lk Hkv D 2
      const int64_t head = (rb * a.Hkv + hks) * D * 2;
      const char* base = reinterpret_cast<const char*>(is_v ? a.v : a.k) + head;
      const uint32_t row_extra = static_cast<uint32_t>((lane / kChunks) * (a.Hkv - 1) * D * 2);
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int q = wave * kPerWave + i;
        const int64_t step = static_cast<int64_t>(i) * kKeysPerCopy * (a.Hkv - 1) * D * 2;
        lds_copy16<false>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst + kWave * 8 * q)), base + step,
                          lane_off(i) + row_extra);
      }
      return;
    }
  }
  // pages straddling the cache end or k_end (or rows outside the launch): per-lane addresses
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int q = wave * kPerWave + i;
    const int r = q * kKeysPerCopy + lane / kChunks;
    const int c = (lane % kChunks) ^ att_sw(r);
    const int kk = min(kb + r, k_end - 1);
    const uint16_t* src = att_row<D>(a, sp, pq, kb, hk, kk, is_v) + 8 * c;
    lds_copy16(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst + kWave * 8 * q)), src);
  }
}

// E4M3 cache, block at kb: the codes of its cached keys into S (row r of K at S + r D, of V at
// S + (64 + r) D; one 1-KB copy = 1024 / D keys), its fresh keys (>= cached) as bf16 rows into the
// block's slots as in att_load.  A block holding both kinds gets both sets of copies; a copy's lanes
// whose key is of the other kind fetch a valid key of the right kind (the last cached key, the first
// fresh row), which the conversion then ignores.  Keys past k_end re-read the last visible key.
template <int D, int NT>
DG_DEV void att_load8(const AttArgs& a, const dg_split& sp, int hk, int kb, int k_end, uint8_t* s8, uint16_t* kdst,
                      uint16_t* vdst) {
  constexpr int kChunks = D / 8;
  constexpr int kKeysPerCopy = kWave / kChunks;
  constexpr int kPerWave = kChunks / (NT / kWave);
  constexpr int kKeysPerCopy8 = 1024 / D;
  constexpr int kPerWave8 = kAttKeys / kKeysPerCopy8 / (NT / kWave);
  static_assert(kPerWave8 >= 1, "one code copy per wave at least");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int kl = min(kb + kAttKeys - 1, k_end - 1);
  if (kb < sp.cached) {
#pragma unroll
    for (int i = 0; i < kPerWave8; ++i) {
      const int q = wave * kPerWave8 + i;
      const int r = q * kKeysPerCopy8 + lane / (D / 16);
      const int kk = min(min(kb + r, k_end - 1), sp.cached - 1);
      const int ti = min(max(sp.page0 + kk / 16, 0), a.page_table_len - 1);
      const int64_t page = min(max(a.page_table[ti], 0), a.n_pages - 1);
      const int64_t off = ((page * a.Hkv + hk) * 16 + (kk & 15)) * D + 16 * (lane % (D / 16));
      const uint32_t klds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s8 + 1024 * q));
      const uint32_t vlds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s8 + kAttKeys * D + 1024 * q));
      const uint8_t* ksrc = a.k_cache8 + off;
      const uint8_t* vsrc = a.v_cache8 + off;
      lds_copy16(klds, ksrc);
      lds_copy16(vlds, vsrc);
    }
  }
  if (kl >= sp.cached) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int q = wave * kPerWave + i;
      const int r = q * kKeysPerCopy + lane / kChunks;
      const int c = (lane % kChunks) ^ att_sw(r);
      const int kk = max(min(kb + r, k_end - 1), sp.cached);
      const int64_t row = min(max(sp.row0 + kk - sp.cached, 0), a.rows - 1);
      const int64_t off = (row * a.Hkv + hk) * D + 8 * c;
      const uint32_t klds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(kdst + kWave * 8 * q));
      const uint32_t vlds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(vdst + kWave * 8 * q));
      const uint16_t* ksrc = a.k + off;
      const uint16_t* vsrc = a.v + off;
      lds_copy16(klds, ksrc);
      lds_copy16(vlds, vsrc);
    }
  }
}

// The cached keys of the block at kb: codes in S -> bf16 (value * scale, exact for a power-of-two
// scale) in the block's swizzled slots.  Each thread converts 8-code chunks u = tid + 256 j.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
template <int D, int NT>
DG_DEV void att_convert8(const AttArgs& a, const dg_split& sp, int kb, int k_end, const uint8_t* s8, uint16_t* kdst,
                         uint16_t* vdst) {
  constexpr int kChunks = D / 8;
#pragma unroll
  for (int j = 0; j < kAttKeys * kChunks / NT; ++j) {
    const int u = threadIdx.x + NT * j;
    const int r = u / kChunks, c = u % kChunks;
    if (min(kb + r, k_end - 1) >= sp.cached) continue;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const uint2 q = *reinterpret_cast<const uint2*>(s8 + (kv * kAttKeys + r) * D + 8 * c);
      const float sc = kv == 0 ? a.k_scale : a.v_scale;
      const bf16x2v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, sc, false);
      const bf16x2v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, sc, true);
      const bf16x2v p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, sc, false);
      const bf16x2v p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, sc, true);
      bf16x8 w;
      w[0] = p0[0]; w[1] = p0[1]; w[2] = p1[0]; w[3] = p1[1];
      w[4] = p2[0]; w[5] = p2[1]; w[6] = p3[0]; w[7] = p3[1];
      uint16_t* dst = kv == 0 ? kdst : vdst;
      *reinterpret_cast<bf16x8*>(dst + 8 * att_kslot<D>(r, c)) = w;
    }
  }
}

// Waits for every outstanding copy, so that after the next barrier K and V of the block are visible.
DG_DEV void att_wait() { __builtin_amdgcn_s_waitcnt(vmcnt_only(0)); }

typedef short short4v __attribute__((ext_vector_type(4)));

// Causal rows' K/V of one KV head into the pages at positions cached + j (16-byte chunks).
template <int D, int NT>
DG_DEV void att_append(const AttArgs& a, const dg_split& sp, int hk, int j0, int j1) {
  constexpr int kChunks = D / 8;
  const int n = (j1 - j0) * kChunks;
  for (int u = threadIdx.x; u < 2 * n; u += NT) {
    const bool is_v = u >= n;
    const int w = is_v ? u - n : u;
    const int j = j0 + w / kChunks, c = w % kChunks;
    if (sp.row0 + j < 0 || sp.row0 + j >= a.rows) continue;  // a descriptor outside the packed rows
    const int pos = sp.cached + j;
    const int ti = min(max(sp.page0 + pos / 16, 0), a.page_table_len - 1);
    const int64_t page = min(max(a.page_table[ti], 0), a.n_pages - 1);
    const int64_t src = ((static_cast<int64_t>(sp.row0) + j) * a.Hkv + hk) * D + 8 * c;
    const int64_t dst = ((page * a.Hkv + hk) * 16 + (pos & 15)) * D + 8 * c;
    const uint16_t* from = is_v ? a.v : a.k;
    uint16_t* to = is_v ? a.v_cache_w : a.k_cache_w;
    *reinterpret_cast<uint4*>(to + dst) = *reinterpret_cast<const uint4*>(from + src);
  }
}

// E4M3 cache: the causal rows' K/V quantised into the pages (x / scale, clamped to +-448, nearest
// even), 8 values per thread and step.
template <int D, int NT>
DG_DEV void att_append8(const AttArgs& a, const dg_split& sp, int hk, int j0, int j1) {
  constexpr int kChunks = D / 8;
  const int n = (j1 - j0) * kChunks;
  for (int u = threadIdx.x; u < 2 * n; u += NT) {
    const bool is_v = u >= n;
    const int w = is_v ? u - n : u;
    const int j = j0 + w / kChunks, c = w % kChunks;
    if (sp.row0 + j < 0 || sp.row0 + j >= a.rows) continue;  // a descriptor outside the packed rows
    const int pos = sp.cached + j;
    const int ti = min(max(sp.page0 + pos / 16, 0), a.page_table_len - 1);
    const int64_t page = min(max(a.page_table[ti], 0), a.n_pages - 1);
    const int64_t src = ((static_cast<int64_t>(sp.row0) + j) * a.Hkv + hk) * D + 8 * c;
    const int64_t dst = ((page * a.Hkv + hk) * 16 + (pos & 15)) * D + 8 * c;
    const uint4 x = *reinterpret_cast<const uint4*>((is_v ? a.v : a.k) + src);
    const float inv = 1.0f / (is_v ? a.v_scale : a.k_scale);
    auto q = [&](float f) { return fminf(fmaxf(f * inv, -448.f), 448.f); };
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(q(bf16_lo(x.x)), q(bf16_hi(x.x)), 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(q(bf16_lo(x.y)), q(bf16_hi(x.y)), lo, true);
    uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(q(bf16_lo(x.z)), q(bf16_hi(x.z)), 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(q(bf16_lo(x.w)), q(bf16_hi(x.w)), hi, true);
    *reinterpret_cast<uint2*>((is_v ? a.v_cache8_w : a.k_cache8_w) + dst) = make_uint2(lo, hi);
  }
}

// ---------------------------------------------------------------- the attention kernel
// Eight waves of 16 packed query rows (two waves per SIMD at up to 256 registers each, so one
// wave's softmax and reads overlap the other's MFMAs), on v_mfma_f32_16x16x32_bf16; each lane
// keeps its row's online-softmax state (max in log2 units, sum) and P stays in registers as the B
// operand of the PV product.  Operand layouts (lane l, group g = l / 16, t = l % 16):
//   S^T tile (16 keys x 16 rows) = K Q^T: A = K (key t, d 8 g .. 8 g + 7 of the 32-d step),
//     B = Q^T (row t, the same d), C: row t, keys 4 g .. 4 g + 3 of the tile;
//   O^T tile (16 d x 16 rows) += V^T P^T over a 32-key chunk: MFMA k-slots 8 g .. 8 g + 3 hold keys
//     4 g .. 4 g + 3 of the chunk's first 16-key tile and slots 8 g + 4 .. 8 g + 7 the same keys of
//     its second tile, which is exactly the P this lane holds (no exchange); the V^T operand for that
//     order is two transposing LDS reads (4 keys x 16 d each).
// A row's 64 scores of a block are spread over the four groups; its max and sum are combined with
// v_permlane16_swap / v_permlane32_swap (no LDS traffic).
// threads of a workgroup at head size D
__host__ __device__ constexpr int att_threads(int D) { return att_tile_rows(D) / 16 * kWave; }

DG_DEV float quad_group_max(float v) {
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = fmaxf(__int_as_float(r16[0]), __int_as_float(r16[1]));
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(r32[0]), __int_as_float(r32[1]));
}
DG_DEV float quad_group_sum(float v) {
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = __int_as_float(r16[0]) + __int_as_float(r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r32[0]) + __int_as_float(r32[1]);
}

// A operand of O^T += V^T P^T for a 16-d tile and a 32-key chunk (see the layout above): two
// transposing LDS reads at the lane's address p (its key row and column within the chunk) and 16 key
// rows further.
template <int C8>
DG_DEV bf16x8 att_vfrag16(const char* p) {
  typedef __attribute__((address_space(3))) short4v lds_short4v;
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p + 256 * C8));
  const short4v lohi[2] = {lo, hi};
  bf16x8 v;
  __builtin_memcpy(&v, lohi, sizeof(v));
  return v;
}

// Uniform description of a work item (row tile it.qtile of request it.req, KV head it.hk, key split
// it.split): its descriptor, first packed row and key range.  The tile sees keys [lo of its first
// row, hi of its last row) (both edges grow with the row); the splits cut that range from its first
// 64-aligned block, the last split also taking the one block the alignment can add beyond ns * sk.
struct AttRange {
  dg_split sp;
  int32_t m_tile0, k_begin, k_end, page_lo;
};

DG_DEV int32_t att_u(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
DG_DEV int64_t att_u64(int64_t v) {
  const uint64_t x = static_cast<uint64_t>(v);
  return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(att_u(static_cast<int32_t>(x >> 32)))) << 32) |
                              static_cast<uint32_t>(att_u(static_cast<int32_t>(x & 0xffffffffu))));
}

// The item's fields (equal in every lane after a pick) moved into scalar registers, so that the
// ranges and copy addresses derived from them stay scalar across the walk.
DG_DEV AttItem att_uniform(const AttItem& it) {
  AttItem u;
  u.req = att_u(it.req);
  u.split = att_u(it.split);
  u.hk = att_u(it.hk);
  u.qtile = att_u(it.qtile);
  u.p = AttReqPlan{att_u(it.p.nr), att_u(it.p.qt), att_u(it.p.ns), att_u(it.p.sk)};
  u.part_off = att_u64(it.part_off);
  return u;
}

template <int D>
DG_DEV AttRange att_range(const AttArgs& a, const AttItem& it) {
  constexpr int ROWS = att_tile_rows(D);
  AttRange r;
  r.sp = a.splits[it.req];
  r.m_tile0 = it.qtile * ROWS;
  const int j_last = min(it.p.nr - 1, (r.m_tile0 + ROWS - 1) / a.G);
  const int tile_lo = att_row_keys(r.sp, r.m_tile0 / a.G).x & ~(kAttKeys - 1);
  const int tile_hi = att_row_keys(r.sp, j_last).y;
  r.k_begin = tile_lo + it.split * it.p.sk;
  r.k_end = min(tile_hi, r.k_begin + it.p.sk + (it.split == it.p.ns - 1 ? kAttKeys : 0));
  r.page_lo = r.k_begin / 16;
  r.sp = dg_split{att_u(r.sp.row0), att_u(r.sp.cached), att_u(r.sp.n_causal), att_u(r.sp.n_canvas),
                  att_u(r.sp.page0), att_u(r.sp.window)};
  r.m_tile0 = att_u(r.m_tile0);
  r.k_begin = att_u(r.k_begin);
  r.k_end = att_u(r.k_end);
  r.page_lo = att_u(r.page_lo);
  return r;
}

// Physical ids of the four 16-key pages of the block at kb, read from the page table (indexes and ids
// clamped into range; ids past the request's pages are only used for keys >= cached).
DG_DEV int4 att_block_pages(const AttArgs& a, const dg_split& sp, int kb) {
  auto id = [&](int i) {
    const int ti = min(max(sp.page0 + kb / 16 + i, 0), a.page_table_len - 1);
    return min(max(a.page_table[ti], 0), a.n_pages - 1);
  };
  return make_int4(id(0), id(1), id(2), id(3));
}

// The workgroup's work items t, t + stride, ... below t_end (pick(t, item) names item t).  While an
// item runs its last block, the next item's first K/V block is copied into the free buffer, its Q
// fragments loaded (once the last score MFMAs have read this item's) and its page ids staged, so the
// next item starts without waiting for its own loads (bf16 cache; the E4M3 path loads each item's
// first block when it starts).  Every wave waits for all of its loads before an item's block loop:
// a Q load still in flight there would have the compiler wait on the vector-memory counter inside
// the loop, where that wait also covers the next block's copies and serialises them with the MFMAs.
template <int D, bool E8, class Pick>
DG_DEV void att_walk(const AttArgs& a, AttSmem<D, E8>& sm, int64_t t, int64_t t_end, int64_t stride, Pick pick) {
  constexpr int ROWS = att_tile_rows(D);
  constexpr int NT = att_threads(D);
  constexpr int kDSteps = D / 32;                // MFMA k-steps over D
  constexpr int kDTiles = D / 16;                // 16-wide output tiles over D
  constexpr float kRescaleAbove = 8.f;           // log2 units: move the reference when exceeded by 2^8
  constexpr int kPageRegs = kAttMaxPages / NT;   // staged page ids per thread

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int g = lane >> 4, t16 = lane & 15;
  const bool lead = __builtin_amdgcn_readfirstlane(wave) < kAttCopyWaves;  // the copying waves

  AttItem it{0, 0, 0, 0, AttReqPlan{0, 0, 0, kAttKeys}, 0};
  if (t >= t_end || !pick(t, it)) return;
  it = att_uniform(it);
  AttRange r = att_range<D>(a, it);

  // this lane's packed row of the current item: query row j, head h, keys [lo, hi)
  bool row_ok = false, row_in = false;
  int j = 0, h = 0, row = 0, lo = 0, hi = 0, wave_lo = 0, wave_hi = 0;
  auto set_rows = [&]() {
    const int m = r.m_tile0 + wave * 16 + t16;
    row_ok = m < it.p.nr * a.G;
    j = row_ok ? m / a.G : 0;
    h = it.hk * a.G + (row_ok ? m % a.G : 0);
    row = r.sp.row0 + j;
    row_in = row >= 0 && row < a.rows;
    const int2 rk = row_ok ? att_row_keys(r.sp, j) : make_int2(0, r.sp.cached + it.p.nr);
    lo = rk.x;
    hi = rk.y;
    int wh = hi, wl = lo;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      wh = min(wh, __shfl_xor(wh, o, kWave));
      wl = max(wl, __shfl_xor(wl, o, kWave));
    }
    wave_hi = __builtin_amdgcn_readfirstlane(wh);  // equal in every lane: the mask test branches
    wave_lo = __builtin_amdgcn_readfirstlane(wl);
  };

  // Q^T fragment (B operand) of item (qi, qr): row t16, d 32 s + 8 g .. + 7
  bf16x8 qf[kDSteps];
  auto load_q = [&](const AttItem& qi, const AttRange& qr) {
    const int m = qr.m_tile0 + wave * 16 + t16;
    const bool ok = m < qi.p.nr * a.G;
    const int jq = ok ? m / a.G : 0;
    const int hq = qi.hk * a.G + (ok ? m % a.G : 0);
    const int rc = min(max(qr.sp.row0 + jq, 0), a.rows - 1);
    const uint16_t* qrow = a.q + (static_cast<int64_t>(rc) * a.Hq + hq) * D;
#pragma unroll
    for (int s = 0; s < kDSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s + 8 * g);
  };

  // The physical page ids of a split's prefix positions, staged in LDS for the copies of its blocks
  // after the first (clamped into range): loaded into registers first and stored after other loads
  // have been issued.
  int32_t pv[kPageRegs];
  auto page_hi = [&](const AttRange& pr) {
    return min((min(pr.k_end, pr.sp.cached) + 15) / 16, pr.page_lo + kAttMaxPages);
  };
  auto load_pages = [&](const AttRange& pr) {
    const int ph = page_hi(pr);
#pragma unroll
    for (int i = 0; i < kPageRegs; ++i) {
      const int p = pr.page_lo + tid + i * NT;
      const int ti = min(max(pr.sp.page0 + p, 0), a.page_table_len - 1);
      pv[i] = p < ph ? min(max(a.page_table[ti], 0), a.n_pages - 1) : 0;
    }
  };
  auto store_pages = [&](auto& smem, const AttRange& pr) {
    const int ph = page_hi(pr);
#pragma unroll
    for (int i = 0; i < kPageRegs; ++i) {
      const int p = pr.page_lo + tid + i * NT;
      if (p < ph) smem.pages[p - pr.page_lo] = pv[i];
    }
  };
  // copying waves: K and V of the block at kb of item (ci, cr) into buffer b (pq: its page ids)
  auto copy_block = [&](const AttItem& ci, const AttRange& cr, int4 pq, int kb, int b) {
    att_load<D>(a, cr.sp, pq, ci.hk, kb, cr.k_end, false, sm.K[b]);
    att_load<D>(a, cr.sp, pq, ci.hk, kb, cr.k_end, true, sm.V[b]);
  };

  floatx4 o[kDTiles];
  float m_ref = -INFINITY, l_run = 0.f;

  // Per-lane parts of the operand read addresses (att_kslot's swizzle split into a lane part, a part
  // that is an immediate of each read and a part XORed in per read).  With Kb / Vb the byte offset of
  // the block buffer from the start of the shared struct (a multiple of 1024, so bits 5 - 9 of the
  // sums below come from the lane parts alone), the K read of tile tt and step s is at offset
  // ((Kb + klane) ^ 64 (s & 3)) + 16 kChunks (16 tt) + 256 (s >> 2), and the V read of d tile dt and
  // chunk ch (rows r and r + 16) at ((Vb + vlane) ^ 32 (dt & 7)) + 512 kChunks ch + 256 (dt >> 3)
  // (+ 256 kChunks).
  constexpr int kC8 = D / 8;
  uint32_t klane, vlane;
  {
    const int y = 4 * g + (t16 >> 2), e = (t16 & 3) >> 1;
    klane = t16 * kC8 * 16 + 64 * (t16 >> 2) + 16 * (g ^ (t16 & 3));
    vlane = 16 * kC8 * y + 32 * (y >> 1) + 16 * (e ^ (y & 1)) + 8 * (t16 & 1);
  }

  // The operand reads are software-pipelined by hand, with scheduling barriers between the steps so
  // that the reads stay ahead of the MFMAs that use them (left to itself the scheduler issues each
  // read just before its MFMA, which then waits for the whole LDS latency).
  //
  // S^T = K Q^T for the block in Kb: four 16-key tiles; the K fragments of step s + 2 are read while
  // the MFMAs of step s run (a ring of three steps).
  constexpr int kKRing = D > 128 ? 2 : 3;
  const char* smb = reinterpret_cast<const char*>(&sm);
  auto scores = [&](const uint16_t* Kbuf, floatx4 (&sc)[4]) {
    const uint32_t kw = static_cast<uint32_t>(reinterpret_cast<const char*>(Kbuf) - smb) + klane;
    auto kread = [&](int s, int tt) {
      return *reinterpret_cast<const bf16x8*>(smb + (kw ^ (64 * (s & 3))) + 256 * kC8 * tt + 256 * (s >> 2));
    };
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) sc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
    bf16x8 kf[kKRing][4];
#pragma unroll
    for (int s = 0; s < kKRing - 1 && s < kDSteps; ++s)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) kf[s][tt] = kread(s, tt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kDSteps; ++s) {
      if (s + kKRing - 1 < kDSteps) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) kf[(s + kKRing - 1) % kKRing][tt] = kread(s + kKRing - 1, tt);
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s % kKRing][tt], qf[s], sc[tt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Online softmax of the block at kb (element e of tile tt holds key 16 tt + 4 g + e of this lane's
  // row), then O^T += V^T P^T over its two 32-key chunks with V in Vb: 2 kDTiles steps (chunk, d tile),
  // the V fragments of step t + kVRing read while the MFMA of step t runs, the first ones before the
  // softmax.
  constexpr int kVSteps = 2 * kDTiles;
  constexpr int kVRing = D > 128 ? 4 : 8;
  constexpr int kVEarly = D > 128 ? 2 : 4;  // of which read before the softmax
  auto accumulate = [&](int kb, floatx4 (&sc)[4], const uint16_t* Vbuf) {
    const uint32_t vw = static_cast<uint32_t>(reinterpret_cast<const char*>(Vbuf) - smb) + vlane;
    auto vread = [&](int t) {
      const int c = t / kDTiles, dt = t % kDTiles;
      return att_vfrag16<kC8>(smb + (vw ^ (32 * (dt & 7))) + 512 * kC8 * c + 256 * (dt >> 3));
    };
    bf16x8 vf[kVRing];
#pragma unroll
    for (int t = 0; t < kVEarly; ++t) vf[t] = vread(t);
    __builtin_amdgcn_sched_barrier(0);
    if (kb + kAttKeys > wave_hi || kb < wave_lo) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kb + 16 * tt + 4 * g + e;
          sc[tt][e] = (key >= lo && key < hi) ? sc[tt][e] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[tt][e]);
    mx = quad_group_max(mx);
    const float mb = mx * a.scale_log2;
    const bool grow = mb > m_ref + kRescaleAbove;
    const bool rescale = grow && m_ref != -INFINITY;
    if (__any(rescale)) {
      const float alpha = rescale ? __builtin_amdgcn_exp2f(m_ref - mb) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[dt][e] *= alpha;
    }
    if (grow) m_ref = mb;
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float psum = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[tt][e], a.scale_log2, -m_use));
        psum += p;
        pf[tt >> 1][4 * (tt & 1) + e] = static_cast<__bf16>(p);
      }
    l_run += quad_group_sum(psum);
#pragma unroll
    for (int t = kVEarly; t < kVRing; ++t) vf[t] = vread(t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kVSteps; ++t) {
      const int c = t / kDTiles, dt = t % kDTiles;
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[t % kVRing], pf[c], o[dt], 0, 0, 0);
      if (t + kVRing < kVSteps) vf[t % kVRing] = vread(t + kVRing);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  int buf = 0;
  bool ready = false;  // the current item's Q, page ids and first block are in place
  floatx4 sc[4];
  for (;;) {
    set_rows();
    if (!ready) {
      if constexpr (!E8) {
        // page ids, the first block (its page ids from the table) and Q in flight together
        load_pages(r);
        if (lead && r.k_begin < r.k_end) copy_block(it, r, att_block_pages(a, r.sp, r.k_begin), r.k_begin, buf);
        load_q(it, r);
        store_pages(sm, r);
        att_wait();
        __syncthreads();
      } else {
        load_q(it, r);
        if (r.k_begin < r.k_end) {
          att_load8<D, NT>(a, r.sp, it.hk, r.k_begin, r.k_end, sm.S, sm.K[buf], sm.V[buf]);
          att_wait();
        }
        __syncthreads();
        if (r.k_begin < r.k_end && r.k_begin < r.sp.cached) {
          att_convert8<D, NT>(a, r.sp, r.k_begin, r.k_end, sm.S, sm.K[buf], sm.V[buf]);
          __syncthreads();
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    m_ref = -INFINITY;
    l_run = 0.f;

    bool have_next = false;
    AttItem it_n = it;
    AttRange r_n = r;
    auto find_next = [&]() {
      have_next = t + stride < t_end && pick(t + stride, it_n);
      if (have_next) {
        it_n = att_uniform(it_n);
        r_n = att_range<D>(a, it_n);
      }
    };
    if constexpr (!E8) {
      // the copying waves fetch the next block while every wave works on the current one
      int kb = r.k_begin;
      for (; kb + kAttKeys < r.k_end; kb += kAttKeys) {
        // (the block's four page ids from the staged list: kb - k_begin is a multiple of 64, so the
        // slot is 4-aligned; slots past the staged range are only used for keys >= cached)
        if (lead)
          copy_block(it, r, *reinterpret_cast<const int4*>(sm.pages + ((kb + kAttKeys) / 16 - r.page_lo)),
                     kb + kAttKeys, buf ^ 1);
        scores(sm.K[buf], sc);
        accumulate(kb, sc, sm.V[buf]);
        if (lead) att_wait();
        __syncthreads();
        buf ^= 1;
      }
      if (kb < r.k_end) {
        // the last block: its copy slot fetches the next item's first block instead
        if (lead) {
          find_next();
          if (have_next && r_n.k_begin < r_n.k_end)
            copy_block(it_n, r_n, att_block_pages(a, r_n.sp, r_n.k_begin), r_n.k_begin, buf ^ 1);
        }
        scores(sm.K[buf], sc);
        if (!lead) find_next();
        if (have_next) {
          load_pages(r_n);
          load_q(it_n, r_n);
        }
        accumulate(kb, sc, sm.V[buf]);
        if (have_next) store_pages(sm, r_n);
        att_wait();        // every wave: the next item's Q and page ids (and copies) complete
        __syncthreads();   // its first block and page list visible
        buf ^= 1;
      }
    } else {
      for (int kb = r.k_begin; kb < r.k_end; kb += kAttKeys) {
        const bool more = kb + kAttKeys < r.k_end;
        if (more) att_load8<D, NT>(a, r.sp, it.hk, kb + kAttKeys, r.k_end, sm.S, sm.K[buf ^ 1], sm.V[buf ^ 1]);
        scores(sm.K[buf], sc);
        accumulate(kb, sc, sm.V[buf]);
        if (more) att_wait();
        __syncthreads();
        if (more && kb + kAttKeys < r.sp.cached) {
          att_convert8<D, NT>(a, r.sp, kb + kAttKeys, r.k_end, sm.S, sm.K[buf ^ 1], sm.V[buf ^ 1]);
          __syncthreads();
        }
        buf ^= 1;
      }
    }

    if (row_ok && row_in) {
      // O^T tile dt: this lane holds d = 16 dt + 4 g + e (e = 0 .. 3) of its row
      const bool split_req = it.p.ns > 1;
      const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
      const int64_t ridx = split_req ? (it.part_off + static_cast<int64_t>(it.split) * it.p.nr + j) * a.Hq + h
                                     : static_cast<int64_t>(row) * a.Hq + h;
      uint16_t* orow = (split_req ? a.o_part : a.out) + ridx * D;
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt) {
        uint2 w;
        w.x = static_cast<uint32_t>(f32_to_bf16(o[dt][0] * inv)) | (static_cast<uint32_t>(f32_to_bf16(o[dt][1] * inv)) << 16);
        w.y = static_cast<uint32_t>(f32_to_bf16(o[dt][2] * inv)) | (static_cast<uint32_t>(f32_to_bf16(o[dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = w;
      }
      if (split_req && g == 0) a.ml_part[ridx] = make_float2(m_ref, l_run);
    }

    // append (after the output, whose registers it reuses): the split-0 workgroup writes the causal
    // rows whose first packed row is in its tile
    if (it.split == 0) {
      const int j0 = (r.m_tile0 + a.G - 1) / a.G;
      const int j1 = min(r.sp.n_causal, (r.m_tile0 + ROWS + a.G - 1) / a.G);
      if (j0 < j1) {
        if constexpr (E8)
          att_append8<D, NT>(a, r.sp, it.hk, j0, j1);
        else
          att_append<D, NT>(a, r.sp, it.hk, j0, j1);
      }
    }

    t += stride;
    if (have_next) {
      ready = r.k_begin < r.k_end;  // prefetched by this item's last block (an item without blocks has none)
      it = it_n;
      r = r_n;
      continue;
    }
    ready = false;
    if (t >= t_end || !pick(t, it)) break;
    it = att_uniform(it);
    r = att_range<D>(a, it);
  }
}

// XCD-aware order: the hardware deals workgroup b to XCD b % 8.  The launch's items are cut into 8
// contiguous ranges, one per XCD, and the workgroups of XCD x walk range x with a stride, so the row
// tiles that read the same K/V (same request, split and KV head, consecutive items) run on one XCD
// and share its L2.  Each workgroup first recomputes the launch totals from the descriptors.
template <int D, bool E8>
__global__ __launch_bounds__(att_threads(D), 2) void attend_mfma16_kernel(AttArgs a) {  // two waves per SIMD
  __shared__ __attribute__((aligned(1024))) AttSmem<D, E8> sm;
  // The plans and prefix sums of the first kGroups x 64 requests stay in registers, one request per
  // lane and group (launches of up to that many requests pick their items from registers; larger
  // ones rescan the descriptors per item).  Two groups at head size 128, where the registers allow
  // them (launches of 128 requests, as a batch of draft blocks, are common there); one at 256.
  constexpr int kGroups = D > 128 ? 1 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  AttReqPlan p0, p1;
  int64_t items0, part0, items1 = 0, part1 = 0;
  att_req_counts(a, lane, p0, items0, part0);
  const int64_t inc_i0 = wave_incl_scan(items0), inc_p0 = wave_incl_scan(part0);
  const int64_t tot_i0 = __shfl(inc_i0, kWave - 1, kWave), tot_p0 = __shfl(inc_p0, kWave - 1, kWave);
  int64_t inc_i1 = tot_i0, inc_p1 = tot_p0;
  if constexpr (kGroups > 1) {
    att_req_counts(a, kWave + lane, p1, items1, part1);
    inc_i1 = tot_i0 + wave_incl_scan(items1);
    inc_p1 = tot_p0 + wave_incl_scan(part1);
  }
  const bool one_pass = a.n_req <= kGroups * kWave;
  int64_t n_items, n_part;
  bool ok;
  if (one_pass) {
    n_items = __shfl(inc_i1, kWave - 1, kWave);
    n_part = __shfl(inc_p1, kWave - 1, kWave);
    ok = n_items <= a.item_cap && n_part <= a.part_cap;
  } else {
    ok = att_totals(a, n_items, n_part);
  }
  // the merge kernel has nothing to do when no request of the launch is split (or nothing is done)
  if (a.n_part != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *a.n_part = ok ? n_part : 0;
  if (!ok) return;
  const int64_t per_xcd = (n_items + 7) / 8;
  const int64_t lo = (blockIdx.x % 8) * per_xcd;
  const int64_t hi = min(n_items, lo + per_xcd);
  const int64_t stride = gridDim.x / 8;  // the grid is a multiple of 8
  // (the pick's answer and the walk's bounds are the same in every lane: kept in scalar registers, so
  // that the walk's control flow, and what it carries from item to item, stays scalar)
  auto pick = [&](int64_t ti, AttItem& it) -> bool {
    bool found;
    if (one_pass) {
      found = att_pick(a, ti, 0, p0, items0, inc_i0 - items0, inc_p0 - part0, it);
      if constexpr (kGroups > 1)
        found = found || att_pick(a, ti, kWave, p1, items1, inc_i1 - items1, inc_p1 - part1, it);
    } else {
      it = att_find(a, ti);
      found = it.p.ns != 0;  // not false for ti below the total
    }
    return att_u(found ? 1 : 0) != 0;
  };
  att_walk<D, E8>(a, sm, att_u64(lo + blockIdx.x / 8), att_u64(hi), att_u64(stride), pick);
}

// Combine the KV splits of a split request: out = sum_s c_s Ohat_s / sum_s c_s with
// c_s = 2^(m_s - M) l_s, M = max_s m_s and Ohat_s = O_s / l_s the split's normalised output (so
// sum_s c_s Ohat_s = sum_s 2^(m_s - M) O_s).  Grid (row stride, 1024-value slice of the row's Hq x D
// outputs): a workgroup walks rows blockIdx.x, + gridDim.x, ...; for each it finds the request
// owning the row and that request's first split row from the same per-request counts as the
// attention kernel (a block-wide prefix over the descriptors); rows of one-split requests (written
// by the attention kernel) and rows of no request are skipped, and the whole launch returns at once
// when the attention kernel counted no split rows.  Four consecutive d per thread, every split's
// loads issued before the sums.
template <int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(AttArgs a) {
  if (*a.n_part == 0) return;  // no split request in this launch
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  __shared__ int64_t s_wave[4];
  __shared__ int64_t s_off;
  __shared__ int32_t s_ns, s_nr, s_row0;
  const int64_t e = static_cast<int64_t>(blockIdx.y) * 1024 + 4 * tid;
  const bool has_e = e < static_cast<int64_t>(a.Hq) * D;
  const int h = has_e ? static_cast<int>(e / D) : 0, d = has_e ? static_cast<int>(e - static_cast<int64_t>(h) * D) : 0;
  for (int row = blockIdx.x; row < a.rows; row += gridDim.x) {
    if (tid == 0) s_ns = 0;
    int64_t base = 0;
    for (int r0 = 0; r0 < a.n_req; r0 += 256) {
      AttReqPlan p;
      int64_t items, part;
      att_req_counts(a, r0 + tid, p, items, part);
      const int32_t row0 = r0 + tid < a.n_req ? a.splits[r0 + tid].row0 : 0;
      const int64_t inc = wave_incl_scan(part);
      if (lane == kWave - 1) s_wave[wave] = inc;
      __syncthreads();
      int64_t before = base;
      for (int w = 0; w < wave; ++w) before += s_wave[w];
      if (part > 0 && row >= row0 && row < row0 + p.nr) {
        s_off = before + inc - part;
        s_ns = p.ns;
        s_nr = p.nr;
        s_row0 = row0;
      }
      base += s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
      __syncthreads();
    }
    const int32_t ns = s_ns;
    const int64_t first = s_off + (row - s_row0);  // split row of split 0
    const int32_t nr = s_nr;
    __syncthreads();  // the shared values are read before the next row resets them
    if (ns < 2 || base > a.part_cap || !has_e) continue;  // block-uniform except has_e (no barrier follows)
    float2 ml[kMergeSplits];
    uint2 ov[kMergeSplits];
#pragma unroll
    for (int sidx = 0; sidx < kMergeSplits; ++sidx) {
      if (sidx < ns) {
        const int64_t ridx = (first + static_cast<int64_t>(sidx) * nr) * a.Hq + h;
        ml[sidx] = a.ml_part[ridx];
        ov[sidx] = *reinterpret_cast<const uint2*>(a.o_part + ridx * D + d);
      }
    }
    float M = -INFINITY;
#pragma unroll
    for (int sidx = 0; sidx < kMergeSplits; ++sidx)
      if (sidx < ns) M = fmaxf(M, ml[sidx].x);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int sidx = 0; sidx < kMergeSplits; ++sidx) {
      if (sidx < ns && ml[sidx].x != -INFINITY) {
        const float c = exp2f(ml[sidx].x - M) * ml[sidx].y;
        L += c;
        acc.x = fmaf(c, bf16_lo(ov[sidx].x), acc.x);
        acc.y = fmaf(c, bf16_hi(ov[sidx].x), acc.y);
        acc.z = fmaf(c, bf16_lo(ov[sidx].y), acc.z);
        acc.w = fmaf(c, bf16_hi(ov[sidx].y), acc.w);
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint2 wv;
    wv.x = static_cast<uint32_t>(f32_to_bf16(acc.x * inv)) | (static_cast<uint32_t>(f32_to_bf16(acc.y * inv)) << 16);
    wv.y = static_cast<uint32_t>(f32_to_bf16(acc.z * inv)) | (static_cast<uint32_t>(f32_to_bf16(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(a.out + (static_cast<int64_t>(row) * a.Hq + h) * D + d) = wv;
  }
}

}  // namespace dg
