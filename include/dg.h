/*
 * dg.h -- C ABI of the block-diffusion denoise step on AMD MI355X (gfx950).
 *
 * The library implements one step of block-diffusion decoding as described on
 * the DiffusionGemma/vLLM page (discuss.pytorch.kr, "DiffusionGemma: the first
 * dLLM natively supported by vLLM"), the single-pass-reads page
 * (portfolio.ywsung.com, "DiffusionGemma's execution path merged") and the
 * DFlash page (molayo1419.me, "How DFlash uses block diffusion to remove the
 * speculative-decoding bottleneck"):
 *
 *   dg_canvas_attention  mixed-mask attention over a paged KV prefix
 *   dg_denoise_sample    per-position softmax statistics, entropy, argmax, Gumbel-max candidate
 *   dg_entropy_accept    entropy-budget acceptance + random-token renoising
 *   dg_converged         convergence test, commit of the argmax canvas, block restart
 *   dg_selfcond_embed    P.E self-conditioning + gated MLP -> next-step canvas embedding
 * plus helpers for the structured-read readout, greedy block verification,
 * an fp32 linear layer for the tiny backbone and a device Philox call.
 *
 * Conventions (every entry point):
 *   - Pointer arguments are DEVICE pointers owned by the caller unless stated
 *     otherwise; the library never allocates, frees or synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously.  DG_OK means "validated and enqueued".
 *   - Arguments are validated on the host before anything is launched: a call
 *     that returns an error has launched nothing.  Values *inside* device
 *     buffers (token ids, split descriptors, page ids) are not validated on the
 *     host; page ids and token ids are clamped into range on the device so that a
 *     bad value yields a wrong result, never an out-of-bounds access.
 *   - Results are bitwise deterministic and batch-invariant per request: a
 *     request's outputs depend on its own inputs only, not on the other
 *     requests of a launch, the host-side bounds or the physical page ids
 *     (single-pass-reads page, section on judging the saved launch per request).
 *   - bf16 data is the top 16 bits of an IEEE fp32 (round to nearest even).
 *   - No entry point keeps state between calls and the library is thread-safe,
 *     except dg_denoise_sample_noalloc, whose per-device scratch array is
 *     shared by every call on that device.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dg_status;
typedef void* dg_stream_t; /* hipStream_t */

enum {
  DG_OK = 0,
  DG_E_ARG = -1,          /* null pointer, bad size, inconsistent shapes          */
  DG_E_UNSUPPORTED = -2,  /* dtype / head_dim / page size / alignment not supported */
  DG_E_WORKSPACE = -3,    /* workspace missing or smaller than the *_ws_bytes size  */
  DG_E_HIP = -4,          /* a HIP launch reported an error                          */
  DG_E_SCRATCH = -5       /* larger than the fixed scratch of an allocation-free entry point */
};

enum { DG_F32 = 0, DG_BF16 = 1 };

/* flags of dg_denoise_sample */
enum { DG_SAMPLE_ARGMAX_ONLY = 1 };

/* Philox streams (counter word 3) */
enum { DG_STREAM_GUMBEL = 0, DG_STREAM_RENOISE = 1, DG_STREAM_INIT = 2, DG_STREAM_GUMBEL_INNER = 3 };

int32_t dg_version(void);
const char* dg_status_str(dg_status s);

/* ------------------------------------------------------------------------ *
 * Philox4x32-10 (Salmon et al., SC'11), the noise source of every random
 * choice in the step.  out[i] = Philox(ctr[i], key[i]) for i < n.
 *   ctr: [n][4] uint32, key: [n][2] uint32, out: [n][4] uint32 (device).
 * Keying used by the step (one 64-bit seed per request):
 *   key = (seed & 0xffffffff, seed >> 32), counter = (c0, position, global step, stream);
 *   Gumbel noise of block b (ids 16 b .. 16 b + 15): word (b >> 7) & 3 of counter
 *     (128 (b >> 9) + (b & 127), pos, step, 0);
 *   Gumbel noise of vocabulary element i inside the winning block: word i & 3 of counter
 *     (i >> 2, pos, step, 3);
 *   renoise / init tokens: word 0 of counter (0, pos, step, 1 or 2), token = (w * V) >> 32;
 *   uniform(w) = (2 * (w >> 9) + 1) * 2^-24, Gumbel = -ln(-ln(uniform)).
 * ------------------------------------------------------------------------ */
dg_status dg_philox4x32_10(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out,
                           dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_canvas_attention
 *
 * One launch over a batch of requests, each in its own phase (the per-request
 * causality of the DiffusionGemma/vLLM page, section "Dynamic per-sequence
 * causal attention"; the row split of the single-pass-reads page, section on
 * keeping each row's visibility).  Request r's rows are packed at
 * [row0, row0 + n_causal + n_canvas) of q/k/v/out: first its causal rows,
 * then its canvas rows.
 *   causal row j : sees cache positions 0 .. cached + j; its K/V is written to
 *                  the request's pages at position cached + j (the encoder
 *                  pass: prompt chunk or commit pass).
 *   canvas row   : sees all cached + n_causal cache positions and every canvas
 *                  row of the request (bidirectional decoder pass); its K/V is
 *                  never written.
 * Sliding-window layers (same page, section on symmetric sliding-window
 * attention): with window W > 0 a row at position p (causal row j at
 * cached + j, canvas row j at cached + n_causal + j) keeps only keys at
 * positions p - W .. p if causal, p - W .. p + W if canvas (2W + 1 keys).
 * W <= 0 is a full-attention layer.
 * out = softmax(scale * q k^T over visible keys) v; query head h reads KV head
 * h / (Hq / Hkv).  No position encoding is applied.
 *
 * Layouts (row-major, dtype DG_BF16 or DG_F32 for every tensor):
 *   q [rows][Hq][D], k/v [rows][Hkv][D], out [rows][Hq][D]
 *   k_cache/v_cache [n_pages][Hkv][page_size][D]; position p of request r lives in
 *   physical page page_table[splits[r].page0 + p / page_size], slot p % page_size.
 *   splits: device array of n_req dg_split.
 * Host-side bounds (used to size the grid; the caller guarantees them):
 *   max_rows_per_req >= n_causal + n_canvas and max_keys_per_req >= the span of keys the
 *   request's rows see together: cached + n_causal + n_canvas, or at most
 *   n_causal + n_canvas + 2 * window for a request with a window.
 * Supported: D in {32, 64, 128, 256}, page_size 16, Hq % Hkv == 0; bf16 with D 128 / 256
 * (the MFMA path) also max_keys_per_req <= 261120.
 * Workspace: dg_canvas_attention_ws_bytes(...) bytes (may be 0 -> NULL allowed).
 * ------------------------------------------------------------------------ */
typedef struct dg_split {
  int32_t row0;      /* first packed row of the request                              */
  int32_t cached;    /* tokens already resident in the request's pages (read-only)    */
  int32_t n_causal;  /* causal rows in this launch (K/V appended at cached + j)       */
  int32_t n_canvas;  /* bidirectional canvas rows (K/V not written)                   */
  int32_t page0;     /* offset of the request's page list in page_table                */
  int32_t window;    /* sliding window W (> 0) of the layer, 0 for full attention     */
} dg_split;

size_t dg_canvas_attention_ws_bytes(int32_t n_req, int32_t rows, int32_t max_rows_per_req,
                                    int32_t max_keys_per_req, int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype);
dg_status dg_canvas_attention(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                              int32_t n_pages, const int32_t* page_table, int32_t page_table_len,
                              const dg_split* splits, int32_t n_req, int32_t rows,
                              int32_t max_rows_per_req, int32_t max_keys_per_req, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t page_size, float scale, int32_t dtype, void* out, void* ws,
                              size_t ws_bytes, dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_canvas_attention_e4m3
 *
 * dg_canvas_attention over an E4M3 paged cache (DiffusionGemma/vLLM page,
 * section "Quantized checkpoint support", the FP8 model): k_cache8 / v_cache8
 * hold OCP E4M3 codes in the page layout of dg_canvas_attention, a cached key
 * is k_scale * value(code) (v_scale for values).  Keys at positions >= cached
 * (this launch's causal and canvas rows) are read from k / v at bf16; the
 * causal rows are appended as codes: round-to-nearest-even of x / scale,
 * clamped to +-448.  q, k, v, out: DG_BF16.  k_scale and v_scale must be
 * powers of two (the conversions are then exact).  Supported: D in {128, 256},
 * page_size 16; workspace: dg_canvas_attention_ws_bytes(..., DG_BF16).
 * ------------------------------------------------------------------------ */
dg_status dg_canvas_attention_e4m3(const void* q, const void* k, const void* v, uint8_t* k_cache8,
                                   uint8_t* v_cache8, float k_scale, float v_scale, int32_t n_pages,
                                   const int32_t* page_table, int32_t page_table_len, const dg_split* splits,
                                   int32_t n_req, int32_t rows, int32_t max_rows_per_req, int32_t max_keys_per_req,
                                   int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, float scale, void* out,
                                   void* ws, size_t ws_bytes, dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_denoise_sample
 *
 * For every logit row (DiffusionGemma/vLLM page, section "Entropy-based
 * denoising" for H(p) = -sum p log p; section "DiffusionGemmaModelState and
 * DiffusionSampler", denoise case, for the Gumbel-max candidate), with
 * x = logits / temperature:
 *   row_max = max x,  row_lnz = ln sum exp(x - row_max),
 *   entropy = max(0, row_lnz - sum exp(x - m)(x - m) / sum exp(x - m)),
 *   argmax  = lowest index of the largest logit,
 *   sample  = a Gumbel-max draw in two levels over blocks of 16 ids: the block
 *             b* with the largest ln sum_{i in b} exp(x_i) + G_b, then the lowest
 *             index of the largest x_i + g_i inside b*; G and g from Philox
 *             (see above).  Its law is softmax(x).
 * Row r belongs to request r / rows_per_req at canvas position r % rows_per_req,
 * keyed by seed[request] and step[request].
 *   logits: [rows][ld] (DG_BF16 or DG_F32), ld % 8 == 0, ld >= V, 16-byte aligned.
 *   seed [n_req] uint64, step [n_req] int32, active [n_req] uint8 or NULL (all active);
 *   rows of inactive requests are skipped and their outputs left untouched.
 *   Outputs [rows]: entropy f32, argmax i32, sample i32, row_max f32, row_lnz f32.
 *   flags & DG_SAMPLE_ARGMAX_ONLY: only argmax is computed (others may be NULL).
 * Workspace: dg_denoise_sample_ws_bytes(rows, V) bytes.
 * ------------------------------------------------------------------------ */
size_t dg_denoise_sample_ws_bytes(int32_t rows, int32_t V);
dg_status dg_denoise_sample(const void* logits, int64_t ld, int32_t dtype, int32_t rows, int32_t V,
                            int32_t rows_per_req, const uint64_t* seed, const int32_t* step,
                            const uint8_t* active, float temperature, uint32_t flags, float* entropy,
                            int32_t* argmax, int32_t* sample, float* row_max, float* row_lnz, void* ws,
                            size_t ws_bytes, dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_denoise_sample_noalloc -- dg_denoise_sample for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and results, with its chunk
 * partials in a fixed device array of dg_denoise_sample_noalloc_max_bytes()
 * bytes (8 MiB) that each GPU holds until the process ends, instead of a
 * caller workspace.  Arguments as dg_denoise_sample minus ws / ws_bytes.
 * Calls whose dg_denoise_sample_ws_bytes(rows, V) exceeds the maximum return
 * DG_E_SCRATCH and launch nothing (V = 262144: up to 65535 rows).  The call
 * allocates nothing; every call on a GPU shares that GPU's array, so calls
 * that overlap on one GPU (concurrent streams or threads) race.  The first
 * call on a device looks the array's address up (hipGetSymbolAddress).
 * ------------------------------------------------------------------------ */
size_t dg_denoise_sample_noalloc_max_bytes(void);
dg_status dg_denoise_sample_noalloc(const void* logits, int64_t ld, int32_t dtype, int32_t rows, int32_t V,
                                    int32_t rows_per_req, const uint64_t* seed, const int32_t* step,
                                    const uint8_t* active, float temperature, uint32_t flags, float* entropy,
                                    int32_t* argmax, int32_t* sample, float* row_max, float* row_lnz,
                                    dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_denoise_sample_sc
 *
 * dg_denoise_sample (DG_BF16 logits, full mode) whose streaming pass also
 * writes the probability operand of the self-conditioning contraction
 * (DiffusionGemma/vLLM page, section "Self-conditioning": the full softmax of
 * this step feeds the next pass), so that dg_selfcond_embed_sc does not read
 * the logits again.  Operand layout (opaque to callers, sized by
 * dg_selfcond_operand_bytes(rows, V)): fp16 w[r][k] = 2^15 exp(x_k - ref)
 * for every run of 16384 vocabulary ids, ref being the run's largest x, plus
 * the refs.  Rows of inactive requests are not written.
 * ------------------------------------------------------------------------ */
size_t dg_selfcond_operand_bytes(int32_t rows, int32_t V);
dg_status dg_denoise_sample_sc(const void* logits, int64_t ld, int32_t dtype, int32_t rows, int32_t V,
                               int32_t rows_per_req, const uint64_t* seed, const int32_t* step,
                               const uint8_t* active, float temperature, float* entropy, int32_t* argmax,
                               int32_t* sample, float* row_max, float* row_lnz, void* ws, size_t ws_bytes,
                               void* sc_operand, size_t sc_operand_bytes, dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_entropy_accept
 *
 * Per canvas b (DiffusionGemma/vLLM page, section "Entropy-based denoising"):
 * positions ordered by (entropy, position) ascending are accepted while the
 * running fp64 sum of their entropies stays <= budget; accepted positions take
 * sample[b][pos], every other position gets a random token from Philox stream
 * RENOISE at step[b].
 *   entropy [B][C] f32 (>= 0), sample [B][C] i32, canvas [B][C] i32 (in/out),
 *   accept [B][C] u8 (out, may be NULL), n_accept [B] i32 (out, may be NULL),
 *   seed [B] u64, step [B] i32, active [B] u8 or NULL.  1 <= C <= 1024.
 * ------------------------------------------------------------------------ */
dg_status dg_entropy_accept(const float* entropy, const int32_t* sample, int32_t B, int32_t C, int32_t V,
                            double budget, const uint64_t* seed, const int32_t* step, const uint8_t* active,
                            int32_t* canvas, uint8_t* accept, int32_t* n_accept, dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_converged
 *
 * Per request (DiffusionGemma/vLLM page, sections "Entropy-based denoising"
 * and "DiffusionGemmaModelState and DiffusionSampler"):
 *   prefill case (step_in_block < 0): canvas <- Philox INIT tokens at step_global,
 *     step_in_block <- 0, unchanged <- 0, sc_on <- 0, nothing emitted.
 *   denoise case: unchanged <- (step_in_block > 0 and argmax == prev_argmax over the
 *     whole canvas) ? unchanged + 1 : 0;  converged <- unchanged >= k and mean(entropy) < tau;
 *     if converged or step_in_block + 1 >= max_steps: commit -- out_tokens <- argmax,
 *     steps_used <- step_in_block + 1, num_sampled <- C, canvas <- Philox INIT tokens at
 *     step_global, unchanged <- 0, step_in_block <- 0, sc_on <- 0;
 *     else step_in_block += 1, sc_on <- 1, num_sampled <- 0.  prev_argmax <- argmax.
 *   step_global += 1 in both cases.  committed[b] is 1 exactly when a commit happened.
 *   argmax/prev_argmax/canvas/out_tokens [B][C] i32; entropy [B][C] f32;
 *   unchanged/step_in_block/step_global/steps_used/num_sampled [B] i32; sc_on/committed [B] u8;
 *   seed [B] u64; active [B] u8 or NULL.  The mean is an fp64 sum / C.  1 <= C <= 1024.
 * ------------------------------------------------------------------------ */
dg_status dg_converged(const int32_t* argmax, const float* entropy, int32_t B, int32_t C, int32_t V, int32_t k,
                       double tau, int32_t max_steps, const uint64_t* seed, const uint8_t* active,
                       int32_t* prev_argmax, int32_t* unchanged, int32_t* step_in_block, int32_t* step_global,
                       int32_t* canvas, uint8_t* sc_on, uint8_t* committed, int32_t* out_tokens,
                       int32_t* steps_used, int32_t* num_sampled, dg_stream_t stream);

/* dg_accept_converged: dg_entropy_accept followed by dg_converged in one launch (one workgroup per
 * request).  A request in its prefill case (step_in_block < 0) gets only dg_converged's prefill;
 * every other active request gets the acceptance (renoise keyed by its current step_global, as
 * dg_entropy_accept with step = step_global) and then the convergence test on the accepted canvas.
 * Arguments as in the two entry points (accept and n_accept may be NULL; budget not NaN); results
 * are bitwise those of the two calls in sequence. */
dg_status dg_accept_converged(const float* entropy, const int32_t* sample, const int32_t* argmax, int32_t B,
                              int32_t C, int32_t V, double budget, int32_t k, double tau, int32_t max_steps,
                              const uint64_t* seed, const uint8_t* active, int32_t* prev_argmax, int32_t* unchanged,
                              int32_t* step_in_block, int32_t* step_global, int32_t* canvas, uint8_t* sc_on,
                              uint8_t* committed, int32_t* out_tokens, int32_t* steps_used, int32_t* num_sampled,
                              uint8_t* accept, int32_t* n_accept, dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_selfcond_embed
 *
 * Self-conditioning of the next denoise pass (DiffusionGemma/vLLM page,
 * section "Self-conditioning"), for every canvas row r of B requests x C positions:
 *   p_r = exp(x_r - row_max_r - row_lnz_r)  (this step's softmax; x = logits / temperature)
 *   s_r = p_r . E                            E [V][d]
 *   y_r = (gelu_tanh(s_r W_gate) * (s_r W_up)) W_down      W_gate/W_up [d][hidden], W_down [hidden][d]
 *   x_out_r = E[canvas_r] + (sc_on[request] ? y_r : 0)
 * dtype DG_BF16: logits, E, weights and x_out are bf16; the contractions run on fp16
 *   MFMA against the prepared fp16 copy (dg_selfcond_prepare) with fp32 accumulation.
 * dtype DG_F32: everything fp32 (prepared may be NULL).
 *   logits [rows][ld], ld % 8 == 0; row_max/row_lnz [rows] f32; canvas [rows] i32;
 *   sc_on [B] u8; x_out [rows][d]; s_out [rows][d] f32 or NULL (the P.E result);
 *   y_out [rows][d] f32 or NULL (the gated-MLP output y, for every row whatever sc_on).
 *   DG_BF16: d and hidden multiples of 128, at most 8192 (else DG_E_UNSUPPORTED).
 * Workspace: dg_selfcond_ws_bytes(rows, V, d, hidden, dtype) bytes.
 * ------------------------------------------------------------------------ */
size_t dg_selfcond_prepared_bytes(int32_t V, int32_t d, int32_t hidden, int32_t dtype);
dg_status dg_selfcond_prepare(const void* E, const void* w_gate, const void* w_up, const void* w_down, int32_t V,
                              int32_t d, int32_t hidden, int32_t dtype, void* prepared, size_t prepared_bytes,
                              dg_stream_t stream);
size_t dg_selfcond_ws_bytes(int32_t rows, int32_t V, int32_t d, int32_t hidden, int32_t dtype);
dg_status dg_selfcond_embed(const void* logits, int64_t ld, int32_t dtype, float temperature, const float* row_max,
                            const float* row_lnz, const uint8_t* sc_on, const int32_t* canvas, int32_t B, int32_t C,
                            const void* E, const void* w_gate, const void* w_up, const void* w_down,
                            const void* prepared, int32_t V, int32_t d, int32_t hidden, void* x_out, float* s_out,
                            float* y_out, void* ws, size_t ws_bytes, dg_stream_t stream);

/* Same as dg_selfcond_embed; when pe_start / pe_stop (hipEvent_t) are non-NULL they are
 * recorded on `stream` immediately before and after the P.E contraction kernel, so a caller
 * can time that kernel alone (the bf16 path's dominant launch) with hipEventElapsedTime. */
dg_status dg_selfcond_embed_traced(const void* logits, int64_t ld, int32_t dtype, float temperature,
                                   const float* row_max, const float* row_lnz, const uint8_t* sc_on,
                                   const int32_t* canvas, int32_t B, int32_t C, const void* E, const void* w_gate,
                                   const void* w_up, const void* w_down, const void* prepared, int32_t V, int32_t d,
                                   int32_t hidden, void* x_out, float* s_out, float* y_out, void* ws,
                                   size_t ws_bytes, void* pe_start, void* pe_stop, dg_stream_t stream);

/* dg_selfcond_embed_sc: dg_selfcond_embed (DG_BF16) taking the probability operand written by
 * dg_denoise_sample_sc of the same step instead of the logits; row_max / row_lnz are that call's
 * outputs.  Each P.E split covers one 16384-id run of the operand.  pe_start / pe_stop as in
 * dg_selfcond_embed_traced (may be NULL).  Workspace: dg_selfcond_ws_bytes_sc(rows, V, d, hidden). */
size_t dg_selfcond_ws_bytes_sc(int32_t rows, int32_t V, int32_t d, int32_t hidden);
dg_status dg_selfcond_embed_sc(const void* sc_operand, const float* row_max, const float* row_lnz,
                               const uint8_t* sc_on, const int32_t* canvas, int32_t B, int32_t C, const void* E,
                               const void* prepared, int32_t V, int32_t d, int32_t hidden, void* x_out,
                               float* s_out, float* y_out, void* ws, size_t ws_bytes, void* pe_start,
                               void* pe_stop, dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_lmhead_denoise_sample -- the LM head fused with the denoise sampler.
 *
 * logits[r][v] = scale * sum_k h[r][k] E[v][k] (the embedding table as the
 * output projection; bf16 inputs, fp32 accumulation), then for every row what
 * dg_denoise_sample computes from those logits (DiffusionGemma/vLLM page,
 * sections "Entropy-based denoising" and "DiffusionGemmaModelState and
 * DiffusionSampler": x = logits / temperature, entropy, argmax, the two-level
 * Gumbel-max sample with the same Philox streams, m = max x, ln Z), plus the
 * probability operand of the self-conditioning contraction (section
 * "Self-conditioning"), which dg_selfcond_embed_lm consumes.  The [rows][V]
 * logits are never written to memory.
 * dg_lmhead_prepare: E [V][d] bf16 row-major -> `prepared`
 *   (dg_lmhead_prepared_bytes(V, d) bytes, caller-owned, opaque: the table
 *   re-laid for the kernel's copies), once per table.
 * dg_lmhead_denoise_sample:
 *   h [rows][ldh] bf16 (ldh >= d, ldh % 8 == 0, 16-byte aligned); prepared
 *   from dg_lmhead_prepare; V % 16 == 0, d % 128 == 0, d <= 16384; scale > 0,
 *   temperature > 0 (finite); rows <= 65535, rows % rows_per_req == 0;
 *   seed [rows / rows_per_req] u64, step i32 (the Gumbel noise of row r is
 *   keyed by (seed, r % rows_per_req, step) of its request); active
 *   [rows / rows_per_req] u8 or NULL: the five outputs of inactive requests'
 *   rows are not written (the operand covers every row).
 *   entropy, row_max, row_lnz [rows] f32; argmax, sample [rows] i32.
 *   Workspace: dg_lmhead_ws_bytes(rows, V, d) bytes.  operand: caller-owned,
 *   dg_lmhead_operand_bytes(rows, V) bytes, opaque (fp16 probabilities
 *   relative to one power of two per 16384-id run, those references, each
 *   row's argmax).  Argmax ties resolve to the lowest id.  Not bitwise equal
 *   to dg_denoise_sample on bf16-rounded logits: these logits keep fp32.
 * dg_lmhead_denoise_sample_traced: the same; when k_start / k_stop
 *   (hipEvent_t) are non-NULL they are recorded on `stream` immediately before
 *   and after the fused LM-head kernel, the call's dominant launch.
 * ------------------------------------------------------------------------ */
size_t dg_lmhead_prepared_bytes(int32_t V, int32_t d);
dg_status dg_lmhead_prepare(const void* E, int32_t V, int32_t d, void* prepared, size_t prepared_bytes,
                            dg_stream_t stream);
size_t dg_lmhead_ws_bytes(int32_t rows, int32_t V, int32_t d);
size_t dg_lmhead_operand_bytes(int32_t rows, int32_t V);
dg_status dg_lmhead_denoise_sample(const void* h, int64_t ldh, const void* prepared, int32_t rows, int32_t V,
                                   int32_t d, float scale, int32_t rows_per_req, const uint64_t* seed,
                                   const int32_t* step, const uint8_t* active, float temperature, float* entropy,
                                   int32_t* argmax, int32_t* sample, float* row_max, float* row_lnz, void* ws,
                                   size_t ws_bytes, void* operand, size_t operand_bytes, dg_stream_t stream);
dg_status dg_lmhead_denoise_sample_traced(const void* h, int64_t ldh, const void* prepared, int32_t rows, int32_t V,
                                          int32_t d, float scale, int32_t rows_per_req, const uint64_t* seed,
                                          const int32_t* step, const uint8_t* active, float temperature,
                                          float* entropy, int32_t* argmax, int32_t* sample, float* row_max,
                                          float* row_lnz, void* ws, size_t ws_bytes, void* operand,
                                          size_t operand_bytes, void* k_start, void* k_stop, dg_stream_t stream);

/* dg_selfcond_embed_lm: dg_selfcond_embed_sc on the operand written by dg_lmhead_denoise_sample of
 * the same step (row_max / row_lnz are that call's outputs): s = softmax(x) E (each row's largest
 * probability entering exactly), then the gated MLP and x_out = bf16(E[canvas] + (sc_on ? y : 0)).
 * E is the bf16 table [V][d]; prepared from dg_selfcond_prepare.  V % 16 == 0; other arguments,
 * the workspace (dg_selfcond_ws_bytes_sc) and pe_start / pe_stop as in dg_selfcond_embed_sc. */
dg_status dg_selfcond_embed_lm(const void* lm_operand, const float* row_max, const float* row_lnz,
                               const uint8_t* sc_on, const int32_t* canvas, int32_t B, int32_t C, const void* E,
                               const void* prepared, int32_t V, int32_t d, int32_t hidden, void* x_out, float* s_out,
                               float* y_out, void* ws, size_t ws_bytes, void* pe_start, void* pe_stop,
                               dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_allowed_probs -- structured-read readout (single-pass-reads page,
 * section on answer slots): for slot s with allowed ids ids[offsets[s] ..
 * offsets[s+1]), q = softmax over x = logits[slot_row[s]][id] / temperature
 * restricted to those ids; answer[s] = first listed id with the largest logit.
 *   logits [*][ld] (DG_BF16 / DG_F32); slot_row [n_slots] i32; offsets [n_slots+1] i32;
 *   ids [offsets[n_slots]] i32; q [offsets[n_slots]] f32; answer [n_slots] i32.
 *   Every slot must list 1..64 ids.
 * ------------------------------------------------------------------------ */
dg_status dg_allowed_probs(const void* logits, int64_t ld, int32_t dtype, int32_t n_rows, int32_t n_slots,
                           int32_t V, const int32_t* slot_row, const int32_t* offsets, const int32_t* ids,
                           float temperature, float* q, int32_t* answer, dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * E4M3 embedding-table variant (DiffusionGemma/vLLM page, section "Quantized
 * checkpoint support": the model ships FP8 weights).  The table is stored as
 * OCP E4M3 codes E8 [V][d] (uint8, row-major) times one fp32 scale e_scale.
 *
 * dg_e4m3_decode: out32[i] = e_scale * value(codes[i]) (f32); out16 (may be
 *   NULL) = value(codes[i]) as fp16 (exact).  The conversions the kernels use.
 *   n % 8 == 0; codes, out32, out16 16-byte aligned.
 * dg_selfcond_prepare_e4m3: builds the K-blocked E8^T byte operand and the
 *   fp16 MLP operands (w_gate, w_up, w_down bf16 as in dg_selfcond_prepare)
 *   into `prepared` (dg_selfcond_prepared_bytes_e4m3 bytes).
 * dg_selfcond_embed_sc_e4m3: dg_selfcond_embed_sc with the table E = e_scale *
 *   value(E8): s = softmax(x) E on fp16 MFMA with the E4M3 operand converted to
 *   fp16 after its LDS read (the E stream is 1 byte per element), then the
 *   MLP and x_out = bf16(E[canvas] + (sc_on ? y : 0)).  Workspace:
 *   dg_selfcond_ws_bytes_sc.
 * Supported: d % 256 == 0, hidden % 128 == 0, both <= 8192.
 * ------------------------------------------------------------------------ */
dg_status dg_e4m3_decode(const uint8_t* codes, int64_t n, float scale, float* out32, void* out16,
                         dg_stream_t stream);
size_t dg_selfcond_prepared_bytes_e4m3(int32_t V, int32_t d, int32_t hidden);
dg_status dg_selfcond_prepare_e4m3(const uint8_t* E8, const void* w_gate, const void* w_up, const void* w_down,
                                   int32_t V, int32_t d, int32_t hidden, void* prepared, size_t prepared_bytes,
                                   dg_stream_t stream);
dg_status dg_selfcond_embed_sc_e4m3(const void* sc_operand, const float* row_max, const float* row_lnz,
                                    const uint8_t* sc_on, const int32_t* canvas, int32_t B, int32_t C,
                                    const uint8_t* E8, float e_scale, const void* prepared, int32_t V, int32_t d,
                                    int32_t hidden, void* x_out, float* s_out, float* y_out, void* ws,
                                    size_t ws_bytes, void* pe_start, void* pe_stop, dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_deficit_admit -- one iteration of the deficit token-budget admission of
 * a serving loop (Sangam page, section on the deficit token-budget scheduler).
 * Host function: plain host pointers, no GPU work, no stream.
 * All decode work (decode_tokens: canvas rows and commit-pass rows of the
 * running requests) is scheduled first.  The waiting prefill at the head of the
 * first-come-first-served queue is admitted whole when
 *   (budget - decode_tokens) + *deficit >= queue[0];
 * then *deficit <- 0 and *n_admitted = 1.  Otherwise *deficit grows by
 * budget - decode_tokens (negative when decode work overruns the budget) and
 * *n_admitted = 0.  With an empty queue nothing changes.  Prefills are never
 * split and at most one is admitted per iteration.
 *   budget > 0, decode_tokens >= 0, queue [n_queue] token counts (queue[0] > 0),
 *   deficit in/out, n_admitted out, tokens out (may be NULL): tokens scheduled
 *   this iteration (decode_tokens plus the admitted prefill).
 * ------------------------------------------------------------------------ */
dg_status dg_deficit_admit(int64_t budget, int64_t decode_tokens, const int64_t* queue, int32_t n_queue,
                           int64_t* deficit, int32_t* n_admitted, int64_t* tokens);

/* ------------------------------------------------------------------------ *
 * dg_verify_prefix -- greedy block verification (DFlash page, section "What
 * DFlash does differently", verification step): accepted[b] = index of the
 * first j with draft[b][j] != target[b][j], or L if the whole block matches.
 *   draft/target [B][L] i32, accepted [B] i32.
 * ------------------------------------------------------------------------ */
dg_status dg_verify_prefix(const int32_t* draft, const int32_t* target, int32_t B, int32_t L, int32_t* accepted,
                           dg_stream_t stream);

/* ------------------------------------------------------------------------ *
 * dg_linear -- fp32 C = alpha * A op(B) (+ residual), for the tiny backbone's
 * projections and tied LM head.  A [M][K]; B [K][N] (trans_b = 0) or [N][K]
 * (trans_b = 1); residual [M][N] or NULL; C [M][N].  Row-major fp32.
 * ------------------------------------------------------------------------ */
dg_status dg_linear(const float* A, const float* B, const float* residual, float* C, int32_t M, int32_t N,
                    int32_t K, int32_t trans_b, float alpha, dg_stream_t stream);

/* dg_gather_rows -- out[i][:] = table[idx[i]][:] (fp32 or bf16 rows of width d), the
 * plain embedding lookup of the encoder passes (no self-conditioning). */
dg_status dg_gather_rows(const void* table, int32_t n_table, int32_t d, int32_t dtype, const int32_t* idx,
                         int32_t n, void* out, dg_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
