"""The five synthetic workloads as plain data (sizes and loop constants; no arithmetic).

tiny_loop      : one request, prefix 32, canvas 16, V 1024, d 64, 2 heads x 32, one fp32 layer,
                 logits = 4 h E^T, budget 2.0 nats, k = 2, tau = 0.5, max 32 steps, MLP 64->128->64.
single_canvas  : one request, one 256-token canvas over a 2048-token paged bf16 prefix
                 (page 16, 16 query / 8 KV heads, head_dim 256), logits 256 x 262144 bf16,
                 E 262144 x 4096 bf16, MLP 4096->1024->4096, budget 8, k = 3, tau = 0.3, max 64.
batched        : 32 requests, prefixes U[512, 8192], 256-token canvases, staggered steps.
structured_read: 64 requests, 2048 causal prompt rows + 256 canvas rows each, 8 slots per request
                 with 2-5 allowed ids, V 262144.
block_draft    : 128 requests x 16 masked positions, 5 draft layers with injected context KV
                 (32 query / 8 KV heads, head_dim 128, context U[256, 4096]), V 151936, argmax,
                 greedy verification against targets whose first mismatch is geometric(0.2).
"""
TINY_LOOP = dict(
    name="tiny_loop", seed=0, prefix=32, C=16, V=1024, d=64, Hq=2, Hkv=2, D=32, layers=1,
    w_std=0.02, e_std=1.0 / 8.0, logit_scale=4.0, budget=2.0, k=2, tau=0.5, max_steps=32,
    hidden=128, temperature=1.0, page_size=16,
)

SINGLE_CANVAS = dict(
    name="single_canvas", seed=0, B=1, C=256, L=2048, page_size=16, Hq=16, Hkv=8, D=256,
    V=262144, d=4096, hidden=1024, budget=8.0, k=3, tau=0.3, max_steps=64, temperature=1.0,
    e_std=1.0 / 8.0, w_std=0.02,
)

BATCHED = dict(
    name="batched", seed=0, B=32, C=256, L_min=512, L_max=8192, page_size=16, Hq=16, Hkv=8, D=256,
    V=262144, d=4096, hidden=1024, budget=8.0, k=3, tau=0.3, max_steps=64, temperature=1.0,
)

STRUCTURED_READ = dict(
    name="structured_read", seed=0, B=64, n_causal=2048, C=256, page_size=16, Hq=16, Hkv=8, D=256,
    V=262144, slots=8, min_ids=2, max_ids=5, temperature=1.0,
)

BLOCK_DRAFT = dict(
    name="block_draft", seed=0, B=128, block=16, layers=5, Hq=32, Hkv=8, D=128, L_min=256, L_max=4096,
    page_size=16, V=151936, p_mismatch=0.2,
)

ALL = [TINY_LOOP, SINGLE_CANVAS, BATCHED, STRUCTURED_READ, BLOCK_DRAFT]

# Batched serving loop with deficit token-budget admission (Sangam page, deficit scheduler): requests
# arrive in bursts of `burst` every `arrival_every` iterations with prompts U[P_min, P_max]; each is
# prefilled whole when
# admitted, then denoises `blocks` canvases of C tokens (commit pass after each).  Activations (Q/K/V
# rows) and logits are synthetic pools: the loop exercises scheduling, launch composition, the paged
# cache and the per-request state, not a trained backbone.
SERVING = dict(
    name="serving", seed=0, R=32, C=256, P_min=512, P_max=8192, burst=8, arrival_every=6, page_size=16, Hq=16,
    Hkv=8, D=256, V=262144, token_budget=8192, blocks=2, budget=8.0, k=3, tau=0.3, max_steps=8,
    temperature=1.0, n_pool=2, d=4096, hidden=1024,
)

# The same loop at sizes the oracle runs in seconds (bf16, MFMA attention path).
SERVING_SMALL = dict(
    name="serving_small", seed=0, R=6, C=16, P_min=8, P_max=72, arrival_every=1, page_size=16, Hq=4, Hkv=2,
    D=128, V=2048, token_budget=72, blocks=2, budget=4.0, k=2, tau=0.3, max_steps=4, temperature=1.0,
    n_pool=3, d=128, hidden=128,
)

# The batched workload as a steady-state loop (every request already holds its prefix of
# U[P_min, P_max] tokens and denoises from the first iteration; request r starts at step 2r of its
# block and global step 2r + 1, so one block reaches the 64-step cap every two iterations, runs its
# commit pass and restarts), with self-conditioning.  Pages are sized for the prefix plus `blocks`
# committed blocks.
BATCHED_LOOP = dict(
    name="batched_loop", seed=0, R=32, C=256, P_min=512, P_max=8192, arrival_every=1, page_size=16, Hq=16,
    Hkv=8, D=256, V=262144, token_budget=8192, blocks=2, budget=8.0, k=3, tau=0.3, max_steps=64,
    temperature=1.0, n_pool=2, d=4096, hidden=1024,
)

# The LM head fused with the sampler (logits = scale h E^T never stored): h from
# synth.lmhead_hidden_*, E ~ N(0, 1/64) bf16.  Small: two requests of 20 rows over a vocabulary of
# 16464 ids (two P.E runs, the second ragged, and LM-head tiles past V) with d = 256.  Full: the
# single canvas (256 rows, V = 262144, d = 4096, MLP 4096 -> 1024 -> 4096).
LMHEAD_SMALL = dict(
    name="lmhead_small", seed=0, B=2, C=20, V=16464, d=256, hidden=128, scale=4.0, a_max=1.5, b=0.125,
    temperature=0.8, e_std=1.0 / 8.0, w_std=0.5,
)

LMHEAD = dict(
    name="lmhead_single_canvas", seed=0, B=1, C=256, V=262144, d=4096, hidden=1024, scale=1.0, a_max=0.4, b=0.125,
    temperature=1.0, e_std=1.0 / 8.0, w_std=0.02,
)
