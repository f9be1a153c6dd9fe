"""CPU oracle for the block-diffusion denoise step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 numpy statement of what the denoise step computes, written
from the method's description on the pages it cites.  It exists to check the
HIP library: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path never
routes through it, and it shares no code with ``denoise_step_amd``.

Modules
  philox     Philox4x32-10 and the three mappings (uniform, Gumbel, token)
  sampler    softmax / entropy / argmax / Gumbel-max candidate per row
  accept     entropy-budget acceptance + renoising
  converged  convergence test, commit, block restart
  attention  mixed-mask (causal + canvas) attention over a paged KV prefix
  selfcond   P.E self-conditioning + gated MLP + next-step canvas embedding
  readout    allowed-choice probabilities for single-pass structured reads
  verify     greedy longest-matching-prefix block verification
  backbone   the one-layer fp32 backbone of the tiny closed loop
  loop       the tiny closed denoise loop
  admission  deficit token-budget admission of a serving loop
  serving    the batched serving loop composed from the parts above
  fp8        OCP E4M3 decoding and encoding

Every function here is pinned by a ``-m "not gpu"`` test against values the
pages fix, hand-worked traces, closed forms, brute force, invariants or an
independent library routine; each module header names its pins.
"""
