"""Deficit token-budget admission (test infrastructure: the oracle of dg_deficit_admit).

Follows the Sangam page (llm-wiki.hwlabs.dev), section on the deficit token-budget scheduler:
every iteration has a token budget B; all running decode work is scheduled first and consumes
B_decode tokens; the remaining budget B_remain = B - B_decode together with the deficit D carried
from earlier iterations admits a waiting prefill only whole, when B_remain + D >= its size;
otherwise B_remain is added to D and carried to the next iteration.  Decode work therefore always
goes first, prefills are never split, and the growing deficit lets a prefill larger than any single
iteration's leftover budget enter eventually.

Readings (the page leaves these open):
  * "the prefill" is the head of a first-come-first-served queue; at most one prefill is admitted
    per iteration;
  * admitting a prefill spends the deficit it was owed: D becomes 0;
  * while no prefill waits, D is left unchanged;
  * B_remain is used as defined, B - B_decode, also when decode work exceeds the budget (then the
    deficit shrinks and admission is delayed until decode work falls below the budget again).

Pinned by tests/test_oracle_admission.py: a hand-worked trace (tests/golden/deficit_trace.txt),
the closed form of the admission iteration as the first prefix sum of leftover budget that reaches
the prefill's size, and the three properties the page states (decode first, prefills whole, no
starvation while leftover budget stays positive).
"""
from __future__ import annotations

from dataclasses import dataclass, field


def admit(budget: int, decode_tokens: int, queue: list, deficit: int):
    """One iteration.  queue: prefill sizes in arrival order.

    Returns (n_admitted, new_deficit, tokens_scheduled)."""
    remain = budget - decode_tokens
    if not queue:
        return 0, deficit, decode_tokens
    if remain + deficit >= queue[0]:
        return 1, 0, decode_tokens + queue[0]
    return 0, deficit + remain, decode_tokens


@dataclass
class Trace:
    """Per iteration: prefill ids admitted, tokens scheduled, deficit after the iteration."""
    admitted: list = field(default_factory=list)
    tokens: list = field(default_factory=list)
    deficit: list = field(default_factory=list)


def simulate(budget: int, decode_tokens: list, arrivals: list) -> Trace:
    """Run `admit` over len(decode_tokens) iterations.

    decode_tokens[t]: decode tokens scheduled at iteration t (given, independent of admissions);
    arrivals: (iteration, size) per prefill, in id order; a prefill joins the queue at the start
    of its arrival iteration."""
    tr = Trace()
    queue = []          # (id, size)
    d = 0
    for t, dec in enumerate(decode_tokens):
        for pid, (t_arr, size) in enumerate(arrivals):
            if t_arr == t:
                queue.append((pid, size))
        n, d, tok = admit(budget, dec, [s for _, s in queue], d)
        tr.admitted.append([queue[i][0] for i in range(n)])
        queue = queue[n:]
        tr.tokens.append(tok)
        tr.deficit.append(d)
    return tr
