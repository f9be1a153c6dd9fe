// dg_deficit_admit: the deficit token-budget admission of a serving loop (host code).
//
// Sangam page (llm-wiki.hwlabs.dev), section on the deficit token-budget scheduler: decode work is
// scheduled first; what is left of the iteration's budget, plus the deficit carried from earlier
// iterations, admits the waiting prefill only whole; otherwise the leftover is added to the
// deficit.  The head of a first-come-first-served queue is the waiting prefill, at most one is
// admitted per iteration, admission spends the deficit (D = 0), and D is left alone while nothing
// waits.
#include <stdint.h>

#include "dg.h"

extern "C" dg_status dg_deficit_admit(int64_t budget, int64_t decode_tokens, const int64_t* queue, int32_t n_queue,
                                      int64_t* deficit, int32_t* n_admitted, int64_t* tokens) {
  if (budget <= 0 || decode_tokens < 0 || n_queue < 0 || deficit == nullptr || n_admitted == nullptr ||
      (n_queue > 0 && (queue == nullptr || queue[0] <= 0)))
    return DG_E_ARG;
  const int64_t remain = budget - decode_tokens;  // negative when decode work overruns the budget
  int32_t n = 0;
  int64_t scheduled = decode_tokens;
  if (n_queue > 0) {
    if (remain + *deficit >= queue[0]) {
      n = 1;
      scheduled += queue[0];
      *deficit = 0;
    } else {
      *deficit += remain;
    }
  }
  *n_admitted = n;
  if (tokens != nullptr) *tokens = scheduled;
  return DG_OK;
}
