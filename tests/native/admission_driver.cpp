// Host driver of dg_deficit_admit for the sanitizer test (tests/test_host_sanitizers.py): built with
// g++ under AddressSanitizer and UndefinedBehaviorSanitizer together with the library's host source.
//
// stdin: the number of traces, then per trace "budget n_iter n_pf", n_iter decode-token counts and
// n_pf (arrival iteration, size) pairs in id order.  A trace is run as a serving loop would: arrivals
// join a first-come-first-served queue at the start of their iteration, then one call per iteration.
// stdout: per iteration "admitted_id_or_-1 deficit tokens"; then the status codes of calls with
// invalid arguments (which must not touch their outputs).
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "dg.h"

int main() {
  int n_traces = 0;
  if (scanf("%d", &n_traces) != 1) return 2;
  for (int tr = 0; tr < n_traces; ++tr) {
    long long budget = 0;
    int n_iter = 0, n_pf = 0;
    if (scanf("%lld %d %d", &budget, &n_iter, &n_pf) != 3) return 2;
    std::vector<long long> decode(n_iter);
    for (auto& x : decode)
      if (scanf("%lld", &x) != 1) return 2;
    std::vector<int> t_arr(n_pf);
    std::vector<long long> size(n_pf);
    for (int i = 0; i < n_pf; ++i)
      if (scanf("%d %lld", &t_arr[i], &size[i]) != 2) return 2;
    std::vector<int> queue_id;
    std::vector<int64_t> queue_size;
    int64_t deficit = 0;
    for (int t = 0; t < n_iter; ++t) {
      for (int i = 0; i < n_pf; ++i)
        if (t_arr[i] == t) {
          queue_id.push_back(i);
          queue_size.push_back(size[i]);
        }
      int32_t n = -1;
      int64_t tokens = -1;
      // an exactly sized copy of the queue, so that a read past its end is caught
      std::vector<int64_t> q(queue_size);
      const dg_status st = dg_deficit_admit(budget, decode[t], q.empty() ? nullptr : q.data(),
                                            static_cast<int32_t>(q.size()), &deficit, &n, &tokens);
      if (st != DG_OK) return 3;
      printf("%d %lld %lld\n", n == 1 ? queue_id[0] : -1, static_cast<long long>(deficit),
             static_cast<long long>(tokens));
      if (n == 1) {
        queue_id.erase(queue_id.begin());
        queue_size.erase(queue_size.begin());
      }
    }
  }
  // invalid arguments: rejected with DG_E_ARG, outputs untouched
  int64_t d = 7, tok = 9, one = 5, zero = 0;
  int32_t n = 11;
  const dg_status bad[] = {
      dg_deficit_admit(0, 0, &one, 1, &d, &n, &tok),          // budget <= 0
      dg_deficit_admit(10, -1, &one, 1, &d, &n, &tok),        // negative decode work
      dg_deficit_admit(10, 0, &one, -1, &d, &n, &tok),        // negative queue length
      dg_deficit_admit(10, 0, nullptr, 1, &d, &n, &tok),      // queue missing
      dg_deficit_admit(10, 0, &zero, 1, &d, &n, &tok),        // empty prefill at the head
      dg_deficit_admit(10, 0, &one, 1, nullptr, &n, &tok),    // deficit missing
      dg_deficit_admit(10, 0, &one, 1, &d, nullptr, &tok),    // count missing
  };
  for (dg_status s : bad) printf("status %d\n", s);
  printf("untouched %lld %d %lld\n", static_cast<long long>(d), n, static_cast<long long>(tok));
  // tokens may be NULL; large counts stay exact
  const int64_t big = int64_t{1} << 40;
  const dg_status s = dg_deficit_admit(big, big - 3, &one, 1, &d, &n, nullptr);
  printf("null_tokens %d %d %lld\n", s, n, static_cast<long long>(d));
  return 0;
}
