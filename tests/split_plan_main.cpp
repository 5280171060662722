// Host driver for the split planner: reads "H_v V has_s0 cus n len_0 .. len_{n-1}"
// on stdin and prints the plan as whitespace-separated integers:
// "split n_seg n_prefix n_chain n_fwd" then the index arrays.
#include <cstdio>
#include <vector>

#include "split_plan.h"

int main() {
  int Hv, V, has_s0, cus, n;
  if (std::scanf("%d %d %d %d %d", &Hv, &V, &has_s0, &cus, &n) != 5) return 2;
  std::vector<int32_t> cu(n + 1, 0);
  for (int i = 0; i < n; ++i) {
    int len;
    if (std::scanf("%d", &len) != 1) return 2;
    cu[i + 1] = cu[i] + len;
  }
  gdn::SplitPlan p;
  const bool split = gdn::plan_split(cu.data(), n, Hv, V, has_s0 != 0, cus, p);
  std::printf("%d %d %d %d %d\n", split ? 1 : 0, p.n_seg, p.n_prefix, p.n_chain, p.n_fwd);
  for (int32_t x : p.ints) std::printf("%d ", x);
  std::printf("\n%d\n", gdn::max_prefix_segments(Hv, V, cus));
  return 0;
}
