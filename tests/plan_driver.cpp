// Host build of the in-tile copy schedule (sync_protocols_amd/csrc/fg_plan.hpp)
// for tests/test_copy_plan.py: prints, for the shape given on the command
// line, the tile and the copied non-lead rows of every item of every list.
//   plan_driver n_slabs half_last per_list n_tn GS GN
// Output: "L x ns lead rows" per list, then "I x j tile c0 c1" per item.
#include <cstdio>
#include <cstdlib>

#include "fg_plan.hpp"

int main(int argc, char** argv) {
  if (argc != 7) return 2;
  fg::CopyPlan p{};
  p.n_slabs = atoi(argv[1]);
  p.half_last = atoi(argv[2]);
  p.nx = 8;
  p.per_list = atoi(argv[3]);
  p.n_tn = atoi(argv[4]);
  p.GS = atoi(argv[5]);
  p.GN = atoi(argv[6]);
  p.lead = fg::plan_lead_slabs(p.per_list, p.n_tn);
  for (int x = 0; x < p.nx; ++x) {
    const int ns = fg::plan_ns(p, x);
    printf("L %d %d %d %d\n", x, ns, fg::plan_ld(p, x), fg::plan_rows(p, x));
    for (int j = 0; j < ns * p.n_tn; ++j) {
      int c0 = 0, c1 = 0;
      fg::plan_item_rows(p, x, j, &c0, &c1);
      printf("I %d %d %d %d %d\n", x, j, fg::plan_tile(p, x, j), c0, c1);
    }
  }
  return 0;
}
