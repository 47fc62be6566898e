// Schedule of the in-tile copy: which gathered rows every workgroup copies
// before it starts computing (the lead slabs), and which rows each tile copies
// inside its K loop for the tiles of later rounds. Pure integer arithmetic,
// compiled for the device and, by a CPU test, for the host.
//
// Setting ("PCIe sync protocols" §5 and §6): the compute role takes tiles from
// one list per XCD; list x owns the 256-row slabs x, x + 8, x + 16, ... of
// the gathered buffer (the last slab of the buffer may have 128 rows). A
// tile gates on the arrival counters of its slab's 128-row blocks, so every
// row of a slab must be copied and counted before the slab's first tile
// starts (§6 audit item 3: a consumer never waits on work scheduled after it).
//
// Order of list x's items. The first `lead` slabs of the list, slab by slab,
// each over all column tiles; lead is the smallest slab count whose tiles fill
// one round of the list's workgroups, so every item of the first round reads
// a lead slab. The other slabs follow in groups of GS slabs x GN column tiles
// (the tiles that run together on one XCD then share A and W lines in its L2),
// as in the default order.
//
// Copy. The lead slabs of all lists are the gathered rows [0, 8 * 256 * lead):
// every workgroup copies its share of them first. The other ("non-lead")
// rows of list x, taken in slab order, are dealt to the whole items of the
// list so that the rows of a group of slabs are all copied by items of an
// earlier round than the group's first item: by the end of round r the items
// have copied C(r) = max(need(r + 1), U(r)) rows, where need(r) is the rows of
// the groups whose first item lies in a round <= r and U spreads the rest
// evenly over the rounds before the last group starts; round r's share is
// split evenly over its items.
#pragma once

#ifdef __HIPCC__
#define FG_HD __host__ __device__ __forceinline__
#else
#define FG_HD inline
#endif

namespace fg {

FG_HD int pmin(int a, int b) { return a < b ? a : b; }
FG_HD int pmax(int a, int b) { return a > b ? a : b; }

struct CopyPlan {
  int n_slabs;    // slabs of the gathered buffer: 256 rows, the last one 128 rows when half_last
  int half_last;
  int nx;         // lists (one per XCD)
  int per_list;   // workgroups per list
  int n_tn;       // column tiles per slab
  int GS, GN;     // group shape after the lead slabs (GN divides n_tn)
  int lead;       // lead slabs per list
};

// Lead slabs per list: the fewest whose tiles fill one round of the list.
FG_HD int plan_lead_slabs(int per_list, int n_tn) { return (per_list + n_tn - 1) / n_tn; }

FG_HD int plan_ns(const CopyPlan& p, int x) { return (p.n_slabs - x + p.nx - 1) / p.nx; }
FG_HD int plan_ld(const CopyPlan& p, int x) { return pmin(plan_ns(p, x), p.lead); }

// Rows of list x's slabs after its lead slabs.
FG_HD int plan_rows(const CopyPlan& p, int x) {
  const int ns = plan_ns(p, x), ld = plan_ld(p, x);
  int r = (ns - ld) * 256;
  if (ns > ld && p.half_last && x + p.nx * (ns - 1) == p.n_slabs - 1) r -= 128;
  return r;
}

// Gathered row of non-lead row rho of list x (rows in slab order).
FG_HD int plan_row(const CopyPlan& p, int x, int rho) {
  const int k = plan_ld(p, x) + rho / 256;
  return 256 * (x + p.nx * k) + rho % 256;
}

FG_HD int plan_groups(const CopyPlan& p, int x) { return (plan_ns(p, x) - plan_ld(p, x) + p.GS - 1) / p.GS; }

// Round (item / per_list) of the first item of non-lead group g.
FG_HD int plan_group_round(const CopyPlan& p, int x, int g) {
  return (plan_ld(p, x) * p.n_tn + g * p.GS * p.n_tn) / p.per_list;
}

// Non-lead rows read by the items of rounds <= r.
FG_HD int plan_need(const CopyPlan& p, int x, int r) {
  const int lim = (r + 1) * p.per_list - plan_ld(p, x) * p.n_tn;   // items of those rounds past the lead
  if (lim <= 0) return 0;
  const int per_group = p.GS * p.n_tn;
  const int cnt = pmin(plan_groups(p, x), (lim + per_group - 1) / per_group);
  const long long rows = (long long)cnt * p.GS * 256;
  return (int)(rows < plan_rows(p, x) ? rows : plan_rows(p, x));
}

// Non-lead rows copied by the items of rounds <= r (C(-1) = 0).
FG_HD int plan_target(const CopyPlan& p, int x, int r) {
  const int R = plan_rows(p, x);
  if (r < 0 || R == 0) return 0;
  const int G = plan_groups(p, x);
  const int span = pmax(1, plan_group_round(p, x, G - 1) - 1);
  const int base = plan_need(p, x, 1);
  const long long u = base + (long long)(R - base) * r / span;
  const int need = plan_need(p, x, r + 1);
  const int c = (int)(u < R ? u : R);
  return pmin(R, pmax(need, c));
}

// Non-lead rows [*c0, *c1) copied by whole item j of list x.
FG_HD void plan_item_rows(const CopyPlan& p, int x, int j, int* c0, int* c1) {
  const int r = j / p.per_list, i = j - r * p.per_list;
  const int lo = plan_target(p, x, r - 1), d = plan_target(p, x, r) - lo;
  *c0 = lo + (int)((long long)d * i / p.per_list);
  *c1 = lo + (int)((long long)d * (i + 1) / p.per_list);
}

// Tile (slab * n_tn + column) of item j of list x: the lead slabs first, slab
// by slab over all columns, then groups of GS slabs x GN columns.
FG_HD int plan_tile(const CopyPlan& p, int x, int j) {
  const int ld = plan_ld(p, x), ns = plan_ns(p, x);
  int k, col;
  if (j < ld * p.n_tn) {
    k = j / p.n_tn;
    col = j - k * p.n_tn;
  } else {
    const int jj = j - ld * p.n_tn;
    const int g = jj / (p.GS * p.n_tn);
    const int gs = pmin(p.GS, ns - ld - g * p.GS);
    const int rr = jj - g * p.GS * p.n_tn;
    const int ng = rr / (gs * p.GN), r2 = rr - ng * gs * p.GN;
    const int si = r2 / p.GN, nn = r2 - si * p.GN;
    k = ld + g * p.GS + si;
    col = ng * p.GN + nn;
  }
  return (x + p.nx * k) * p.n_tn + col;
}

}  // namespace fg
