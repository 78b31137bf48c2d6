// Host-side check of the balanced schedule's unit arithmetic (common.h):
// for seeded random launches (heads, key tiles per head, query tiles, segment
// cost, workgroups), every real unit is owned by exactly the workgroup whose
// range covers it, the virtual <-> real maps are consistent and monotone, and
// no workgroup range is empty.  Prints "ok N" with the number of launches
// checked, or the first failure, and exits non-zero on a failure.
#include <cstdio>
#include <cstdlib>
#include <random>

#include "common.h"

using namespace chunkattn;

static int fail(const char* what, int cfg, int a, int b) {
  std::printf("FAIL %s (launch %d: %d, %d)\n", what, cfg, a, b);
  return 1;
}

int main() {
  std::mt19937 rng(1234);
  static AttnParams p;
  int checked = 0;
  for (int cfg = 0; cfg < 400; ++cfg) {
    const int nh = 1 + (int)(rng() % (cfg % 4 == 0 ? 256 : 12));
    const int maxt = cfg % 3 == 0 ? 8 : 600;
    p.n_heads = nh;
    p.n_qtiles = 1 + (int)(rng() % 24);
    p.seg_cost = (int[]){0, 1, 8, 13}[rng() % 4];
    p.tprefix[0] = 0;
    for (int i = 0; i < nh; ++i) p.tprefix[i + 1] = p.tprefix[i] + 1 + (int)(rng() % maxt);
    p.n_units = p.n_qtiles * p.tprefix[nh];
    p.n_vunits = p.n_units + p.n_qtiles * nh * p.seg_cost;
    // the host's bound on the workgroup count
    int gmax = 256;
    if (p.n_units / 8 < gmax) gmax = p.n_units / 8;
    if (p.n_vunits / (p.seg_cost + 1) < gmax) gmax = p.n_vunits / (p.seg_cost + 1);
    if (gmax < 1) continue;
    p.n_wgs = 1 + (int)(rng() % gmax);
    if (p.n_units > 3000000) continue;
    // virtual -> real: endpoints, monotone, real(virtual(u)) = u
    if (sched_real(p, 0) != 0) return fail("real(0)", cfg, sched_real(p, 0), 0);
    if (sched_real(p, p.n_vunits) != p.n_units) return fail("real(end)", cfg, sched_real(p, p.n_vunits), p.n_units);
    int prev = 0;
    for (int v = 0; v < p.n_vunits; ++v) {
      const int r = sched_real(p, v);
      if (r < prev || r > p.n_units) return fail("monotone", cfg, v, r);
      prev = r;
    }
    int vprev = -1;
    for (int u = 0; u < p.n_units; ++u) {
      const int v = sched_virtual(p, u);
      if (v <= vprev || v >= p.n_vunits) return fail("virtual increasing", cfg, u, v);
      vprev = v;
      if (sched_real(p, v) != u) return fail("real(virtual(u)) = u", cfg, u, v);
      // real(v') <= u exactly for v' <= virtual(u)
      if (sched_real(p, v + 1) != u + 1) return fail("real(virtual(u) + 1) = u + 1", cfg, u, v);
    }
    // ranges: non-empty, contiguous, covering; the owner of u covers it
    for (int g = 0; g < p.n_wgs; ++g) {
      const int a = sched_real(p, unit_begin(g, p.n_vunits, p.n_wgs));
      const int b = sched_real(p, unit_begin(g + 1, p.n_vunits, p.n_wgs));
      if (b <= a) return fail("empty range", cfg, g, a);
      for (int u = a; u < b; u += 1 + (b - a) / 64) {
        if (g_of_unit(sched_virtual(p, u), p.n_vunits, p.n_wgs) != g) return fail("owner", cfg, u, g);
      }
      if (g_of_unit(sched_virtual(p, b - 1), p.n_vunits, p.n_wgs) != g) return fail("owner of last", cfg, b - 1, g);
    }
    ++checked;
  }
  if (checked < 200) return fail("too few launches checked", checked, 0, 0);
  std::printf("ok %d\n", checked);
  return 0;
}
