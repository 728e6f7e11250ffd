// Host-side checks of the projection planner (built and run by
// test_plans.py on the CPU, against the library's own plan functions).
// Every plan the library can launch must satisfy what its kernels assume:
// K slices that cover K, staged activations within the LDS, no more units
// a wave than the kernel template holds, grids within the CU count.  The
// device query fails without a GPU, so the plans are those of 256 CUs.
#include <cstdio>

#include "kernels.h"

using namespace moetail;

namespace {

int fails = 0;
int checked = 0;

#define CHECK(cond, ...)                               \
  do {                                                 \
    if (!(cond)) {                                     \
      ++fails;                                         \
      std::printf("FAIL (%s) ", #cond);                \
      std::printf(__VA_ARGS__);                        \
      std::printf("\n");                               \
    }                                                  \
  } while (0)

int tokens_padded(int b) {
  const int nt = (b + 15) / 16;
  return 16 * (nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : 8);
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

ProjPlan check_plan(int b, int rows, int K, bool always, const ProjTuning& t, const char* what) {
  const ProjPlan p = plan_projection(b, rows, K, always, t);
  ++checked;
  if (!p.splits) return p;  // no slice fits the LDS: the entry point refuses the size
  const int tok = tokens_padded(b);
  const int cu = device_cu_count();
  const int target = t.target_blocks > 0 ? t.target_blocks : cu;
#define CTX "%s b=%d rows=%d K=%d splits=%d kps=%d passes=%d waves=%d bps=%d hold=%d", what, b, \
            rows, K, p.splits, p.k_per_split, p.passes, p.waves, p.blocks_per_slice, p.hold
  CHECK(p.k_per_split > 0 && p.k_per_split % 32 == 0, CTX);
  if (p.stream) {
    // the streamed kernel: activations through the LDS chunk ring (fixed
    // LDS), K ranges that cover K, 6 or 7 consumer waves with an 8-deep
    // ring, one unit a wave
    CHECK(p.lds == 4 * 32 * 1024 + 256, CTX);
    CHECK((p.splits - 1) * p.k_per_split < K && K <= p.splits * p.k_per_split, CTX);
    CHECK(p.blocks_per_slice >= 1 && p.splits * p.blocks_per_slice <= target, CTX);
    CHECK((p.waves == 6 || p.waves == 7) && p.pf == 8 && p.mr == 1 && p.hold == 1, CTX);
    CHECK(ceil_div(rows / 16, p.blocks_per_slice * p.waves) <= 1, CTX);
    CHECK(rows % 16 == 0 && K % 8 == 0, CTX);
    return p;
  }
  CHECK(p.pitch >= p.k_per_split, CTX);
  CHECK(p.lds == (size_t)tok * p.pitch * 2 && p.lds <= 160 * 1024, CTX);
  CHECK(p.blocks_per_slice >= 1, CTX);
  CHECK(p.splits * p.blocks_per_slice <= (target > p.splits ? target : p.splits), CTX);
  const int mr = p.mr > 0 ? p.mr : 1;
  CHECK(rows % (16 * mr) == 0, CTX);
  const int per_wave = ceil_div(rows / (16 * mr), p.blocks_per_slice * p.waves);
  if (p.passes > 1) {
    CHECK(K == p.splits * p.passes * p.k_per_split, CTX);
    CHECK(mr == 1 && (p.waves == 8 || p.waves == 12), CTX);
    CHECK(per_wave <= p.hold && p.hold <= 4, CTX);
    CHECK(!(p.waves == 12 && tok == 64 && p.hold > 1), CTX);
    CHECK(!(tok == 128 && p.hold > 1), CTX);  // 8 token blocks: one unit a wave
    CHECK(p.lds <= 160 * 1024, CTX);
  } else {
    CHECK((p.splits - 1) * p.k_per_split < K && K <= p.splits * p.k_per_split, CTX);
    if (p.hold) CHECK(mr == 1 && p.pf == 8 && p.waves <= 8 && tok <= 64, CTX);
  }
#undef CTX
  return p;
}

// The fused tail's grouped grid of the down (rows H, K = I) and up (rows H,
// K = L) projections, on the plans of their own entry points.
void check_group(int b, int H, int I, int L, const ProjTuning& td, const ProjTuning& tu,
                 bool must_exist, const char* what) {
  const ProjPlan dn = check_plan(b, H, I, false, td, what);
  const ProjPlan up = check_plan(b, H, L, false, tu, what);
  if (!dn.splits || !up.splits) return;
  const GroupPlan g = plan_group(b, dn, H, up, H);
  ++checked;
  const int tok = tokens_padded(b);
#define CTX "%s group b=%d H=%d I=%d L=%d bps=%d/%d waves=%d hold=%d mp=%d", what, b, H, I, L, \
            g.bps0, g.bps1, g.waves, g.hold, g.mp
  if (must_exist) CHECK(g.waves > 0, CTX);
  if (!g.waves) return;
  CHECK(g.bps0 >= 1 && g.bps1 >= 1, CTX);
  const int pw0 = ceil_div(H / 16, g.bps0 * g.waves);
  const int pw1 = ceil_div(H / 16, g.bps1 * g.waves);
  if (g.stream) {
    // both streamed: one grid running each plan's own splits in turn, one
    // unit of each a wave
    CHECK(dn.stream && up.stream && g.waves == dn.waves && g.waves == up.waves, CTX);
    CHECK(g.bps0 == dn.blocks_per_slice && g.bps1 == up.blocks_per_slice && g.hold == 2, CTX);
    CHECK(pw0 <= 1 && pw1 <= 1, CTX);
    CHECK(g.bps0 * dn.splits <= device_cu_count() && g.bps1 * up.splits <= device_cu_count(),
          CTX);
    return;
  }
  CHECK(g.bps0 * dn.splits + g.bps1 * up.splits <= device_cu_count(), CTX);
  if (g.mp) {
    CHECK(dn.passes > 1 || up.passes > 1, CTX);
    CHECK(g.waves == 8 || g.waves == 12, CTX);
    CHECK(pw0 <= g.hold && pw1 <= g.hold && g.hold <= 4, CTX);
    CHECK(!(g.waves == 12 && tok == 64 && g.hold > 1), CTX);
    CHECK(!(tok == 128 && g.hold > 1), CTX);
    // (A single-pass side runs as one pass of its own slices, in units of
    // one tile whatever its plan's tiles per unit: each tile's chain keeps
    // its k order, so the sums are those of its own launch.)
  } else {
    CHECK(dn.passes <= 1 && up.passes <= 1 && (g.waves == 7 || g.waves == 8), CTX);
    if (g.hold) CHECK(tok <= 64 && pw0 <= 4 && pw1 <= 4, CTX);
  }
#undef CTX
}

}  // namespace

int main() {
  const ProjTuning dflt{0, 0, 0, 0, 0, 0};
  // Tuning overrides (MOETAIL_<KIND>_* in the library), including ones that
  // cannot fit and fall back.
  const ProjTuning over[] = {
      {2, 7, 0, 0, 0, 0},  {8, 16, 0, 0, 0, 0}, {2, 4, 0, 2, 4, 0},  {8, 8, 0, 2, 8, 0},
      {2, 8, 100, 0, 0, 0}, {8, 14, 37, 0, 0, 0}, {1, 0, 0, 0, 0, 0}, {0, 0, 0, 0, 0, 1},
      {0, 0, 0, 0, 0, 2},  {0, 0, 64, 0, 0, 2}, {0, 0, 64, 0, 0, 4}, {1, 0, 0, 0, 0, 2},
      {0, 8, 64, 0, 0, 2}, {0, 0, 16, 0, 0, 2}, {0, 0, 4, 0, 0, 2},  {0, 12, 8, 0, 0, 2},
      {3, 0, 0, 0, 0, 0},  {0, 0, 8, 0, 0, 4},  {0, 12, 0, 0, 0, 2}, {5, 0, 0, 0, 0, 2}};
  struct Shape {
    int rows, K;
    bool always;
  };
  const Shape shapes[] = {{12288, 7168, true}, {7168, 6144, false}, {7168, 3584, false},
                          {512, 3584, false},  {2048, 1024, true},  {1024, 1024, false},
                          {640, 512, true},    {512, 320, false},   {512, 1024, false},
                          {384, 512, true},    {256, 128, false},   {128, 64, true}};
  const int bs[] = {1, 2, 5, 8, 15, 16, 17, 31, 32, 33, 40, 48, 63, 64, 65, 100, 127, 128};
  for (int b : bs) {
    for (const Shape& s : shapes) {
      check_plan(b, s.rows, s.K, s.always, dflt, "default");
      for (const ProjTuning& t : over) check_plan(b, s.rows, s.K, s.always, t, "override");
    }
    // the tail's real shapes: a grouped plan must exist at every size up to
    // 64 tokens (above, the down and up projections may run as two launches)
    check_group(b, 7168, 6144, 3584, dflt, dflt, true, "tail");
    check_group(b, 512, 320, 1024, dflt, dflt, b <= 64, "tail small");
    check_group(b, 512, 128, 544, dflt, dflt, b <= 64, "tail ragged");
    for (const ProjTuning& td : over)
      for (const ProjTuning& tu : over) check_group(b, 512, 320, 1024, td, tu, false, "tail override");
  }
  std::printf("checked %d plans, %d failures\n", checked, fails);
  return fails ? 1 : 0;
}
