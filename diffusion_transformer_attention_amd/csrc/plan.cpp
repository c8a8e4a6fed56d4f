// Host-side work plan of the balanced forward (dit_attn_fwd_balanced): which
// query tiles run whole and how the rest are cut into key chunks.  Pure
// arithmetic on the sizes; the launches are in attn_bf16.hip.
#include "launch.h"

namespace ditattn {

BalancedPlan balanced_plan(int B, int H, int Nq, int Nkv, int D, int slots) {
  // Costs in key-tile steps of one workgroup (64 keys x 256 rows): a
  // workgroup's fixed cost (query load, epilogue, the gap before the next) is
  // about 6 steps; an extra launch about 6; HBM moves ~8 MB per step at
  // D = 128 (the step shrinks with D).
  constexpr double kFixed = 6.0, kLaunch = 6.0, kStepBytes = 8.0e6;
  BalancedPlan pl{};
  const int n_qtiles = (Nq + kFwdQueryTile - 1) / kFwdQueryTile;
  const int64_t total = (int64_t)B * H * n_qtiles;
  const int nt = (Nkv + kFwdKeyTile - 1) / kFwdKeyTile;
  pl.whole = (int)(total > 0x7fffffff ? 0x7fffffff : total);  // the plain launch rejects more
  pl.nsplit = 1;
  if (slots < 1 || total < 1 || total > 0x7fffffff || nt < 2) return pl;
  const int64_t whole = total / slots * slots, R = total - whole;
  if (R == 0) return pl;
  const double step_bytes = kStepBytes * D / 128.0;
  auto cost = [&](int per, int s) {  // per key tiles per chunk, s chunks
    const double waves = (double)((R * s + slots - 1) / slots);
    double t = waves * (kFixed + per);
    if (s > 1) t += 2 * kLaunch + (double)R * kFwdQueryTile * s * (D + 1) * 4.0 * 2.0 / step_bytes;
    return t;
  };
  const double c1 = cost(nt, 1);
  double best = c1;
  for (int s0 = 2; s0 <= 32 && s0 <= nt; ++s0) {
    const int per = (nt + s0 - 1) / s0, s = (nt + per - 1) / per;
    const double t = cost(per, s);
    if (t < best - 1e-9) {
      best = t;
      pl.nsplit = s;
      pl.kc = per * kFwdKeyTile;
    }
  }
  if (pl.nsplit == 1 || best > 0.97 * c1) {
    pl.nsplit = 1;
    pl.kc = 0;
    return pl;
  }
  pl.whole = (int)whole;
  pl.row0 = (whole / n_qtiles) * (int64_t)Nq + (whole % n_qtiles) * (int64_t)kFwdQueryTile;
  pl.rows = (int64_t)B * H * Nq - pl.row0;
  pl.units = (int)(R * pl.nsplit);
  pl.ws_bytes = (size_t)pl.nsplit * pl.rows * (D + 1) * sizeof(float);
  return pl;
}

}  // namespace ditattn
