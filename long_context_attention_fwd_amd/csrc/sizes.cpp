// sizes.cpp -- host-only sizing rules of the launchers: workspace layouts of
// the backward and the number of key ranges of the split-KV forward.  Kept
// apart from the kernels so that the argument-validation layer (api.cpp)
// also builds and runs without device code (the host sanitizer build).
#include <algorithm>

#include "launch.hpp"

namespace lcattn {

long long bwd_delta_floats(int B, int Hq, long long Nq) {
  // Dv rows, padded to a multiple of 64 floats (256 bytes)
  return ((long long)B * Hq * Nq + 63) / 64 * 64;
}

long long bwd_part_floats(int B, int Hq, int Hkv, long long Nk, int D) {
  return Hq != Hkv ? 2LL * B * Hq * Nk * D : 0;  // per-query-head dK, dV partials
}

long long bwd_workspace_bytes(int B, int Hq, int Hkv, long long Nq, long long Nk, int D) {
  return (bwd_delta_floats(B, Hq, Nq) + bwd_part_floats(B, Hq, Hkv, Nk, D)) * 4;
}

int fwd_split_count(int B, int Hq, int Hkv, long long Nq, long long Nk, int causal, int n_splits) {
  if (n_splits > 0) return n_splits;
  const int G = Hq / Hkv;
  const int HP = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  const long long span = (kFwdWaves / HP) * 32;
  const long long wgs = (Nq + span - 1) / span * (Hq / HP) * B;
  const long long tiles = (Nk + kFwdKeyTile - 1) / kFwdKeyTile;
  // about one and a half workgroups per compute unit, ranges of at least 16
  // key tiles (measured: 4K tokens x 4 heads run fastest with 4 ranges, 16K x
  // 4 query heads on one KV head with 2, 32K x 4 heads unsplit)
  long long n = (384 + wgs - 1) / wgs;
  n = std::min<long long>(n, std::max<long long>(1, tiles / 16));
  (void)causal;
  return (int)std::max<long long>(1, std::min<long long>(n, 64));
}

// Query tiles of `span` rows that see at least one key of key range r (key
// tiles [r * st, (r + 1) * st) of 64 keys): tile qt sees keys below
// kv_end(qt) = min(Nk, max(0, dpos + last row of qt + 1)) when causal, all Nk
// otherwise; kv_end grows with qt, so those tiles are qt >= q0(r) and the
// count is n_qt - q0(r).  The forward kernel decodes its compact grid with
// the same rule.
long long splitkv_range_tiles(long long Nq, long long Nk, long long dpos, int causal, int span, int st, int r) {
  const long long n_qt = (Nq + span - 1) / span;
  const long long x = (long long)r * st * 64;  // first key of the range
  if (x >= Nk) return 0;
  if (!causal) return n_qt;
  const long long y = x - dpos;  // a tile has work iff its last row >= y
  if (y <= 0) return n_qt;
  if (y + 1 > Nq) return 0;
  return n_qt - ((y + span) / span - 1);
}

long long splitkv_pairs(long long Nq, long long Nk, long long dpos, int causal, int span, int n_splits) {
  const long long tiles = (Nk + 63) / 64;
  const int st = (int)((tiles + n_splits - 1) / n_splits);
  long long total = 0;
  for (int r = 0; r < n_splits; ++r) total += splitkv_range_tiles(Nq, Nk, dpos, causal, span, st, r);
  return total;
}

int splitkv_split_count(int B, int Hq, int Hkv, long long Nq, long long Nk, int causal, int n_splits) {
  if (n_splits > 0) return n_splits;
  const int G = Hq / Hkv;
  const int HP = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  const int span = (kFwdWaves / HP) * 32;
  const long long layers = (long long)(Hq / HP) * B;
  const long long tiles = (Nk + 63) / 64;
  // unsplit, enough workgroups for the GPU already
  if ((Nq + span - 1) / span * layers >= 384) return 1;
  // the most ranges whose workgroups with work still get a compute unit each
  // (the launch is the compact grid of those workgroups; 256 compute units)
  int best = 1;
  for (int n = 2; n <= std::min<long long>(64, tiles); ++n)
    if (splitkv_pairs(Nq, Nk, 0, causal, span, n) * layers <= 256) best = n;
  return best;
}

}  // namespace lcattn
