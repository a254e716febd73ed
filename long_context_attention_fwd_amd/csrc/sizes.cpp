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

}  // namespace lcattn
