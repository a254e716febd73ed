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

long long bwd_split_part_floats(int B, int Hq, int Hkv, long long Nk, int D, const BwdSplit& s) {
  return s.rkv > 1 ? 2LL * s.rkv * B * Hq * Nk * D : bwd_part_floats(B, Hq, Hkv, Nk, D);
}

long long bwd_split_dq_floats(int B, int Hq, long long Nq, int D, const BwdSplit& s) {
  return s.rq > 1 ? (long long)s.rq * B * Hq * Nq * D : 0;
}

// A backward whose dK/dV grid (one workgroup per 128 keys and query head)
// leaves compute units idle is limited by its longest workgroups: the first
// key tile walks every query tile, the last query tile every key tile.  Cut
// into ranges, every workgroup of either pass does at most about the work of
// 1024 query rows x 128 keys at D = 64: the dK/dV pass takes query ranges of
// 1024 * 64 / D rows, the dQ pass key ranges of 512 * 64 / D keys (its
// workgroups hold 256 query rows).  At most 8 ranges a pass, and their fp32
// partials within 64 MiB.  (Measured on the glossary example's backward
// [1, 4, 4096, 64]: 4 and 8 ranges 95 us against 121 us unsplit, fewer ranges
// 97-128 us; [1, 8, 1024, 128]: 2 and 4 ranges 58 us against 77 us.)
BwdSplit bwd_split_plan(int B, int Hq, int Hkv, long long Nq, long long Nk, int D) {
  const long long wkv = (long long)B * Hq * ((Nk + 127) / 128);
  if (wkv >= 256 || Hq % Hkv) return BwdSplit{};
  const long long nqt = (Nq + 63) / 64, nkt = (Nk + 63) / 64;
  long long rkv = std::min<long long>(8, (nqt + 16 * 64 / D - 1) / (16 * 64 / D));
  long long rq = std::min<long long>(8, (nkt + 8 * 64 / D - 1) / (8 * 64 / D));
  for (;;) {
    BwdSplit t;
    t.qst = (int)((nqt + rkv - 1) / rkv);
    t.rkv = (int)((nqt + t.qst - 1) / t.qst);
    t.kst = (int)((nkt + rq - 1) / rq);
    t.rq = (int)((nkt + t.kst - 1) / t.kst);
    if (t.rkv == 1) t.qst = 1 << 30;
    if (t.rq == 1) t.kst = 1 << 30;
    const long long extra = (t.rkv > 1 ? 2LL * t.rkv * B * Hq * Nk * D : 0) + bwd_split_dq_floats(B, Hq, Nq, D, t);
    if (extra * 4 <= (64LL << 20)) return t;
    if (rkv == 1 && rq == 1) return BwdSplit{};
    if (rkv >= rq) --rkv; else --rq;
  }
}

long long bwd_workspace_bytes(int B, int Hq, int Hkv, long long Nq, long long Nk, int D) {
  const BwdSplit s = bwd_split_plan(B, Hq, Hkv, Nq, Nk, D);
  return (bwd_delta_floats(B, Hq, Nq) + bwd_split_part_floats(B, Hq, Hkv, Nk, D, s) +
          bwd_split_dq_floats(B, Hq, Nq, D, s)) * 4;
}

long long bwd_ds_head_elems(long long N, int causal) {
  const long long nqt = (N + 63) / 64, nkt2 = (N + 127) / 128 * 2;
  return bwd_ds_row_start(nqt, causal, nkt2) * kDsBlockElems;
}

long long bwd_ds_offset_bytes(int B, int Hq, int Hkv, long long N, int D) {
  return (bwd_workspace_bytes(B, Hq, Hkv, N, N, D) + 255) / 256 * 256;
}

long long bwd_ds_workspace_bytes(int B, int Hq, int Hkv, long long N, int D, int causal) {
  // a dK/dV grid below one workgroup per compute unit (the small problems
  // whose passes are split and run side by side) keeps the dQ pass
  if ((long long)B * Hq * ((N + 127) / 128) < 256) return 0;
  return bwd_ds_offset_bytes(B, Hq, Hkv, N, D) + 2LL * B * Hq * bwd_ds_head_elems(N, causal);
}

long long bwd_block_ds_head_elems(long long Nq, long long Nk) {
  return (Nq + 63) / 64 * ((Nk + 127) / 128 * 2) * kDsBlockElems;
}

long long bwd_block_ds_offset_bytes(int B, int Hq, int Hkv, long long Nk, int D) {
  return (bwd_part_floats(B, Hq, Hkv, Nk, D) * 4 + 255) / 256 * 256;
}

long long bwd_block_ds_workspace_bytes(int B, int Hq, int Hkv, long long Nq, long long Nk, int D) {
  if ((long long)B * Hq * ((Nk + 127) / 128) < 256) return 0;
  return bwd_block_ds_offset_bytes(B, Hq, Hkv, Nk, D) + 2LL * B * Hq * bwd_block_ds_head_elems(Nq, Nk);
}

int fwd_split_count(int B, int Hq, int Hkv, long long Nq, long long Nk, int causal, int n_splits) {
  if (n_splits > 0) return n_splits;
  const int G = Hq / Hkv;
  const int HP = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  const long long span = (kFwdWaves / HP) * 32;
  const long long wgs = (Nq + span - 1) / span * (Hq / HP) * B;
  const long long tiles = (Nk + kFwdKeyTile - 1) / kFwdKeyTile;
  // about one and a half workgroups per compute unit, ranges of at least 16
  // key tiles (measured on the split forward before its grid held only the
  // pairs with work: 4K tokens x 4 heads fastest with 4 ranges, 16K x 4 query
  // heads on one KV head with 2, 32K x 4 heads unsplit; a zigzag ring step of
  // two 4096-token chunk calls fastest with the 3 it gives)
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
