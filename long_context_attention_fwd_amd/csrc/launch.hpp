// launch.hpp -- host-side launchers of the gfx950 kernels (internal to the library).
//
// Each launcher assumes its arguments were validated by api.cpp: pointers are
// device pointers, aligned, sized and non-overlapping as the public header
// states, and every size fits the index arithmetic of the kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcattn {

// out[a * rep + i, b, :] = in[b, a, :] (i < rep), rows of row_bytes (a
// power-of-two multiple of 16), for up to kMaxRelayoutBatch tensors with rows
// of one size, in one launch.
constexpr int kMaxRelayoutBatch = 8;
struct TransposeJob {
  const void* in;
  void* out;
  unsigned A, Bn, rep;
};
// a_fast: a-tiles fastest in the workgroup order (else b-tiles fastest)
hipError_t launch_transpose_rows_batch(const TransposeJob* jobs, int n, unsigned row_bytes, bool a_fast,
                                       hipStream_t stream);
// out[b, a, :] = sum over i < rep of in[a * rep + i, b, :] (bf16 out)
hipError_t launch_sum_replicas(const void* in, bool in_f32, uint16_t* out, long long A, long long Bn, int D, int rep,
                               hipStream_t stream);

// forward kernel geometry (shared by the launcher and the split-count heuristic)
constexpr int kFwdWaves = 8;     // waves per workgroup
constexpr int kFwdKeyTile = 64;  // keys per tile
constexpr int kBwdDqWaves = 8;   // waves per workgroup of the backward's dQ pass (32 query rows each)

// The attention kernels number their workgroups in 32 bits: a launch whose
// grid has 2^31 or more workgroups is refused (hipErrorInvalidConfiguration).
inline bool grid_fits(const dim3& g) { return (unsigned long long)g.x * g.y * g.z < (1ull << 31); }

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int Hq, Hkv, G;
  long long Nq, Nk;
  float scale_log2;  // softmax scale times log2(e)
  int causal;
  long long q_pos0, k_pos0;
  // split of the keys: workgroup z = s * B + b covers key tiles
  // [s * split_tiles, (s + 1) * split_tiles) and writes part s of o / lse,
  // part_stride elements apart in o (part_stride / D in lse)
  int n_splits = 1;
  int split_tiles = 1 << 30;
  long long part_stride = 0;
  int B = 1;  // batch (grid z = split * B + batch)
  // element strides (batch, head, token) of q, of k and v, and of o; the
  // head dimension is contiguous.  Zero: contiguous [B, H, N, D].
  long long qs[3] = {0, 0, 0}, ks[3] = {0, 0, 0}, os[3] = {0, 0, 0};
  // fp32 output only: accum != 0 merges this call's result into the running
  // (o, lse) already there (log-sum-exp rule) instead of overwriting them;
  // o_final, if set, also receives the (merged) O rounded to bf16,
  // contiguous [B, Hq, Nq, D]
  int accum = 0;
  uint16_t* o_final = nullptr;
  // split forward: grid x enumerates only the (key range, query tile) pairs
  // with work (range-major, longest query tiles first within a range)
  int compact = 0;
};

// (strides left at zero are filled in for contiguous [B, H, N, D] tensors)
hipError_t launch_attn_fwd(const FwdArgs& a, int B, int D, bool out_f32, hipStream_t stream);
// Up to kMaxFwdGroup independent fp32-output calls (contiguous tensors, the
// same B, Hq, Hkv, D, scale and mask kind) in one launch.
constexpr int kMaxFwdGroup = 4;
hipError_t launch_attn_fwd_group(const FwdArgs* calls, int n, int B, int D, hipStream_t stream);
// The same calls with each call's keys cut into `splits` ranges computed side
// by side: fp32 partials of call c in parts[c] ([splits, B, Hq, Nq, D] O,
// then [splits, B, Hq, Nq] LSE), then one merge per call of its partials and
// its running result (o, lse of calls[c], merged unless accum == 0) into that
// running result, and o_final.
hipError_t launch_attn_fwd_group_split(const FwdArgs* calls, float* const* parts, int n, int B, int D, int splits,
                                       hipStream_t stream);

// Forward over n_splits key ranges side by side (fp32 partials in o_parts /
// lse_parts, [n_splits, B, Hq, Nq(, D)]), then their LSE merge into o (bf16)
// and lse.
hipError_t launch_attn_fwd_splitkv(const FwdArgs& a, int B, int D, int n_splits, float* o_parts, float* lse_parts,
                                   hipStream_t stream);
// Number of key ranges for a ring step's grouped accumulate calls
// (attn_fwd_split_suggest, whose grid is not compacted): n_splits if > 0,
// else about one and a half workgroups per compute unit with ranges of at
// least 16 key tiles.
int fwd_split_count(int B, int Hq, int Hkv, long long Nq, long long Nk, int causal, int n_splits);
// attn_fwd_splitkv's ranges: n_splits if > 0; else 1 when the unsplit grid
// fills the GPU, otherwise the most ranges whose (range, query tile) pairs
// with work fit one workgroup per compute unit
int splitkv_split_count(int B, int Hq, int Hkv, long long Nq, long long Nk, int causal, int n_splits);
// (range, query tile) pairs with work of the split forward (n_splits ranges
// of whole key tiles; query tiles of `span` rows; dpos = q_pos0 - k_pos0)
long long splitkv_pairs(long long Nq, long long Nk, long long dpos, int causal, int span, int n_splits);

// Geometry of the split forward's partials: a query tile of `span` rows
// (row i of the Nq rows of a head lies in tile i / span) has a partial for
// every key range that starts before its last visible key, ranges being
// split_tiles tiles of key_tile keys; the ranges after it wrote nothing.
struct MergeSplits {
  int span = 0;
  int split_tiles = 0;
  int key_tile = 0;
  long long Nq = 0, Nk = 0;
  long long dpos = 0;  // q_pos0 - k_pos0
  int causal = 0;
};

// o[row] = LSE merge of the n_parts partials of each row; with `splits`, a
// row reads only the partials its query tile has (fewer than n_parts when
// its keys end early)
hipError_t launch_partial_merge(const void* o_parts, bool parts_f32, const float* lse_parts, int n_parts,
                                uint16_t* o, float* lse, long long rows, int D, hipStream_t stream,
                                const MergeSplits* splits = nullptr);
// fp32 partials of the split forward (geometry sp) merged into a running
// fp32 result o_run, lse_run (which counts as one more part unless first);
// o_final (optional) receives the merged O in bf16
hipError_t launch_merge_into(const float* o_parts, const float* lse_parts, int n_parts, const MergeSplits& sp,
                             float* o_run, float* lse_run, bool first, uint16_t* o_final, long long rows, int D,
                             hipStream_t stream);

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* d_o;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  // <dO_i, O_i> per query row (fp32): written by the launch first when o is
  // set, else given
  float* delta;
  float* part;  // grouped-query attention: per-query-head fp32 dK, dV partials
  int Hq, Hkv, G;
  long long Nq, Nk;  // query rows; keys (the whole sequence, or one KV block)
  float scale;
  int causal;
  // q_pos0 - k_pos0: key j is visible to query i iff j <= i + dpos (causal);
  // clamped to [-Nq, Nk], which keeps every mask sum in the int range for
  // Nq, Nk < 2^30
  int dpos = 0;
  // dQ output: 0 -> bf16 dq only; 1 -> fp32 dq_acc overwritten; 2 -> added
  // into dq_acc (a ring over KV blocks); with 1 and 2, dq (bf16) also
  // receives the accumulated value if set
  int dq_mode = 0;
  float* dq_acc = nullptr;
  // dK, dV output, the same three modes on dk_acc / dv_acc (fp32) with dk, dv
  // (bf16) optional when set
  int dkv_mode = 0;
  float* dk_acc = nullptr;
  float* dv_acc = nullptr;
  // element strides (batch, head, token) of q, o, d_o and dq (qs) and of k,
  // v, dk and dv (ks); the head dimension is contiguous.  Zero: contiguous
  // [B, H, N, D].  lse, the delta, the fp32 accumulators and the workspace
  // are always contiguous.
  long long qs[3] = {0, 0, 0}, ks[3] = {0, 0, 0};
  // Split passes (filled in by the launcher from a BwdSplit): the dK/dV pass
  // over rkv ranges of qst 64-row query tiles, its fp32 partials at part
  // ([rkv, B, Hq, Nk, D] for dK, then the same for dV) when rkv > 1 or the
  // heads are grouped; the dQ pass over rq ranges of kst 64-key tiles, its
  // fp32 partials (scaled) at dq_part ([rq, B, Hq, Nq, D]) when rq > 1.  A
  // range that no query (key) of a workgroup's tile sees writes nothing.
  int B = 1;
  int rkv = 1, qst = 1 << 30;
  int rq = 1, kst = 1 << 30;
  float* dq_part = nullptr;
  // dQ as a product of stored dS (attn_bwd given the larger workspace): the
  // dK/dV pass also writes dS^T in blocks (layout at bwd_ds_row_start) at ds,
  // ds_head elements per (batch, query head), and a product pass forms
  // dQ = scale dS K from them; null: the dQ pass recomputes S and dP
  uint16_t* ds = nullptr;
  long long ds_head = 0;
  // 1: every query tile's row of blocks has the same length (nkt2; block
  // calls, whose offsets make the compact causal rows irregular)
  int ds_uniform = 0;
};

// Stored dS: per (batch, query head), dS^T in blocks of 64 keys x 64 query
// rows (bf16, row-major [key][query], kDsBlockElems elements).  Query tile qt
// (rows 64 qt ..) has a row of blocks for key tiles [0, len(qt)): causal
// (Nq = Nk, no offset), len = 2 (qt / 2) + 2, the key-tile pairs of the dK/dV
// workgroups that see the tile; otherwise every key tile, rounded up to pairs
// (nkt2).  Rows follow one another: row qt starts at block bwd_ds_row_start.
constexpr long long kDsBlockElems = 64 * 64;
constexpr long long bwd_ds_row_start(long long qt, int causal, long long nkt2) {
  return causal ? 2 * (qt >> 1) * ((qt >> 1) + 1) + (qt & 1) * (2 * (qt >> 1) + 2) : qt * nkt2;
}

// How a small backward problem splits its passes (one per call shape): the
// dK/dV pass over rkv query ranges of qst 64-row tiles, the dQ pass over rq
// key ranges of kst 64-key tiles; 1: not split.
struct BwdSplit {
  int rkv = 1, qst = 1 << 30;
  int rq = 1, kst = 1 << 30;
};
BwdSplit bwd_split_plan(int B, int Hq, int Hkv, long long Nq, long long Nk, int D);

// Backward workspace: Dv per query row (fp32, padded to 64 floats), then, for
// grouped-query attention (Hq != Hkv), per-query-head fp32 partials of dK and
// dV ([B, Hq, Nk, D] each).  bwd_workspace_bytes is that of attn_bwd, whose
// split plan (bwd_split_plan) also holds rkv partials of dK and dV and rq of
// dQ: Dv | dK, dV partials (bwd_split_part_floats) | dQ partials.
long long bwd_delta_floats(int B, int Hq, long long Nq);
long long bwd_part_floats(int B, int Hq, int Hkv, long long Nk, int D);
long long bwd_split_part_floats(int B, int Hq, int Hkv, long long Nk, int D, const BwdSplit& s);
long long bwd_split_dq_floats(int B, int Hq, long long Nq, int D, const BwdSplit& s);
long long bwd_workspace_bytes(int B, int Hq, int Hkv, long long Nq, long long Nk, int D);
// attn_bwd's workspace with room for stored dS: the workspace above, padded
// to 256 bytes (bwd_ds_offset_bytes, where the blocks start), then the blocks
// (bwd_ds_head_elems per batch and query head).  0 for small problems (a
// dK/dV grid below 256 workgroups), which keep the recomputing dQ pass
// beside the dK/dV pass.
long long bwd_ds_head_elems(long long N, int causal);
long long bwd_ds_offset_bytes(int B, int Hq, int Hkv, long long N, int D);
long long bwd_ds_workspace_bytes(int B, int Hq, int Hkv, long long N, int D, int causal);
// A block call's workspace with room for stored dS: its grouped-query
// partials padded to 256 bytes, then uniform rows (nqt x nkt2 blocks per
// batch and query head); 0 below 256 dK/dV workgroups.
long long bwd_block_ds_head_elems(long long Nq, long long Nk);
long long bwd_block_ds_offset_bytes(int B, int Hq, int Hkv, long long Nk, int D);
long long bwd_block_ds_workspace_bytes(int B, int Hq, int Hkv, long long Nq, long long Nk, int D);

// allow_side: a problem whose dK/dV grid has fewer than two workgroups per
// compute unit runs its dQ pass on the library's side stream of the device
// (forked from and joined back into `stream`); false keeps every launch on
// `stream` and creates nothing (the allocation-free entry point)
// split: run the passes as bwd_split_plan says (a.part, a.dq_part then point
// at its partials; attn_bwd and its strided and allocation-free forms); else
// unsplit (block calls, whose workspace holds the grouped-query partials only)
hipError_t launch_attn_bwd(const BwdArgs& a, int B, int D, hipStream_t stream, bool allow_side, bool split);
// Up to kMaxBwdGroup independent block-backward calls (contiguous tensors, Dv
// given, the same B, Hq, Hkv, D, scale and mask kind): one dK/dV launch and
// one dQ launch for all of them.
constexpr int kMaxBwdGroup = 4;
hipError_t launch_attn_bwd_group(const BwdArgs* calls, int n, int B, int D, hipStream_t stream);

// The allocation-free backward's scratch: kNoAllocScratchBytes of device
// memory per GPU, held by the library until the process ends.  *ptr receives
// the device address of the copy on the GPU that `stream` belongs to (looked
// up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(160) << 20;
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);
// Dv_i = <dO_i, O_i> for rows query rows of width D
hipError_t launch_bwd_delta(const uint16_t* o, const uint16_t* d_o, float* delta, long long rows, int D,
                            hipStream_t stream);

}  // namespace lcattn
