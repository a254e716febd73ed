/*
 * attn.h -- C ABI of the MI355X (gfx950) long-context causal attention library.
 *
 * What it computes.  Exact scaled-dot-product attention with a causal mask,
 * O = softmax(scale * Q K^T + mask) V, plus the per-row log-sum-exp (natural
 * log) of the scaled, masked scores.  This is the call the example program on
 * the "Context Parallelism" glossary page (Ultralytics, German edition,
 * section "Praktische Anwendung und Kompromisse") makes on [batch, heads,
 * sequence, head_dim] bf16 tensors with the causal flag set, followed by a
 * backward pass of a loss of the output.  The ring form (partial attention
 * against one KV block, then a combine that equals full attention) is from the
 * same page, section "So funktioniert Kontextparallelität"; the sequence-to-
 * head exchange is the Ulysses all-to-all of "Million-Token-Kontexte im
 * Training ..." (section "Ulysses: Die Sequenz als Verteilungseinheit") and of
 * "Ulysses Sequence Parallelism: как тренировать модели с контекстом в миллион
 * токенов" (section "Как работает Ulysses: технические детали"), carried out on
 * one GPU.
 *
 * Conventions shared by every entry point.
 *  - Pointers are device pointers (hipMalloc / torch CUDA tensors), 16-byte
 *    aligned, all tensors contiguous row-major in the layouts stated below.
 *  - bf16 tensors hold raw bfloat16 words; LSE and fp32 tensors hold float.
 *  - Ownership: the caller owns every buffer, including the backward
 *    workspace.  The library allocates and frees no device memory.  Its global
 *    state: a thread-local error text, the records of the optional
 *    measurement hook below, the per-GPU address of attn_bwd_noalloc's scratch
 *    array, and the backward's side streams (one with two events per caller
 *    stream, for up to 64 caller streams; see attn_bwd), all created at first
 *    use and kept until the process ends.
 *  - Asynchrony: each call validates its arguments on the host, then enqueues
 *    its kernels on `hip_stream` (a hipStream_t; NULL = the default stream)
 *    and returns.  Work a call puts on the side stream is forked from and
 *    joined back into `hip_stream` with events, so everything a call does is
 *    ordered on `hip_stream`.  A validation failure returns a nonzero status
 *    before anything is launched and leaves the outputs untouched.  A launch
 *    failure returns ATTN_ERR_HIP.  Faults inside kernels surface at the
 *    caller's next synchronisation.
 *  - Every element of every output is written, including masked rows.
 *  - Inputs and outputs must not overlap.
 */
#ifndef LCATTN_ATTN_H
#define LCATTN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size is <= 0 or sizes are inconsistent */
  ATTN_ERR_UNSUPPORTED = 3, /* valid but not implemented (e.g. D not 64/128) */
  ATTN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  ATTN_ERR_ALIAS = 5,       /* an output overlaps an input */
  ATTN_ERR_WORKSPACE = 6,   /* workspace missing or too small */
  ATTN_ERR_HIP = 7          /* the HIP runtime reported an error */
};

enum { ATTN_BF16 = 0, ATTN_FP32 = 1 };

/*
 * attn_fwd -- fused causal attention forward with per-row log-sum-exp.
 *
 * q    [B, Hq,  Nq, D] bf16       k, v [B, Hkv, Nk, D] bf16
 * o    [B, Hq,  Nq, D] bf16 (o_dtype = ATTN_BF16) or float (ATTN_FP32)
 * lse  [B, Hq,  Nq]    float, natural log of sum_j exp(S_ij)
 *
 * S_ij = scale * <q_i, k_j>.  With causal != 0, key j is visible to query i
 * iff k_pos0 + j <= q_pos0 + i (global token positions), so a call with a KV
 * sub-range and its offsets is one ring step's partial attention.  Query head
 * h reads key/value head h / (Hq / Hkv) (grouped-query attention).  A row
 * with no visible key gets o = 0 and lse = -inf.  fp32 o keeps partial results
 * unrounded for attn_partial_merge.
 *
 * Requires B, Hq, Hkv, Nq, Nk >= 1; Hkv divides Hq; D in {64, 128};
 * q_pos0, k_pos0 >= 0; scale finite.  Deterministic: repeated calls give
 * bit-identical outputs.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
             int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D, float scale, int causal,
             int64_t q_pos0, int64_t k_pos0, void* hip_stream);

/*
 * attn_fwd_strided -- attn_fwd on tensors given by element strides, so that
 * attention can read a Ulysses shard in the token-major layout the exchange
 * delivers ([N, H, D] rows: token stride H*D, head stride D) and write O the
 * same way, without a separate relayout pass.
 *
 * q_strides, kv_strides, o_strides: host arrays of 3 element strides (batch,
 * head, token) of q, of k and v (shared), and of o; the D elements of a row
 * are contiguous.  Every stride keeps rows 16-byte aligned (a multiple of 8
 * for bf16, of 4 for fp32 o); token strides are >= D and < 2^24; o's rows
 * must not overlap one another (ATTN_ERR_ALIAS), and o, lse must not overlap
 * the address ranges of q, k, v.  lse stays contiguous [B, Hq, Nq].  Results
 * are bit-identical to attn_fwd on the same values.  Otherwise as attn_fwd.
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
                     int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D, float scale, int causal,
                     int64_t q_pos0, int64_t k_pos0, const int64_t* q_strides, const int64_t* kv_strides,
                     const int64_t* o_strides, void* hip_stream);

/*
 * attn_fwd_accumulate -- one step of a streaming ring on one GPU: attention of
 * q against one KV block, merged in place into a running result.
 *
 * o_acc [B, Hq, Nq, D] float and lse_acc [B, Hq, Nq] float hold the running
 * attention of q over the KV blocks of the previous calls.  With first != 0
 * they are overwritten with this block's result (as attn_fwd with ATTN_FP32
 * output); otherwise this block's (O_b, LSE_b) is merged into them by the
 * attn_partial_merge rule ("So funktioniert Kontextparallelität": combining
 * partial attention over disjoint key blocks gives full attention), which
 * replaces the per-block partial buffers and the separate merge pass of the
 * ring.  o_final (optional, bf16 [B, Hq, Nq, D]) also receives the merged O
 * rounded to bf16, for the last block.  k, v, k_pos0 describe the block
 * (global positions as in attn_fwd).  Calls on the same o_acc must be
 * ordered (one stream).  Otherwise as attn_fwd.
 */
int attn_fwd_accumulate(const void* q, const void* k, const void* v, float* o_acc, float* lse_acc, void* o_final,
                        int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D, float scale, int causal,
                        int64_t q_pos0, int64_t k_pos0, int first, void* hip_stream);

/*
 * attn_fwd_accumulate_group -- up to ATTN_MAX_FWD_GROUP independent
 * attn_fwd_accumulate calls in one launch.  In a ring step a rank's query
 * chunks each attend to the key/value chunk that just arrived ("Context
 * Parallelism", section "So funktioniert Kontextparallelität"); their
 * running results are distinct, so the calls are independent, and one
 * launch gives the GPU all their workgroups at once.  Each entry of calls (a
 * host array of n) is one call with the meaning of attn_fwd_accumulate's
 * arguments; B, Hq, Hkv, D, scale and causal are shared.  No call's outputs
 * (o_acc, lse_acc, o_final) may overlap another call's outputs or inputs
 * (ATTN_ERR_ALIAS): calls that update the same running result must be
 * separate, ordered launches.  Results are bit-identical to the calls made
 * one by one.  Every entry is validated before anything is launched; the
 * status names the first failing entry in attn_last_error.
 */
#define ATTN_MAX_FWD_GROUP 4
typedef struct {
  const void* q;    /* [B, Hq, Nq, D] bf16 */
  const void* k;    /* [B, Hkv, Nk, D] bf16 */
  const void* v;    /* [B, Hkv, Nk, D] bf16 */
  float* o_acc;     /* [B, Hq, Nq, D] float, running output */
  float* lse_acc;   /* [B, Hq, Nq] float, running log-sum-exp */
  void* o_final;    /* optional bf16 [B, Hq, Nq, D]: the merged O */
  int64_t Nq, Nk;   /* query rows, keys of the block */
  int64_t q_pos0, k_pos0;  /* global positions of the first query and key */
  int first;        /* nonzero: overwrite o_acc, lse_acc instead of merging */
} attn_accumulate_call;
int attn_fwd_accumulate_group(const attn_accumulate_call* calls, int n, int B, int Hq, int Hkv, int D, float scale,
                              int causal, void* hip_stream);

/*
 * attn_fwd_accumulate_group_split -- attn_fwd_accumulate_group with each
 * call's key/value block cut into n_splits ranges of key tiles that run side
 * by side, for calls too small to fill the GPU (a ring step of a short chunk:
 * the query rows alone give a few workgroups per compute unit at most).  Each
 * range's attention goes, in fp32, into the call's workspace; then one merge
 * pass per call combines the ranges that hold visible keys with the running
 * result (o_acc, lse_acc; not read when first) by the attn_partial_merge rule
 * ("So funktioniert Kontextparallelität") and writes o_acc, lse_acc and
 * o_final.  The sums are grouped differently from attn_fwd_accumulate, so
 * results agree with it up to rounding, not bit for bit; n_splits = 1 still
 * takes this path (one range, then the merge).
 *
 * Each entry: an attn_accumulate_call with the meaning of
 * attn_fwd_accumulate_group's entries, and its workspace (device memory of
 * at least attn_fwd_accumulate_workspace_size(B, Hq, call.Nq, D, n_splits)
 * bytes, 16-byte aligned, apart from every argument and every other
 * workspace; contents unspecified on return).  1 <= n_splits <= 64 and
 * B * n * n_splits <= 65535.  attn_fwd_split_suggest gives the library's
 * choice of n_splits for n_calls such calls side by side (1: no split).
 * Validation as attn_fwd_accumulate_group, workspaces included.
 */
typedef struct {
  attn_accumulate_call call;
  void* workspace;          /* fp32 partials of the call's key ranges */
  size_t workspace_bytes;
} attn_accumulate_split_call;
int attn_fwd_split_suggest(int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int causal, int n_calls);
size_t attn_fwd_accumulate_workspace_size(int B, int Hq, int64_t Nq, int D, int n_splits);
int attn_fwd_accumulate_group_split(const attn_accumulate_split_call* calls, int n, int B, int Hq, int Hkv, int D,
                                    float scale, int causal, int n_splits, void* hip_stream);

/*
 * attn_fwd_splitkv_workspace_size -- bytes of device workspace attn_fwd_splitkv
 * needs for the same arguments: fp32 partial outputs and log-sum-exps of every
 * key range, n * B*Hq*Nq*(D + 1) floats for n ranges (n_splits > 0: that many;
 * n_splits <= 0: the number attn_fwd_splitkv chooses).  Returns 0 for invalid
 * sizes or n_splits > 64.
 */
size_t attn_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D, int causal,
                                       int n_splits);

/*
 * attn_fwd_splitkv -- attn_fwd with the keys split into ranges that run side by
 * side, for short sequences where one workgroup per query block leaves most
 * of the GPU idle and the longest row sets the time.
 *
 * Same arguments, layouts, masking and results as attn_fwd with o in bf16
 * (up to fp32 rounding order).  The keys are cut into n contiguous ranges of
 * whole 64-key tiles; each range's attention (fp32 O and LSE) is the partial
 * attention of "So funktioniert Kontextparallelität" for one KV block, and the
 * ranges are combined by the attn_partial_merge rule.  n_splits in [1, 64]
 * fixes n; n_splits <= 0 lets the library choose: unsplit when the plain
 * grid already has 384 or more workgroups, else the most ranges whose
 * (range, query tile) pairs with work fit one workgroup per compute unit.
 * Only those pairs are launched; a range no query of a tile sees writes no
 * partial and the merge skips it.  The workspace (caller-owned, >=
 * attn_fwd_splitkv_workspace_size bytes, 16-byte aligned, not overlapping
 * any argument) is scratch; its contents on return are unspecified.
 * Deterministic.  Errors as attn_fwd, plus ATTN_ERR_WORKSPACE and
 * ATTN_ERR_UNSUPPORTED for n_splits > 64.
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D, float scale, int causal,
                     int64_t q_pos0, int64_t k_pos0, int n_splits, void* workspace, size_t workspace_bytes,
                     void* hip_stream);

/*
 * attn_partial_merge -- log-sum-exp merge of partial attention results.
 *
 * o_parts   [n_parts, B, H, N, D] bf16 or float (part_dtype)
 * lse_parts [n_parts, B, H, N]    float
 * o         [B, H, N, D] bf16,  lse [B, H, N] float
 *
 * Part b must be attention of the same queries over a block of keys, the
 * blocks being disjoint.  Then LSE = M + ln sum_b exp(LSE_b - M) with
 * M = max_b LSE_b, and O = sum_b exp(LSE_b - LSE) O_b, which is attention
 * over the union of the blocks ("So funktioniert Kontextparallelität": the
 * ring result equals full attention).  Parts with LSE_b = -inf weigh zero;
 * a row empty in every part gives o = 0, lse = -inf.  Requires n_parts >= 1,
 * D in {64, 128}.
 */
int attn_partial_merge(const void* o_parts, int part_dtype, const float* lse_parts, int n_parts,
                       void* o, float* lse, int B, int H, int64_t N, int D, void* hip_stream);

/*
 * attn_bwd_workspace_size -- bytes of device workspace attn_bwd needs: the
 * per-row <dO, O> in fp32 and, for grouped-query attention (Hq != Hkv),
 * per-query-head fp32 partials of dK and dV (2 * B*Hq*N*D floats) that are
 * summed over each group.  A small problem (fewer than 256 dK/dV workgroups,
 * i.e. B * Hq * ceil(N / 128) < 256) also splits its passes into ranges:
 * rkv query ranges of dK, dV partials (2 * rkv * B*Hq*N*D floats, replacing
 * the grouped-query ones) and rq key ranges of dQ partials (rq * B*Hq*N*D
 * floats), at most 8 ranges a pass and 64 MiB for the two.  Returns 0 for
 * invalid sizes.
 */
size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int64_t N, int D);

/*
 * attn_bwd_ds_workspace_size -- bytes of workspace with which attn_bwd (and
 * attn_bwd_strided) forms dq from stored dS instead of recomputing it.
 * dq = scale dS K needs, per query row, dS against every key it sees; the
 * recomputing dQ pass forms S = Q K^T and dO V^T a second time for that
 * (seven products per visible pair instead of five).  With this workspace
 * the dK/dV pass also writes the dS it forms (bf16, the same rounding the
 * products use) in 64 x 64 blocks -- every block at or left of the diagonal
 * when causal, all of them otherwise: about B * Hq * N^2 bytes causal, twice
 * that otherwise -- and a product pass reads them back: dq = scale dS K.
 * Layout: attn_bwd_workspace_size bytes rounded up to 256, then the blocks.
 * Returns 0 (path not available) for invalid sizes and for small problems
 * (fewer than 256 dK/dV workgroups: B * Hq * ceil(N / 128) < 256), whose
 * passes run as attn_bwd describes.
 */
size_t attn_bwd_ds_workspace_size(int B, int Hq, int Hkv, int64_t N, int D, int causal);

/*
 * attn_bwd -- gradients of sum(O * dO) with respect to q, k and v.
 *
 * q, o, d_o, dq [B, Hq, N, D] bf16;  k, v, dk, dv [B, Hkv, N, D] bf16;
 * lse [B, Hq, N] float from attn_fwd on the same inputs (Nq = Nk = N, equal
 * offsets).  P is recomputed from q, k and lse; with Dv_i = <dO_i, O_i>,
 * dS = P * (dO V^T - Dv), dq = scale dS K, dk = scale dS^T Q, dv = P^T dO,
 * accumulated in fp32 and rounded once to bf16.  For grouped-query attention
 * dk, dv of a key/value head sum over the query heads that read it.  The
 * workspace (caller-owned, >= attn_bwd_workspace_size bytes, 16-byte aligned)
 * is scratch; its contents on return are unspecified.  The glossary example
 * backpropagates the mean of O^2, i.e. d_o = 2 O / numel.
 * Small problems (fewer than 256 dK/dV workgroups: the glossary example's
 * [1, 4, 4096, 64]) are limited by their longest workgroups, the first key
 * tile against every query and the last query tile against every key: the
 * dK/dV pass then runs over ranges of about 1024 * 64 / D query rows and the
 * dQ pass over ranges of about 512 * 64 / D keys, each range writing fp32
 * partials into the workspace that a reduce kernel sums in a fixed order
 * (deterministic; the grouping of the sums differs from the unsplit passes,
 * so results agree with attn_bwd_block over the whole sequence to rounding,
 * not bit for bit).
 * With workspace_bytes >= attn_bwd_ds_workspace_size (nonzero), dq comes
 * from the stored dS (that function describes it): dk and dv are the same
 * bits as with the minimal workspace; dq sums the same terms over keys in
 * the same order, but its dS is formed from P after P's rounding to bf16 (as
 * dk's is), so it agrees with the recomputing pass to rounding.
 * When the dK/dV pass has fewer than two workgroups per compute unit (short
 * sequences, ring steps), the dQ pass runs beside it on a side stream of the
 * library's own, forked from hip_stream after Dv and joined back before the
 * call returns; results are the same bits either way.  Each caller stream
 * has its own side stream (default priority, created on its first such call;
 * up to 64 caller streams, further ones run single-stream), so no ordering
 * between different caller streams is added.  Calls from several host
 * threads are serialised around the fork and join.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
             const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
             int B, int Hq, int Hkv, int64_t N, int D, float scale, int causal, void* hip_stream);

/*
 * attn_bwd_noalloc -- attn_bwd without a workspace argument and without any
 * device allocation, for callers that cannot allocate: code under HIP graph
 * capture, tight training loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, layout and results as attn_bwd given attn_bwd_workspace_size
 * bytes of workspace (the same kernels, with dq from the recomputing pass;
 * outputs bit-identical), minus workspace / workspace_bytes.  The scratch those
 * kernels need (attn_bwd_workspace_size bytes: Dv per query row, the
 * grouped-query dK/dV partials and a small problem's range partials) lives in a
 * device array inside the library, attn_bwd_noalloc_max_scratch() bytes
 * (160 MiB) per GPU, held from the first call on that GPU until the process
 * ends.  A call that needs more returns ATTN_ERR_WORKSPACE before any GPU
 * work.  The array serves the GPU of hip_stream; every call on one GPU
 * shares it, so calls that may overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  Nothing in it needs
 * to start at zero.  The first call on a GPU looks up the array's device
 * address (not a device allocation); an error there returns ATTN_ERR_HIP.
 * Every launch stays on hip_stream (no side stream is created or used).
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                     const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int64_t N, int D,
                     float scale, int causal, void* hip_stream);

/* Bytes of scratch attn_bwd_noalloc holds per GPU (its size limit). */
size_t attn_bwd_noalloc_max_scratch(void);

/*
 * attn_bwd_strided -- attn_bwd on tensors given by element strides, so that
 * the backward of a Ulysses shard reads Q, K, V, O, dO in the token-major
 * layout the exchange delivers ([N, H, D] rows: token stride H*D, head
 * stride D; "Million-Token-Kontexte im Training ...", section "Ulysses: Die
 * Sequenz als Verteilungseinheit") and writes dQ, dK, dV the same way,
 * without relayout passes -- the backward counterpart of attn_fwd_strided.
 *
 * q_strides: host array of 3 element strides (batch, head, token) shared by
 * q, o, d_o and dq; kv_strides: the same for k, v, dk and dv.  The D
 * elements of a row are contiguous; every stride keeps rows 16-byte aligned
 * (a multiple of 8), token strides are >= D and < 2^24, and the rows of dq
 * (dk, dv) under these strides must not overlap one another (ATTN_ERR_ALIAS).
 * lse [B, Hq, N] and the workspace stay contiguous.  Outputs must not
 * overlap the address ranges of the inputs or one another.  Results are
 * bit-identical to attn_bwd on the same values.  Otherwise as attn_bwd.
 */
int attn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                     int64_t N, int D, float scale, int causal, const int64_t* q_strides,
                     const int64_t* kv_strides, void* hip_stream);

/*
 * attn_bwd_delta -- Dv_i = <dO_i, O_i> in fp32 for every query row: the
 * per-row term of dS that attn_bwd_block takes as an input.  o, d_o
 * [B, Hq, Nq, D] bf16 (o the final output of the forward, after every KV
 * block); delta [B, Hq, Nq] float, caller-owned, must not overlap o or d_o.
 * D in {64, 128}; 16-byte aligned pointers.
 */
int attn_bwd_delta(const void* o, const void* d_o, float* delta, int B, int Hq, int64_t Nq, int D,
                   void* hip_stream);

/*
 * attn_bwd_block_workspace_size -- bytes of device workspace attn_bwd_block
 * needs: 0 when Hq == Hkv, else per-query-head fp32 partials of dK and dV
 * (2 * B*Hq*Nk*D floats).  Returns 0 also for invalid sizes.
 */
size_t attn_bwd_block_workspace_size(int B, int Hq, int Hkv, int64_t Nk, int D);

/*
 * attn_bwd_block_ds_workspace_size -- bytes of workspace with which
 * attn_bwd_block forms dq from stored dS, as attn_bwd does with
 * attn_bwd_ds_workspace_size: the dK/dV pass also writes the dS it forms, in
 * 64 x 64 bf16 blocks, and a product pass adds scale dS K to dq (or dq_acc).
 * Layout: attn_bwd_block_workspace_size bytes rounded up to 256, then, per
 * batch and query head, ceil(Nq / 64) rows of 2 ceil(Nk / 128) blocks (the
 * position offsets make the causal rows irregular, so every row has room for
 * every block; only the blocks a row sees are written and read).  Returns 0
 * (path not available) for invalid sizes and for fewer than 256 dK/dV
 * workgroups (B * Hq * ceil(Nk / 128) < 256).  attn_bwd_block_group keeps the
 * recomputing pass.
 */
size_t attn_bwd_block_ds_workspace_size(int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D);

/*
 * attn_bwd_block -- the backward of one ring step: the gradients that flow
 * through one KV block's part of the attention of q ("So funktioniert
 * Kontextparallelität" on the "Context Parallelism" glossary page: each
 * device attends its queries to one KV block at a time).  Because the
 * forward's full attention is the LSE-merge of the per-block partials, P over
 * block b is exp(scale q_i.k_j - LSE_i) with the global LSE, and
 *   dS_ij = P_ij (dO_i.v_j - Dv_i)   (Dv from attn_bwd_delta on the final O),
 *   dq_i += scale sum_{j in b} dS_ij k_j,
 *   dk_j  = scale sum_i dS_ij q_i,   dv_j = sum_i P_ij dO_i   (j in b),
 * so summing dq over the blocks, and running every block, gives attn_bwd's
 * gradients exactly up to rounding.
 *
 * q, d_o [B, Hq, Nq, D] bf16; lse, delta [B, Hq, Nq] float (global LSE of the
 * forward over all blocks, and Dv); k, v [B, Hkv, Nk, D] bf16: the block.
 * Positions are global as in attn_fwd (q_pos0, k_pos0): key j is visible to
 * query i iff k_pos0 + j <= q_pos0 + i when causal.
 *
 * Outputs, each optional but at least one of dq_acc / dq and one of the pairs
 * (dk_acc, dv_acc) / (dk, dv):
 *   dq_acc [B, Hq, Nq, D] float: overwritten with this block's dq, or, with
 *     dq_accumulate != 0, this block's dq added to it (a ring over blocks);
 *   dq [B, Hq, Nq, D] bf16: the value dq_acc holds after the call rounded to
 *     bf16 (or, without dq_acc, this block's dq);
 *   dk_acc, dv_acc [B, Hkv, Nk, D] float: the same for dk, dv with
 *     dkv_accumulate (a block whose gradients arrive from several query
 *     shards); dk, dv [B, Hkv, Nk, D] bf16: rounded copies.
 * Keys that no query sees get zero gradients.  Requires Nq, Nk < 2^30;
 * workspace >= attn_bwd_block_workspace_size bytes (may be null when that
 * is 0; contents unspecified on return); with at least
 * attn_bwd_block_ds_workspace_size bytes (nonzero) dq comes from stored dS
 * (dk, dv the same bits; dq agrees to rounding).  Outputs must not overlap
 * inputs or one another.  Calls accumulating into the same buffers must be
 * ordered (one stream).  Deterministic.  Otherwise as attn_bwd.
 */
int attn_bwd_block(const void* q, const void* k, const void* v, const void* d_o, const float* lse,
                   const float* delta, float* dq_acc, float* dk_acc, float* dv_acc, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D,
                   float scale, int causal, int64_t q_pos0, int64_t k_pos0, int dq_accumulate, int dkv_accumulate,
                   void* hip_stream);

/*
 * attn_bwd_block_group -- up to ATTN_MAX_BWD_GROUP independent attn_bwd_block
 * calls in one dK/dV launch and one dQ launch (plus, for grouped-query
 * attention, one small reduction per call).  On a ring whose ranks hold two
 * query chunks and receive two key/value chunks per step (zigzag sharding of
 * "So funktioniert Kontextparallelität"), the step's visible (query chunk,
 * key chunk) pairs that share neither chunk -- (q1, k1) with (q2, k2), and
 * (q1, k2) with (q2, k1) -- are independent: their dQ and their dK, dV go to
 * different accumulators.  Each call's fields mean what the arguments of
 * attn_bwd_block mean; B, Hq, Hkv, D, scale and causal are shared.  Every call
 * is validated as attn_bwd_block (errors name the call); in addition no call
 * may write what another call reads or writes (ATTN_ERR_ALIAS).  Results are
 * bit-identical to the same calls made one at a time with the recomputing dQ
 * pass (a workspace below attn_bwd_block_ds_workspace_size; a group call's
 * workspace may be larger, it is not used for stored dS).  Requires 1 <= n <=
 * ATTN_MAX_BWD_GROUP and B * n <= 65535.
 */
#define ATTN_MAX_BWD_GROUP 4
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  const float* lse;
  const float* delta;
  float* dq_acc;
  float* dk_acc;
  float* dv_acc;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;
  size_t workspace_bytes;
  int64_t Nq, Nk, q_pos0, k_pos0;
  int dq_accumulate, dkv_accumulate;
} attn_bwd_block_call;
int attn_bwd_block_group(const attn_bwd_block_call* calls, int n, int B, int Hq, int Hkv, int D, float scale,
                         int causal, void* hip_stream);

/*
 * seq_to_head_relayout -- the Ulysses all-to-all's data movement on one GPU.
 *
 * in  [P, N/P, H, D]: shard p holds tokens p*N/P .. (p+1)*N/P - 1, all heads.
 * out [P, H/P, N, D]: rank r holds heads r*H/P .. (r+1)*H/P - 1, all tokens.
 * out[r, h', n, :] = in[n / (N/P), n % (N/P), r*(H/P) + h', :] -- the
 * transpose [N, H, D] -> [H, N, D].  A bit copy of elem_bytes-wide words
 * (2 for bf16, 4 for float).  Requires P | N, D*elem_bytes 16 times a power
 * of two, and P | H -- or, for fewer heads than ranks (key/value heads of
 * grouped-query attention, H < P), H | P: then each head is replicated to
 * the P/H consecutive ranks whose query heads read it, out [P, 1, N, D] with
 * out[r, 0, n, :] = in[n / (N/P), n % (N/P), r / (P/H), :].  in and out must
 * not overlap.  For key/value tensors pass H = Hkv.
 */
int seq_to_head_relayout(const void* in, void* out, int P, int64_t N, int H, int D, int elem_bytes,
                         void* hip_stream);

/*
 * head_to_seq_relayout -- the inverse: in [P, H/P, N, D] -> out [P, N/P, H, D]
 * (P | H; replicated heads, H < P, are ATTN_ERR_UNSUPPORTED here: their
 * gradients must be summed, see head_to_seq_reduce).
 */
int head_to_seq_relayout(const void* in, void* out, int P, int64_t N, int H, int D, int elem_bytes,
                         void* hip_stream);

/*
 * seq_to_head_relayout_batch / head_to_seq_relayout_batch -- the relayouts
 * of several tensors in one launch: tensor j (j < n) is moved exactly as
 * seq_to_head_relayout (head_to_seq_relayout) would move ins[j] into
 * outs[j] with H = H[j]; P, N, D and elem_bytes are shared.  Ulysses
 * exchanges the query, key and value matrices in one all-to-all step
 * ("Million-Token-Kontexte im Training ...", section "Ulysses: Die Sequenz
 * als Verteilungseinheit"); one launch over all of them (and dO, or O and
 * the gradients on the way back) avoids the ramp-up and drain of a launch
 * per tensor.  ins, outs and H
 * are host arrays of n entries, 1 <= n <= ATTN_MAX_RELAYOUT_BATCH; each
 * tensor is validated as in the single call (status and tensor index in
 * attn_last_error), and no output may overlap any input or another output
 * (ATTN_ERR_ALIAS).  Nothing is launched on any error.
 */
#define ATTN_MAX_RELAYOUT_BATCH 8
int seq_to_head_relayout_batch(int n, const void* const* ins, void* const* outs, const int* H, int P, int64_t N,
                               int D, int elem_bytes, void* hip_stream);
int head_to_seq_relayout_batch(int n, const void* const* ins, void* const* outs, const int* H, int P, int64_t N,
                               int D, int elem_bytes, void* hip_stream);

/*
 * head_to_seq_reduce -- the inverse exchange of gradients of heads that
 * several ranks shared: with R = P/H ranks per head when H < P (else R = 1),
 * in [P, max(1, H/P), N, D] (flattened: [H*R, N, D], rank-major), out
 * [P, N/P, H, D] bf16 with out[n / (N/P), n % (N/P), h, :] = the sum over
 * i < R of in[h*R + i, n, :], added in fp32 in the order i = 0, 1, ... and
 * rounded once to bf16 (nearest even).  A key/value head read by the query
 * heads of R ranks gets the sum of their dK (dV) parts, which is its
 * gradient.  in_dtype ATTN_BF16 or ATTN_FP32 (e.g. attn_bwd_block's fp32
 * accumulators); R = 1 is the plain inverse relayout with a conversion.
 * Requires P | N, H | P or P | H, D a multiple of 8; in and out must not
 * overlap.
 */
int head_to_seq_reduce(const void* in, int in_dtype, void* out, int P, int64_t N, int H, int D, void* hip_stream);

/*
 * Measurement hook (not part of the computation).  While enabled, every
 * kernel the library launches is bracketed by two HIP events recorded on its
 * launch stream (at most 8192 launches are held).  attn_trace_collect waits
 * for those events, writes per-kernel totals -- the kernel's name into
 * names + i*name_len (NUL-terminated), the summed milliseconds into
 * total_ms[i] and the launch count into calls[i] for i < max_kernels --
 * releases the records and returns the number of distinct kernels, or
 * -ATTN_ERR_HIP if an event could not be read.  The events are created once
 * and reused.  Thread-safe.
 */
int attn_trace_enable(int on);
int attn_trace_collect(char* names, int name_len, double* total_ms, int* calls, int max_kernels);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Detail of the calling thread's last failure ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LCATTN_ATTN_H */
