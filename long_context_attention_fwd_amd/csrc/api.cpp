// api.cpp -- the library's C ABI: argument validation, dispatch, status codes.
//
// Every entry point validates on the host first and returns a status without
// touching the GPU when validation fails, so the error paths are testable on a
// machine without a GPU.  Kernels are enqueued on the caller's stream (the
// backward of a small problem forks its dQ pass onto a side stream of the
// library and joins it back); the library allocates no device memory, and its
// only state is a thread-local error text, the measurement hook's records and
// per-GPU handles created at first use (scratch address, side stream).
#include "attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <algorithm>
#include <utility>

#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

constexpr int kMaxSplits = 64;  // key ranges of attn_fwd_splitkv

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checked product of non-negative sizes; false on overflow of int64.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool elems(int64_t* out, std::initializer_list<int64_t> dims) {
  int64_t n = 1;
  for (int64_t d : dims)
    if (!mul_ok(n, d, &n)) return false;
  *out = n;
  return true;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "invalid shape";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case ATTN_ERR_ALIAS: return "output overlaps input";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

// Validation shared by attn_fwd and attn_fwd_splitkv; fills the kernel
// arguments on success.
int fwd_check(const char* name, const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
              int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D, float scale, int causal, int64_t q_pos0,
              int64_t k_pos0, lcattn::FwdArgs* a, bool contiguous = true) {
  if (!q || !k || !v || !o || !lse) return fail(ATTN_ERR_NULL, "%s: q, k, v, o and lse must be non-null", name);
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || D < 1)
    return fail(ATTN_ERR_SHAPE, "%s: sizes must be >= 1 (B=%d Hq=%d Hkv=%d Nq=%lld Nk=%lld D=%d)", name, B, Hq,
                Hkv, (long long)Nq, (long long)Nk, D);
  if (Hq % Hkv) return fail(ATTN_ERR_SHAPE, "%s: Hkv=%d does not divide Hq=%d", name, Hkv, Hq);
  if (q_pos0 < 0 || k_pos0 < 0) return fail(ATTN_ERR_SHAPE, "%s: position offsets must be >= 0", name);
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: D=%d (supported: 64, 128)", name, D);
  if (o_dtype != ATTN_BF16 && o_dtype != ATTN_FP32)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: o_dtype=%d (ATTN_BF16 or ATTN_FP32)", name, o_dtype);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: scale must be finite and > 0", name);
  if (Hq / Hkv > 1 && Hq > 65535 * 4) return fail(ATTN_ERR_UNSUPPORTED, "%s: too many heads", name);
  int64_t nq_el, nk_el, nl;
  if (!elems(&nq_el, {B, Hq, Nq, D}) || !elems(&nk_el, {B, Hkv, Nk, D}) || !elems(&nl, {B, Hq, Nq}) ||
      nq_el > (INT64_MAX / 8))
    return fail(ATTN_ERR_SHAPE, "%s: tensor sizes overflow", name);
  if (Nq >= INT32_MAX || Nk >= INT32_MAX || B > 65535 || Hq > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: sequence lengths must be < 2^31, B and Hq <= 65535", name);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(ATTN_ERR_ALIGN, "%s: pointers must be 16-byte aligned", name);
  if (contiguous) {
    const size_t ob = (size_t)nq_el * (o_dtype == ATTN_FP32 ? 4 : 2);
    const size_t lb = (size_t)nl * 4;
    const void* ins[3] = {q, k, v};
    const size_t inb[3] = {(size_t)nq_el * 2, (size_t)nk_el * 2, (size_t)nk_el * 2};
    for (int i = 0; i < 3; ++i)
      if (overlap(o, ob, ins[i], inb[i]) || overlap(lse, lb, ins[i], inb[i]))
        return fail(ATTN_ERR_ALIAS, "%s: outputs overlap inputs", name);
    if (overlap(o, ob, lse, lb)) return fail(ATTN_ERR_ALIAS, "%s: o overlaps lse", name);
  }

  a->q = static_cast<const uint16_t*>(q);
  a->k = static_cast<const uint16_t*>(k);
  a->v = static_cast<const uint16_t*>(v);
  a->o = o;
  a->lse = lse;
  a->Hq = Hq;
  a->Hkv = Hkv;
  a->G = Hq / Hkv;
  a->Nq = Nq;
  a->Nk = Nk;
  a->scale_log2 = scale * 1.4426950408889634f;
  a->causal = causal ? 1 : 0;
  a->q_pos0 = q_pos0;
  a->k_pos0 = k_pos0;
  return ATTN_OK;
}

// Strides (batch, head, token; elements) of a [B, H, N, D] tensor whose head
// dimension is contiguous.  Every row starts 16-byte aligned; the token
// stride is at least D and below 2^24 (per-lane tile offsets are 32-bit); an output's
// rows must not overlap one another.  *span = elements from the first to one
// past the last element.
int stride_check(const char* name, const char* what, const int64_t* st, int B, int H, int64_t N, int D,
                 int elem_bytes, bool output, int64_t* span) {
  if (!st) return fail(ATTN_ERR_NULL, "%s: %s strides must be non-null", name, what);
  const int64_t cnt[3] = {B, H, N};
  int64_t sp = D;
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return fail(ATTN_ERR_SHAPE, "%s: %s strides must be >= 0", name, what);
    if ((st[i] * elem_bytes) % 16)
      return fail(ATTN_ERR_ALIGN, "%s: %s strides must keep rows 16-byte aligned", name, what);
    int64_t ext;
    if (!mul_ok(cnt[i] - 1, st[i], &ext) || ext > INT64_MAX / 4 - sp)
      return fail(ATTN_ERR_SHAPE, "%s: %s extent overflows", name, what);
    sp += ext;
  }
  if (st[2] < D) return fail(ATTN_ERR_SHAPE, "%s: %s token stride must be >= D", name, what);
  if (st[2] >= (int64_t(1) << 24))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: %s token stride must be < 2^24 elements", name, what);
  if (output) {
    // sort the dimensions of more than one element by stride; each must step
    // past everything inside it
    int64_t s2[3], c2[3];
    int m = 0;
    for (int i = 0; i < 3; ++i)
      if (cnt[i] > 1) { s2[m] = st[i]; c2[m] = cnt[i]; ++m; }
    for (int i = 0; i < m; ++i)
      for (int j = i + 1; j < m; ++j)
        if (s2[j] < s2[i]) { std::swap(s2[i], s2[j]); std::swap(c2[i], c2[j]); }
    int64_t inner = D;
    for (int i = 0; i < m; ++i) {
      if (s2[i] < inner) return fail(ATTN_ERR_ALIAS, "%s: %s rows overlap one another", name, what);
      inner = s2[i] * c2[i];
    }
  }
  *span = sp;
  return ATTN_OK;
}

// Workspace bytes of attn_fwd_splitkv for n key ranges: fp32 partial O, then
// fp32 partial LSE.  0 on overflow.
size_t splitkv_bytes(int B, int Hq, int64_t Nq, int D, int n) {
  int64_t el;
  if (!elems(&el, {n, B, Hq, Nq, D + 1}) || el > INT64_MAX / 4) return 0;
  return (size_t)el * 4;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, int B, int Hq,
             int Hkv, int64_t Nq, int64_t Nk, int D, float scale, int causal, int64_t q_pos0, int64_t k_pos0,
             void* hip_stream) {
  lcattn::FwdArgs a;
  const int st = fwd_check("attn_fwd", q, k, v, o, o_dtype, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, q_pos0,
                           k_pos0, &a);
  if (st != ATTN_OK) return st;
  return hip_status(lcattn::launch_attn_fwd(a, B, D, o_dtype == ATTN_FP32, static_cast<hipStream_t>(hip_stream)),
                    "attn_fwd launch");
}

int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, int B, int Hq,
                     int Hkv, int64_t Nq, int64_t Nk, int D, float scale, int causal, int64_t q_pos0,
                     int64_t k_pos0, const int64_t* q_strides, const int64_t* kv_strides, const int64_t* o_strides,
                     void* hip_stream) {
  lcattn::FwdArgs a;
  const char* name = "attn_fwd_strided";
  int st = fwd_check(name, q, k, v, o, o_dtype, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, q_pos0, k_pos0, &a,
                     false);
  if (st != ATTN_OK) return st;
  const int ob = o_dtype == ATTN_FP32 ? 4 : 2;
  int64_t qsp, ksp, osp;
  if ((st = stride_check(name, "q", q_strides, B, Hq, Nq, D, 2, false, &qsp)) != ATTN_OK) return st;
  if ((st = stride_check(name, "k/v", kv_strides, B, Hkv, Nk, D, 2, false, &ksp)) != ATTN_OK) return st;
  if ((st = stride_check(name, "o", o_strides, B, Hq, Nq, D, ob, true, &osp)) != ATTN_OK) return st;
  int64_t nl;
  elems(&nl, {B, Hq, Nq});
  const void* ins[3] = {q, k, v};
  const size_t inb[3] = {(size_t)qsp * 2, (size_t)ksp * 2, (size_t)ksp * 2};
  for (int i = 0; i < 3; ++i)
    if (overlap(o, (size_t)osp * ob, ins[i], inb[i]) || overlap(lse, (size_t)nl * 4, ins[i], inb[i]))
      return fail(ATTN_ERR_ALIAS, "%s: outputs overlap inputs", name);
  if (overlap(o, (size_t)osp * ob, lse, (size_t)nl * 4)) return fail(ATTN_ERR_ALIAS, "%s: o overlaps lse", name);
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = q_strides[i];
    a.ks[i] = kv_strides[i];
    a.os[i] = o_strides[i];
  }
  return hip_status(lcattn::launch_attn_fwd(a, B, D, o_dtype == ATTN_FP32, static_cast<hipStream_t>(hip_stream)),
                    "attn_fwd_strided launch");
}

int attn_fwd_accumulate(const void* q, const void* k, const void* v, float* o_acc, float* lse_acc, void* o_final,
                        int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D, float scale, int causal,
                        int64_t q_pos0, int64_t k_pos0, int first, void* hip_stream) {
  lcattn::FwdArgs a;
  const char* name = "attn_fwd_accumulate";
  const int st = fwd_check(name, q, k, v, o_acc, ATTN_FP32, lse_acc, B, Hq, Hkv, Nq, Nk, D, scale, causal, q_pos0,
                           k_pos0, &a);
  if (st != ATTN_OK) return st;
  if (o_final) {
    if (!aligned16(o_final)) return fail(ATTN_ERR_ALIGN, "%s: o_final must be 16-byte aligned", name);
    int64_t nq_el, nk_el, nl;
    elems(&nq_el, {B, Hq, Nq, D});
    elems(&nk_el, {B, Hkv, Nk, D});
    elems(&nl, {B, Hq, Nq});
    const void* bufs[5] = {q, k, v, o_acc, lse_acc};
    const size_t sizes[5] = {(size_t)nq_el * 2, (size_t)nk_el * 2, (size_t)nk_el * 2, (size_t)nq_el * 4,
                             (size_t)nl * 4};
    for (int i = 0; i < 5; ++i)
      if (overlap(o_final, (size_t)nq_el * 2, bufs[i], sizes[i]))
        return fail(ATTN_ERR_ALIAS, "%s: o_final overlaps another argument", name);
  }
  a.accum = first ? 0 : 1;
  a.o_final = static_cast<uint16_t*>(o_final);
  return hip_status(lcattn::launch_attn_fwd(a, B, D, true, static_cast<hipStream_t>(hip_stream)), "attn_fwd_accumulate launch");
}

static_assert(ATTN_MAX_FWD_GROUP == lcattn::kMaxFwdGroup, "group limit of the header and the kernel");
static_assert(ATTN_MAX_BWD_GROUP == lcattn::kMaxBwdGroup, "group limit of the header and the kernels");

}  // extern "C"

namespace {

// Validation of a group of accumulate calls (each as attn_fwd_accumulate; no
// call's outputs may overlap another call's inputs or outputs); fills the
// kernel arguments and each call's byte ranges (inputs q, k, v; outputs
// o_acc, lse_acc, o_final).
int accumulate_group_check(const char* name, const attn_accumulate_call* const* calls, int n, int B, int Hq,
                           int Hkv, int D, float scale, int causal, lcattn::FwdArgs* args,
                           const void* (*in_p)[3], size_t (*in_b)[3], const void* (*out_p)[3],
                           size_t (*out_b)[3]) {
  if (n < 1 || n > ATTN_MAX_FWD_GROUP) return fail(ATTN_ERR_SHAPE, "%s: n=%d calls (1 .. %d)", name, n, ATTN_MAX_FWD_GROUP);
  for (int c = 0; c < n; ++c)
    if (!calls[c]) return fail(ATTN_ERR_NULL, "%s: null call array", name);
  for (int c = 0; c < n; ++c) {
    const attn_accumulate_call& x = *calls[c];
    int st = fwd_check(name, x.q, x.k, x.v, x.o_acc, ATTN_FP32, x.lse_acc, B, Hq, Hkv, x.Nq, x.Nk, D, scale, causal,
                       x.q_pos0, x.k_pos0, &args[c]);
    int64_t nq_el = 0, nk_el = 0, nl = 0;
    elems(&nq_el, {B, Hq, x.Nq, D});
    elems(&nk_el, {B, Hkv, x.Nk, D});
    elems(&nl, {B, Hq, x.Nq});
    if (st == ATTN_OK && x.o_final) {
      if (!aligned16(x.o_final)) st = fail(ATTN_ERR_ALIGN, "%s: o_final must be 16-byte aligned", name);
      const void* bufs[5] = {x.q, x.k, x.v, x.o_acc, x.lse_acc};
      const size_t sizes[5] = {(size_t)nq_el * 2, (size_t)nk_el * 2, (size_t)nk_el * 2, (size_t)nq_el * 4,
                               (size_t)nl * 4};
      for (int i = 0; st == ATTN_OK && i < 5; ++i)
        if (overlap(x.o_final, (size_t)nq_el * 2, bufs[i], sizes[i]))
          st = fail(ATTN_ERR_ALIAS, "%s: o_final overlaps another argument", name);
    }
    if (st != ATTN_OK) {
      char detail[sizeof(g_last_error)];
      snprintf(detail, sizeof(detail), "%s", g_last_error);
      return fail(st, "%s (call %d)", detail, c);
    }
    in_p[c][0] = x.q; in_b[c][0] = (size_t)nq_el * 2;
    in_p[c][1] = x.k; in_b[c][1] = (size_t)nk_el * 2;
    in_p[c][2] = x.v; in_b[c][2] = (size_t)nk_el * 2;
    out_p[c][0] = x.o_acc; out_b[c][0] = (size_t)nq_el * 4;
    out_p[c][1] = x.lse_acc; out_b[c][1] = (size_t)nl * 4;
    out_p[c][2] = x.o_final; out_b[c][2] = x.o_final ? (size_t)nq_el * 2 : 0;
    args[c].accum = x.first ? 0 : 1;
    args[c].o_final = static_cast<uint16_t*>(x.o_final);
  }
  for (int c = 0; c < n; ++c)
    for (int d = 0; d < n; ++d) {
      if (c == d) continue;
      for (int i = 0; i < 3; ++i) {
        if (!out_p[c][i]) continue;
        for (int j = 0; j < 3; ++j) {
          if (overlap(out_p[c][i], out_b[c][i], in_p[d][j], in_b[d][j]))
            return fail(ATTN_ERR_ALIAS, "%s: outputs of call %d overlap inputs of call %d", name, c, d);
          if (out_p[d][j] && overlap(out_p[c][i], out_b[c][i], out_p[d][j], out_b[d][j]))
            return fail(ATTN_ERR_ALIAS, "%s: outputs of calls %d and %d overlap", name, c, d);
        }
      }
    }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_accumulate_group(const attn_accumulate_call* calls, int n, int B, int Hq, int Hkv, int D, float scale,
                              int causal, void* hip_stream) {
  const char* name = "attn_fwd_accumulate_group";
  if (!calls) return fail(ATTN_ERR_NULL, "%s: null call array", name);
  if (n < 1 || n > ATTN_MAX_FWD_GROUP) return fail(ATTN_ERR_SHAPE, "%s: n=%d calls (1 .. %d)", name, n, ATTN_MAX_FWD_GROUP);
  if ((int64_t)B * n > 65535) return fail(ATTN_ERR_UNSUPPORTED, "%s: B * n must be <= 65535", name);
  const attn_accumulate_call* ptrs[ATTN_MAX_FWD_GROUP];
  for (int c = 0; c < n; ++c) ptrs[c] = &calls[c];
  lcattn::FwdArgs args[ATTN_MAX_FWD_GROUP];
  const void* in_p[ATTN_MAX_FWD_GROUP][3];
  size_t in_b[ATTN_MAX_FWD_GROUP][3];
  const void* out_p[ATTN_MAX_FWD_GROUP][3];
  size_t out_b[ATTN_MAX_FWD_GROUP][3];
  const int st = accumulate_group_check(name, ptrs, n, B, Hq, Hkv, D, scale, causal, args, in_p, in_b, out_p, out_b);
  if (st != ATTN_OK) return st;
  return hip_status(lcattn::launch_attn_fwd_group(args, n, B, D, static_cast<hipStream_t>(hip_stream)),
                    "attn_fwd_accumulate_group launch");
}

int attn_fwd_split_suggest(int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int causal, int n_calls) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Nq < 1 || Nk < 1 || n_calls < 1) return 1;
  // the choice for one call of n_calls times the rows: the calls run side by side
  return lcattn::fwd_split_count(B, Hq, Hkv, Nq * n_calls, Nk, causal, 0);
}

size_t attn_fwd_accumulate_workspace_size(int B, int Hq, int64_t Nq, int D, int n_splits) {
  if (B < 1 || Hq < 1 || Nq < 1 || D < 1 || n_splits < 1 || n_splits > kMaxSplits) return 0;
  return splitkv_bytes(B, Hq, Nq, D, n_splits);
}

int attn_fwd_accumulate_group_split(const attn_accumulate_split_call* calls, int n, int B, int Hq, int Hkv, int D,
                                    float scale, int causal, int n_splits, void* hip_stream) {
  const char* name = "attn_fwd_accumulate_group_split";
  if (!calls) return fail(ATTN_ERR_NULL, "%s: null call array", name);
  if (n < 1 || n > ATTN_MAX_FWD_GROUP) return fail(ATTN_ERR_SHAPE, "%s: n=%d calls (1 .. %d)", name, n, ATTN_MAX_FWD_GROUP);
  if (n_splits < 1 || n_splits > kMaxSplits)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: n_splits=%d (1 .. %d)", name, n_splits, kMaxSplits);
  if ((int64_t)B * n * n_splits > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: B * n * n_splits must be <= 65535", name);
  const attn_accumulate_call* ptrs[ATTN_MAX_FWD_GROUP];
  for (int c = 0; c < n; ++c) ptrs[c] = &calls[c].call;
  lcattn::FwdArgs args[ATTN_MAX_FWD_GROUP];
  const void* in_p[ATTN_MAX_FWD_GROUP][3];
  size_t in_b[ATTN_MAX_FWD_GROUP][3];
  const void* out_p[ATTN_MAX_FWD_GROUP][3];
  size_t out_b[ATTN_MAX_FWD_GROUP][3];
  const int st = accumulate_group_check(name, ptrs, n, B, Hq, Hkv, D, scale, causal, args, in_p, in_b, out_p, out_b);
  if (st != ATTN_OK) return st;
  // workspaces: large enough, aligned, apart from every argument and one another
  float* parts[ATTN_MAX_FWD_GROUP];
  size_t need[ATTN_MAX_FWD_GROUP];
  for (int c = 0; c < n; ++c) {
    const attn_accumulate_split_call& x = calls[c];
    need[c] = splitkv_bytes(B, Hq, x.call.Nq, D, n_splits);
    if (need[c] == 0) return fail(ATTN_ERR_SHAPE, "%s: workspace size overflows (call %d)", name, c);
    if (!x.workspace || x.workspace_bytes < need[c])
      return fail(ATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (call %d)", name, need[c], c);
    if (!aligned16(x.workspace)) return fail(ATTN_ERR_ALIGN, "%s: workspace must be 16-byte aligned (call %d)", name, c);
    parts[c] = static_cast<float*>(x.workspace);
  }
  for (int c = 0; c < n; ++c)
    for (int d = 0; d < n; ++d) {
      for (int j = 0; j < 3; ++j) {
        if (overlap(calls[c].workspace, need[c], in_p[d][j], in_b[d][j]) ||
            (out_p[d][j] && overlap(calls[c].workspace, need[c], out_p[d][j], out_b[d][j])))
          return fail(ATTN_ERR_ALIAS, "%s: workspace of call %d overlaps an argument of call %d", name, c, d);
      }
      if (d != c && overlap(calls[c].workspace, need[c], calls[d].workspace, need[d]))
        return fail(ATTN_ERR_ALIAS, "%s: workspaces of calls %d and %d overlap", name, c, d);
    }
  return hip_status(lcattn::launch_attn_fwd_group_split(args, parts, n, B, D, n_splits,
                                                        static_cast<hipStream_t>(hip_stream)),
                    "attn_fwd_accumulate_group_split launch");
}

size_t attn_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D, int causal,
                                       int n_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Nq < 1 || Nk < 1 || D < 1 || n_splits > kMaxSplits) return 0;
  return splitkv_bytes(B, Hq, Nq, D, lcattn::splitkv_split_count(B, Hq, Hkv, Nq, Nk, causal, n_splits));
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int64_t Nq, int64_t Nk, int D, float scale, int causal, int64_t q_pos0, int64_t k_pos0,
                     int n_splits, void* workspace, size_t workspace_bytes, void* hip_stream) {
  lcattn::FwdArgs a;
  const int st = fwd_check("attn_fwd_splitkv", q, k, v, o, ATTN_BF16, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal,
                           q_pos0, k_pos0, &a);
  if (st != ATTN_OK) return st;
  if (n_splits > kMaxSplits)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_splitkv: n_splits=%d (at most %d)", n_splits, kMaxSplits);
  const int n = lcattn::splitkv_split_count(B, Hq, Hkv, Nq, Nk, causal, n_splits);
  if ((int64_t)B * n > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_splitkv: B * n_splits must be <= 65535");
  const size_t need = splitkv_bytes(B, Hq, Nq, D, n);
  if (need == 0) return fail(ATTN_ERR_SHAPE, "attn_fwd_splitkv: workspace size overflows");
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "attn_fwd_splitkv: workspace of %zu bytes needed", need);
  if (!aligned16(workspace)) return fail(ATTN_ERR_ALIGN, "attn_fwd_splitkv: workspace must be 16-byte aligned");
  int64_t nq_el, nk_el, nl;
  elems(&nq_el, {B, Hq, Nq, D});
  elems(&nk_el, {B, Hkv, Nk, D});
  elems(&nl, {B, Hq, Nq});
  const void* bufs[5] = {q, k, v, o, lse};
  const size_t sizes[5] = {(size_t)nq_el * 2, (size_t)nk_el * 2, (size_t)nk_el * 2, (size_t)nq_el * 2,
                           (size_t)nl * 4};
  for (int i = 0; i < 5; ++i)
    if (overlap(workspace, need, bufs[i], sizes[i]))
      return fail(ATTN_ERR_ALIAS, "attn_fwd_splitkv: workspace overlaps an input or output");
  float* o_parts = static_cast<float*>(workspace);
  float* lse_parts = o_parts + (size_t)n * nq_el;
  return hip_status(lcattn::launch_attn_fwd_splitkv(a, B, D, n, o_parts, lse_parts,
                                                    static_cast<hipStream_t>(hip_stream)),
                    "attn_fwd_splitkv launch");
}

int attn_partial_merge(const void* o_parts, int part_dtype, const float* lse_parts, int n_parts, void* o,
                       float* lse, int B, int H, int64_t N, int D, void* hip_stream) {
  if (!o_parts || !lse_parts || !o || !lse) return fail(ATTN_ERR_NULL, "attn_partial_merge: null pointer");
  if (n_parts < 1 || B < 1 || H < 1 || N < 1 || D < 1)
    return fail(ATTN_ERR_SHAPE, "attn_partial_merge: sizes and n_parts must be >= 1");
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_partial_merge: D=%d (supported: 64, 128)", D);
  if (part_dtype != ATTN_BF16 && part_dtype != ATTN_FP32)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_partial_merge: part_dtype=%d", part_dtype);
  int64_t rows, parts_el, out_el;
  if (!elems(&rows, {B, H, N}) || !elems(&parts_el, {n_parts, rows, D}) || !elems(&out_el, {rows, D}) ||
      parts_el > INT64_MAX / 8 || (rows * (D / 8) + 255) / 256 > INT32_MAX)
    return fail(ATTN_ERR_SHAPE, "attn_partial_merge: tensor sizes overflow");
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse))
    return fail(ATTN_ERR_ALIGN, "attn_partial_merge: pointers must be 16-byte aligned");
  const size_t pb = (size_t)parts_el * (part_dtype == ATTN_FP32 ? 4 : 2);
  const size_t plb = (size_t)n_parts * rows * 4, ob = (size_t)out_el * 2, lb = (size_t)rows * 4;
  if (overlap(o, ob, o_parts, pb) || overlap(o, ob, lse_parts, plb) || overlap(lse, lb, o_parts, pb) ||
      overlap(lse, lb, lse_parts, plb) || overlap(o, ob, lse, lb))
    return fail(ATTN_ERR_ALIAS, "attn_partial_merge: outputs overlap inputs");
  return hip_status(lcattn::launch_partial_merge(o_parts, part_dtype == ATTN_FP32, lse_parts, n_parts,
                                                 static_cast<uint16_t*>(o), lse, rows, D,
                                                 static_cast<hipStream_t>(hip_stream)),
                    "attn_partial_merge launch");
}

size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int64_t N, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1 || Hq % Hkv) return 0;
  int64_t el;
  if (!elems(&el, {B, Hq, N, D}) || el > INT64_MAX / 16) return 0;
  return (size_t)lcattn::bwd_workspace_bytes(B, Hq, Hkv, N, N, D);
}

size_t attn_bwd_ds_workspace_size(int B, int Hq, int Hkv, int64_t N, int D, int causal) {
  if (attn_bwd_workspace_size(B, Hq, Hkv, N, D) == 0 || (D != 64 && D != 128)) return 0;
  // the stored blocks: at most B * Hq * N^2 elements (checked against
  // overflow before multiplying out)
  const double approx = (double)B * Hq * ((double)N + 128) * ((double)N + 128) * 2.0;
  if (approx > 9.0e18) return 0;
  return (size_t)lcattn::bwd_ds_workspace_bytes(B, Hq, Hkv, N, D, causal ? 1 : 0);
}

// attn_bwd and attn_bwd_strided: validation and launch.  Null strides:
// contiguous [B, H, N, D] tensors.
static int bwd_entry(const char* name, const void* q, const void* k, const void* v, const void* o, const void* d_o,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
                     int Hq, int Hkv, int64_t N, int D, float scale, int causal, const int64_t* q_strides,
                     const int64_t* kv_strides, void* hip_stream, bool use_scratch = false) {
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv)
    return fail(ATTN_ERR_NULL, "%s: tensor pointers must be non-null", name);
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1) return fail(ATTN_ERR_SHAPE, "%s: sizes must be >= 1", name);
  if (Hq % Hkv) return fail(ATTN_ERR_SHAPE, "%s: Hkv=%d does not divide Hq=%d", name, Hkv, Hq);
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: D=%d (supported: 64, 128)", name, D);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(ATTN_ERR_UNSUPPORTED, "%s: scale must be > 0", name);
  int64_t nq_el, nk_el, nl;
  if (!elems(&nq_el, {B, Hq, N, D}) || !elems(&nk_el, {B, Hkv, N, D}) || !elems(&nl, {B, Hq, N}) ||
      nq_el > INT64_MAX / 8)
    return fail(ATTN_ERR_SHAPE, "%s: tensor sizes overflow", name);
  if (N >= INT32_MAX || B > 65535 || Hq > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: N must be < 2^31, B and Hq <= 65535", name);
  const size_t need_min = attn_bwd_workspace_size(B, Hq, Hkv, N, D);
  // a workspace with room for the stored dS takes the product pass for dQ
  const size_t need_ds = use_scratch ? 0 : attn_bwd_ds_workspace_size(B, Hq, Hkv, N, D, causal);
  const bool use_ds = need_ds != 0 && workspace && workspace_bytes >= need_ds;
  const size_t need = use_ds ? need_ds : need_min;
  if (use_scratch) {
    if (need > lcattn::kNoAllocScratchBytes)
      return fail(ATTN_ERR_WORKSPACE, "%s: needs %zu bytes of scratch; the library holds %zu per GPU", name, need,
                  lcattn::kNoAllocScratchBytes);
  } else if (!workspace || workspace_bytes < need) {
    return fail(ATTN_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", name, need, workspace_bytes);
  }
  const void* ptrs[10] = {q, k, v, o, d_o, lse, dq, dk, dv, use_scratch ? q : workspace};
  for (int i = 0; i < 10; ++i)
    if (!aligned16(ptrs[i])) return fail(ATTN_ERR_ALIGN, "%s: pointers must be 16-byte aligned", name);
  // byte extents from each base (the whole tensor when contiguous)
  size_t qb = (size_t)nq_el * 2, kb = (size_t)nk_el * 2;
  const size_t lb = (size_t)nl * 4;
  const bool strided = q_strides || kv_strides;
  if (strided) {
    int64_t qsp, ksp;
    int st;
    if ((st = stride_check(name, "q", q_strides, B, Hq, N, D, 2, false, &qsp)) != ATTN_OK) return st;
    if ((st = stride_check(name, "k/v", kv_strides, B, Hkv, N, D, 2, false, &ksp)) != ATTN_OK) return st;
    // the gradients take the strides of their inputs: their rows must not overlap
    if ((st = stride_check(name, "dq", q_strides, B, Hq, N, D, 2, true, &qsp)) != ATTN_OK) return st;
    if ((st = stride_check(name, "dk/dv", kv_strides, B, Hkv, N, D, 2, true, &ksp)) != ATTN_OK) return st;
    qb = (size_t)qsp * 2;
    kb = (size_t)ksp * 2;
  }
  const void* ins[6] = {q, k, v, o, d_o, lse};
  const size_t inb[6] = {qb, kb, kb, qb, qb, lb};
  // the library's scratch is memory of its own, apart from every caller buffer
  const void* outs[4] = {dq, dk, dv, use_scratch ? nullptr : workspace};
  const size_t outb[4] = {qb, kb, kb, use_scratch ? 0 : need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], outb[i], ins[j], inb[j])) return fail(ATTN_ERR_ALIAS, "%s: outputs overlap inputs", name);
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return fail(ATTN_ERR_ALIAS, "%s: outputs overlap", name);
  }
  if (use_scratch) {  // every argument is valid: now the GPU's copy of the scratch
    const hipError_t e = lcattn::noalloc_scratch(static_cast<hipStream_t>(hip_stream), &workspace);
    if (e != hipSuccess) return hip_status(e, "attn_bwd_noalloc scratch");
  }
  lcattn::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.d_o = static_cast<const uint16_t*>(d_o);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.delta = static_cast<float*>(workspace);
  a.part = a.delta + lcattn::bwd_delta_floats(B, Hq, N);
  if (use_ds) {
    a.ds = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                       lcattn::bwd_ds_offset_bytes(B, Hq, Hkv, N, D));
    a.ds_head = lcattn::bwd_ds_head_elems(N, causal ? 1 : 0);
  }
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Nq = N;
  a.Nk = N;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  if (strided)
    for (int i = 0; i < 3; ++i) {
      a.qs[i] = q_strides[i];
      a.ks[i] = kv_strides[i];
    }
  char what[64];
  snprintf(what, sizeof(what), "%s launch", name);
  return hip_status(lcattn::launch_attn_bwd(a, B, D, static_cast<hipStream_t>(hip_stream), !use_scratch, true), what);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
             int64_t N, int D, float scale, int causal, void* hip_stream) {
  return bwd_entry("attn_bwd", q, k, v, o, d_o, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, D, scale,
                   causal, nullptr, nullptr, hip_stream);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                     void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int64_t N, int D, float scale, int causal,
                     void* hip_stream) {
  return bwd_entry("attn_bwd_noalloc", q, k, v, o, d_o, lse, dq, dk, dv, nullptr, 0, B, Hq, Hkv, N, D, scale, causal,
                   nullptr, nullptr, hip_stream, true);
}

size_t attn_bwd_noalloc_max_scratch(void) { return lcattn::kNoAllocScratchBytes; }

int attn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                     int64_t N, int D, float scale, int causal, const int64_t* q_strides,
                     const int64_t* kv_strides, void* hip_stream) {
  if (!q_strides || !kv_strides) return fail(ATTN_ERR_NULL, "attn_bwd_strided: strides must be non-null");
  return bwd_entry("attn_bwd_strided", q, k, v, o, d_o, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N,
                   D, scale, causal, q_strides, kv_strides, hip_stream);
}

int attn_bwd_delta(const void* o, const void* d_o, float* delta, int B, int Hq, int64_t Nq, int D,
                   void* hip_stream) {
  if (!o || !d_o || !delta) return fail(ATTN_ERR_NULL, "attn_bwd_delta: pointers must be non-null");
  if (B < 1 || Hq < 1 || Nq < 1 || D < 1) return fail(ATTN_ERR_SHAPE, "attn_bwd_delta: sizes must be >= 1");
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd_delta: D=%d (supported: 64, 128)", D);
  int64_t el, rows;
  if (!elems(&el, {B, Hq, Nq, D}) || !elems(&rows, {B, Hq, Nq}) || el > INT64_MAX / 8 ||
      (rows * (D / 8) + 255) / 256 > INT32_MAX)
    return fail(ATTN_ERR_SHAPE, "attn_bwd_delta: tensor sizes overflow");
  if (!aligned16(o) || !aligned16(d_o) || !aligned16(delta))
    return fail(ATTN_ERR_ALIGN, "attn_bwd_delta: pointers must be 16-byte aligned");
  if (overlap(delta, (size_t)rows * 4, o, (size_t)el * 2) || overlap(delta, (size_t)rows * 4, d_o, (size_t)el * 2))
    return fail(ATTN_ERR_ALIAS, "attn_bwd_delta: delta overlaps an input");
  return hip_status(lcattn::launch_bwd_delta(static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(d_o),
                                             delta, rows, D, static_cast<hipStream_t>(hip_stream)),
                    "attn_bwd_delta launch");
}

size_t attn_bwd_block_workspace_size(int B, int Hq, int Hkv, int64_t Nk, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nk < 1 || D < 1 || Hq % Hkv) return 0;
  int64_t el;
  if (!elems(&el, {B, Hq, Nk, D}) || el > INT64_MAX / 16) return 0;
  return (size_t)lcattn::bwd_part_floats(B, Hq, Hkv, Nk, D) * 4;
}

size_t attn_bwd_block_ds_workspace_size(int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || Hq % Hkv || (D != 64 && D != 128)) return 0;
  int64_t el;
  if (!elems(&el, {B, Hq, Nk, D}) || el > INT64_MAX / 16) return 0;
  // the uniform rows: B * Hq * ceil(Nq / 64) * ceil(Nk / 128) * 2 blocks of
  // 8 KiB (checked against overflow before multiplying out)
  const double approx = (double)B * Hq * ((double)Nq + 64) * ((double)Nk + 128) * 2.0;
  if (approx > 9.0e18) return 0;
  return (size_t)lcattn::bwd_block_ds_workspace_bytes(B, Hq, Hkv, Nq, Nk, D);
}

// Validation of one block-backward call; fills the kernel arguments and the
// byte ranges of its inputs (6) and outputs (7, null when absent).  allow_ds:
// a workspace of attn_bwd_block_ds_workspace_size bytes selects the stored-dS
// dQ (single calls; the grouped launch keeps the recomputing pass).
static int bwd_block_check(const char* name, const void* q, const void* k, const void* v, const void* d_o,
                           const float* lse, const float* delta, float* dq_acc, float* dk_acc, float* dv_acc,
                           void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq,
                           int Hkv, int64_t Nq, int64_t Nk, int D, float scale, int causal, int64_t q_pos0,
                           int64_t k_pos0, int dq_accumulate, int dkv_accumulate, lcattn::BwdArgs* args,
                           const void* (&ins)[6], size_t (&inb)[6], const void* (&outs)[7], size_t (&outb)[7],
                           bool allow_ds = false) {
  if (!q || !k || !v || !d_o || !lse || !delta)
    return fail(ATTN_ERR_NULL, "%s: q, k, v, d_o, lse and delta must be non-null", name);
  if (!dq_acc && !dq) return fail(ATTN_ERR_NULL, "%s: dq_acc or dq must be set", name);
  if (!dk_acc != !dv_acc || !dk != !dv)
    return fail(ATTN_ERR_NULL, "%s: dk_acc and dv_acc (and dk and dv) are set together", name);
  if (!dk_acc && !dk) return fail(ATTN_ERR_NULL, "%s: dk_acc/dv_acc or dk/dv must be set", name);
  if ((dq_accumulate && !dq_acc) || (dkv_accumulate && !dk_acc))
    return fail(ATTN_ERR_NULL, "%s: accumulating needs the fp32 accumulators", name);
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || D < 1)
    return fail(ATTN_ERR_SHAPE, "%s: sizes must be >= 1", name);
  if (Hq % Hkv) return fail(ATTN_ERR_SHAPE, "%s: Hkv=%d does not divide Hq=%d", name, Hkv, Hq);
  if (q_pos0 < 0 || k_pos0 < 0) return fail(ATTN_ERR_SHAPE, "%s: position offsets must be >= 0", name);
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: D=%d (supported: 64, 128)", name, D);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(ATTN_ERR_UNSUPPORTED, "%s: scale must be > 0", name);
  int64_t nq_el, nk_el, nl, hk_el;
  if (!elems(&nq_el, {B, Hq, Nq, D}) || !elems(&nk_el, {B, Hkv, Nk, D}) || !elems(&nl, {B, Hq, Nq}) ||
      !elems(&hk_el, {B, Hq, Nk, D}) || nq_el > INT64_MAX / 8 || hk_el > INT64_MAX / 16)
    return fail(ATTN_ERR_SHAPE, "%s: tensor sizes overflow", name);
  if (Nq >= (int64_t(1) << 30) || Nk >= (int64_t(1) << 30) || B > 65535 || Hq > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: Nq and Nk must be < 2^30, B and Hq <= 65535", name);
  const size_t need_min = attn_bwd_block_workspace_size(B, Hq, Hkv, Nk, D);
  const size_t need_ds = allow_ds ? attn_bwd_block_ds_workspace_size(B, Hq, Hkv, Nq, Nk, D) : 0;
  const bool use_ds = need_ds != 0 && workspace && workspace_bytes >= need_ds;
  const size_t need = use_ds ? need_ds : need_min;
  if (need && (!workspace || workspace_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", name, need, workspace_bytes);
  const void* all[13] = {q, k, v, d_o, lse, delta, dq_acc, dk_acc, dv_acc, dq, dk, dv, need ? workspace : nullptr};
  for (int i = 0; i < 13; ++i)
    if (all[i] && !aligned16(all[i])) return fail(ATTN_ERR_ALIGN, "%s: pointers must be 16-byte aligned", name);
  const size_t qb = (size_t)nq_el * 2, kb = (size_t)nk_el * 2, lb = (size_t)nl * 4;
  const void* in_[6] = {q, k, v, d_o, lse, delta};
  const size_t inb_[6] = {qb, kb, kb, qb, lb, lb};
  const void* out_[7] = {dq_acc, dk_acc, dv_acc, dq, dk, dv, need ? workspace : nullptr};
  const size_t outb_[7] = {qb * 2, kb * 2, kb * 2, qb, kb, kb, need};
  for (int i = 0; i < 7; ++i) {
    outs[i] = out_[i];
    outb[i] = out_[i] ? outb_[i] : 0;
    if (i < 6) {
      ins[i] = in_[i];
      inb[i] = inb_[i];
    }
  }
  for (int i = 0; i < 7; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], outb[i], ins[j], inb[j])) return fail(ATTN_ERR_ALIAS, "%s: outputs overlap inputs", name);
    for (int j = i + 1; j < 7; ++j)
      if (outs[j] && overlap(outs[i], outb[i], outs[j], outb[j]))
        return fail(ATTN_ERR_ALIAS, "%s: outputs overlap", name);
  }
  lcattn::BwdArgs& a = *args;
  a = lcattn::BwdArgs{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = nullptr;  // Dv is given
  a.d_o = static_cast<const uint16_t*>(d_o);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.delta = const_cast<float*>(delta);
  a.part = static_cast<float*>(workspace);
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.dpos = (int)std::max(-Nq, std::min(q_pos0 - k_pos0, Nk));
  a.dq_mode = dq_acc ? (dq_accumulate ? 2 : 1) : 0;
  a.dq_acc = dq_acc;
  a.dkv_mode = dk_acc ? (dkv_accumulate ? 2 : 1) : 0;
  a.dk_acc = dk_acc;
  a.dv_acc = dv_acc;
  if (use_ds) {
    a.ds = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                       lcattn::bwd_block_ds_offset_bytes(B, Hq, Hkv, Nk, D));
    a.ds_head = lcattn::bwd_block_ds_head_elems(Nq, Nk);
    a.ds_uniform = 1;
  }
  return ok();
}

int attn_bwd_block(const void* q, const void* k, const void* v, const void* d_o, const float* lse,
                   const float* delta, float* dq_acc, float* dk_acc, float* dv_acc, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D,
                   float scale, int causal, int64_t q_pos0, int64_t k_pos0, int dq_accumulate, int dkv_accumulate,
                   void* hip_stream) {
  lcattn::BwdArgs a;
  const void* ins[6];
  size_t inb[6];
  const void* outs[7];
  size_t outb[7];
  const int st = bwd_block_check("attn_bwd_block", q, k, v, d_o, lse, delta, dq_acc, dk_acc, dv_acc, dq, dk, dv,
                                 workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, D, scale, causal, q_pos0, k_pos0,
                                 dq_accumulate, dkv_accumulate, &a, ins, inb, outs, outb, true);
  if (st != ATTN_OK) return st;
  return hip_status(lcattn::launch_attn_bwd(a, B, D, static_cast<hipStream_t>(hip_stream), true, false),
                    "attn_bwd_block launch");
}

int attn_bwd_block_group(const attn_bwd_block_call* calls, int n, int B, int Hq, int Hkv, int D, float scale,
                         int causal, void* hip_stream) {
  const char* name = "attn_bwd_block_group";
  if (!calls) return fail(ATTN_ERR_NULL, "%s: null call array", name);
  if (n < 1 || n > ATTN_MAX_BWD_GROUP)
    return fail(ATTN_ERR_SHAPE, "%s: n=%d calls (1 .. %d)", name, n, ATTN_MAX_BWD_GROUP);
  if ((int64_t)B * n > 65535) return fail(ATTN_ERR_UNSUPPORTED, "%s: B * n must be <= 65535", name);
  lcattn::BwdArgs args[ATTN_MAX_BWD_GROUP];
  const void* ins[ATTN_MAX_BWD_GROUP][6];
  size_t inb[ATTN_MAX_BWD_GROUP][6];
  const void* outs[ATTN_MAX_BWD_GROUP][7];
  size_t outb[ATTN_MAX_BWD_GROUP][7];
  for (int c = 0; c < n; ++c) {
    const attn_bwd_block_call& x = calls[c];
    const int st = bwd_block_check(name, x.q, x.k, x.v, x.d_o, x.lse, x.delta, x.dq_acc, x.dk_acc, x.dv_acc, x.dq,
                                   x.dk, x.dv, x.workspace, x.workspace_bytes, B, Hq, Hkv, x.Nq, x.Nk, D, scale,
                                   causal, x.q_pos0, x.k_pos0, x.dq_accumulate, x.dkv_accumulate, &args[c], ins[c],
                                   inb[c], outs[c], outb[c]);
    if (st != ATTN_OK) {
      char detail[sizeof(g_last_error)];
      snprintf(detail, sizeof(detail), "%s", g_last_error);
      return fail(st, "%s (call %d)", detail, c);
    }
  }
  // the calls run side by side: no call may write what another reads or writes
  for (int c = 0; c < n; ++c)
    for (int d = 0; d < n; ++d) {
      if (c == d) continue;
      for (int i = 0; i < 7; ++i) {
        if (!outs[c][i]) continue;
        for (int j = 0; j < 6; ++j)
          if (overlap(outs[c][i], outb[c][i], ins[d][j], inb[d][j]))
            return fail(ATTN_ERR_ALIAS, "%s: outputs of call %d overlap inputs of call %d", name, c, d);
        for (int j = 0; j < 7; ++j)
          if (outs[d][j] && overlap(outs[c][i], outb[c][i], outs[d][j], outb[d][j]))
            return fail(ATTN_ERR_ALIAS, "%s: outputs of calls %d and %d overlap", name, c, d);
      }
    }
  return hip_status(lcattn::launch_attn_bwd_group(args, n, B, D, static_cast<hipStream_t>(hip_stream)),
                    "attn_bwd_block_group launch");
}

// Validates one tensor of a relayout and fills its job; returns a status.
static int relayout_job(const char* name, bool to_head, const void* in, void* out, int P, int64_t N, int H, int D,
                        int elem_bytes, lcattn::TransposeJob* job, size_t* in_bytes, size_t* out_bytes) {
  if (!in || !out) return fail(ATTN_ERR_NULL, "%s: null pointer", name);
  if (P < 1 || N < 1 || H < 1 || D < 1) return fail(ATTN_ERR_SHAPE, "%s: sizes must be >= 1", name);
  if (N % P) return fail(ATTN_ERR_SHAPE, "%s: P=%d does not divide N=%lld", name, P, (long long)N);
  if (H < P && !to_head)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: H=%d < P=%d: replicated heads are summed by head_to_seq_reduce", name, H,
                P);
  if (H < P && P % H) return fail(ATTN_ERR_SHAPE, "%s: H=%d does not divide P=%d", name, H, P);
  if (H >= P && H % P) return fail(ATTN_ERR_SHAPE, "%s: P=%d does not divide H=%d", name, P, H);
  const int rep = H < P ? P / H : 1;  // ranks that share one head
  if (elem_bytes != 2 && elem_bytes != 4) return fail(ATTN_ERR_UNSUPPORTED, "%s: elem_bytes must be 2 or 4", name);
  const int64_t row_bytes = (int64_t)D * elem_bytes;
  if (row_bytes % 16 || ((row_bytes / 16) & (row_bytes / 16 - 1)))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: D*elem_bytes=%lld must be 16 times a power of two", name,
                (long long)row_bytes);
  int64_t units, out_units;
  if (!elems(&units, {N, H, row_bytes / 16}) || !elems(&out_units, {N, H, rep, row_bytes / 16}) ||
      out_units >= (int64_t(1) << 32))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: tensor has 2^32 or more 16-byte units", name);
  if (!aligned16(in) || !aligned16(out)) return fail(ATTN_ERR_ALIGN, "%s: pointers must be 16-byte aligned", name);
  if (overlap(in, (size_t)units * 16, out, (size_t)out_units * 16))
    return fail(ATTN_ERR_ALIAS, "%s: in and out overlap", name);
  // seq->head: out[h][n] = in[n][h] (A = H, Bn = N); head->seq: out[n][h] = in[h][n].
  job->in = in;
  job->out = out;
  job->A = to_head ? (unsigned)H : (unsigned)N;
  job->Bn = to_head ? (unsigned)N : (unsigned)H;
  job->rep = (unsigned)rep;
  *in_bytes = (size_t)units * 16;
  *out_bytes = (size_t)out_units * 16;
  return ATTN_OK;
}

static int relayout(const char* name, bool to_head, const void* in, void* out, int P, int64_t N, int H, int D,
                    int elem_bytes, void* hip_stream) {
  lcattn::TransposeJob job;
  size_t ib, ob;
  const int st = relayout_job(name, to_head, in, out, P, N, H, D, elem_bytes, &job, &ib, &ob);
  if (st != ATTN_OK) return st;
  // head groups fastest in both directions: consecutive workgroups then walk
  // the token-major side ([N, H, D]: the input of seq->head, the output of
  // head->seq) sequentially, measured 6% (seq->head) and 18% (head->seq)
  // faster than the other order
  return hip_status(lcattn::launch_transpose_rows_batch(&job, 1, (unsigned)(D * elem_bytes), to_head,
                                                        static_cast<hipStream_t>(hip_stream)),
                    name);
}

static_assert(ATTN_MAX_RELAYOUT_BATCH == lcattn::kMaxRelayoutBatch, "batch limit of the header and the kernel");

static int relayout_batch(const char* name, bool to_head, int n, const void* const* ins, void* const* outs,
                          const int* H, int P, int64_t N, int D, int elem_bytes, void* hip_stream) {
  if (!ins || !outs || !H) return fail(ATTN_ERR_NULL, "%s: null array", name);
  if (n < 1 || n > ATTN_MAX_RELAYOUT_BATCH)
    return fail(ATTN_ERR_SHAPE, "%s: n=%d tensors (1 .. %d)", name, n, ATTN_MAX_RELAYOUT_BATCH);
  lcattn::TransposeJob jobs[ATTN_MAX_RELAYOUT_BATCH];
  size_t ib[ATTN_MAX_RELAYOUT_BATCH], ob[ATTN_MAX_RELAYOUT_BATCH];
  unsigned long long blocks = 0;
  for (int j = 0; j < n; ++j) {
    const int st = relayout_job(name, to_head, ins[j], outs[j], P, N, H[j], D, elem_bytes, &jobs[j], &ib[j], &ob[j]);
    if (st != ATTN_OK) {
      char detail[sizeof(g_last_error)];
      snprintf(detail, sizeof(detail), "%s", g_last_error);
      return fail(st, "%s (tensor %d)", detail, j);
    }
    blocks += (unsigned long long)jobs[j].A * jobs[j].Bn;  // >= the workgroups of the job
  }
  if (blocks > 0xFFFFFFFFull) return fail(ATTN_ERR_UNSUPPORTED, "%s: too many rows in one launch", name);
  // every output is written while every input is still being read
  for (int j = 0; j < n; ++j)
    for (int i = 0; i < n; ++i) {
      if (i != j && overlap(ins[i], ib[i], outs[j], ob[j]))
        return fail(ATTN_ERR_ALIAS, "%s: output %d overlaps input %d", name, j, i);
      if (i < j && overlap(outs[i], ob[i], outs[j], ob[j]))
        return fail(ATTN_ERR_ALIAS, "%s: outputs %d and %d overlap", name, i, j);
    }
  return hip_status(lcattn::launch_transpose_rows_batch(jobs, n, (unsigned)(D * elem_bytes), to_head,
                                                        static_cast<hipStream_t>(hip_stream)),
                    name);
}

int seq_to_head_relayout(const void* in, void* out, int P, int64_t N, int H, int D, int elem_bytes,
                         void* hip_stream) {
  return relayout("seq_to_head_relayout", true, in, out, P, N, H, D, elem_bytes, hip_stream);
}

int head_to_seq_relayout(const void* in, void* out, int P, int64_t N, int H, int D, int elem_bytes,
                         void* hip_stream) {
  return relayout("head_to_seq_relayout", false, in, out, P, N, H, D, elem_bytes, hip_stream);
}

int seq_to_head_relayout_batch(int n, const void* const* ins, void* const* outs, const int* H, int P, int64_t N,
                               int D, int elem_bytes, void* hip_stream) {
  return relayout_batch("seq_to_head_relayout_batch", true, n, ins, outs, H, P, N, D, elem_bytes, hip_stream);
}

int head_to_seq_relayout_batch(int n, const void* const* ins, void* const* outs, const int* H, int P, int64_t N,
                               int D, int elem_bytes, void* hip_stream) {
  return relayout_batch("head_to_seq_relayout_batch", false, n, ins, outs, H, P, N, D, elem_bytes, hip_stream);
}

int head_to_seq_reduce(const void* in, int in_dtype, void* out, int P, int64_t N, int H, int D, void* hip_stream) {
  const char* name = "head_to_seq_reduce";
  if (!in || !out) return fail(ATTN_ERR_NULL, "%s: null pointer", name);
  if (P < 1 || N < 1 || H < 1 || D < 1) return fail(ATTN_ERR_SHAPE, "%s: sizes must be >= 1", name);
  if (N % P) return fail(ATTN_ERR_SHAPE, "%s: P=%d does not divide N=%lld", name, P, (long long)N);
  if (H < P ? P % H : H % P) return fail(ATTN_ERR_SHAPE, "%s: H=%d and P=%d: one must divide the other", name, H, P);
  if (in_dtype != ATTN_BF16 && in_dtype != ATTN_FP32)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: in_dtype=%d (ATTN_BF16 or ATTN_FP32)", name, in_dtype);
  if (D % 8) return fail(ATTN_ERR_UNSUPPORTED, "%s: D=%d must be a multiple of 8", name, D);
  const int rep = H < P ? P / H : 1;
  int64_t out_el, in_el;
  if (!elems(&out_el, {N, H, D}) || !elems(&in_el, {N, H, rep, D}) || in_el > INT64_MAX / 8 ||
      (out_el / 8 + 255) / 256 > INT32_MAX)
    return fail(ATTN_ERR_SHAPE, "%s: tensor sizes overflow", name);
  if (!aligned16(in) || !aligned16(out)) return fail(ATTN_ERR_ALIGN, "%s: pointers must be 16-byte aligned", name);
  if (overlap(in, (size_t)in_el * (in_dtype == ATTN_FP32 ? 4 : 2), out, (size_t)out_el * 2))
    return fail(ATTN_ERR_ALIAS, "%s: in and out overlap", name);
  return hip_status(lcattn::launch_sum_replicas(in, in_dtype == ATTN_FP32, static_cast<uint16_t*>(out), H, N, D, rep,
                                                static_cast<hipStream_t>(hip_stream)),
                    name);
}

}  // extern "C"
