// C ABI of libfa.so: argument validation, then the kernel launchers.
//
// Every check runs before any work is enqueued, so a rejected call never
// touches the stream or device memory (and can be exercised on a machine
// without a GPU).  The only HIP calls a call makes before its checks pass are
// reads of the current device and its compute-unit count, which size the
// launch plans and workspaces.
#include "fa.h"

#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

static_assert(FA_STATIC_SCRATCH_BYTES == fa::kStaticScratchBytes, "scratch size");

namespace {

struct Range {
  uintptr_t lo;
  uintptr_t hi;  // one past the end
};

Range range_of(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Shape, head-dim and scale checks shared by every entry point.  On success
// writes the element count of one [B, H, N, d] tensor and of one [B, H, N]
// statistic.  d is 64 or 128 everywhere; the bf16 entry points (wide = true)
// also take 256.
int check_common(int B, int H, int N, int d, float scale, size_t* tensor_elems,
                 size_t* row_elems, bool wide = false) {
  if (B < 0 || H < 0 || N < 0 || N > FA_MAX_N) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && !(wide && d == 256)) return FA_ERR_HEADDIM;
  const long long bh = (long long)B * (long long)H;
  if (bh > INT_MAX) return FA_ERR_SHAPE;
  // grid size: one workgroup per (batch*head, 64-row tile) at most
  if (bh * (((long long)N + 63) / 64) > INT_MAX) return FA_ERR_SHAPE;
  // every elementwise grid (one thread per 8 features of a row) stays < 2^31 blocks
  if (bh * (long long)N > (1LL << 34)) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  *row_elems = (size_t)bh * (size_t)N;
  *tensor_elems = *row_elems * (size_t)d;
  return FA_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// True if any output overlaps an input or another output.
bool any_alias(const Range* in, int nin, const Range* out, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(out[i], in[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(out[i], out[j])) return true;
  }
  return false;
}

// Grouped-query head counts: H query heads share Hkv key / value heads, each
// key / value head serving H / Hkv consecutive query heads.
int check_heads(int H, int Hkv) {
  if (H == 0) return Hkv >= 0 ? FA_OK : FA_ERR_SHAPE;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_SHAPE;
  return FA_OK;
}

int fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  size_t te = 0, re = 0;
  int st = check_common(B, H, N, d, scale, &te, &re, true);
  if (st != FA_OK) return st;
  st = check_heads(H, Hkv);
  if (st != FA_OK) return st;
  if (re == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return FA_ERR_ALIGN;
  const size_t tb = te * 2;
  const size_t kvb = tb / (size_t)(H / Hkv);
  const Range in[3] = {range_of(q, tb), range_of(k, kvb), range_of(v, kvb)};
  const Range out[2] = {range_of(o, tb), range_of(lse, re * 4)};
  if (any_alias(in, 3, out, 2)) return FA_ERR_ALIAS;
  const fa::FwdPlan pl = fa::fwd_plan(B * H, H / Hkv, N, N, d, false, fa::device_cus());
  return from_hip(fa::launch_fwd_bf16_kv(q, k, v, o, lse, nullptr, B * H, N, N, d, H / Hkv,
                                         causal != 0, scale, pl, stream));
}

// The three backward stages on validated arguments.  hsplit > 1 needs the
// split partials after the plain workspace (grouped-query heads only).
int bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, void* workspace, int B, int H,
               int Hkv, int Nq, int Nk, int d, int hsplit, int causal, float scale,
               hipStream_t stream) {
  const bool has_q = (size_t)B * H * Nq > 0;
  const size_t kve = H > 0 ? (size_t)B * (size_t)Hkv * (size_t)Nk * (size_t)d : 0;
  const int BH = B * H;
  hipError_t e = hipSuccess;
  if (has_q) e = fa::launch_bwd_pre(o, dout, lse, workspace, BH, Nq, d, stream);
  if (e == hipSuccess && kve > 0) {
    if (has_q)
      e = fa::launch_bwd_main(q, k, v, dout, dk, dv, workspace, BH, Nq, Nk, d, H / Hkv, hsplit,
                              causal != 0, scale, stream);
    else   // no queries: every key's gradient is 0
      e = fa::launch_zero_bf16(dk, dv, kve, stream);
  }
  if (e == hipSuccess && has_q)
    e = fa::launch_bwd_finalize(q, k, v, dout, dq, workspace, BH, Nq, Nk, d, H / Hkv,
                                causal != 0, scale, stream);
  return from_hip(e);
}

int bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
             float scale, hipStream_t stream) {
  size_t te = 0, re = 0;
  int st = check_common(B, H, Nq, d, scale, &te, &re, true);
  if (st != FA_OK) return st;
  if (Nk < 0 || Nk > FA_MAX_N) return FA_ERR_SHAPE;
  st = check_heads(H, Hkv);
  if (st != FA_OK) return st;
  const size_t kve = H > 0 ? (size_t)B * (size_t)Hkv * (size_t)Nk * (size_t)d : 0;
  if (re == 0 && kve == 0) return FA_OK;
  const bool has_q = re > 0, has_k = kve > 0;
  if ((has_q && (!q || !o || !dout || !lse || !dq || !workspace)) ||
      (has_k && (!k || !v || !dk || !dv)))
    return FA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(dout) ||
      misaligned(lse) || misaligned(dq) || misaligned(dk) || misaligned(dv) ||
      misaligned(workspace))
    return FA_ERR_ALIGN;
  size_t need = fa::bwd_workspace_bytes(B * H, Nq, d);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  // a larger workspace lets grouped-query heads split over more workgroups
  int hsplit = has_q && has_k && H != Hkv
                   ? fa::bwd_head_split(B * Hkv, H / Hkv, Nq, Nk, d, causal != 0,
                                        fa::device_cus())
                   : 1;
  if (hsplit > 1) {
    const size_t full = need + fa::bwd_split_bytes(B * Hkv, Nk, d, hsplit);
    if (workspace_bytes >= full)
      need = full;
    else
      hsplit = 1;
  }
  const size_t tb = te * 2, kvb = kve * 2;
  const Range in[6] = {range_of(q, tb),    range_of(k, kvb),   range_of(v, kvb),
                       range_of(o, tb),    range_of(dout, tb), range_of(lse, re * 4)};
  const Range out[4] = {range_of(dq, tb), range_of(dk, kvb), range_of(dv, kvb),
                        range_of(workspace, need)};
  if (any_alias(in, 6, out, 4)) return FA_ERR_ALIAS;
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Hkv, Nq, Nk, d, hsplit,
                    causal, scale, stream);
}

// Nq query rows against Nk keys: sizes of q / o ([B, H, Nq, d]), k / v
// ([B, Hkv, Nk, d]) and lse ([B, H, Nq]) in elements.
int check_kv(int B, int H, int Hkv, int Nq, int Nk, int d, float scale, size_t* q_elems,
             size_t* kv_elems, size_t* rows) {
  size_t te = 0, re = 0;
  int st = check_common(B, H, Nq, d, scale, &te, &re, true);
  if (st != FA_OK) return st;
  if (Nk < 0 || Nk > FA_MAX_N) return FA_ERR_SHAPE;
  st = check_heads(H, Hkv);
  if (st != FA_OK) return st;
  *q_elems = te;
  *rows = re;
  *kv_elems = H > 0 ? (size_t)B * (size_t)Hkv * (size_t)Nk * (size_t)d : 0;
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_fwd_kv_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d) {
  size_t te = 0, re = 0;
  if (check_common(B, H, Nq, d, 1.f, &te, &re, true) != FA_OK) return 0;
  if (Nk < 0 || Nk > FA_MAX_N || re == 0 || check_heads(H, Hkv) != FA_OK) return 0;
  return fa::fwd_workspace_bytes(B * H, H / Hkv, Nq, Nk, d, fa::device_cus());
}

int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
              size_t workspace_bytes, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
              float scale, hipStream_t stream) {
  size_t qe = 0, kve = 0, re = 0;
  int st = check_kv(B, H, Hkv, Nq, Nk, d, scale, &qe, &kve, &re);
  if (st != FA_OK) return st;
  if (re == 0) return FA_OK;
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return FA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse) ||
      misaligned(workspace))
    return FA_ERR_ALIGN;
  const int cus = fa::device_cus();
  const size_t need = fa::fwd_workspace_bytes(B * H, H / Hkv, Nq, Nk, d, cus);
  if (need > 0 && workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (need > 0 && !workspace) return FA_ERR_NULL;
  const Range in[3] = {range_of(q, qe * 2), range_of(k, kve * 2), range_of(v, kve * 2)};
  const Range out[3] = {range_of(o, qe * 2), range_of(lse, re * 4),
                        range_of(workspace, need)};
  if (any_alias(in, 3, out, 3)) return FA_ERR_ALIAS;
  const fa::FwdPlan pl = fa::fwd_plan(B * H, H / Hkv, Nq, Nk, d, need > 0, cus);
  return from_hip(fa::launch_fwd_bf16_kv(q, k, v, o, lse, need > 0 ? workspace : nullptr, B * H,
                                         Nq, Nk, d, H / Hkv, causal != 0, scale, pl, stream));
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, int causal, float scale, hipStream_t stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, H, N, d, causal, scale, stream);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, float q_scale,
               float k_scale, float v_scale, int B, int H, int N, int d, int causal, float scale,
               hipStream_t stream) {
  size_t te = 0, re = 0;
  int st = check_common(B, H, N, d, scale, &te, &re);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_HEADDIM;
  const float score = scale * q_scale * k_scale;
  if (!isfinite(q_scale) || !isfinite(k_scale) || !isfinite(v_scale) || !isfinite(score))
    return FA_ERR_SCALE;
  if (re == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return FA_ERR_ALIGN;
  const Range in[3] = {range_of(q, te), range_of(k, te), range_of(v, te)};
  const Range out[2] = {range_of(o, te * 2), range_of(lse, re * 4)};
  if (any_alias(in, 3, out, 2)) return FA_ERR_ALIAS;
  return from_hip(
      fa::launch_fwd_fp8(q, k, v, o, lse, B * H, N, d, causal != 0, score, v_scale, stream));
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
               int N, int d, int causal, float scale, hipStream_t stream) {
  size_t te = 0, re = 0;
  int st = check_common(B, H, N, d, scale, &te, &re);
  if (st != FA_OK) return st;
  if (re == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return FA_ERR_ALIGN;
  const size_t tb = te * 4;
  const Range in[3] = {range_of(q, tb), range_of(k, tb), range_of(v, tb)};
  const Range out[2] = {range_of(o, tb), range_of(lse, re * 4)};
  if (any_alias(in, 3, out, 2)) return FA_ERR_ALIAS;
  return from_hip(fa::launch_fwd_f32(q, k, v, o, lse, B * H, N, d, causal != 0, scale, stream));
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  size_t te = 0, re = 0;
  if (check_common(B, H, N, d, 1.0f, &te, &re, true) != FA_OK) return 0;
  return fa::bwd_workspace_bytes(B * H, N, d);
}

size_t fa_bwd_kv_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d) {
  size_t te = 0, re = 0;
  if (check_common(B, H, Nq, d, 1.0f, &te, &re, true) != FA_OK) return 0;
  if (Nk < 0 || Nk > FA_MAX_N || check_heads(H, Hkv) != FA_OK) return 0;
  if (H == 0) return fa::bwd_workspace_bytes(0, Nq, d);
  return fa::bwd_kv_workspace_bytes(B * H, H / Hkv, Nq, Nk, d, fa::device_cus());
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale,
           hipStream_t stream) {
  return bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, N, N,
                  d, causal, scale, stream);
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, int B, int H, int Hkv, int N, int d, int causal,
               float scale, hipStream_t stream) {
  return bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Hkv, N,
                  N, d, causal, scale, stream);
}

int fa_bwd_kv(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, void* workspace,
              size_t workspace_bytes, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
              float scale, hipStream_t stream) {
  return bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Hkv, Nq,
                  Nk, d, causal, scale, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   int causal, float scale, hipStream_t stream) {
  size_t te = 0, re = 0;
  int st = check_common(B, H, N, d, scale, &te, &re, true);
  if (st != FA_OK) return st;
  if (re == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(dout) ||
      misaligned(lse) || misaligned(dq) || misaligned(dk) || misaligned(dv))
    return FA_ERR_ALIGN;
  if (fa::bwd_workspace_bytes(B * H, N, d) > fa::kStaticScratchBytes) return FA_ERR_SCRATCH;
  const size_t tb = te * 2;
  const Range in[6] = {range_of(q, tb), range_of(k, tb),    range_of(v, tb),
                       range_of(o, tb), range_of(dout, tb), range_of(lse, re * 4)};
  const Range out[3] = {range_of(dq, tb), range_of(dk, tb), range_of(dv, tb)};
  if (any_alias(in, 6, out, 3)) return FA_ERR_ALIAS;
  void* scratch = nullptr;
  if (fa::static_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, scratch, B, H, H, N, N, d, 1, causal,
                    scale, stream);
}

int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, void* workspace,
                      size_t workspace_bytes, int B, int H, int N, int d, hipStream_t stream) {
  size_t te = 0, re = 0;
  int st = check_common(B, H, N, d, 1.0f, &te, &re, true);
  if (st != FA_OK) return st;
  if (re == 0) return FA_OK;
  if (!o || !dout || !lse || !workspace) return FA_ERR_NULL;
  if (misaligned(o) || misaligned(dout) || misaligned(lse) || misaligned(workspace))
    return FA_ERR_ALIGN;
  const size_t need = fa::bwd_workspace_bytes(B * H, N, d);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  const size_t tb = te * 2;
  const Range in[3] = {range_of(o, tb), range_of(dout, tb), range_of(lse, re * 4)};
  const Range out[1] = {range_of(workspace, need)};
  if (any_alias(in, 3, out, 1)) return FA_ERR_ALIAS;
  return from_hip(fa::launch_bwd_pre(o, dout, lse, workspace, B * H, N, d, stream));
}

int fa_bwd_main(const void* q, const void* k, const void* v, const void* dout, void* dk,
                void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                int causal, float scale, hipStream_t stream) {
  size_t te = 0, re = 0;
  int st = check_common(B, H, N, d, scale, &te, &re, true);
  if (st != FA_OK) return st;
  if (re == 0) return FA_OK;
  if (!q || !k || !v || !dout || !dk || !dv || !workspace) return FA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(dout) || misaligned(dk) ||
      misaligned(dv) || misaligned(workspace))
    return FA_ERR_ALIGN;
  const size_t need = fa::bwd_workspace_bytes(B * H, N, d);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  const size_t tb = te * 2;
  const Range in[4] = {range_of(q, tb), range_of(k, tb), range_of(v, tb), range_of(dout, tb)};
  const Range out[3] = {range_of(dk, tb), range_of(dv, tb), range_of(workspace, need)};
  if (any_alias(in, 4, out, 3)) return FA_ERR_ALIAS;
  return from_hip(fa::launch_bwd_main(q, k, v, dout, dk, dv, workspace, B * H, N, N, d, 1, 1,
                                      causal != 0, scale, stream));
}

int fa_bwd_finalize(const void* q, const void* k, const void* v, const void* dout, void* dq,
                    const void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                    int causal, float scale, hipStream_t stream) {
  size_t te = 0, re = 0;
  int st = check_common(B, H, N, d, scale, &te, &re, true);
  if (st != FA_OK) return st;
  if (re == 0) return FA_OK;
  if (!dq || !workspace) return FA_ERR_NULL;
  if (d != 64 && (!q || !k || !v || !dout)) return FA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(dout) || misaligned(dq) ||
      misaligned(workspace))
    return FA_ERR_ALIGN;
  const size_t need = fa::bwd_workspace_bytes(B * H, N, d);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  const size_t tb = te * 2;
  const Range in[5] = {range_of(workspace, need), range_of(q, tb), range_of(k, tb),
                       range_of(v, tb), range_of(dout, tb)};
  const Range out[1] = {range_of(dq, tb)};
  if (any_alias(in, d == 64 ? 1 : 5, out, 1)) return FA_ERR_ALIAS;
  return from_hip(fa::launch_bwd_finalize(q, k, v, dout, dq, workspace, B * H, N, N, d, 1,
                                          causal != 0, scale, stream));
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "invalid shape (B, H or N negative, N too large, size overflow, or H not a "
             "multiple of Hkv)";
    case FA_ERR_HEADDIM:
      return "unsupported head dimension (64 or 128; the bf16 entry points also take 256)";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_HIP: return "HIP kernel launch failed";
    case FA_ERR_WORKSPACE: return "workspace too small";
    case FA_ERR_SCRATCH:
      return "problem needs more scratch than the library's static buffer holds "
             "(fa_bwd_noalloc: at most FA_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
