// Kernel launchers called by the C ABI layer (fa_api.cpp).  Arguments are
// already validated there; each launcher only enqueues work on `stream` and
// returns the launch status.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

// BH = batch * query heads; `group` consecutive query heads share one key /
// value head (K and V hold BH / group heads).
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int BH, int N, int d, int group, bool causal, float scale,
                           hipStream_t stream);

// Nq query rows against Nk keys (bottom-right causal alignment).  With a
// workspace of fwd_workspace_bytes(), the keys may be split across
// workgroups and merged by a second kernel; with ws == nullptr never.
struct FwdPlan {
  int decode;   // 1: packed-rows decode kernel
  int nsplit;   // key ranges (1: none)
  int klen;     // keys per range
};
FwdPlan fwd_plan(int BH, int group, int Nq, int Nk, int d, bool has_ws);
size_t fwd_workspace_bytes(int BH, int group, int Nq, int Nk, int d);
hipError_t launch_fwd_bf16_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                              void* ws, int BH, int Nq, int Nk, int d, int group, bool causal,
                              float scale, hipStream_t stream);

// e4m3 Q, K, V (one byte per element), d = 128; score_scale already holds
// scale * q_scale * k_scale; O = v_scale * softmax(...) (fp8 V).
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                          int BH, int N, int d, bool causal, float score_scale, float v_scale,
                          hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int BH, int N, int d, bool causal, float scale, hipStream_t stream);

// Backward: per-row L2 = lse*log2(e) and D = rowsum(dO * O) plus dQ
// accumulator zeroing, the key-tile kernel (dK, dV, atomic dQ), then dQ
// conversion.  `ws` holds L2 and D (BH * roundup(N, 64) floats each, 256-byte
// aligned regions) followed by the fp32 dQ accumulator (BH * N * d floats).
size_t bwd_workspace_bytes(int BH, int N, int d);
hipError_t launch_bwd_pre(const void* o, const void* dout, const float* lse, void* ws, int BH,
                          int N, int d, hipStream_t stream);
// BH = batch * query heads; `group` query heads share each key / value head.
// Nq query rows (the workspace is sized by them) against Nk keys, causal
// alignment as in launch_fwd_bf16_kv.  hsplit > 1 (a divisor of group) deals
// each group's query heads to hsplit workgroups per key tile; their float32
// dK / dV partials ([2][hsplit][BH / group][Nk][d], bwd_split_bytes) follow
// the bwd_workspace_bytes part of `ws` and a reduction kernel sums them.
int bwd_head_split(int BHkv, int group, int Nq, int Nk, int d, bool causal);
size_t bwd_split_bytes(int BHkv, int Nk, int d, int hsplit);
// Workspace for the largest split either masking may choose.
size_t bwd_kv_workspace_bytes(int BH, int group, int Nq, int Nk, int d);
hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const void* dout,
                           void* dk, void* dv, void* ws, int BH, int Nq, int Nk, int d, int group,
                           int hsplit, bool causal, float scale, hipStream_t stream);
// Two bf16 tensors of `elems` elements each (a multiple of 8) set to 0.
hipError_t launch_zero_bf16(void* a, void* b, size_t elems, hipStream_t stream);
// d = 64: dQ = bf16(accumulator); d = 128, 256: the query-stationary dQ
// kernel (recomputes S and dP; no accumulator).
hipError_t launch_bwd_finalize(const void* q, const void* k, const void* v, const void* dout,
                               void* dq, const void* ws, int BH, int Nq, int Nk, int d, int group,
                               bool causal, float scale, hipStream_t stream);

}  // namespace fa
