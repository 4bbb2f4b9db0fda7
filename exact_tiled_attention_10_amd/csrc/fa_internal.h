// Kernel launchers and launch plans called by the C ABI layer (fa_api.cpp).
// Arguments are already validated there; each launcher only enqueues work on
// `stream` and returns the launch status.  The plans (fa_plan.cpp) are plain
// host arithmetic: they size workspaces and pick grids, with the device's
// compute-unit count passed in.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

// ---------------------------------------------------------------------------
// tile geometry shared by the kernels and the plans
// ---------------------------------------------------------------------------
// Queries per forward workgroup: 256 (8 waves x 32) for d = 128, 128 (4 waves
// x 32) for d = 64 and 256.
constexpr int fwd_rows_per_tile(int d) { return d == 128 ? 256 : 128; }
// Keys per forward key tile of the plans' split arithmetic (a multiple of
// every forward kernel's key tile).
constexpr int kFwdSplitKeys = 64;
// Queries per block streamed past a backward key tile.
constexpr int kBwdQueryBlock = 64;
// Keys per backward key-tile workgroup: 256 at d = 64 (8 waves x 32), 128 at
// d = 128 and 256 (4 waves x 32).
constexpr int bwd_keys_per_tile(int d) { return d == 64 ? 256 : 128; }

// ---------------------------------------------------------------------------
// per-device state (fa_device.hip)
// ---------------------------------------------------------------------------
// Compute units of the current device (read once per device; 256, MI355X's
// count, when no device can be queried, e.g. on a host without a GPU).
int device_cus();

// The no-allocation backward's scratch: a static device array of
// kStaticScratchBytes per device.  Writes the current device's address of it
// to *ptr (looked up with hipGetSymbolAddress once per device, with that
// device current).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(void** ptr);

// ---------------------------------------------------------------------------
// plans (fa_plan.cpp)
// ---------------------------------------------------------------------------
// Nq query rows against Nk keys (bottom-right causal alignment).  With a
// workspace of fwd_workspace_bytes(), the keys may be split across
// workgroups and merged by a second kernel; without one never.
struct FwdPlan {
  int decode;   // 1: packed-rows decode kernel
  int nsplit;   // key ranges (1: none)
  int klen;     // keys per range
};
FwdPlan fwd_plan(int BH, int group, int Nq, int Nk, int d, bool has_ws, int cus);
size_t fwd_workspace_bytes(int BH, int group, int Nq, int Nk, int d, int cus);

// Backward workspace: per row L2 = lse*log2(e) and D = rowsum(dO * O)
// (BH * roundup(N, 64) floats each, 256-byte aligned regions), then at d = 64
// the fp32 dQ accumulator (BH * N * d floats).
size_t bwd_workspace_bytes(int BH, int N, int d);
// Grouped-query heads: hsplit > 1 (a divisor of group) deals each group's
// query heads to hsplit workgroups per key tile; their float32 dK / dV
// partials ([2][hsplit][BH / group][Nk][d], bwd_split_bytes) follow the
// bwd_workspace_bytes part of the workspace and a reduction kernel sums them.
int bwd_head_split(int BHkv, int group, int Nq, int Nk, int d, bool causal, int cus);
size_t bwd_split_bytes(int BHkv, int Nk, int d, int hsplit);
// Workspace for the largest split either masking may choose.
size_t bwd_kv_workspace_bytes(int BH, int group, int Nq, int Nk, int d, int cus);

// ---------------------------------------------------------------------------
// launchers (fa_fwd.hip, fa_bwd.hip)
// ---------------------------------------------------------------------------
// BH = batch * query heads; `group` consecutive query heads share one key /
// value head (K and V hold BH / group heads).  `plan` comes from fwd_plan
// (nsplit > 1 needs ws of fwd_workspace_bytes()).
hipError_t launch_fwd_bf16_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                              void* ws, int BH, int Nq, int Nk, int d, int group, bool causal,
                              float scale, const FwdPlan& plan, hipStream_t stream);

// e4m3 Q, K, V (one byte per element), d = 128; score_scale already holds
// scale * q_scale * k_scale; O = v_scale * softmax(...) (fp8 V).
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                          int BH, int N, int d, bool causal, float score_scale, float v_scale,
                          hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int BH, int N, int d, bool causal, float scale, hipStream_t stream);

// Backward: per-row L2 and D plus dQ accumulator zeroing, the key-tile
// kernel (dK, dV; atomic dQ at d = 64), then dQ.
hipError_t launch_bwd_pre(const void* o, const void* dout, const float* lse, void* ws, int BH,
                          int N, int d, hipStream_t stream);
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
