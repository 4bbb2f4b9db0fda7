/*
 * fa.h -- C ABI of the exact tiled attention library (libfa.so, gfx950).
 *
 * Computes exact attention O = softmax(scale * Q K^T) V and its gradients on
 * one MI355X, tiled so the N x N score matrix never exists in device memory.
 *
 * The operation ("Flash Attention, From First Principles", sections "What is
 * attention?" and "Stop 3: the pour"; "LLM Architecture Refresh [3]: Flash
 * Attention Is Exact, and Here's the Proof", sections 2, 4 and 7):
 *
 *   S   = scale * Q K^T                      (per batch b, head h)
 *   S_ij = -inf where causal and j > i        (key j visible to query i iff j <= i)
 *   P   = softmax(S) row-wise;  O = P V
 *   lse_i = log(sum_j exp(S_ij))             (natural log, scaled-score units)
 *
 * The saved statistic lse is the log-sum-exp L = m + log(l) of "FlashAttention
 * from scratch: how it works and how to code it", Follow-up questions; the
 * backward rebuilds P = exp(S - L) from it instead of storing P.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout   Every tensor is a contiguous row-major [B, H, N, d] array (query,
 *          key, value, output and gradient tensors alike); lse and the
 *          backward's D are contiguous [B, H, N] float arrays.  Queries and
 *          keys have the same length N.
 * Pointers All pointers are DEVICE pointers (memory from hipMalloc or any
 *          allocator handing out device memory).  Tensor pointers must be
 *          16-byte aligned.  Inputs are only read.  Outputs must not overlap
 *          any input or each other.
 * Ownership The caller owns every buffer, including the backward workspace.
 *          The library allocates nothing, keeps no mutable global state and
 *          may be called from several host threads at once.
 * Streams  Work is enqueued on `stream` (0 = the null stream) and the call
 *          returns without waiting.  Faults during execution surface at the
 *          caller's next synchronisation on that stream.
 * Errors   Every call returns an int status (FA_OK == 0).  Arguments are
 *          validated before any work is enqueued, so a rejected call touches
 *          neither the stream nor device memory; the only HIP calls made
 *          before the checks pass read the current device and its compute-
 *          unit count (which size the launch plans and workspaces).
 *          B*H*N == 0 is a valid no-op.  Nothing is thrown across the ABI.
 * Sizes    d must be 64 or 128; the bfloat16 entry points (the forwards
 *          fa_fwd, fa_fwd_gqa, fa_fwd_kv and the backwards) also take
 *          d = 256; fa_fwd_fp8 takes 128 only.  B, H >= 0; 0 <= N <= FA_MAX_N.
 * Scale    Any finite float (the usual value is 1/sqrt(d)).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL                        */
  FA_ERR_SHAPE = 2,     /* B, H or N negative, N > FA_MAX_N, overflow, or a
                           head count H that Hkv does not divide             */
  FA_ERR_HEADDIM = 3,   /* d not supported by the entry point (see Sizes)     */
  FA_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned            */
  FA_ERR_ALIAS = 5,     /* an output overlaps an input or another output      */
  FA_ERR_SCALE = 6,     /* scale is NaN or infinite                           */
  FA_ERR_HIP = 7,       /* a kernel launch was rejected by the HIP runtime    */
  FA_ERR_WORKSPACE = 8, /* workspace smaller than required                    */
  FA_ERR_SCRATCH = 9    /* fa_bwd_noalloc: the problem needs more scratch than
                           the static buffer holds (FA_STATIC_SCRATCH_BYTES)  */
};

/* Largest supported sequence length (keeps every per-head offset in 31 bits). */
#define FA_MAX_N (1 << 22)

/*
 * fa_fwd -- forward pass, bfloat16 tensors.
 *
 *   q, k, v  [B, H, N, d] bfloat16 inputs (read only).
 *   o        [B, H, N, d] bfloat16 output, O rounded to nearest even.
 *   lse      [B, H, N] float32 output, natural-log log-sum-exp of each row of
 *            scale * Q K^T over its visible keys.
 *   causal   0 = every key visible; nonzero = key j visible to query i iff j <= i.
 *   scale    multiplies Q K^T before the softmax.
 *
 * Scores, the running max / running sum and the output accumulator are fp32;
 * the probability tile is rounded to bfloat16 for the P V product.  Tiles
 * whose keys all lie in the future of every query of the tile are skipped
 * ("LLM Architecture Refresh [3]", section 7).  d = 64, 128 or 256 (d = 256
 * runs a kernel with one wave per SIMD: its accumulator and query tile do not
 * fit the two-wave schedule; "Flash Attention, From First Principles", "The
 * rent arithmetic", on tiles shrinking as d grows).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float scale,
           hipStream_t stream);

/*
 * fa_fwd_gqa -- forward pass with grouped-query attention, bfloat16 tensors.
 *
 *   q, o        [B, H, N, d];  k, v  [B, Hkv, N, d];  lse [B, H, N].
 *   Hkv         key / value heads, 1 <= Hkv <= H with H a multiple of Hkv
 *               (Hkv = 1: multi-query attention; Hkv = H: same as fa_fwd).
 *
 * Query head h attends with key / value head h / (H / Hkv): each key / value
 * head serves H / Hkv consecutive query heads.  The pages only name
 * multi-query and grouped-query attention ("Flash Attention, From First
 * Principles", "Honesty time -- the confession list", item 6; "LLM
 * Architecture Refresh [3]", section 6, the KV-cache vs score-matrix table);
 * the grouping is the usual consecutive one.  Otherwise exactly fa_fwd: same
 * operation per head, rules, rounding and errors.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, int causal, float scale,
               hipStream_t stream);

/*
 * fa_fwd_kv -- forward pass of Nq queries against Nk keys (cross-attention,
 * a prompt or generated tokens against a key/value cache), bfloat16 tensors.
 *
 *   q, o        [B, H, Nq, d];  k, v  [B, Hkv, Nk, d];  lse [B, H, Nq].
 *   Hkv         key / value heads as in fa_fwd_gqa (Hkv = H: one per head).
 *   Nq, Nk      0 <= Nq, Nk <= FA_MAX_N, independent.
 *   causal      the queries are the LAST Nq positions of the sequence: query i
 *               sees key j iff j <= i + (Nk - Nq) (bottom-right alignment;
 *               for Nq = Nk exactly the rule of fa_fwd).  A query that sees
 *               no key (with causal masking the first Nq - Nk queries when
 *               Nq > Nk; every query when Nk = 0) gets O = 0 and lse = -inf.
 *   workspace   device memory of at least fa_fwd_kv_workspace_size(B, H, Hkv,
 *               Nq, Nk, d) bytes, 16-byte aligned; may be NULL when that size
 *               is 0.
 *
 * The pages define attention for one length n ("LLM Architecture Refresh
 * [3]", the notes before the references, which also point out that
 * generation splits a sequence into a prompt and new tokens); the alignment
 * above is the reading that places the queries at the end.  When every query
 * row that reads a key / value head fits in one wave ((H / Hkv) * Nq <= 32,
 * d = 64 or 128: decode), one wave computes all of them against a range of
 * keys, so each key and value byte is read once per key / value head.  When
 * the work alone would leave most of the GPU idle (decode, few heads, small
 * Nq), the keys are split into ranges handled by separate workgroups, each writing
 * a normalised partial output and its log-sum-exp to the workspace, and a
 * second kernel merges the ranges by the block law of "Flash Attention, From
 * First Principles", "The scaffold": lse = log sum_r e^{lse_r},
 * O = sum_r e^{lse_r - lse} O_r.  The result is the same exact attention.
 * Errors as fa_fwd, plus FA_ERR_WORKSPACE for a workspace that is too small;
 * k and v may be NULL when Nk == 0.
 */
size_t fa_fwd_kv_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d);
int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
              void* workspace, size_t workspace_bytes, int B, int H, int Hkv,
              int Nq, int Nk, int d, int causal, float scale,
              hipStream_t stream);

/*
 * fa_fwd_fp8 -- forward pass with 8-bit floating-point inputs (the FA-3
 * direction of "LLM Architecture Refresh [3]", section 8).
 *
 *   q, k, v   [B, H, N, d] OCP e4m3 ("float8 e4m3fn") bytes, one byte per
 *             element; the values they stand for are q_scale * q, k_scale * k
 *             and v_scale * v (one dequantisation factor per tensor).
 *   o         [B, H, N, d] bfloat16 output;  lse [B, H, N] float32 output.
 *   d         128 only (FA_ERR_HEADDIM otherwise).
 *
 * Computes the attention of the dequantised tensors: S = scale * q_scale *
 * k_scale * (q k^T), lse and O = v_scale * softmax(S) v.  Both products run
 * on the fp8 matrix cores with fp32 accumulation; the probabilities are
 * rounded to e4m3 (3 mantissa bits) for the P V product, while the running
 * max, the running sum and lse are fp32 from the unrounded probabilities.  So
 * lse is as accurate as the bf16 path's, and each output element carries an
 * error of at most about 2^-4 of the probability-weighted |v| it averages
 * (plus the bf16 rounding of O); the tests state the bound per element.
 * Errors as fa_fwd, plus FA_ERR_SCALE for a non-finite scale factor or
 * product of factors.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               float q_scale, float k_scale, float v_scale, int B, int H, int N,
               int d, int causal, float scale, hipStream_t stream);

/*
 * fa_fwd_f32 -- forward pass, float32 tensors end to end.
 *
 * Same operation, layout and rules as fa_fwd with every tensor float32 and
 * every product carried out in float32 (fp32 MFMA).
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o,
               float* lse, int B, int H, int N, int d, int causal, float scale,
               hipStream_t stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs.
 *
 * Returns 0 for invalid shapes.  The workspace holds, per row, lse * log2(e)
 * and -D = -rowsum(dO * O) (float32, each head padded to a multiple of 64 rows)
 * and, at d = 64 only, the float32 dQ accumulator ([B, H, N, d]).
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * fa_bwd_kv_workspace_size -- bytes of device workspace with which fa_bwd_gqa
 * and fa_bwd_kv run at full speed: fa_bwd_workspace_size(B, H, Nq, d) plus,
 * when grouped-query heads are split (below), room for float32 partial dK
 * and dV sums.  Returns 0 for invalid shapes (as the fa_bwd_kv checks).
 *
 * Under causal masking the first key tiles see every query and the last few
 * almost none, and with few key / value heads the key tiles holding all H / Hkv
 * query heads' work would set the backward's time.  Given this workspace, the
 * key-tile kernel deals each group's query heads to several workgroups (a
 * divisor of H / Hkv, chosen from the shapes) that write float32 partials,
 * and a reduction kernel sums them in a fixed order (deterministic).  With
 * only fa_bwd_workspace_size bytes the split is not used; results agree to
 * bf16 rounding either way.
 */
size_t fa_bwd_kv_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d);

/*
 * fa_bwd -- backward pass, bfloat16 tensors.
 *
 *   q, k, v, o  [B, H, N, d] bfloat16: the forward's inputs and output.
 *   dout        [B, H, N, d] bfloat16: gradient of the loss w.r.t. O
 *               (named for the dO of the pages; `do` is a C keyword).
 *   lse         [B, H, N] float32 from fa_fwd on the same inputs.
 *   dq, dk, dv  [B, H, N, d] bfloat16 outputs.
 *   workspace   device buffer of at least fa_bwd_workspace_size(B, H, N, d)
 *               bytes, 16-byte aligned; contents on entry are ignored and
 *               overwritten.  workspace_bytes is its size.
 *
 * Recomputes every probability tile from Q, K and lse ("FlashAttention from
 * scratch", Follow-up questions): P = exp(S - L); dV += P^T dO; dP = dO V^T;
 * D = rowsum(dO * O); dS = P * (dP - D); dK += scale * dS^T Q; dQ += scale *
 * dS K.  dK and dV accumulate per key tile.  dQ is accumulated separately:
 * at d = 64 across key tiles in the float32 workspace with atomic adds (dQ
 * may then differ between runs in its last bits); at d = 128 and 256 by a
 * second pass that owns query tiles and recomputes S and dP (no atomics,
 * deterministic).  d = 64, 128 or 256.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
           int causal, float scale, hipStream_t stream);

/*
 * fa_bwd_gqa -- backward pass with grouped-query attention, bfloat16 tensors.
 *
 *   q, o, dout, dq  [B, H, N, d];  k, v, dk, dv  [B, Hkv, N, d];  lse [B, H, N].
 *   workspace       at least fa_bwd_workspace_size(B, H, N, d) bytes (it is
 *                   sized by the query heads); fa_bwd_kv_workspace_size(B, H,
 *                   Hkv, N, N, d) bytes allow the head split described there.
 *
 * The gradient of fa_fwd_gqa: dK and dV of a key / value head sum the
 * contributions of the H / Hkv query heads that share it (the chain rule
 * through the shared head); each workgroup owns a key tile of one key / value
 * head and walks its query heads (or its share of them) in turn, so the sum
 * stays in registers.  Otherwise exactly fa_bwd.
 */
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes, int B, int H, int Hkv,
               int N, int d, int causal, float scale, hipStream_t stream);

/*
 * fa_bwd_kv -- backward pass of fa_fwd_kv (Nq queries against Nk keys,
 * bottom-right causal alignment, grouped-query heads), bfloat16 tensors.
 *
 *   q, o, dout, dq  [B, H, Nq, d];  k, v, dk, dv  [B, Hkv, Nk, d];
 *   lse [B, H, Nq] as fa_fwd_kv returned it.
 *   workspace       at least fa_bwd_workspace_size(B, H, Nq, d) bytes;
 *                   fa_bwd_kv_workspace_size(B, H, Hkv, Nq, Nk, d) bytes
 *                   allow the grouped-query head split described there.
 *
 * Gradients of sum(O * dO) as for fa_bwd: query rows with no visible key get
 * dQ = 0; keys no query sees get dK = dV = 0 (with Nq = 0 every key, and
 * then only k, v, dk and dv need to be given).  Errors as fa_bwd.
 */
int fa_bwd_kv(const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, void* dq, void* dk, void* dv,
              void* workspace, size_t workspace_bytes, int B, int H, int Hkv,
              int Nq, int Nk, int d, int causal, float scale, hipStream_t stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, operation, results and errors as fa_bwd minus
 * the workspace: the library uses its own static device buffer of
 * FA_STATIC_SCRATCH_BYTES instead (a file-scope device array, one per GPU,
 * held from the library's first use on that GPU until the process ends).
 * The call allocates nothing: no hipMalloc, no hipFree, no allocating library
 * routine.
 *
 *   Limit       fa_bwd_workspace_size(B, H, N, d) must not exceed
 *               FA_STATIC_SCRATCH_BYTES, else FA_ERR_SCRATCH (nothing is
 *               launched).  64 MiB holds about 254 thousand rows (B*H*N) at
 *               d = 64, whose workspace carries the float32 dQ accumulator
 *               ([4, 16, 2048, 64] uses 33 MiB), and about 8.3 million rows at
 *               d = 128 and 256 (two floats per row).
 *   Sharing     every call on one GPU uses that GPU's one buffer, which keeps
 *               the last call's contents (each call clears what must start at
 *               zero with a kernel, not a memset).  Calls that overlap on one
 *               GPU -- on different streams, or from different host threads
 *               without ordering -- RACE on the buffer; serialise them.
 *   First call  on a GPU, looks the buffer's address up on that device (the
 *               device current at the call) and keeps it.
 */
#define FA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk,
                   void* dv, int B, int H, int N, int d, int causal, float scale,
                   hipStream_t stream);

/*
 * The three stages fa_bwd runs, in order, on the same stream.  Calling them in
 * sequence with the same arguments is exactly fa_bwd; they exist for callers
 * that schedule or time the stages separately.  Each validates like fa_bwd
 * (its own pointers only) and reads/writes the workspace as documented.
 *
 * fa_bwd_preprocess -- lse * log2(e) and -D = -rowsum(dO * O) into the
 *                      workspace; at d = 64 zeroes the workspace's fp32 dQ
 *                      accumulator.
 * fa_bwd_main       -- the key-tile kernel: recomputes P from q, k and the
 *                      workspace's log-sum-exp and writes dk and dv; at d = 64
 *                      it also adds scale * dS K into the dQ accumulator
 *                      (float atomics).  Needs the preprocess stage's
 *                      workspace contents.
 * fa_bwd_finalize   -- dq: at d = 64 bf16(dQ accumulator) (q, k, v, dout,
 *                      causal and scale are not read and may be NULL / any);
 *                      at d = 128 and 256 the query-tile dQ kernel, which
 *                      needs them and the preprocess stage's workspace.
 */
int fa_bwd_preprocess(const void* o, const void* dout, const float* lse,
                      void* workspace, size_t workspace_bytes, int B, int H,
                      int N, int d, hipStream_t stream);
int fa_bwd_main(const void* q, const void* k, const void* v, const void* dout,
                void* dk, void* dv, void* workspace, size_t workspace_bytes,
                int B, int H, int N, int d, int causal, float scale,
                hipStream_t stream);
int fa_bwd_finalize(const void* q, const void* k, const void* v,
                    const void* dout, void* dq, const void* workspace,
                    size_t workspace_bytes, int B, int H, int N, int d, int causal,
                    float scale, hipStream_t stream);

/* fa_status_string -- static, human-readable text for a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
