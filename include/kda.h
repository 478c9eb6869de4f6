/*
 * kda.h -- C ABI of libkda.so: Kimi Delta Attention (KDA) forward pass on
 * AMD MI355X (gfx950).
 *
 * The operator (a gated delta rule; interface constraints from the refft.com
 * "FlashKDA: High-performance KDA CUDA kernels for SM90+ GPUs" summary,
 * sections "How does FlashKDA's stateful/streaming (chunked) support work?"
 * and "How to seamlessly replace flash-linear-attention's chunk_kda"):
 * per chain (a batch row, or one packed sequence) and value head h, with a
 * state S in R^{K x V} and for each token t
 *
 *     qn = q_t / sqrt(|q_t|^2 + 1e-6),  kn = k_t / sqrt(|k_t|^2 + 1e-6)
 *     g_t = -exp(A_log[h]) * softplus(g_raw_t)      (<= 0; per key channel,
 *                                                    or one value per token
 *                                                    and head)
 *     b_t = sigmoid(beta_logit_t)
 *     S_t = (I - b_t kn kn^T) Diag(exp(g_t)) S_{t-1} + b_t kn v_t^T
 *     o_t = scale * S_t^T qn
 *
 * The gate activation, the sigmoid and the q/k L2 normalisation all run
 * inside the kernels; callers pass raw values.  K = V = 128 only (the
 * FlashKDA summary: the implementation assumes K = V = 128).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Every tensor pointer is a caller-owned DEVICE pointer to contiguous
 *   row-major memory, 16-byte aligned.  The entry points never allocate or
 *   free device memory and create no streams.  Device state the library
 *   holds: the static scratch array of kda_fwd_noalloc (one copy per device,
 *   loaded with the library's code object and held until the process ends),
 *   and, only while the timing diagnostics below are enabled, the HIP events
 *   they record (created on first use per thread and reused).
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *   default stream).  Nothing synchronises the host.
 * - Arguments are validated on the host before anything is enqueued; on a
 *   validation failure nothing is enqueued, a status is returned and
 *   kda_last_error() describes the problem.  Launch failures return
 *   KDA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *   synchronisation.  No C++ exception crosses this ABI.
 * - Token layout: q, k are [B, T, H_qk, 128]; v and out are [B, T, H, 128];
 *   value head h reads q/k head h / (H / H_qk) (contiguous groups, so
 *   H % H_qk == 0).  bf16 tensors hold IEEE bfloat16.
 * - g_raw is bf16 [B, T, H, 128] when gate_per_channel = 1 (KDA), or
 *   bf16 [B, T, H] when gate_per_channel = 0 (one decay per token and head:
 *   the gated delta rule with grouped value heads benchmarked on the
 *   FlashQLA H200 page, "FORWARD BENCHMARKS" table).
 * - beta_logits is fp32 [B, T, H]; A_log is fp32 [H].
 * - State layout is [C, H, V, K] with state[c][h][v][k] = S[k][v], where
 *   C = B (dense) or N (packed sequences).  A state is fp32 or bf16; when
 *   both an initial and a final state are given their dtypes must match.
 *   initial_state = NULL means a zero state; final_state = NULL means the
 *   final state is not written.  initial_state may equal final_state (the
 *   state is read before it is overwritten).
 * - Precise mode: with the environment variable KDA_PRECISE=1 the
 *   per-channel delta-rule forward (kda_fwd, kda_fwd_varlen, kda_fwd_noalloc
 *   with gate_per_channel = 1) runs as one persistent cooperative kernel
 *   that adds low parts (x - fp16(x)) to the fp16 operands of the state
 *   update: about 2-3x lower final-state error when keys within a chunk are
 *   nearly parallel with strong writes and little decay, at about 1.5x the
 *   time.  Check its launches with kda_fwd_check.  Other calls, and devices
 *   without cooperative launch, take the default two-kernel path.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,                  /* a required pointer is NULL */
  KDA_ERR_SHAPE = 2,                 /* a size is negative, K or V != 128, H % H_qk != 0, or tokens,
                                        sequences x H or chunks x H do not fit in int32 */
  KDA_ERR_DTYPE = 3,                 /* unknown state dtype */
  KDA_ERR_STATE_DTYPE_MISMATCH = 4,  /* initial and final state dtypes differ */
  KDA_ERR_WORKSPACE = 5,             /* workspace NULL or smaller than kda_fwd_workspace_bytes() */
  KDA_ERR_ALIGN = 6,                 /* a pointer is not 16-byte aligned */
  KDA_ERR_HIP = 7                    /* the HIP runtime reported an error */
} kda_status;

/* The two range markers widen the enum to every int value, so a dtype outside
 * the three named ones, passed from C, is still a value of the type (and is
 * rejected with KDA_ERR_DTYPE) rather than undefined behaviour in C++. */
typedef enum {
  KDA_STATE_NONE = 0,
  KDA_STATE_BF16 = 1,
  KDA_STATE_FP32 = 2,
  KDA_STATE_RANGE_MIN_ = -2147483647 - 1,
  KDA_STATE_RANGE_MAX_ = 2147483647
} kda_state_dtype;

/*
 * Bytes of device workspace kda_fwd (N = 0) or kda_fwd_varlen (N > 0
 * packed sequences, B = 1) needs for these sizes.  Returns 0 for invalid
 * sizes.  The workspace holds per-chunk intermediates and the chunk
 * schedule; its contents need not be initialised and are garbage afterwards.
 */
size_t kda_fwd_workspace_bytes(int B, int T, int H_qk, int H, int N);

/*
 * Chunked forward pass over B independent rows of T tokens (the cuLA KDA
 * fixed-length table's B x T workload).  States are [B, H, V, K].
 * B == 0 is a successful no-op.  T == 0 writes no output and sets
 * final_state (if given) to initial_state, or to zero when initial_state is
 * NULL.
 */
kda_status kda_fwd(const void* q, const void* k, const void* v, const void* g_raw,
                   const float* beta_logits, const float* A_log, float scale,
                   int gate_per_channel, const void* initial_state, kda_state_dtype init_dtype,
                   void* out, void* final_state, kda_state_dtype final_dtype, int B, int T,
                   int H_qk, int H, int K, int V, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Allocation-free variant of kda_fwd, for callers that cannot call
 * hipMalloc (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments are those of kda_fwd without the
 * workspace: its intermediates go to a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES (one copy per device, whose address is looked up
 * once per device on the first call there).  Sizes whose workspace
 * (kda_fwd_workspace_bytes(B, T, H_qk, H, 0)) exceeds that capacity are
 * rejected with KDA_ERR_WORKSPACE before anything is enqueued: about 1000
 * (64-token chunk, head) pairs, e.g. B = 1, T = 4032, H = 16, on the default
 * path; the precise mode's records live in fixed rings that fit for any T.  Calls on one
 * device share its scratch: calls that overlap on one device (on different
 * streams, or from different threads without ordering) race and give
 * undefined results.  Nothing in the scratch needs to start at zero.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_fwd_noalloc(const void* q, const void* k, const void* v, const void* g_raw,
                           const float* beta_logits, const float* A_log, float scale,
                           int gate_per_channel, const void* initial_state, kda_state_dtype init_dtype,
                           void* out, void* final_state, kda_state_dtype final_dtype, int B, int T,
                           int H_qk, int H, int K, int V, void* stream);

/*
 * Chunked forward pass over N packed sequences (the FlashKDA summary: with
 * cu_seqlens, B must be 1 and the state is [N, H, V, K]; the cuLA KDA varlen
 * table's workload).  The token tensors have B = 1 and T = total tokens.
 * cu_seqlens is a DEVICE int32 array of N + 1 offsets with cu_seqlens[0] = 0,
 * non-decreasing, cu_seqlens[N] = T; it is read on the device (no host
 * copy).  Its contents are a precondition: they are only checked when the
 * environment variable KDA_DEBUG=1 is set, which synchronises the stream.
 * Zero-length sequences are allowed (their final state equals their initial
 * state).  N == 0 is a successful no-op.  T == 0 (all sequences empty)
 * writes no output and sets each final state to its initial state, or to
 * zero when initial_state is NULL.
 */
kda_status kda_fwd_varlen(const void* q, const void* k, const void* v, const void* g_raw,
                          const float* beta_logits, const float* A_log, float scale,
                          int gate_per_channel, const void* initial_state,
                          kda_state_dtype init_dtype, void* out, void* final_state,
                          kda_state_dtype final_dtype, const int32_t* cu_seqlens, int N, int T,
                          int H_qk, int H, int K, int V, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * One decode step: every batch row advances by exactly one token (the cuLA
 * single-token decode table's workload shape: batch up to 256, 64 heads,
 * head dim 128).  q, k: bf16 [B, H_qk, 128]; v: bf16 [B, H, 128]; g_raw:
 * bf16 [B, H, 128] or [B, H]; beta_logits: fp32 [B, H]; state: [B, H, V, K]
 * updated in place; out: bf16 [B, H, 128].  B == 0 is a successful no-op.
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g_raw,
                           const float* beta_logits, const float* A_log, float scale,
                           int gate_per_channel, void* state, kda_state_dtype state_dtype,
                           void* out, int B, int H_qk, int H, int K, int V, void* stream);

/*
 * Decay-only linear attention ("lightning attention": the cuLA benchmark
 * page times its chunked no-state / varlen forward and its single-token
 * decode, in the lightning-attention section, without defining it).  Read as
 * the KDA recurrence without the delta rule:
 *   S_t = Diag(exp(g_t)) S_{t-1} + k_t v_t^T,   o_t = scale * S_t^T q_t,
 * with g_t = -exp(A_log[h]) * softplus(g_raw_t) (one scalar per token-head
 * when gate_per_channel == 0, the per-head decay of lightning attention, or
 * per channel), q and k used as given (no normalisation), no write strength.
 * Arguments, layouts, shapes, workspace (kda_fwd_workspace_bytes), errors
 * and the B/N/T == 0 behaviour are those of kda_fwd / kda_fwd_varlen /
 * kda_decode_step without beta_logits.
 */
kda_status kda_la_fwd(const void* q, const void* k, const void* v, const void* g_raw, const float* A_log,
                      float scale, int gate_per_channel, const void* initial_state,
                      kda_state_dtype init_dtype, void* out, void* final_state,
                      kda_state_dtype final_dtype, int B, int T, int H_qk, int H, int K, int V,
                      void* workspace, size_t workspace_bytes, void* stream);
kda_status kda_la_fwd_varlen(const void* q, const void* k, const void* v, const void* g_raw,
                             const float* A_log, float scale, int gate_per_channel,
                             const void* initial_state, kda_state_dtype init_dtype, void* out,
                             void* final_state, kda_state_dtype final_dtype,
                             const int32_t* cu_seqlens, int N, int T, int H_qk, int H, int K, int V,
                             void* workspace, size_t workspace_bytes, void* stream);
kda_status kda_la_decode_step(const void* q, const void* k, const void* v, const void* g_raw,
                              const float* A_log, float scale, int gate_per_channel, void* state,
                              kda_state_dtype state_dtype, void* out, int B, int H_qk, int H, int K,
                              int V, void* stream);

/*
 * Backward pass of kda_fwd, for both gate modes: gate_per_channel = 1 (KDA,
 * one decay per key channel: the method of the cuLA KDA and FlashKDA pages)
 * and gate_per_channel = 0 (the gated delta rule with grouped value heads
 * whose backward the FlashQLA H200 page times, "BACKWARD BENCHMARKS" table).
 * The pages do not define the backward; it is read as the gradient of a
 * scalar loss through kda_fwd.  Returns the gradients of
 *     L = sum(dout * out) + sum(dfinal * final_state)
 * where (out, final_state) = kda_fwd with the same inputs, with respect to
 * q, k, v, g_raw, beta_logits, A_log and initial_state.
 *
 * Inputs: q, k, v, g_raw (bf16 [B, T, H, 128] or [B, T, H]), beta_logits,
 * A_log, scale as for kda_fwd; initial_state fp32 [B, H, V, K] or NULL (zero
 * state); dout bf16 [B, T, H, 128]; dfinal fp32 [B, H, V, K] or NULL (zero).
 * Outputs, fp32, caller-allocated, each written whole (no accumulation into
 * what they held): dq, dk [B, T, H_qk, 128] (summed over the value heads of
 * each q/k head); dv [B, T, H, 128]; dg_raw in g_raw's layout;
 * dbeta_logits [B, T, H]; dA_log [H]; dinitial_state [B, H, V, K], or NULL
 * (not written).
 *
 * The forward is recomputed inside the call (the state entering every
 * 64-token chunk is kept in the workspace, fp16), so nothing from an earlier
 * kda_fwd call is needed.  Workspace bytes:
 * kda_bwd_workspace_bytes(B, T, H_qk, H, 0) (N > 0: kda_bwd_varlen), the same
 * for both gate modes, 256-byte aligned, contents garbage before and after.
 * dq, dk (when H > H_qk) and dA_log are accumulated with float atomics, so
 * their last bits may differ from run to run; every other output is the same
 * bit for bit on every call (sums inside a workgroup are formed in a fixed
 * order).  Other errors and the B/N/T == 0
 * behaviour follow kda_fwd / kda_fwd_varlen (T == 0: dinitial_state = dfinal,
 * or zero).
 */
size_t kda_bwd_workspace_bytes(int B, int T, int H_qk, int H, int N);
kda_status kda_bwd(const void* q, const void* k, const void* v, const void* g_raw,
                   const float* beta_logits, const float* A_log, float scale, int gate_per_channel,
                   const float* initial_state, const void* dout, const float* dfinal, float* dq,
                   float* dk, float* dv, float* dg_raw, float* dbeta_logits, float* dA_log,
                   float* dinitial_state, int B, int T, int H_qk, int H, int K, int V,
                   void* workspace, size_t workspace_bytes, void* stream);
/* The same over N packed sequences (B = 1, cu_seqlens as for kda_fwd_varlen;
 * states [N, H, V, K]). */
kda_status kda_bwd_varlen(const void* q, const void* k, const void* v, const void* g_raw,
                          const float* beta_logits, const float* A_log, float scale,
                          int gate_per_channel, const float* initial_state, const void* dout,
                          const float* dfinal, float* dq, float* dk, float* dv, float* dg_raw,
                          float* dbeta_logits, float* dA_log, float* dinitial_state,
                          const int32_t* cu_seqlens, int N, int T, int H_qk, int H, int K, int V,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Diagnostics: per-kernel timing with HIP events (used by the benchmark).
 * While enabled on the calling thread, each kernel launched by the entry
 * points above is bracketed by two hipEventRecord calls on the caller's
 * stream.  kda_kernel_timing_read() waits for those events, writes the total
 * milliseconds and launch count per kernel id into the caller's arrays
 * (up to max_kernels entries), forgets them, and returns the number of
 * kernel ids (or -1 on a HIP error).  Kernel ids: 0 schedule, 1 chunk-local,
 * 2 recurrence, 3 decode, 4 fused forward, 5 backward coefficients,
 * 6 backward chains (chunk states and their gradients), 7 backward
 * gradients.  The events are created by the library and reused.
 */
void kda_kernel_timing_enable(int enable);
int kda_kernel_timing_read(double* total_ms, int* launches, int max_kernels);
const char* kda_kernel_name(int id);

/*
 * Waits for `stream`, then reports whether the last forward call on
 * `workspace` (NULL: the current device's kda_fwd_noalloc scratch) met an
 * internal error: for the per-channel delta-rule forward, which runs as one
 * persistent kernel whose workgroups exchange chunk records through the L2
 * of their XCD, a bounded wait that timed out or a workgroup on an
 * unexpected XCD.  The results of such a call are invalid.  Returns KDA_OK
 * when no error was recorded, KDA_ERR_HIP (with a description) otherwise.
 */
kda_status kda_fwd_check(const void* workspace, void* stream);

/* Static, human-readable name of a status code. */
const char* kda_status_string(kda_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* kda_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
