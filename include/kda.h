/*
 * kda.h -- C ABI of libkda: the Kimi Delta Attention (KDA) forward operator
 * on AMD Instinct MI355X (gfx950).
 *
 * KDA is the channel-wise gated delta rule. Per (sequence, head), with a
 * d_k x d_v fp32 state S (row i = key channel i, column j = value channel j):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * with alpha_t = exp(log_alpha_t) one gate per key channel and beta_t one
 * scalar per head. Sources: "Kimi Linear爆发背后的秘密：重新定义长上下文推理效率"
 * (xugj520.cn), section "Kimi Delta Attention的技术内核" (the recurrence) and
 * section "硬件效率的深度优化" (chunk-parallel inside a chunk, recurrent across
 * chunks, WY representation, UT transform); the 2025 attention/MoE review
 * (lanjinlin.com.cn), sections "GatedDeltaNet解读" (per-token loop: decay,
 * correction against the decayed state, rank-1 write, read-out from the
 * updated state, initial/final state of a sequence; state laid out as
 * [heads, head_k_dim, head_v_dim]) and "KLA" (o_t = S_t^T q_t, Diag(alpha_t));
 * "线性注意力机制Kimi Linear架构解析与优化实践" (coreui.cn), section 2.1 (alpha per key
 * channel (B,H,D_k), beta per head (B,H,1)), section 2.2 (64-token chunks),
 * section 3.2 (the recurrent state kept in one contiguous cache) and
 * section 4.2 (the gate carried in log space).
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is DEVICE memory on the current HIP device,
 *    owned by the caller. The library never allocates or frees device memory
 *    and never synchronises; all of a call's work is enqueued on `stream`, in
 *    order, so a call can be captured in a HIP graph.
 *  - Every pointer must be 16-byte aligned; tensors are dense, row-major,
 *    with the layouts given below (last dimension contiguous).
 *  - Arguments are validated on the host before anything is enqueued. A
 *    status other than KDA_OK means nothing was enqueued, except
 *    KDA_ERR_HIP, which reports a failed kernel launch. With KDA_DEBUG_SYNC=1
 *    in the environment (read once, a debugging aid, not for use under graph
 *    capture) every call also waits for its work on `stream` and reports an
 *    error while it ran as KDA_ERR_HIP.
 *  - Device-side contents are the caller's contract and are not checked:
 *    cu_seqlens must be non-decreasing from 0 to T_total, log_alpha finite
 *    and <= 0, slot indices distinct and in range. Stability of the
 *    recurrence needs beta_t ||k_t||^2 in [0, 2] (e.g. ||k_t|| <= 1 and
 *    beta_t in [0, 2]).
 *  - bf16 prefill: its pairwise key/query products run on fp16 operands, so
 *    every q and k component must be below 6.5e4 in magnitude. A chunk in
 *    which some 16-token sub-chunk decays by more than e^10 in a channel, or
 *    in which a q or k component times the decay over half a sub-chunk could
 *    pass 3e4, evaluates its diagonal 16 x 16 blocks element by element in
 *    fp32 instead (slower, same result); v, the states and the outputs have
 *    no such bound (they are scaled by powers of two before every fp16
 *    conversion).
 *  - Test overrides, read from the environment: KDA_SEG_CHUNKS=n (at every
 *    call) cuts the state passes of the bf16 prefill into segments of n
 *    chunks (at most the chunk count; with d_k = d_v a sequence's segment 0
 *    has floor(5 n / 8) chunks, at least one), and KDA_PREFILL_KERNEL=valu
 *    (once per process) runs bf16 inputs through the fp32 prefill kernels.
 *    The workspace size depends on both: query it under the environment of
 *    the call.
 *  - The library's only global state is a per-device cache of the compute
 *    unit count and of the address of kda_chunk_fwd_ex_noalloc's static
 *    scratch (both atomic), and that scratch itself. Calls are thread-safe
 *    and take no lock; calls on different streams that write the same memory
 *    (outputs, states, a shared workspace) race.
 *  - No C++ exception crosses this interface.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* NULL, misaligned pointer or out-of-range size */
    KDA_ERR_UNSUPPORTED = 2, /* valid but not implemented: head dims, chunk size, dtype pair */
    KDA_ERR_WORKSPACE = 3,   /* workspace smaller than kda_chunk_fwd_workspace_size() */
    KDA_ERR_HIP = 4          /* a HIP launch failed; see hipGetLastError() */
} kda_status_t;

typedef enum {
    KDA_F32 = 0,  /* IEEE binary32 */
    KDA_BF16 = 1  /* bfloat16; outputs are rounded to nearest even */
} kda_dtype_t;

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char *kda_status_string(kda_status_t status);

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes; 0 means the
 * call may pass workspace = NULL (or the sizes are invalid). A function of its
 * arguments and of the test overrides above.
 */
size_t kda_chunk_fwd_workspace_size(int32_t N, int32_t T_total, int32_t H,
                                    int32_t d_k, int32_t d_v,
                                    kda_dtype_t in_dtype);

/*
 * Chunkwise-parallel KDA prefill over N packed variable-length sequences.
 *
 * Sequence n covers tokens [cu_seqlens[n], cu_seqlens[n+1]) of the packed
 * token axis. Each sequence starts from initial_state[n] (zeros if
 * initial_state is NULL) and is cut into 64-token chunks from its own first
 * token; the last chunk may be partial. The result is the recurrence above
 * evaluated exactly up to floating-point rounding: the chunk size is not
 * part of the result.
 *
 *   q, k        [T_total, H, d_k]   in_dtype
 *   v           [T_total, H, d_v]   in_dtype
 *   log_alpha   [T_total, H, d_k]   fp32, natural-log channel gate, <= 0
 *   beta        [T_total, H]        fp32
 *   cu_seqlens  [N + 1]             int32, device memory
 *   initial_state [N, H, d_k, d_v]  fp32, or NULL for zeros
 *   final_state   [N, H, d_k, d_v]  fp32 output, or NULL (not written);
 *                                   may be the same pointer as initial_state
 *   o           [T_total, H, d_v]   out_dtype output
 *   scale       multiplies o only (not the state); 1.0 gives o_t = S_t^T q_t
 *   chunk_size  must be 64
 *   workspace   device scratch of workspace_bytes (may be NULL if the size
 *               query returns 0)
 *
 * Sizes: N >= 1, H >= 1, 0 <= T_total <= 2^31 - 65, N H < 2^27,
 * T_total H max(d_k, d_v) <= 2^40, d_k and d_v in {64, 128}. With
 * T_total = 0 the token arrays (q, k, v, log_alpha, beta, o) may be NULL.
 * dtype pairs: (F32 in, F32 out), (BF16 in, BF16 out), (BF16 in, F32 out).
 * Internal arithmetic: fp32 state and accumulation; the state is fp32 at
 * every chunk boundary.
 * A sequence of length 0 leaves final_state[n] = initial_state[n] (or 0).
 */
kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           const int32_t *cu_seqlens, int32_t N,
                           int32_t T_total, int32_t H, int32_t d_k,
                           int32_t d_v, kda_dtype_t in_dtype,
                           kda_dtype_t out_dtype, float scale,
                           const float *initial_state, float *final_state,
                           void *o, int32_t chunk_size, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * One recurrent decode step for B independent sequences, updating an fp32
 * state cache in place (one token per sequence).
 *
 *   q, k        [B, H, d_k]   in_dtype
 *   v           [B, H, d_v]   in_dtype
 *   log_alpha   [B, H, d_k]   fp32
 *   beta        [B, H]        fp32
 *   state_cache [num_slots, H, d_k, d_v] fp32, read and written in place
 *   slot_idx    [B] int32 device array of distinct slots in [0, num_slots),
 *               or NULL for slot b = b (then B <= num_slots)
 *   o           [B, H, d_v]   out_dtype output
 *
 * Per (b, h): S' = Diag(exp(log_alpha)) S; u = beta (v - S'^T k);
 * S = S' + k u^T; o = scale * S^T q.
 * Sizes: B >= 1, H >= 1, num_slots >= 1, d_k and d_v in {64, 128}.
 * dtype pairs as for kda_chunk_fwd.
 */
kda_status_t kda_decode_step(const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta,
                             float *state_cache, const int32_t *slot_idx,
                             void *o, int32_t B, int32_t H, int32_t d_k,
                             int32_t d_v, int32_t num_slots,
                             kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                             float scale, hipStream_t stream);

/*
 * Extended entry points: the steps just before and just after the operator,
 * and the serving layout of the states. `opt` may be NULL; a zero-filled
 * kda_options_t (or NULL) gives exactly kda_chunk_fwd / kda_decode_step.
 *
 * Sources: the 2025 attention/MoE review (lanjinlin.com.cn), section
 * "GatedDeltaNet解读": the gates g and beta are produced from two inputs (a, b),
 * the key/query heads serve groups of value heads, and the read-out is
 * RMS-normalised and multiplied by an output gate z; its MiniMax section fuses
 * the group RMS norm, the sigmoid gate and the product into one kernel.
 * "线性注意力机制Kimi Linear架构解析与优化实践" (coreui.cn), section 3.2: the
 * recurrent states kept in one contiguous cache indexed per sequence.
 * The pages do not give KDA's gate activation; this library uses
 *     log_alpha = -gate_scale * softplus(gate_x),  beta = sigmoid(beta_y),
 * with softplus(x) = ln(1 + e^x) and sigmoid(y) = 1 / (1 + e^-y).
 */
typedef enum {
    KDA_ACT_NONE = 0,    /* o <- o * z */
    KDA_ACT_SIGMOID = 1  /* o <- o * sigmoid(z) */
} kda_act_t;

typedef struct {
    /* Grouped value heads: q and k have num_k_heads heads ([*, num_k_heads,
     * d_k]); value head h uses key head h / (H / num_k_heads). H must be a
     * multiple of num_k_heads. 0 means H (no grouping). */
    int32_t num_k_heads;
    /* Gate pre-activations, in_dtype. gate_x [*, H, d_k] replaces log_alpha
     * (which must then be NULL); beta_y [*, H] replaces beta (which must then
     * be NULL). gate_scale > 0 and finite when gate_x is set. */
    const void *gate_x;
    const void *beta_y;
    float gate_scale;
    /* Output epilogue, per token and value head, in fp32 before the output
     * rounding: if norm != 0, o <- o / sqrt(mean_j o_j^2 + norm_eps), then
     * times norm_weight [d_v] (fp32, NULL = 1); then, if out_gate
     * ([*, H, d_v], in_dtype) is set, o <- o * act(out_gate). norm_eps >= 0. */
    int32_t norm;
    float norm_eps;
    const float *norm_weight;
    const void *out_gate;
    kda_act_t out_gate_act;
    /* Prefill only: states in a slot cache. With state_slots ([N] int32,
     * device) set, initial_state and final_state are caches
     * [num_slots, H, d_k, d_v] (usually the same pointer): sequence n starts
     * from slot state_slots[n] of initial_state and writes its final state to
     * the same slot of final_state. A negative slot marks padding: the
     * sequence starts from zeros and its final state is not written. Slots of
     * different sequences must differ. num_slots >= 1. */
    const int32_t *state_slots;
    int32_t num_slots;
} kda_options_t;

/*
 * kda_chunk_fwd with options. H is the number of value heads (the heads of
 * v, log_alpha / gate_x, beta / beta_y, o and the states); the workspace is
 * kda_chunk_fwd_workspace_size(N, T_total, H, d_k, d_v, in_dtype).
 * Every option is available for both input types (on the fp32 path the
 * epilogue runs as a second pass over o). Errors as for kda_chunk_fwd, plus
 * KDA_ERR_INVALID_ARG for inconsistent options; kda_chunk_fwd itself returns
 * KDA_ERR_INVALID_ARG when log_alpha or beta is NULL and T_total > 0.
 * With T_total = 0 no gate is read: neither gate form need be given (and
 * gate_x, beta_y and out_gate may be NULL), but giving both forms of one gate
 * is still an error.
 */
kda_status_t kda_chunk_fwd_ex(const void *q, const void *k, const void *v,
                              const float *log_alpha, const float *beta,
                              const int32_t *cu_seqlens, int32_t N,
                              int32_t T_total, int32_t H, int32_t d_k,
                              int32_t d_v, kda_dtype_t in_dtype,
                              kda_dtype_t out_dtype, float scale,
                              const float *initial_state, float *final_state,
                              void *o, int32_t chunk_size, void *workspace,
                              size_t workspace_bytes, const kda_options_t *opt,
                              hipStream_t stream);

/*
 * kda_decode_step with options (state_slots and num_slots of `opt` are not
 * used: decode has slot_idx). H is the number of value heads.
 */
kda_status_t kda_decode_step_ex(const void *q, const void *k, const void *v,
                                const float *log_alpha, const float *beta,
                                float *state_cache, const int32_t *slot_idx,
                                void *o, int32_t B, int32_t H, int32_t d_k,
                                int32_t d_v, int32_t num_slots,
                                kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                                float scale, const kda_options_t *opt,
                                hipStream_t stream);

/*
 * Bytes of the library's static scratch, the workspace of
 * kda_chunk_fwd_ex_noalloc: one array per GPU in the library's code object,
 * held from the first use of the library on that GPU until the process ends.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/*
 * kda_chunk_fwd_ex without the workspace arguments, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The call allocates nothing and calls no
 * allocating routine; its workspace is the library's static scratch of the
 * current device (KDA_NOALLOC_SCRATCH_BYTES).
 *  - Returns KDA_ERR_WORKSPACE, with nothing enqueued, when
 *    kda_chunk_fwd_workspace_size(N, T_total, H, d_k, d_v, in_dtype) exceeds
 *    KDA_NOALLOC_SCRATCH_BYTES (e.g. a 4,096-token bf16 call at H = 32 and
 *    d = 128 fits, and one 16 times larger does not); KDA_ERR_HIP if the
 *    scratch's address cannot be obtained. Every other argument and error is
 *    as for kda_chunk_fwd_ex.
 *  - Every call on a GPU uses that GPU's one scratch array, which keeps the
 *    previous call's contents (no call needs it cleared: each writes what it
 *    reads). Calls that overlap on one GPU (different streams, or host
 *    threads, without ordering between them) race on it and must not be made.
 */
kda_status_t kda_chunk_fwd_ex_noalloc(const void *q, const void *k, const void *v,
                                      const float *log_alpha, const float *beta,
                                      const int32_t *cu_seqlens, int32_t N,
                                      int32_t T_total, int32_t H, int32_t d_k,
                                      int32_t d_v, kda_dtype_t in_dtype,
                                      kda_dtype_t out_dtype, float scale,
                                      const float *initial_state, float *final_state,
                                      void *o, int32_t chunk_size,
                                      const kda_options_t *opt, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
