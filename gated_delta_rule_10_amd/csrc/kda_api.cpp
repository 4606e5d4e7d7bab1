// C-ABI layer of libkda: host-side argument validation, kernel selection and
// error mapping. Reads no device memory, allocates nothing and never
// synchronises; see include/kda.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "kda.h"
#include "kda_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

bool dtype_pair_ok(kda_dtype_t in, kda_dtype_t out) {
    if (in == KDA_F32) return out == KDA_F32;
    if (in == KDA_BF16) return out == KDA_BF16 || out == KDA_F32;
    return false;
}

bool dtype_valid(kda_dtype_t d) { return d == KDA_F32 || d == KDA_BF16; }

// Debug override of the prefill kernel for bf16 inputs: KDA_PREFILL_KERNEL=valu
// selects the fp32 vector-ALU kernel. Read once per process.
bool force_valu() {
    static const bool f = [] {
        const char *e = std::getenv("KDA_PREFILL_KERNEL");
        return e && std::strcmp(e, "valu") == 0;
    }();
    return f;
}

// Debugging aid: KDA_DEBUG_SYNC=1 waits for each call's work, so that an error while
// it runs is reported by that call (as KDA_ERR_HIP). Read once per process; not for
// use under graph capture.
bool debug_sync() {
    static const bool f = [] {
        const char *e = std::getenv("KDA_DEBUG_SYNC");
        return e && std::strcmp(e, "1") == 0;
    }();
    return f;
}
hipError_t finish(hipError_t e, hipStream_t stream) {
    if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(stream);
    if (e == hipSuccess && debug_sync()) e = hipGetLastError();
    return e;
}

}  // namespace

namespace {

// Options: neutral values when `opt` is NULL; otherwise checked against the
// sizes. `tokens`: the call has tokens (without any, no gate is read and both
// gate forms may be absent). Returns KDA_OK or the status to report.
kda_status_t check_options(const kda_options_t *opt, int32_t H, bool has_log_alpha, bool has_beta,
                           bool prefill, bool tokens, kda_options_t &o) {
    o = kda_options_t{};
    if (opt) o = *opt;
    if (o.num_k_heads == 0) o.num_k_heads = H;
    if (o.num_k_heads < 1 || H % o.num_k_heads != 0) return KDA_ERR_INVALID_ARG;
    // one gate form of each kind, never both
    if ((o.gate_x && has_log_alpha) || (o.beta_y && has_beta)) return KDA_ERR_INVALID_ARG;
    if (tokens && ((!o.gate_x && !has_log_alpha) || (!o.beta_y && !has_beta))) return KDA_ERR_INVALID_ARG;
    if (o.gate_x && !(o.gate_scale > 0.f && o.gate_scale < 3.0e38f)) return KDA_ERR_INVALID_ARG;
    if (!(o.norm_eps >= 0.f && o.norm_eps < 3.0e38f)) return KDA_ERR_INVALID_ARG;
    if (o.out_gate_act != KDA_ACT_NONE && o.out_gate_act != KDA_ACT_SIGMOID) return KDA_ERR_INVALID_ARG;
    const void *ptrs[] = {o.gate_x, o.beta_y, o.norm_weight, o.out_gate, o.state_slots};
    for (const void *p : ptrs)
        if (!aligned16(p)) return KDA_ERR_INVALID_ARG;
    if (prefill && o.state_slots && o.num_slots < 1) return KDA_ERR_INVALID_ARG;
    if (!prefill) {
        o.state_slots = nullptr;
        o.num_slots = 0;
    }
    return KDA_OK;
}

kda_status_t chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
                       const int32_t *cu_seqlens, int32_t N, int32_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                       kda_dtype_t in_dtype, kda_dtype_t out_dtype, float scale, const float *initial_state,
                       float *final_state, void *o, int32_t chunk_size, void *workspace, size_t workspace_bytes,
                       const kda_options_t *opt, hipStream_t stream, bool noalloc = false) {
    if (N < 1 || H < 1 || T_total < 0) return KDA_ERR_INVALID_ARG;
    if (!dtype_valid(in_dtype) || !dtype_valid(out_dtype)) return KDA_ERR_INVALID_ARG;
    if (!cu_seqlens || !aligned16(cu_seqlens)) return KDA_ERR_INVALID_ARG;
    kda_options_t op;
    const kda_status_t os = check_options(opt, H, log_alpha != nullptr, beta != nullptr, true, T_total > 0, op);
    if (os != KDA_OK) return os;
    if (T_total > 0) {
        const void *req[] = {q, k, v, op.gate_x ? op.gate_x : log_alpha, op.beta_y ? op.beta_y : beta, o};
        for (const void *p : req)
            if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
    }
    if (!aligned16(log_alpha) || !aligned16(beta)) return KDA_ERR_INVALID_ARG;
    if (!aligned16(initial_state) || !aligned16(final_state) || !aligned16(workspace))
        return KDA_ERR_INVALID_ARG;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v) || chunk_size != 64) return KDA_ERR_UNSUPPORTED;
    if (!dtype_pair_ok(in_dtype, out_dtype)) return KDA_ERR_UNSUPPORTED;
    // grid sizes are int32 on the device side, and so are token counts rounded up to whole chunks
    if (static_cast<int64_t>(N) * H * 16 > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if (T_total > INT32_MAX - 64) return KDA_ERR_INVALID_ARG;
    if (static_cast<int64_t>(T_total) * H * (d_k > d_v ? d_k : d_v) > (int64_t(1) << 40))
        return KDA_ERR_INVALID_ARG;
    const size_t need = kda_chunk_fwd_workspace_size(N, T_total, H, d_k, d_v, in_dtype);
    if (noalloc) {  // the library's static scratch, once every argument has passed
        if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
        workspace = nullptr;
        workspace_bytes = need;
        if (need > 0 && !(workspace = kda::noalloc_scratch())) return KDA_ERR_HIP;
    }
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;

    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = log_alpha; a.beta = beta; a.cu_seqlens = cu_seqlens;
    a.s0 = initial_state; a.sT = final_state; a.o = o;
    a.N = N; a.T = T_total; a.H = H; a.K = d_k; a.V = d_v; a.scale = scale;
    a.in_dtype = in_dtype; a.out_dtype = out_dtype;
    a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.Hk = op.num_k_heads; a.gx = op.gate_x; a.by = op.beta_y; a.gscale = op.gate_scale;
    a.norm = op.norm != 0; a.eps = op.norm_eps; a.nw = op.norm_weight; a.z = op.out_gate;
    a.zact = op.out_gate_act; a.slots = op.state_slots; a.nslots = op.num_slots;
    const bool epi = a.norm || a.z;
    hipError_t e;
    if (in_dtype == KDA_BF16 && !force_valu()) {
        e = kda::launch_prefill_mfma(a, stream);
    } else {
        e = kda::launch_prefill_valu(a, stream);
        if (e == hipSuccess && epi && T_total > 0) e = kda::launch_epilogue(a, stream);
    }
    return finish(e, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t decode_step(const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
                         float *state_cache, const int32_t *slot_idx, void *o, int32_t B, int32_t H, int32_t d_k,
                         int32_t d_v, int32_t num_slots, kda_dtype_t in_dtype, kda_dtype_t out_dtype, float scale,
                         const kda_options_t *opt, hipStream_t stream) {
    if (B < 1 || H < 1 || num_slots < 1) return KDA_ERR_INVALID_ARG;
    if (!dtype_valid(in_dtype) || !dtype_valid(out_dtype)) return KDA_ERR_INVALID_ARG;
    kda_options_t op;
    const kda_status_t os = check_options(opt, H, log_alpha != nullptr, beta != nullptr, false, true, op);
    if (os != KDA_OK) return os;
    const void *req[] = {q, k, v, op.gate_x ? op.gate_x : log_alpha, op.beta_y ? op.beta_y : beta, state_cache, o};
    for (const void *p : req)
        if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
    if (!aligned16(slot_idx) || !aligned16(log_alpha) || !aligned16(beta)) return KDA_ERR_INVALID_ARG;
    if (!slot_idx && B > num_slots) return KDA_ERR_INVALID_ARG;
    if (static_cast<int64_t>(B) * H > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
    if (!dtype_pair_ok(in_dtype, out_dtype)) return KDA_ERR_UNSUPPORTED;

    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = log_alpha; a.beta = beta; a.state = state_cache;
    a.slot_idx = slot_idx; a.o = o; a.B = B; a.H = H; a.K = d_k; a.V = d_v;
    a.slots = num_slots; a.scale = scale; a.in_dtype = in_dtype; a.out_dtype = out_dtype;
    a.Hk = op.num_k_heads; a.gx = op.gate_x; a.by = op.beta_y; a.gscale = op.gate_scale;
    a.norm = op.norm != 0; a.eps = op.norm_eps; a.nw = op.norm_weight; a.z = op.out_gate;
    a.zact = op.out_gate_act;
    return finish(kda::launch_decode(a, stream), stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_string(kda_status_t s) {
    switch (s) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: NULL or misaligned pointer, or size out of range";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head dims must be 64 or 128, chunk size 64, dtype pair F32/F32, BF16/BF16 or BF16/F32";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace smaller than kda_chunk_fwd_workspace_size()";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: kernel launch failed";
    }
    return "unknown kda_status_t";
}

size_t kda_chunk_fwd_workspace_size(int32_t N, int32_t T_total, int32_t H, int32_t d_k,
                                    int32_t d_v, kda_dtype_t in_dtype) {
    if (N < 1 || H < 1 || T_total < 0 || T_total > INT32_MAX - 64 || !head_dim_ok(d_k) || !head_dim_ok(d_v))
        return 0;
    // both paths stage every chunk's state-independent operands in the workspace
    if (in_dtype == KDA_BF16 && !force_valu()) return kda::prefill_mfma_workspace(N, T_total, H, d_k, d_v);
    return kda::prefill_valu_workspace(N, T_total, H, d_k);
}


kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, const int32_t *cu_seqlens, int32_t N, int32_t T_total,
                           int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t in_dtype,
                           kda_dtype_t out_dtype, float scale, const float *initial_state,
                           float *final_state, void *o, int32_t chunk_size, void *workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    // the plain form needs both gate tensors
    if (T_total > 0 && (!log_alpha || !beta)) return KDA_ERR_INVALID_ARG;
    return chunk_fwd(q, k, v, log_alpha, beta, cu_seqlens, N, T_total, H, d_k, d_v, in_dtype, out_dtype, scale,
                     initial_state, final_state, o, chunk_size, workspace, workspace_bytes, nullptr, stream);
}

kda_status_t kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *log_alpha,
                              const float *beta, const int32_t *cu_seqlens, int32_t N, int32_t T_total,
                              int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t in_dtype,
                              kda_dtype_t out_dtype, float scale, const float *initial_state,
                              float *final_state, void *o, int32_t chunk_size, void *workspace,
                              size_t workspace_bytes, const kda_options_t *opt, hipStream_t stream) {
    return chunk_fwd(q, k, v, log_alpha, beta, cu_seqlens, N, T_total, H, d_k, d_v, in_dtype, out_dtype, scale,
                     initial_state, final_state, o, chunk_size, workspace, workspace_bytes, opt, stream);
}

kda_status_t kda_chunk_fwd_ex_noalloc(const void *q, const void *k, const void *v, const float *log_alpha,
                                      const float *beta, const int32_t *cu_seqlens, int32_t N, int32_t T_total,
                                      int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t in_dtype,
                                      kda_dtype_t out_dtype, float scale, const float *initial_state,
                                      float *final_state, void *o, int32_t chunk_size, const kda_options_t *opt,
                                      hipStream_t stream) {
    return chunk_fwd(q, k, v, log_alpha, beta, cu_seqlens, N, T_total, H, d_k, d_v, in_dtype, out_dtype, scale,
                     initial_state, final_state, o, chunk_size, nullptr, 0, opt, stream, true);
}

kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                             const float *beta, float *state_cache, const int32_t *slot_idx,
                             void *o, int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                             int32_t num_slots, kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                             float scale, hipStream_t stream) {
    if (!log_alpha || !beta) return KDA_ERR_INVALID_ARG;
    return decode_step(q, k, v, log_alpha, beta, state_cache, slot_idx, o, B, H, d_k, d_v, num_slots, in_dtype,
                       out_dtype, scale, nullptr, stream);
}

kda_status_t kda_decode_step_ex(const void *q, const void *k, const void *v, const float *log_alpha,
                                const float *beta, float *state_cache, const int32_t *slot_idx,
                                void *o, int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                                int32_t num_slots, kda_dtype_t in_dtype, kda_dtype_t out_dtype,
                                float scale, const kda_options_t *opt, hipStream_t stream) {
    return decode_step(q, k, v, log_alpha, beta, state_cache, slot_idx, o, B, H, d_k, d_v, num_slots, in_dtype,
                       out_dtype, scale, opt, stream);
}

}  // extern "C"
