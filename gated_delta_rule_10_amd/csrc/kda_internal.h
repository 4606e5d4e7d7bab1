// Internal launch interface between the C-ABI layer (kda_api.cpp) and the
// HIP kernels. Not installed; the public interface is include/kda.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

struct PrefillArgs {
    const void *q, *k, *v;       // [T, H, K|K|V] in_dtype
    const float *g;              // log alpha [T, H, K]
    const float *beta;           // [T, H]
    const int32_t *cu_seqlens;   // [N + 1] device
    const float *s0;             // [N, H, K, V] or nullptr
    float *sT;                   // [N, H, K, V] or nullptr
    void *o;                     // [T, H, V] out_dtype
    int32_t N, T, H, K, V;
    float scale;
    kda_dtype_t in_dtype, out_dtype;
    void *ws;                    // caller workspace (the per-chunk records)
    size_t ws_bytes;
    // options (kda_options_t); neutral values give the plain operator
    int32_t Hk;                  // key/query heads; value head h uses key head h / (H / Hk)
    const void *gx;              // gate pre-activation [T, H, K] in_dtype (replaces g) or nullptr
    const void *by;              // beta pre-activation [T, H] in_dtype (replaces beta) or nullptr
    float gscale;                // log alpha = -gscale * softplus(gx)
    int32_t norm;                // RMS-normalise o over d_v
    float eps;
    const float *nw;             // [V] or nullptr
    const void *z;               // output gate [T, H, V] in_dtype or nullptr
    int32_t zact;                // kda_act_t
    const int32_t *slots;        // [N] state slots or nullptr (s0 / sT are then caches)
    int32_t nslots;
};

struct DecodeArgs {
    const void *q, *k, *v;   // [B, H, K|K|V]
    const float *g;          // [B, H, K]
    const float *beta;       // [B, H]
    float *state;            // [slots, H, K, V]
    const int32_t *slot_idx; // [B] or nullptr
    void *o;                 // [B, H, V]
    int32_t B, H, K, V, slots;
    float scale;
    kda_dtype_t in_dtype, out_dtype;
    int32_t Hk;
    const void *gx, *by;
    float gscale;
    int32_t norm;
    float eps;
    const float *nw;
    const void *z;
    int32_t zact;
};

// Each launcher enqueues its kernel(s) on `stream` and returns the launch
// status (hipGetLastError after the launch).
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_prefill_valu(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream);
// o <- epilogue(o) in place, per (token, head) row (the fp32-path epilogue)
hipError_t launch_epilogue(const PrefillArgs &a, hipStream_t stream);

// Workspace bytes of the matrix-core prefill (0 for d_k/d_v it cannot run).
size_t prefill_mfma_workspace(int32_t N, int32_t T, int32_t H, int32_t K, int32_t V);
// workspace of the fp32 vector-ALU path: one fp32 record per (chunk slot, head)
size_t prefill_valu_workspace(int32_t N, int32_t T, int32_t H, int32_t K);

// Device address of the current device's copy of the static scratch of
// kda_chunk_fwd_ex_noalloc (KDA_NOALLOC_SCRATCH_BYTES), looked up once per
// device; nullptr if the lookup fails.
void *noalloc_scratch();

}  // namespace kda
