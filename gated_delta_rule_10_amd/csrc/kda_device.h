// Device helpers shared by the KDA kernels: element loads/stores for the two
// I/O types (fp32 and bf16 carried as raw 16-bit patterns).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

using bf16_t = uint16_t;  // raw bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct io;

template <> struct io<float> {
    __device__ __forceinline__ static float load(const float *p) { return *p; }
    __device__ __forceinline__ static void store(float *p, float x) { *p = x; }
    __device__ __forceinline__ static float4 load4(const float *p) {
        return *reinterpret_cast<const float4 *>(p);
    }
    __device__ __forceinline__ static void store4(float *p, float4 x) {
        *reinterpret_cast<float4 *>(p) = x;
    }
};

template <> struct io<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t *p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void store(bf16_t *p, float x) { *p = f32_to_bf16(x); }
    __device__ __forceinline__ static float4 load4(const bf16_t *p) {
        const uint2 w = *reinterpret_cast<const uint2 *>(p);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
    }
    __device__ __forceinline__ static void store4(bf16_t *p, float4 x) {
        uint2 w;
        w.x = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
        w.y = static_cast<uint32_t>(f32_to_bf16(x.z)) | (static_cast<uint32_t>(f32_to_bf16(x.w)) << 16);
        *reinterpret_cast<uint2 *>(p) = w;
    }
};

// Read-only int32 metadata (offsets, sequence bounds, slot indices) that no
// kernel of the launch writes: read through the constant address space, so that
// a uniform index becomes a scalar load. A vector load would be counted with the
// stores in flight, and its first use would wait for all of them.
__device__ __forceinline__ int32_t ld_meta(const int32_t *p, int i) {
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

// Gate activations of the extended entry points (kda_options_t):
// log alpha = -scale * softplus(x), softplus(x) = ln(1 + e^x) = max(x, 0) + ln(1 + e^-|x|);
// beta = sigmoid(y) = 1 / (1 + e^-y).
__device__ __forceinline__ float log_alpha_from(float x, float scale) {
    return -scale * (fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x))));
}
__device__ __forceinline__ float sigmoid_f(float y) { return 1.f / (1.f + __expf(-y)); }
// output gate act(z): KDA_ACT_NONE -> z, KDA_ACT_SIGMOID -> sigmoid(z)
__device__ __forceinline__ float out_gate_act(float z, int act) { return act == KDA_ACT_SIGMOID ? sigmoid_f(z) : z; }

__device__ __forceinline__ float4 operator*(float4 a, float s) {
    return make_float4(a.x * s, a.y * s, a.z * s, a.w * s);
}
__device__ __forceinline__ float4 operator+(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 operator-(float4 a, float4 b) {
    return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}
__device__ __forceinline__ float4 fma4(float4 a, float s, float4 c) {
    return make_float4(fmaf(a.x, s, c.x), fmaf(a.y, s, c.y), fmaf(a.z, s, c.z), fmaf(a.w, s, c.w));
}

}  // namespace kda
