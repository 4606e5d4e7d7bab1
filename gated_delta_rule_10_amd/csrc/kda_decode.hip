// KDA single-token decode: one read-modify-write of the fp32 state cache.
//
// Per (b, h), with S the d_k x d_v state of slot s(b) (row i = key channel i):
//   S' = Diag(exp(g)) S;  r = S'^T k;  p = S'^T q;  u = beta (v - r)
//   S  = S' + k u^T  (in place);  o = scale * (p + (k . q) u)
// The last line is S^T q for the updated S, expanded so that the state is
// read and written exactly once. Token loop of the 2025 attention review
// page, section "GatedDeltaNet解读" (decay, correction against the decayed
// state, rank-1 write, read-out from the updated state), with the gate per key
// channel as in its section "KLA"; the state cache is one contiguous
// [slots, H, d_k, d_v] array as in "线性注意力机制Kimi Linear架构解析与优化实践", section 3.2.
//
// Mapping: one 256-thread workgroup per (b, h). A state row of d_v floats is
// covered by d_v/4 lanes reading float4, so one wave load instruction reads
// 64 * 16 B = 1 KiB of consecutive rows (fully coalesced). Each lane keeps its
// d_k*d_v/1024 float4s in registers between the read and the write. The two
// column reductions over d_k run in registers, across lanes of a wave with
// xor-shuffles, and across the four waves through 2 KiB of LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kDecWaves = 4;

template <int K, int V, typename TIn, typename TOut>
__global__ __launch_bounds__(64 * kDecWaves) void decode_kernel(DecodeArgs a) {
    constexpr int LPR = V / 4;                       // lanes per state row
    constexpr int RPI = 64 / LPR;                    // rows per wave load
    constexpr int ITERS = K / (kDecWaves * RPI);     // float4 per lane
    static_assert(ITERS * kDecWaves * RPI == K, "row mapping must cover d_k");
    __shared__ float4 red_r[kDecWaves][LPR];
    __shared__ float4 red_p[kDecWaves][LPR];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c4 = lane % LPR, rsub = lane / LPR;
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H;
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    float *S = a.state + (static_cast<size_t>(slot) * a.H + h) * static_cast<size_t>(K * V);
    // value head h reads key head h / (H / Hk)
    const size_t bhk = static_cast<size_t>(b) * a.Hk + h / (a.H / a.Hk);
    const TIn *qp = static_cast<const TIn *>(a.q) + bhk * K;
    const TIn *kp = static_cast<const TIn *>(a.k) + bhk * K;
    const TIn *vp = static_cast<const TIn *>(a.v) + static_cast<size_t>(bh) * V;
    const float *gp = a.g + static_cast<size_t>(bh) * K;
    const TIn *gxp = static_cast<const TIn *>(a.gx) + static_cast<size_t>(bh) * K;

    float4 s[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int row = (it * kDecWaves + w) * RPI + rsub;
        s[it] = io<float>::load4(S + row * V + c4 * 4);
    }
    float kr[ITERS];
    float4 r4 = make_float4(0.f, 0.f, 0.f, 0.f), p4 = r4;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int row = (it * kDecWaves + w) * RPI + rsub;
        const float al = __expf(a.gx ? log_alpha_from(io<TIn>::load(gxp + row), a.gscale) : gp[row]);
        const float kv = io<TIn>::load(kp + row), qv = io<TIn>::load(qp + row);
        s[it] = s[it] * al;
        r4 = fma4(s[it], kv, r4);
        p4 = fma4(s[it], qv, p4);
        kr[it] = kv;
    }
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) {
        r4.x += __shfl_xor(r4.x, m); r4.y += __shfl_xor(r4.y, m);
        r4.z += __shfl_xor(r4.z, m); r4.w += __shfl_xor(r4.w, m);
        p4.x += __shfl_xor(p4.x, m); p4.y += __shfl_xor(p4.y, m);
        p4.z += __shfl_xor(p4.z, m); p4.w += __shfl_xor(p4.w, m);
    }
    if (rsub == 0) {
        red_r[w][c4] = r4;
        red_p[w][c4] = p4;
    }
    float kq = 0.f;
    for (int i = lane; i < K; i += 64) kq += io<TIn>::load(kp + i) * io<TIn>::load(qp + i);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) kq += __shfl_xor(kq, m);
    __syncthreads();
    float4 r = red_r[0][c4], p = red_p[0][c4];
#pragma unroll
    for (int ww = 1; ww < kDecWaves; ++ww) {
        r = r + red_r[ww][c4];
        p = p + red_p[ww][c4];
    }
    const float bt = a.by ? sigmoid_f(io<TIn>::load(static_cast<const TIn *>(a.by) + bh)) : a.beta[bh];
    const float4 u = (io<TIn>::load4(vp + c4 * 4) - r) * bt;
    float4 ov = fma4(u, kq, p) * a.scale;
    if (a.norm) {  // o / sqrt(mean o^2 + eps) over the LPR lanes of the row (uniform branch)
        float ss = ov.x * ov.x + ov.y * ov.y + ov.z * ov.z + ov.w * ov.w;
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m);
        ov = ov * rsqrtf(ss / V + a.eps);
        if (a.nw) {
            const float4 wv = io<float>::load4(a.nw + c4 * 4);
            ov = make_float4(ov.x * wv.x, ov.y * wv.y, ov.z * wv.z, ov.w * wv.w);
        }
    }
    if (a.z) {
        const float4 zv = io<TIn>::load4(static_cast<const TIn *>(a.z) + static_cast<size_t>(bh) * V + c4 * 4);
        ov = make_float4(ov.x * out_gate_act(zv.x, a.zact), ov.y * out_gate_act(zv.y, a.zact),
                         ov.z * out_gate_act(zv.z, a.zact), ov.w * out_gate_act(zv.w, a.zact));
    }
    if (w == 0 && rsub == 0) {
        TOut *op = static_cast<TOut *>(a.o) + static_cast<size_t>(bh) * V;
        io<TOut>::store4(op + c4 * 4, ov);
    }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int row = (it * kDecWaves + w) * RPI + rsub;
        io<float>::store4(S + row * V + c4 * 4, fma4(u, kr[it], s[it]));
    }
}

template <int K, int V>
hipError_t launch_kv(const DecodeArgs &a, hipStream_t st) {
    const dim3 grid(a.B * a.H), block(64 * kDecWaves);
    if (a.in_dtype == KDA_F32)
        hipLaunchKernelGGL((decode_kernel<K, V, float, float>), grid, block, 0, st, a);
    else if (a.out_dtype == KDA_BF16)
        hipLaunchKernelGGL((decode_kernel<K, V, bf16_t, bf16_t>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((decode_kernel<K, V, bf16_t, float>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
    if (a.K == 128 && a.V == 128) return launch_kv<128, 128>(a, st);
    if (a.K == 128 && a.V == 64) return launch_kv<128, 64>(a, st);
    if (a.K == 64 && a.V == 128) return launch_kv<64, 128>(a, st);
    return launch_kv<64, 64>(a, st);
}

}  // namespace kda
