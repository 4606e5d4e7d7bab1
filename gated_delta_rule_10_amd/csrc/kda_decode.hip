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
// Mapping: two 512-thread workgroups per (b, h), each with half of the d_v
// columns: the column reductions run over d_k only, so the halves are
// independent (they both read the small inputs). The RMS norm of the output
// epilogue needs whole rows and keeps one workgroup per (b, h). A state row of
// NC floats is covered by NC/4 lanes reading float4, so one wave load
// instruction reads 64 * 16 B = 1 KiB in rows of NC * 4 bytes. Each lane keeps
// its d_k*NC/1024 float4s in registers between the read and the write. The small
// inputs are loaded first, so that they arrive while the state loads are in
// flight: one load per key channel of the gate, k and q (staged through LDS as
// (alpha, k, q) for the lanes of every row), and each lane's four columns of v,
// and of the norm weight and output gate when given. The two column reductions
// over d_k run in registers, across lanes of a wave with xor-shuffles, and
// across the eight waves through LDS.
//
// The state is read and written with nontemporal accesses: each byte is touched
// once per step, and a model's caches (one per layer) far exceed the 256 MB
// Infinity Cache, so streaming past the caches is what each step costs from HBM
// (measured with the caches cycled: 47.3 against 54.0 us per step at B = 64,
// H = 32, d = 128). A single cache small enough to stay in the Infinity Cache
// between steps no longer benefits from it (48.8 against 42.1 us).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef float nf4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float *p) {
    const nf4 v = __builtin_nontemporal_load(reinterpret_cast<const nf4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(float *p, float4 x) {
    __builtin_nontemporal_store(nf4{x.x, x.y, x.z, x.w}, reinterpret_cast<nf4 *>(p));
}

constexpr int kDecWaves = 8;
constexpr int kDecSplit = 2;  // workgroups per (b, h), each with d_v / kDecSplit columns

template <int K, int V, int NC, typename TIn, typename TOut>
__global__ __launch_bounds__(64 * kDecWaves) void decode_kernel(DecodeArgs a) {
    constexpr int LPR = NC / 4;                      // lanes per state row (NC of its d_v columns)
    constexpr int RPI = 64 / LPR;                    // rows per wave load
    constexpr int ITERS = K / (kDecWaves * RPI);     // float4 per lane
    static_assert(ITERS * kDecWaves * RPI == K, "row mapping must cover d_k");
    static_assert(K % 64 == 0 && K <= 64 * kDecWaves, "one key channel per thread of the first waves");
    __shared__ float4 vec[K];  // (alpha, k, q, -) per key channel
    __shared__ float kqp[K / 64];
    __shared__ float4 red_r[kDecWaves][LPR];
    __shared__ float4 red_p[kDecWaves][LPR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c4 = lane % LPR, rsub = lane / LPR;
    const int bh = blockIdx.x / (V / NC), col0 = NC * (blockIdx.x - bh * (V / NC));
    const int b = bh / a.H, h = bh - b * a.H;
    // value head h reads key head h / (H / Hk)
    const size_t bhk = static_cast<size_t>(b) * a.Hk + h / (a.H / a.Hk);

    // ---- small inputs first
    float gk = 0.f, kk = 0.f, qk = 0.f;
    if (tid < K) {
        gk = a.gx ? io<TIn>::load(static_cast<const TIn *>(a.gx) + static_cast<size_t>(bh) * K + tid)
                  : a.g[static_cast<size_t>(bh) * K + tid];
        kk = io<TIn>::load(static_cast<const TIn *>(a.k) + bhk * K + tid);
        qk = io<TIn>::load(static_cast<const TIn *>(a.q) + bhk * K + tid);
    }
    const float4 vv = io<TIn>::load4(static_cast<const TIn *>(a.v) + static_cast<size_t>(bh) * V + col0 + c4 * 4);
    const float braw = a.by ? io<TIn>::load(static_cast<const TIn *>(a.by) + bh) : a.beta[bh];
    float4 zv = make_float4(1.f, 1.f, 1.f, 1.f), wv = zv;
    if (a.z) zv = io<TIn>::load4(static_cast<const TIn *>(a.z) + static_cast<size_t>(bh) * V + col0 + c4 * 4);
    if (a.norm && a.nw) wv = io<float>::load4(a.nw + col0 + c4 * 4);

    // ---- the state
    const int slot = a.slot_idx ? ld_meta(a.slot_idx, b) : b;
    float *S = a.state + (static_cast<size_t>(slot) * a.H + h) * static_cast<size_t>(K * V);
    float4 s[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int row = (it * kDecWaves + w) * RPI + rsub;
        s[it] = load_stream(S + row * V + col0 + c4 * 4);
    }

    if (tid < K) {
        const float al = __expf(a.gx ? log_alpha_from(gk, a.gscale) : gk);
        vec[tid] = make_float4(al, kk, qk, 0.f);
        float kq = kk * qk;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) kq += __shfl_xor(kq, m);
        if (lane == 0) kqp[w] = kq;
    }
    __syncthreads();

    // S' = Diag(alpha) S; r = S'^T k; p = S'^T q
    float4 r4 = make_float4(0.f, 0.f, 0.f, 0.f), p4 = r4;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int row = (it * kDecWaves + w) * RPI + rsub;
        const float4 c = vec[row];
        s[it] = s[it] * c.x;
        r4 = fma4(s[it], c.y, r4);
        p4 = fma4(s[it], c.z, p4);
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
    __syncthreads();
    float4 r = red_r[0][c4], p = red_p[0][c4];
#pragma unroll
    for (int ww = 1; ww < kDecWaves; ++ww) {
        r = r + red_r[ww][c4];
        p = p + red_p[ww][c4];
    }
    float kq = kqp[0];
#pragma unroll
    for (int i = 1; i < K / 64; ++i) kq += kqp[i];
    const float bt = a.by ? sigmoid_f(braw) : braw;
    const float4 u = (vv - r) * bt;
    float4 ov = fma4(u, kq, p) * a.scale;
    if (a.norm) {  // o / sqrt(mean o^2 + eps) over the LPR lanes of the row (uniform branch; NC == V)
        float ss = ov.x * ov.x + ov.y * ov.y + ov.z * ov.z + ov.w * ov.w;
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m);
        ov = ov * rsqrtf(ss / V + a.eps);
        ov = make_float4(ov.x * wv.x, ov.y * wv.y, ov.z * wv.z, ov.w * wv.w);
    }
    if (a.z) {
        ov = make_float4(ov.x * out_gate_act(zv.x, a.zact), ov.y * out_gate_act(zv.y, a.zact),
                         ov.z * out_gate_act(zv.z, a.zact), ov.w * out_gate_act(zv.w, a.zact));
    }
    if (w == 0 && rsub == 0) {
        TOut *op = static_cast<TOut *>(a.o) + static_cast<size_t>(bh) * V;
        io<TOut>::store4(op + col0 + c4 * 4, ov);
    }
    // S = S' + k u^T
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int row = (it * kDecWaves + w) * RPI + rsub;
        store_stream(S + row * V + col0 + c4 * 4, fma4(u, vec[row].y, s[it]));
    }
}

template <int K, int V, int NC>
hipError_t launch_nc(const DecodeArgs &a, hipStream_t st) {
    const dim3 grid(a.B * a.H * (V / NC)), block(64 * kDecWaves);
    if (a.in_dtype == KDA_F32)
        hipLaunchKernelGGL((decode_kernel<K, V, NC, float, float>), grid, block, 0, st, a);
    else if (a.out_dtype == KDA_BF16)
        hipLaunchKernelGGL((decode_kernel<K, V, NC, bf16_t, bf16_t>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((decode_kernel<K, V, NC, bf16_t, float>), grid, block, 0, st, a);
    return hipGetLastError();
}

// The RMS norm of the output epilogue spans a whole row of d_v columns, so it
// keeps one workgroup per (b, h); otherwise kDecSplit workgroups share the columns.
template <int K, int V>
hipError_t launch_kv(const DecodeArgs &a, hipStream_t st) {
    if (a.norm || kDecSplit == 1) return launch_nc<K, V, V>(a, st);
    return launch_nc<K, V, V / kDecSplit>(a, st);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
    if (a.K == 128 && a.V == 128) return launch_kv<128, 128>(a, st);
    if (a.K == 128 && a.V == 64) return launch_kv<128, 64>(a, st);
    if (a.K == 64 && a.V == 128) return launch_kv<64, 128>(a, st);
    return launch_kv<64, 64>(a, st);
}

}  // namespace kda
