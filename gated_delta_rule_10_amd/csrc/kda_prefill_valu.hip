// KDA chunk prefill, fp32 vector-ALU kernel (the fp32-input path).
//
// Chunkwise form ("Kimi Linear爆发背后的秘密" page, section "硬件效率的深度优化":
// parallel inside a chunk, recurrent across chunks, WY representation, UT
// transform; 64-token chunks as in "线性注意力机制Kimi Linear架构解析与优化实践",
// section 2.2; cumulative decay in log space, its section 4.2). For a chunk of
// n <= 64 tokens with incoming state S and G_r = sum_{s<=r} g_s per channel:
//   A  = strict_lower(Diag(beta) [sum_i k_r[i] k_s[i] e^{G_r[i]-G_s[i]}])
//   P  = lower_incl([sum_i q_r[i] k_s[i] e^{G_r[i]-G_s[i]}])
//   T  = (I + A)^{-1}                               (UT transform)
//   U' = T Diag(beta) (V - (K . e^G) S)             (WY pseudo-values)
//   O  = scale ((Q . e^G) S + P U')
//   S  <- Diag(e^{G_n}) S + (K . e^{G_n - G})^T U'
// Substituting S_r = Diag(e^{G_r})S + sum_{s<=r} Diag(e^{G_r-G_s}) k_s u_s^T
// into the token recurrence gives (I + A) U' = Diag(beta)(V - (K.e^G) S),
// hence these lines exactly.
//
// Every quantity is fp32; the pairwise decays are evaluated element by
// element (one exp per (r, s, channel)), so no factorisation can overflow.
// Rows past the end of a partial chunk are zero-filled with g = 0 and
// beta = 0, which makes them contribute nothing.
//
// Mapping: one 256-thread workgroup per (sequence, head, 16 value columns);
// the chunk's q/k/G tiles, A/T, P, the 16-column state slice and the
// pseudo-values live in LDS (about 149 KB at d_k = 128).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;    // chunk length
constexpr int kVT = 16;   // value columns per workgroup
constexpr int kNT = 256;  // threads per workgroup

template <int K>
struct ValuSmem {
    static constexpr int KP = K + 1, CP = kC + 1;
    float G[kC * KP];   // cumulative log decay, then K . e^{G_n - G}
    float KK[kC * KP];  // k, then K . e^G
    float QQ[kC * KP];  // q, then Q . e^G
    float A[kC * CP];   // strict-lower A, then T = (I + A)^{-1} below the diagonal
    float P[kC * CP];
    float S[K * kVT];
    float X[kC * kVT];  // v, then Diag(beta)(V - (K.e^G) S)
    float U[kC * kVT];  // U'
    float glast[K];
    float gam[K];
    float bet[kC];
};

template <int K, int V, typename TIn, typename TOut>
__global__ __launch_bounds__(kNT) void prefill_valu_kernel(PrefillArgs a) {
    constexpr int KP = K + 1, CP = kC + 1;
    constexpr int NVT = V / kVT;
    __shared__ ValuSmem<K> sm;
    const int tid = threadIdx.x;
    int bid = blockIdx.x;
    const int vt = bid % NVT;
    bid /= NVT;
    const int h = bid % a.H, n = bid / a.H;
    const int j0 = vt * kVT;
    const int H = a.H;
    const int tbeg = a.cu_seqlens[n], tend = a.cu_seqlens[n + 1];
    const TIn *qg = static_cast<const TIn *>(a.q);
    const TIn *kg = static_cast<const TIn *>(a.k);
    const TIn *vg = static_cast<const TIn *>(a.v);
    TOut *og = static_cast<TOut *>(a.o);
    // states: [N, H, K, V], or with slots a cache [slots, H, K, V] read and written at slot[n]
    // (a negative slot: zero initial state, final state not written)
    const int slot = a.slots ? a.slots[n] : n;
    const size_t sbase = (static_cast<size_t>(slot) * H + h) * static_cast<size_t>(K) * V;
    const float *s0 = slot >= 0 ? a.s0 : nullptr;
    float *sT = slot >= 0 ? a.sT : nullptr;
    const int Hk = a.Hk, hk = h / (H / Hk);  // key head of value head h

    for (int idx = tid; idx < K * kVT; idx += kNT) {
        const int i = idx / kVT, c = idx % kVT;
        sm.S[idx] = s0 ? s0[sbase + static_cast<size_t>(i) * V + j0 + c] : 0.f;
    }

    for (int t0 = tbeg; t0 < tend; t0 += kC) {
        const int nt = min(kC, tend - t0);
        __syncthreads();
        for (int idx = tid; idx < kC * K; idx += kNT) {
            const int r = idx / K, i = idx % K;
            const bool ok = r < nt;
            const size_t off = (static_cast<size_t>(t0 + r) * H + h) * K + i;
            const size_t offk = (static_cast<size_t>(t0 + r) * Hk + hk) * K + i;
            sm.KK[r * KP + i] = ok ? io<TIn>::load(kg + offk) : 0.f;
            sm.QQ[r * KP + i] = ok ? io<TIn>::load(qg + offk) : 0.f;
            float gv = 0.f;
            if (ok) gv = a.gx ? log_alpha_from(io<TIn>::load(static_cast<const TIn *>(a.gx) + off), a.gscale) : a.g[off];
            sm.G[r * KP + i] = gv;
        }
        for (int idx = tid; idx < kC * kVT; idx += kNT) {
            const int r = idx / kVT, c = idx % kVT;
            sm.X[idx] = r < nt ? io<TIn>::load(vg + (static_cast<size_t>(t0 + r) * H + h) * V + j0 + c)
                               : 0.f;
        }
        if (tid < kC) {
            float bv = 0.f;
            if (tid < nt) {
                const size_t off = static_cast<size_t>(t0 + tid) * H + h;
                bv = a.by ? sigmoid_f(io<TIn>::load(static_cast<const TIn *>(a.by) + off)) : a.beta[off];
            }
            sm.bet[tid] = bv;
        }
        __syncthreads();
        if (tid < K) {  // inclusive cumulative sum of log alpha over the chunk
            float acc = 0.f;
            for (int r = 0; r < kC; ++r) {
                acc += sm.G[r * KP + tid];
                sm.G[r * KP + tid] = acc;
            }
            sm.glast[tid] = acc;
            sm.gam[tid] = __expf(acc);
        }
        __syncthreads();
        for (int p = tid; p < kC * kC; p += kNT) {  // A and P, one (r, s) pair each
            const int r = p / kC, s = p % kC;
            float aa = 0.f, pp = 0.f;
            if (s <= r) {
                for (int i = 0; i < K; ++i) {
                    const float ks = sm.KK[s * KP + i] * __expf(sm.G[r * KP + i] - sm.G[s * KP + i]);
                    aa = fmaf(sm.KK[r * KP + i], ks, aa);
                    pp = fmaf(sm.QQ[r * KP + i], ks, pp);
                }
            }
            sm.A[r * CP + s] = s < r ? sm.bet[r] * aa : 0.f;
            sm.P[r * CP + s] = pp;
        }
        __syncthreads();
        // T = (I + A)^{-1}, row by row: T[r][c] = -sum_{c<=s<r} A[r][s] T[s][c],
        // T[c][c] = 1. Row r of T overwrites row r of A once it is complete.
        for (int r = 1; r < kC; ++r) {
            float t = 0.f;
            if (tid < r) {
                t = -sm.A[r * CP + tid];
                for (int s = tid + 1; s < r; ++s) t = fmaf(-sm.A[r * CP + s], sm.A[s * CP + tid], t);
            }
            __syncthreads();
            if (tid < r) sm.A[r * CP + tid] = t;
            __syncthreads();
        }
        for (int idx = tid; idx < kC * K; idx += kNT) {  // decayed operands, in place
            const int r = idx / K, i = idx % K;
            const float G = sm.G[r * KP + i];
            const float e1 = __expf(G), e2 = __expf(sm.glast[i] - G);
            const float kv = sm.KK[r * KP + i];
            sm.KK[r * KP + i] = kv * e1;
            sm.QQ[r * KP + i] *= e1;
            sm.G[r * KP + i] = kv * e2;
        }
        __syncthreads();
        for (int idx = tid; idx < kC * kVT; idx += kNT) {  // X = Diag(beta)(V - (K.e^G) S)
            const int r = idx / kVT, c = idx % kVT;
            float acc = 0.f;
            for (int i = 0; i < K; ++i) acc = fmaf(sm.KK[r * KP + i], sm.S[i * kVT + c], acc);
            sm.X[idx] = sm.bet[r] * (sm.X[idx] - acc);
        }
        __syncthreads();
        for (int idx = tid; idx < kC * kVT; idx += kNT) {  // U' = T X
            const int r = idx / kVT, c = idx % kVT;
            float acc = sm.X[idx];
            for (int s = 0; s < r; ++s) acc = fmaf(sm.A[r * CP + s], sm.X[s * kVT + c], acc);
            sm.U[idx] = acc;
        }
        __syncthreads();
        for (int idx = tid; idx < kC * kVT; idx += kNT) {  // O = (Q.e^G) S + P U'
            const int r = idx / kVT, c = idx % kVT;
            if (r < nt) {
                float acc = 0.f;
                for (int i = 0; i < K; ++i) acc = fmaf(sm.QQ[r * KP + i], sm.S[i * kVT + c], acc);
                for (int s = 0; s <= r; ++s) acc = fmaf(sm.P[r * CP + s], sm.U[s * kVT + c], acc);
                io<TOut>::store(og + (static_cast<size_t>(t0 + r) * H + h) * V + j0 + c, a.scale * acc);
            }
        }
        __syncthreads();
        for (int idx = tid; idx < K * kVT; idx += kNT) {  // S <- e^{G_n} S + (K.e^{G_n-G})^T U'
            const int i = idx / kVT, c = idx % kVT;
            float acc = sm.gam[i] * sm.S[idx];
            for (int r = 0; r < kC; ++r) acc = fmaf(sm.G[r * KP + i], sm.U[r * kVT + c], acc);
            sm.S[idx] = acc;
        }
    }
    if (sT) {
        for (int idx = tid; idx < K * kVT; idx += kNT) {
            const int i = idx / kVT, c = idx % kVT;
            sT[sbase + static_cast<size_t>(i) * V + j0 + c] = sm.S[idx];
        }
    }
}

// Output epilogue in place, one wave per (token, head) row of V values:
// o <- o / sqrt(mean o^2 + eps) (* weight), then o <- o * act(z).
template <int V, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void epilogue_kernel(PrefillArgs a) {
    constexpr int PER = V / 64;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
    if (row >= a.T * a.H) return;
    TOut *op = static_cast<TOut *>(a.o) + static_cast<size_t>(row) * V;
    float x[PER];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        x[e] = io<TOut>::load(op + e * 64 + l);
        ss += x[e] * x[e];
    }
    if (a.norm) {
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m);
        const float inv = rsqrtf(ss / V + a.eps);
#pragma unroll
        for (int e = 0; e < PER; ++e) x[e] *= inv * (a.nw ? a.nw[e * 64 + l] : 1.f);
    }
    if (a.z) {
        const TIn *zp = static_cast<const TIn *>(a.z) + static_cast<size_t>(row) * V;
#pragma unroll
        for (int e = 0; e < PER; ++e) x[e] *= out_gate_act(io<TIn>::load(zp + e * 64 + l), a.zact);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) io<TOut>::store(op + e * 64 + l, x[e]);
}

template <int V>
hipError_t launch_epi(const PrefillArgs &a, hipStream_t st) {
    const dim3 grid((static_cast<unsigned>(a.T) * a.H + 3) / 4), block(256);
    if (a.in_dtype == KDA_F32)
        hipLaunchKernelGGL((epilogue_kernel<V, float, float>), grid, block, 0, st, a);
    else if (a.out_dtype == KDA_BF16)
        hipLaunchKernelGGL((epilogue_kernel<V, bf16_t, bf16_t>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((epilogue_kernel<V, bf16_t, float>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int K, int V>
hipError_t launch_kv(const PrefillArgs &a, hipStream_t st) {
    const dim3 grid(a.N * a.H * (V / kVT)), block(kNT);
    if (a.in_dtype == KDA_F32)
        hipLaunchKernelGGL((prefill_valu_kernel<K, V, float, float>), grid, block, 0, st, a);
    else if (a.out_dtype == KDA_BF16)
        hipLaunchKernelGGL((prefill_valu_kernel<K, V, bf16_t, bf16_t>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((prefill_valu_kernel<K, V, bf16_t, float>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_epilogue(const PrefillArgs &a, hipStream_t st) {
    return a.V == 128 ? launch_epi<128>(a, st) : launch_epi<64>(a, st);
}

hipError_t launch_prefill_valu(const PrefillArgs &a, hipStream_t st) {
    if (a.K == 128 && a.V == 128) return launch_kv<128, 128>(a, st);
    if (a.K == 128 && a.V == 64) return launch_kv<128, 64>(a, st);
    if (a.K == 64 && a.V == 128) return launch_kv<64, 128>(a, st);
    return launch_kv<64, 64>(a, st);
}

}  // namespace kda
