// KDA chunk prefill, fp32 vector-ALU kernels (the fp32-input path).
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
// Every quantity is fp32. The pairwise decays are the products
// e^{G_r} e^{-G_s} (one exp per token and channel) while the chunk decays by
// less than e^80 in every channel, so neither factor leaves the normal fp32
// range; a chunk that decays further evaluates e^{G_r - G_s} element by element.
// Rows past the end of a partial chunk are zero-filled with g = 0 and
// beta = 0, which makes them contribute nothing.
//
// Two kernels:
//  * valu_prep_kernel, one 256-thread workgroup per (chunk, head), all in
//    parallel: everything that does not depend on the state (the cumulative
//    decay, A, P, T = (I + A)^{-1}, the decayed operands) into an fp32 record
//    in the workspace;
//  * valu_state_kernel, one 256-thread workgroup per (sequence, head, 16 value
//    columns), sequential over the chunks of the sequence: the state-dependent
//    products, with the chunk's record, the state slice and the pseudo-values
//    in LDS (about 149 KB at d_k = 128).
// Record slots: chunk c of sequence n has id floor(cu[n] / 64) + n + c. The ids
// increase with n and c and stay distinct (floor(a/64) + ceil(b/64) <=
// floor((a + b)/64) + 1), and they stay below ceil(T/64) + N; an empty
// sequence leaves one id unused.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;    // chunk length
constexpr int kVT = 16;   // value columns per workgroup of the state pass
constexpr int kNT = 256;  // threads per workgroup

// fp32 record of one (chunk, head), row-major, each part 256-B aligned
template <int K>
struct ValuRec {
    static constexpr size_t TB = 0;                    // [64][64] T Diag(beta), zero above the diagonal
    static constexpr size_t P = TB + kC * kC * 4;      // [64][64] P, zero above the diagonal
    static constexpr size_t KE = P + kC * kC * 4;      // [64][K] K . e^G
    static constexpr size_t QE = KE + kC * K * 4;      // [64][K] Q . e^G
    static constexpr size_t KG = QE + kC * K * 4;      // [64][K] K . e^{G_n - G}
    static constexpr size_t GAM = KG + kC * K * 4;     // [K] e^{G_n}
    static constexpr size_t BYTES = (GAM + K * 4 + 255) / 256 * 256;
};

// record slots per head: an upper bound of the chunk ids
inline size_t valu_slots(int32_t T, int32_t N) { return static_cast<size_t>((T + kC - 1) / kC) + N; }

__device__ __forceinline__ int valu_base(const int32_t *cu, int n) { return cu[n] / kC + n; }

// record id -> (sequence n, chunk c inside it); false for an unused id
__device__ __forceinline__ bool valu_item(const int32_t *cu, int N, int id, int &n, int &c) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (valu_base(cu, mid) <= id) lo = mid; else hi = mid - 1;
    }
    n = lo;
    c = id - valu_base(cu, lo);
    return c >= 0 && c < (cu[lo + 1] - cu[lo] + kC - 1) / kC;
}

template <int K>
struct PrepSm {
    static constexpr int KP = K + 1, CP = kC + 1;
    float G[kC * KP];   // cumulative log decay
    float KK[kC * KP];  // k
    float QQ[kC * KP];  // q
    float A[kC * CP];   // strict-lower A, then T = (I + A)^{-1} below the diagonal
    float P[kC * CP];
    float glast[K];
    float bet[kC];
};

template <int K, typename TIn>
__global__ __launch_bounds__(kNT) void valu_prep_kernel(PrefillArgs a, char *recs, int nslot) {
    constexpr int KP = K + 1, CP = kC + 1;
    using R = ValuRec<K>;
    __shared__ PrepSm<K> sm;
    const int tid = threadIdx.x;
    const int H = a.H, id = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    int n, c;
    if (!valu_item(a.cu_seqlens, a.N, id, n, c)) return;
    const int t0 = a.cu_seqlens[n] + c * kC, nt = min(kC, a.cu_seqlens[n + 1] - t0);
    const TIn *qg = static_cast<const TIn *>(a.q);
    const TIn *kg = static_cast<const TIn *>(a.k);
    const int Hk = a.Hk, hk = h / (H / Hk);  // key head of value head h
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
    }
    // G never increases along the chunk, so e^{-G} stays below e^80 everywhere when the
    // last row does: then e^{G_r - G_s} = e^{G_r} e^{-G_s} and A, P are plain products
    const bool exact = __syncthreads_or(tid < K && sm.glast[tid] < -80.f);
    if (!exact) {
        // in place: k -> K.e^G, q -> Q.e^G, G -> K.e^{-G}
        for (int idx = tid; idx < kC * K; idx += kNT) {
            const int r = idx / K, i = idx % K;
            const float G = sm.G[r * KP + i], e1 = __expf(G), e2 = __expf(-G);
            const float kv = sm.KK[r * KP + i];
            sm.KK[r * KP + i] = kv * e1;
            sm.QQ[r * KP + i] *= e1;
            sm.G[r * KP + i] = kv * e2;
        }
        __syncthreads();
        // A = Diag(beta) strict_lower((K.e^G)(K.e^{-G})^T), P = lower((Q.e^G)(K.e^{-G})^T):
        // thread tid owns the 4 x 4 tile of rows 4 (tid / 16) .., columns 4 (tid % 16) ..
        const int rb = 4 * (tid / 16), cb = 4 * (tid % 16);
        float aa[4][4] = {}, pp[4][4] = {};
        if (cb <= rb + 3) {
            for (int i = 0; i < K; ++i) {
                float kr[4], qr[4], kc[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    kr[m] = sm.KK[(rb + m) * KP + i];
                    qr[m] = sm.QQ[(rb + m) * KP + i];
                    kc[m] = sm.G[(cb + m) * KP + i];
                }
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int nn = 0; nn < 4; ++nn) {
                        aa[m][nn] = fmaf(kr[m], kc[nn], aa[m][nn]);
                        pp[m][nn] = fmaf(qr[m], kc[nn], pp[m][nn]);
                    }
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int nn = 0; nn < 4; ++nn) {
                const int r = rb + m, s2 = cb + nn;
                sm.A[r * CP + s2] = s2 < r ? sm.bet[r] * aa[m][nn] : 0.f;
                sm.P[r * CP + s2] = s2 <= r ? pp[m][nn] : 0.f;
            }
    } else {
        // a channel decays by more than e^80 over the chunk: e^{G_r - G_s} per element,
        // A and P on and below the diagonal, one (r, s) pair each: p = r (r + 1) / 2 + s
        // (the entries above the diagonal are never read; the record gets zeros there)
        for (int p = tid; p < kC * (kC + 1) / 2; p += kNT) {
            int r = static_cast<int>((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
            if ((r + 1) * (r + 2) / 2 <= p) ++r;  // float rounding, either way
            if (r * (r + 1) / 2 > p) --r;
            const int s2 = p - r * (r + 1) / 2;
            float aa = 0.f, pp = 0.f;
            for (int i = 0; i < K; ++i) {
                const float ks = sm.KK[s2 * KP + i] * __expf(sm.G[r * KP + i] - sm.G[s2 * KP + i]);
                aa = fmaf(sm.KK[r * KP + i], ks, aa);
                pp = fmaf(sm.QQ[r * KP + i], ks, pp);
            }
            sm.A[r * CP + s2] = s2 < r ? sm.bet[r] * aa : 0.f;
            sm.P[r * CP + s2] = pp;
        }
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
    char *rec = recs + (static_cast<size_t>(h) * nslot + id) * R::BYTES;
    float *tb = reinterpret_cast<float *>(rec + R::TB), *pm = reinterpret_cast<float *>(rec + R::P);
    for (int p = tid; p < kC * kC; p += kNT) {
        const int r = p / kC, s = p % kC;
        const float t = s < r ? sm.A[r * CP + s] : (s == r ? 1.f : 0.f);
        tb[p] = t * sm.bet[s];
        pm[p] = s <= r ? sm.P[r * CP + s] : 0.f;
    }
    float *ke = reinterpret_cast<float *>(rec + R::KE), *qe = reinterpret_cast<float *>(rec + R::QE);
    float *kgn = reinterpret_cast<float *>(rec + R::KG);
    for (int idx = tid; idx < kC * K; idx += kNT) {
        const int r = idx / K, i = idx % K;
        if (!exact) {  // the LDS holds K.e^G, Q.e^G and K.e^{-G}
            ke[idx] = sm.KK[r * KP + i];
            qe[idx] = sm.QQ[r * KP + i];
            kgn[idx] = sm.G[r * KP + i] * __expf(sm.glast[i]);
        } else {
            const float G = sm.G[r * KP + i];
            const float e1 = __expf(G), e2 = __expf(sm.glast[i] - G);
            const float kv = sm.KK[r * KP + i];
            ke[idx] = kv * e1;
            qe[idx] = sm.QQ[r * KP + i] * e1;
            kgn[idx] = kv * e2;
        }
    }
    if (tid < K) reinterpret_cast<float *>(rec + R::GAM)[tid] = __expf(sm.glast[tid]);
}

template <int K>
struct StateSm {
    static constexpr int KP = K + 1, CP = kC + 1;
    float KE[kC * KP];  // K . e^G
    float QE[kC * KP];  // Q . e^G
    float KG[kC * KP];  // K . e^{G_n - G}
    float TB[kC * CP];  // T Diag(beta)
    float P[kC * CP];
    float S[K * kVT];
    float X[kC * kVT];  // v, then V - (K.e^G) S
    float U[kC * kVT];  // U'
    float gam[K];
};

template <int K, int V, typename TIn, typename TOut>
__global__ __launch_bounds__(kNT) void valu_state_kernel(PrefillArgs a, const char *recs, int nslot) {
    constexpr int KP = K + 1, CP = kC + 1;
    constexpr int NVT = V / kVT;
    using R = ValuRec<K>;
    __shared__ StateSm<K> sm;
    const int tid = threadIdx.x;
    int bid = blockIdx.x;
    const int vt = bid % NVT;
    bid /= NVT;
    const int h = bid % a.H, n = bid / a.H;
    const int j0 = vt * kVT;
    const int H = a.H;
    const int tbeg = a.cu_seqlens[n], tend = a.cu_seqlens[n + 1];
    const TIn *vg = static_cast<const TIn *>(a.v);
    TOut *og = static_cast<TOut *>(a.o);
    // states: [N, H, K, V], or with slots a cache [slots, H, K, V] read and written at slot[n]
    // (a negative slot: zero initial state, final state not written)
    const int slot = a.slots ? a.slots[n] : n;
    const size_t sbase = (static_cast<size_t>(slot) * H + h) * static_cast<size_t>(K) * V;
    const float *s0 = slot >= 0 ? a.s0 : nullptr;
    float *sT = slot >= 0 ? a.sT : nullptr;
    const char *hrec = recs + static_cast<size_t>(h) * nslot * R::BYTES;
    const int base = valu_base(a.cu_seqlens, n);

    for (int idx = tid; idx < K * kVT; idx += kNT) {
        const int i = idx / kVT, c = idx % kVT;
        sm.S[idx] = s0 ? s0[sbase + static_cast<size_t>(i) * V + j0 + c] : 0.f;
    }

    for (int t0 = tbeg, c = 0; t0 < tend; t0 += kC, ++c) {
        const int nt = min(kC, tend - t0);
        const char *rec = hrec + static_cast<size_t>(base + c) * R::BYTES;
        __syncthreads();
        {
            // 16-byte loads; the LDS rows are padded by one word, so the stores are single words
            const float4 *tb = reinterpret_cast<const float4 *>(rec + R::TB);
            const float4 *pm = reinterpret_cast<const float4 *>(rec + R::P);
            for (int p = tid; p < kC * kC / 4; p += kNT) {
                const int r = (4 * p) / kC, s = (4 * p) % kC;
                const float4 x = tb[p], y = pm[p];
                float *dt = &sm.TB[r * CP + s], *dp = &sm.P[r * CP + s];
                dt[0] = x.x; dt[1] = x.y; dt[2] = x.z; dt[3] = x.w;
                dp[0] = y.x; dp[1] = y.y; dp[2] = y.z; dp[3] = y.w;
            }
            const float4 *ke = reinterpret_cast<const float4 *>(rec + R::KE);
            const float4 *qe = reinterpret_cast<const float4 *>(rec + R::QE);
            const float4 *kgn = reinterpret_cast<const float4 *>(rec + R::KG);
            for (int p = tid; p < kC * K / 4; p += kNT) {
                const int r = (4 * p) / K, i = (4 * p) % K;
                const float4 x = ke[p], y = qe[p], z = kgn[p];
                float *d0 = &sm.KE[r * KP + i], *d1 = &sm.QE[r * KP + i], *d2 = &sm.KG[r * KP + i];
                d0[0] = x.x; d0[1] = x.y; d0[2] = x.z; d0[3] = x.w;
                d1[0] = y.x; d1[1] = y.y; d1[2] = y.z; d1[3] = y.w;
                d2[0] = z.x; d2[1] = z.y; d2[2] = z.z; d2[3] = z.w;
            }
            if (tid < K) sm.gam[tid] = reinterpret_cast<const float *>(rec + R::GAM)[tid];
        }
        for (int idx = tid; idx < kC * kVT; idx += kNT) {
            const int r = idx / kVT, cc = idx % kVT;
            sm.X[idx] = r < nt ? io<TIn>::load(vg + (static_cast<size_t>(t0 + r) * H + h) * V + j0 + cc) : 0.f;
        }
        __syncthreads();
        // Thread tid owns column cc = tid % 16 and the rows r0 + 16 m (m < NR) of the
        // 64 x 16 products, so that one state (or U') value serves NR rows.
        constexpr int NR = kC * kVT / kNT, NS = K * kVT / kNT;
        static_assert(NR * kNT == kC * kVT && NS * kNT == K * kVT, "whole tiles per thread");
        const int cc = tid % kVT, r0 = tid / kVT;
        {  // X = V - (K.e^G) S
            float acc[NR] = {};
            for (int i = 0; i < K; ++i) {
                const float sv = sm.S[i * kVT + cc];
#pragma unroll
                for (int m = 0; m < NR; ++m) acc[m] = fmaf(sm.KE[(r0 + 16 * m) * KP + i], sv, acc[m]);
            }
#pragma unroll
            for (int m = 0; m < NR; ++m) sm.X[(r0 + 16 * m) * kVT + cc] -= acc[m];
        }
        __syncthreads();
        for (int idx = tid; idx < kC * kVT; idx += kNT) {  // U' = T Diag(beta) X
            const int r = idx / kVT, cc = idx % kVT;
            float acc = 0.f;
            for (int s = 0; s <= r; ++s) acc = fmaf(sm.TB[r * CP + s], sm.X[s * kVT + cc], acc);
            sm.U[idx] = acc;
        }
        __syncthreads();
        {  // O = (Q.e^G) S + P U' (P is zero above the diagonal)
            float acc[NR] = {};
            for (int i = 0; i < K; ++i) {
                const float sv = sm.S[i * kVT + cc];
#pragma unroll
                for (int m = 0; m < NR; ++m) acc[m] = fmaf(sm.QE[(r0 + 16 * m) * KP + i], sv, acc[m]);
            }
            for (int s2 = 0; s2 < kC; ++s2) {
                const float uv = sm.U[s2 * kVT + cc];
#pragma unroll
                for (int m = 0; m < NR; ++m) acc[m] = fmaf(sm.P[(r0 + 16 * m) * CP + s2], uv, acc[m]);
            }
#pragma unroll
            for (int m = 0; m < NR; ++m) {
                const int r = r0 + 16 * m;
                if (r < nt) io<TOut>::store(og + (static_cast<size_t>(t0 + r) * H + h) * V + j0 + cc, a.scale * acc[m]);
            }
        }
        __syncthreads();
        {  // S <- e^{G_n} S + (K.e^{G_n-G})^T U'; thread tid owns rows r0 + 16 m of S
            float acc[NS];
#pragma unroll
            for (int m = 0; m < NS; ++m) acc[m] = sm.gam[r0 + 16 * m] * sm.S[(r0 + 16 * m) * kVT + cc];
            for (int r = 0; r < kC; ++r) {
                const float uv = sm.U[r * kVT + cc];
#pragma unroll
                for (int m = 0; m < NS; ++m) acc[m] = fmaf(sm.KG[r * KP + r0 + 16 * m], uv, acc[m]);
            }
#pragma unroll
            for (int m = 0; m < NS; ++m) sm.S[(r0 + 16 * m) * kVT + cc] = acc[m];
        }
    }
    __syncthreads();
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
    const int nslot = static_cast<int>(valu_slots(a.T, a.N));
    char *recs = static_cast<char *>(a.ws);
    if (a.T > 0) {
        const dim3 pg(static_cast<unsigned>(nslot) * a.H), pb(kNT);
        if (a.in_dtype == KDA_F32) hipLaunchKernelGGL((valu_prep_kernel<K, float>), pg, pb, 0, st, a, recs, nslot);
        else hipLaunchKernelGGL((valu_prep_kernel<K, bf16_t>), pg, pb, 0, st, a, recs, nslot);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 grid(static_cast<unsigned>(a.N) * a.H * (V / kVT)), block(kNT);
    if (a.in_dtype == KDA_F32)
        hipLaunchKernelGGL((valu_state_kernel<K, V, float, float>), grid, block, 0, st, a, recs, nslot);
    else if (a.out_dtype == KDA_BF16)
        hipLaunchKernelGGL((valu_state_kernel<K, V, bf16_t, bf16_t>), grid, block, 0, st, a, recs, nslot);
    else
        hipLaunchKernelGGL((valu_state_kernel<K, V, bf16_t, float>), grid, block, 0, st, a, recs, nslot);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_epilogue(const PrefillArgs &a, hipStream_t st) {
    return a.V == 128 ? launch_epi<128>(a, st) : launch_epi<64>(a, st);
}

size_t prefill_valu_workspace(int32_t N, int32_t T, int32_t H, int32_t K) {
    if (T <= 0) return 0;
    const size_t rb = K == 128 ? ValuRec<128>::BYTES : ValuRec<64>::BYTES;
    return valu_slots(T, N) * static_cast<size_t>(H) * rb;
}

hipError_t launch_prefill_valu(const PrefillArgs &a, hipStream_t st) {
    if (a.K == 128 && a.V == 128) return launch_kv<128, 128>(a, st);
    if (a.K == 128 && a.V == 64) return launch_kv<128, 64>(a, st);
    if (a.K == 64 && a.V == 128) return launch_kv<64, 128>(a, st);
    return launch_kv<64, 64>(a, st);
}

}  // namespace kda
