// KDA chunk prefill on the gfx950 matrix cores (bf16 inputs).
//
// The chunkwise form ("Kimi Linear爆发背后的秘密" page, section "硬件效率的深度优化":
// parallel inside a chunk, recurrent across chunks, WY representation, UT
// transform, second-level chunking needing only two pairwise matrices; 64-token
// chunks and log-space cumulative decay from "线性注意力机制Kimi Linear架构解析与优化实践",
// sections 2.2 and 4.2). For a chunk of n <= 64 tokens, incoming state S,
// G_r = sum_{s<=r} g_s per key channel:
//   A  = strict_lower(Diag(beta) [sum_i k_r[i] k_s[i] e^{G_r[i]-G_s[i]}])
//   P  = lower_incl([sum_i q_r[i] k_s[i] e^{G_r[i]-G_s[i]}])
//   T  = (I + A)^{-1}
//   U' = T Diag(beta) (V - (K . e^G) S)
//   O  = scale ((Q . e^G) S + P U')
//   S <- Diag(e^{G_n}) S + (K . e^{G_n-G})^T U'
//
// Two kernels.
//  * prep (one workgroup per chunk and head, all chunks in parallel): every
//    quantity that does not depend on the state. The 64x64 pairwise matrices
//    are built from 16-token sub-chunks: for a row in sub-chunk i and a column
//    in sub-chunk j <= i, e^{G_r-G_s} = e^{G_r-G_b} e^{G_b-G_s} with b the last
//    token before sub-chunk i, so every factor is <= 1 except, on the diagonal
//    sub-chunk, e^{G_b-G_s} <= e^{(decay over 16 tokens)}. Those products run
//    as fp16 16x16x32 MFMAs with fp32 accumulation. Sub-chunks whose decay in
//    some channel exceeds e^10 over 16 tokens take an exact fp32 per-element
//    path for their diagonal block instead. T is inverted in fp32 (forward
//    substitution on the 16x16 diagonal blocks, block recurrence below them).
//    Results are written to the workspace as fp16 MFMA operand fragments in
//    exactly the register layout the scan kernel consumes.
//  * scan (one workgroup per sequence, head and 16 value columns): the
//    sequential pass over chunks. The state slice lives in MFMA accumulators
//    (fp32); every value-side operand (state, V - K S, U') is scaled per value
//    column by a power of two before its fp16 conversion, so the fp16 range
//    never limits the magnitude of v or of the state. One workgroup barrier per
//    chunk.
//
// MFMA fragment conventions (v_mfma_f32_16x16x32_f16, lane l, r = l % 16,
// g = l / 16): A operand holds A[r][k(g, e)], B operand B[k(g, e)][r], result
// D[4g + e'][r], e = 0..7, e' = 0..3. Along every contraction index this file
// uses k(g, e) = 4g + e for e < 4 and 16 + 4g + (e - 4) for e >= 4, which is
// exactly the set of rows a lane holds of two stacked 16x16 results, so a
// product's result feeds the next product's B operand from registers.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;
constexpr float kFastRange = 10.f;  // max decay exponent of one sub-chunk on the fp16 path

__device__ __forceinline__ f4 mfma(half8 a, half8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ int kidx(int g, int e) { return e < 4 ? 4 * g + e : 12 + 4 * g + e; }

template <int SH>
__device__ __forceinline__ float dpp_row_shr(float v) {
    // lanes whose source lies outside their 16-lane row read 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + SH, 0xF, 0xF, false));
}

// Power-of-two scale for a column whose largest magnitude is m: returns s and
// sets inv = 1/s such that m * inv lies in [2^14, 2^15).
__device__ __forceinline__ float col_scale(float m, float &inv) {
    int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xFFu) - 127;
    e = max(-100, min(e, 110));
    inv = __uint_as_float(static_cast<uint32_t>(127 + 14 - e) << 23);
    return __uint_as_float(static_cast<uint32_t>(127 - 14 + e) << 23);
}

// max over the four lanes l, l^16, l^32, l^48 (one column of an MFMA result):
// a lane swap of a register with itself pairs every lane with its partner
__device__ __forceinline__ float col_max(float m) {
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// Per (chunk, head) record in the workspace; every fragment is 64 lanes x 16 B.
template <int K>
struct Rec {
    static constexpr int NCB = K / 32, NCT = K / 16;
    static constexpr size_t FRAG = 1024;
    static constexpr size_t KEXP = 0;                        // [i 4][cb NCB]  (K.e^G)
    static constexpr size_t QG = KEXP + 4 * NCB * FRAG;      // [i 4][cb NCB]  (Q.e^G)
    static constexpr size_t KGT = QG + 4 * NCB * FRAG;       // [ct NCT][ks 2] (K.e^{G_n-G})^T
    static constexpr size_t TM = KGT + 2 * NCT * FRAG;       // 6 lower blocks of T
    static constexpr size_t PM = TM + 6 * FRAG;              // 6 lower blocks of P
    static constexpr size_t GAM = PM + 6 * FRAG;             // e^{G_n} [K] fp32
    static constexpr size_t BET = GAM + 4 * K;               // beta [64] fp32
    static constexpr size_t BYTES = (BET + 4 * kC + 255) / 256 * 256;
};
// (row block i, 32-wide k step ks) -> fragment index for the lower-triangular T and P
__device__ __forceinline__ int tri(int i, int ks) { return i < 2 ? i : 2 * i - 2 + ks; }
// (row block i, column block j <= i) -> B-operand variant of column block j
__device__ __forceinline__ int vblk(int i, int j) { return (j == 0 ? 0 : j == 1 ? 4 : j == 2 ? 7 : 9) + i - j; }

constexpr size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// chunk capacity: an upper bound of sum_n ceil(len_n / 64); records are stored
// head-major, record (chunk c, head h) at index h * capacity + c, so one head's
// consecutive chunks are adjacent in memory
__host__ __device__ __forceinline__ size_t a_nc(const PrefillArgs &a) {
    return static_cast<size_t>((a.T + kC - 1) / kC) + a.N;
}

// ---------------------------------------------------------------------------
// chunk offsets: off[n] = sum_{m<n} ceil(len_m / 64), off[N] = total chunks
__global__ __launch_bounds__(256) void chunk_offsets_kernel(const int32_t *cu, int32_t N,
                                                             int32_t *off) {
    __shared__ int32_t buf[256];
    __shared__ int32_t carry;
    const int t = threadIdx.x;
    if (t == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + t;
        int nc = 0;
        if (n < N) nc = (max(cu[n + 1] - cu[n], 0) + kC - 1) / kC;
        buf[t] = nc;
        __syncthreads();
        for (int s = 1; s < 256; s <<= 1) {
            const int x = t >= s ? buf[t - s] : 0;
            __syncthreads();
            buf[t] += x;
            __syncthreads();
        }
        if (n < N) off[n] = carry + buf[t] - nc;
        __syncthreads();
        if (t == 255) carry += buf[255];
        __syncthreads();
    }
    if (t == 0) off[N] = carry;
}

// ---------------------------------------------------------------------------
// prep: state-independent work of one chunk of one head
template <int K>
struct PrepSmem {
    static constexpr int NCB = K / 32, LD = 65;
    float tot[4][K];       // decay of each sub-chunk per channel (log, <= 0)
    float fac[K][16];      // per-channel factors, see prep_kernel
    float beta[kC];
    union {
        struct {
            half8 colv[10][NCB][64];  // B operands of the pairwise products
            _Float16 kgT[K][kC + 8];  // (K.e^{G_n-G}) transposed [channel][token]
        } a;
        struct {
            float A[kC][LD];
            float P[kC][LD];
            float T[kC][LD];
            float X[4][16][17];
        } b;
    } u;
};

template <int K>
__global__ __launch_bounds__(256) void prep_kernel(PrefillArgs a, const int32_t *off, char *recs) {
    constexpr int NCB = K / 32, NCT = K / 16;
    using R = Rec<K>;
    __shared__ PrepSmem<K> sm;
    const int H = a.H;
    const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (c >= off[a.N]) return;
    int lo = 0, hi = a.N - 1;  // sequence n with off[n] <= c < off[n + 1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const int n = lo;
    const int t0 = a.cu_seqlens[n] + (c - off[n]) * kC;
    const int nt = min(kC, a.cu_seqlens[n + 1] - t0);
    char *rec = recs + (static_cast<size_t>(h) * a_nc(a) + c) * R::BYTES;

    const int tid = threadIdx.x, l = tid & 63, r = l & 15, g = l >> 4;
    // wave index as a scalar: branches on it must be real jumps, because a
    // matrix instruction inside an EXEC-masked block still writes its result
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tr = 16 * w + r;  // token of this lane inside the chunk
    const bool valid = tr < nt;
    const size_t row = (static_cast<size_t>(t0 + (valid ? tr : 0)) * H + h) * K;
    const bf16_t *qp = static_cast<const bf16_t *>(a.q) + row;
    const bf16_t *kp = static_cast<const bf16_t *>(a.k) + row;
    const float *gp = a.g + row;

    // ---- load this lane's 8 channels per 32-channel block, scan the log decay over the sub-chunk
    float kx[NCB][8], qx[NCB][8], s[NCB][8];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int ch = 32 * cb + 16 * hf + 4 * g;
            float4 gv = make_float4(0.f, 0.f, 0.f, 0.f), kv = gv, qv = gv;
            if (valid) {
                gv = *reinterpret_cast<const float4 *>(gp + ch);
                kv = io<bf16_t>::load4(kp + ch);
                qv = io<bf16_t>::load4(qp + ch);
            }
            s[cb][4 * hf + 0] = gv.x; s[cb][4 * hf + 1] = gv.y;
            s[cb][4 * hf + 2] = gv.z; s[cb][4 * hf + 3] = gv.w;
            kx[cb][4 * hf + 0] = kv.x; kx[cb][4 * hf + 1] = kv.y;
            kx[cb][4 * hf + 2] = kv.z; kx[cb][4 * hf + 3] = kv.w;
            qx[cb][4 * hf + 0] = qv.x; qx[cb][4 * hf + 1] = qv.y;
            qx[cb][4 * hf + 2] = qv.z; qx[cb][4 * hf + 3] = qv.w;
        }
    }
    if (g == 0) sm.beta[tr] = valid ? a.beta[static_cast<size_t>(t0 + tr) * H + h] : 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = s[cb][e];
            v += dpp_row_shr<1>(v);
            v += dpp_row_shr<2>(v);
            v += dpp_row_shr<4>(v);
            v += dpp_row_shr<8>(v);
            s[cb][e] = v;  // G_r - G_b: log decay from the sub-chunk start to token r (inclusive)
        }
    if (r == 15) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.tot[w][32 * cb + kidx(g, e)] = s[cb][e];
    }
    __syncthreads();

    // ---- per-channel factors: 0..3 e^{G_{b_w}} (decay before sub-chunk w), 4..7 decay after
    // sub-chunk w to the chunk end, 8..11 inverse decay of sub-chunk w (clamped; fast path
    // only), 12 e^{tot1}, 13 e^{tot1+tot2}, 14 e^{tot2} (between sub-chunks), 15 e^{G_n}
    int bad = 0;
    if (tid < K) {
        const float d0 = sm.tot[0][tid], d1 = sm.tot[1][tid], d2 = sm.tot[2][tid], d3 = sm.tot[3][tid];
        float *f = sm.fac[tid];
        f[0] = 1.f; f[1] = __expf(d0); f[2] = __expf(d0 + d1); f[3] = __expf(d0 + d1 + d2);
        f[4] = __expf(d1 + d2 + d3); f[5] = __expf(d2 + d3); f[6] = __expf(d3); f[7] = 1.f;
        f[8] = __expf(fminf(-d0, 80.f)); f[9] = __expf(fminf(-d1, 80.f));
        f[10] = __expf(fminf(-d2, 80.f)); f[11] = __expf(fminf(-d3, 80.f));
        f[12] = __expf(d1); f[13] = __expf(d1 + d2); f[14] = __expf(d2);
        f[15] = __expf(d0 + d1 + d2 + d3);
        bad = fmaxf(fmaxf(-d0, -d1), fmaxf(-d2, -d3)) > kFastRange;
    }
    const bool slow = __syncthreads_or(bad);

    // ---- elementwise: decayed operands
    half8 kr[NCB], qr[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        half8 kexp, qg, cv0, cv1, cv2, cv3;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = 32 * cb + kidx(g, e);
            const float *f = sm.fac[ch];
            const float rho = __expf(s[cb][e]);                  // e^{G_r - G_b} <= 1
            const float tau = __expf(sm.tot[w][ch] - s[cb][e]);  // e^{G_{b'} - G_r} <= 1, b' = sub-chunk end
            const float krv = kx[cb][e] * rho, qrv = qx[cb][e] * rho;
            kr[cb][e] = static_cast<_Float16>(krv);
            qr[cb][e] = static_cast<_Float16>(qrv);
            kexp[e] = static_cast<_Float16>(krv * f[w]);
            qg[e] = static_cast<_Float16>(qrv * f[w]);
            const float kt = kx[cb][e] * tau;
            sm.u.a.kgT[ch][tr] = static_cast<_Float16>(kt * f[4 + w]);
            // column operands of column block w for row blocks i = w..3: k_s e^{G_{b_i} - G_s}
            cv0[e] = static_cast<_Float16>(slow ? 0.f : kt * f[8 + w]);  // i = w (>= 1)
            cv1[e] = static_cast<_Float16>(kt);                           // i = w + 1
            cv2[e] = static_cast<_Float16>(kt * (w == 0 ? f[12] : f[14]));  // i = w + 2
            cv3[e] = static_cast<_Float16>(kt * f[13]);                   // i = 3 (w = 0)
        }
        *reinterpret_cast<half8 *>(rec + R::KEXP + ((w * NCB + cb) * 64 + l) * 16) = kexp;
        *reinterpret_cast<half8 *>(rec + R::QG + ((w * NCB + cb) * 64 + l) * 16) = qg;
        sm.u.a.colv[vblk(w, w)][cb][l] = cv0;
        if (w + 1 < 4) sm.u.a.colv[vblk(w + 1, w)][cb][l] = cv1;
        if (w + 2 < 4) sm.u.a.colv[vblk(w + 2, w)][cb][l] = cv2;
        if (w == 0) sm.u.a.colv[vblk(3, 0)][cb][l] = cv3;
    }
    __syncthreads();

    // ---- (K.e^{G_n-G})^T fragments: [channel tile ct][token step ks]
    for (int f = w; f < 2 * NCT; f += 4) {
        const int ct = f >> 1, ks = f & 1;
        half8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = sm.u.a.kgT[16 * ct + r][32 * ks + kidx(g, e)];
        *reinterpret_cast<half8 *>(rec + R::KGT + (f * 64 + l) * 16) = v;
    }

    // ---- pairwise products for row block w: A_wj, P_wj, j <= w
    f4 accA[4], accP[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        accA[j] = zero4();
        accP[j] = zero4();
        if (j <= w) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const half8 b = sm.u.a.colv[vblk(w, j)][cb][l];
                accA[j] = mfma(kr[cb], b, accA[j]);
                accP[j] = mfma(qr[cb], b, accP[j]);
            }
        }
    }
    __syncthreads();  // colv / kgT no longer read; the union now holds A, P, T

#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rl = 4 * g + e, rowi = 16 * w + rl, col = 16 * j + r;
            float av = 0.f, pv = 0.f;
            if (j < w) { av = accA[j][e]; pv = accP[j][e]; }
            if (j == w) { av = r < rl ? accA[j][e] : 0.f; pv = r <= rl ? accP[j][e] : 0.f; }
            sm.u.b.A[rowi][col] = av * sm.beta[rowi];
            sm.u.b.P[rowi][col] = pv;
            sm.u.b.T[rowi][col] = 0.f;
        }
    if (slow) {
        // exact diagonal block: e^{G_r - G_s} per element, s <= r inside sub-chunk w
        for (int ss = 0; ss < 16; ++ss) {
            float pa = 0.f, pp = 0.f;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float s_s = __shfl(s[cb][e], ss + 16 * g);
                    const float k_s = __shfl(kx[cb][e], ss + 16 * g);
                    const float t = ss <= r ? k_s * __expf(fminf(s[cb][e] - s_s, 0.f)) : 0.f;
                    pa = fmaf(kx[cb][e], t, pa);
                    pp = fmaf(qx[cb][e], t, pp);
                }
            pa += __shfl_xor(pa, 16); pa += __shfl_xor(pa, 32);
            pp += __shfl_xor(pp, 16); pp += __shfl_xor(pp, 32);
            if (g == 0) {
                sm.u.b.A[16 * w + r][16 * w + ss] = ss < r ? pa * sm.beta[16 * w + r] : 0.f;
                sm.u.b.P[16 * w + r][16 * w + ss] = ss <= r ? pp : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by forward substitution (lane r = column)
    {
        float t[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc = rr == r ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < rr; ++m) acc = fmaf(-sm.u.b.A[16 * w + rr][16 * w + m], t[m], acc);
            t[rr] = acc;
        }
        if (g == 0) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) sm.u.b.T[16 * w + rr][16 * w + r] = t[rr];
        }
    }
    __syncthreads();
    // blocks below the diagonal: T_wj = -T_ww sum_{m=j}^{w-1} A_wm T_mj, by distance w - j
    for (int lev = 1; lev <= 3; ++lev) {
        const int j = w - lev;
        if (j >= 0) {
            float x[4] = {0.f, 0.f, 0.f, 0.f};
            for (int m = j; m < w; ++m)
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    const float tv = sm.u.b.T[16 * m + kk][16 * j + r];
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = fmaf(sm.u.b.A[16 * w + 4 * g + e][16 * m + kk], tv, x[e]);
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.u.b.X[w][4 * g + e][r] = x[e];
        }
        __syncthreads();
        if (j >= 0) {
            float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const float xv = sm.u.b.X[w][kk][r];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = fmaf(-sm.u.b.T[16 * w + 4 * g + e][16 * w + kk], xv, y[e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.u.b.T[16 * w + 4 * g + e][16 * j + r] = y[e];
        }
        __syncthreads();
    }

    // ---- T and P fragments of row block w (A operands, contraction over tokens)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        if (ks <= (w >> 1)) {
            half8 tf, pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = 32 * ks + kidx(g, e);
                tf[e] = static_cast<_Float16>(sm.u.b.T[16 * w + r][col]);
                pf[e] = static_cast<_Float16>(sm.u.b.P[16 * w + r][col]);
            }
            *reinterpret_cast<half8 *>(rec + R::TM + (tri(w, ks) * 64 + l) * 16) = tf;
            *reinterpret_cast<half8 *>(rec + R::PM + (tri(w, ks) * 64 + l) * 16) = pf;
        }
    }
    if (tid < K) reinterpret_cast<float *>(rec + R::GAM)[tid] = sm.fac[tid][15];
    if (tid < kC) reinterpret_cast<float *>(rec + R::BET)[tid] = sm.beta[tid];
}

// ---------------------------------------------------------------------------
// scan: sequential pass over the chunks of one (sequence, head, 16 value columns)
template <int K>
struct Frags {
    float4 v;              // this thread's 4 columns of one token of V        (staged to LDS)
    float aux;             // beta (threads 0..63) or e^{G_n} (threads 64..191) (staged to LDS)
    half8 t[2];            // T fragments w and w + 4 (w + 4 exists for w < 2)  (staged to LDS)
    half8 kexp[4], qg[4];  // this wave's channel block, all four token row blocks
    half8 kgt[2][2];       // this wave's two channel tiles x two token steps
    half8 p[2];            // this wave's output row block
};

// Operand loads of chunk c (clamped to the last chunk, so they are unconditional),
// in four parts that the chunk loop spreads over the previous chunk's work: one
// burst of all of them saturates the CU's vector memory pipeline.
template <int K, int V>
struct FragLoader {
    const char *rec;
    const bf16_t *vrow;
    bool vok;

    __device__ __forceinline__ FragLoader(const char *recs, size_t nc, int c, int clast, int H, int h,
                                          const bf16_t *vg, int tbeg, int tend, int cbeg, int j0, int tid) {
        c = min(c, clast);
        rec = recs + (static_cast<size_t>(h) * nc + c) * Rec<K>::BYTES;
        const int tok = tbeg + (c - cbeg) * kC + (tid >> 2);
        vok = tok < tend;
        vrow = vg + (static_cast<size_t>(min(tok, tend - 1)) * H + h) * V + j0 + (tid & 3) * 4;
    }
    __device__ __forceinline__ void part0(Frags<K> &f, int tid, int w, int l) const {
        using R = Rec<K>;
        const float4 vv = io<bf16_t>::load4(vrow);
        f.v = vok ? vv : make_float4(0.f, 0.f, 0.f, 0.f);
        if (tid < 64) f.aux = reinterpret_cast<const float *>(rec + R::BET)[tid];
        else if (tid < 64 + K) f.aux = reinterpret_cast<const float *>(rec + R::GAM)[tid - 64];
        f.t[0] = *reinterpret_cast<const half8 *>(rec + R::TM + (w * 64 + l) * 16);
        if (w < 2) f.t[1] = *reinterpret_cast<const half8 *>(rec + R::TM + ((w + 4) * 64 + l) * 16);
    }
    __device__ __forceinline__ void part1(Frags<K> &f, int w, int l) const {
        using R = Rec<K>;
        constexpr int NCB = K / 32;
        if (w < NCB) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                f.kexp[i] = *reinterpret_cast<const half8 *>(rec + R::KEXP + ((i * NCB + w) * 64 + l) * 16);
        }
    }
    __device__ __forceinline__ void part2(Frags<K> &f, int w, int l) const {
        using R = Rec<K>;
        constexpr int NCB = K / 32;
        if (w < NCB) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                f.qg[i] = *reinterpret_cast<const half8 *>(rec + R::QG + ((i * NCB + w) * 64 + l) * 16);
        }
    }
    __device__ __forceinline__ void part3(Frags<K> &f, int w, int l) const {
        using R = Rec<K>;
        constexpr int NCB = K / 32;
        if (w < NCB) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    f.kgt[tt][ks] = *reinterpret_cast<const half8 *>(rec + R::KGT + (((2 * w + tt) * 2 + ks) * 64 + l) * 16);
        }
        f.p[0] = *reinterpret_cast<const half8 *>(rec + R::PM + (tri(w, 0) * 64 + l) * 16);
        if (w >= 2) f.p[1] = *reinterpret_cast<const half8 *>(rec + R::PM + (tri(w, 1) * 64 + l) * 16);
    }
};

template <int K, int V, typename TOut>
struct ScanSmem {
    static constexpr int NCB = K / 32;
    f4 partX[2][NCB][4][64];  // (K.e^G) S_w / sig_w per wave w (channel block)
    f4 partO[2][NCB][4][64];  // (Q.e^G) S_w / sig_w
    float sig[2][NCB][64];    // sig_w of the lane's column
    float vT[2][16][kC + 4];
    float bet[2][kC];
    float gam[2][K];
    half8 t[2][6][64];        // T fragments of the current / next chunk
};

// Stage the chunk data that every wave needs (V transposed, beta, e^{G_n}, T) into LDS buffer b.
template <int K, int V, typename TOut>
__device__ __forceinline__ void stage(ScanSmem<K, V, TOut> &sm, int b, const Frags<K> &f, int tid) {
    const int stok = tid >> 2, sc4 = (tid & 3) * 4;
    sm.vT[b][sc4 + 0][stok] = f.v.x;
    sm.vT[b][sc4 + 1][stok] = f.v.y;
    sm.vT[b][sc4 + 2][stok] = f.v.z;
    sm.vT[b][sc4 + 3][stok] = f.v.w;
    if (tid < 64) sm.bet[b][tid] = f.aux;
    else if (tid < 64 + K) sm.gam[b][tid - 64] = f.aux;
    const int w = tid >> 6, l = tid & 63;
    sm.t[b][w][l] = f.t[0];
    if (w < 2) sm.t[b][w + 4][l] = f.t[1];
}

#define KDA_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// One chunk of the state pass. `f` holds chunk c's operands (V, beta, e^{G_n}
// and T already staged in LDS buffer `buf`); the loads of the next chunk into
// `fn` are issued in parts between the phases. Returns the output rows
// 16w + 4g + e of column j0 + r in `out`.
template <int K, int V, typename TOut>
__device__ __forceinline__ void scan_chunk(ScanSmem<K, V, TOut> &sm, const Frags<K> &f, Frags<K> &fn,
                                           const FragLoader<K, V> &ld, f4 (&S)[2], int buf, float scale,
                                           int tid, int w, int l, int r, int g, f4 &out) {
    constexpr int NCB = K / 32;
    const bool hasS = w < NCB;
    ld.part0(fn, tid, w, l);
    KDA_SCHED_FENCE();
    // (a) partial products with this wave's channel block of the state
    if (hasS) {
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(S[0][e]), fabsf(S[1][e])));
        float inv;
        const float sig = col_scale(col_max(m), inv);
        half8 sf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sf[e] = static_cast<_Float16>(S[0][e] * inv);
            sf[4 + e] = static_cast<_Float16>(S[1][e] * inv);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sm.partX[buf][w][i][l] = mfma(f.kexp[i], sf, zero4());
            sm.partO[buf][w][i][l] = mfma(f.qg[i], sf, zero4());
        }
        sm.sig[buf][w][l] = sig;
    }
    KDA_SCHED_FENCE();
    ld.part1(fn, w, l);
    KDA_SCHED_FENCE();
    __syncthreads();

    // (b) X = Diag(beta)(V - (K.e^G) S) for all 64 tokens, column j0 + r
    f4 X[4];
    float mx = 0.f;
    float sw[NCB];
#pragma unroll
    for (int ww = 0; ww < NCB; ++ww) sw[ww] = sm.sig[buf][ww][l];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f4 ks = sm.partX[buf][0][i][l] * sw[0];
#pragma unroll
        for (int ww = 1; ww < NCB; ++ww) ks += sm.partX[buf][ww][i][l] * sw[ww];
        const f4 vv = *reinterpret_cast<const f4 *>(&sm.vT[buf][r][16 * i + 4 * g]);
        const f4 bb = *reinterpret_cast<const f4 *>(&sm.bet[buf][16 * i + 4 * g]);
        X[i] = bb * (vv - ks);
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(X[i][e]));
    }
    float invx;
    const float sigx = col_scale(col_max(mx), invx);
    half8 xf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xf[ks][e] = static_cast<_Float16>(X[2 * ks][e] * invx);
            xf[ks][4 + e] = static_cast<_Float16>(X[2 * ks + 1][e] * invx);
        }

    KDA_SCHED_FENCE();
    ld.part2(fn, w, l);
    KDA_SCHED_FENCE();
    // (c) U' = T X
    f4 U[4];
    U[0] = mfma(sm.t[buf][0][l], xf[0], zero4());
    U[1] = mfma(sm.t[buf][1][l], xf[0], zero4());
    U[2] = mfma(sm.t[buf][3][l], xf[1], mfma(sm.t[buf][2][l], xf[0], zero4()));
    U[3] = mfma(sm.t[buf][5][l], xf[1], mfma(sm.t[buf][4][l], xf[0], zero4()));
    // U holds U' / sigx; pick U' / sigu with the column maximum of U' in [2^14, 2^15)
    float mu = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) mu = fmaxf(mu, fabsf(U[i][e]));
    float invu;
    const float sigu = col_scale(col_max(mu) * sigx, invu);
    const float ru = sigx * invu;
    half8 uf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uf[ks][e] = static_cast<_Float16>(U[2 * ks][e] * ru);
            uf[ks][4 + e] = static_cast<_Float16>(U[2 * ks + 1][e] * ru);
        }

    KDA_SCHED_FENCE();
    ld.part3(fn, w, l);
    KDA_SCHED_FENCE();
    // (d) S <- Diag(e^{G_n}) S + (K.e^{G_n-G})^T U'
    if (hasS) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const f4 gm = *reinterpret_cast<const f4 *>(&sm.gam[buf][16 * (2 * w + tt) + 4 * g]);
            f4 acc = S[tt] * gm * invu;
            acc = mfma(f.kgt[tt][0], uf[0], acc);
            acc = mfma(f.kgt[tt][1], uf[1], acc);
            S[tt] = acc * sigu;
        }
    }

    // (e) O rows of token block w = (Q.e^G) S + P U'
    {
        f4 ov = sm.partO[buf][0][w][l] * sw[0];
#pragma unroll
        for (int ww = 1; ww < NCB; ++ww) ov += sm.partO[buf][ww][w][l] * sw[ww];
        f4 pu = mfma(f.p[0], uf[0], zero4());
        if (w >= 2) pu = mfma(f.p[1], uf[1], pu);
        out = (ov + pu * sigu) * scale;
    }
}

template <int K, int V, typename TOut>
__global__ __launch_bounds__(256) void scan_kernel(PrefillArgs a, const int32_t *off, const char *recs) {
    constexpr int NCB = K / 32, NV = V / 16;
    __shared__ ScanSmem<K, V, TOut> sm;

    // blockIdx -> (unit, value tile) with the NV tiles of a unit on one XCD
    const int bid = blockIdx.x, xcd = bid & 7, q8 = bid >> 3;
    const int vt = q8 % NV, unit = (q8 / NV) * 8 + xcd;
    if (unit >= a.N * a.H) return;
    const int n = unit / a.H, h = unit - (unit / a.H) * a.H, j0 = vt * 16;
    const int H = a.H;
    const int tid = threadIdx.x, l = tid & 63, r = l & 15, g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool hasS = w < NCB;
    const size_t sbase = (static_cast<size_t>(n) * H + h) * static_cast<size_t>(K) * V;

    f4 S[2] = {zero4(), zero4()};  // S[16 (2w + tt) + 4g + e][j0 + r]
    if (hasS && a.s0) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[tt][e] = a.s0[sbase + static_cast<size_t>(16 * (2 * w + tt) + 4 * g + e) * V + j0 + r];
    }
    const int cbeg = off[n], cend = off[n + 1];
    const int tbeg = a.cu_seqlens[n], tend = a.cu_seqlens[n + 1];
    const size_t nc = a_nc(a);
    const bf16_t *vg = static_cast<const bf16_t *>(a.v);
    TOut *og = static_cast<TOut *>(a.o);

    if (cbeg < cend) {
        // operands of chunk c + 1 load while chunk c is processed; the copy at the
        // top of the loop waits for loads issued one chunk earlier
        Frags<K> nx;
        const int clast = cend - 1;
        {
            const FragLoader<K, V> ld(recs, nc, cbeg, clast, H, h, vg, tbeg, tend, cbeg, j0, tid);
            ld.part0(nx, tid, w, l);
            ld.part1(nx, w, l);
            ld.part2(nx, w, l);
            ld.part3(nx, w, l);
        }

        // The output of chunk c is stored at the start of iteration c + 1, after the
        // wait for the prefetched operands: stores and loads share one completion
        // counter, so a store issued just before that wait would stall it.
        auto store_out = [&](int c, const f4 &ov) {
            const int t0 = tbeg + (c - cbeg) * kC;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tok = t0 + 16 * w + 4 * g + e;
                if (tok < tend) io<TOut>::store(og + (static_cast<size_t>(tok) * H + h) * V + j0 + r, ov[e]);
            }
        };
        f4 out = zero4();
        int buf = 0;
        for (int c = cbeg; c < cend; ++c, buf ^= 1) {
            const Frags<K> cu = nx;
            // Chunk c's shared data goes to LDS buffer c & 1 before chunk c's barrier.
            // That buffer was last read by chunk c - 2; a wave that reaches this point
            // has passed chunk c - 1's barrier, which no wave reaches before it has
            // finished chunk c - 2, so the writes cannot overtake those reads.
            stage<K, V, TOut>(sm, buf, cu, tid);
            if (c > cbeg) store_out(c - 1, out);
            const FragLoader<K, V> ld(recs, nc, c + 1, clast, H, h, vg, tbeg, tend, cbeg, j0, tid);
            scan_chunk<K, V, TOut>(sm, cu, nx, ld, S, buf, a.scale, tid, w, l, r, g, out);
        }
        store_out(cend - 1, out);
    }
    if (hasS && a.sT) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                a.sT[sbase + static_cast<size_t>(16 * (2 * w + tt) + 4 * g + e) * V + j0 + r] = S[tt][e];
    }
}

template <int K, int V>
hipError_t launch_kv(const PrefillArgs &a, hipStream_t st) {
    using R = Rec<K>;
    const size_t nc_max = a_nc(a);
    int32_t *off = static_cast<int32_t *>(a.ws);
    char *recs = static_cast<char *>(a.ws) + align256(static_cast<size_t>(a.N + 1) * 4);
    hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(256), 0, st, a.cu_seqlens, a.N, off);
    if (a.T > 0)
        hipLaunchKernelGGL((prep_kernel<K>), dim3(static_cast<unsigned>(nc_max * a.H)), dim3(256), 0, st,
                           a, off, recs);
    const unsigned units = static_cast<unsigned>(a.N) * a.H;
    const dim3 grid(((units + 7) / 8) * 8 * (V / 16));
    if (a.out_dtype == KDA_BF16)
        hipLaunchKernelGGL((scan_kernel<K, V, bf16_t>), grid, dim3(256), 0, st, a, off, recs);
    else
        hipLaunchKernelGGL((scan_kernel<K, V, float>), grid, dim3(256), 0, st, a, off, recs);
    (void)sizeof(R);
    return hipGetLastError();
}

template <int K>
size_t workspace_k(int32_t N, int32_t T, int32_t H) {
    const size_t nc_max = static_cast<size_t>((T + kC - 1) / kC) + N;
    return align256(static_cast<size_t>(N + 1) * 4) + nc_max * H * Rec<K>::BYTES;
}

}  // namespace

size_t prefill_mfma_workspace(int32_t N, int32_t T, int32_t H, int32_t K, int32_t V) {
    (void)V;
    return K == 128 ? workspace_k<128>(N, T, H) : workspace_k<64>(N, T, H);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t st) {
    if (a.K == 128 && a.V == 128) return launch_kv<128, 128>(a, st);
    if (a.K == 128 && a.V == 64) return launch_kv<128, 64>(a, st);
    if (a.K == 64 && a.V == 128) return launch_kv<64, 128>(a, st);
    return launch_kv<64, 64>(a, st);
}

}  // namespace kda
