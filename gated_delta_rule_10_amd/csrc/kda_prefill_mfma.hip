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
// U' enters only those two products, so with B = T Diag(beta), X = V - (K . e^G) S,
// Y = B^T (K . e^{G_n-G}):  O = scale ((Q . e^G) S + (P B) X),  S <- Diag(e^{G_n}) S + Y^T X.
//
// Kernels.
//  * prep (persistent, all (chunk, head) items in parallel): every quantity that
//    does not depend on the state. The 64x64 pairwise matrices are built from
//    16-token sub-chunks: for a row in sub-chunk i and a column in sub-chunk
//    j <= i, e^{G_r-G_s} = e^{G_r-G_m} e^{G_m-G_s} with m after the 8th token of
//    sub-chunk i, so every column factor below the diagonal is <= 1 and, on the
//    diagonal, each factor is at most the decay over half a sub-chunk. Those
//    products run as fp16 16x16x32 MFMAs with fp32 accumulation. Sub-chunks whose
//    decay in some channel exceeds e^10 over 16 tokens, or whose operands would
//    leave the fp16 range, take an exact fp32 per-element path for their diagonal
//    block instead. T is inverted in fp32 (forward
//    substitution on the 16x16 diagonal blocks, fp32 MFMA block recurrence
//    below them); Y and P B are fp16 MFMA products of T Diag(beta) with the
//    decayed keys and with P. Results are written to the workspace as fp16 MFMA
//    operand fragments in exactly the register layout the state passes consume.
//  * state passes over segments of consecutive chunks (see below): a map pass,
//    a prefix over segments and an output pass. The state lives in MFMA
//    accumulators (fp32); every value-side operand (state, X = V - K S) is
//    scaled per value column by a power of two for its fp16 conversion (the
//    state is held scaled, its scale changed only when its range requires), so
//    the fp16 range never limits the magnitude of v or of the state.
//
// Options of kda_chunk_fwd_ex: the gates from bf16 pre-activations are formed
// in prep at the end of the item before the one that uses them (off the start
// of an item, where every wave waits for them); grouped key heads only change
// which q/k rows prep reads; slot-indexed states only change where the state
// passes read the initial and write the final state; the RMS-norm / output-gate
// epilogue runs in the output pass on an fp32 tile of each chunk's outputs.
//
// MFMA fragment conventions (v_mfma_f32_16x16x32_f16, lane l, r = l % 16,
// g = l / 16): A operand holds A[r][k(g, e)], B operand B[k(g, e)][r], result
// D[4g + e'][r], e = 0..7, e' = 0..3. Along every contraction index this file
// uses k(g, e) = 4g + e for e < 4 and 16 + 4g + (e - 4) for e >= 4, which is
// exactly the set of rows a lane holds of two stacked 16x16 results, so a
// product's result feeds the next product's B operand from registers.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;
constexpr float kFastRange = 10.f;  // max decay exponent of one sub-chunk on the fp16 path
// Bound of the fp16 diagonal column operand k_s e^{G_b - G_s} (<= max|k| e^{decay of the
// sub-chunk}), below the fp16 maximum 65504; above it the exact fp32 path is taken.
constexpr float kFastOperand = 3.0e4f;

__device__ __forceinline__ f4 mfma(half8 a, half8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }
// Stores of data that is read at most once more, by a later pass (chunk records)
// or not at all by this library (outputs): nontemporal, so they stream past the
// caches instead of evicting lines that are still in use.
template <typename T>
__device__ __forceinline__ void store_stream(T *p, T v) { __builtin_nontemporal_store(v, p); }
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
// With B = T Diag(beta): Y = B^T (K.e^{G_n-G}) and PB = P B, the only two ways the
// state passes use B (U' = B X enters the state update as (K.e^{G_n-G})^T U' = Y^T X
// and the outputs as P U' = PB X), so U' itself is never formed.
template <int K>
struct Rec {
    static constexpr int NCB = K / 32, NCT = K / 16;
    static constexpr size_t FRAG = 1024;
    static constexpr size_t KEXP = 0;                        // [i 4][cb NCB]  (K.e^G)
    static constexpr size_t QG = KEXP + 4 * NCB * FRAG;      // [i 4][cb NCB]  (Q.e^G)
    static constexpr size_t YT = QG + 4 * NCB * FRAG;        // [ct NCT][ks 2] Y^T
    static constexpr size_t PB = YT + 2 * NCT * FRAG;        // 6 lower blocks of P B
    static constexpr size_t GAM = PB + 6 * FRAG;             // e^{G_n} [K] fp32
    static constexpr size_t BYTES = (GAM + 4 * K + 255) / 256 * 256;
};
// (row block i, 32-wide k step ks) -> fragment index for the lower-triangular P B
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
// chunk and segment offsets: off[n] = sum_{m<n} ceil(len_m / 64), off[N] = total
// chunks; soff[n] = sum_{m<n} G_m segments. A sequence of at most L chunks is one
// segment; a longer one has a segment 0 of L0 <= L chunks and then segments of L
// chunks (the last one shorter): G = 1 + ceil((chunks - L0) / L).
__global__ __launch_bounds__(256) void chunk_offsets_kernel(const int32_t *cu, int32_t N, int32_t L, int32_t L0,
                                                             int32_t *off, int32_t *soff) {
    __shared__ int32_t buf[2][256];
    __shared__ int32_t carry[2];
    const int t = threadIdx.x;
    if (t < 2) carry[t] = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + t;
        int nc = 0, ns = 0;
        if (n < N) {
            nc = (max(cu[n + 1] - cu[n], 0) + kC - 1) / kC;
            ns = nc <= L ? 1 : 1 + (nc - L0 + L - 1) / L;
        }
        buf[0][t] = nc;
        buf[1][t] = ns;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int x0 = t >= d ? buf[0][t - d] : 0, x1 = t >= d ? buf[1][t - d] : 0;
            __syncthreads();
            buf[0][t] += x0;
            buf[1][t] += x1;
            __syncthreads();
        }
        if (n < N) {
            off[n] = carry[0] + buf[0][t] - nc;
            soff[n] = carry[1] + buf[1][t] - ns;
        }
        __syncthreads();
        if (t == 255) {
            carry[0] += buf[0][255];
            carry[1] += buf[1][255];
        }
        __syncthreads();
    }
    if (t == 0) {
        off[N] = carry[0];
        soff[N] = carry[1];
    }
}

// ---------------------------------------------------------------------------
// prep: state-independent work of one chunk of one head
template <int K>
struct PrepSmem {
    // row stride of the fp32 64 x 64 matrices: with 68 (= 4 mod 64) words, the
    // accumulator layout (rows 4g + e, column r) and the A-operand reads (row r,
    // columns 4s + g) both spread a wave's 64 lanes over distinct banks
    static constexpr int NCB = K / 32, LD = 68;
    _Float16 kgT[K][kC + 8];  // (K.e^{G_n-G}) transposed [channel][token], read last for Y
    float beta[kC];
    float kmax[4];  // max |k_i|, |q_i| over the tokens and channels of each sub-chunk
    union {
        struct {  // decay factors and the operands of the pairwise products
            float tot[4][K];          // decay of each sub-chunk per channel (log, <= 0)
            float mid[4][K];          // decay from each sub-chunk's start through its 8th token (log, <= 0)
            float fac[19][K + 4];     // per-channel factors, see prep_kernel
            half8 colv[10][NCB][64];  // B operands of the pairwise products
        } a;
        struct {  // then the pairwise matrices and the UT transform
            float A[kC][LD];
            float P[kC][LD];
            float T[kC][LD];
        } b;
    } u;
};

// prep workgroups resident per compute unit (its LDS use allows two)
constexpr int kPrepWgsPerCu = 2;

// One (chunk, head) work item of prep: chunk c of sequence n, tokens [t0, t0 + nt).
struct PrepItem {
    int c, h, n, t0, nt;
};
__device__ __forceinline__ PrepItem prep_item(const PrefillArgs &a, const int32_t *off, int u) {
    const int c = u / a.H, h = u - (u / a.H) * a.H;
    int lo = 0, hi = a.N - 1;  // sequence n with off[n] <= c < off[n + 1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ld_meta(off, mid) <= c) lo = mid; else hi = mid - 1;
    }
    const int t0 = ld_meta(a.cu_seqlens, lo) + (c - ld_meta(off, lo)) * kC;
    return PrepItem{c, h, lo, t0, min(kC, ld_meta(a.cu_seqlens, lo + 1) - t0)};
}

// The inputs one lane reads for a work item: token 16w + r of the chunk and, per
// 32-channel block, the 8 consecutive channels o(g) .. o(g) + 7 with
// o(g) = 16 (g & 1) + 8 (g >> 1), so every k, q (and bf16 gate) load is 16 bytes.
// One v_permlane16_swap per register pair (it exchanges the odd 16-lane rows of
// its first operand with the even rows of its second) then leaves lane g with
// channels 4g .. 4g + 3 in the first result and 16 + 4g .. 16 + 4g + 3 in the
// second: the chain order k(g, e) of the MFMA operands. With GX the log decay
// comes from bf16 gate pre-activations (log alpha = -gscale softplus(x)) instead
// of fp32 log alpha.
__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void swap16(float &a, float &b) {
    uint32_t x = __float_as_uint(a), y = __float_as_uint(b);
    swap16(x, y);
    a = __uint_as_float(x);
    b = __uint_as_float(y);
}

template <int K, bool GX>
struct PrepRaw {
    float4 gv[K / 32][2];  // fp32 log alpha: channels o(g) .. + 3 and o(g) + 4 .. + 7 (without GX)
    uint4 xv[K / 32];      // bf16 gate pre-activation, 8 channels (with GX)
    uint4 kv[K / 32], qv[K / 32];
    uint32_t betaw;  // beta as loaded: fp32 bits, or bf16 bits of its pre-activation
    bool valid;  // token inside the sequence (else its k, q, decay and beta count as zero)

    // Loads are unconditional: a token past the sequence end reads token t0 of the chunk.
    // q and k come from key head h / (H / Hk) of the value head h.
    __device__ __forceinline__ void load(const PrefillArgs &a, const PrepItem &it, bool ok, int tr, int g) {
        load_gates(a, it, ok, tr, g);
        load_kq(a, it, tr, g);
    }
    // The next item's inputs load in parts rather than in one burst, which together with
    // the current item's stores held the CU's vector-memory pipeline (64 KB of loads and
    // 32 KB of stores per workgroup): its beta and the decay of channel block cb right
    // after the current item stores its K.e^G and Q.e^G fragments of block cb (the
    // elementwise phase), its k and q once the pairwise products have consumed the
    // current row operands (load_kq). load() takes an item's inputs at once.
    __device__ __forceinline__ void load_gates(const PrefillArgs &a, const PrepItem &it, bool ok, int tr, int g) {
        valid = ok && tr < it.nt;
        const size_t t = static_cast<size_t>(it.t0 + (valid ? tr : 0));
        const size_t tok = t * a.H + it.h;
        const size_t row = tok * K;
        const int o = 16 * (g & 1) + 8 * (g >> 1);
#pragma unroll
        for (int cb = 0; cb < K / 32; ++cb) {
            const int ch = 32 * cb + o;
            if constexpr (GX) {
                xv[cb] = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.gx) + row + ch);
            } else {
                gv[cb][0] = *reinterpret_cast<const float4 *>(a.g + row + ch);
                gv[cb][1] = *reinterpret_cast<const float4 *>(a.g + row + ch + 4);
            }
        }
        // raw bits: converting here would make the wave wait for the load at once
        if (a.by) betaw = static_cast<const bf16_t *>(a.by)[tok];
        else betaw = reinterpret_cast<const uint32_t *>(a.beta)[tok];
    }
    // the decay of channel block cb only (with valid as set by load_gates_meta)
    __device__ __forceinline__ void load_gate_block(const PrefillArgs &a, const PrepItem &it, int tr, int g, int cb) {
        const size_t t = static_cast<size_t>(it.t0 + (valid ? tr : 0));
        const size_t row = (t * a.H + it.h) * K;
        const int ch = 32 * cb + 16 * (g & 1) + 8 * (g >> 1);
        if constexpr (GX) {
            xv[cb] = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.gx) + row + ch);
        } else {
            gv[cb][0] = *reinterpret_cast<const float4 *>(a.g + row + ch);
            gv[cb][1] = *reinterpret_cast<const float4 *>(a.g + row + ch + 4);
        }
    }
    // valid and beta of an item
    __device__ __forceinline__ void load_gates_meta(const PrefillArgs &a, const PrepItem &it, bool ok, int tr) {
        valid = ok && tr < it.nt;
        const size_t t = static_cast<size_t>(it.t0 + (valid ? tr : 0));
        const size_t tok = t * a.H + it.h;
        if (a.by) betaw = static_cast<const bf16_t *>(a.by)[tok];
        else betaw = reinterpret_cast<const uint32_t *>(a.beta)[tok];
    }
    // k and q of an item (valid as set by load_gates for the same item)
    __device__ __forceinline__ void load_kq(const PrefillArgs &a, const PrepItem &it, int tr, int g) {
        const size_t t = static_cast<size_t>(it.t0 + (valid ? tr : 0));
        const size_t rowk = (t * a.Hk + it.h / (a.H / a.Hk)) * K;
        const int o = 16 * (g & 1) + 8 * (g >> 1);
#pragma unroll
        for (int cb = 0; cb < K / 32; ++cb) {
            const int ch = 32 * cb + o;
            kv[cb] = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.k) + rowk + ch);
            qv[cb] = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.q) + rowk + ch);
        }
    }
    // beta (sigmoid of the bf16 pre-activation when given), 0 past the sequence end
    __device__ __forceinline__ float beta(const PrefillArgs &a) const {
        if (!valid) return 0.f;
        return a.by ? sigmoid_f(__uint_as_float(betaw << 16)) : __uint_as_float(betaw);
    }
    // With GX: the gate pre-activations as fp32 log alpha in gv, in the layout of
    // fp32 gates (channels o .. o + 3, o + 4 .. o + 7). Called once the loads have
    // landed, away from the start of the item that uses them.
    __device__ __forceinline__ void activate(float gscale) {
        if constexpr (GX) {
#pragma unroll
            for (int cb = 0; cb < K / 32; ++cb) {
                const uint32_t w4[4] = {xv[cb].x, xv[cb].y, xv[cb].z, xv[cb].w};
                float f[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[2 * e] = log_alpha_from(__uint_as_float(w4[e] << 16), gscale);
                    f[2 * e + 1] = log_alpha_from(__uint_as_float(w4[e] & 0xFFFF0000u), gscale);
                }
                gv[cb][0] = make_float4(f[0], f[1], f[2], f[3]);
                gv[cb][1] = make_float4(f[4], f[5], f[6], f[7]);
            }
        }
    }
    // max |k_i|, |q_i| of the loaded channels, from the bf16 bits (sign cleared, two values
    // per word compared as 16-bit integers, whose order is that of the magnitudes)
    __device__ __forceinline__ float absmax() const {
        typedef uint16_t us2 __attribute__((ext_vector_type(2)));
        us2 m = {0, 0};
#pragma unroll
        for (int cb = 0; cb < K / 32; ++cb) {
            const uint32_t w[8] = {kv[cb].x, kv[cb].y, kv[cb].z, kv[cb].w, qv[cb].x, qv[cb].y, qv[cb].z, qv[cb].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w[i] & 0x7FFF7FFFu));
        }
        return __uint_as_float(static_cast<uint32_t>(m.x > m.y ? m.x : m.y) << 16);
    }
    // k, q and the inclusive scan of the log decay over the 16-token sub-chunk
    // (lanes r of a 16-lane row are its consecutive tokens), channels in chain order
    __device__ __forceinline__ void unpack(float (&kx)[K / 32][8], float (&qx)[K / 32][8], float (&sc)[K / 32][8],
                                           float gscale) const {
#pragma unroll
        for (int cb = 0; cb < K / 32; ++cb) {
            uint4 kk = kv[cb], qq = qv[cb];
            swap16(kk.x, kk.z);
            swap16(kk.y, kk.w);
            swap16(qq.x, qq.z);
            swap16(qq.y, qq.w);
            float gg[8];
            {  // fp32 log alpha (with GX, as activate() left it)
                float4 p = gv[cb][0], q4 = gv[cb][1];
                swap16(p.x, q4.x);
                swap16(p.y, q4.y);
                swap16(p.z, q4.z);
                swap16(p.w, q4.w);
                gg[0] = p.x; gg[1] = p.y; gg[2] = p.z; gg[3] = p.w;
                gg[4] = q4.x; gg[5] = q4.y; gg[6] = q4.z; gg[7] = q4.w;
            }
            const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w}, qw[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kx[cb][2 * e] = __uint_as_float(kw[e] << 16);
                kx[cb][2 * e + 1] = __uint_as_float(kw[e] & 0xFFFF0000u);
                qx[cb][2 * e] = __uint_as_float(qw[e] << 16);
                qx[cb][2 * e + 1] = __uint_as_float(qw[e] & 0xFFFF0000u);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[cb][e] = gg[e];
        }
        // tokens past the sequence end (only in a sequence's last chunk: a wave-uniform branch)
        if (__builtin_amdgcn_ballot_w64(!valid) != 0) {
#pragma unroll
            for (int cb = 0; cb < K / 32; ++cb)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sc[cb][e] = valid ? sc[cb][e] : 0.f;
                    kx[cb][e] = valid ? kx[cb][e] : 0.f;
                    qx[cb][e] = valid ? qx[cb][e] : 0.f;
                }
        }
#pragma unroll
        for (int cb = 0; cb < K / 32; ++cb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = sc[cb][e];
                v += dpp_row_shr<1>(v);
                v += dpp_row_shr<2>(v);
                v += dpp_row_shr<4>(v);
                v += dpp_row_shr<8>(v);
                sc[cb][e] = v;  // G_r - G_b: log decay from the sub-chunk start to token r (inclusive)
            }
    }
};

// Persistent: each workgroup walks the (chunk, head) items with stride gridDim.x
// and loads the next item's inputs into registers while it finishes the current
// one, so the input loads of one item overlap the pairwise products, the UT
// transform and the stores of the previous one.
template <int K, bool GX>
__global__ __launch_bounds__(256, kPrepWgsPerCu) void prep_kernel(PrefillArgs a, const int32_t *off, char *recs) {
    constexpr int NCB = K / 32, NCT = K / 16;
    using R = Rec<K>;
    __shared__ PrepSmem<K> sm;
    const int total = ld_meta(off, a.N) * a.H;
    const int tid = threadIdx.x, l = tid & 63, r = l & 15, g = l >> 4;
    // wave index as a scalar: branches on it must be real jumps, because a
    // matrix instruction inside an EXEC-masked block still writes its result
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tr = 16 * w + r;  // token of this lane inside the chunk
    int u = blockIdx.x;
    PrepItem nx = prep_item(a, off, u < total ? u : 0);
    PrepRaw<K, GX> raw;
    raw.load(a, nx, u < total, tr, g);
    raw.activate(a.gscale);
    float kqmax = raw.absmax();  // of the item whose inputs the registers hold
    for (; u < total; u += gridDim.x) {
    const PrepItem it = nx;
    const int c = it.c, h = it.h;
    char *rec = recs + (static_cast<size_t>(h) * a_nc(a) + c) * R::BYTES;

    float kx[NCB][8], qx[NCB][8], s[NCB][8];
    raw.unpack(kx, qx, s, a.gscale);
    if (g == 0) sm.beta[tr] = raw.beta(a);
    {  // max |k_i|, |q_i| of this sub-chunk: the lane's (taken when its loads landed), over
       // its 16-lane row, then the 4 rows
        float m = kqmax;
        m = fmaxf(m, dpp_row_shr<1>(m));
        m = fmaxf(m, dpp_row_shr<2>(m));
        m = fmaxf(m, dpp_row_shr<4>(m));
        m = fmaxf(m, dpp_row_shr<8>(m));
        m = col_max(m);
        if (l == 15) sm.kmax[w] = m;
    }
    if (r == 15 || r == 7) {
        float(*dst)[K] = r == 15 ? sm.u.a.tot : sm.u.a.mid;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[w][32 * cb + kidx(g, e)] = s[cb][e];
    }
    __syncthreads();

    // ---- per-channel factors. The pairwise products of a row in sub-chunk i take their
    // reference at m_i, after the 8th token of sub-chunk i: e^{G_r - G_s} =
    // e^{G_r - G_{m_i}} e^{G_{m_i} - G_s}, so both factors of a diagonal block stay within
    // e^{(decay over 8 tokens)}, and every column factor of a block below it is <= 1. A
    // chunk on the exact diagonal path (slow) takes the reference at the sub-chunk start
    // instead (mu = 0 below), which keeps every row operand <= |k|.
    // Rows, with mu_w the reference's decay inside sub-chunk w: 0..3 e^{G_{b_w} + mu_w}
    // (K.e^G and Q.e^G from the row operands), 4..7 decay after sub-chunk w to the chunk
    // end, 8..11 e^{mu_w - tot_w} (diagonal column operand, clamped), 12..14 e^{mu_{w+1}},
    // 15..16 e^{tot_{w+1} + mu_{w+2}}, 17 e^{tot1 + tot2 + mu_3} (column operands of the
    // blocks below the diagonal), 18 e^{G_n}.
    // Two threads per channel, each with half of the rows. The first also checks whether
    // the fast path applies: every sub-chunk's decay within e^kFastRange, and its fp16
    // operands within range: a row operand (k or q times e^{G_r - G_m}) is at most
    // max|k, q| e^{-mu}, a diagonal column operand at most max|k| e^{mu - tot}.
    auto factors = [&](bool start_ref) {
        int bad = 0;
        if (tid < 2 * K) {
            const int ch = tid & (K - 1);
            const float d0 = sm.u.a.tot[0][ch], d1 = sm.u.a.tot[1][ch], d2 = sm.u.a.tot[2][ch], d3 = sm.u.a.tot[3][ch];
            float mu[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) mu[i] = start_ref ? 0.f : sm.u.a.mid[i][ch];
            if (start_ref && tid < K) {  // the elementwise phase reads the reference from mid
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.u.a.mid[i][ch] = 0.f;
            }
            if (tid < K) {
                float emu[4], fd[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    emu[i] = __expf(mu[i]);
                    fd[i] = __expf(fminf(mu[i] - (i == 0 ? d0 : i == 1 ? d1 : i == 2 ? d2 : d3), 80.f));
                    sm.u.a.fac[8 + i][ch] = fd[i];
                    if (i > 0) sm.u.a.fac[11 + i][ch] = emu[i];
                    const float d = i == 0 ? d0 : i == 1 ? d1 : i == 2 ? d2 : d3;
                    bad |= -d > kFastRange || !(sm.kmax[i] <= kFastOperand * emu[i]) ||
                           !(sm.kmax[i] * fd[i] <= kFastOperand);
                }
                sm.u.a.fac[0][ch] = emu[0];
            } else {
                sm.u.a.fac[1][ch] = __expf(d0 + mu[1]);
                sm.u.a.fac[2][ch] = __expf(d0 + d1 + mu[2]);
                sm.u.a.fac[3][ch] = __expf(d0 + d1 + d2 + mu[3]);
                sm.u.a.fac[4][ch] = __expf(d1 + d2 + d3);
                sm.u.a.fac[5][ch] = __expf(d2 + d3);
                sm.u.a.fac[6][ch] = __expf(d3);
                sm.u.a.fac[7][ch] = 1.f;
                sm.u.a.fac[15][ch] = __expf(d1 + mu[2]);
                sm.u.a.fac[16][ch] = __expf(d2 + mu[3]);
                sm.u.a.fac[17][ch] = __expf(d1 + d2 + mu[3]);
                sm.u.a.fac[18][ch] = __expf(d0 + d1 + d2 + d3);
            }
        }
        return bad;
    };
    const int bad = factors(false);
    const bool slow = __syncthreads_or(bad);
    if (slow) {  // rare: the exact diagonal path, with the reference at the sub-chunk starts
        (void)factors(true);
        __syncthreads();
    }

    if (tid < K) store_stream(reinterpret_cast<float *>(rec + R::GAM) + tid, sm.u.a.fac[18][tid]);

    // ---- elementwise: decayed operands
    {
        const int un = u + static_cast<int>(gridDim.x);
        nx = prep_item(a, off, un < total ? un : 0);
    }
    half8 kr[NCB], qr[NCB];
    // this lane's 8 channels of a 32-channel block (chain order) from a per-channel table row
    auto row8 = [&](const float *rowp, int cb, float (&o)[8]) {
        const f4 lo4 = *reinterpret_cast<const f4 *>(rowp + 32 * cb + 4 * g);
        const f4 hi4 = *reinterpret_cast<const f4 *>(rowp + 32 * cb + 16 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[e] = lo4[e];
            o[4 + e] = hi4[e];
        }
    };
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        half8 kexp, qg, cv0, cv1, cv2, cv3;
        float tw[8], mw[8], fb[8], fa[8], fi[8], f1[8], f2[8], f3[8];
        row8(sm.u.a.tot[w], cb, tw);
        row8(sm.u.a.mid[w], cb, mw);
        row8(sm.u.a.fac[w], cb, fb);
        row8(sm.u.a.fac[4 + w], cb, fa);
        row8(sm.u.a.fac[8 + w], cb, fi);
        row8(sm.u.a.fac[12 + min(w, 2)], cb, f1);
        row8(sm.u.a.fac[w == 0 ? 15 : 16], cb, f2);
        row8(sm.u.a.fac[17], cb, f3);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = 32 * cb + kidx(g, e);
            // e^{G_r - G_m} (m: the reference of this row's products; at most e^{8-token decay}
            // on the fast path, <= 1 from the sub-chunk start on the slow path, where mid is 0)
            const float rho = __expf(s[cb][e] - mw[e]);
            const float tau = __expf(tw[e] - s[cb][e]);  // e^{G_{b'} - G_r} <= 1, b' = sub-chunk end
            const float krv = kx[cb][e] * rho, qrv = qx[cb][e] * rho;
            kr[cb][e] = static_cast<_Float16>(krv);
            qr[cb][e] = static_cast<_Float16>(qrv);
            kexp[e] = static_cast<_Float16>(krv * fb[e]);
            qg[e] = static_cast<_Float16>(qrv * fb[e]);
            const float kt = kx[cb][e] * tau;
            sm.kgT[ch][tr] = static_cast<_Float16>(kt * fa[e]);
            // column operands of column block w for row blocks i = w..3: k_s e^{G_{m_i} - G_s}
            // (i = w on the slow path: unbounded, but its products are replaced by the exact ones)
            cv0[e] = static_cast<_Float16>(kt * fi[e]);                 // i = w
            cv1[e] = static_cast<_Float16>(kt * f1[e]);                 // i = w + 1
            cv2[e] = static_cast<_Float16>(kt * f2[e]);                 // i = w + 2
            cv3[e] = static_cast<_Float16>(kt * f3[e]);                 // i = 3 (w = 0)
        }
        store_stream(reinterpret_cast<half8 *>(rec + R::KEXP + ((w * NCB + cb) * 64 + l) * 16), kexp);
        store_stream(reinterpret_cast<half8 *>(rec + R::QG + ((w * NCB + cb) * 64 + l) * 16), qg);
        // the next item's beta and block cb of its decay (this item's are unpacked)
        if (cb == 0) raw.load_gates_meta(a, nx, u + static_cast<int>(gridDim.x) < total, tr);
        raw.load_gate_block(a, nx, tr, g, cb);
        sm.u.a.colv[vblk(w, w)][cb][l] = cv0;
        if (w + 1 < 4) sm.u.a.colv[vblk(w + 1, w)][cb][l] = cv1;
        if (w + 2 < 4) sm.u.a.colv[vblk(w + 2, w)][cb][l] = cv2;
        if (w == 0) sm.u.a.colv[vblk(3, 0)][cb][l] = cv3;
    }
    __syncthreads();

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
    raw.load_kq(a, nx, tr, g);  // this item's row operands are consumed: the next item's k and q
    __syncthreads();  // the factors and colv are no longer read; the union now holds A, P, T

    // blocks j <= w of A (strictly lower on the diagonal) and P (lower); the T and P
    // fragments of even row blocks w also span block w + 1, which must read zero
    {
        const f4 bet = *reinterpret_cast<const f4 *>(&sm.beta[16 * w + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j > w + 1 || (j == w + 1 && (w & 1))) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rl = 4 * g + e, rowi = 16 * w + rl, col = 16 * j + r;
                if (j <= w) {
                    float av = accA[j][e], pv = accP[j][e];
                    if (j == w) {
                        av = r < rl ? av : 0.f;
                        pv = r <= rl ? pv : 0.f;
                    }
                    sm.u.b.A[rowi][col] = av * bet[e];
                    sm.u.b.P[rowi][col] = pv;
                } else {
                    sm.u.b.P[rowi][col] = 0.f;
                    sm.u.b.T[rowi][col] = 0.f;
                }
            }
        }
    }
    if (slow) {
        // exact diagonal block: e^{G_r - G_s} per element, s <= r inside sub-chunk w
        // (this item's inputs are read again: the registers now hold the next item's)
        PrepRaw<K, GX> cr;
        cr.load(a, it, true, tr, g);
        cr.activate(a.gscale);
        cr.unpack(kx, qx, s, a.gscale);
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
    // blocks below the diagonal: T_wj = -T_ww sum_{m=j}^{w-1} A_wm T_mj, by distance w - j,
    // as fp32 16x16x4 matrix products (lane (r, g): A operand X[r][k], B operand Y[k][r],
    // result Z[4g + e][r]). X = sum_m A_wm T_mj contracts k = 4s + g in step s; Y = -T_ww X
    // contracts k = 4g + s in step s, so that X's result registers are Y's B operands.
    for (int lev = 1; lev <= 3; ++lev) {
        const int j = w - lev;
        if (j >= 0) {
            f4 x = zero4();
            for (int m = j; m < w; ++m)
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    x = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.u.b.A[16 * w + r][16 * m + 4 * s4 + g],
                                                             sm.u.b.T[16 * m + 4 * s4 + g][16 * j + r], x, 0, 0, 0);
            f4 y = zero4();
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(-sm.u.b.T[16 * w + r][16 * w + 4 * g + s4], x[s4], y, 0, 0,
                                                         0);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.u.b.T[16 * w + 4 * g + e][16 * j + r] = y[e];
        }
        __syncthreads();
    }

    // ---- Y^T and P B fragments (A operands, contraction over tokens), B = T Diag(beta).
    // Both are products with B^T on the left, whose rows are tokens: a 16x16 result block
    // D[4g + e][r] holds for lane (r, g) tokens 4g + e of its block, which is one half of
    // what a fragment lane holds along the contraction (tokens 4g + e, then 16 + 4g + e),
    // so the result blocks of tokens 2 ks and 2 ks + 1 make fragment ks.
    // bt[tb][ks]: rows 16 tb + r of B^T, tokens 32 ks + k(g, e); B^T[t][s] = T[s][t] beta[t]
    // is zero for s < t (ks < tb / 2 is never used; T's blocks above the diagonal that
    // the others span were zeroed above).
    half8 bt[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const float bb = sm.beta[16 * tb + r];
#pragma unroll
        for (int ks = tb >> 1; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                bt[tb][ks][e] = static_cast<_Float16>(sm.u.b.T[32 * ks + kidx(g, e)][16 * tb + r] * bb);
    }
    {  // Y = B^T (K.e^{G_n-G}) for this wave's channel tiles
        typedef _Float16 half4 __attribute__((ext_vector_type(4)));
        constexpr int CPW = NCT / 4;
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
            const int ct = w * CPW + q;
            half8 kf[2];  // B operands: tokens 32 ks + k(g, e) of channel 16 ct + r
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const half4 lo = *reinterpret_cast<const half4 *>(&sm.kgT[16 * ct + r][32 * ks + 4 * g]);
                const half4 hi = *reinterpret_cast<const half4 *>(&sm.kgT[16 * ct + r][32 * ks + 16 + 4 * g]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kf[ks][e] = lo[e];
                    kf[ks][4 + e] = hi[e];
                }
            }
            f4 d[4];
            d[0] = mfma(bt[0][1], kf[1], mfma(bt[0][0], kf[0], zero4()));
            d[1] = mfma(bt[1][1], kf[1], mfma(bt[1][0], kf[0], zero4()));
            d[2] = mfma(bt[2][1], kf[1], zero4());
            d[3] = mfma(bt[3][1], kf[1], zero4());
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                half8 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[e] = static_cast<_Float16>(d[2 * ks][e]);
                    y[4 + e] = static_cast<_Float16>(d[2 * ks + 1][e]);
                }
                store_stream(reinterpret_cast<half8 *>(rec + R::YT + ((ct * 2 + ks) * 64 + l) * 16), y);
            }
        }
    }
    {  // P B of row block w: (P B)^T blocks (tb, w) = sum_ks bt[tb][ks] P^T, zero for tb > w
        half8 pf[2] = {};  // B operands: P[16 w + r][32 ks + k(g, e)] (ks = 1 only below row block 2)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks <= (w >> 1)) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pf[ks][e] = static_cast<_Float16>(sm.u.b.P[16 * w + r][32 * ks + kidx(g, e)]);
            }
        }
        f4 d[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            d[tb] = zero4();
            if (tb <= w) {
#pragma unroll
                for (int ks = tb >> 1; ks < 2; ++ks)
                    if (ks <= (w >> 1)) d[tb] = mfma(bt[tb][ks], pf[ks], d[tb]);
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks <= (w >> 1)) {
                half8 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = static_cast<_Float16>(d[2 * ks][e]);
                    v[4 + e] = static_cast<_Float16>(d[2 * ks + 1][e]);
                }
                store_stream(reinterpret_cast<half8 *>(rec + R::PB + (tri(w, ks) * 64 + l) * 16), v);
            }
        }
    }
    raw.activate(a.gscale);  // the next item's gates
    kqmax = raw.absmax();     // and the magnitude of its k, q
    __syncthreads();  // the next item rewrites the LDS this one read last
    }
}

// ---------------------------------------------------------------------------
// State passes. The chunks of a sequence are cut into segments of consecutive
// chunks (a segment 0 of L0 chunks, then segments of L). Every chunk maps its
// incoming state affinely,
//   S <- (Diag(e^{G_n}) - Y^T (K.e^G)) S + Y^T V,
// so a segment does too: S_out = M S_in + N, with M (d_k x d_k) the segment run
// from the identity with V = 0 and N (d_k x d_v) the segment run from zero.
//  * seg_kernel, every segment but the last of each sequence, in parallel:
//    segment 0 runs from the initial state (its end state enters segment 1; with
//    d_k = d_v it also writes its outputs there), a middle segment runs from the
//    identity for M and from zero for N, both in one workgroup;
//  * prefix_kernel: S_in(g + 1) = M_g S_in(g) + N_g along the middle segments;
//  * out_kernel, every other segment in parallel from its incoming state, with
//    outputs; the last segment of a sequence writes the final state.
// A workgroup covers all columns of one (segment, head) state (and of M); each
// wave holds d_k rows of 32 columns (map pass) or 16 (output pass) in MFMA
// accumulators, two waves per SIMD. A chunk's record is copied global -> LDS once
// per workgroup with direct-to-LDS loads, one chunk ahead, into a two-buffer ring
// (the output pass starts K.e^G and Q.e^G of the chunk after next too), so that no
// record is streamed by more than one compute unit at a time; while one wave of a
// SIMD waits on the memory pipeline the other computes.

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kPad = 32;  // bytes after every 1 KB LDS copy of V or O rows: 4-row groups hit distinct banks

// 64 x V bf16 tile (V, or the output) in LDS: copies of 1 KB (1024 / 2V token rows) + padding
template <int V>
struct VTile {
    static constexpr int RPI = 1024 / (2 * V);
    static constexpr int NI = kC / RPI;
    static constexpr int BYTES = NI * (1024 + kPad);
    __device__ __forceinline__ static int off(int t, int col) {
        return (t / RPI) * (1024 + kPad) + (t % RPI) * (2 * V) + 2 * col;
    }
};

template <int K, int V>
struct ScanBuf {
    static constexpr int VT = static_cast<int>(Rec<K>::BYTES);
    static constexpr int BYTES = VT + VTile<V>::BYTES;
};

// Direct-to-LDS copies (LDS[M0 + inst_offset + size * lane] = global[addr + inst_offset]).
// They are issued as inline assembly, so the compiler does not see them as LDS
// stores and does not make reads of the other ring buffer wait for them: every
// copy is awaited explicitly (vmcnt) before the workgroup barrier that precedes
// the first read of its buffer. M0 is used by nothing else in these kernels.
// (readfirstlane returns a signed int: both halves go through uint32_t before
// widening, so that a low word with bit 31 set is not sign-extended into the high one)
__device__ __forceinline__ uint32_t sgpr_u32(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}
__device__ __forceinline__ uint32_t lds_addr(const char *p) {
    return sgpr_u32(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)p)));
}
__device__ __forceinline__ uint64_t uniform_addr(const void *p) {
    const uint64_t b = reinterpret_cast<uint64_t>(p);
    return (static_cast<uint64_t>(sgpr_u32(static_cast<uint32_t>(b >> 32))) << 32) |
           static_cast<uint64_t>(sgpr_u32(static_cast<uint32_t>(b)));
}
// (the clobber keeps the compiler from assuming an M0 value across these; the
// warning only says it will not save and restore M0 around them)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Record reads (dma16, dma4) are nontemporal: a pass reads each record byte once.
// 16 bytes per lane from uniform base + per-lane 32-bit offset
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, const char *lds) {
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "s"(lds_addr(lds)), "v"(voff), "s"(uniform_addr(base))
                     : "memory", "m0");
}
// 16 bytes per lane from a per-lane 64-bit address
__device__ __forceinline__ void dma16v(const void *addr, const char *lds) {
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(lds_addr(lds)), "v"(reinterpret_cast<uint64_t>(addr))
                     : "memory", "m0");
}
// 4 bytes per lane, 64 lanes = 256 B, uniform base + 4 lane
__device__ __forceinline__ void dma4(const void *base, uint32_t voff, const char *lds) {
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2 nt"
                     :
                     : "s"(lds_addr(lds)), "v"(voff), "s"(uniform_addr(base))
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// Copy chunk data into LDS buffer `dst`, spread over the NW waves: the record
// fragments the pass reads (all of them with outputs, else K.e^G and Y^T), e^{G_n},
// and (HASV) the 64 x V tile of V. Tokens past the sequence end read the last token
// (finite; their columns of Y^T and P B are zero).
// PART (with FULL): 0 = the whole record, 1 = only K.e^G and Q.e^G (copied early),
// 2 = everything but K.e^G and Q.e^G.
template <int K, int V, bool FULL, bool HASV, int NW, int PART = 0>
__device__ __forceinline__ void copy_chunk(char *dst, const char *rec, const bf16_t *vg, int t0, int tend,
                                           int H, int h, int w, int l) {
    using R = Rec<K>;
    constexpr int NKX = 4 * (K / 32);
    constexpr int KG0 = static_cast<int>(R::YT / 1024);
    constexpr int NF = FULL ? static_cast<int>(R::GAM / 1024) : NKX + 2 * (K / 16);
    static_assert(PART == 0 || FULL, "parts of the full record only");
    constexpr int F0 = PART == 2 ? KG0 : 0, F1 = PART == 1 ? KG0 : NF;
    const uint32_t lo = static_cast<uint32_t>(l) * 16u;
    for (int f = F0 + w; f < F1; f += NW) {
        const int fi = (FULL || f < NKX) ? f : f - NKX + KG0;
        dma16(rec + fi * 1024, lo, dst + fi * 1024);
    }
    if (PART == 1) return;
    // e^{G_n} [K] fp32 in copies of 256 B
    static_assert(K % 64 == 0, "e^{G_n} span");
    if (w == NW - 1) {
        const uint32_t l4 = static_cast<uint32_t>(l) * 4u;
#pragma unroll
        for (int q = 0; q < K / 64; ++q) dma4(rec + R::GAM + q * 256, l4, dst + R::GAM + q * 256);
    }
    if (HASV) {
        using VT = VTile<V>;
        constexpr int LPR = 2 * V / 16;  // lanes per token row
        for (int q = w; q < VT::NI; q += NW) {
            const int tok = min(t0 + q * VT::RPI + l / LPR, tend - 1);
            dma16v(vg + (static_cast<size_t>(tok) * H + h) * V + (l % LPR) * 8,
                   dst + ScanBuf<K, V>::VT + q * (1024 + kPad));
        }
    }
}

// fp32 -> bf16 bits, round to nearest even (the gfx950 conversion instruction)
__device__ __forceinline__ bf16_t bf16_rne(float x) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(x)); }

// Fragment reads of a chunk buffer go through a per-buffer lane base (the LDS
// address of buf + 16 l) that the compiler cannot fold into constants: every
// fragment offset inside a record is below 64 KB, so each read then takes its
// offset from the ds_read immediate, also for the buffer that starts above 64 KB
// (otherwise each read of that buffer needs its own address instruction).
typedef __attribute__((address_space(3))) const char lds_cchar;
__device__ __forceinline__ lds_cchar *frag_base(const char *buf, int l) {
    uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)buf)) + 16u * static_cast<uint32_t>(l);
    __asm__("" : "+v"(a));
    return reinterpret_cast<lds_cchar *>(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ half8 lds_frag(lds_cchar *fb, size_t off) {
    return *reinterpret_cast<const __attribute__((address_space(3))) half8 *>(fb + off);
}

// Workgroup barrier without a memory fence: callers wait for the counters they
// need first (a fence would also wait for the copies in flight into the other buffer).
__device__ __forceinline__ void wg_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }         // vm, exp, lgkm = 0
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }    // lgkmcnt(0)

// One chunk for one wave holding NB 16-column blocks of the state, S[j][ct] =
// rows 16 ct + 4g + e of column col0 + 16 j + r, held as S / sc[j] with a power of
// two sc[j] per column (ChunkScale) that changes only when the held values leave the
// range of their fp16 conversion. part_a: (K.e^G) S and (OUT) (Q.e^G) S, and
// X = V - (K.e^G) S as an fp16 operand (V = 0 without HASV); part_b: the state
// update S <- Diag(e^{G_n}) S + Y^T X and (OUT) the outputs O = (Q.e^G) S + (P B) X of
// tokens 16i + 4g + e in out[j][i].
// X is held in the state's own scale when every column of the wave has X / sc below
// 2^15 and its largest magnitude at least 2^-3 (or zero): then its fp16 elements carry
// an error of at most half an fp16 ulp of that largest magnitude (subnormal ones far
// less), as in a scale of its own, and the update and the outputs need no factor
// between two scales (the decayed state is the accumulator of the update's MFMAs,
// (Q.e^G) S that of the outputs'). Otherwise (a wave-uniform branch) X takes its own
// power-of-two scale sigx: X's size beside the state does not bound its effect, since
// a strong decay leaves little of the state beside the update.
template <int NB>
struct ChunkScale {
    float sc[NB], isc[NB];  // sc and 1 / sc, both powers of two
    __device__ __forceinline__ ChunkScale() {
#pragma unroll
        for (int j = 0; j < NB; ++j) sc[j] = isc[j] = 1.f;
    }
};
template <int K, int V, int NB, bool OUT, bool HASV>
struct ChunkStep {
    static constexpr int NCB = K / 32, NCT = K / 16;
    using R = Rec<K>;
    float sigs[NB], sigx[NB], ix[NB];  // with own_x: X held as X / sigx, ix = 1 / sigx
    bool own_x;
    half8 xf[NB][2];
    f4 oa[NB][4];

    static __device__ __forceinline__ float vval(const char *buf, int t, int col) {
        return bf16_to_f32(*reinterpret_cast<const bf16_t *>(buf + ScanBuf<K, V>::VT + VTile<V>::off(t, col)));
    }

    // The held values are the fp16 operand itself while every column's largest magnitude
    // lies in [2^-13, 2^15): below 2^-14 an element is subnormal in fp16, and its absolute
    // error (2^-25 at most) stays under half an fp16 ulp of that largest magnitude. When a
    // column of the wave leaves the range, its columns are brought to [2^14, 2^15) (a
    // wave-uniform branch, rare once a state has formed). The scale is that of col_scale,
    // within [2^-114, 2^96]: a column whose true magnitude falls below 2^-127 (a map
    // decayed away) keeps sc = 2^-114 and fits as it is, and zero columns fit.
    __device__ __forceinline__ void part_a(const char *buf, lds_cchar *fb, f4 (&S)[NB][NCT], ChunkScale<NB> &cs,
                                           int col0, int l, int r, int g) {
        half8 sf[NB][NCB];
        float m[NB];
        bool fit = true;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            float mj = 0.f;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) mj = fmaxf(mj, fabsf(S[j][ct][e]));
            m[j] = col_max(mj);
            fit = fit && m[j] < 0x1p15f && (m[j] >= 0x1p-13f || m[j] == 0.f || cs.sc[j] == 0x1p-114f);
        }
        if (__builtin_amdgcn_ballot_w64(!fit) != 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (m[j] > 0.f) {
                    float inv;
                    const float s = col_scale(m[j] * cs.sc[j], inv);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int e = 0; e < 4; ++e) S[j][ct][e] = (S[j][ct][e] * cs.sc[j]) * inv;
                    cs.sc[j] = s;
                    cs.isc[j] = inv;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            sigs[j] = cs.sc[j];
#pragma unroll
            for (int kb = 0; kb < NCB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sf[j][kb][e] = static_cast<_Float16>(S[j][2 * kb][e]);
                    sf[j][kb][4 + e] = static_cast<_Float16>(S[j][2 * kb + 1][e]);
                }
        }
        f4 xa[NB][4];
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xa[j][i] = zero4();
                if (OUT) oa[j][i] = zero4();
            }
#pragma unroll
        for (int kb = 0; kb < NCB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half8 kx = lds_frag(fb, R::KEXP + (i * NCB + kb) * 1024);
#pragma unroll
                for (int j = 0; j < NB; ++j) xa[j][i] = mfma(kx, sf[j][kb], xa[j][i]);
                if (OUT) {
                    const half8 qx = lds_frag(fb, R::QG + (i * NCB + kb) * 1024);
#pragma unroll
                    for (int j = 0; j < NB; ++j) oa[j][i] = mfma(qx, sf[j][kb], oa[j][i]);
                }
            }
        // X / sc = V / sc - (K.e^G)(S / sc)
        f4 X[NB][4];
        bool held = true;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            float mj = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // without V, X / sc = -xa: the sign goes onto the packed fp16 operand
                    float xv = xa[j][i][e];
                    if (HASV) xv = fmaf(vval(buf, 16 * i + 4 * g + e, col0 + 16 * j + r), cs.isc[j], -xv);
                    X[j][i][e] = xv;
                    mj = fmaxf(mj, fabsf(xv));
                }
            const float mx = col_max(mj);
            held = held && mx < 0x1p15f && (mx >= 0x1p-3f || mx == 0.f);
        }
        own_x = __builtin_amdgcn_ballot_w64(!held) != 0;
        if (own_x) {
            // X in true units, then its own scale. X / sc is not finite only where V / sc
            // passed 2^128: |(K.e^G)(S / sc)| < 2^38 (fp16 operands, d_k <= 128), so there
            // V exceeds sc (K.e^G)(S / sc) by more than 2^90 and X = V in fp32.
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                float mt = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float xt = X[j][i][e] * cs.sc[j];
                        if (HASV && !(fabsf(X[j][i][e]) <= 0x1.fffffep127f))
                            xt = vval(buf, 16 * i + 4 * g + e, col0 + 16 * j + r);
                        X[j][i][e] = xt;
                        mt = fmaxf(mt, fabsf(xt));
                    }
                float invx;
                sigx[j] = col_scale(col_max(mt), invx);
                ix[j] = invx;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) X[j][i][e] *= invx;
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xf[j][ks][e] = static_cast<_Float16>(X[j][2 * ks][e]);
                    xf[j][ks][4 + e] = static_cast<_Float16>(X[j][2 * ks + 1][e]);
                }
        if (!HASV) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    u4 w = __builtin_bit_cast(u4, xf[j][ks]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[q] ^= 0x80008000u;
                    xf[j][ks] = __builtin_bit_cast(half8, w);
                }
        }
    }

    __device__ __forceinline__ void part_b(const char *buf, lds_cchar *fb, f4 (&S)[NB][NCT], ChunkScale<NB> &cs,
                                           f4 (&out)[NB][4], float scale, int g) {
        if (!own_x) {
            // S / sc <- Diag(e^{G_n}) (S / sc) + Y^T (X / sc): the decayed state is the
            // accumulator of the two MFMAs
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f4 gm = *reinterpret_cast<const f4 *>(buf + R::GAM + (16 * ct + 4 * g) * 4);
                const half8 y0 = lds_frag(fb, R::YT + (ct * 2 + 0) * 1024);
                const half8 y1 = lds_frag(fb, R::YT + (ct * 2 + 1) * 1024);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    f4 d;
#pragma unroll
                    for (int e = 0; e < 4; ++e) d[e] = S[j][ct][e] * gm[e];
                    S[j][ct] = mfma(y1, xf[j][1], mfma(y0, xf[j][0], d));
                }
            }
            if (OUT) {
                // O = sc ((Q.e^G)(S / sc) + (P B)(X / sc))
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const half8 p0 = lds_frag(fb, R::PB + tri(i, 0) * 1024);
                    half8 p1 = p0;
                    if (i >= 2) p1 = lds_frag(fb, R::PB + tri(i, 1) * 1024);
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        f4 px = mfma(p0, xf[j][0], oa[j][i]);
                        if (i >= 2) px = mfma(p1, xf[j][1], px);
                        const float os = sigs[j] * scale;
#pragma unroll
                        for (int e = 0; e < 4; ++e) out[j][i][e] = px[e] * os;
                    }
                }
            }
            return;
        }
        // S <- Diag(e^{G_n}) S + Y^T X  (X held as X / sigx, S as S / sc). An update more
        // than 2^100 times the held state's scale restarts that column's scale at sigx (the
        // state is then negligible beside it), so that sigx / sc stays finite.
        float fx[NB];
        bool big = false;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            fx[j] = sigx[j] * cs.isc[j];
            big = big || !(fx[j] <= 0x1p100f);
        }
        if (__builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (!(fx[j] <= 0x1p100f)) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int e = 0; e < 4; ++e) S[j][ct][e] = (S[j][ct][e] * cs.sc[j]) * ix[j];
                    cs.sc[j] = sigx[j];
                    cs.isc[j] = ix[j];
                    fx[j] = 1.f;
                }
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const f4 gm = *reinterpret_cast<const f4 *>(buf + R::GAM + (16 * ct + 4 * g) * 4);
            const half8 y0 = lds_frag(fb, R::YT + (ct * 2 + 0) * 1024);
            const half8 y1 = lds_frag(fb, R::YT + (ct * 2 + 1) * 1024);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const f4 acc = mfma(y1, xf[j][1], mfma(y0, xf[j][0], zero4()));
#pragma unroll
                for (int e = 0; e < 4; ++e) S[j][ct][e] = fmaf(fx[j], acc[e], S[j][ct][e] * gm[e]);
            }
        }
        if (OUT) {
            // O = (Q.e^G) S + (P B) X
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half8 p0 = lds_frag(fb, R::PB + tri(i, 0) * 1024);
                half8 p1 = p0;
                if (i >= 2) p1 = lds_frag(fb, R::PB + tri(i, 1) * 1024);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    f4 px = mfma(p0, xf[j][0], zero4());
                    if (i >= 2) px = mfma(p1, xf[j][1], px);
                    const float os = sigs[j] * scale, ox = sigx[j] * scale;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[j][i][e] = fmaf(oa[j][i][e], os, px[e] * ox);
                }
            }
        }
    }
};

// Output epilogue (kda_options_t), per token and value head, on the fp32 outputs:
// o <- o / sqrt(mean o^2 + eps) * weight if norm, then o <- o * act(z) if z.
struct Epi {
    const bf16_t *z;
    const float *nw;
    float eps;
    int norm, zact;
};

// fp32 64 x V output tile in LDS; the 16-column blocks of row t are permuted by
// XOR with (t / 4) % 4, so the four row groups a wave writes at once hit
// distinct banks while a 16-column block stays contiguous for the row reads.
template <int V>
__device__ __forceinline__ int ftile_off(int row, int col) {
    return (row * V + (col ^ (16 * ((row >> 2) & 3)))) * 4;
}

// The chunks [cb, ce) of one segment (tokens from tbeg; the sequence ends at tend)
// on a workgroup of NW waves. Waves 0 .. CW - 1 issue the copies (the V tile when
// COPYV); an active wave advances its state columns col0 .. col0 + 16 NB - 1
// (with V when HASV). With OUT, the outputs of every chunk go to `og` through an
// LDS tile written once all waves have read the chunk's K.e^G, Q.e^G and V, and
// stored by whole rows at the next chunk: bf16 in the V region of the chunk's
// buffer; with EPI fp32 (in the K.e^G / Q.e^G region, or in `ftd` when that is
// too small), normalised and gated on the way out. fp32 outputs without EPI are
// stored directly from the registers.
template <int K, int V, int NB, bool OUT, bool HASV, bool COPYV, int NW, int CW, bool EPI, typename TOut>
__device__ __forceinline__ void run_segment(char *lb0, char *lb1, char *ftd, f4 (&S)[NB][K / 16], const char *hrec,
                                            int cb, int ce, int tbeg, int tend, const bf16_t *vg, TOut *og, int H,
                                            int h, float scale, const Epi &ep, bool active, int tid, int w, int l,
                                            int r, int g, int col0) {
    constexpr size_t RB = Rec<K>::BYTES;
    constexpr bool TILE = OUT && (EPI || sizeof(TOut) == 2);
    constexpr int NT = 64 * NW;
    constexpr int NP = kC * 2 * V / 16 / NT;  // 16-byte bf16 output pieces per thread
    constexpr int TPR = V / 16;               // threads per row of the fp32 tile (16 columns each)
    static_assert(!TILE || EPI || NP * NT == kC * 2 * V / 16, "output tile pieces");
    static_assert(!EPI || TPR * kC == NT, "one 16-column piece of the fp32 tile per thread");
    using VT = VTile<V>;
    // With bf16 output tiles (no epilogue, whose fp32 tile reuses that region), the
    // K.e^G and Q.e^G fragments of chunk c + 2 are copied into chunk c's buffer as soon
    // as chunk c has read them, and the rest at chunk c + 1. A copy wave then waits for
    // chunk c + 1 with vmcnt(EW): its last vector-memory operations are the EW early
    // copies, and the counter also counts its output stores, so at most EW loads are then
    // outstanding whatever the order in which stores retire. Loads retire in the order
    // they were issued (the rule every partial vmcnt wait rests on), so those are the
    // early copies, and every copy of chunk c + 1 has landed.
    constexpr bool LA = OUT && TILE && !EPI && COPYV;
    constexpr int EW = LA ? 8 * (K / 32) / CW : 0;
    static_assert(!LA || (8 * (K / 32)) % CW == 0, "early copies spread evenly over the copy waves");
    static_assert(EW <= 15, "early copies within the low vmcnt field");
    if (cb >= ce) return;
    f4 out[NB][4];
    ChunkScale<NB> cs;  // the state is held as S / cs.sc across the chunks (ChunkStep)
    if (w < CW) copy_chunk<K, V, OUT, COPYV, CW>(lb0, hrec + static_cast<size_t>(cb) * RB, vg, tbeg, tend, H, h, w, l);

    // epilogue: this thread's row and 16 columns of the fp32 tile, its weights, and
    // the output gate of the chunk whose tile is pending
    const int erow = tid / TPR, ecol = 16 * (tid % TPR);
    float ew[16];
    u4 zq[2] = {u4{0u, 0u, 0u, 0u}, u4{0u, 0u, 0u, 0u}};
    if (EPI) {
#pragma unroll
        for (int c = 0; c < 16; ++c) ew[c] = ep.nw ? ep.nw[ecol + c] : 1.f;
    }
    auto ftb = [&](char *buf) -> char * { return ftd ? ftd : buf; };
    auto epi_read = [&](const char *fb, f4 (&x)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = *reinterpret_cast<const f4 *>(fb + ftile_off<V>(erow, ecol + 4 * q));
    };
    auto epi_store = [&](const f4 (&x)[4], int t0) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = x[q][e];
        if (ep.norm) {
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) ss = fmaf(v[c], v[c], ss);
#pragma unroll
            for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m);
            const float inv = rsqrtf(ss / V + ep.eps);
#pragma unroll
            for (int c = 0; c < 16; ++c) v[c] *= inv * ew[c];
        }
        if (ep.z) {
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const uint32_t wd = zq[c >> 3][(c >> 1) & 3];
                v[c] *= out_gate_act(__uint_as_float((c & 1) ? (wd & 0xFFFF0000u) : (wd << 16)), ep.zact);
            }
        }
        const int tok = t0 + erow;
        if (tok < tend) {
            TOut *dst = og + (static_cast<size_t>(tok) * H + h) * V + ecol;
            if constexpr (sizeof(TOut) == 2) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    u4 pk;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pk[e] = static_cast<uint32_t>(bf16_rne(v[8 * q + 2 * e])) |
                                (static_cast<uint32_t>(bf16_rne(v[8 * q + 2 * e + 1])) << 16);
                    reinterpret_cast<u4 *>(dst)[q] = pk;
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    reinterpret_cast<f4 *>(dst)[q] = f4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
            }
        }
    };

    lds_cchar *const fb0 = frag_base(lb0, l), *const fb1 = frag_base(lb1, l);
    auto body = [&](char *cur, lds_cchar *fbc, char *oth, int c) {
        const int tc = tbeg + (c - cb) * kC;
        // this wave's copies of chunk c, its stores and its LDS writes are done (the early
        // copies of chunk c + 1, issued last, may still be in flight)
        if (LA && c > cb && c + 1 < ce && w < CW) __builtin_amdgcn_s_waitcnt(EW);
        else wait_all();
        wg_barrier();
        u4 pc[(EPI || NP == 0) ? 1 : NP];
        f4 fx[4];
        if (TILE && c > cb) {
            if (EPI) {
                epi_read(ftb(oth), fx);
            } else {
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    const int p = q * NT + tid, row = p / (2 * V / 16), pi = p % (2 * V / 16);
                    pc[q] = *reinterpret_cast<const u4 *>(oth + ScanBuf<K, V>::VT + VT::off(row, pi * 8));
                }
            }
            wait_lds();
        }
        if (TILE) wg_barrier();  // every wave has read the previous output tile
        if (c + 1 < ce && w < CW) {
            bool rest = false;  // chunk c + 1's K.e^G and Q.e^G went out during chunk c - 1
            if constexpr (LA) {
                rest = c > cb;
                if (rest)
                    copy_chunk<K, V, OUT, COPYV, CW, 2>(oth, hrec + static_cast<size_t>(c + 1) * RB, vg, tc + kC, tend,
                                                        H, h, w, l);
            }
            if (!rest)
                copy_chunk<K, V, OUT, COPYV, CW>(oth, hrec + static_cast<size_t>(c + 1) * RB, vg, tc + kC, tend, H, h,
                                                 w, l);
        }
        if (TILE && c > cb) {
            if (EPI) {
                epi_store(fx, tc - kC);
            } else {
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    const int p = q * NT + tid, row = p / (2 * V / 16), pi = p % (2 * V / 16);
                    const int tok = tc - kC + row;
                    if (tok < tend)
                        store_stream(reinterpret_cast<u4 *>(og + (static_cast<size_t>(tok) * H + h) * V + pi * 8), pc[q]);
                }
            }
        }
        if (EPI && ep.z) {  // output gate of chunk c, used when its tile is stored
            const int tok = tc + erow;
            zq[0] = zq[1] = u4{0u, 0u, 0u, 0u};
            if (tok < tend) {
                const u4 *zp = reinterpret_cast<const u4 *>(ep.z + (static_cast<size_t>(tok) * H + h) * V + ecol);
                zq[0] = zp[0];
                zq[1] = zp[1];
            }
        }
        ChunkStep<K, V, NB, OUT, HASV> st;
        if (active) st.part_a(cur, fbc, S, cs, col0, l, r, g);
        if (TILE) wg_barrier();  // every wave has read K.e^G, Q.e^G and V of chunk c: the tile may go there
        if constexpr (LA) {
            if (c + 2 < ce && w < CW)
                copy_chunk<K, V, OUT, COPYV, CW, 1>(cur, hrec + static_cast<size_t>(c + 2) * RB, vg, tc + 2 * kC, tend, H,
                                                    h, w, l);
        }
        if (active) st.part_b(cur, fbc, S, cs, out, scale, g);
        if (OUT && active) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 16 * i + 4 * g + e, col = col0 + 16 * j + r;
                        if (EPI) {
                            *reinterpret_cast<float *>(ftb(cur) + ftile_off<V>(t, col)) = out[j][i][e];
                        } else if (TILE) {
                            *reinterpret_cast<bf16_t *>(cur + ScanBuf<K, V>::VT + VT::off(t, col)) =
                                bf16_rne(out[j][i][e]);
                        } else if (tc + t < tend) {
                            io<TOut>::store(og + (static_cast<size_t>(tc + t) * H + h) * V + col, out[j][i][e]);
                        }
                    }
        }
    };
    // two chunks per iteration, so that each buffer is a distinct LDS object: copies
    // into one never make reads of the other wait
    for (int c = cb; c < ce; c += 2) {
        body(lb0, fb0, lb1, c);
        if (c + 1 >= ce) break;
        body(lb1, fb1, lb0, c + 1);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)  // the state itself for the caller
#pragma unroll
        for (int ct = 0; ct < K / 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[j][ct][e] *= cs.sc[j];
    if (TILE) {
        wait_all();
        wg_barrier();
        char *last = ((ce - 1 - cb) & 1) ? lb1 : lb0;
        const int t0 = tbeg + (ce - 1 - cb) * kC;
        if (EPI) {
            f4 fx[4];
            epi_read(ftb(last), fx);
            epi_store(fx, t0);
        } else {
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                const int p = q * NT + tid, row = p / (2 * V / 16), pi = p % (2 * V / 16);
                const int tok = t0 + row;
                const u4 v = *reinterpret_cast<const u4 *>(last + ScanBuf<K, V>::VT + VT::off(row, pi * 8));
                if (tok < tend) store_stream(reinterpret_cast<u4 *>(og + (static_cast<size_t>(tok) * H + h) * V + pi * 8), v);
            }
        }
    }
}

// state slice of a wave: S[j][ct][e] = X[16 ct + 4g + e][col0 + 16 j + r] of a row-major
// d_k x ld matrix X (nullptr: zero)
template <int K, int NB>
__device__ __forceinline__ void load_state(f4 (&S)[NB][K / 16], const float *x, int ld, int col0, int r, int g) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int ct = 0; ct < K / 16; ++ct) S[j][ct] = zero4();
    if (!x) return;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int ct = 0; ct < K / 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[j][ct][e] = x[static_cast<size_t>(16 * ct + 4 * g + e) * ld + col0 + 16 * j + r];
}
template <int K, int NB>
__device__ __forceinline__ void store_state(const f4 (&S)[NB][K / 16], float *x, int ld, int col0, int r, int g) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int ct = 0; ct < K / 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[static_cast<size_t>(16 * ct + 4 * g + e) * ld + col0 + 16 * j + r] = S[j][ct][e];
}

// global segment s -> (sequence n, index gl inside it, segment count G of n)
struct SegInfo {
    int n, gl, G;
};
__device__ __forceinline__ SegInfo seg_of(const int32_t *soff, int N, int s) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (soff[mid] <= s) lo = mid; else hi = mid - 1;
    }
    return SegInfo{lo, s - soff[lo], soff[lo + 1] - soff[lo]};
}

// chunks [cb, ce) of a segment and its first token (the plan of chunk_offsets_kernel)
struct SegRange {
    int cb, ce, tbeg;
};
__device__ __forceinline__ SegRange seg_range(const PrefillArgs &a, const int32_t *off, const SegInfo &si, int L,
                                              int L0) {
    const int c0 = off[si.n], c1 = off[si.n + 1];
    int cb = c0, ce = c1;
    if (si.G > 1) {
        cb = si.gl == 0 ? c0 : c0 + L0 + (si.gl - 1) * L;
        ce = min(c1, si.gl == 0 ? c0 + L0 : cb + L);
    }
    return SegRange{cb, ce, a.cu_seqlens[si.n] + (cb - c0) * kC};
}

// initial / final state of sequence n, head h: [N, H, d_k, d_v] arrays, or slot
// caches when slots are given (a negative slot: zero initial state, no final state)
__device__ __forceinline__ const float *state_in(const PrefillArgs &a, int n, int h) {
    const int slot = a.slots ? a.slots[n] : n;
    return (a.s0 && slot >= 0) ? a.s0 + (static_cast<size_t>(slot) * a.H + h) * a.K * a.V : nullptr;
}
__device__ __forceinline__ float *state_out(const PrefillArgs &a, int n, int h) {
    const int slot = a.slots ? a.slots[n] : n;
    return (a.sT && slot >= 0) ? a.sT + (static_cast<size_t>(slot) * a.H + h) * a.K * a.V : nullptr;
}

struct SegBufs {
    float *sin;   // [segments, H, d_k, d_v] incoming state of each segment
    float *mapm;  // [segments, H, d_k, d_k] M of middle segments
    float *mapn;  // [segments, H, d_k, d_v] N of middle segments
};

// One workgroup per (segment, head), (d_k + d_v) / 32 waves of 32 columns (two
// 16-column blocks, so that every fragment read from LDS serves both): the first
// d_k / 32 waves carry M (from the identity, V = 0) of a middle segment (and idle
// on segment 0 when d_k != d_v), and issue all the chunk copies (their products are the lighter ones:
// letting every wave copy makes the pass slower); the others carry N (from zero), or
// on segment 0 the state from the initial state.
// With d_k = d_v (SEG0OUT), segment 0 is shorter than the others and its workgroup
// runs the output pass of segment 0 instead (the workgroup then has the output
// pass's d_v / 16 waves): its incoming state is known, so its outputs need not wait
// for the prefix, and the output pass that follows has one segment fewer per
// sequence. Its end state is the incoming state of segment 1 either way.
constexpr int kSegNB = 2;  // 16-column blocks per wave in the map pass
template <int K, int V, typename TOut, bool EPI>
__global__ __launch_bounds__(64 * (K + V) / (16 * kSegNB)) void seg_kernel(PrefillArgs a, const int32_t *off,
                                                                           const int32_t *soff, int L, int L0,
                                                                           const char *recs, SegBufs sb) {
    constexpr int NB = kSegNB, NW = (K + V) / (16 * NB), WM = K / (16 * NB);
    constexpr bool SEG0OUT = K == V;
    __shared__ __attribute__((aligned(16))) char lb0[ScanBuf<K, V>::BYTES];
    __shared__ __attribute__((aligned(16))) char lb1[ScanBuf<K, V>::BYTES];
    const int H = a.H;
    const int s = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (s >= soff[a.N]) return;
    const SegInfo si = seg_of(soff, a.N, s);
    if (si.gl >= si.G - 1) return;    // the last segment has no successor
    const int tid = threadIdx.x, l = tid & 63, r = l & 15, g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const SegRange sr = seg_range(a, off, si, L, L0);
    const int tend = a.cu_seqlens[si.n + 1];
    const char *hrec = recs + static_cast<size_t>(h) * a_nc(a) * Rec<K>::BYTES;
    const bf16_t *vg = static_cast<const bf16_t *>(a.v);
    const size_t skv = (static_cast<size_t>(s) * H + h) * K * V;
    if constexpr (SEG0OUT) {
        if (si.gl == 0) {
            constexpr int OW = V / 16;
            static_assert(OW == NW, "the output pass's waves are the map pass's");
            static_assert(static_cast<size_t>(kC) * V * 4 <= Rec<K>::YT, "the fp32 epilogue tile fits a buffer");
            f4 S1[1][K / 16];
            const int col0 = 16 * w;
            load_state<K, 1>(S1, state_in(a, si.n, h), V, col0, r, g);
            const Epi ep{static_cast<const bf16_t *>(a.z), a.nw, a.eps, a.norm, a.zact};
            run_segment<K, V, 1, true, true, true, OW, OW, EPI, TOut>(lb0, lb1, nullptr, S1, hrec, sr.cb, sr.ce,
                                                                      sr.tbeg, tend, vg, static_cast<TOut *>(a.o), H,
                                                                      h, a.scale, ep, true, tid, w, l, r, g, col0);
            store_state<K, 1>(S1, sb.sin + skv + static_cast<size_t>(H) * K * V, V, col0, r, g);
            return;
        }
    }
    f4 S[NB][K / 16];
    if (w < WM) {
        const int col0 = 16 * NB * w;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int ct = 0; ct < K / 16; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[j][ct][e] = (16 * ct + 4 * g + e == col0 + 16 * j + r) ? 1.f : 0.f;
        run_segment<K, V, NB, false, false, true, NW, WM, false, float>(lb0, lb1, nullptr, S, hrec, sr.cb, sr.ce,
                                                                        sr.tbeg, tend, vg, nullptr, H, h, 1.f, Epi{},
                                                                        si.gl > 0, tid, w, l, r, g, col0);
        if (si.gl > 0) store_state<K, NB>(S, sb.mapm + (static_cast<size_t>(s) * H + h) * K * K, K, col0, r, g);
    } else {
        const int col0 = 16 * NB * (w - WM);
        const float *init = si.gl == 0 ? state_in(a, si.n, h) : nullptr;
        load_state<K, NB>(S, init, V, col0, r, g);
        run_segment<K, V, NB, false, true, true, NW, WM, false, float>(lb0, lb1, nullptr, S, hrec, sr.cb, sr.ce,
                                                                       sr.tbeg, tend, vg, nullptr, H, h, 1.f, Epi{},
                                                                       true, tid, w, l, r, g, col0);
        store_state<K, NB>(S, si.gl == 0 ? sb.sin + skv + static_cast<size_t>(H) * K * V : sb.mapn + skv, V, col0, r,
                           g);
    }
}

// For a sequence cut into several segments when d_k != d_v (segment 0 then goes
// through the output pass): a copy of its initial state (zeros without one) as the
// incoming state of its segment 0, which the output pass reads. The output pass
// writes final states (which may alias the initial states) while other segments of
// it still run, so segment 0 reads this copy.
// Each state is copied by kSeedParts workgroups, so that a few long sequences still
// spread the copies over many compute units.
constexpr int kSeedParts = 16;
template <int K, int V>
__global__ __launch_bounds__(256) void seed_kernel(PrefillArgs a, const int32_t *soff, SegBufs sb) {
    constexpr int NQ = K * V / 4, PQ = NQ / kSeedParts;  // float4 per state, per part
    static_assert(NQ % kSeedParts == 0, "whole parts");
    const int item = blockIdx.x / kSeedParts, part = blockIdx.x - item * kSeedParts;
    const int n = item / a.H, h = item - (item / a.H) * a.H;
    if (n >= a.N || soff[n + 1] - soff[n] < 2) return;
    const float4 *src = reinterpret_cast<const float4 *>(state_in(a, n, h));
    float4 *dst = reinterpret_cast<float4 *>(sb.sin + (static_cast<size_t>(soff[n]) * a.H + h) * K * V);
    for (int i = part * PQ + static_cast<int>(threadIdx.x); i < (part + 1) * PQ; i += 256)
        dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

// S_in(g + 1) = M_g S_in(g) + N_g for the middle segments g of one (sequence, head),
// 16 state columns per workgroup, in fp32 (16x16x4 fp32 MFMAs: exact products,
// fp32 sums). Wave w computes rows 16w .. 16w + 15 of the tile: lane (r, q) feeds
// row 16w + r of M over the columns K/4 q .. K/4 (q + 1) - 1 as A operands, loaded
// one step ahead, and the same rows of the tile (transposed in LDS) as B operands;
// the accumulator starts from N_g. The steps are sequential, so the time per step
// is one chain of K/4 MFMAs and one barrier.
// Workgroups go to the 8 XCDs in turn (workgroup b to XCD b % 8), and the d_v / 16
// tiles of one (sequence, head) all read its whole M_g at every step, so they are
// placed on one XCD to share its L2: (sequence, head) u = 8 (b / 8 / NV) + b % 8,
// tile (b / 8) % NV.
constexpr int kXcds = 8;
template <int K, int V>
__global__ __launch_bounds__(64 * K / 16) void prefix_kernel(const int32_t *soff, int N, int H, SegBufs sb) {
    constexpr int NV = V / 16, KQ = K / 4, NT = 64 * K / 16;
    __shared__ __attribute__((aligned(16))) float xt[2][16][K + 4];  // the tile, [buffer][column][row]
    const int b = blockIdx.x, xi = b / kXcds, vt = xi % NV, nh = (xi / NV) * kXcds + b % kXcds;
    const int n = nh / H, h = nh - (nh / H) * H;
    if (n >= N) return;
    const int s0 = soff[n], G = soff[n + 1] - s0;
    if (G < 3) return;
    const int tid = threadIdx.x, l = tid & 63, r = l & 15, q = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t kv = static_cast<size_t>(K) * V;
    const int c0 = 16 * vt;
    static_assert(NT == 4 * K, "one float4 of the K x 16 tile per thread");
    {  // S_in(1): row tid / 4, columns 4 (tid % 4) .. + 3
        const int row = tid >> 2, cq = 4 * (tid & 3);
        const float4 v = *reinterpret_cast<const float4 *>(sb.sin + (static_cast<size_t>(s0 + 1) * H + h) * kv +
                                                          static_cast<size_t>(row) * V + c0 + cq);
        xt[0][cq][row] = v.x;
        xt[0][cq + 1][row] = v.y;
        xt[0][cq + 2][row] = v.z;
        xt[0][cq + 3][row] = v.w;
    }
    const int mrow = 16 * w + r;
    // operands of step gl: M_gl row mrow, columns KQ q ..; N_gl rows 16w + 4q + e, column c0 + r
    auto load_step = [&](float4 (&am)[KQ / 4], f4 &an, int gl) {
        const float4 *mg = reinterpret_cast<const float4 *>(
            sb.mapm + (static_cast<size_t>(s0 + gl) * H + h) * K * K + static_cast<size_t>(mrow) * K + KQ * q);
#pragma unroll
        for (int j = 0; j < KQ / 4; ++j) am[j] = mg[j];
        const float *ng = sb.mapn + (static_cast<size_t>(s0 + gl) * H + h) * kv + c0 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) an[e] = ng[static_cast<size_t>(16 * w + 4 * q + e) * V];
    };
    auto step = [&](const float4 (&am)[KQ / 4], f4 y, int gl, int cur) {
        const float4 *xb = reinterpret_cast<const float4 *>(&xt[cur][r][KQ * q]);
#pragma unroll
        for (int j = 0; j < KQ / 4; ++j) {
            const float4 x = xb[j];
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(am[j].x, x.x, y, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(am[j].y, x.y, y, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(am[j].z, x.z, y, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(am[j].w, x.w, y, 0, 0, 0);
        }
        // y[e] = S_in(gl + 1)[16w + 4q + e][c0 + r]
        float *dst = sb.sin + (static_cast<size_t>(s0 + gl + 1) * H + h) * kv + c0 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[static_cast<size_t>(16 * w + 4 * q + e) * V] = y[e];
        *reinterpret_cast<f4 *>(&xt[cur ^ 1][r][16 * w + 4 * q]) = y;
        __syncthreads();
    };
    // two register sets in turn: the loads of the next step overlap the current one
    float4 m0[KQ / 4], m1[KQ / 4];
    f4 n0, n1;
    load_step(m0, n0, 1);
    __syncthreads();
    for (int gl = 1; gl <= G - 2; gl += 2) {
        load_step(m1, n1, min(gl + 1, G - 2));
        step(m0, n0, gl, 0);
        if (gl + 1 > G - 2) break;
        load_step(m0, n0, min(gl + 2, G - 2));
        step(m1, n1, gl + 1, 1);
    }
}

template <int K, int V, typename TOut, bool EPI>
__global__ __launch_bounds__(64 * V / 16) void out_kernel(PrefillArgs a, const int32_t *off, const int32_t *soff,
                                                          int L, int L0, const char *recs, SegBufs sb) {
    constexpr int NB = 1, NW = V / 16;
    // the fp32 epilogue tile goes into the K.e^G / Q.e^G region of a chunk buffer when it fits
    constexpr bool FTD = EPI && static_cast<size_t>(kC) * V * 4 > Rec<K>::YT;
    __shared__ __attribute__((aligned(16))) char lb0[ScanBuf<K, V>::BYTES];
    __shared__ __attribute__((aligned(16))) char lb1[ScanBuf<K, V>::BYTES];
    __shared__ __attribute__((aligned(16))) char ftd[FTD ? kC * V * 4 : 16];
    const int H = a.H;
    const int s = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
    if (s >= soff[a.N]) return;
    const SegInfo si = seg_of(soff, a.N, s);
    if (K == V && si.G > 1 && si.gl == 0) return;  // segment 0's outputs came from the map pass
    const int tid = threadIdx.x, l = tid & 63, r = l & 15, g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col0 = 16 * NB * w;
    const SegRange sr = seg_range(a, off, si, L, L0);
    const int cb = sr.cb, ce = sr.ce, tbeg = sr.tbeg, tend = a.cu_seqlens[si.n + 1];
    f4 S[NB][K / 16];
    const float *init = si.G == 1 ? state_in(a, si.n, h) : sb.sin + (static_cast<size_t>(s) * H + h) * K * V;
    load_state<K, NB>(S, init, V, col0, r, g);
    const Epi ep{static_cast<const bf16_t *>(a.z), a.nw, a.eps, a.norm, a.zact};
    run_segment<K, V, NB, true, true, true, NW, NW, EPI, TOut>(
        lb0, lb1, FTD ? ftd : nullptr, S, recs + static_cast<size_t>(h) * a_nc(a) * Rec<K>::BYTES, cb, ce, tbeg, tend,
        static_cast<const bf16_t *>(a.v), static_cast<TOut *>(a.o), H, h, a.scale, ep, true, tid, w, l, r, g, col0);
    if (si.gl == si.G - 1) {
        float *fin = state_out(a, si.n, h);
        if (fin) store_state<K, NB>(S, fin, V, col0, r, g);
    }
}

// Compute units of the current device, queried once per device (relaxed atomics:
// threads that race on a first query store the same value).
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Segment plan. With d_k = d_v the map pass also runs the output pass of each
// sequence's segment 0 (seg_kernel), at about 0.6 of the map pass's rate per chunk
// (4.2 against 2.6 us per chunk at 128K tokens), so segment 0 gets 5/8 of the
// others' L chunks and both passes then take about L chunks' time.
constexpr int kSeg0Eighths = 5;
int seg0_chunks(int L, bool seg0out) { return seg0out ? std::max(1, kSeg0Eighths * L / 8) : L; }

// Chunks per segment: enough segments to give every compute unit a (segment,
// head) in each state pass for one long sequence at this size (with segment 0
// counted at its shorter length), and at least 16 chunks each. KDA_SEG_CHUNKS
// overrides it (tests of the segment bookkeeping at small sizes), up to the chunk count.
int seg_chunks(int32_t N, int32_t T, int32_t H, bool seg0out) {
    const int64_t nc = (static_cast<int64_t>(T) + kC - 1) / kC + N;
    if (const char *e = std::getenv("KDA_SEG_CHUNKS")) {
        const int v = std::atoi(e);
        if (v >= 1) return static_cast<int>(std::min<int64_t>(v, nc));
    }
    // (G - 1) segments of L and one of 5 L / 8 per long sequence, G - 1 = 256 / H
    const int64_t den = 8 * 256 + (seg0out ? kSeg0Eighths * static_cast<int64_t>(H) : 0);
    return static_cast<int>(std::max<int64_t>(16, (8 * nc * H + den - 1) / den));
}

template <int K, int V>
struct WsLayout {
    int L, L0;
    size_t nc, nseg, off, soff, recs, sin, mapn, mapm, bytes;
    WsLayout(int32_t N, int32_t T, int32_t H) {
        L = seg_chunks(N, T, H, K == V);
        L0 = seg0_chunks(L, K == V);
        nc = static_cast<size_t>((static_cast<int64_t>(T) + kC - 1) / kC) + N;
        // sum over sequences of ceil(chunks / L), plus one for each sequence longer than L
        nseg = (nc + L - 1) / L + N + std::min<size_t>(N, (nc + L - 1) / L);
        off = 0;
        soff = align256(static_cast<size_t>(N + 1) * 4);
        recs = soff + align256(static_cast<size_t>(N + 1) * 4);
        sin = recs + nc * H * Rec<K>::BYTES;
        mapn = sin + nseg * H * K * V * 4;
        mapm = mapn + nseg * H * K * V * 4;
        bytes = mapm + nseg * H * K * K * 4;
    }
};

template <int K, int V>
hipError_t launch_out(const PrefillArgs &a, const int32_t *off, const int32_t *soff, int L, int L0, const char *recs,
                      const SegBufs &sb, size_t units, hipStream_t st) {
    const dim3 og(static_cast<unsigned>(units)), ob(64 * V / 16);
    const bool epi = a.norm || a.z;
    if (a.out_dtype == KDA_BF16) {
        if (epi) hipLaunchKernelGGL((out_kernel<K, V, bf16_t, true>), og, ob, 0, st, a, off, soff, L, L0, recs, sb);
        else hipLaunchKernelGGL((out_kernel<K, V, bf16_t, false>), og, ob, 0, st, a, off, soff, L, L0, recs, sb);
    } else {
        if (epi) hipLaunchKernelGGL((out_kernel<K, V, float, true>), og, ob, 0, st, a, off, soff, L, L0, recs, sb);
        else hipLaunchKernelGGL((out_kernel<K, V, float, false>), og, ob, 0, st, a, off, soff, L, L0, recs, sb);
    }
    return hipGetLastError();
}

// the map pass; with d_k = d_v it also writes segment 0's outputs (output type and epilogue)
template <int K, int V>
hipError_t launch_seg(const PrefillArgs &a, const int32_t *off, const int32_t *soff, int L, int L0, const char *recs,
                      const SegBufs &sb, size_t units, hipStream_t st) {
    const dim3 gg(static_cast<unsigned>(units)), gb(64 * (K + V) / (16 * kSegNB));
    const bool epi = a.norm || a.z;
    if constexpr (K == V) {
        if (a.out_dtype == KDA_BF16) {
            if (epi) hipLaunchKernelGGL((seg_kernel<K, V, bf16_t, true>), gg, gb, 0, st, a, off, soff, L, L0, recs, sb);
            else hipLaunchKernelGGL((seg_kernel<K, V, bf16_t, false>), gg, gb, 0, st, a, off, soff, L, L0, recs, sb);
        } else {
            if (epi) hipLaunchKernelGGL((seg_kernel<K, V, float, true>), gg, gb, 0, st, a, off, soff, L, L0, recs, sb);
            else hipLaunchKernelGGL((seg_kernel<K, V, float, false>), gg, gb, 0, st, a, off, soff, L, L0, recs, sb);
        }
    } else {
        (void)epi;
        hipLaunchKernelGGL((seg_kernel<K, V, float, false>), gg, gb, 0, st, a, off, soff, L, L0, recs, sb);
    }
    return hipGetLastError();
}

template <int K, int V>
hipError_t launch_kv(const PrefillArgs &a, hipStream_t st) {
    const WsLayout<K, V> lay(a.N, a.T, a.H);
    char *ws = static_cast<char *>(a.ws);
    int32_t *off = reinterpret_cast<int32_t *>(ws + lay.off);
    int32_t *soff = reinterpret_cast<int32_t *>(ws + lay.soff);
    char *recs = ws + lay.recs;
    const SegBufs sb{reinterpret_cast<float *>(ws + lay.sin), reinterpret_cast<float *>(ws + lay.mapm),
                     reinterpret_cast<float *>(ws + lay.mapn)};
    hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(256), 0, st, a.cu_seqlens, a.N, lay.L, lay.L0, off, soff);
    if (a.T > 0) {
        const size_t items = lay.nc * a.H;
        const size_t wgs = std::min(items, static_cast<size_t>(kPrepWgsPerCu) * cu_count());
        if (a.gx)
            hipLaunchKernelGGL((prep_kernel<K, true>), dim3(static_cast<unsigned>(wgs)), dim3(256), 0, st, a, off,
                               recs);
        else
            hipLaunchKernelGGL((prep_kernel<K, false>), dim3(static_cast<unsigned>(wgs)), dim3(256), 0, st, a, off,
                               recs);
    }
    // every sequence has at most ceil(T / 64) chunks: one segment if that fits in L
    const int64_t maxc = (static_cast<int64_t>(a.T) + kC - 1) / kC;
    const size_t units = lay.nseg * a.H;
    if (maxc <= lay.L) return launch_out<K, V>(a, off, soff, lay.L, lay.L0, recs, sb, units, st);

    if (K != V)
        hipLaunchKernelGGL((seed_kernel<K, V>), dim3(static_cast<unsigned>(a.N) * a.H * kSeedParts), dim3(256), 0, st,
                           a, soff, sb);
    const hipError_t e = launch_seg<K, V>(a, off, soff, lay.L, lay.L0, recs, sb, units, st);
    if (e != hipSuccess) return e;
    if (maxc > static_cast<int64_t>(lay.L0) + lay.L)  // some sequence has three or more segments
        hipLaunchKernelGGL((prefix_kernel<K, V>),
                           dim3(static_cast<unsigned>((static_cast<int64_t>(a.N) * a.H + kXcds - 1) / kXcds) * kXcds *
                                (V / 16)),
                           dim3(64 * K / 16), 0, st, soff, a.N, a.H, sb);
    return launch_out<K, V>(a, off, soff, lay.L, lay.L0, recs, sb, units, st);
}

// Workspace of kda_chunk_fwd_ex_noalloc. In host code this name is the runtime's
// stand-in for the device array, not a device address: only the address from
// hipGetSymbolAddress (taken per device, below) goes to kernels.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

}  // namespace

void *noalloc_scratch() {
    static std::atomic<void *> addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        // with `dev` current: each GPU holds its own copy of the array at its own address
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev].store(p, std::memory_order_release);
    }
    return p;
}

size_t prefill_mfma_workspace(int32_t N, int32_t T, int32_t H, int32_t K, int32_t V) {
    if (K == 128 && V == 128) return WsLayout<128, 128>(N, T, H).bytes;
    if (K == 128 && V == 64) return WsLayout<128, 64>(N, T, H).bytes;
    if (K == 64 && V == 128) return WsLayout<64, 128>(N, T, H).bytes;
    return WsLayout<64, 64>(N, T, H).bytes;
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t st) {
    if (a.K == 128 && a.V == 128) return launch_kv<128, 128>(a, st);
    if (a.K == 128 && a.V == 64) return launch_kv<128, 64>(a, st);
    if (a.K == 64 && a.V == 128) return launch_kv<64, 128>(a, st);
    return launch_kv<64, 64>(a, st);
}

}  // namespace kda
