/*
 * kda_oracle.c -- plain, slow, fp64 CPU evaluation of Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE. This file is the correctness oracle that the HIP
 * library is compared against. Only the test-suite, the package smoke check
 * and the CPU-baseline leg of the benchmark may load it. It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes, for every sequence n and head h on its own
 * (row i of S belongs to key channel i, column j to value channel j):
 *
 *     S = initial state of (n, h), or the K x V zero matrix
 *     for every token t of sequence n, in order:
 *         S'  = Diag(exp(g_t)) S           decay: row i scaled by alpha_t[i]
 *         u   = beta_t (v_t - S'^T k_t)    prediction error on the decayed state
 *         S   = S' + k_t u^T               rank-1 delta-rule write
 *         o_t = scale * S^T q_t            read-out from the updated state
 *     final state of (n, h) = S
 *
 * Sources (the web pages on Kimi Delta Attention):
 *  - "Kimi Linear爆发背后的秘密：重新定义长上下文推理效率" (xugj520.cn), section
 *    "Kimi Delta Attention的技术内核": the recurrence
 *    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T.
 *  - 2025 attention/MoE architecture review (lanjinlin.com.cn), section
 *    "GatedDeltaNet解读": the expansion S_{t-1}alpha_t + beta_t k_t (v_t -
 *    S_{t-1}alpha_t k_t) of the gated delta rule and its per-token loop
 *    (decay the state by exp(g_t) first, form the value correction against
 *    the decayed state, add the rank-1 update, read the output from the
 *    updated state, save the final state). The same page, section "KLA",
 *    gives o_t = S_t^T q_t and makes the gate channel-wise, Diag(alpha_t).
 *  - "线性注意力机制Kimi Linear架构解析与优化实践" (coreui.cn), section 2.1: alpha is
 *    per key channel (B, H, D_k), beta one scalar per head (B, H, 1). The
 *    gate enters as log alpha (natural log), as in its section 4.2.
 *
 * Expanding the matrix form gives exactly the four lines above:
 * (I - b k k^T) S' + b k v^T = S' + k (b (v - S'^T k))^T.
 *
 * Arithmetic: every input is read from fp32 containers (bf16 and fp32 values
 * are exact in fp32) and converted to double; all arithmetic is fp64, in the
 * order written above, with libm's exp. Outputs are fp64.
 *
 * Parallelism: the work is split over (sequence, head, block of value
 * columns). Column j of S obeys its own recurrence given (k, alpha, beta),
 * so the split changes no arithmetic of any output element.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_COLS 32 /* value columns per task */

/* One (sequence, head, column block) task over tokens [t0, t1). */
static void oracle_task(const float *q, const float *k, const float *v,
                        const float *g, const float *beta, int64_t t0,
                        int64_t t1, int h, int H, int K, int V, int j0, int nj,
                        double scale, const float *s0, /* K x V of (n,h) or NULL */
                        double *o,                     /* [T_total, H, V] */
                        double *sfin,                  /* K x V of (n,h) or NULL */
                        double *S,                     /* scratch nj x K (column-major) */
                        double *alpha, double *kk, double *qq)
{
    for (int j = 0; j < nj; ++j)
        for (int i = 0; i < K; ++i)
            S[(size_t)j * K + i] = s0 ? (double)s0[(size_t)i * V + j0 + j] : 0.0;

    for (int64_t t = t0; t < t1; ++t) {
        const size_t bk = ((size_t)t * H + h) * (size_t)K;
        const size_t bv = ((size_t)t * H + h) * (size_t)V;
        const double b = (double)beta[(size_t)t * H + h];
        for (int i = 0; i < K; ++i) {
            alpha[i] = exp((double)g[bk + i]);
            kk[i] = (double)k[bk + i];
            qq[i] = (double)q[bk + i];
        }
        for (int j = 0; j < nj; ++j) {
            double *s = S + (size_t)j * K;
            /* S' = Diag(alpha_t) S */
            for (int i = 0; i < K; ++i)
                s[i] = alpha[i] * s[i];
            /* r = (S'^T k_t)_j */
            double r = 0.0;
            for (int i = 0; i < K; ++i)
                r += s[i] * kk[i];
            /* u_j = beta_t (v_t[j] - r) */
            const double u = b * ((double)v[bv + j0 + j] - r);
            /* S = S' + k_t u^T */
            for (int i = 0; i < K; ++i)
                s[i] = s[i] + kk[i] * u;
            /* o_t[j] = scale * (S^T q_t)_j */
            double acc = 0.0;
            for (int i = 0; i < K; ++i)
                acc += s[i] * qq[i];
            o[bv + j0 + j] = scale * acc;
        }
    }
    if (sfin)
        for (int j = 0; j < nj; ++j)
            for (int i = 0; i < K; ++i)
                sfin[(size_t)i * V + j0 + j] = S[(size_t)j * K + i];
}

/*
 * Prefill over packed variable-length sequences.
 *   q, k, log_alpha : [T_total, H, K]   (fp32 containers)
 *   v               : [T_total, H, V]
 *   beta            : [T_total, H]
 *   cu_seqlens      : [N + 1] host array, 0 = cu[0] <= cu[1] <= ... <= cu[N] = T_total
 *   initial_state   : [N, H, K, V] or NULL (zeros)
 *   o               : [T_total, H, V] fp64 output
 *   final_state     : [N, H, K, V] fp64 output, or NULL
 *   nthreads        : OpenMP threads, <= 0 for the runtime default
 * Returns 0 on success, -1 on invalid arguments (nothing is written then).
 */
int kda_oracle_prefill(const float *q, const float *k, const float *v,
                       const float *log_alpha, const float *beta,
                       const int32_t *cu_seqlens, int32_t N, int32_t H,
                       int32_t K, int32_t V, double scale,
                       const float *initial_state, double *o,
                       double *final_state, int32_t nthreads)
{
    if (!cu_seqlens || N < 1 || H < 1 || K < 1 || V < 1 || !o)
        return -1;
    if (cu_seqlens[0] != 0)
        return -1;
    for (int32_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -1;
    const int64_t T_total = cu_seqlens[N];
    if (T_total > 0 && (!q || !k || !v || !log_alpha || !beta))
        return -1;

    const int nblk = (V + ORACLE_COLS - 1) / ORACLE_COLS;
    const int64_t ntask = (int64_t)N * H * nblk;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)K * ORACLE_COLS);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)K * 3);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t task = 0; task < ntask; ++task) {
            const int blk = (int)(task % nblk);
            const int h = (int)((task / nblk) % H);
            const int n = (int)(task / ((int64_t)nblk * H));
            const int j0 = blk * ORACLE_COLS;
            const int nj = (V - j0) < ORACLE_COLS ? (V - j0) : ORACLE_COLS;
            const size_t sofs = ((size_t)n * H + h) * (size_t)K * V;
            oracle_task(q, k, v, log_alpha, beta, cu_seqlens[n],
                        cu_seqlens[n + 1], h, H, K, V, j0, nj, scale,
                        initial_state ? initial_state + sofs : NULL, o,
                        final_state ? final_state + sofs : NULL, S, alpha,
                        alpha + K, alpha + 2 * K);
        }
        free(S);
        free(alpha);
    }
    return 0;
}

/*
 * One decode step: the same token update applied to a state cache in place.
 *   q, k, log_alpha : [B, H, K];  v : [B, H, V];  beta : [B, H]
 *   state           : [num_slots, H, K, V] fp64, updated in place
 *   slot_idx        : [B] host array of distinct slots, or NULL (b -> b)
 *   o               : [B, H, V] fp64 output
 * Returns 0 on success, -1 on invalid arguments (nothing is written then).
 */
int kda_oracle_decode(const float *q, const float *k, const float *v,
                      const float *log_alpha, const float *beta, double *state,
                      const int32_t *slot_idx, int32_t B, int32_t H, int32_t K,
                      int32_t V, int32_t num_slots, double scale, double *o,
                      int32_t nthreads)
{
    if (!q || !k || !v || !log_alpha || !beta || !state || !o || B < 1 ||
        H < 1 || K < 1 || V < 1 || num_slots < 1)
        return -1;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t s = slot_idx ? slot_idx[b] : b;
        if (s < 0 || s >= num_slots)
            return -1;
    }
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *alpha = (double *)malloc(sizeof(double) * (size_t)K);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
            const int32_t b = (int32_t)(bh / H), h = (int32_t)(bh % H);
            const int32_t slot = slot_idx ? slot_idx[b] : b;
            double *S = state + ((size_t)slot * H + h) * (size_t)K * V;
            const size_t bk = (size_t)bh * K, bv = (size_t)bh * V;
            const double bt = (double)beta[bh];
            for (int i = 0; i < K; ++i)
                alpha[i] = exp((double)log_alpha[bk + i]);
            for (int j = 0; j < V; ++j) {
                /* S' = Diag(alpha) S, column j; r = (S'^T k)_j */
                double r = 0.0;
                for (int i = 0; i < K; ++i) {
                    const double sd = alpha[i] * S[(size_t)i * V + j];
                    S[(size_t)i * V + j] = sd;
                    r += sd * (double)k[bk + i];
                }
                /* u_j = beta (v_j - r);  S = S' + k u^T;  o_j = scale (S^T q)_j */
                const double u = bt * ((double)v[bv + j] - r);
                double acc = 0.0;
                for (int i = 0; i < K; ++i) {
                    const double sn = S[(size_t)i * V + j] + (double)k[bk + i] * u;
                    S[(size_t)i * V + j] = sn;
                    acc += sn * (double)q[bk + i];
                }
                o[bv + j] = scale * acc;
            }
        }
        free(alpha);
    }
    return 0;
}
