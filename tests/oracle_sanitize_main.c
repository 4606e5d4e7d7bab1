/*
 * Driver for the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (host code only; built and run by tests/test_oracle_sanitizers.py). Every
 * buffer is a heap allocation of exactly the size the oracle's interface
 * states, so a read or write past any of them is reported.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_prefill(const float *q, const float *k, const float *v, const float *log_alpha, const float *beta,
                       const int32_t *cu_seqlens, int32_t N, int32_t H, int32_t K, int32_t V, double scale,
                       const float *initial_state, double *o, double *final_state, int32_t nthreads);
int kda_oracle_decode(const float *q, const float *k, const float *v, const float *log_alpha, const float *beta,
                      double *state, const int32_t *slot_idx, int32_t B, int32_t H, int32_t K, int32_t V,
                      int32_t num_slots, double scale, double *o, int32_t nthreads);

static uint32_t lcg = 12345u;
static float unit(void) { /* uniform in (-1, 1) */
    lcg = lcg * 1664525u + 1013904223u;
    return (float)((double)(lcg >> 8) / 8388608.0 - 1.0);
}
static float *fill(size_t n, float lo, float hi) {
    float *x = malloc(sizeof(float) * n);
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * 0.5f * (unit() + 1.0f);
    return x;
}

int main(void) {
    /* three sequences, one empty, the last spanning a partial column block (V = 33) */
    const int32_t N = 3, H = 2, K = 4, V = 33;
    const int32_t cu[4] = {0, 5, 5, 75};
    const int32_t T = cu[N];
    float *q = fill((size_t)T * H * K, -1.f, 1.f), *k = fill((size_t)T * H * K, -1.f, 1.f);
    float *v = fill((size_t)T * H * V, -1.f, 1.f);
    float *g = fill((size_t)T * H * K, -0.5f, 0.f), *b = fill((size_t)T * H, 0.f, 1.f);
    float *s0 = fill((size_t)N * H * K * V, -0.1f, 0.1f);
    double *o = malloc(sizeof(double) * (size_t)T * H * V);
    double *sT = malloc(sizeof(double) * (size_t)N * H * K * V);
    if (kda_oracle_prefill(q, k, v, g, b, cu, N, H, K, V, 0.5, s0, o, sT, 2) != 0) return 1;
    if (kda_oracle_prefill(q, k, v, g, b, cu, N, H, K, V, 1.0, NULL, o, NULL, 1) != 0) return 2;
    const int32_t bad[4] = {0, 5, 4, 75}; /* decreasing: rejected before anything is written */
    if (kda_oracle_prefill(q, k, v, g, b, bad, N, H, K, V, 1.0, NULL, o, NULL, 1) != -1) return 3;

    /* decode: two sequences into slots 3 and 0 of a four-slot cache */
    const int32_t B = 2, slots = 4;
    const int32_t slot_idx[2] = {3, 0};
    double *state = malloc(sizeof(double) * (size_t)slots * H * K * V);
    for (size_t i = 0; i < (size_t)slots * H * K * V; ++i) state[i] = 0.01 * unit();
    double *od = malloc(sizeof(double) * (size_t)B * H * V);
    if (kda_oracle_decode(q, k, v, g, b, state, slot_idx, B, H, K, V, slots, 1.0, od, 2) != 0) return 4;
    const int32_t out_of_range[2] = {4, 0};
    if (kda_oracle_decode(q, k, v, g, b, state, out_of_range, B, H, K, V, slots, 1.0, od, 1) != -1) return 5;

    double sum = 0.0;
    for (size_t i = 0; i < (size_t)T * H * V; ++i) sum += fabs(o[i]);
    for (size_t i = 0; i < (size_t)B * H * V; ++i) sum += fabs(od[i]);
    printf("checksum %.6f\n", sum);
    free(q); free(k); free(v); free(g); free(b); free(s0); free(o); free(sT); free(state); free(od);
    return isfinite(sum) ? 0 : 6;
}
