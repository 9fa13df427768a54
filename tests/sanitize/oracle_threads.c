/*
 * oracle_threads.c -- thread-pool check of the fp64 oracle, built with a sanitizer.
 *
 * Test infrastructure: compiled together with oracle/gdn_oracle.c by
 * tests/test_sanitizers.py (gcc -fsanitize=thread, or address+undefined) and run as
 * a plain executable, so the sanitizer runtime instruments the whole process.
 *
 * It runs prefill (from a nonzero S0) and replay on a small ragged batch with one
 * thread and with eight, and requires the results to be bit-identical: every
 * (sequence, v-head) chain is sequential, so the thread count cannot change them.
 * Inputs come from a fixed 64-bit LCG (only test data; none of the method's math).
 * Exit status 0 = pass; any other value, or a sanitizer report, = fail.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn_oracle_prefill(int64_t n_seqs, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                       const double *q, const double *k, const double *v, const double *g,
                       const double *beta, const int64_t *cu_seqlens, const double *S0,
                       double scale, double *S_out, double *o_out, int32_t n_threads);
int gdn_oracle_replay(int64_t n_seqs, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                      const double *q, const double *k, const double *v, const double *g,
                      const double *beta, const int64_t *cu_seqlens, const int64_t *r,
                      double scale, double *S_out, double *o_out, int32_t n_threads);

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;

static double uniform(void)   /* [-1, 1) */
{
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg_state >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static double *fill(size_t n, double lo, double hi)
{
    double *p = malloc(n * sizeof(double));
    if (!p) exit(3);
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (uniform() + 1.0);
    return p;
}

int main(void)
{
    enum { N = 5, HQK = 2, HV = 4, DK = 8, DV = 6 };
    const int64_t lens[N] = {0, 1, 17, 40, 9};
    int64_t cu[N + 1] = {0}, r[N];
    for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + lens[n];
    const int64_t T = cu[N];
    int64_t T_out = 0;
    for (int n = 0; n < N; ++n) { r[n] = lens[n] / 2 + (n & 1); if (r[n] > lens[n]) r[n] = lens[n]; T_out += r[n]; }

    double *q = fill((size_t)T * HQK * DK, -1, 1), *k = fill((size_t)T * HQK * DK, -0.4, 0.4);
    double *v = fill((size_t)T * HV * DV, -1, 1), *g = fill((size_t)T * HV, -0.5, 0.0);
    double *beta = fill((size_t)T * HV, 0, 1), *S0 = fill((size_t)N * HV * DK * DV, -1, 1);
    const size_t nS = (size_t)N * HV * DK * DV;
    double *S1 = calloc(nS, sizeof(double)), *S8 = calloc(nS, sizeof(double));
    double *o1 = calloc((size_t)T * HV * DV, sizeof(double)), *o8 = calloc((size_t)T * HV * DV, sizeof(double));
    if (!S1 || !S8 || !o1 || !o8) return 3;

    int bad = 0;
    if (gdn_oracle_prefill(N, HQK, HV, DK, DV, q, k, v, g, beta, cu, S0, 0.35, S1, o1, 1) ||
        gdn_oracle_prefill(N, HQK, HV, DK, DV, q, k, v, g, beta, cu, S0, 0.35, S8, o8, 8)) return 4;
    bad |= memcmp(S1, S8, nS * sizeof(double)) != 0;
    bad |= memcmp(o1, o8, (size_t)T * HV * DV * sizeof(double)) != 0;

    if (gdn_oracle_replay(N, HQK, HV, DK, DV, q, k, v, g, beta, cu, r, 0.35, S1, o1, 1) ||
        gdn_oracle_replay(N, HQK, HV, DK, DV, q, k, v, g, beta, cu, r, 0.35, S8, o8, 8)) return 4;
    bad |= memcmp(S1, S8, nS * sizeof(double)) != 0;
    bad |= memcmp(o1, o8, (size_t)T_out * HV * DV * sizeof(double)) != 0;

    double norm = 0.0;
    for (size_t i = 0; i < nS; ++i) norm += S1[i] * S1[i];
    if (!(norm > 0.0) || !isfinite(norm)) bad = 1;   /* the check must see real work */

    free(q); free(k); free(v); free(g); free(beta); free(S0);
    free(S1); free(S8); free(o1); free(o8);
    printf("oracle thread check: %s\n", bad ? "MISMATCH" : "ok");
    return bad ? 1 : 0;
}
