/*
 * gdn_oracle.c -- fp64 CPU oracle for the Gated DeltaNet replay / prefill path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header or constant
 * with the HIP library, and nothing on the product path may call it.
 *
 * What it computes (plain definition, token by token, in double precision):
 *
 *   Gated delta rule (Gated DeltaNet, the linear-attention layer the Tail-Replay
 *   pages rebuild; gist.science technical summary, "Mecanismos Principais": the
 *   recurrence equations are replayed over a short tail starting from a zero state):
 *
 *       S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *       o_t = scale * S_t^T q_t,            alpha_t = exp(g_t),
 *
 *   with S_t a d_k x d_v matrix per (sequence, v-head).  The update is evaluated as
 *       p = S^T k;  S = alpha*S - (alpha*beta) k p^T + beta k v^T
 *   which never forms (I - beta k k^T).  g = -inf gives alpha = 0 exactly.
 *
 *   Replay (Tail-Replay, arXiv 2608.30310 abstract and the technical summary's
 *   "Reconstrucao de Estado Independente"): for sequence n with matched prefix
 *   [cu[n], cu[n+1]) and replay length r_n, run the recurrence from S = 0 over the
 *   last r_n tokens [cu[n+1]-r_n, cu[n+1]).  o rows are packed per sequence in order.
 *
 *   Prefill (the full-prefill baseline the pages compare against): run the
 *   recurrence over the whole sequence from S0 (or zero).
 *
 * Layouts (row-major, packed varlen):
 *   q, k  [T, h_qk, d_k]      v [T, h_v, d_v]      g, beta [T, h_v]
 *   S0, S [N, h_v, d_k, d_v]  o [T_out, h_v, d_v]
 * v-head h reads q/k head floor(h * h_qk / h_v).
 *
 * Work is split over (sequence, v-head) chains with POSIX threads; each chain is
 * sequential, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t n_seqs;
    int32_t h_qk, h_v, d_k, d_v;
    const double *q, *k, *v, *g, *beta;
    const int64_t *cu;       /* [n_seqs + 1] */
    const int64_t *r;        /* [n_seqs] or NULL (prefill) */
    const double *S0;        /* [n_seqs, h_v, d_k, d_v] or NULL */
    double scale;
    double *S_out;           /* [n_seqs, h_v, d_k, d_v] */
    double *o_out;           /* [T_out, h_v, d_v] or NULL */
    const int64_t *o_row0;   /* first o row of each sequence */
    int64_t n_chains;
    int64_t next;            /* work counter */
    pthread_mutex_t lock;
} job_t;

/* One (sequence, v-head) chain of the recurrence. */
static void run_chain(const job_t *J, int64_t chain, double *p)
{
    const int64_t n = chain / J->h_v;
    const int32_t h = (int32_t)(chain % J->h_v);
    const int32_t hk = (int32_t)(((int64_t)h * J->h_qk) / J->h_v);
    const int32_t dk = J->d_k, dv = J->d_v;
    const int64_t end = J->cu[n + 1];
    const int64_t start = J->r ? end - J->r[n] : J->cu[n];
    double *S = J->S_out + (n * J->h_v + h) * (int64_t)dk * dv;

    if (!J->r && J->S0)
        memcpy(S, J->S0 + (n * J->h_v + h) * (int64_t)dk * dv, sizeof(double) * dk * dv);
    else
        memset(S, 0, sizeof(double) * dk * dv);

    for (int64_t t = start; t < end; ++t) {
        const double *kt = J->k + (t * J->h_qk + hk) * (int64_t)dk;
        const double *qt = J->q + (t * J->h_qk + hk) * (int64_t)dk;
        const double *vt = J->v + (t * J->h_v + h) * (int64_t)dv;
        const double a = exp(J->g[t * J->h_v + h]);
        const double b = J->beta[t * J->h_v + h];
        const double ab = a * b;

        /* p = S^T k */
        for (int32_t j = 0; j < dv; ++j) p[j] = 0.0;
        for (int32_t i = 0; i < dk; ++i) {
            const double ki = kt[i];
            const double *Si = S + (int64_t)i * dv;
            for (int32_t j = 0; j < dv; ++j) p[j] += ki * Si[j];
        }
        /* S = a S - (a b) k p^T + b k v^T */
        for (int32_t i = 0; i < dk; ++i) {
            const double ki = kt[i];
            double *Si = S + (int64_t)i * dv;
            for (int32_t j = 0; j < dv; ++j)
                Si[j] = a * Si[j] - ab * ki * p[j] + b * ki * vt[j];
        }
        /* o_t = scale * S_t^T q_t, from the state after the update */
        if (J->o_out) {
            double *ot = J->o_out + ((J->o_row0[n] + (t - start)) * J->h_v + h) * (int64_t)dv;
            for (int32_t j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i) {
                const double qi = qt[i];
                const double *Si = S + (int64_t)i * dv;
                for (int32_t j = 0; j < dv; ++j) ot[j] += qi * Si[j];
            }
            for (int32_t j = 0; j < dv; ++j) ot[j] *= J->scale;
        }
    }
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *p = (double *)malloc(sizeof(double) * (size_t)J->d_v);
    if (!p) return NULL;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t c = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (c >= J->n_chains) break;
        run_chain(J, c, p);
    }
    free(p);
    return NULL;
}

static int run_job(job_t *J, int32_t n_threads)
{
    int64_t *row0 = (int64_t *)malloc(sizeof(int64_t) * (size_t)(J->n_seqs + 1));
    if (!row0) return -1;
    row0[0] = 0;
    for (int64_t n = 0; n < J->n_seqs; ++n)
        row0[n + 1] = row0[n] + (J->r ? J->r[n] : J->cu[n + 1] - J->cu[n]);
    J->o_row0 = row0;
    J->n_chains = J->n_seqs * J->h_v;
    J->next = 0;
    pthread_mutex_init(&J->lock, NULL);
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    if ((int64_t)n_threads > J->n_chains) n_threads = (int32_t)(J->n_chains > 0 ? J->n_chains : 1);
    pthread_t tid[256];
    int started = 0;
    for (int32_t i = 1; i < n_threads; ++i)
        if (pthread_create(&tid[started], NULL, worker, J) == 0) ++started;
    worker(J);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    pthread_mutex_destroy(&J->lock);
    free(row0);
    return 0;
}

static int check_dims(int64_t n_seqs, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                      const int64_t *cu)
{
    if (n_seqs < 0 || h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return -1;
    if (h_v % h_qk != 0) return -1;
    if (!cu) return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    return 0;
}

/* Full prefill over every sequence, from S0 (NULL = zero state). */
int gdn_oracle_prefill(int64_t n_seqs, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                       const double *q, const double *k, const double *v, const double *g,
                       const double *beta, const int64_t *cu_seqlens, const double *S0,
                       double scale, double *S_out, double *o_out, int32_t n_threads)
{
    if (check_dims(n_seqs, h_qk, h_v, d_k, d_v, cu_seqlens)) return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.n_seqs = n_seqs; J.h_qk = h_qk; J.h_v = h_v; J.d_k = d_k; J.d_v = d_v;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
    J.cu = cu_seqlens; J.r = NULL; J.S0 = S0; J.scale = scale;
    J.S_out = S_out; J.o_out = o_out;
    return run_job(&J, n_threads);
}

/* Tail replay: zero state, last r[n] tokens of each sequence. */
int gdn_oracle_replay(int64_t n_seqs, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                      const double *q, const double *k, const double *v, const double *g,
                      const double *beta, const int64_t *cu_seqlens, const int64_t *r,
                      double scale, double *S_out, double *o_out, int32_t n_threads)
{
    if (check_dims(n_seqs, h_qk, h_v, d_k, d_v, cu_seqlens) || !r) return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (r[n] < 0 || r[n] > cu_seqlens[n + 1] - cu_seqlens[n]) return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.n_seqs = n_seqs; J.h_qk = h_qk; J.h_v = h_v; J.d_k = d_k; J.d_v = d_v;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
    J.cu = cu_seqlens; J.r = r; J.S0 = NULL; J.scale = scale;
    J.S_out = S_out; J.o_out = o_out;
    return run_job(&J, n_threads);
}

/* Relative Frobenius distance per state: ||A - B||_F / ||B||_F, or ||A||_F when
 * ||B||_F = 0.  Returns the number of non-finite entries seen in A. */
int64_t gdn_oracle_state_relerr(const double *A, const double *B, int64_t n_states,
                                int64_t state_elems, double *out)
{
    int64_t nonfinite = 0;
    for (int64_t s = 0; s < n_states; ++s) {
        const double *a = A + s * state_elems, *b = B + s * state_elems;
        double num = 0.0, den = 0.0;
        for (int64_t i = 0; i < state_elems; ++i) {
            if (!isfinite(a[i])) ++nonfinite;
            const double d = a[i] - b[i];
            num += d * d;
            den += b[i] * b[i];
        }
        out[s] = den > 0.0 ? sqrt(num / den) : sqrt(num);
    }
    return nonfinite;
}
