/*
 * kda_oracle.c -- plain, slow fp64 CPU oracle for the Kimi Delta Attention
 * (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU product
 * path never calls it, and it shares no code, header or constant with the
 * GPU path.
 *
 * What it computes (the per-token definition, nothing more): for every
 * token t of a sequence and every head, the state S (d_k x d_v) moves by
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,          alpha_t = exp(log_alpha_t),
 * i.e. a per-key-channel decay of the previous state corrected by a delta
 * rule scaled by beta_t ("Kimi Delta Attention: la atencion lineal detras
 * de Kimi K2 y Qwen3", TL;DR and section "Cómo funciona Kimi Delta
 * Attention paso a paso"; the transition is the diagonal-plus-low-rank
 * matrix of "Cos'è Kimi Delta Attention (KDA)?", section "Gating per
 * canale: cosa rende KDA diverso", which is also where the per-channel
 * gate is set apart from Gated DeltaNet's per-head one).  The first page
 * scales the query by 1/sqrt(d_k); here the scale is an argument.
 *
 * The state is stored as S[c][j], c = key channel (rows), j = value
 * channel (columns), so Diag(alpha_t) scales rows.  The first page keeps
 * the transpose (d_v x d_k) and decays along its key axis: the same map.
 *
 * Numbers: every input arrives as float32 (bf16 and fp32 stored values
 * widen to float32 exactly) and is widened to double; all arithmetic and
 * all outputs are double.  The output scale is an argument; callers pass
 * 1/sqrt(d_k) to follow the first page.
 *
 * Layouts (row-major, contiguous):
 *   q, k        [total_T][H][d_k]
 *   v           [total_T][H][d_v]
 *   log_alpha   [total_T][H][d_k]
 *   beta        [total_T][H]
 *   h0, hT, S   [N][H][d_k][d_v]     (h0 may be NULL: zero initial state)
 *   o           [total_T][H][d_v]
 *   cu_seqlens  [N+1] sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1
 *
 * Parallelism: sequences and heads never interact, so (sequence, head)
 * pairs are handed to worker threads; each pair runs the plain token loop.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const float *q, *k, *v, *log_alpha, *beta;
    const double *h0;     /* NULL => zeros */
    const int64_t *cu_seqlens;
    int64_t N, H, dk, dv;
    double scale;
    double *o, *hT;       /* hT may be NULL */
    /* work distribution */
    int64_t next;         /* next (seq, head) item, guarded by mu */
    pthread_mutex_t mu;
    int failed;
} job_t;

/* One token: S <- M S + beta k v^T with the transition
 * M = (I - beta k k^T) Diag(alpha), then o = scale S^T q.
 *
 * M is a diagonal matrix plus a rank-one term, the DPLR structure the
 * second page names for KDA's per-channel gate.  Expanding it,
 *   M S + beta k v^T = Diag(alpha) S + k w^T,   w = beta (v - S^T Diag(alpha) k),
 * so the token costs two sweeps over the state: the first forms the
 * row vector u = k^T Diag(alpha) S, the second rewrites every key row c as
 * alpha_c S[c,:] + k_c w and adds q_c times the new row into o. */
static void kda_token(double *S, double *u, double *w, int64_t dk, int64_t dv,
                      const float *q, const float *k, const float *v,
                      const float *log_alpha, double beta, double scale,
                      double *o)
{
    for (int64_t j = 0; j < dv; ++j) u[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
        const double ac = exp((double)log_alpha[c]);
        const double kc = (double)k[c];
        const double *row = S + c * dv;
        for (int64_t j = 0; j < dv; ++j) u[j] += (ac * row[j]) * kc;
    }
    for (int64_t j = 0; j < dv; ++j) w[j] = beta * ((double)v[j] - u[j]);

    for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
        const double ac = exp((double)log_alpha[c]);
        const double kc = (double)k[c], qc = (double)q[c];
        double *row = S + c * dv;
        for (int64_t j = 0; j < dv; ++j) {
            const double s = ac * row[j] + kc * w[j];
            row[j] = s;
            o[j] += s * qc;
        }
    }
    for (int64_t j = 0; j < dv; ++j) o[j] *= scale;
}

static int run_pair(job_t *J, int64_t n, int64_t h)
{
    const int64_t dk = J->dk, dv = J->dv, H = J->H;
    double *S = (double *)malloc((size_t)(dk * dv) * sizeof(double));
    double *u = (double *)malloc((size_t)dv * sizeof(double));
    double *w = (double *)malloc((size_t)dv * sizeof(double));
    if (!S || !u || !w) { free(S); free(u); free(w); return 1; }

    const int64_t sidx = (n * H + h) * dk * dv;
    if (J->h0) memcpy(S, J->h0 + sidx, (size_t)(dk * dv) * sizeof(double));
    else       memset(S, 0, (size_t)(dk * dv) * sizeof(double));

    for (int64_t t = J->cu_seqlens[n]; t < J->cu_seqlens[n + 1]; ++t) {
        const int64_t th = t * H + h;
        kda_token(S, u, w, dk, dv,
                  J->q + th * dk, J->k + th * dk, J->v + th * dv,
                  J->log_alpha + th * dk, (double)J->beta[th], J->scale,
                  J->o + th * dv);
    }
    if (J->hT) memcpy(J->hT + sidx, S, (size_t)(dk * dv) * sizeof(double));
    free(S); free(u); free(w);
    return 0;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t total = J->N * J->H;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t item = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (item >= total) break;
        if (run_pair(J, item / J->H, item % J->H)) {
            pthread_mutex_lock(&J->mu);
            J->failed = 1;
            pthread_mutex_unlock(&J->mu);
        }
    }
    return NULL;
}

static int run_job(job_t *J, int nthreads)
{
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    const int64_t total = J->N * J->H;
    if (nthreads > total) nthreads = (int)(total > 0 ? total : 1);
    J->next = 0;
    J->failed = 0;
    pthread_mutex_init(&J->mu, NULL);
    pthread_t *th = (pthread_t *)malloc((size_t)nthreads * sizeof(pthread_t));
    if (!th) return 1;
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, J) == 0) ++started;
        else th[i] = 0;
    }
    worker(J);                          /* the calling thread works too */
    for (int i = 1; i < nthreads; ++i)
        if (th[i]) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J->mu);
    (void)started;
    return J->failed;
}

/* Prefill over a packed variable-length batch.  Returns 0 on success,
 * 1 on an allocation failure, 2 on a malformed argument. */
int kdaref_prefill(const float *q, const float *k, const float *v,
                   const float *log_alpha, const float *beta,
                   const double *h0, const int64_t *cu_seqlens,
                   int64_t N, int64_t H, int64_t dk, int64_t dv, double scale,
                   double *o, double *hT, int nthreads)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return 2;
    if (cu_seqlens[0] != 0) return 2;
    for (int64_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 2;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta;
    J.h0 = h0; J.cu_seqlens = cu_seqlens;
    J.N = N; J.H = H; J.dk = dk; J.dv = dv; J.scale = scale;
    J.o = o; J.hT = hT;
    return run_job(&J, nthreads);
}

/* One decode step: one token per sequence, state S [N][H][d_k][d_v]
 * updated in place, o [N][H][d_v].  Same per-token body as prefill. */
int kdaref_decode_step(const float *q, const float *k, const float *v,
                       const float *log_alpha, const float *beta,
                       double *S, int64_t N, int64_t H, int64_t dk, int64_t dv,
                       double scale, double *o)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !S) return 2;
    double *u = (double *)malloc((size_t)dv * sizeof(double));
    double *w = (double *)malloc((size_t)dv * sizeof(double));
    if (!u || !w) { free(u); free(w); return 1; }
    for (int64_t nh = 0; nh < N * H; ++nh)
        kda_token(S + nh * dk * dv, u, w, dk, dv,
                  q + nh * dk, k + nh * dk, v + nh * dv,
                  log_alpha + nh * dk, (double)beta[nh], scale, o + nh * dv);
    free(u); free(w);
    return 0;
}
