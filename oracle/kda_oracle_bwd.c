/*
 * kda_oracle_bwd.c -- plain, slow fp64 CPU oracle for the gradients of the
 * Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY, like kda_oracle.c: only the test suite, the
 * smoke check and the benchmark's CPU leg may load it, and it shares no
 * code, header or constant with the GPU path.
 *
 * What it computes: the reverse-mode derivative of the per-token
 * recurrence S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T,
 * o_t = scale S_t^T q ("Kimi Delta Attention: la atencion lineal detras de
 * Kimi K2 y Qwen3", section "Cómo funciona Kimi Delta Attention paso a
 * paso"; the diagonal-plus-low-rank transition of "Cos'è Kimi Delta
 * Attention (KDA)?", section "Gating per canale: cosa rende KDA diverso").
 * With the state stored S[c][j] (c = key channel, j = value channel), one
 * token expands into
 *
 *   D = Diag(alpha) S_prev,  u = D^T k,  r = v - u,  w = beta r,
 *   S = D + k w^T,           o = scale S^T q,
 *
 * and the adjoints run through those definitions in reverse; given
 * L = the adjoint of S (from the later tokens, or dhT after the last one)
 * and dO = the adjoint of o:
 *     o = scale S^T q:   L  += scale q dO^T;        dq = scale S dO
 *     S = D + k w^T:     dD  = L;  dk = L w;        dw = L^T k
 *     w = beta (v - u):  dbeta = dw . r;  dv = beta dw;  du = -beta dw
 *     u = D^T k:         dD += k du^T;    dk += D du
 *     D = Diag(alpha) S_prev:  dlog_alpha[c] = sum_j dD[c][j] D[c][j];
 *                        L = Diag(alpha) dD
 *   and after the first token of the sequence dh0 = L.
 *
 * The states before each token are needed in reverse order: the forward
 * pass keeps the state every kSeg tokens, and the backward pass recomputes
 * the kSeg states of one segment at a time from its checkpoint.
 *
 * Numbers: inputs arrive as float32 (bf16 and fp32 values widen exactly),
 * the adjoints dO and dhT as double; all arithmetic and outputs are double.
 * Layouts as in kda_oracle.c; dO is [total_T][H][d_v], dhT and dh0
 * [N][H][d_k][d_v], and the gradients take the layouts of their inputs
 * (dlog_alpha [total_T][H][d_k], dbeta [total_T][H]).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { kSeg = 64 };

typedef struct {
    const float *q, *k, *v, *log_alpha, *beta;
    const double *h0, *dO, *dhT;   /* h0, dhT may be NULL (zeros) */
    const int64_t *cu;
    int64_t N, H, dk, dv;
    double scale;
    double *dq, *dk_, *dv_, *dla, *dbeta, *dh0;   /* dh0 may be NULL */
    int64_t next;
    pthread_mutex_t mu;
    int failed;
} bjob_t;

/* forward of one token on S (in place), keeping what the backward needs:
 * the decayed state D, the residual r = v - D^T k and w = beta r */
static void fwd_token(double *S, double *D, double *r, double *w, int64_t dk, int64_t dv,
                      const float *k, const float *v, const float *la, double beta)
{
    for (int64_t c = 0; c < dk; ++c) {
        const double a = exp((double)la[c]);
        for (int64_t j = 0; j < dv; ++j) D[c * dv + j] = a * S[c * dv + j];
    }
    for (int64_t j = 0; j < dv; ++j) {
        double u = 0.0;
        for (int64_t c = 0; c < dk; ++c) u += D[c * dv + j] * (double)k[c];
        r[j] = (double)v[j] - u;
        w[j] = beta * r[j];
    }
    for (int64_t c = 0; c < dk; ++c)
        for (int64_t j = 0; j < dv; ++j) S[c * dv + j] = D[c * dv + j] + (double)k[c] * w[j];
}

static int run_pair(bjob_t *J, int64_t n, int64_t h)
{
    const int64_t dk = J->dk, dv = J->dv, H = J->H, SE = dk * dv;
    const int64_t t0 = J->cu[n], t1 = J->cu[n + 1], len = t1 - t0;
    const int64_t nseg = (len + kSeg - 1) / kSeg;
    double *ck = (double *)malloc((size_t)((nseg > 0 ? nseg : 1) * SE) * sizeof(double));
    double *segS = (double *)malloc((size_t)((kSeg + 1) * SE) * sizeof(double));
    double *D = (double *)malloc((size_t)SE * sizeof(double));
    double *L = (double *)malloc((size_t)SE * sizeof(double));
    double *dD = (double *)malloc((size_t)SE * sizeof(double));
    double *r = (double *)malloc((size_t)dv * sizeof(double));
    double *w = (double *)malloc((size_t)dv * sizeof(double));
    double *dw = (double *)malloc((size_t)dv * sizeof(double));
    int rc = 0;
    if (!ck || !segS || !D || !L || !dD || !r || !w || !dw) { rc = 1; goto out; }

    /* forward: checkpoint the state before every kSeg-th token */
    {
        double *S = segS;
        const int64_t sidx = (n * H + h) * SE;
        if (J->h0) memcpy(S, J->h0 + sidx, (size_t)SE * sizeof(double));
        else       memset(S, 0, (size_t)SE * sizeof(double));
        for (int64_t t = t0; t < t1; ++t) {
            if ((t - t0) % kSeg == 0) memcpy(ck + ((t - t0) / kSeg) * SE, S, (size_t)SE * sizeof(double));
            const int64_t th = t * H + h;
            fwd_token(S, D, r, w, dk, dv, J->k + th * dk, J->v + th * dv,
                      J->log_alpha + th * dk, (double)J->beta[th]);
        }
        if (J->dhT) memcpy(L, J->dhT + sidx, (size_t)SE * sizeof(double));
        else        memset(L, 0, (size_t)SE * sizeof(double));
    }

    /* backward, one segment at a time from the last */
    for (int64_t s = nseg - 1; s >= 0; --s) {
        const int64_t a0 = t0 + s * kSeg;
        const int64_t a1 = a0 + kSeg < t1 ? a0 + kSeg : t1;
        /* states before each token of the segment: segS[i] precedes token a0 + i */
        memcpy(segS, ck + s * SE, (size_t)SE * sizeof(double));
        for (int64_t t = a0; t + 1 < a1; ++t) {
            const int64_t i = t - a0, th = t * H + h;
            memcpy(segS + (i + 1) * SE, segS + i * SE, (size_t)SE * sizeof(double));
            fwd_token(segS + (i + 1) * SE, D, r, w, dk, dv, J->k + th * dk, J->v + th * dv,
                      J->log_alpha + th * dk, (double)J->beta[th]);
        }
        for (int64_t t = a1 - 1; t >= a0; --t) {
            const int64_t i = t - a0, th = t * H + h;
            const float *q = J->q + th * dk, *k = J->k + th * dk, *v = J->v + th * dv;
            const float *la = J->log_alpha + th * dk;
            const double beta = (double)J->beta[th];
            const double *dO = J->dO + th * dv;
            /* the state after the token goes to the slot of the state
             * before token i+1, which the reverse walk has already used */
            double *S = segS + (i + 1) * SE;
            memcpy(S, segS + i * SE, (size_t)SE * sizeof(double));
            fwd_token(S, D, r, w, dk, dv, k, v, la, beta);

            /* o = scale S^T q */
            for (int64_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    L[c * dv + j] += J->scale * (double)q[c] * dO[j];
                    acc += S[c * dv + j] * dO[j];
                }
                J->dq[th * dk + c] = J->scale * acc;
            }
            /* S = D + k w^T */
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < dk; ++c) acc += L[c * dv + j] * (double)k[c];
                dw[j] = acc;
            }
            double db = 0.0;
            for (int64_t j = 0; j < dv; ++j) {
                db += dw[j] * r[j];                       /* w = beta (v - u) */
                J->dv_[th * dv + j] = beta * dw[j];
            }
            J->dbeta[th] = db;
            for (int64_t c = 0; c < dk; ++c) {
                double dkc = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    const double du = -beta * dw[j];
                    dkc += L[c * dv + j] * w[j];          /* from S = D + k w^T */
                    dkc += D[c * dv + j] * du;            /* from u = D^T k */
                    dD[c * dv + j] = L[c * dv + j] + (double)k[c] * du;
                }
                J->dk_[th * dk + c] = dkc;
            }
            /* D = Diag(alpha) S_prev */
            for (int64_t c = 0; c < dk; ++c) {
                const double a = exp((double)la[c]);
                double g = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    g += dD[c * dv + j] * D[c * dv + j];
                    L[c * dv + j] = a * dD[c * dv + j];
                }
                J->dla[th * dk + c] = g;
            }
        }
    }
    if (J->dh0) memcpy(J->dh0 + (n * H + h) * SE, L, (size_t)SE * sizeof(double));
out:
    free(ck); free(segS); free(D); free(L); free(dD); free(r); free(w); free(dw);
    return rc;
}

static void *worker(void *arg)
{
    bjob_t *J = (bjob_t *)arg;
    const int64_t total = J->N * J->H;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t item = J->next++;
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

/* Gradients of <o, dO> + <hT, dhT> with respect to q, k, v, log_alpha,
 * beta and h0.  Returns 0 on success, 1 on an allocation failure, 2 on a
 * malformed argument. */
int kdaref_backward(const float *q, const float *k, const float *v,
                    const float *log_alpha, const float *beta, const double *h0,
                    const int64_t *cu_seqlens, int64_t N, int64_t H, int64_t dk, int64_t dv,
                    double scale, const double *dO, const double *dhT,
                    double *dq, double *dk_, double *dv_, double *dla, double *dbeta,
                    double *dh0, int nthreads)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens || !dO) return 2;
    if (cu_seqlens[0] != 0) return 2;
    for (int64_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 2;
    bjob_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta;
    J.h0 = h0; J.dO = dO; J.dhT = dhT; J.cu = cu_seqlens;
    J.N = N; J.H = H; J.dk = dk; J.dv = dv; J.scale = scale;
    J.dq = dq; J.dk_ = dk_; J.dv_ = dv_; J.dla = dla; J.dbeta = dbeta; J.dh0 = dh0;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    const int64_t total = N * H;
    if (nthreads > total) nthreads = (int)(total > 0 ? total : 1);
    pthread_mutex_init(&J.mu, NULL);
    pthread_t *th = (pthread_t *)malloc((size_t)nthreads * sizeof(pthread_t));
    if (!th) { pthread_mutex_destroy(&J.mu); return 1; }
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, worker, &J) != 0) th[i] = 0;
    worker(&J);
    for (int i = 1; i < nthreads; ++i)
        if (th[i]) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return J.failed;
}
