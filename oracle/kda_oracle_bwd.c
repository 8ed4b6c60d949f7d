/*
 * KDA backward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain fp64 reverse-mode evaluation of the gradients of the KDA forward that
 * kda_oracle.c computes (same layouts, same readings). The articles say only the
 * forward kernels were released and that training still goes through the Triton
 * implementation (kucoin.com news flash): the backward pass is the method's next
 * step, and this is its definition, derived here by the chain rule from the
 * per-token forward, nothing more. Only the tests may load it; it shares no code
 * with the HIP sources.
 *
 * Forward, per token t (a = exp(max(g_t, lower_bound)) per key row):
 *   S1  = Diag(a) S_{t-1}
 *   u   = S1^T k          r = v - u          d = beta r
 *   S_t = S1 + k d^T
 *   o_t = scale S_t^T q
 * Given dL/do_t for every token and dL/dS_final (zero when none is given), walk the
 * tokens backwards with dS = dL/dS_t:
 *   dS   += scale q do_t^T                 (o_t reads S_t)
 *   dq    = scale S_t do_t
 *   dd    = dS^T k                          (S_t = S1 + k d^T)
 *   dk    = dS d
 *   dbeta = dd . r,   dv = beta dd,   du = -beta dd
 *   dS1   = dS + k du^T                     (u = S1^T k)
 *   dk   += S1 du
 *   dg_i  = sum_j S1[i][j] dS1[i][j]   where g_i >= lower_bound, else 0
 *   dS    = Diag(a) dS1                     (S1 = Diag(a) S_{t-1})
 * and d initial_state = dS after the first token. The clamp passes the gradient
 * where g >= lower_bound (the value g = lower_bound itself included, as a clamp
 * from below does) and stops it below.
 *
 * The states S_{t-1} of a chain are kept from a forward pass over it (dk x dv
 * doubles per token: test sizes only).
 *
 * Layouts as kda_oracle.c; gradients: dq, dk [T, H, dk], dv [T, H, dv], dg [T, H, dk],
 * dbeta [T, H], d_initial_state [N, H, dk, dv] (may be NULL). d_final_state may be NULL.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *s0, *dout, *dfin;
    double scale, lower_bound;
    const int64_t *cu;
    int64_t n_seqs, n_heads, dk, dv;
    double *dq, *dkk, *dvv, *dg, *dbeta, *ds0;
    int64_t next;
    int failed;
    pthread_mutex_t lock;
} bwd_job;

/* One (sequence, head) chain. Returns 0, or -2 when memory fails. */
static int run_chain_bwd(bwd_job *J, int64_t n, int64_t h)
{
    const int64_t H = J->n_heads, dk = J->dk, dv = J->dv;
    const int64_t bos = J->cu[n], eos = J->cu[n + 1], len = eos - bos;
    const size_t sz = (size_t)(dk * dv);
    double *states = (double *)malloc(sizeof(double) * sz * (size_t)(len > 0 ? len : 1));
    double *S = (double *)malloc(sizeof(double) * sz);
    double *S1 = (double *)malloc(sizeof(double) * sz);
    double *dS = (double *)malloc(sizeof(double) * sz);
    double *a = (double *)malloc(sizeof(double) * (size_t)dk);
    double *vec = (double *)malloc(sizeof(double) * (size_t)(4 * dv));
    if (!states || !S || !S1 || !dS || !a || !vec) {
        free(states); free(S); free(S1); free(dS); free(a); free(vec);
        return -2;
    }
    double *u = vec, *r = vec + dv, *d = vec + 2 * dv, *dd = vec + 3 * dv;

    /* forward over the chain, keeping the state before every token */
    if (J->s0)
        memcpy(S, J->s0 + (n * H + h) * dk * dv, sz * sizeof(double));
    else
        memset(S, 0, sz * sizeof(double));
    for (int64_t t = bos; t < eos; ++t) {
        memcpy(states + (size_t)(t - bos) * sz, S, sz * sizeof(double));
        const double *kt = J->k + (t * H + h) * dk;
        const double *vt = J->v + (t * H + h) * dv;
        const double *gt = J->g + (t * H + h) * dk;
        const double bt = J->beta[t * H + h];
        for (int64_t i = 0; i < dk; ++i) {
            const double ai = exp(gt[i] < J->lower_bound ? J->lower_bound : gt[i]);
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= ai;
        }
        for (int64_t j = 0; j < dv; ++j) u[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) u[j] += kt[i] * S[i * dv + j];
        for (int64_t j = 0; j < dv; ++j) d[j] = bt * (vt[j] - u[j]);
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += kt[i] * d[j];
    }

    /* backward */
    if (J->dfin)
        memcpy(dS, J->dfin + (n * H + h) * dk * dv, sz * sizeof(double));
    else
        memset(dS, 0, sz * sizeof(double));
    for (int64_t t = eos - 1; t >= bos; --t) {
        const double *qt = J->q + (t * H + h) * dk;
        const double *kt = J->k + (t * H + h) * dk;
        const double *vt = J->v + (t * H + h) * dv;
        const double *gt = J->g + (t * H + h) * dk;
        const double *dot = J->dout + (t * H + h) * dv;
        const double bt = J->beta[t * H + h];
        const double *Sprev = states + (size_t)(t - bos) * sz;
        double *dqt = J->dq + (t * H + h) * dk;
        double *dkt = J->dkk + (t * H + h) * dk;
        double *dvt = J->dvv + (t * H + h) * dv;
        double *dgt = J->dg + (t * H + h) * dk;

        /* recompute the token: S1, u, r, d and S_t (into S) */
        for (int64_t i = 0; i < dk; ++i) {
            a[i] = exp(gt[i] < J->lower_bound ? J->lower_bound : gt[i]);
            for (int64_t j = 0; j < dv; ++j) S1[i * dv + j] = a[i] * Sprev[i * dv + j];
        }
        for (int64_t j = 0; j < dv; ++j) u[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) u[j] += kt[i] * S1[i * dv + j];
        for (int64_t j = 0; j < dv; ++j) {
            r[j] = vt[j] - u[j];
            d[j] = bt * r[j];
        }
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = S1[i * dv + j] + kt[i] * d[j];

        /* o_t = scale S_t^T q */
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] += J->scale * qt[i] * dot[j];
        for (int64_t i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dv; ++j) acc += S[i * dv + j] * dot[j];
            dqt[i] = J->scale * acc;
        }
        /* S_t = S1 + k d^T */
        for (int64_t j = 0; j < dv; ++j) dd[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) dd[j] += dS[i * dv + j] * kt[i];
        for (int64_t i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dv; ++j) acc += dS[i * dv + j] * d[j];
            dkt[i] = acc;
        }
        /* d = beta (v - u) */
        double db = 0.0;
        for (int64_t j = 0; j < dv; ++j) {
            db += dd[j] * r[j];
            dvt[j] = bt * dd[j];
            u[j] = -bt * dd[j];                /* u now holds du */
        }
        J->dbeta[t * H + h] = db;
        /* u = S1^T k: dS1 = dS + k du^T (into dS), dk += S1 du */
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] += kt[i] * u[j];
        for (int64_t i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dv; ++j) acc += S1[i * dv + j] * u[j];
            dkt[i] += acc;
        }
        /* S1 = Diag(a) S_{t-1}: gate gradient, then dS_{t-1} */
        for (int64_t i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dv; ++j) acc += S1[i * dv + j] * dS[i * dv + j];
            dgt[i] = gt[i] >= J->lower_bound ? acc : 0.0;
            for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] *= a[i];
        }
    }
    if (J->ds0)
        memcpy(J->ds0 + (n * H + h) * dk * dv, dS, sz * sizeof(double));
    free(states); free(S); free(S1); free(dS); free(a); free(vec);
    return 0;
}

static void *bwd_worker(void *arg)
{
    bwd_job *J = (bwd_job *)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t item = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (item >= J->n_seqs * J->n_heads)
            break;
        if (run_chain_bwd(J, item / J->n_heads, item % J->n_heads) != 0) {
            pthread_mutex_lock(&J->lock);
            J->failed = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

/* Returns 0 on success, -1 on a bad argument, -2 when memory or threads fail. */
int kda_oracle_bwd(const double *q, const double *k, const double *v, const double *g,
                   const double *beta, double scale, const int64_t *cu_seqlens,
                   int64_t n_seqs, int64_t n_heads, int64_t dk, int64_t dv,
                   const double *initial_state, double lower_bound, const double *d_out,
                   const double *d_final_state, double *dq, double *dkk, double *dvv, double *dg,
                   double *dbeta, double *d_initial_state, int n_threads)
{
    if (!cu_seqlens || n_seqs < 1 || n_heads < 1 || dk < 1 || dv < 1 || cu_seqlens[0] != 0)
        return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -1;
    if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !g || !beta || !d_out || !dq || !dkk || !dvv || !dg ||
                                   !dbeta))
        return -1;

    bwd_job J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.s0 = initial_state;
    J.dout = d_out; J.dfin = d_final_state;
    J.scale = scale; J.lower_bound = lower_bound;
    J.cu = cu_seqlens; J.n_seqs = n_seqs; J.n_heads = n_heads; J.dk = dk; J.dv = dv;
    J.dq = dq; J.dkk = dkk; J.dvv = dvv; J.dg = dg; J.dbeta = dbeta; J.ds0 = d_initial_state;
    J.next = 0;
    J.failed = 0;
    pthread_mutex_init(&J.lock, NULL);

    const int64_t items = n_seqs * n_heads;
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > items)
        n_threads = (int)items;
    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!tids) {
        pthread_mutex_destroy(&J.lock);
        return -2;
    }
    int started = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&tids[i], NULL, bwd_worker, &J) != 0)
            break;
        ++started;
    }
    if (started == 0)
        bwd_worker(&J);
    for (int i = 0; i < started; ++i)
        pthread_join(tids[i], NULL);
    free(tids);
    pthread_mutex_destroy(&J.lock);
    return J.failed ? -2 : 0;
}
