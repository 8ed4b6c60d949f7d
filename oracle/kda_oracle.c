/*
 * KDA forward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct fp64 CPU evaluation of the Kimi Delta
 * Attention forward recurrence, one token at a time. It exists so that the
 * GPU kernels have something independent to be checked against. Only the
 * tests, the package smoke check and the benchmark's CPU-baseline leg may
 * load it; nothing on the GPU path calls it, and it shares no code, header
 * or constant with the HIP sources.
 *
 * What it computes (per sequence n, per head h, independently):
 *
 *   S_0     = initial_state[n,h]  (dk x dv; zeros when none is given)
 *   for t over the tokens of sequence n, in order:
 *     a_t   = exp(max(g_t, lower_bound))            per key channel
 *     S'    = Diag(a_t) S_{t-1}                     decay acts on key rows
 *     u_t   = beta_t (v_t - S'^T k_t)               delta-rule error
 *     S_t   = S' + k_t u_t^T
 *     o_t   = scale * S_t^T q_t                     read-out after the write
 *   final_state[n,h] = S_T
 *
 * S' + k_t u_t^T expands to (I - beta_t k_t k_t^T) Diag(a_t) S_{t-1}
 * + beta_t k_t v_t^T, which is the gated delta rule with a per-channel gate
 * that the FlashKDA articles describe (smzdm "KDA 内核到底难在哪": KDA refines
 * Gated DeltaNet by giving each channel its own decay and folds history into a
 * fixed-size state; the decay is bounded below by lower_bound = -5). The
 * order "decay, then delta write, then read" and the key axis carrying the
 * decay are the readings this project takes of that description.
 *
 * Layouts (row-major, contiguous):
 *   q, k   [T, H, dk]    v [T, H, dv]    g [T, H, dk]    beta [T, H]
 *   cu_seqlens [N+1] with 0 = c_0 <= c_1 <= ... <= c_N = T
 *   initial_state, final_state [N, H, dk, dv]   (row = key channel)
 *   out [T, H, dv]
 *
 * pairs: optional list of (n, h) pairs (2*n_pairs int64); when given, only
 * those chains are evaluated (their o rows and final_state blocks are
 * written; everything else in out/final_state is left untouched).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *s0;
    double scale, lower_bound;
    const int64_t *cu;
    int64_t n_seqs, n_heads, dk, dv;
    double *out, *fin;
    const int64_t *pairs;
    int64_t n_items;
    int64_t next; /* next work item, guarded by lock */
    pthread_mutex_t lock;
} oracle_job;

/* One (sequence, head) chain, token by token. S is dk x dv, row = key channel. */
static void run_chain(const oracle_job *J, int64_t n, int64_t h, double *S, double *kv)
{
    const int64_t H = J->n_heads, dk = J->dk, dv = J->dv;
    const int64_t bos = J->cu[n], eos = J->cu[n + 1];

    if (J->s0)
        memcpy(S, J->s0 + (n * H + h) * dk * dv, (size_t)(dk * dv) * sizeof(double));
    else
        memset(S, 0, (size_t)(dk * dv) * sizeof(double));

    for (int64_t t = bos; t < eos; ++t) {
        const double *qt = J->q + (t * H + h) * dk;
        const double *kt = J->k + (t * H + h) * dk;
        const double *vt = J->v + (t * H + h) * dv;
        const double *gt = J->g + (t * H + h) * dk;
        const double bt = J->beta[t * H + h];

        /* decay: row i of S scales by exp(max(g_i, lower_bound)) */
        for (int64_t i = 0; i < dk; ++i) {
            double gi = gt[i] < J->lower_bound ? J->lower_bound : gt[i];
            double a = exp(gi);
            double *row = S + i * dv;
            for (int64_t j = 0; j < dv; ++j)
                row[j] *= a;
        }
        /* kv = S^T k  (what the decayed state currently predicts for key k) */
        for (int64_t j = 0; j < dv; ++j)
            kv[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
            const double *row = S + i * dv;
            const double ki = kt[i];
            for (int64_t j = 0; j < dv; ++j)
                kv[j] += ki * row[j];
        }
        /* u = beta (v - S^T k), then the rank-one write S += k u^T */
        for (int64_t j = 0; j < dv; ++j)
            kv[j] = bt * (vt[j] - kv[j]);
        for (int64_t i = 0; i < dk; ++i) {
            double *row = S + i * dv;
            const double ki = kt[i];
            for (int64_t j = 0; j < dv; ++j)
                row[j] += ki * kv[j];
        }
        /* o = scale * S^T q */
        double *ot = J->out + (t * H + h) * dv;
        for (int64_t j = 0; j < dv; ++j)
            ot[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
            const double *row = S + i * dv;
            const double qi = qt[i];
            for (int64_t j = 0; j < dv; ++j)
                ot[j] += qi * row[j];
        }
        for (int64_t j = 0; j < dv; ++j)
            ot[j] *= J->scale;
    }
    if (J->fin)
        memcpy(J->fin + (n * H + h) * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    double *S = (double *)malloc((size_t)(J->dk * J->dv) * sizeof(double));
    double *kv = (double *)malloc((size_t)J->dv * sizeof(double));
    if (!S || !kv) {
        free(S);
        free(kv);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t item = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (item >= J->n_items)
            break;
        int64_t n, h;
        if (J->pairs) {
            n = J->pairs[2 * item];
            h = J->pairs[2 * item + 1];
        } else {
            n = item / J->n_heads;
            h = item % J->n_heads;
        }
        run_chain(J, n, h, S, kv);
    }
    free(S);
    free(kv);
    return NULL;
}

/* Returns 0 on success, -1 on a bad argument, -2 when memory or threads fail. */
int kda_oracle_fwd(const double *q, const double *k, const double *v, const double *g,
                   const double *beta, double scale, const int64_t *cu_seqlens,
                   int64_t n_seqs, int64_t n_heads, int64_t dk, int64_t dv,
                   const double *initial_state, double lower_bound, double *out,
                   double *final_state, const int64_t *pairs, int64_t n_pairs,
                   int n_threads)
{
    if (!cu_seqlens || n_seqs < 1 || n_heads < 1 || dk < 1 || dv < 1 || !out)
        return -1;
    if (cu_seqlens[0] != 0)
        return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -1;
    if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !g || !beta))
        return -1;
    if (pairs)
        for (int64_t i = 0; i < n_pairs; ++i)
            if (pairs[2 * i] < 0 || pairs[2 * i] >= n_seqs || pairs[2 * i + 1] < 0 ||
                pairs[2 * i + 1] >= n_heads)
                return -1;

    oracle_job J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.s0 = initial_state;
    J.scale = scale; J.lower_bound = lower_bound;
    J.cu = cu_seqlens; J.n_seqs = n_seqs; J.n_heads = n_heads; J.dk = dk; J.dv = dv;
    J.out = out; J.fin = final_state;
    J.pairs = pairs;
    J.n_items = pairs ? n_pairs : n_seqs * n_heads;
    J.next = 0;
    pthread_mutex_init(&J.lock, NULL);

    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > J.n_items)
        n_threads = (int)(J.n_items > 0 ? J.n_items : 1);

    int rc = 0;
    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!tids) {
        pthread_mutex_destroy(&J.lock);
        return -2;
    }
    int started = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&tids[i], NULL, worker, &J) != 0)
            break;
        ++started;
    }
    if (started == 0) {
        /* no thread could start: run inline */
        if (worker(&J) != NULL)
            rc = -2;
    }
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(tids[i], &ret);
        if (ret != NULL)
            rc = -2;
    }
    free(tids);
    pthread_mutex_destroy(&J.lock);
    return rc;
}
