/*
 * abi_demo.c -- the KDA library driven through its C ABI alone (include/kda.h), with
 * no Python and no torch: device buffers from hipMalloc, one kda_fwd over a packed
 * batch of three sequences (one of them empty) with initial states, then one
 * kda_decode step per sequence that continues in place from the final states. The
 * results are checked against the fp64 oracle (oracle/libkda_oracle.so, test
 * infrastructure) run over the same sequences extended by the decode tokens.
 *
 * Test code: __graft_entry__.build() compiles it to tests/abi_demo_bin, and
 * tests/test_gpu_abi_demo.py runs it on the GPU. Exit status 0 when every output
 * passes the parity gate (relative L2 <= 1e-2, max-abs <= 2e-2 RMS).
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

/* the oracle's C entry point (oracle/kda_oracle.c) */
int kda_oracle_fwd(const double *q, const double *k, const double *v, const double *g,
                   const double *beta, double scale, const int64_t *cu_seqlens, int64_t n_seqs,
                   int64_t n_heads, int64_t dk, int64_t dv, const double *initial_state,
                   double lower_bound, double *out, double *final_state, const int64_t *pairs,
                   int64_t n_pairs, int n_threads);

#define D 128
#define NSEQ 3
#define NH 4

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(2);                                                                \
        }                                                                           \
    } while (0)

/* xorshift64* and Box-Muller: this program's own seeded inputs */
static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double urand(void) {
    rng ^= rng >> 12, rng ^= rng << 25, rng ^= rng >> 27;
    return (double)((rng * 0x2545f4914f6cdd1dull) >> 11) * (1.0 / 9007199254740992.0);
}
static double nrand(void) {
    double u = urand(), w = urand();
    if (u < 1e-300) u = 1e-300;
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * w);
}
/* fp32 -> bf16 bits, round to nearest even; and back */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
static double from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

typedef struct { double rel_l2, max_abs_rms; } parity_t;
static parity_t parity(const float *got, const double *ref, size_t n) {
    double e2 = 0, r2 = 0, emax = 0;
    for (size_t i = 0; i < n; ++i) {
        const double e = (double)got[i] - ref[i];
        e2 += e * e, r2 += ref[i] * ref[i];
        if (fabs(e) > emax || e != e) emax = fabs(e);
    }
    parity_t p = {sqrt(e2 / r2), emax / sqrt(r2 / (double)n)};
    return p;
}

int main(void) {
    const int lens[NSEQ] = {37, 0, 100};
    int T = 0;
    for (int n = 0; n < NSEQ; ++n) T += lens[n];
    const int TE = T + NSEQ;                  /* tokens with each sequence's decode token */
    const size_t row = (size_t)NH * D, st_elems = (size_t)NSEQ * NH * D * D;
    const float scale = (float)(1.0 / sqrt((double)D));

    /* extended sequences, token-major, sequence n = its prompt then its decode token */
    uint16_t *q = malloc(TE * row * 2), *k = malloc(TE * row * 2), *v = malloc(TE * row * 2);
    float *g = malloc(TE * row * 4), *beta = malloc((size_t)TE * NH * 4), *s0 = malloc(st_elems * 4);
    for (int t = 0; t < TE; ++t)
        for (int h = 0; h < NH; ++h) {
            double xq[D], xk[D], nq = 0, nk = 0;
            for (int c = 0; c < D; ++c) xq[c] = nrand(), nq += xq[c] * xq[c];
            for (int c = 0; c < D; ++c) xk[c] = nrand(), nk += xk[c] * xk[c];
            for (int c = 0; c < D; ++c) {
                const size_t i = ((size_t)t * NH + h) * D + c;
                q[i] = to_bf16((float)(xq[c] / sqrt(nq)));
                k[i] = to_bf16((float)(xk[c] / sqrt(nk)));
                v[i] = to_bf16((float)nrand());
                const double z = nrand();
                const double sp = z > 0 ? z + log1p(exp(-z)) : log1p(exp(z));   /* softplus */
                g[i] = (float)fmax(-sp, -5.0);
            }
            beta[(size_t)t * NH + h] = (float)(1.0 / (1.0 + exp(-nrand())));
        }
    for (size_t i = 0; i < st_elems; ++i) s0[i] = (float)(0.02 * nrand());

    /* packed prompt batch (T tokens) and the decode batch (one token per sequence) */
    int cu[NSEQ + 1], ext_row[NSEQ + 1];
    int64_t cu_ext[NSEQ + 1];
    cu[0] = 0, cu_ext[0] = 0;
    for (int n = 0; n < NSEQ; ++n) cu[n + 1] = cu[n] + lens[n], cu_ext[n + 1] = cu_ext[n] + lens[n] + 1;
    for (int n = 0; n < NSEQ; ++n) ext_row[n] = (int)cu_ext[n];
    uint16_t *qp = malloc(T * row * 2 + 2), *kp = malloc(T * row * 2 + 2), *vp = malloc(T * row * 2 + 2);
    float *gp = malloc(T * row * 4 + 4), *bp = malloc((size_t)T * NH * 4 + 4);
    uint16_t *qd = malloc(NSEQ * row * 2), *kd = malloc(NSEQ * row * 2), *vd = malloc(NSEQ * row * 2);
    float *gd = malloc(NSEQ * row * 4), *bd = malloc((size_t)NSEQ * NH * 4);
    for (int n = 0; n < NSEQ; ++n) {
        const size_t src = (size_t)ext_row[n] * row, dst = (size_t)cu[n] * row, L = (size_t)lens[n];
        memcpy(qp + dst, q + src, L * row * 2), memcpy(kp + dst, k + src, L * row * 2);
        memcpy(vp + dst, v + src, L * row * 2), memcpy(gp + dst, g + src, L * row * 4);
        memcpy(bp + (size_t)cu[n] * NH, beta + (size_t)ext_row[n] * NH, L * NH * 4);
        const size_t last = (size_t)(ext_row[n] + lens[n]);
        memcpy(qd + n * row, q + last * row, row * 2), memcpy(kd + n * row, k + last * row, row * 2);
        memcpy(vd + n * row, v + last * row, row * 2), memcpy(gd + n * row, g + last * row, row * 4);
        memcpy(bd + (size_t)n * NH, beta + last * NH, NH * 4);
    }

    /* device buffers */
    void *d_q, *d_k, *d_v, *d_qd, *d_kd, *d_vd;
    float *d_g, *d_b, *d_gd, *d_bd, *d_s, *d_out, *d_outd;
    int32_t *d_cu;
    HIP_OK(hipMalloc(&d_q, T * row * 2 + 2)); HIP_OK(hipMalloc(&d_k, T * row * 2 + 2));
    HIP_OK(hipMalloc(&d_v, T * row * 2 + 2)); HIP_OK(hipMalloc((void **)&d_g, T * row * 4 + 4));
    HIP_OK(hipMalloc((void **)&d_b, (size_t)T * NH * 4 + 4)); HIP_OK(hipMalloc((void **)&d_cu, sizeof cu));
    HIP_OK(hipMalloc((void **)&d_s, st_elems * 4)); HIP_OK(hipMalloc((void **)&d_out, T * row * 4 + 4));
    HIP_OK(hipMalloc(&d_qd, NSEQ * row * 2)); HIP_OK(hipMalloc(&d_kd, NSEQ * row * 2));
    HIP_OK(hipMalloc(&d_vd, NSEQ * row * 2)); HIP_OK(hipMalloc((void **)&d_gd, NSEQ * row * 4));
    HIP_OK(hipMalloc((void **)&d_bd, (size_t)NSEQ * NH * 4)); HIP_OK(hipMalloc((void **)&d_outd, NSEQ * row * 4));
    HIP_OK(hipMemcpy(d_q, qp, T * row * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_k, kp, T * row * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_v, vp, T * row * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_g, gp, T * row * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_b, bp, (size_t)T * NH * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_cu, cu, sizeof cu, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_s, s0, st_elems * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_qd, qd, NSEQ * row * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_kd, kd, NSEQ * row * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_vd, vd, NSEQ * row * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_gd, gd, NSEQ * row * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_bd, bd, (size_t)NSEQ * NH * 4, hipMemcpyHostToDevice));

    /* prefill, the final state written in place over the initial state, then one decode step */
    printf("%s\n", kda_version());
    int rc = kda_fwd(d_q, d_k, d_v, d_g, d_b, scale, d_cu, NSEQ, T, NH, D, d_s, d_out, d_s, NULL);
    if (rc != KDA_OK) {
        fprintf(stderr, "kda_fwd: %s\n", kda_status_string(rc));
        return 2;
    }
    rc = kda_decode(d_qd, d_kd, d_vd, d_gd, d_bd, scale, NSEQ, NH, D, d_s, d_s, d_outd, NULL);
    if (rc != KDA_OK) {
        fprintf(stderr, "kda_decode: %s\n", kda_status_string(rc));
        return 2;
    }
    HIP_OK(hipDeviceSynchronize());
    float *out = malloc(T * row * 4 + 4), *outd = malloc(NSEQ * row * 4), *fin = malloc(st_elems * 4);
    HIP_OK(hipMemcpy(out, d_out, T * row * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(outd, d_outd, NSEQ * row * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(fin, d_s, st_elems * 4, hipMemcpyDeviceToHost));

    /* the oracle over the extended sequences, from the same bf16-rounded values */
    double *Q = malloc(TE * row * 8), *K = malloc(TE * row * 8), *V = malloc(TE * row * 8);
    double *G = malloc(TE * row * 8), *B = malloc((size_t)TE * NH * 8), *S0 = malloc(st_elems * 8);
    double *O = malloc(TE * row * 8), *F = malloc(st_elems * 8);
    for (size_t i = 0; i < TE * row; ++i)
        Q[i] = from_bf16(q[i]), K[i] = from_bf16(k[i]), V[i] = from_bf16(v[i]), G[i] = g[i];
    for (size_t i = 0; i < (size_t)TE * NH; ++i) B[i] = beta[i];
    for (size_t i = 0; i < st_elems; ++i) S0[i] = s0[i];
    if (kda_oracle_fwd(Q, K, V, G, B, (double)scale, cu_ext, NSEQ, NH, D, D, S0, -5.0, O, F, NULL, 0, 4) != 0) {
        fprintf(stderr, "oracle failed\n");
        return 2;
    }
    /* reference rows of the prompt tokens and of the decode tokens */
    double *Op = malloc(T * row * 8 + 8), *Od = malloc(NSEQ * row * 8);
    for (int n = 0; n < NSEQ; ++n) {
        memcpy(Op + (size_t)cu[n] * row, O + (size_t)ext_row[n] * row, (size_t)lens[n] * row * 8);
        memcpy(Od + (size_t)n * row, O + (size_t)(ext_row[n] + lens[n]) * row, row * 8);
    }
    const parity_t po = parity(out, Op, T * row), pd = parity(outd, Od, NSEQ * row), pf = parity(fin, F, st_elems);
    printf("prefill o: rel_l2 %.3g max_abs/rms %.3g\n", po.rel_l2, po.max_abs_rms);
    printf("decode o:  rel_l2 %.3g max_abs/rms %.3g\n", pd.rel_l2, pd.max_abs_rms);
    printf("state:     rel_l2 %.3g max_abs/rms %.3g\n", pf.rel_l2, pf.max_abs_rms);
    const int ok = po.rel_l2 <= 1e-2 && po.max_abs_rms <= 2e-2 && pd.rel_l2 <= 1e-2 && pd.max_abs_rms <= 2e-2 &&
                   pf.rel_l2 <= 1e-2 && pf.max_abs_rms <= 2e-2;
    printf("%s\n", ok ? "PASS" : "FAIL");
    return ok ? 0 : 1;
}
