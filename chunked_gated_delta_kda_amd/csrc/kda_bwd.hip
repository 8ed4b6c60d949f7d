// kda_bwd.hip -- gradients of the KDA forward on gfx950 (a first backward kernel).
//
// The articles release the forward kernels only and leave training to the Triton
// implementation (kucoin.com news flash); this is the backward pass, derived by the
// chain rule from the per-token recurrence (a = exp(max(g, -5)) per key row):
//
//   S1 = Diag(a) S_{t-1};  u = S1^T k;  r = v - u;  d = beta r;  S_t = S1 + k d^T;
//   o_t = scale S_t^T q
//
// Walking the tokens backwards with dS = dL/dS_t (dL/dS_final to start):
//
//   dS += scale q do^T;         dq = scale (S1 do + k (d . do))
//   dd = dS^T k;   dk = dS d;   dbeta = dd . r;   dv = beta dd;   du = -beta dd
//   dS1 = dS + k du^T;          dk += S1 du;      dg_i = sum_j S1_ij dS1_ij (g_i >= -5)
//   dS = Diag(a) dS1
//
// One workgroup per (sequence, head): the state and its gradient (fp32, 128 x 129:
// one padding column makes both row and column walks free of LDS bank conflicts)
// live in LDS; each step is a few elementwise passes and reductions over rows or
// columns of the two tiles. The reverse walk needs the state before every token: a
// forward pass stores a checkpoint every BLK tokens in the workspace, then, block by
// block from the last, the tokens of a block are recomputed forward from their
// checkpoint with the state before each token stored to a per-chain buffer of BLK
// states, and walked backwards from it. Work per token is O(dk dv) on the vector
// units: this kernel is correct and simple, not fast (no MFMA, one chain per CU).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda.h"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int D = KDA_HEAD_DIM;
constexpr int NT = 256;
constexpr int LD = D + 1;        // padded row of the LDS tiles
constexpr float LB = KDA_LOWER_BOUND;

struct BwdLds {
    float S[D * LD];     // the state (S_{t-1}, then S1 in place)
    float dS[D * LD];    // dL/dS_t, then dS1, then dL/dS_{t-1}
    float q[D], k[D], v[D], e[D], g[D], dout[D];
    float u[D], r[D], d[D], dd[D], du[D];
    float part[2][D];    // partial sums of the two halves of a reduction
    float dot;           // d . do
    float beta;
};

// thread -> column tid % 128, rows [64 (tid / 128), +64): a wave's accesses to one row
// are 64 consecutive words
__device__ __forceinline__ int col_of(int tid) { return tid & (D - 1); }
__device__ __forceinline__ int row0_of(int tid) { return (tid >> 7) * 64; }

// sum over rows i of X[i][j] w[i], for column j = tid % 128 (both halves), into out[j]
__device__ __forceinline__ void reduce_rows(const float *X, const float *w, float *out, BwdLds &L) {
    const int tid = threadIdx.x, j = col_of(tid), i0 = row0_of(tid);
    float acc = 0.f;
    for (int i = i0; i < i0 + 64; ++i) acc = fmaf(X[i * LD + j], w[i], acc);
    L.part[tid >> 7][j] = acc;
    __syncthreads();
    if (tid < D) out[tid] = L.part[0][tid] + L.part[1][tid];
    __syncthreads();
}

// sum over columns j of X[i][j] w[j], for row i = tid % 128 (both halves of j): returns it
// in threads 0..127
__device__ __forceinline__ float reduce_cols(const float *X, const float *w, BwdLds &L) {
    const int tid = threadIdx.x, i = tid & (D - 1), j0 = (tid >> 7) * 64;
    float acc = 0.f;
    for (int j = j0; j < j0 + 64; ++j) acc = fmaf(X[i * LD + j], w[j], acc);
    L.part[tid >> 7][i] = acc;
    __syncthreads();
    const float s = tid < D ? L.part[0][tid] + L.part[1][tid] : 0.f;
    __syncthreads();
    return s;
}

__device__ __forceinline__ void load_tile(float *X, const float *src) {
    const int tid = threadIdx.x, j = col_of(tid), i0 = row0_of(tid);
    for (int i = i0; i < i0 + 64; ++i) X[i * LD + j] = src ? src[(int64_t)i * D + j] : 0.f;
}
__device__ __forceinline__ void store_tile(float *dst, const float *X) {
    const int tid = threadIdx.x, j = col_of(tid), i0 = row0_of(tid);
    for (int i = i0; i < i0 + 64; ++i) dst[(int64_t)i * D + j] = X[i * LD + j];
}

// inputs of token row th (= t H + h) into the LDS vectors
__device__ __forceinline__ void load_token(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                                           const float *beta, const float *dout, int64_t th, BwdLds &L) {
    const int tid = threadIdx.x;
    if (tid < D) {
        const int64_t o = th * D + tid;
        L.q[tid] = __uint_as_float((uint32_t)q[o] << 16);
        L.k[tid] = __uint_as_float((uint32_t)k[o] << 16);
        L.v[tid] = __uint_as_float((uint32_t)v[o] << 16);
        const float gi = g[o];
        L.g[tid] = gi;
        L.e[tid] = __expf(fmaxf(gi, LB));
        if (dout) L.dout[tid] = dout[o];
    }
    if (tid == 0) L.beta = beta[th];
    __syncthreads();
}

// one token forward on the LDS state: S <- S1 + k d^T (u, r, d left in LDS)
__device__ __forceinline__ void fwd_token(BwdLds &L) {
    const int tid = threadIdx.x, j = col_of(tid), i0 = row0_of(tid);
    for (int i = i0; i < i0 + 64; ++i) L.S[i * LD + j] *= L.e[i];
    __syncthreads();
    reduce_rows(L.S, L.k, L.u, L);
    if (tid < D) {
        L.r[tid] = L.v[tid] - L.u[tid];
        L.d[tid] = L.beta * L.r[tid];
    }
    __syncthreads();
    for (int i = i0; i < i0 + 64; ++i) L.S[i * LD + j] = fmaf(L.k[i], L.d[j], L.S[i * LD + j]);
    __syncthreads();
}

// State checkpoints: chunk_off[n] (blocks of BLK tokens before sequence n) indexes ck,
// [blocks, H, 128, 128]; buf holds BLK states per (sequence, head).
constexpr int BLK = 32;

__global__ __launch_bounds__(NT) void bwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float scale, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int N, int T, int H, const float *__restrict__ s0,
    const float *__restrict__ dout, const float *__restrict__ dsf, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dg, float *__restrict__ dbeta,
    float *__restrict__ ds0, float *__restrict__ ck, float *__restrict__ buf) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    BwdLds &L = *(BwdLds *)lds_raw;
    const int h = blockIdx.x % H, n = blockIdx.x / H;
    const int tid = threadIdx.x, j = col_of(tid), i0 = row0_of(tid);
    const int64_t bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
    const int64_t len = eos - bos;
    const int nblk = (int)((len + BLK - 1) / BLK);
    const int64_t sbase = ((int64_t)n * H + h) * D * D;
    float *ckc = ck + ((int64_t)chunk_off[n] * H + h) * D * D;   // this chain's block b: ckc + b H D D
    float *bufc = buf + ((int64_t)n * H + h) * BLK * D * D;

    // ---- forward: a checkpoint before every block of BLK tokens
    load_tile(L.S, s0 ? s0 + sbase : nullptr);
    __syncthreads();
    for (int64_t t = bos; t < eos; ++t) {
        if ((t - bos) % BLK == 0) store_tile(ckc + ((t - bos) / BLK) * H * D * D, L.S);
        load_token(q, k, v, g, beta, nullptr, t * H + h, L);
        fwd_token(L);
    }

    // ---- backward, block by block from the last
    load_tile(L.dS, dsf ? dsf + sbase : nullptr);
    __syncthreads();
    for (int b = nblk - 1; b >= 0; --b) {
        const int64_t tb = bos + (int64_t)b * BLK, te = min(eos, tb + BLK);
        load_tile(L.S, ckc + (int64_t)b * H * D * D);
        __syncthreads();
        for (int64_t t = tb; t < te; ++t) {      // the state before each token of the block
            store_tile(bufc + (t - tb) * D * D, L.S);
            load_token(q, k, v, g, beta, nullptr, t * H + h, L);
            fwd_token(L);
        }
        for (int64_t t = te - 1; t >= tb; --t) {
            const int64_t th = t * H + h;
            __syncthreads();                      // every thread's last reads of S are done
            load_tile(L.S, bufc + (t - tb) * D * D);
            load_token(q, k, v, g, beta, dout, th, L);
            // S1 = Diag(a) S_{t-1}; u, r, d
            for (int i = i0; i < i0 + 64; ++i) L.S[i * LD + j] *= L.e[i];
            __syncthreads();
            reduce_rows(L.S, L.k, L.u, L);
            if (tid < D) {
                L.r[tid] = L.v[tid] - L.u[tid];
                L.d[tid] = L.beta * L.r[tid];
            }
            // o_t = scale S_t^T q
            for (int i = i0; i < i0 + 64; ++i) L.dS[i * LD + j] = fmaf(scale * L.q[i], L.dout[j], L.dS[i * LD + j]);
            __syncthreads();
            if (tid < 64) {   // d . do, one wave
                float p = L.d[tid] * L.dout[tid] + L.d[tid + 64] * L.dout[tid + 64];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
                if (tid == 0) L.dot = p;
            }
            const float a_i = reduce_cols(L.S, L.dout, L);       // (S1 do)_i
            const float b_i = reduce_cols(L.dS, L.d, L);         // (dS d)_i
            reduce_rows(L.dS, L.k, L.dd, L);                     // dd = dS^T k
            if (tid < D) dq[th * D + tid] = scale * (a_i + L.k[tid] * L.dot);
            if (tid < D) {
                const float ddj = L.dd[tid];
                dv[th * D + tid] = L.beta * ddj;
                L.du[tid] = -L.beta * ddj;
            }
            if (tid < 64) {   // dbeta = dd . r, one wave
                float p = L.dd[tid] * L.r[tid] + L.dd[tid + 64] * L.r[tid + 64];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
                if (tid == 0) dbeta[th] = p;
            }
            __syncthreads();
            // u = S1^T k:  dS1 = dS + k du^T,  dk += S1 du
            for (int i = i0; i < i0 + 64; ++i) L.dS[i * LD + j] = fmaf(L.k[i], L.du[j], L.dS[i * LD + j]);
            __syncthreads();
            const float c_i = reduce_cols(L.S, L.du, L);         // (S1 du)_i
            // dg_i = sum_j S1_ij dS1_ij
            {
                const int i = tid & (D - 1), jb = (tid >> 7) * 64;
                float acc = 0.f;
                for (int jj = jb; jj < jb + 64; ++jj) acc = fmaf(L.S[i * LD + jj], L.dS[i * LD + jj], acc);
                L.part[tid >> 7][i] = acc;
            }
            __syncthreads();
            if (tid < D) {
                dk[th * D + tid] = b_i + c_i;
                const float dgi = L.part[0][tid] + L.part[1][tid];
                dg[th * D + tid] = L.g[tid] >= LB ? dgi : 0.f;
            }
            // S1 = Diag(a) S_{t-1}: dS_{t-1} = Diag(a) dS1
            for (int i = i0; i < i0 + 64; ++i) L.dS[i * LD + j] *= L.e[i];
        }
    }
    __syncthreads();
    if (ds0) store_tile(ds0 + sbase, L.dS);
}

}  // namespace

hipError_t launch_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                      float scale, const int32_t *cu_safe, const int32_t *chunk_off, int N, int T, int H,
                      const float *s0, const float *dout, const float *dsf, float *dq, float *dk, float *dv,
                      float *dg, float *dbeta, float *ds0, float *ck, float *buf, hipStream_t st) {
    constexpr int lds = (int)sizeof(BwdLds);
    static_assert(lds <= 160 * 1024, "LDS");
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)bwd_kernel, lds, lds_set) != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_kernel, dim3((unsigned)((int64_t)N * H)), dim3(NT), lds, st, q, k, v, g, beta, scale,
                       cu_safe, chunk_off, N, T, H, s0, dout, dsf, dq, dk, dv, dg, dbeta, ds0, ck, buf);
    return hipGetLastError();
}

int bwd_block_tokens() { return BLK; }

}  // namespace kda
