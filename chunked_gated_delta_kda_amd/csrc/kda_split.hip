// kda_split.hip -- the two-kernel KDA forward: a chunk-parallel prep kernel
// over (chunk, head) that writes one record per chunk-head, and a sequential
// recurrence kernel over (sequence, head, 16-column state slice).
//
// The split into a wide "prepare" phase over every (sequence, head, chunk) and
// a narrow serial phase over (sequence, head) follows the two-kernel layout the
// FlashKDA write-up describes (smzdm.com, "KDA 内核到底难在哪"); the kernels
// themselves are this library's gfx950 design (see kda_device.hpp).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

static_assert(Rec::BYTES == REC_BYTES, "record size mismatch");

// ---------------------------------------------------------------- chunk map
// One workgroup. chunk_off[n] = number of 16-token chunks before sequence n
// (chunk_off[N] = total); order[] lists sequences longest first (ties by
// index) when N <= ORDER_MAX, else in input order.
constexpr int MAP_THREADS = 256;
constexpr int ORDER_MAX = 2048;

__global__ __launch_bounds__(MAP_THREADS) void chunk_map_kernel(const int32_t *__restrict__ cu,
                                                                 int N, int T,
                                                                 int32_t *__restrict__ chunk_off,
                                                                 int32_t *__restrict__ order) {
    __shared__ int32_t part[MAP_THREADS];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += MAP_THREADS) {
        const int n = base + tid;
        int32_t c = 0;
        if (n < N) {
            const int32_t len = cu ? cu[n + 1] - cu[n] : T;
            c = (len + C - 1) / C;
        }
        part[tid] = c;
        __syncthreads();
        for (int s = 1; s < MAP_THREADS; s <<= 1) {   // inclusive Hillis-Steele scan
            const int32_t x = tid >= s ? part[tid - s] : 0;
            __syncthreads();
            part[tid] += x;
            __syncthreads();
        }
        if (n < N) chunk_off[n + 1] = carry + part[tid];
        __syncthreads();
        if (tid == MAP_THREADS - 1) carry += part[tid];
        __syncthreads();
    }
    if (tid == 0) chunk_off[0] = 0;
    if (N <= ORDER_MAX) {
        for (int n = tid; n < N; n += MAP_THREADS) {
            const int32_t ln = cu ? cu[n + 1] - cu[n] : T;
            int rank = 0;
            for (int m = 0; m < N; ++m) {
                const int32_t lm = cu ? cu[m + 1] - cu[m] : T;
                rank += (lm > ln) || (lm == ln && m < n);
            }
            order[rank] = n;
        }
    } else {
        for (int n = tid; n < N; n += MAP_THREADS) order[n] = n;
    }
}

// ---------------------------------------------------------------- prep
// One wave per (chunk, head). Grid: max_chunks * H blocks of 64 threads; blocks
// past the real chunk count exit.
__global__ __launch_bounds__(64) void prep_kernel(const uint16_t *__restrict__ q,
                                                  const uint16_t *__restrict__ k,
                                                  const float *__restrict__ g,
                                                  const float *__restrict__ beta,
                                                  const int32_t *__restrict__ cu, int N, int T,
                                                  int H, float scale,
                                                  const int32_t *__restrict__ chunk_off,
                                                  char *__restrict__ recs) {
    __shared__ PrepLds L;
    const int ci = blockIdx.x / H, h = blockIdx.x % H;
    if (ci >= chunk_off[N]) return;
    // sequence owning chunk ci: largest n with chunk_off[n] <= ci
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= ci) lo = mid; else hi = mid - 1;
    }
    const int n = lo;
    const int64_t bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
    const int64_t t0 = bos + (int64_t)C * (ci - chunk_off[n]);
    const int nc = (int)min<int64_t>(C, eos - t0);
    prep_chunk(q, k, g, beta, t0, nc, h, H, scale, L, recs + ((int64_t)ci * H + h) * Rec::BYTES);
}

// ---------------------------------------------------------------- recurrence
// NW waves per block, one 16-column state slice each; block covers 16*NW
// value columns of one (sequence, head). Blocks of one (sequence, head) are
// given consecutive logical ids, and xcd_remap keeps them on one XCD.
template <int NW>
__global__ __launch_bounds__(64 * NW) void recur_kernel(
    const char *__restrict__ recs, const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order, int N, int T, int H,
    const float *__restrict__ s0, float *__restrict__ out, float *__restrict__ sfin) {
    constexpr int PARTS = D / (16 * NW);
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int part = bid % PARTS;
    const int sh = bid / PARTS;
    const int h = sh % H;
    const int n = order[sh / H];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, gq = l >> 4;
    const int col = (part * NW + w) * 16 + c;
    const int64_t bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
    const int ci0 = chunk_off[n], ci1 = chunk_off[n + 1];
    const int64_t HD = (int64_t)H * D;

    f32x4 S[8];
    const int64_t sbase = ((int64_t)n * H + h) * D * D + col;
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            S[b][j] = s0 ? s0[sbase + (int64_t)(16 * b + 4 * gq + j) * D] : 0.f;

    if (ci0 < ci1) {
        StepIn cur, nxt;
        load_step(cur, recs + ((int64_t)ci0 * H + h) * Rec::BYTES, v + (bos * H + h) * D + col,
                  HD, (int)min<int64_t>(C, eos - bos));
        for (int ci = ci0; ci < ci1; ++ci) {
            const int64_t t0 = bos + (int64_t)C * (ci - ci0);
            const int nc = (int)min<int64_t>(C, eos - t0);
            if (ci + 1 < ci1) {
                const int64_t t1 = t0 + C;
                load_step(nxt, recs + ((int64_t)(ci + 1) * H + h) * Rec::BYTES,
                          v + (t1 * H + h) * D + col, HD, (int)min<int64_t>(C, eos - t1));
            }
            const f32x4 o = recur_step(cur, S);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * gq + j < nc) out[((t0 + 4 * gq + j) * H + h) * D + col] = o[j];
            cur = nxt;
        }
    }
    if (sfin) {
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) sfin[sbase + (int64_t)(16 * b + 4 * gq + j) * D] = S[b][j];
    }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_chunk_map(const int32_t *cu, int N, int T, int32_t *chunk_off, int32_t *order,
                            hipStream_t st) {
    hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(MAP_THREADS), 0, st, cu, N, T, chunk_off,
                       order);
    return hipGetLastError();
}

hipError_t launch_prep(const uint16_t *q, const uint16_t *k, const float *g, const float *beta,
                       const int32_t *cu, int N, int T, int H, float scale,
                       const int32_t *chunk_off, char *recs, int64_t max_chunks, hipStream_t st) {
    const int64_t blocks = max_chunks * H;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)blocks), dim3(64), 0, st, q, k, g, beta, cu, N,
                       T, H, scale, chunk_off, recs);
    return hipGetLastError();
}

hipError_t launch_recur(const char *recs, const uint16_t *v, const int32_t *cu,
                        const int32_t *chunk_off, const int32_t *order, int N, int T, int H,
                        const float *s0, float *out, float *sfin, int waves, hipStream_t st) {
    const int64_t sh = (int64_t)N * H;
    switch (waves) {
    case 1:
        hipLaunchKernelGGL(recur_kernel<1>, dim3((unsigned)(sh * 8)), dim3(64), 0, st, recs, v, cu,
                           chunk_off, order, N, T, H, s0, out, sfin);
        break;
    case 2:
        hipLaunchKernelGGL(recur_kernel<2>, dim3((unsigned)(sh * 4)), dim3(128), 0, st, recs, v,
                           cu, chunk_off, order, N, T, H, s0, out, sfin);
        break;
    case 4:
        hipLaunchKernelGGL(recur_kernel<4>, dim3((unsigned)(sh * 2)), dim3(256), 0, st, recs, v,
                           cu, chunk_off, order, N, T, H, s0, out, sfin);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kda
