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
                                                                 int32_t *__restrict__ order,
                                                                 int32_t *__restrict__ err) {
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
    if (tid == 0) {
        chunk_off[0] = 0;
        *err = 0;
    }
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
// NW waves per block, one 16-column state slice each; a block covers 16*NW
// value columns of one (sequence, head). Chunk records and the block's V tile
// stream through an NSLOT-deep LDS ring filled by direct global->LDS loads
// (no registers held while in flight), NSLOT-1 chunks ahead of the compute.
// Blocks of one (sequence, head) get consecutive logical ids; xcd_remap keeps
// them on one XCD so they share the record reads in L2.
template <int NW>
struct Ring {
    static constexpr int REC_LOADS = Rec::BYTES / 1024;              // 1 KiB wave loads
    static constexpr int VCOLS = 16 * NW;                            // value columns per block
    static constexpr int V_BYTES = 16 * VCOLS * 2;                   // [16 tokens][VCOLS] bf16
    static constexpr int V_LOADS = (V_BYTES + 1023) / 1024;
    static constexpr int V_LANE = 16;                                // bytes per lane
    static constexpr int V_LPR = VCOLS * 2 / V_LANE;                 // lanes per token row
    static constexpr int V_ACTIVE = V_BYTES / V_LOADS / V_LANE;      // lanes with data per load
    static constexpr int LOADS = REC_LOADS + V_LOADS;
    static constexpr int SLOT = Rec::BYTES + V_LOADS * 1024;
    static constexpr int loads_of(int w) { return (LOADS - w + NW - 1) / NW; }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]; others left open
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

#define KDA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Issue this wave's share of the loads of one chunk (record + V tile) into an LDS slot.
template <int NW>
__device__ __forceinline__ void ring_fill(char *slot, const char *rec, const uint16_t *v,
                                          int64_t t0, int nc, int h, int H, int vcol0) {
    using R = Ring<NW>;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < R::LOADS; ++i) {
        if (i % NW != w) continue;
        if (i < R::REC_LOADS) {
            __builtin_amdgcn_global_load_lds((const void *)(rec + i * 1024 + l * 16),
                                             KDA_LDS(slot + i * 1024), 16, 0, 0);
        } else {
            const int j = i - R::REC_LOADS;
            const int row = j * (64 / R::V_LPR) + l / R::V_LPR;
            const int col = vcol0 + (l % R::V_LPR) * (R::V_LANE / 2);
            const int64_t t = t0 + (row < nc ? row : nc - 1);   // rows past the end: finite filler
            if (R::V_ACTIVE == 64 || l < R::V_ACTIVE)
                __builtin_amdgcn_global_load_lds((const void *)(v + (t * H + h) * D + col),
                                                 KDA_LDS(slot + Rec::BYTES + j * 1024), R::V_LANE, 0, 0);
        }
    }
}

template <int NW, int NSLOT>
__device__ __forceinline__ void ring_wait(int w) {
    // own loads of the chunk about to be consumed are done once at most the
    // loads of the NSLOT-2 younger chunks are still outstanding
    using R = Ring<NW>;
    if (w == 0) wait_vmcnt<(NSLOT - 2) * R::loads_of(0)>();
    else if (NW > 1 && w == NW - 1) wait_vmcnt<(NSLOT - 2) * R::loads_of(NW > 1 ? NW - 1 : 0)>();
    else wait_vmcnt<(NSLOT - 2) * R::loads_of(NW > 2 ? 1 : 0)>();
}

template <int NW, int NSLOT>
__global__ __launch_bounds__(64 * NW) void recur_kernel(
    const char *__restrict__ recs, const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order, int N, int T, int H,
    const float *__restrict__ s0, float *__restrict__ out, float *__restrict__ sfin) {
    using R = Ring<NW>;
    static_assert(NSLOT >= 2, "ring needs two slots");
    static_assert(R::loads_of(0) - R::loads_of(NW - 1) <= 1, "unbalanced ring loads");
    extern __shared__ __attribute__((aligned(16))) char ring[];
    constexpr int PARTS = D / (16 * NW);
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int part = bid % PARTS;
    const int sh = bid / PARTS;
    const int h = sh % H;
    const int n = order[sh / H];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, gq = l >> 4;
    const int vcol0 = part * R::VCOLS;            // first value column of this block
    const int col = vcol0 + w * 16 + c;           // this lane's value column
    const int64_t bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
    const int ci0 = chunk_off[n], ci1 = chunk_off[n + 1];

    f32x4 S[8];
    const int64_t sbase = ((int64_t)n * H + h) * D * D + col;
    if (s0) {
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[b][j] = s0[sbase + (int64_t)(16 * b + 4 * gq + j) * D];
    } else {
#pragma unroll
        for (int b = 0; b < 8; ++b) S[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int nch = ci1 - ci0;
    // every chunk index past the end is clamped to the last chunk (a harmless reload
    // into a slot nobody reads) so that each wave issues the same loads per step
    auto fill = [&](int it) {
        const int k = it < nch ? it : nch - 1;
        const int64_t t0 = bos + (int64_t)C * k;
        ring_fill<NW>(ring + (it % NSLOT) * R::SLOT, recs + ((int64_t)(ci0 + k) * H + h) * Rec::BYTES,
                      v, t0, (int)min<int64_t>(C, eos - t0), h, H, vcol0);
    };
    if (nch > 0) {
#pragma unroll
        for (int it = 0; it < NSLOT - 1; ++it) fill(it);
        for (int it = 0; it < nch; ++it) {
            ring_wait<NW, NSLOT>(w);
            __builtin_amdgcn_s_barrier();         // all waves: slot it ready, slot it-1 released
            __builtin_amdgcn_sched_barrier(0);
            fill(it + NSLOT - 1);
            __builtin_amdgcn_sched_barrier(0);
            const char *slot = ring + (it % NSLOT) * R::SLOT;
            StepIn st;
            read_rec(st, slot);
            read_vtile(st, (const uint16_t *)(slot + Rec::BYTES), R::VCOLS, w * 16);
            const f32x4 o = recur_step(st, S);
            const int64_t t0 = bos + (int64_t)C * it;
            const int nc = (int)min<int64_t>(C, eos - t0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * gq + j < nc) out[((t0 + 4 * gq + j) * H + h) * D + col] = o[j];
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
                            int32_t *err, hipStream_t st) {
    hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(MAP_THREADS), 0, st, cu, N, T, chunk_off,
                       order, err);
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

template <int NW, int NSLOT>
static hipError_t launch_recur_t(const char *recs, const uint16_t *v, const int32_t *cu,
                                 const int32_t *chunk_off, const int32_t *order, int N, int T,
                                 int H, const float *s0, float *out, float *sfin, hipStream_t st) {
    const size_t lds = (size_t)NSLOT * Ring<NW>::SLOT;
    auto kern = recur_kernel<NW, NSLOT>;
    static bool attr_set = false;   // raising the dynamic LDS limit is per-kernel, idempotent
    if (!attr_set) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess)
            return hipErrorInvalidValue;
        attr_set = true;
    }
    const int64_t blocks = (int64_t)N * H * (D / (16 * NW));
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * NW), lds, st, recs, v, cu,
                       chunk_off, order, N, T, H, s0, out, sfin);
    return hipGetLastError();
}

hipError_t launch_recur(const char *recs, const uint16_t *v, const int32_t *cu,
                        const int32_t *chunk_off, const int32_t *order, int N, int T, int H,
                        const float *s0, float *out, float *sfin, int waves, hipStream_t st) {
    switch (waves) {
    case 1: return launch_recur_t<1, 4>(recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, st);
    case 2: return launch_recur_t<2, 4>(recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, st);
    case 4: return launch_recur_t<4, 3>(recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
