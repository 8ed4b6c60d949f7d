// kda_fused.hip -- the single-kernel KDA forward. Chunk-local intermediates
// never leave the chip: producer waves turn raw q/k/g/beta chunks into chunk
// records in an LDS ring, consumer waves run the sequential state recurrence
// on them, in one workgroup per (sequence, head, value-column part).
//
// Keeping the whole prefill in one kernel, with producers preparing later
// chunks into a small ring of on-chip slots that a consumer drains in order,
// is the organisation the fused B200 kernel in the FlashKDA coverage used
// (smzdm.com, "反转二"); here the ring lives in LDS and the hand-off is
// a pair of per-slot counters in LDS.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

// Bounded spin: a wave that waits longer than this many polls gives up, flags
// the error and leaves its loop, so a logic error cannot hang the device.
constexpr int SPIN_LIMIT = 1 << 24;

__device__ __forceinline__ int lds_load_acquire(int *p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store_release(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_add_release(int *p, int v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Waits until pred(*p) holds; returns false after SPIN_LIMIT polls.
template <class Pred>
__device__ __forceinline__ bool spin_until(int *p, Pred pred) {
    for (int i = 0; i < SPIN_LIMIT; ++i) {
        if (pred(lds_load_acquire(p))) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// NW consumer waves (16 value columns each) + NP producer waves; NSLOT records
// in the LDS ring. Producer p prepares chunks p, p+NP, ...; slot s holds chunks
// s, s+NSLOT, ...; ready[s] = index of the chunk it holds, done[s] = number of
// consumer passes over it so far.
template <int NW, int NP, int NSLOT>
struct FusedLayout {
    static constexpr int FLAGS = 256;                        // ready[NSLOT], done[NSLOT], error
    static constexpr int SLOTS = FLAGS;
    static constexpr int SCRATCH = SLOTS + NSLOT * Rec::BYTES;
    static constexpr int BYTES = SCRATCH + NP * (int)sizeof(PrepLds);
};

template <int NW, int NP, int NSLOT>
__global__ __launch_bounds__(64 * (NW + NP)) void fused_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ order, int N, int T, int H, float scale,
    const float *__restrict__ s0, float *__restrict__ out, float *__restrict__ sfin,
    int *__restrict__ err, int *dev_err) {
    using LY = FusedLayout<NW, NP, NSLOT>;
    static_assert(LY::FLAGS >= (2 * NSLOT + 1) * 4, "flag area too small");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    int *ready = (int *)lds;
    int *done = ready + NSLOT;
    int *failed = done + NSLOT;

    constexpr int PARTS = D / (16 * NW);
    const int bid = xcd_remap(blockIdx.x, gridDim.x, PARTS);
    const int part = bid % PARTS;
    const int sh = bid / PARTS;
    const int h = sh % H;
    const int n = order[sh / H];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, gq = l >> 4;
    const int64_t bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
    const int nch = (int)((eos - bos + C - 1) / C);

    if (threadIdx.x < NSLOT) {
        ready[threadIdx.x] = -1;
        done[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) *failed = 0;
    __syncthreads();

    if (w >= NW) {
        // ------------------------------------------------------------ producer
        const int p = w - NW;
        PrepLds &L = *(PrepLds *)(lds + LY::SCRATCH + p * (int)sizeof(PrepLds));
        for (int i = p; i < nch; i += NP) {
            const int s = i % NSLOT;
            const int need = (i / NSLOT) * NW;   // consumer passes over earlier occupants
            if (!spin_until(&done[s], [&](int x) { return x >= need; })) {
                *failed = 1;
                break;
            }
            if (lds_load_acquire(failed)) break;
            const int64_t t0 = bos + (int64_t)C * i;
            prep_chunk(q, k, g, beta, t0, (int)min<int64_t>(C, eos - t0), h, H, scale, L,
                       lds + LY::SLOTS + s * Rec::BYTES);
            __builtin_amdgcn_s_waitcnt(0);
            if (l == 0) lds_store_release(&ready[s], i);
        }
        return;
    }

    // ---------------------------------------------------------------- consumer
    const int col = (part * NW + w) * 16 + c;
    const int64_t HD = (int64_t)H * D;
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

    // V for this lane's column, rows 4g..4g+3 of a chunk (rows past the end read the
    // last valid row and are zeroed), one chunk ahead of its use
    auto load_v = [&](int i, uint16_t (&vv)[4]) {
        const int ii = i < nch ? i : nch - 1;
        const int64_t t0 = bos + (int64_t)C * ii;
        const int nc = (int)min<int64_t>(C, eos - t0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 4 * gq + j;
            const uint16_t x = v[(t0 + (t < nc ? t : nc - 1)) * HD + (int64_t)h * D + col];
            vv[j] = (t < nc && i < nch) ? x : (uint16_t)0;
        }
    };
    uint16_t vcur[4], vnxt[4];
    if (nch > 0) load_v(0, vcur);
    bool ok = true;
    for (int i = 0; i < nch; ++i) {
        load_v(i + 1, vnxt);
        const int s = i % NSLOT;
        if (!spin_until(&ready[s], [&](int x) { return x == i; })) {
            *failed = 1;
            ok = false;
            break;
        }
        const char *slot = lds + LY::SLOTS + s * Rec::BYTES;
        StepIn st;
        read_rec(st, slot);
        st.v = __builtin_bit_cast(bf16x4, (ushort4{vcur[0], vcur[1], vcur[2], vcur[3]}));
        __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): slot reads landed before release
        if (l == 0) lds_add_release(&done[s], 1);
        const f32x4 o = recur_step(st, S);
        const int64_t t0 = bos + (int64_t)C * i;
        const int nc = (int)min<int64_t>(C, eos - t0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (4 * gq + j < nc) out[((t0 + 4 * gq + j) * H + h) * D + col] = o[j];
#pragma unroll
        for (int j = 0; j < 4; ++j) vcur[j] = vnxt[j];
    }
    if (!ok || lds_load_acquire(failed)) {
        if (l == 0) {
            atomicOr(err, 1);
            if (dev_err) atomicOr(dev_err, 1);
        }
        return;
    }
    if (sfin) {
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) sfin[sbase + (int64_t)(16 * b + 4 * gq + j) * D] = S[b][j];
    }
}

template <int NW, int NP, int NSLOT>
static hipError_t launch_fused_t(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const float *g, const float *beta, const int32_t *cu,
                                 const int32_t *order, int N, int T, int H, float scale,
                                 const float *s0, float *out, float *sfin, int *err,
                                 hipStream_t st) {
    using LY = FusedLayout<NW, NP, NSLOT>;
    auto kern = fused_kernel<NW, NP, NSLOT>;
    static std::atomic<uint64_t> lds_set{0};
    if (const hipError_t e = ensure_lds_limit((const void *)kern, LY::BYTES, lds_set); e != hipSuccess) return e;
    const int64_t blocks = (int64_t)N * H * (D / (16 * NW));
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * (NW + NP)), LY::BYTES, st, q, k,
                       v, g, beta, cu, order, N, T, H, scale, s0, out, sfin, err, device_error_word());
    return hipGetLastError();
}

hipError_t launch_fused(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                        const float *beta, const int32_t *cu, const int32_t *order, int N, int T,
                        int H, float scale, const float *s0, float *out, float *sfin, int *err,
                        int waves, hipStream_t st) {
    // three producer waves: measured on MI355X (config 3, four slices per block, ms per
    // call for 2 | 3 producers and 3 ring slots) 0.206 | 0.164; 3 or 4 producers with 2
    // slots 0.211 (the consumers wait for the ring); 4 producers and 3 slots do not fit
    // in LDS
    switch (waves) {
    case 1: return launch_fused_t<1, 3, 3>(q, k, v, g, beta, cu, order, N, T, H, scale, s0, out, sfin, err, st);
    case 2: return launch_fused_t<2, 3, 3>(q, k, v, g, beta, cu, order, N, T, H, scale, s0, out, sfin, err, st);
    case 4: return launch_fused_t<4, 3, 3>(q, k, v, g, beta, cu, order, N, T, H, scale, s0, out, sfin, err, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
