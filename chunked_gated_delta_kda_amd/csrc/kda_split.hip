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

// Write-only sink for the output rows of a partial chunk: the output waves store
// every row unconditionally (rows past the chunk end go here), which keeps their
// stores out of branches so that the waits for their in-flight loads stay exact.
__device__ float store_sink[64];

// ---------------------------------------------------------------- chunk map
// One workgroup. First the sequence offsets are sanitised into cu_safe[N+1]: each
// offset clamped to [0, T] and raised to the largest offset before it, so that the
// ranges are ordered, inside [0, T], and add up to at most T tokens; every later
// kernel reads cu_safe, so malformed cu_seqlens cannot send an access outside the
// inputs, the outputs or the workspace (whose record area is sized for T tokens).
// The error word is set to ERR_CU_SEQLENS when the offsets were not 0 = c_0 <= c_1
// <= ... <= c_N = T (and the bit is ORed into the device error word). Then chunk_off[n] = number of cl-token chunks before sequence n
// (chunk_off[N] = total), and order[] lists sequences longest first (ties by index)
// when N <= ORDER_MAX, else in input order.
constexpr int MAP_THREADS = 256;
constexpr int ORDER_MAX = 2048;
constexpr int ERR_CU_SEQLENS = 2;   // (bit 0 is the fused kernel's wait timeout)

// Inclusive scan over the workgroup (MAP_THREADS threads): shuffles within each wave,
// then one exchange of the wave totals through LDS. op is max or +; both treat 0 as
// the identity for the non-negative values scanned here.
template <bool MAX>
__device__ __forceinline__ int32_t block_scan(int32_t v, int32_t *wsum) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(v, off);
        if (lane >= off) v = MAX ? max(v, y) : v + y;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    int32_t pre = 0;
    for (int i = 0; i < w; ++i) pre = MAX ? max(pre, wsum[i]) : pre + wsum[i];
    __syncthreads();   // wsum free for the next scan
    return MAX ? max(pre, v) : pre + v;
}

__global__ __launch_bounds__(MAP_THREADS) void chunk_map_kernel(const int32_t *__restrict__ cu,
                                                                 int N, int T,
                                                                 int32_t *__restrict__ cu_safe,
                                                                 int32_t *__restrict__ chunk_off,
                                                                 int32_t *__restrict__ order,
                                                                 int32_t *__restrict__ err,
                                                                 int32_t *dev_err, int cl) {
    __shared__ int32_t wsum[MAP_THREADS / 64];
    __shared__ int32_t last;   // the scan's last value: the carry into the next MAP_THREADS
    __shared__ int32_t lcs[ORDER_MAX + 1];   // the sanitised offsets again, for N <= ORDER_MAX
    const int tid = threadIdx.x;
    const bool in_lds = N <= ORDER_MAX;
    // sanitised offsets: running maximum of the clamped offsets
    int bad = 0;
    int32_t carry = 0;   // the same in every thread
    for (int base = 0; base <= N; base += MAP_THREADS) {
        const int n = base + tid;
        int32_t x = 0;
        if (n <= N) {
            const int32_t raw = cu ? cu[n] : (n == 0 ? 0 : T);
            x = min(max(raw, 0), T);
            if (n == 0) bad |= raw != 0;
            else bad |= raw < (cu ? cu[n - 1] : 0);
            if (n == N) bad |= raw != T;
        }
        const int32_t m = max(carry, block_scan<true>(x, wsum));
        if (n <= N) {
            cu_safe[n] = m;
            if (in_lds) lcs[n] = m;
        }
        if (tid == MAP_THREADS - 1) last = m;
        __syncthreads();
        carry = last;
        __syncthreads();
    }
    bad = __syncthreads_or(bad);
    // chunk counts of the sanitised ranges (written by this workgroup above)
    const int32_t *cs = in_lds ? lcs : cu_safe;
    carry = 0;
    for (int base = 0; base < N; base += MAP_THREADS) {
        const int n = base + tid;
        const int32_t c = n < N ? (cs[n + 1] - cs[n] + cl - 1) / cl : 0;
        const int32_t incl = carry + block_scan<false>(c, wsum);
        if (n < N) chunk_off[n + 1] = incl;
        if (tid == MAP_THREADS - 1) last = incl;
        __syncthreads();
        carry = last;
        __syncthreads();
    }
    if (tid == 0) {
        chunk_off[0] = 0;
        *err = bad ? ERR_CU_SEQLENS : 0;
        if (bad && dev_err) atomicOr(dev_err, ERR_CU_SEQLENS);
    }
    if (in_lds) {
        for (int n = tid; n < N; n += MAP_THREADS) {
            const int32_t ln = lcs[n + 1] - lcs[n];
            int rank = 0;
            for (int m = 0; m < N; ++m) {
                const int32_t lm = lcs[m + 1] - lcs[m];
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
// Record of chunk ci (global index), head h.
__device__ __forceinline__ void prep_one(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                         const float *__restrict__ g, const float *__restrict__ beta,
                                         const int32_t *__restrict__ cu, int N, int T, int H,
                                         float scale, const int32_t *__restrict__ chunk_off,
                                         char *__restrict__ recs, int ci, int h, PrepLds &L) {
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


__global__ __launch_bounds__(64) void prep_kernel(const uint16_t *__restrict__ q,
                                                  const uint16_t *__restrict__ k,
                                                  const float *__restrict__ g,
                                                  const float *__restrict__ beta,
                                                  const int32_t *__restrict__ cu, int N, int T,
                                                  int H, float scale,
                                                  const int32_t *__restrict__ chunk_off,
                                                  char *__restrict__ recs, int fb, int fe) {
    __shared__ PrepLds L;
    int h;
    const int ci = seg_chunk_of(chunk_off, N, H, fb, fe, blockIdx.x, h);
    if (ci < 0) return;
    prep_one(q, k, g, beta, cu, N, T, H, scale, chunk_off, recs, ci, h, L);
}

// ---------------------------------------------------------------- recurrence
// NW waves per block, one 16-column state slice each; a block covers 16*NW
// value columns of one (sequence, head). Chunk records and the block's V tile
// stream through an NSLOT-deep LDS ring filled by direct global->LDS loads
// (no registers held while in flight), NSLOT-1 chunks ahead of the compute.
// Blocks of one (sequence, head) get consecutive logical ids; xcd_remap keeps
// them on one XCD so they share the record reads in L2, and deals chains to XCDs in turn.
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


// Issue this wave's share of the loads of one chunk (record + V tile) into an LDS slot.
// (NSLOT only makes each ring shape its own specialization: clang's host pass rejects a
// second instantiation of this device template from another kernel specialization.)
template <int NW, int NSLOT>
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

// Loads of a sequence's chunk `it` (of nch) into its ring slot. Every chunk index past
// the end is clamped to the last chunk (a harmless reload into a slot nobody reads) so
// that each wave issues the same loads per step.
template <int NW, int NSLOT>
__device__ __forceinline__ void ring_fill_chunk(char *ring, int it, int nch, int64_t bos, int64_t eos, int ci0,
                                                const char *recs, const uint16_t *v, int h, int H, int vcol0) {
    const int k = it < nch ? it : nch - 1;
    const int64_t t0 = bos + (int64_t)C * k;
    ring_fill<NW, NSLOT>(ring + (it % NSLOT) * Ring<NW>::SLOT, recs + ((int64_t)(ci0 + k) * H + h) * Rec::BYTES, v, t0,
                  (int)min<int64_t>(C, eos - t0), h, H, vcol0);
}

template <int NW, int NSLOT, int W = 0>
__device__ __forceinline__ void ring_wait(int w) {
    // own loads of the chunk about to be consumed are done once at most the
    // loads of the NSLOT-2 younger chunks are still outstanding (wave W issues
    // loads_of(W) loads per chunk; w is uniform across the wave)
    using R = Ring<NW>;
    if constexpr (W + 1 < NW) {
        if (w != W) {
            ring_wait<NW, NSLOT, W + 1>(w);
            return;
        }
    }
    wait_vmcnt<(NSLOT - 2) * R::loads_of(W)>();
}

// Segments [fb, fe) of every sequence as in the paired recurrence below: the state
// enters from s0 (or zeros) at a sequence's first chunk and from `carry` otherwise, and
// leaves to sfin after its last chunk and to `carry` otherwise.
template <int NW, int NSLOT>
__device__ __forceinline__ void recur_ring_block(
    int bid, char *ring, const char *__restrict__ recs, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order,
    int N, int T, int H, const float *s0, float *__restrict__ out, float *sfin, float *carry, int fb,
    int fe) {
    using R = Ring<NW>;
    static_assert(NSLOT >= 2, "ring needs two slots");
    static_assert(R::loads_of(0) - R::loads_of(NW - 1) <= 1, "unbalanced ring loads");
    constexpr int PARTS = D / (16 * NW);
    const int part = bid % PARTS;
    const int sh = bid / PARTS;
    const int h = sh % H;
    const int n = order[sh / H];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, gq = l >> 4;
    const int vcol0 = part * R::VCOLS;            // first value column of this block
    const int col = vcol0 + w * 16 + c;           // this lane's value column
    const int64_t seq_bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
    const int seq_c0 = chunk_off[n], seq_c1 = chunk_off[n + 1];
    const int ci0 = seq_c0 + seg_chunk(seq_c1 - seq_c0, fb);   // this launch's chunks of the sequence
    const int ci1 = seq_c0 + seg_chunk(seq_c1 - seq_c0, fe);
    // a sequence without chunks copies its initial state in the first segment
    if (ci0 >= ci1 && !(seq_c0 == seq_c1 && fb == 0)) return;
    const int64_t bos = seq_bos + (int64_t)C * (ci0 - seq_c0);
    const float *sin = ci0 == seq_c0 ? s0 : carry;
    float *sout = ci1 == seq_c1 ? sfin : carry;

    f32x4 S[8];
    const int64_t sbase = ((int64_t)n * H + h) * D * D + col;
    if (sin) {
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[b][j] = sin[sbase + (int64_t)(16 * b + 4 * gq + j) * D];
    } else {
#pragma unroll
        for (int b = 0; b < 8; ++b) S[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int nch = ci1 - ci0;
    if (nch > 0) {
#pragma unroll
        for (int it = 0; it < NSLOT - 1; ++it)
            ring_fill_chunk<NW, NSLOT>(ring, it, nch, bos, eos, ci0, recs, v, h, H, vcol0);
        for (int it = 0; it < nch; ++it) {
            ring_wait<NW, NSLOT>(w);
            __builtin_amdgcn_s_barrier();         // all waves: slot it ready, slot it-1 released
            __builtin_amdgcn_sched_barrier(0);
            ring_fill_chunk<NW, NSLOT>(ring, it + NSLOT - 1, nch, bos, eos, ci0, recs, v, h, H, vcol0);
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
    if (sout) {
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) sout[sbase + (int64_t)(16 * b + 4 * gq + j) * D] = S[b][j];
    }
}

template <int NW, int NSLOT>
__global__ __launch_bounds__(64 * NW) void recur_kernel(
    const char *__restrict__ recs, const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order, int N, int T, int H,
    const float *__restrict__ s0, float *__restrict__ out, float *__restrict__ sfin) {
    extern __shared__ __attribute__((aligned(16))) char ring[];
    recur_ring_block<NW, NSLOT>(xcd_remap(blockIdx.x, gridDim.x, D / (16 * NW)), ring, recs, v, cu, chunk_off,
                                order, N, T, H, s0, out, sfin, sfin, 0, SEG_ONE);
}


// ---------------------------------------------------------------- paired recurrence
// NW 16-column slices per block; per slice one chain wave and two output waves.
// The chain wave (w < NW) runs only the state chain: V_new = U - W S (state hi
// part), S <- D S + K~^T V_new; each chunk it publishes the pre-update state
// (fp32) and V_new (hi|lo) in a snapshot. Output wave parity p (chunks m with
// m % 2 == p) forms O = Q+ S + P V_new of its chunk off the chain, in two halves
// over the two chunks after it (key blocks 0-3, then 4-7 and P V_new), so that
// each output wave does half a chunk of work per chunk. One barrier per chunk
// (the ring's); snapshots rotate through three buffers. A dedicated loader wave
// issues every ring load.
// Waves w and w+4 of a block share a SIMD (and its matrix unit), so the roles are
// placed to keep each chain wave's SIMD free of output work:
//   NW = 1: chain 0 | output p0 | output p1 | loader
//   NW = 2: chain 0, chain 1 | output (slice 0, p0), (slice 1, p0) | loader | idle |
//           output (slice 0, p1), (slice 1, p1)
// (the idle wave only keeps the barrier count, so that SIMD 1 hosts chain 1 alone).
// Ring depth (chunks) of the paired recurrence. Measured on MI355X (ms per call, ring of
// 4 | 5 | 6): one slice per block, 65536 tokens x 8 heads 2.275 | 2.174 | 2.168, 8192 x 32
// 0.428 | 0.423 | 0.422; two slices per block, 8192 x 32 0.430 | 0.437 | 0.440 and 8 x
// 1024 x 16 0.187 | 0.190 | 0.191.
template <int NW>
constexpr int pair_nslot() { return NW == 1 ? 5 : 4; }


// A launch covers the segment [fb, fe) of every sequence (seg_chunk; launches over
// consecutive segments, in order on one stream, cover a batch). A sequence's state
// enters from initial_state (or zeros) at its first chunk and from `carry` otherwise,
// and leaves to final_state after its last chunk and to `carry` otherwise (carry may
// be final_state itself). Sequences without chunks copy initial to final state in
// the launch of the first segment. With zero_v the chain runs as if every v were 0 (the
// part of the chain that is linear in the entry state alone; outputs are then not valid).
template <int NW, int NSLOT>
__device__ __forceinline__ void recur_pair_block(
    int bid, char *ring, const char *__restrict__ recs, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off,
    const int32_t *__restrict__ order, int N, int T, int H, const float *s0,
    float *__restrict__ out, float *sfin, float *carry, int fb, int fe, bool zero_v = false) {
    using R = Ring<NW>;         // V tile geometry of NW slices
    using PL = PairLayout<NW>;
    constexpr int REC_LOADS = Rec::CHAIN / 1024;       // the chain's part of the record
    constexpr int LOADS = REC_LOADS + R::V_LOADS;
    constexpr int SLOT = Rec::CHAIN + R::V_LOADS * 1024;
    static_assert(NSLOT >= 3, "the chain reads one chunk ahead of the one it computes");
    static_assert((NSLOT - 2) * LOADS < 64, "ring deeper than the vmcnt range");
    char *snaps = ring + NSLOT * SLOT;

    constexpr int PARTS = D / (16 * NW);
    const int part = bid % PARTS;
    const int sh = bid / PARTS;
    const int h = sh % H;
    const int n = order[sh / H];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, gq = l >> 4;
    const bool chain = w < NW;
    const bool loader = w == PL::LOADER;     // issues every ring load; computes nothing
    const bool idle = w == PL::IDLE;
    const int parity = (w == PL::out_wave(0, 1) || w == PL::out_wave(NW - 1, 1)) ? 1 : 0;
    const int slice = chain ? w : ((loader || idle) ? 0 : (w == PL::out_wave(0, parity) ? 0 : 1));
    const int vcol0 = part * R::VCOLS;
    const int col = vcol0 + slice * 16 + c;
    const int64_t seq_bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
    const int seq_c0 = chunk_off[n], seq_c1 = chunk_off[n + 1];
    const int ci0 = seq_c0 + seg_chunk(seq_c1 - seq_c0, fb);   // this launch's chunks of the sequence
    const int ci1 = seq_c0 + seg_chunk(seq_c1 - seq_c0, fe);
    const int64_t sbase = ((int64_t)n * H + h) * D * D + col;
    if (ci0 >= ci1) {
        if (seq_c0 == seq_c1 && fb == 0 && chain && sfin) {
#pragma unroll
            for (int b = 0; b < 8; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t o = sbase + (int64_t)(16 * b + 4 * gq + j) * D;
                    sfin[o] = s0 ? s0[o] : 0.f;
                }
        }
        return;
    }
    const int nch = ci1 - ci0;
    const int64_t bos = seq_bos + (int64_t)C * (ci0 - seq_c0);   // first token of this launch's part
    const float *sin = ci0 == seq_c0 ? s0 : carry;
    float *sout = ci1 == seq_c1 ? sfin : carry;
    auto snap_of = [&](int it) { return snaps + ((it % PL::SNAPS) * NW + slice) * PL::SNAP; };
    auto sync = [] {
        __builtin_amdgcn_s_barrier();      // slots it, it+1 ready; slot it-1 released
        __builtin_amdgcn_sched_barrier(0);
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bf16x4 z4 = {};

    if (loader) {
        // ring fill (the vector-memory pipe is busy for most of a chunk's worth of
        // time; no compute wave waits on it). Sharing the loads with the idle wave,
        // one loading wave on each chain wave's SIMD, measured slower.
        auto fill = [&](int it) {
            const int k = it < nch ? it : nch - 1;
            const int64_t t0 = bos + (int64_t)C * k;
            const int nc = (int)min<int64_t>(C, eos - t0);
            char *slot = ring + (it % NSLOT) * SLOT;
            const char *rec = recs + ((int64_t)(ci0 + k) * H + h) * Rec::BYTES;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                if (i < REC_LOADS) {
                    __builtin_amdgcn_global_load_lds((const void *)(rec + i * 1024 + l * 16),
                                                     KDA_LDS(slot + i * 1024), 16, 0, 0);
                } else {
                    const int j = i - REC_LOADS;
                    const int row = j * (64 / R::V_LPR) + l / R::V_LPR;
                    const int cc = vcol0 + (l % R::V_LPR) * (R::V_LANE / 2);
                    const int64_t t = t0 + (row < nc ? row : nc - 1);
                    if (R::V_ACTIVE == 64 || l < R::V_ACTIVE)
                        __builtin_amdgcn_global_load_lds((const void *)(v + (t * H + h) * D + cc),
                                                         KDA_LDS(slot + Rec::CHAIN + j * 1024), 16, 0, 0);
                }
            }
        };
#pragma unroll
        for (int it = 0; it < NSLOT - 1; ++it) fill(it);
        for (int it = 0; it < nch; ++it) {
            // chunks it and it+1 have landed once at most the loads of the NSLOT-3
            // younger chunks remain outstanding
            wait_vmcnt<(NSLOT - 3) * LOADS>();
            sync();
            fill(it + NSLOT - 1);
        }
        sync();
        sync();
        wait_vmcnt<0>();     // no ring write still in flight when the wave ends
        return;
    }

    if (idle) {
        for (int it = 0; it < nch + 2; ++it) sync();
        return;
    }

    if (chain) {
        f32x4 S[8];
        if (sin) {
#pragma unroll
            for (int b = 0; b < 8; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) S[b][j] = sin[sbase + (int64_t)(16 * b + 4 * gq + j) * D];
        } else {
#pragma unroll
            for (int b = 0; b < 8; ++b) S[b] = zero;
        }
        // inputs of one chunk, read from its ring slot one chunk ahead of use
        struct ChainIn {
            bf16x8 wn[4], kt[8], tb;
            f32x2 e;             // lane-permuted state decay
            uint16_t vv[4];      // V[4g+j][col], combined only where used
        };
        auto chain_read = [&](ChainIn &x, int it) {
            const char *slot = ring + (it % NSLOT) * SLOT;
            x.tb = *(const bf16x8 *)(slot + Rec::TB + l * 16);
            const uint16_t *vt = (const uint16_t *)(slot + Rec::CHAIN);
#pragma unroll
            for (int j = 0; j < 4; ++j) x.vv[j] = zero_v ? (uint16_t)0 : vt[(4 * gq + j) * R::VCOLS + slice * 16 + c];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) x.wn[kb] = *(const bf16x8 *)(slot + Rec::WN + kb * 1024 + l * 16);
#pragma unroll
            for (int b = 0; b < 8; ++b) x.kt[b] = *(const bf16x8 *)(slot + Rec::KT + b * 1024 + l * 16);
            x.e = *(const f32x2 *)(slot + Rec::EGP + l * 8);
        };
        // one chunk: publish S (pre-update) and V_new, then update S
        auto chain_step = [&](const ChainIn &x, int it) {
            char *snap = snap_of(it);
            bf16x8 shi[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) shi[kb] = cat(to_bf16x4(S[2 * kb]), to_bf16x4(S[2 * kb + 1]));
            // combine the V values here, not where they were read (the compiler would
            // otherwise do it at the read and wait for the read to land)
            uint32_t v0 = x.vv[0], v1 = x.vv[1], v2 = x.vv[2], v3 = x.vv[3];
            asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
            const bf16x4 vin = __builtin_bit_cast(bf16x4, (uint2{v0 | (v1 << 16), v2 | (v3 << 16)}));
            // U - W S over four independent accumulators (plus T Diag(beta) V)
            f32x4 a0 = mfma(x.wn[0], shi[0], zero), a1 = mfma(x.wn[1], shi[1], zero);
            f32x4 a2 = mfma(x.wn[2], shi[2], zero), a3 = mfma(x.wn[3], shi[3], zero);
            const f32x4 u = mfma(x.tb, cat(vin, vin), zero);
            // the decayed state, formed while the products above run
            f32x4 Sd[8];
            Sd[0] = decay_block<0>(S[0], x.e);
            Sd[1] = decay_block<1>(S[1], x.e);
            Sd[2] = decay_block<2>(S[2], x.e);
            Sd[3] = decay_block<3>(S[3], x.e);
            Sd[4] = decay_block<4>(S[4], x.e);
            Sd[5] = decay_block<5>(S[5], x.e);
            Sd[6] = decay_block<6>(S[6], x.e);
            Sd[7] = decay_block<7>(S[7], x.e);
#pragma unroll
            for (int b = 0; b < 8; ++b) *(f32x4 *)(snap + (b * 64 + l) * 16) = S[b];
            bf16x4 vh, vl;
            split4((a0 + a1) + (a2 + a3) + u, vh, vl);
            *(bf16x8 *)(snap + 8 * 64 * 16 + l * 16) = cat(vh, vl);
            const bf16x8 vhh = cat(vh, vh), vl0 = cat(vl, z4);
            // two passes over each half of the key blocks so that no MFMA waits on
            // the one just before it
#pragma unroll
            for (int hb = 0; hb < 8; hb += 4) {
                f32x4 tmp[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) tmp[b] = mfma(x.kt[hb + b], vhh, Sd[hb + b]);
#pragma unroll
                for (int b = 0; b < 4; ++b) S[hb + b] = mfma(x.kt[hb + b], vl0, tmp[b]);
            }
        };

        // After each barrier every LDS access of the wave issued before it (a chunk
        // ago) is waited for explicitly: the LDS counter completes in order and
        // counts at most 15, so waits placed per use after the next chunk's reads
        // have been issued would also wait for those.
        auto sync_chain = [&] {
            sync();
            __builtin_amdgcn_s_waitcnt(0xc07f);
        };
        // the first chunk's inputs are read (and waited for) before the loop, so that
        // every step starts with its inputs complete
        ChainIn A, B;
        sync();
        chain_read(A, 0);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        for (int it = 0; it < nch; it += 2) {   // unrolled by two: A and B alternate
            if (it + 1 < nch) chain_read(B, it + 1);
            chain_step(A, it);
            if (it + 1 >= nch) break;
            sync_chain();
            if (it + 2 < nch) chain_read(A, it + 2);
            chain_step(B, it + 1);
            if (it + 2 >= nch) break;
            sync_chain();
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);     // the last snapshot is written
        sync();
        sync();
        if (sout) {
#pragma unroll
            for (int b = 0; b < 8; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) sout[sbase + (int64_t)(16 * b + 4 * gq + j) * D] = S[b][j];
        }
        return;
    }

    // ---- output wave: chunks m = parity, parity + 2, ...; the first half of chunk
    // m's output after barrier m+1, the rest after barrier m+2. Its Q+ and P pieces
    // come straight from global memory into registers, four chunks ahead.
    struct OutIn {
        bf16x8 qh[4], ql[4], pp;
    };
    auto load = [&](OutIn &x, int m) {
        const char *rec = recs + ((int64_t)(ci0 + m) * H + h) * Rec::BYTES;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            x.qh[kb] = *(const bf16x8 *)(rec + Rec::QH + kb * 1024 + l * 16);
            x.ql[kb] = *(const bf16x8 *)(rec + Rec::QL + kb * 1024 + l * 16);
        }
        x.pp = *(const bf16x8 *)(rec + Rec::PP + l * 16);
    };
    f32x4 oa = zero, ob = zero;
    auto half_qs = [&](const OutIn &x, int m, int kb0) {
        const char *snap = snap_of(m);
#pragma unroll
        for (int kb = kb0; kb < kb0 + 2; ++kb) {
            const f32x4 a = *(const f32x4 *)(snap + ((2 * kb) * 64 + l) * 16);
            const f32x4 b = *(const f32x4 *)(snap + ((2 * kb + 1) * 64 + l) * 16);
            bf16x4 ah, al, bh, bl;
            split4(a, ah, al);
            split4(b, bh, bl);
            const bf16x8 shi = cat(ah, bh), slo = cat(al, bl);
            oa = mfma(x.qh[kb], shi, oa);
            ob = mfma(x.qh[kb], slo, ob);
            oa = mfma(x.ql[kb], shi, oa);
        }
    };
    auto first = [&](const OutIn &x, int m) {
        oa = zero;
        ob = zero;
        half_qs(x, m, 0);
        __builtin_amdgcn_s_waitcnt(0xc07f);   // snapshot reads done before the next barrier
    };
    auto finish = [&](const OutIn &x, int m) {
        const char *snap = snap_of(m);
        const bf16x8 vs = *(const bf16x8 *)(snap + 8 * 64 * 16 + l * 16);   // V_new hi | lo
        half_qs(x, m, 2);
        const bf16x4 vh = __builtin_shufflevector(vs, vs, 0, 1, 2, 3);
        const bf16x4 vl = __builtin_shufflevector(vs, vs, 4, 5, 6, 7);
        ob = mfma(x.pp, cat(vh, vh), ob);
        ob = mfma(x.pp, cat(vl, z4), ob);
        const f32x4 o = oa + ob;
        const int64_t t0 = bos + (int64_t)C * m;
        const int nc = (int)min<int64_t>(C, eos - t0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float *dst = 4 * gq + j < nc ? out + ((t0 + 4 * gq + j) * H + h) * D + col : store_sink + l;
            *dst = o[j];
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
    };
    OutIn X, Y;                      // chunks m = parity + 4i and parity + 4i + 2
    // loads are issued unconditionally (past the end they repeat the last chunk), so
    // that the compiler can count them exactly in its waits
    auto cl = [&](int m) { return m < nch ? m : nch - 1; };
    load(X, cl(parity));
    load(Y, cl(parity + 2));
    int nb = 0;
    for (; nb < parity + 1; ++nb) sync();
    for (int m = parity; m < nch; m += 4) {
        sync(); ++nb;
        first(X, m);
        sync(); ++nb;
        finish(X, m);
        load(X, cl(m + 4));
        if (m + 2 >= nch) break;
        sync(); ++nb;
        first(Y, m + 2);
        sync(); ++nb;
        finish(Y, m + 2);
        load(Y, cl(m + 6));
    }
    for (; nb < nch + 2; ++nb) sync();
}

template <int NW, int NSLOT>
struct PairLds {
    static constexpr int BYTES = NSLOT * (Rec::CHAIN + Ring<NW>::V_LOADS * 1024) +
                                 PairLayout<NW>::SNAPS * NW * PairLayout<NW>::SNAP;
};


template <int NW, int NSLOT>
__global__ __launch_bounds__(64 * PairLayout<NW>::WAVES) void recur_pair_kernel(
    const char *__restrict__ recs, const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order, int N, int T, int H,
    const float *s0, float *__restrict__ out, float *sfin, float *carry, int fb, int fe) {
    extern __shared__ __attribute__((aligned(16))) char ring[];
    recur_pair_block<NW, NSLOT>(xcd_remap(blockIdx.x, gridDim.x, D / (16 * NW)), ring, recs, v, cu, chunk_off,
                                order, N, T, H, s0, out, sfin, carry, fb, fe);
}

// ---------------------------------------------------------------- per-chain choice of shape
// Many chains of unequal length: the paired form has the lowest latency per chunk but
// holds a CU per 32 columns of one chain; the eight-wave ring form (one block per
// chain, each wave forming its own outputs) moves more chain-chunks per CU but takes
// ~3x longer per chunk. The chains that set the end time are those longer than the
// balanced share of a CU, (all chains' chunks) / 256 CUs: they get four paired blocks
// (two 16-column slices each), every other chain one eight-wave block. Sequences come
// longest first, so the long chains are the first L of the order and their blocks are
// dispatched first. The grid is sized for the case where every chain is long; blocks
// past the ones in use exit at the end of the grid (spare blocks interleaved with
// working ones were measured to halve the working blocks' throughput).
// Over segments [fb, fe) (as the paired recurrence above; by default the form runs
// whole), blocks from 4 N H on prepare the records of the next segment [pb, pe),
// HYBRID_PREP_WAVES chunk-heads per block, as in recur_prep_kernel. They are dispatched
// after every recurrence block.
constexpr int HYBRID_RING = 4;   // ring depth of the eight-wave blocks (fits in the paired block's LDS)
constexpr int HYBRID_PREP_WAVES = 4;

template <int NSLOT>
__global__ __launch_bounds__(64 * PairLayout<2>::WAVES) void recur_hybrid_kernel(
    const char *__restrict__ recs, const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order, int N, int T, int H,
    const float *s0, float *__restrict__ out, float *sfin, float *carry, int fb, int fe,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, float scale, char *__restrict__ recs_out, int pb, int pe) {
    static_assert(PairLayout<2>::WAVES == 8, "both shapes run eight waves");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int NH = N * H;
    const int b = blockIdx.x;
    if (b >= 4 * NH) {
        constexpr int PW = HYBRID_PREP_WAVES;
        const int w = threadIdx.x >> 6;
        if (w >= PW) return;
        const int64_t idx = (int64_t)(b - 4 * NH) * PW + w;
        int h;
        const int ci = seg_chunk_of(chunk_off, N, H, pb, pe, idx, h);
        if (ci < 0) return;
        prep_one(q, k, g, beta, cu, N, T, H, scale, chunk_off, recs_out, ci, h,
                 *(PrepLds *)(lds + w * (int)sizeof(PrepLds)));
        return;
    }
    const int64_t share = ((int64_t)chunk_off[N] * H + 255) / 256;
    int nlong = 0;   // sequences with more chunks than the share (the same count in every block)
    for (int base = 0; base < N; base += 64 * PairLayout<2>::WAVES) {
        const int s = base + (int)threadIdx.x;
        nlong += __syncthreads_count(s < N && chunk_off[s + 1] - chunk_off[s] > share);
    }
    const int L = nlong * H;              // long chains: the first L in chain order
    if (b < 4 * L) {
        recur_pair_block<2, NSLOT>(xcd_remap(b, 4 * L, 4), lds, recs, v, cu, chunk_off, order, N, T, H, s0, out,
                                   sfin, carry, fb, fe);
    } else if (b < 4 * L + (NH - L)) {
        recur_ring_block<8, HYBRID_RING>(L + xcd_remap(b - 4 * L, NH - L, 1), lds, recs, v, cu, chunk_off, order,
                                         N, T, H, s0, out, sfin, carry, fb, fe);
    }
}

// ---------------------------------------------------------------- recurrence + next prep
// One launch that runs the paired recurrence over the segment [fb, fe) in
// blocks [0, RB) and prepares the records of the next segment [pb, pe) in the
// remaining blocks, PREP_WAVES chunk-heads per block (one per wave). Workgroups
// are dispatched in index order and the LDS request admits one block per CU, so
// the recurrence blocks take their CUs first and the prep blocks fill the CUs
// the recurrence leaves idle, instead of waiting for the recurrence to finish.
template <int NW>
struct RecurPrep {
    static constexpr int PREP_WAVES = PairLayout<NW>::WAVES < 4 ? PairLayout<NW>::WAVES : 4;
};

template <int NW, int NSLOT>
__global__ __launch_bounds__(64 * PairLayout<NW>::WAVES) void recur_prep_kernel(
    const char *__restrict__ recs_in, const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order, int N, int T, int H,
    const float *s0, float *__restrict__ out, float *sfin, float *carry, int fb, int fe, int RB,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, float scale, char *__restrict__ recs_out, int pb, int pe) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    if ((int)blockIdx.x < RB) {
        recur_pair_block<NW, NSLOT>(xcd_remap(blockIdx.x, RB, D / (16 * NW)), lds, recs_in, v, cu, chunk_off,
                                    order, N, T, H, s0, out, sfin, carry, fb, fe);
        return;
    }
    constexpr int PW = RecurPrep<NW>::PREP_WAVES;
    const int w = threadIdx.x >> 6;
    if (w >= PW) return;
    const int64_t idx = (int64_t)(blockIdx.x - RB) * PW + w;
    int h;
    const int ci = seg_chunk_of(chunk_off, N, H, pb, pe, idx, h);
    if (ci < 0) return;
    prep_one(q, k, g, beta, cu, N, T, H, scale, chunk_off, recs_out, ci, h,
             *(PrepLds *)(lds + w * (int)sizeof(PrepLds)));
}

// ---------------------------------------------------------------- launchers
hipError_t launch_chunk_map(const int32_t *cu, int N, int T, int32_t *cu_safe, int32_t *chunk_off,
                            int32_t *order, int32_t *err, int cl, hipStream_t st) {
    hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(MAP_THREADS), 0, st, cu, N, T, cu_safe, chunk_off,
                       order, err, device_error_word(), cl);
    return hipGetLastError();
}

hipError_t launch_prep(const uint16_t *q, const uint16_t *k, const float *g, const float *beta,
                       const int32_t *cu, int N, int T, int H, float scale,
                       const int32_t *chunk_off, char *recs, int fb, int fe, int64_t M,
                       hipStream_t st) {
    const int64_t blocks = seg_chunks_bound(M, N, fb, fe) * H;
    if (blocks <= 0 || fe <= fb) return hipSuccess;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)blocks), dim3(64), 0, st, q, k, g, beta, cu, N,
                       T, H, scale, chunk_off, recs, fb, fe);
    return hipGetLastError();
}

template <int NW, int NSLOT>
static hipError_t launch_recur_t(const char *recs, const uint16_t *v, const int32_t *cu,
                                 const int32_t *chunk_off, const int32_t *order, int N, int T,
                                 int H, const float *s0, float *out, float *sfin, hipStream_t st) {
    const size_t lds = (size_t)NSLOT * Ring<NW>::SLOT;
    auto kern = recur_kernel<NW, NSLOT>;
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)kern, (int)lds, lds_set) != hipSuccess) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)N * H * (D / (16 * NW));
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * NW), lds, st, recs, v, cu,
                       chunk_off, order, N, T, H, s0, out, sfin);
    return hipGetLastError();
}

template <int NW, int NSLOT>
static hipError_t launch_recur_pair(const char *recs, const uint16_t *v, const int32_t *cu,
                                    const int32_t *chunk_off, const int32_t *order, int N, int T,
                                    int H, const float *s0, float *out, float *sfin, float *carry,
                                    int fb, int fe, hipStream_t st) {
    constexpr int lds = PairLds<NW, NSLOT>::BYTES;
    static_assert(lds <= 160 * 1024, "LDS");
    auto kern = recur_pair_kernel<NW, NSLOT>;
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)kern, lds, lds_set) != hipSuccess) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)N * H * (D / (16 * NW));
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * PairLayout<NW>::WAVES), lds, st,
                       recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, carry, fb, fe);
    return hipGetLastError();
}

// a.fb..a.fe: the recurrence's segment; a.pb..a.pe: the segment to prepare (none if equal)
static hipError_t launch_recur_hybrid(const RecurPrepArgs &a, hipStream_t st) {
    constexpr int pair = PairLds<2, pair_nslot<2>()>::BYTES;
    constexpr int ring = HYBRID_RING * Ring<8>::SLOT;
    constexpr int rl = pair > ring ? pair : ring;
    constexpr int prep = HYBRID_PREP_WAVES * (int)sizeof(PrepLds);
    constexpr int lds = rl > prep ? rl : prep;
    // more than 80 KiB: never two blocks on one CU
    static_assert(lds <= 160 * 1024 && lds > 80 * 1024, "LDS");
    auto kern = recur_hybrid_kernel<pair_nslot<2>()>;
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)kern, lds, lds_set) != hipSuccess) return hipErrorInvalidValue;
    constexpr int PW = HYBRID_PREP_WAVES;
    const int64_t rb = (int64_t)a.N * a.H * 4;
    const int64_t pblocks = a.pe > a.pb ? (seg_chunks_bound(a.M, a.N, a.pb, a.pe) * a.H + PW - 1) / PW : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)(rb + pblocks)), dim3(64 * PairLayout<2>::WAVES), lds, st, a.recs,
                       a.v, a.cu, a.chunk_off, a.order, a.N, a.T, a.H, a.s0, a.out, a.sfin, a.carry, a.fb, a.fe,
                       a.q, a.k, a.g, a.beta, a.scale, a.recs, a.pb, a.pe);
    return hipGetLastError();
}

template <int NW, int NSLOT>
static hipError_t launch_recur_prep_t(const RecurPrepArgs &a, hipStream_t st) {
    constexpr int PW = RecurPrep<NW>::PREP_WAVES;
    constexpr int pair = PairLds<NW, NSLOT>::BYTES;
    constexpr int prep = PW * (int)sizeof(PrepLds);
    constexpr int lds = pair > prep ? pair : prep;
    // more than 80 KiB: never two blocks on one CU (the prep blocks must not share
    // a CU with a recurrence block)
    static_assert(lds <= 160 * 1024 && lds > 80 * 1024, "LDS");
    auto kern = recur_prep_kernel<NW, NSLOT>;
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)kern, lds, lds_set) != hipSuccess) return hipErrorInvalidValue;
    const int64_t rb = (int64_t)a.N * a.H * (D / (16 * NW));
    const int64_t pblocks = a.pe > a.pb ? (seg_chunks_bound(a.M, a.N, a.pb, a.pe) * a.H + PW - 1) / PW : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)(rb + pblocks)), dim3(64 * PairLayout<NW>::WAVES), lds, st, a.recs, a.v,
                       a.cu, a.chunk_off, a.order, a.N, a.T, a.H, a.s0, a.out, a.sfin, a.carry,
                       a.fb, a.fe, (int)rb, a.q, a.k, a.g, a.beta, a.scale, a.recs,
                       a.pb, a.pe);
    return hipGetLastError();
}

hipError_t launch_recur_range(const char *recs, const uint16_t *v, const int32_t *cu,
                              const int32_t *chunk_off, const int32_t *order, int N, int T, int H,
                              const float *s0, float *out, float *sfin, float *carry, int waves,
                              int fb, int fe, hipStream_t st) {
    switch (waves) {
    case 101: return launch_recur_pair<1, pair_nslot<1>()>(recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, carry, fb, fe, st);
    case 102: return launch_recur_pair<2, pair_nslot<2>()>(recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, carry, fb, fe, st);
    case 9: {
        const RecurPrepArgs a{const_cast<char *>(recs), nullptr, nullptr, v, nullptr, nullptr, 0.f, cu, chunk_off,
                              order, N, T, H, s0, out, sfin, carry, fb, fe, 0, 0, 0};
        return launch_recur_hybrid(a, st);
    }
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_recur_prep(const RecurPrepArgs &a, int waves, hipStream_t st) {
    switch (waves) {
    case 9: return launch_recur_hybrid(a, st);
    case 101: return launch_recur_prep_t<1, pair_nslot<1>()>(a, st);
    case 102: return launch_recur_prep_t<2, pair_nslot<2>()>(a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_recur(const char *recs, const uint16_t *v, const int32_t *cu,
                        const int32_t *chunk_off, const int32_t *order, int N, int T, int H,
                        const float *s0, float *out, float *sfin, int waves, hipStream_t st) {
    switch (waves) {
    case 101: case 102: case 9:
        return launch_recur_range(recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, sfin,
                                  waves, 0, SEG_ONE, st);
    case 8: return launch_recur_t<8, 2>(recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, st);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- parts of long sequences
// A sequence's chain of chunk steps is affine in its entry state: S_out = M S_in + B
// (every step is linear in the state plus a term from the chunk's v). With few long
// chains the paired recurrence leaves most CUs idle while each block walks thousands
// of chunks, so every sequence is cut into P parts of about equal chunk count, each a
// virtual sequence (contiguous in tokens and records). Pass 1 runs every part twice in
// one launch, from S_in = 0 with the true v (final state B) and from S_in = I with v = 0
// (final state M, the part's linear map itself, so no subtraction of two runs loses its
// digits); the composition kernel walks the parts of each sequence in order, S_{p+1} = M_p S_p + B_p
// from the sequence's initial state, and writes each part's entry state and the final
// state; pass 2 re-runs every part from its entry state and writes the outputs. The
// chain is then P times shorter for three passes of it, two of them side by side.

// virtual batch: part p of sequence n (at position n of `order`) is virtual sequence n P + p,
// covering its chunks [seg(c, p/P), seg(c, (p+1)/P)); also fills the identity entry states
__global__ __launch_bounds__(256) void parts_setup_kernel(const int32_t *cu_safe, const int32_t *chunk_off,
                                                          const int32_t *order, int N, int P, int cl, int32_t *vcu,
                                                          int32_t *vco, int32_t *vorder, float *ident,
                                                          int64_t nstates) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = tid; v < (int64_t)N * P; v += nth) {
        const int n = (int)(v / P), p = (int)(v % P);
        const int c0 = chunk_off[n], c = chunk_off[n + 1] - c0;
        const int k = seg_chunk(c, (int)(((int64_t)p * SEG_ONE) / P));
        vco[v] = c0 + k;
        vcu[v] = min(cu_safe[n + 1], cu_safe[n] + cl * k);
        vorder[v] = order[n] * P + p;
        if (v == (int64_t)N * P - 1) {
            vco[v + 1] = chunk_off[N];
            vcu[v + 1] = cu_safe[N];
        }
    }
    for (int64_t i = tid; i < nstates * D * D; i += nth) {
        const int rc = (int)(i % (D * D));
        ident[i] = rc / D == rc % D ? 1.f : 0.f;
    }
}

// pass 1: blocks [0, G/2) run every part from a zero state, blocks [G/2, G) from the identity
// with v taken as 0. Both halves also write outputs (not the true ones) to `out`; pass 2, a
// later launch on the same stream, overwrites every one of them.
template <int NW, int NSLOT>
__global__ __launch_bounds__(64 * PairLayout<NW>::WAVES) void recur_parts_kernel(
    const char *__restrict__ recs, const uint16_t *__restrict__ v, const int32_t *__restrict__ vcu,
    const int32_t *__restrict__ vco, const int32_t *__restrict__ vorder, int NV, int T, int H,
    const float *ident, float *out, float *rb, float *ri) {
    extern __shared__ __attribute__((aligned(16))) char ring[];
    const int RB = (int)(gridDim.x / 2);
    const bool id = (int)blockIdx.x >= RB;
    const int b = id ? (int)blockIdx.x - RB : (int)blockIdx.x;
    recur_pair_block<NW, NSLOT>(xcd_remap(b, RB, D / (16 * NW)), ring, recs, v, vcu, vco, vorder, NV, T, H,
                                id ? ident : nullptr, out, id ? ri : rb, id ? ri : rb, 0, SEG_ONE, id);
}

// Composition over the parts of each sequence, one block per (sequence, head, 16 value
// columns): the columns of a state evolve independently under M. Per part p, in order:
// the entry state S is written out, then S <- M_p S + B_p in fp32, on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32: A lane l holds M[row l % 16][k l / 16], B holds
// S[k l / 16][col l % 16], the result rows 4 (l / 16) + j of column l % 16). Each of the
// four waves owns 32 rows. M_p (64 KiB) goes through LDS with rows padded to 132 floats
// (a wave's 16 rows x 4 k of an A operand fall in 64 distinct banks), loaded with whole
// 16-byte accesses; the next part's M is loaded into registers during this part's product.
constexpr int COMBINE_LD = D + 4;
constexpr int COMBINE_LDS = (2 * D * COMBINE_LD + D * 16) * (int)sizeof(float);

// With vcu (the parts' token offsets; NULL: every map applies), a part's map is applied only
// where it is needed: forwards (rev = 0) that of part p while part p + 1 has tokens;
// backwards (rev = 1: the arrays hold part p at index P - 1 - p) that of part p, p >= 1,
// while part p has tokens. The parts with tokens of a sequence come first.
__global__ __launch_bounds__(256) void parts_combine_kernel(const float *s0, const float *rb, const float *ri,
                                                            int N, int P, int H, float *sin, float *sfin, int sbf,
                                                            const int32_t *vcu, int rev) {
    extern __shared__ __attribute__((aligned(16))) float combine_lds[];
    float(*Ms)[D][COMBINE_LD] = (float(*)[D][COMBINE_LD])combine_lds;   // [2][D][D + 4]
    float(*S)[16] = (float(*)[16])(combine_lds + 2 * D * COMBINE_LD);     // [D][16]
    const int cs = blockIdx.x % 8, h = (blockIdx.x / 8) % H, n = blockIdx.x / (8 * H);
    // with vcu, a sequence of one part (or none) has nothing to compose: its part reads the
    // sequence's own entry state and exit gradient
    if (vcu && (P < 2 || vcu[n * P + 1] >= vcu[n * P + 2])) return;
    const int t = threadIdx.x, w = t >> 6, l = t & 63, col0 = cs * 16;
    const int lc = l & 15, lk = l >> 4;    // MFMA: column (or row) l % 16, k slot l / 16
    for (int i = t; i < D * 16; i += 256) {
        const int rr = i / 16, cc = i % 16;
        const int64_t i0 = ((int64_t)n * H + h) * D * D + (int64_t)rr * D + col0 + cc;
        S[rr][cc] = !s0 ? 0.f : sbf ? __uint_as_float((uint32_t)((const uint16_t *)s0)[i0] << 16) : s0[i0];
    }
    auto base_of = [&](int p) { return (((int64_t)n * P + p) * H + h) * D * D; };
    // with vcu: whether step p applies its map, and whether its entry state is read later
    auto has_tokens = [&](int part) { return vcu[n * P + part] < vcu[n * P + part + 1]; };
    auto applies = [&](int p) {
        const int pp = rev ? P - 1 - p : p;   // the part whose map step p applies
        return !vcu || (rev ? pp >= 1 && has_tokens(pp) : pp + 1 < P && has_tokens(pp + 1));
    };
    auto entry_read = [&](int p) {
        const int pp = rev ? P - 1 - p : p;
        return !vcu || pp == 0 || has_tokens(pp);
    };
    float4 mreg[16];   // one part's M: 16 float4 per thread, element 4 (t + 256 j)
    f32x4 breg[2];     // and its B at this lane's result positions
    auto load_m = [&](int p) {
        if (!applies(p)) return;
        const float4 *src = (const float4 *)(ri + base_of(p));
#pragma unroll
        for (int j = 0; j < 16; ++j) mreg[j] = src[t + 256 * j];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                breg[rt][j] = rb[base_of(p) + (int64_t)(32 * w + 16 * rt + 4 * lk + j) * D + col0 + lc];
    };
    auto store_m = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = 4 * (t + 256 * j), row = e / D, col = e % D;
            *(float4 *)&Ms[buf][row][col] = mreg[j];
        }
    };
    if (P > 0) {
        load_m(0);
        store_m(0);
    }
    __syncthreads();
    for (int p = 0; p < P; ++p) {
        const int64_t base = base_of(p);
        const bool apply = applies(p);
        f32x4 acc[2] = {breg[0], breg[1]};
        if (p + 1 < P) load_m(p + 1);
        const float(*M)[COMBINE_LD] = Ms[p & 1];
        if (apply) {
#pragma unroll 8
            for (int kk = 0; kk < D / 4; ++kk) {
                const float b = S[4 * kk + lk][lc];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    acc[rt] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(M[32 * w + 16 * rt + lc][4 * kk + lk], b, acc[rt], 0, 0, 0);
            }
        }
        // the entry state of part p, then (after every wave's reads of S) the new state
        if (entry_read(p)) {
            for (int i = t; i < D * 16 / 4; i += 256) {
                const int rr = i / 4, c4 = (i % 4) * 4;
                *(float4 *)(sin + base + (int64_t)rr * D + col0 + c4) = *(const float4 *)&S[rr][c4];
            }
        }
        __syncthreads();   // every read of S and of this part's M is done
        if (apply) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) S[32 * w + 16 * rt + 4 * lk + j][lc] = acc[rt][j];
        }
        if (p + 1 < P) store_m((p + 1) & 1);
        __syncthreads();
    }
    if (sfin) {
        for (int i = t; i < D * 16; i += 256) {
            const int rr = i / 16, cc = i % 16;
            const int64_t i0 = ((int64_t)n * H + h) * D * D + (int64_t)rr * D + col0 + cc;
            if (sbf) ((uint16_t *)sfin)[i0] = (uint16_t)(pack2(S[rr][cc], 0.f) & 0xffffu);   // round to nearest even
            else sfin[i0] = S[rr][cc];
        }
    }
}

// the composition of the parts' affine maps, for other users of the same scheme (the backward)
hipError_t launch_parts_compose(const float *s0, const float *rb, const float *ri, int N, int P, int H, float *sin,
                                float *sfin, const int32_t *vcu, bool rev, hipStream_t st) {
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)parts_combine_kernel, COMBINE_LDS, lds_set) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(parts_combine_kernel, dim3((unsigned)(N * H * 8)), dim3(256), COMBINE_LDS, st, s0, rb, ri, N, P,
                       H, sin, sfin, 0, vcu, (int)rev);
    return hipGetLastError();
}

// setup, pass 1 (two-slice paired blocks: 8 N P H of them), composition, pass 2 (one-slice
// paired blocks, no state written: the composition wrote the final state)
hipError_t launch_parts(const char *recs, const uint16_t *v, const int32_t *cu_safe, const int32_t *chunk_off,
                        const int32_t *order, int N, int T, int H, int P, const float *s0, float *out,
                        float *sfin, int32_t *vcu, int32_t *vco, int32_t *vorder, float *ident, float *rb,
                        float *ri, float *sin, bool h32, bool sbf, int pass2_waves, hipStream_t st) {
    const int NV = N * P;
    const int64_t ns = (int64_t)NV * H;
    hipLaunchKernelGGL(parts_setup_kernel, dim3(512), dim3(256), 0, st, cu_safe, chunk_off, order, N, P,
                       h32 ? 32 : C, vcu, vco, vorder, ident, ns);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    if (h32) {
        if (launch_h32_parts_pass1(recs, v, vcu, vco, vorder, NV, T, H, ident, out, rb, ri, st) != hipSuccess)
            return hipErrorLaunchFailure;
    } else {
        constexpr int NW = 2, NS = pair_nslot<2>();
        constexpr int lds = PairLds<NW, NS>::BYTES;
        auto kern = recur_parts_kernel<NW, NS>;
        static std::atomic<uint64_t> lds_set{0};
        if (ensure_lds_limit((const void *)kern, lds, lds_set) != hipSuccess) return hipErrorInvalidValue;
        const int64_t rbk = (int64_t)NV * H * (D / (16 * NW));
        hipLaunchKernelGGL(kern, dim3((unsigned)(2 * rbk)), dim3(64 * PairLayout<NW>::WAVES), lds, st, recs, v, vcu,
                           vco, vorder, NV, T, H, (const float *)ident, out, rb, ri);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    static std::atomic<uint64_t> combine_lds_set{0};
    if (ensure_lds_limit((const void *)parts_combine_kernel, COMBINE_LDS, combine_lds_set) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(parts_combine_kernel, dim3((unsigned)(N * H * 8)), dim3(256), COMBINE_LDS, st, s0,
                       (const float *)rb, (const float *)ri, N, P, H, sin, sfin, (int)sbf, (const int32_t *)nullptr, 0);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    if (h32) return launch_recur_h32_range(recs, v, vcu, vco, vorder, NV, T, H, sin, out, nullptr, nullptr,
                                           pass2_waves, 0, SEG_ONE, false, st);
    return launch_recur_range(recs, v, vcu, vco, vorder, NV, T, H, sin, out, nullptr, nullptr, 101, 0, SEG_ONE, st);
}

}  // namespace kda
