// kda_launch.hpp -- host-side launchers of the gfx950 KDA kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace kda {

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once per device
// (one process may drive several GPUs; concurrent callers may both set it, which is
// harmless). `done` is the calling launcher's own bit set of devices (64 at most; a
// device beyond that has the attribute set at every call).
inline hipError_t ensure_lds_limit(const void *kern, int bytes, std::atomic<uint64_t> &done) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

constexpr int REC_BYTES = 23552;   // bytes of one 16-token chunk record (Rec::BYTES)
constexpr int REC32_BYTES = 50176; // bytes of one 32-token chunk record (Rec32::BYTES)

// Segments of the split path. A launch over the segment [fb, fe) covers, of every
// sequence with c chunks, its local chunks [seg_chunk(c, fb), seg_chunk(c, fe)): fb <= fe
// are fractions of a sequence in units of 1/SEG_ONE, and [0, SEG_ONE) is all of it. So
// every sequence advances in every launch, however the lengths in a batch are spread.
constexpr int SEG_ONE = 1 << 16;
__host__ __device__ inline int seg_chunk(int c, int f) { return (int)(((int64_t)c * f) >> 16); }
// Upper bound on the chunks of all sequences inside [fb, fe) when they have at most M in all.
inline int64_t seg_chunks_bound(int64_t M, int N, int fb, int fe) {
    if (fb == 0 && fe == SEG_ONE) return M;
    const int64_t b = (M * (int64_t)(fe - fb) + SEG_ONE - 1) / SEG_ONE + N;
    return b < M ? b : M;
}

// sanitised sequence offsets cu_safe[N+1] (ordered, inside [0, T]; the error word gets
// 2 when cu was malformed, else 0), chunk offsets of cl-token chunks (cl = 16 or 32),
// longest-first order. Later kernels take cu_safe as their cu.
hipError_t launch_chunk_map(const int32_t *cu, int N, int T, int32_t *cu_safe, int32_t *chunk_off,
                            int32_t *order, int32_t *err, int cl, hipStream_t st);

// Records (16-token chunks; 32-token with prep32) of the segment [fb, fe); M bounds the
// batch's chunk count.
hipError_t launch_prep32(const uint16_t *q, const uint16_t *k, const float *g, const float *beta,
                         const int32_t *cu, int N, int T, int H, float scale,
                         const int32_t *chunk_off, char *recs, int fb, int fe, int64_t M,
                         hipStream_t st);

hipError_t launch_prep(const uint16_t *q, const uint16_t *k, const float *g, const float *beta,
                       const int32_t *cu, int N, int T, int H, float scale,
                       const int32_t *chunk_off, char *recs, int fb, int fe, int64_t M,
                       hipStream_t st);

// paired recurrence over the segment [fb, fe); waves in {101, 102, 201, 202}
hipError_t launch_recur_range(const char *recs, const uint16_t *v, const int32_t *cu,
                              const int32_t *chunk_off, const int32_t *order, int N, int T, int H,
                              const float *s0, float *out, float *sfin, float *carry, int waves,
                              int fb, int fe, hipStream_t st);

// One launch: paired recurrence over the segment [fb, fe) plus the records of the
// segment [pb, pe) (the next one), prepared on the CUs the recurrence leaves idle.
struct RecurPrepArgs {
    char *recs;
    const uint16_t *q, *k, *v;
    const float *g, *beta;
    float scale;
    const int32_t *cu, *chunk_off, *order;
    int N, T, H;
    const float *s0;
    float *out, *sfin, *carry;
    int fb, fe, pb, pe;
    int64_t M;          // bound on the batch's chunk count
};
hipError_t launch_recur_prep(const RecurPrepArgs &a, int waves, hipStream_t st);
// 32-token forms (waves 301: one slice per block, 302: two): recurrence over the segment
// [fb, fe), alone or with the prep of [pb, pe) on the idle CUs
hipError_t launch_recur32_range(const char *recs, const uint16_t *v, const int32_t *cu,
                                const int32_t *chunk_off, const int32_t *order, int N, int T,
                                int H, const float *s0, float *out, float *sfin, float *carry,
                                int waves, int fb, int fe, hipStream_t st);
hipError_t launch_recur32_prep(const RecurPrepArgs &a, int waves, hipStream_t st);

hipError_t launch_recur(const char *recs, const uint16_t *v, const int32_t *cu,
                        const int32_t *chunk_off, const int32_t *order, int N, int T, int H,
                        const float *s0, float *out, float *sfin, int waves, hipStream_t st);

// Token-by-token recurrence: one block per (sequence, head, tile of dvt value columns),
// dvt in {128, 64, 32}. one_token_per_seq: sequence n is token n (decode step, cu unused).
// States s0 / sfin are fp32, or bf16 with bf16_state (one token per sequence only).
hipError_t launch_recurrent(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                            const float *beta, float scale, const int32_t *cu, int N, int T, int H,
                            bool one_token_per_seq, const void *s0, float *out, void *sfin, bool bf16_state,
                            int dvt, hipStream_t st);
// value-column tile of launch_recurrent for this many (sequence, head) chains over a
// batch of `tokens` tokens in `seqs` sequences, with an fp32 or a bf16 state
int recurrent_tile(int64_t chains, int64_t tokens, int64_t seqs, bool bf16_state);

hipError_t launch_fused(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                        const float *beta, const int32_t *cu, const int32_t *order, int N, int T,
                        int H, float scale, const float *s0, float *out, float *sfin, int *err,
                        int waves, hipStream_t st);

// The recurrence over P parts of every sequence (few long chains); the buffers hold N P H
// states each (ident, rb, ri, sin) and N P + 1 (vcu, vco) or N P (vorder) entries.
hipError_t launch_parts(const char *recs, const uint16_t *v, const int32_t *cu_safe, const int32_t *chunk_off,
                        const int32_t *order, int N, int T, int H, int P, const float *s0, float *out,
                        float *sfin, int32_t *vcu, int32_t *vco, int32_t *vorder, float *ident, float *rb,
                        float *ri, float *sin, hipStream_t st);
}  // namespace kda
