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

// Device error word of the current device: one int32 in device memory that kernels OR
// their error bits into (KDA_DEVERR_* of kda.h) and that only kda_device_errors clears.
// Resolved once per device; nullptr if the runtime cannot resolve it (kernels then skip it).
int32_t *device_error_word();

constexpr int REC_BYTES = 23552;   // bytes of one 16-token chunk record (Rec::BYTES)
constexpr int RECH_BYTES = 37888;  // bytes of one 32-token chunk record of forms 401/402 (RecH::BYTES)

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

// Records (16-token chunks) of the segment [fb, fe); M bounds the batch's chunk count.

hipError_t launch_prep(const uint16_t *q, const uint16_t *k, const float *g, const float *beta,
                       const int32_t *cu, int N, int T, int H, float scale,
                       const int32_t *chunk_off, char *recs, int fb, int fe, int64_t M,
                       hipStream_t st);

// paired recurrence over the segment [fb, fe); waves in {101, 102, 9}
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
    bool g_bf16 = false;      // g holds bf16 bits (forms 401/402 only)
    bool state_bf16 = false;  // s0 and sfin hold bf16 bits (forms 401/402 only)
};
hipError_t launch_recur_prep(const RecurPrepArgs &a, int waves, hipStream_t st);

// 32-token chunks with fp16 recurrence operands (kda_h32.hip): records of the segment
// [fb, fe); recurrence forms 401 (one 16-column slice per block) and 402 (two), alone or
// with the prep of [pb, pe); pass 1 of the recurrence over parts.
// g_bf16: g holds bf16 bits; sbf: s0 and sfin hold bf16 bits (the carry stays fp32).
hipError_t launch_prep_h32(const uint16_t *q, const uint16_t *k, const void *g, bool g_bf16, const float *beta,
                           const int32_t *cu, int N, int T, int H, float scale, const int32_t *chunk_off,
                           char *recs, int fb, int fe, int64_t M, hipStream_t st);
// The same for the first segment [0, fe) with the chunk map formed in the launch (no
// chunk-map launch before it): cu is the caller's offsets, and the launch stores cu_safe,
// chunk_off, order and the error word as launch_chunk_map does (32-token chunks). Only for
// prep_h32_maps(N), batches of at most 63 sequences.
bool prep_h32_maps(int N);
hipError_t launch_prep_h32_map(const uint16_t *q, const uint16_t *k, const void *g, bool g_bf16, const float *beta,
                               const int32_t *cu, int N, int T, int H, float scale, char *recs, int fe, int64_t M,
                               int32_t *cu_safe, int32_t *chunk_off, int32_t *order, int32_t *err, hipStream_t st);
hipError_t launch_recur_h32_range(const char *recs, const uint16_t *v, const int32_t *cu, const int32_t *chunk_off,
                                  const int32_t *order, int N, int T, int H, const float *s0, float *out, float *sfin,
                                  float *carry, int waves, int fb, int fe, bool sbf, hipStream_t st);
hipError_t launch_recur_h32_prep(const RecurPrepArgs &a, int waves, hipStream_t st);
hipError_t launch_h32_parts_pass1(const char *recs, const uint16_t *v, const int32_t *vcu, const int32_t *vco,
                                  const int32_t *vorder, int NV, int T, int H, const float *ident, float *out,
                                  float *rb, float *ri, hipStream_t st);

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
// The token loop over a packed batch (the recurrent variant of the forward), with g and the
// initial/final states as fp32 or bf16 (g_bf16, s_bf16: bf16 bits).
hipError_t launch_recurrent_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const void *g, bool g_bf16,
                                const float *beta, float scale, const int32_t *cu, int N, int T, int H,
                                const void *s0, float *out, void *sfin, bool s_bf16, int dvt, hipStream_t st);
// value-column tile of launch_recurrent for this many (sequence, head) chains over a
// batch of `tokens` tokens in `seqs` sequences, with an fp32 or a bf16 state
int recurrent_tile(int64_t chains, int64_t tokens, int64_t seqs, bool bf16_state);

// The composition over parts of affine maps S <- M S + B (ri, rb: [N P][H][128][128] fp32):
// sin receives each part's entry state, sfin (or NULL) the last exit state, s0 (or NULL:
// zeros) entering part 0. With vcu (the parts' token offsets) only the maps that are needed
// apply (see parts_combine_kernel); rev: the arrays hold the parts in reverse order.
hipError_t launch_parts_compose(const float *s0, const float *rb, const float *ri, int N, int P, int H, float *sin,
                                float *sfin, const int32_t *vcu, bool rev, hipStream_t st);

// Workspace of the backward over up to P parts per sequence (P > 1): the parts as virtual
// sequences (vcu, vco: N P + 1 offsets each), and four [N P][H][128][128] fp32 arrays (rb and
// ri hold the forward maps, then the gradient maps; sinf and sinb the entry states and the
// exit gradients of the parts). A sequence of c blocks of tokens takes ceil(c / lstar)
// parts (at most P), the slots after them being empty.
struct BwdParts {
    int P, lstar;
    int32_t *vcu, *vco;
    float *rb, *ri, *sinf, *sinb;
};

// The backward (kda_bwd.hip) with `waves` (8 or 4) waves per workgroup, 128 / (8 waves)
// workgroups per (sequence, head). With 8: zeroes dq, dk, dg, dbeta, which the two
// workgroups of a chain add into; with 4: the workgroups write partial sums to psum
// (bwd_partial_floats(T, H, waves) floats) and a last kernel adds them in a fixed order.
// chunk_off counts blocks of bwd_block_tokens() tokens per sequence (the chunk map at that
// chunk length); ck holds a state per block and head. With parts (parts.P > 1) each
// sequence is cut into P parts of whole blocks, run as sequences of their own.
hipError_t launch_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                      float scale, const int32_t *cu_safe, const int32_t *chunk_off, int N,
                      int T, int H, const float *s0, const float *dout, const float *dsf, float *dq, float *dk,
                      float *dv, float *dg, float *dbeta, float *ds0, float *ck, float *psum, int waves,
                      const BwdParts &parts, hipStream_t st);
inline int64_t bwd_partial_floats(int64_t T, int64_t H, int waves) {
    return waves == 8 ? 0 : (int64_t)(16 / waves) * T * H * (3 * 128 + 1);
}
int bwd_block_tokens();

hipError_t launch_fused(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                        const float *beta, const int32_t *cu, const int32_t *order, int N, int T,
                        int H, float scale, const float *s0, float *out, float *sfin, int *err,
                        int waves, hipStream_t st);

// The recurrence over P parts of every sequence (few long chains); the buffers hold N P H
// states each (ident, rb, ri, sin) and N P + 1 (vcu, vco) or N P (vorder) entries. h32:
// over 32-token fp16 records (forms 401/402), else 16-token records.
hipError_t launch_parts(const char *recs, const uint16_t *v, const int32_t *cu_safe, const int32_t *chunk_off,
                        const int32_t *order, int N, int T, int H, int P, const float *s0, float *out,
                        float *sfin, int32_t *vcu, int32_t *vco, int32_t *vorder, float *ident, float *rb,
                        float *ri, float *sin, bool h32, bool sbf, int pass2_waves, hipStream_t st);
}  // namespace kda
