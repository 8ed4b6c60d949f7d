// kda_api.cpp -- the C ABI declared in include/kda.h: argument validation,
// variant choice, workspace, launches. No exception crosses the interface.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kda.h"
#include "kda_launch.hpp"

namespace {

constexpr size_t ALIGN = 256;
constexpr int KDA_MAX_SEGMENTS = 8;
static_assert(KDA_SEGMENT_ONE == kda::SEG_ONE, "segment fraction unit");

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// chunks of cl tokens: an upper bound over any split of T tokens into N sequences
int64_t max_chunks(int64_t N, int64_t T, int cl = KDA_CHUNK) { return (T + cl - 1) / cl + N; }

// The recurrence forms 301/302 consume 32-token chunk records; all others 16-token ones.
int chunk_len(int waves) { return waves >= 300 ? 32 : KDA_CHUNK; }
size_t rec_bytes(int waves) { return waves >= 300 ? kda::REC32_BYTES : kda::REC_BYTES; }

// Workspace: chunk offsets [N+1], sequence order [N], an error word, the sanitised
// sequence offsets [N+1], and (split variant only) a state carry buffer [N, H, 128, 128]
// fp32 when the chunk range is cut into segments, followed by one chunk record per
// (chunk, head).
struct Layout {
    size_t chunk_off, order, err, cu, carry, recs, parts, total;
};

constexpr int MAX_PARTS = 16;
constexpr size_t STATE_BYTES = (size_t)KDA_HEAD_DIM * KDA_HEAD_DIM * sizeof(float);

// Parts per sequence of the split variant's recurrence (1: whole sequences; see
// launch_parts). Pass 1 runs 8 N P H two-slice paired blocks and pass 2 8 N P H one-slice
// blocks, so P <= 32 / (N H) keeps each pass within one round of the 256 CUs; three
// passes over a P times shorter chain pay from P = 3, down to parts of 64 chunks. Measured
// on MI355X (ms, whole | in P parts; best of 4 alternating rounds), one sequence of T
// tokens x H heads: 65536 x 8 2.16 | 1.74 (3), 1.41 (4); 32768 x 8 1.09 | 0.76 (4); 16384 x
// 8 0.551 | 0.481 (3), 0.412 (4); 12288 x 8 0.419 | 0.365 (3); 8192 x 8 0.275 | 0.253 (3),
// 0.223 (4); 65536 x 4 2.08 | 1.26 (4), 0.79 (8); 8192 x 4 0.269 | 0.201 (4), 0.177 (8);
// 4096 x 2 0.142 | 0.126 (4), 0.122 (8); two sequences of 16384 x 4 0.554 | 0.418 (4);
// but 32768 x 16 1.21 | 1.41 (2). KDA_PARTS (1..MAX_PARTS) overrides, for the 16-token
// forms.
int split_parts(int64_t N, int64_t T, int64_t H, int waves) {
    if (waves >= 300) return 1;
    if (const char *e = std::getenv("KDA_PARTS")) {
        const int p = std::atoi(e);
        if (p >= 1 && p <= MAX_PARTS) return p;
    }
    if (waves != 101) return 1;
    int64_t p = 32 / (N * H);
    const int64_t by_len = max_chunks(N, T) / 64;
    if (by_len < p) p = by_len;
    if (p > MAX_PARTS) p = MAX_PARTS;
    return p >= 3 ? (int)p : 1;
}

Layout ws_layout(int64_t N, int64_t T, int64_t H, int variant, int segments, int waves, int parts = 1) {
    Layout L{};
    if (variant == KDA_VARIANT_RECURRENT) return L;  // reads cu_seqlens directly, no workspace
    L.chunk_off = 0;
    L.order = align_up(sizeof(int32_t) * (size_t)(N + 1));
    L.err = L.order + align_up(sizeof(int32_t) * (size_t)N);
    L.cu = L.err + ALIGN;
    L.carry = L.cu + align_up(sizeof(int32_t) * (size_t)(N + 1));
    L.recs = L.carry;
    L.total = L.recs;
    if (variant == KDA_VARIANT_SPLIT) {
        if (segments > 1)
            L.recs = L.carry + (size_t)N * H * KDA_HEAD_DIM * KDA_HEAD_DIM * sizeof(float);
        L.parts = L.recs + align_up((size_t)max_chunks(N, T, chunk_len(waves)) * (size_t)H * rec_bytes(waves));
        L.total = L.parts;
        if (parts > 1)   // identity, zero-run, identity-run and entry states; virtual cu, chunk offsets, order
            L.total += 4 * (size_t)N * parts * H * STATE_BYTES + 3 * align_up(sizeof(int32_t) * (size_t)(N * parts + 1));
    }
    return L;
}

// Shape limits: grid sizes stay far below 2^31 blocks and token-head offsets fit int64.
bool shape_ok(int64_t N, int64_t T, int64_t H) {
    if (N < 1 || T < 0 || H < 1) return false;
    if (max_chunks(N, T) * H > (int64_t)1 << 30) return false;
    if (N * H * 8 > (int64_t)1 << 30) return false;
    return true;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + nb && pb < pa + na;
}


// Recurrence block shape. 9: per chain, paired or eight-wave (below). 1, 2, 4 or 8:
// waves per block, each owning 16 value columns
// and forming its own outputs; the block's waves share each chunk record through one
// LDS ring (3 chunks deep for 4 waves, 2 for 8; 42 and 83 are the other depths). 0:
// the key-split form, four waves per 16-column slice. 101, 102: the paired form (1 or
// 2 slices per block, a chain wave and two output waves per slice, one loader wave).
// KDA_RECUR_WAVES overrides the choice, for tuning.
int recur_waves(int64_t N, int64_t H, const char *env = "KDA_RECUR_WAVES") {
    if (const char *e = std::getenv(env)) {
        const int w = std::atoi(e);
        if (w == 0 || w == 1 || w == 2 || w == 4 || w == 42 || w == 8 || w == 83 || w == 9 || w == 101 ||
            w == 102 || w == 201 || w == 202 || w == 301 || w == 302)
            return w;
    }
    // Measured on MI355X (ms, best segment count each; one slice per block 101 | two
    // slices 102), one sequence of 8192 tokens: 20 heads 0.326 | 0.370; 24 heads 0.356 |
    // 0.384; 28 heads 0.391 | 0.401; 32 heads 0.408 | 0.417; 40 heads 0.673 | 0.460 (101
    // needs two rounds of blocks from 33 chains). Then (ms; paired 102 | eight-wave 8):
    // 128 chains (8 x 1024 tokens, 16 heads) 0.181 | 0.205; 192 chains 0.476 | 0.478; 512
    // chains of 2048 tokens 1.23 | 1.00; 8192 chains of 64 tokens 1.18 | 0.72; but 384
    // chains of skewed lengths (12 sequences, 32768 tokens, 32 heads) 1.29 | 2.43, where
    // the longest chain sets the end time. From 192 chains the hybrid (9) picks per chain
    // on the device: paired for chains longer than a CU's balanced share, eight-wave
    // otherwise.
    const int64_t chains = N * H;
    if (chains <= 32) return 101;
    if (chains < 192) return 102;
    return 9;
}

// Number of segments of the split variant. With S > 1 the launches are
// prep(segment 0), then recurrence(s) fused with prep(s+1) for s < S-1, then
// recurrence(S-1): the prep of later segments runs on the CUs the recurrence leaves
// idle, which pays when the recurrence has fewer blocks than the chip has CUs. 1 for
// the other recurrence forms. KDA_SEGMENTS (1..KDA_MAX_SEGMENTS) overrides (the hybrid
// form included).
int split_segments(int64_t N, int64_t T, int64_t H, int waves) {
    if (waves < 100 && waves != 9) return 1;
    if (const char *e = std::getenv("KDA_SEGMENTS")) {
        const int s = std::atoi(e);
        if (s >= 1 && s <= KDA_MAX_SEGMENTS) return s;
    }
    // The hybrid runs whole: its prep of a next segment waits for every recurrence block
    // to be dispatched, and the chains below the longest keep the CUs busy for most of a
    // segment. Measured on MI355X (ms for 1 | 2 | 3 segments, best of 4 alternating
    // rounds): 12 skewed sequences of 32768 tokens x 32 heads 1.172 | 1.222 | 1.257; 6
    // skewed sequences of 22528 tokens x 32 heads 0.950 | 0.910 | 0.907; 8 x 4096 x 32
    // 1.023 | 1.052 | 1.075; 16 x 2048 x 32 1.032 | 1.084 | 1.124; 16 x 1024 x 16 0.263 |
    // 0.299 | 0.322. KDA_SEGMENTS selects segments for it (parity-tested).
    if (waves == 9) return 1;
    // The prep of a segment (work ~ the chain count) runs on the CUs the recurrence
    // leaves idle and must fit under its time: segments only with at least 2.5 idle CUs
    // per chain. Measured on MI355X (ms, 8192 tokens; unsegmented | segmented): 101 with
    // 20 heads (96 idle CUs) 0.359 | 0.326, 24 heads (64) 0.371 | 0.356, 28 heads (32)
    // 0.391 | 0.401; 102 with 32 heads (128) 0.447 | 0.417, 40 heads (96) 0.476 | 0.460,
    // 48 heads (64) 0.511 | 0.527, 56 heads (32) 0.548 | 0.602.
    const int64_t chains = N * H;
    const int64_t blocks = chains * (8 / (waves % 100));
    if (2 * (256 - blocks) < 5 * chains) return 1;
    // S segments hide (1 - 1/S) of the prep (~7 ns per chunk-head on the whole chip)
    // and add S - 1 launches (~5 us each): S = sqrt(prep / 5 us), i.e. sqrt(chunk-heads
    // / 500), at most 6. Measured on MI355X (ms for 1 | 2 | 3 | 6 segments): 256 tokens x
    // 2 heads 0.024 | 0.028 | 0.032 | 0.051; 4096 x 8 0.160 | 0.159 | 0.160 | 0.170;
    // 4096 x 32 0.229 | 0.218 | 0.216 | 0.228; 8192 x 32: 3 0.442, 4 0.439, 6 0.435,
    // 8 0.441; 65536 x 8: 4 2.308, 6 2.305, 8 2.321.
    const double chunk_heads = (double)max_chunks(N, T) * (double)H;
    const int s = (int)std::lround(std::sqrt(chunk_heads / 500.0));
    return s < 1 ? 1 : s > 6 ? 6 : s;
}

// Start of segment sg of S, as a fraction of every sequence's chunks in units of
// 1/SEG_ONE (segment_frac(S, S) = SEG_ONE). Segment sizes grow geometrically by a ratio
// r: the first segment's prep runs alone, so a small first segment shortens it, while
// each later prep (work per chunk ~ the chain count) must still fit under the previous
// segment's recurrence (time per chunk independent of the chain count).
// r = min(2, 1 + 8 / chains); measured on MI355X (ms for r = 1, 1.3, 1.6, 2): 8192 tokens x
// 32 heads 0.433, 0.428, 0.435, 0.454; 65536 x 8 2.307, 2.293, 2.280, 2.277.
// KDA_SEGMENT_RATIO overrides r, for tuning.
double segment_ratio(int64_t chains) {
    if (const char *e = std::getenv("KDA_SEGMENT_RATIO")) {
        const double r = std::atof(e);
        if (r >= 1.0 && r <= 4.0) return r;
    }
    const double r = 1.0 + 8.0 / (double)(chains > 0 ? chains : 1);
    return r > 2.0 ? 2.0 : r;
}
int segment_frac(int sg, int S, int64_t chains) {
    if (sg <= 0) return 0;
    if (sg >= S) return kda::SEG_ONE;
    const double r = segment_ratio(chains);
    const double f = r == 1.0 ? (double)sg / S : (std::pow(r, sg) - 1.0) / (std::pow(r, S) - 1.0);
    return (int)std::lround(f * kda::SEG_ONE);
}

// Consumer waves per block of the fused kernel (1, 2 or 4; 16 value columns each).
// KDA_FUSED_WAVES overrides the choice, for tuning.
int fused_waves(int64_t N, int64_t H) {
    if (const char *e = std::getenv("KDA_FUSED_WAVES")) {
        const int w = std::atoi(e);
        if (w == 1 || w == 2 || w == 4) return w;
    }
    // measured on MI355X: 2 chains (config 1) 1 or 2 slices per block tie; 128 chains
    // (config 3): 4 slices 0.22 ms, 2 slices 0.34 ms, 1 slice 0.66 ms
    const int64_t chains = N * H;
    if (chains <= 16) return 1;
    if (chains <= 64) return 2;
    return 4;
}

}  // namespace

extern "C" {

const char *kda_version(void) { return "kda-mi355x 0.1.0 (gfx950)"; }

const char *kda_status_string(int s) {
    switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is out of range";
    case KDA_ERR_UNSUPPORTED: return "unsupported argument (head_dim must be 128; scale finite; known variant)";
    case KDA_ERR_ALLOC: return "workspace allocation failed or caller workspace too small";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
    case KDA_ERR_DEVICE: return "HIP device error";
    case KDA_ERR_ALIAS: return "final_state partially overlaps initial_state";
    default: return "unknown status";
    }
}

int kda_select_variant(int32_t num_seqs, int32_t total_tokens, int32_t num_heads) {
    (void)num_heads;
    if (const char *e = std::getenv("KDA_VARIANT")) {
        if (!std::strcmp(e, "split")) return KDA_VARIANT_SPLIT;
        if (!std::strcmp(e, "fused")) return KDA_VARIANT_FUSED;
        if (!std::strcmp(e, "recurrent")) return KDA_VARIANT_RECURRENT;
    }
    // The token loop costs ~0.9 us per token of the longest sequence (plus ~11 us); the
    // split variant at least ~17 us (measured on MI355X, 32 heads, ms split | token
    // loop: 1 sequence of 8 tokens 0.017 | 0.012, of 16 tokens 0.017 | 0.021; 256
    // sequences of 1 token 0.313 | 0.102, of 8 tokens 0.328 | 0.192, of 16 tokens 0.341
    // | 0.333). The host cannot see the lengths, only T and N; with T <= max(8, 2N) even
    // the most skewed split of the T tokens (one sequence of T - N + 1) keeps the token
    // loop ahead of the split variant.
    if ((int64_t)total_tokens <= 8 || (int64_t)total_tokens <= 2 * (int64_t)num_seqs)
        return KDA_VARIANT_RECURRENT;
    return KDA_VARIANT_SPLIT;
}

int32_t kda_launch_plan(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                        int32_t variant, kda_launch_info *info, int32_t max_launches) {
    if (!shape_ok(num_seqs, total_tokens, num_heads)) return 0;
    const int v = variant == KDA_VARIANT_AUTO
                      ? kda_select_variant(num_seqs, total_tokens, num_heads)
                      : variant;
    const int waves = v == KDA_VARIANT_SPLIT ? recur_waves(num_seqs, num_heads) : 0;
    const int cl = v == KDA_VARIANT_SPLIT ? chunk_len(waves) : KDA_CHUNK;
    kda_launch_info plan[2 + KDA_MAX_SEGMENTS];
    int n = 0;
    if (v == KDA_VARIANT_RECURRENT) {
        plan[n++] = {KDA_KERNEL_RECURRENT, 0, 0, 0, 0, 1};
        for (int i = 0; info && i < n && i < max_launches; ++i) info[i] = plan[i];
        return n;
    }
    plan[n++] = {KDA_KERNEL_CHUNK_MAP, 0, 0, 0, 0, cl};
    if (v == KDA_VARIANT_SPLIT) {
        const int segs = split_segments(num_seqs, total_tokens, num_heads, waves);
        auto bound = [&](int sg) { return (int32_t)segment_frac(sg, segs, (int64_t)num_seqs * num_heads); };
        if (split_parts(num_seqs, total_tokens, num_heads, waves) > 1) {
            plan[n++] = {KDA_KERNEL_PREP, 0, KDA_SEGMENT_ONE, 0, 0, cl};
            plan[n++] = {KDA_KERNEL_PARTS, 0, 0, 0, KDA_SEGMENT_ONE, cl};
            for (int i = 0; info && i < n && i < max_launches; ++i) info[i] = plan[i];
            return n;
        }
        plan[n++] = {KDA_KERNEL_PREP, 0, bound(1), 0, 0, cl};
        for (int sg = 0; sg + 1 < segs; ++sg)
            plan[n++] = {KDA_KERNEL_RECUR_PREP, bound(sg + 1), bound(sg + 2), bound(sg), bound(sg + 1), cl};
        plan[n++] = {KDA_KERNEL_RECUR, 0, 0, bound(segs - 1), KDA_SEGMENT_ONE, cl};
    } else {
        plan[n++] = {KDA_KERNEL_FUSED, 0, KDA_SEGMENT_ONE, 0, KDA_SEGMENT_ONE, cl};
    }
    for (int i = 0; info && i < n && i < max_launches; ++i) info[i] = plan[i];
    return n;
}

size_t kda_workspace_bytes(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                           int32_t variant) {
    if (!shape_ok(num_seqs, total_tokens, num_heads)) return 0;
    const int v = variant == KDA_VARIANT_AUTO
                      ? kda_select_variant(num_seqs, total_tokens, num_heads)
                      : variant;
    const int waves = v == KDA_VARIANT_SPLIT ? recur_waves(num_seqs, num_heads) : 0;
    const int segs = v == KDA_VARIANT_SPLIT ? split_segments(num_seqs, total_tokens, num_heads, waves) : 1;
    const int parts = v == KDA_VARIANT_SPLIT ? split_parts(num_seqs, total_tokens, num_heads, waves) : 1;
    return ws_layout(num_seqs, total_tokens, num_heads, v, segs, waves, parts).total;
}

int kda_fwd_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
               float scale, const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens,
               int32_t num_heads, int32_t head_dim, const float *initial_state, float *out,
               float *final_state, void *stream, const kda_options *opt) {
    // ---- host-side validation, before anything is enqueued
    const int n_ev = opt ? opt->n_stage_events : 0;
    if (n_ev != 0 && (n_ev < 2 || n_ev > KDA_MAX_STAGE_EVENTS || !opt->stage_events))
        return KDA_ERR_UNSUPPORTED;
    if (opt && opt->reserved != 0) return KDA_ERR_UNSUPPORTED;
    const int variant = opt ? opt->variant : KDA_VARIANT_AUTO;
    if (variant != KDA_VARIANT_AUTO && variant != KDA_VARIANT_SPLIT && variant != KDA_VARIANT_FUSED &&
        variant != KDA_VARIANT_RECURRENT)
        return KDA_ERR_UNSUPPORTED;
    if (head_dim != KDA_HEAD_DIM) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return KDA_ERR_UNSUPPORTED;
    if (!shape_ok(num_seqs, total_tokens, num_heads)) return KDA_ERR_SHAPE;
    if (!cu_seqlens && num_seqs != 1) return KDA_ERR_SHAPE;
    if (!out && total_tokens > 0) return KDA_ERR_NULL;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta)) return KDA_ERR_NULL;
    const size_t state_bytes = (size_t)num_seqs * num_heads * KDA_HEAD_DIM * KDA_HEAD_DIM * 4;
    if (initial_state && final_state && (const void *)initial_state != (const void *)final_state &&
        overlaps(initial_state, state_bytes, final_state, state_bytes))
        return KDA_ERR_ALIAS;

    const int chosen = variant == KDA_VARIANT_AUTO
                           ? kda_select_variant(num_seqs, total_tokens, num_heads)
                           : variant;
    hipStream_t st = (hipStream_t)stream;
    const int N = num_seqs, T = total_tokens, H = num_heads;
    const int waves = chosen == KDA_VARIANT_SPLIT ? recur_waves(N, H) : fused_waves(N, H);
    const int segs = chosen == KDA_VARIANT_SPLIT ? split_segments(N, T, H, waves) : 1;
    const int parts = chosen == KDA_VARIANT_SPLIT ? split_parts(N, T, H, waves) : 1;
    const Layout lay = ws_layout(N, T, H, chosen, segs, waves, parts);
    const int cl = chosen == KDA_VARIANT_SPLIT ? chunk_len(waves) : KDA_CHUNK;
    const bool c32 = cl == 32;

    // profiling events: [0] before the first kernel launch, [i] after the i-th (all on
    // the caller's stream, where every kernel runs in order)
    void **ev = n_ev ? opt->stage_events : nullptr;
    int kidx = 0;
    auto around = [&](hipStream_t s, auto &&launch) -> bool {
        if (ev && kidx == 0 && hipEventRecord((hipEvent_t)ev[0], s) != hipSuccess) return false;
        if (launch() != hipSuccess) return false;
        ++kidx;
        if (ev && kidx < n_ev && hipEventRecord((hipEvent_t)ev[kidx], s) != hipSuccess) return false;
        return true;
    };
    const uint16_t *q16 = (const uint16_t *)q, *k16 = (const uint16_t *)k, *v16 = (const uint16_t *)v;

    if (chosen == KDA_VARIANT_RECURRENT) {
        const int dvt = kda::recurrent_tile((int64_t)N * H, T, N, false);
        const bool ok = around(st, [&] {
            return kda::launch_recurrent(q16, k16, v16, g, beta, scale, cu_seqlens, N, T, H, false, initial_state,
                                         out, final_state, false, dvt, st);
        });
        return ok ? KDA_OK : KDA_ERR_LAUNCH;
    }

    char *ws = nullptr;
    bool owned = false;
    if (opt && opt->workspace) {
        if (opt->workspace_bytes < lay.total) return KDA_ERR_ALLOC;
        ws = (char *)opt->workspace;
    } else {
        if (hipMallocAsync((void **)&ws, lay.total, st) != hipSuccess) {
            (void)hipGetLastError();
            return KDA_ERR_ALLOC;
        }
        owned = true;
    }
    int32_t *chunk_off = (int32_t *)(ws + lay.chunk_off);
    int32_t *order = (int32_t *)(ws + lay.order);
    int32_t *err = (int32_t *)(ws + lay.err);
    int32_t *cus = (int32_t *)(ws + lay.cu);   // sanitised cu_seqlens, written by the chunk map
    char *recs = ws + lay.recs;

    bool ok = around(st, [&] { return kda::launch_chunk_map(cu_seqlens, N, T, cus, chunk_off, order, err, cl, st); });
    if (ok && chosen == KDA_VARIANT_SPLIT) {
        const int64_t M = max_chunks(N, T, cl);
        auto prep = [&](int b, int e) {
            return c32 ? kda::launch_prep32(q16, k16, g, beta, cus, N, T, H, scale, chunk_off, recs, b, e, M, st)
                       : kda::launch_prep(q16, k16, g, beta, cus, N, T, H, scale, chunk_off, recs, b, e, M, st);
        };
        auto recur_range = [&](float *carry, int b, int e) {
            return c32 ? kda::launch_recur32_range(recs, v16, cus, chunk_off, order, N, T, H, initial_state, out, final_state, carry, waves, b, e, st)
                       : kda::launch_recur_range(recs, v16, cus, chunk_off, order, N, T, H, initial_state, out, final_state, carry, waves, b, e, st);
        };
        if (parts > 1) {
            const int NV = N * parts;
            const size_t sb = (size_t)NV * H * STATE_BYTES;
            const size_t ib = align_up(sizeof(int32_t) * (size_t)(NV + 1));
            char *pw = ws + lay.parts;
            float *ident = (float *)pw, *rb = (float *)(pw + sb), *ri = (float *)(pw + 2 * sb);
            float *sin = (float *)(pw + 3 * sb);
            int32_t *vcu = (int32_t *)(pw + 4 * sb), *vco = (int32_t *)(pw + 4 * sb + ib);
            int32_t *vorder = (int32_t *)(pw + 4 * sb + 2 * ib);
            ok = around(st, [&] { return prep(0, kda::SEG_ONE); }) &&
                 around(st, [&] {
                     return kda::launch_parts(recs, v16, cus, chunk_off, order, N, T, H, parts, initial_state, out,
                                              final_state, vcu, vco, vorder, ident, rb, ri, sin, st);
                 });
        } else if (segs == 1) {
            ok = around(st, [&] { return prep(0, kda::SEG_ONE); }) &&
                 around(st, [&] {
                     return waves >= 100 ? recur_range(final_state, 0, kda::SEG_ONE)
                                         : kda::launch_recur(recs, v16, cus, chunk_off, order, N, T, H, initial_state, out, final_state, waves, st);
                 });
        } else {
            kda::RecurPrepArgs a{recs, q16, k16, v16, g, beta, scale, cus, chunk_off, order,
                                 N, T, H, initial_state, out, final_state,
                                 final_state ? final_state : (float *)(ws + lay.carry), 0, 0, 0, 0, M};
            auto bound = [&](int sg) { return segment_frac(sg, segs, (int64_t)N * H); };
            ok = around(st, [&] { return prep(0, bound(1)); });
            for (int sg = 0; ok && sg + 1 < segs; ++sg) {
                a.fb = bound(sg), a.fe = bound(sg + 1), a.pb = bound(sg + 1), a.pe = bound(sg + 2);
                ok = around(st, [&] { return c32 ? kda::launch_recur32_prep(a, waves, st) : kda::launch_recur_prep(a, waves, st); });
            }
            ok = ok && around(st, [&] { return recur_range(a.carry, bound(segs - 1), kda::SEG_ONE); });
        }
    } else if (ok) {
        ok = around(st, [&] { return kda::launch_fused(q16, k16, v16, g, beta, cus, order, N, T, H, scale, initial_state, out, final_state, err, waves, st); });
    }
    int rc = KDA_OK;
    if (!ok) {
        rc = KDA_ERR_LAUNCH;
        if (std::getenv("KDA_DEBUG")) {
            const hipError_t e = hipGetLastError();
            std::fprintf(stderr, "kda_fwd: launch failed (variant %d): %s\n", chosen,
                         hipGetErrorString(e));
        }
    }
    if (owned && hipFreeAsync(ws, st) != hipSuccess && rc == KDA_OK) rc = KDA_ERR_DEVICE;
    return rc;
}

int kda_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
            float scale, const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens,
            int32_t num_heads, int32_t head_dim, const float *initial_state, float *out,
            float *final_state, void *stream) {
    return kda_fwd_ex(q, k, v, g, beta, scale, cu_seqlens, num_seqs, total_tokens, num_heads,
                      head_dim, initial_state, out, final_state, stream, nullptr);
}

int kda_decode(const void *q, const void *k, const void *v, const float *g, const float *beta,
               float scale, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
               const float *state_in, float *state_out, float *out, void *stream) {
    return kda_decode_ex(q, k, v, g, beta, scale, num_seqs, num_heads, head_dim, state_in, state_out, out, stream,
                         KDA_STATE_F32);
}

int kda_decode_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  float scale, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                  const void *state_in, void *state_out, float *out, void *stream, int32_t state_dtype) {
    if (head_dim != KDA_HEAD_DIM) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return KDA_ERR_UNSUPPORTED;
    if (state_dtype != KDA_STATE_F32 && state_dtype != KDA_STATE_BF16) return KDA_ERR_UNSUPPORTED;
    if (!shape_ok(num_seqs, num_seqs, num_heads)) return KDA_ERR_SHAPE;
    if (!q || !k || !v || !g || !beta || !out) return KDA_ERR_NULL;
    const size_t state_bytes =
        (size_t)num_seqs * num_heads * KDA_HEAD_DIM * KDA_HEAD_DIM * (state_dtype == KDA_STATE_BF16 ? 2 : 4);
    if (state_in && state_out && (const void *)state_in != (const void *)state_out &&
        overlaps(state_in, state_bytes, state_out, state_bytes))
        return KDA_ERR_ALIAS;
    hipStream_t st = (hipStream_t)stream;
    const int dvt = kda::recurrent_tile((int64_t)num_seqs * num_heads, num_seqs, num_seqs,
                                        state_dtype == KDA_STATE_BF16);
    if (kda::launch_recurrent((const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, g, beta, scale,
                              nullptr, num_seqs, num_seqs, num_heads, true, state_in, out, state_out,
                              state_dtype == KDA_STATE_BF16, dvt, st) != hipSuccess)
        return KDA_ERR_LAUNCH;
    return KDA_OK;
}

}  // extern "C"
