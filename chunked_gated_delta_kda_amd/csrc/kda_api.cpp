// kda_api.cpp -- the C ABI declared in include/kda.h: argument validation,
// variant choice, workspace, launches. No exception crosses the interface.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kda.h"
#include "kda_launch.hpp"

namespace kda {

// Error bits raised on the device by any call on this device (see kda_device_errors).
__device__ int32_t device_error_bits;

int32_t *device_error_word() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
    static std::atomic<int32_t *> cache[64];
    if (dev < 64) {
        if (int32_t *p = cache[dev].load(std::memory_order_acquire)) return p;
    }
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(device_error_bits)) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (dev < 64) cache[dev].store((int32_t *)p, std::memory_order_release);
    return (int32_t *)p;
}

// Scratch of kda_fwd_noalloc: every device the library runs on holds one copy. In host
// code the array's name is only a stand-in for the symbol: its device address comes
// from noalloc_scratch().
static __device__ __align__(256) unsigned char noalloc_scratch_dev[KDA_NOALLOC_SCRATCH_BYTES];

// Device address of the current device's scratch, resolved once per device
// (hipGetSymbolAddress with that device current); nullptr on failure.
static void *noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
    static std::atomic<void *> cache[64];
    if (dev < 64) {
        if (void *p = cache[dev].load(std::memory_order_acquire)) return p;
    }
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch_dev)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (dev < 64) cache[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace kda

namespace {

constexpr size_t ALIGN = 256;
constexpr int KDA_MAX_SEGMENTS = 8;
static_assert(KDA_SEGMENT_ONE == kda::SEG_ONE, "segment fraction unit");

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// chunks of cl tokens: an upper bound over any split of T tokens into N sequences
int64_t max_chunks(int64_t N, int64_t T, int cl = KDA_CHUNK) { return (T + cl - 1) / cl + N; }

// Forms 401/402 consume 32-token chunk records with fp16 operands (kda_h32.hip); all
// others 16-token ones.
bool fp16_form(int waves) { return waves == 401 || waves == 402; }
int chunk_len(int waves) { return fp16_form(waves) ? 32 : KDA_CHUNK; }
size_t rec_bytes(int waves) { return fp16_form(waves) ? kda::RECH_BYTES : kda::REC_BYTES; }

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
    if (const char *e = std::getenv("KDA_PARTS")) {
        const int p = std::atoi(e);
        if (p >= 1 && p <= MAX_PARTS) return p;
    }
    if (waves != 101 && waves != 401) return 1;
    // Over 32-token records pass 1 runs four-slice blocks without outputs (2 per part and
    // entry state) and pass 2 the two-slice form when the one-slice form would not fit one
    // round: P = 64 / chains, with parts of 64 chunks or more. Measured on MI355X (ms for
    // P = 1, 2, 4, 8, 16): 65536 tokens x 8 heads 1.75, 1.59, 0.970, 0.729, 0.840; 32768 x
    // 8 0.885, 0.818, 0.523, 0.418, 0.474; 2 x 16384 x 4 0.389, 0.386, 0.270, 0.248, 0.307;
    // 16384 x 4 0.336, 0.353, 0.224, 0.181, 0.207; 2 x 65536 x 8 1.99, 1.88, 1.34, 1.44,
    // 1.53; 8192 x 16 (P = 1, 3, 4, 8) 0.236, 0.237, 0.221, 0.251; 2 x 8192 x 8 0.242, 0.238,
    // 0.221, 0.255; but 8192 x 32 (P = 1, 2, 4, 8, 16) 0.359, 0.369, 0.395, 0.444, 0.539 and
    // 4096 x 4 (P = 1, 3, 4, 8) 0.099, 0.103, 0.098, 0.108.
    if (waves == 401) {
        int64_t p = 64 / (N * H);
        const int64_t by_len = T / N / 32 / 64;
        if (by_len < p) p = by_len;
        if (p > MAX_PARTS) p = MAX_PARTS;
        return p >= 3 ? (int)p : 1;
    }
    int64_t p = 32 / (N * H);
    const int64_t by_len = max_chunks(N, T) / 64;
    if (by_len < p) p = by_len;
    if (p > MAX_PARTS) p = MAX_PARTS;
    return p >= 3 ? (int)p : 1;
}

// Recurrence form of pass 2 of the recurrence over parts (32-token records): 401 (one
// 16-column slice per block, 8 blocks per part) while the parts fit one round of the
// 256 CUs that way, else 402 (two slices, 4 blocks per part; see split_parts).
// KDA_PARTS_FORM overrides, for tuning.
int parts_pass2_waves(int64_t N, int64_t H, int P) {
    if (const char *e = std::getenv("KDA_PARTS_FORM")) {
        const int w = std::atoi(e);
        if (w == 401 || w == 402) return w;
    }
    return N * H * P * 8 <= 256 ? 401 : 402;
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


// Recurrence block shape. 9: per chain, paired or eight-wave (below). 8: eight waves
// per block, each owning 16 value columns and forming its own outputs; the block's waves
// share each chunk record through one LDS ring 2 chunks deep. 101, 102: the paired form
// (1 or 2 slices per block, a chain wave and two output waves per slice, one loader
// wave). 401, 402: the paired form over 32-token chunks with fp16 operands (kda_h32.hip).
// KDA_RECUR_WAVES overrides the choice, for tuning.
int recur_waves(int64_t N, int64_t T, int64_t H, const char *env = "KDA_RECUR_WAVES") {
    if (const char *e = std::getenv(env)) {
        const int w = std::atoi(e);
        if (w == 8 || w == 9 || w == 101 || w == 102 || w == 401 || w == 402) return w;
    }
    // The 32-token fp16 forms (401: one 16-column slice per block, 402: two) take one
    // serial step per 32 tokens. Measured on MI355X (ms per call; 401 | 402 | paired
    // 16-token 101 or 102): one sequence of 8192 tokens x 32 heads 0.341 | 0.364 | 0.438;
    // 8 x 1024 tokens x 16 heads 0.185 | 0.153 | 0.190; 65536 x 8 (over parts) 1.084 |
    // 1.64 | 1.43; 4 x 4096 x 8 0.170 | 0.198; 2 x 8192 x 16 0.327 | 0.351. With many
    // chains (ms; 402 | hybrid 9 | eight-wave 8 over 16-token records): 12 skewed
    // sequences (32768 tokens) x 32 heads 0.991 | 1.238 | -; 24 x 1024 x 32 0.736 |
    // 0.807 | 0.752; 16 x 2048 x 32 0.949 | 1.044 | 0.949; 8 x 2048 x 32 0.505 | 0.537 |
    // 0.504; but 24 x 512 x 16 0.226 | 0.258 | 0.210; 256 x 256 x 32 2.22 | 2.30 | 2.09;
    // 64 x 128 x 32 0.370 | 0.356 | 0.304; 256 x 16 x 32 0.672 | 0.431 | 0.336. So from
    // 192 chains 402 where sequences average 1024 tokens or more, else the hybrid, which
    // picks per chain on the device (paired blocks for chains longer than a CU's
    // balanced share, one eight-wave block otherwise) and so keeps one long sequence in
    // a batch of short ones off a slow eight-wave block.
    const int64_t chains = N * H;
    // 25-32 chains of 8192 tokens or more: the two-slice form on half the CUs, with the
    // prep of the next segment on the other half (split_segments), beats the one-slice
    // form on all of them. Measured on MI355X (ms; 401 | 402 over 3, 4, 5 segments): 8192
    // tokens x 32 heads 0.361 | 0.356, 0.344, 0.345; 16384 x 32 0.681 | 0.660, 0.654,
    // 0.665; but 8192 x 24 0.305 | 0.313, 0.310, 0.313; 2 x 4096 x 16 0.177 | 0.191,
    // 0.195, 0.204; 4096 x 32 0.173 | 0.188, 0.194, 0.202; 8192 x 16 0.222 | 0.283. With
    // 4 segments (segment ratio 1.0 | 1.25 | 1.6): 8192 x 32 0.355 | 0.346 | 0.361 (401:
    // 0.360); 8192 x 28 0.337 | 0.325 | 0.340 (401: 0.348); 32768 x 32 1.277 | 1.262 |
    // 1.275 (401: 1.326).
    if (chains > 24 && chains <= 32 && T >= 8192 * N) return 402;
    if (chains <= 32) return 401;
    if (chains < 192) return 402;
    return T >= 1024 * N ? 402 : 9;
}

// The split path's first prep forms the chunk map itself (no chunk-map launch) for the
// 32-token forms the shape picks by itself and batches of at most 63 sequences.
bool map_in_prep(int64_t N, int64_t T, int64_t H) {
    return fp16_form(recur_waves(N, T, H)) && kda::prep_h32_maps((int)N);
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
    // the two-slice 32-token form on 25-32 long chains (recur_waves): 5 segments (with
    // segment_ratio's r = 1.05; 4 with r = 1.25 before the last segment ran the one-slice
    // form, measured best of 3-5 then)
    if (waves == 402 && N * H <= 32) return 5;
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
// The two-slice 32-token form on 25-32 chains (five segments, the last one in the
// one-slice form on all CUs): r = 1.05. Measured on MI355X (ms warm, cold; 4 segments with
// r = 1.25 -> 5 with r = 1.05; alternating builds, 2 rounds): 8192 tokens x 32 heads
// 0.346 -> 0.338, 0.388 -> 0.377; 2 x 16384 x 16 0.357 -> 0.347, 0.398 -> 0.389; 8192 x
// 28 0.316 -> 0.316, 0.358 -> 0.359; 16384 x 32 0.646 -> 0.656, 0.694 -> 0.703.
// KDA_SEGMENT_RATIO overrides r, for tuning.
double segment_ratio(int64_t chains, int waves) {
    if (const char *e = std::getenv("KDA_SEGMENT_RATIO")) {
        const double r = std::atof(e);
        if (r >= 1.0 && r <= 4.0) return r;
    }
    if (waves == 402 && chains <= 32) return 1.05;
    const double r = 1.0 + 8.0 / (double)(chains > 0 ? chains : 1);
    return r > 2.0 ? 2.0 : r;
}
int segment_frac(int sg, int S, int64_t chains, int waves) {
    if (sg <= 0) return 0;
    if (sg >= S) return kda::SEG_ONE;
    const double r = segment_ratio(chains, waves);
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
    case KDA_ERR_SCRATCH: return "kda_fwd_noalloc: more sequences than its fixed scratch holds (KDA_NOALLOC_MAX_SEQS)";
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
    const int waves = v == KDA_VARIANT_SPLIT ? recur_waves(num_seqs, total_tokens, num_heads) : 0;
    const int cl = v == KDA_VARIANT_SPLIT ? chunk_len(waves) : KDA_CHUNK;
    kda_launch_info plan[2 + KDA_MAX_SEGMENTS];
    int n = 0;
    if (v == KDA_VARIANT_RECURRENT) {
        plan[n++] = {KDA_KERNEL_RECURRENT, 0, 0, 0, 0, 1};
        for (int i = 0; info && i < n && i < max_launches; ++i) info[i] = plan[i];
        return n;
    }
    if (v != KDA_VARIANT_SPLIT || !map_in_prep(num_seqs, total_tokens, num_heads))
        plan[n++] = {KDA_KERNEL_CHUNK_MAP, 0, 0, 0, 0, cl};
    if (v == KDA_VARIANT_SPLIT) {
        const int segs = split_segments(num_seqs, total_tokens, num_heads, waves);
        auto bound = [&](int sg) { return (int32_t)segment_frac(sg, segs, (int64_t)num_seqs * num_heads, waves); };
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
    const int waves = v == KDA_VARIANT_SPLIT ? recur_waves(num_seqs, total_tokens, num_heads) : 0;
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
    const int g_dtype = opt ? opt->g_dtype : KDA_DTYPE_F32;
    const int s_dtype = opt ? opt->state_dtype : KDA_DTYPE_F32;
    if ((g_dtype != KDA_DTYPE_F32 && g_dtype != KDA_DTYPE_BF16) || (s_dtype != KDA_DTYPE_F32 && s_dtype != KDA_DTYPE_BF16))
        return KDA_ERR_UNSUPPORTED;
    const bool g_bf16 = g_dtype == KDA_DTYPE_BF16, s_bf16 = s_dtype == KDA_DTYPE_BF16;
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
    const size_t state_bytes = (size_t)num_seqs * num_heads * KDA_HEAD_DIM * KDA_HEAD_DIM * (s_bf16 ? 2 : 4);
    if (initial_state && final_state && (const void *)initial_state != (const void *)final_state &&
        overlaps(initial_state, state_bytes, final_state, state_bytes))
        return KDA_ERR_ALIAS;

    const int chosen = variant == KDA_VARIANT_AUTO
                           ? kda_select_variant(num_seqs, total_tokens, num_heads)
                           : variant;
    // bf16 g or bf16 states: the 32-token forms and the token loop read them; the fused
    // variant does not
    if ((g_bf16 || s_bf16) && chosen == KDA_VARIANT_FUSED) return KDA_ERR_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    const int N = num_seqs, T = total_tokens, H = num_heads;
    int waves = chosen == KDA_VARIANT_SPLIT ? recur_waves(N, T, H) : fused_waves(N, H);
    if (chosen == KDA_VARIANT_SPLIT && (g_bf16 || s_bf16) && !fp16_form(waves))
        waves = (int64_t)N * H <= 32 ? 401 : 402;
    const int segs = chosen == KDA_VARIANT_SPLIT ? split_segments(N, T, H, waves) : 1;
    const int parts = chosen == KDA_VARIANT_SPLIT ? split_parts(N, T, H, waves) : 1;
    const Layout lay = ws_layout(N, T, H, chosen, segs, waves, parts);
    const int cl = chosen == KDA_VARIANT_SPLIT ? chunk_len(waves) : KDA_CHUNK;
    const bool h32 = fp16_form(waves);

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
            return kda::launch_recurrent_fwd(q16, k16, v16, g, g_bf16, beta, scale, cu_seqlens, N, T, H,
                                             initial_state, out, final_state, s_bf16, dvt, st);
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

    // the chunk map: a launch of its own, or formed by the first prep (map_in_prep)
    const bool mapped = chosen == KDA_VARIANT_SPLIT && h32 && map_in_prep(N, T, H);
    bool ok = mapped ||
              around(st, [&] { return kda::launch_chunk_map(cu_seqlens, N, T, cus, chunk_off, order, err, cl, st); });
    if (ok && chosen == KDA_VARIANT_SPLIT) {
        const int64_t M = max_chunks(N, T, cl);
        auto prep = [&](int b, int e) {
            if (mapped && b == 0)
                return kda::launch_prep_h32_map(q16, k16, g, g_bf16, beta, cu_seqlens, N, T, H, scale, recs, e, M,
                                                cus, chunk_off, order, err, st);
            if (h32) return kda::launch_prep_h32(q16, k16, g, g_bf16, beta, cus, N, T, H, scale, chunk_off, recs, b, e, M, st);
            return kda::launch_prep(q16, k16, g, beta, cus, N, T, H, scale, chunk_off, recs, b, e, M, st);
        };
        auto recur_range = [&](float *carry, int b, int e) {
            if (h32) return kda::launch_recur_h32_range(recs, v16, cus, chunk_off, order, N, T, H, initial_state, out, final_state, carry, waves, b, e, s_bf16, st);
            return kda::launch_recur_range(recs, v16, cus, chunk_off, order, N, T, H, initial_state, out, final_state, carry, waves, b, e, st);
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
                                              final_state, vcu, vco, vorder, ident, rb, ri, sin, h32, s_bf16,
                                              parts_pass2_waves(N, H, parts), st);
                 });
        } else if (segs == 1) {
            ok = around(st, [&] { return prep(0, kda::SEG_ONE); }) &&
                 around(st, [&] {
                     return waves >= 100 ? recur_range(final_state, 0, kda::SEG_ONE)
                                         : kda::launch_recur(recs, v16, cus, chunk_off, order, N, T, H, initial_state, out, final_state, waves, st);
                 });
        } else {
            // the state crosses segment boundaries in fp32: through final_state where it is fp32,
            // else through the workspace's carry buffer
            kda::RecurPrepArgs a{recs, q16, k16, v16, g, beta, scale, cus, chunk_off, order,
                                 N, T, H, initial_state, out, final_state,
                                 final_state && !s_bf16 ? final_state : (float *)(ws + lay.carry), 0, 0, 0, 0, M,
                                 g_bf16, s_bf16};
            // the form chosen for the segments (waves changes for the last one below)
            const int seg_waves = waves;
            auto bound = [&](int sg) { return segment_frac(sg, segs, (int64_t)N * H, seg_waves); };
            ok = around(st, [&] { return prep(0, bound(1)); });
            for (int sg = 0; ok && sg + 1 < segs; ++sg) {
                a.fb = bound(sg), a.fe = bound(sg + 1), a.pb = bound(sg + 1), a.pe = bound(sg + 2);
                ok = around(st, [&] {
                    return h32 ? kda::launch_recur_h32_prep(a, waves, st) : kda::launch_recur_prep(a, waves, st);
                });
            }
            // The last segment has no prep beside it: with at most 32 chains the one-slice
            // form takes all CUs (same state layout as the two-slice form's carry).
            // Measured on MI355X, 8192 tokens x 32 heads: 0.3539 -> 0.3499 ms (alternating
            // builds in one process, 4 rounds each).
            if (waves == 402 && (int64_t)N * H <= 32) waves = 401;
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

// Backward workspace: the head of the forward's (chunk offsets at KDA_BWD_BLOCK tokens,
// order, error word, sanitised offsets), then a state per block of KDA_BWD_BLOCK tokens
// and head.
// Waves per backward workgroup: 8 (two workgroups per (sequence, head), their sums added
// onto zeroed outputs) or 4 (four workgroups per chain, partial sums added by a last
// kernel, so that a batch of few chains occupies more CUs). Measured on MI355X (ms per
// call, 8 | 4 | 2 waves): 256 tokens x 2 heads 0.484 | 0.341 | 0.345; 8192 x 32 heads
// 16.9 | 11.2 | 11.2; 8 x 1024 x 8 heads 2.22 | 1.55 | 2.13; 4 x 2048 x 24 heads 4.67 |
// 4.71 | 5.37; 8 x 1024 x 16 heads 2.51 | 2.61 | 3.26. So 4 below 96 chains (unless its
// partial sums would pass 8 GiB), else 8; two waves never paid. KDA_BWD_WAVES overrides
// the choice (tests, tuning).
static int bwd_waves(int64_t N, int64_t T, int64_t H) {
    if (const char *e = std::getenv("KDA_BWD_WAVES")) {
        const int w = std::atoi(e);
        if (w == 8 || w == 4) return w;
    }
    if (N * H >= 96) return 8;
    return kda::bwd_partial_floats(T, H, 4) * 4 > ((int64_t)8 << 30) ? 8 : 4;
}

// The backward over parts of each sequence (few or skewed long chains): slots for up to P
// parts per sequence, a sequence taking one part per lstar tokens (rounded up, at least
// one). lstar = 1024 tokens, or more where the batch alone fills 1024 blocks (two or four
// per (sequence, head) and part): T H blocks / 1024. P = T / lstar as a power of two, at
// most 16; P = 1: no parts. A part costs a forward-state and a gradient-state pass on top
// of its backward, and the compositions; a sequence of one part costs neither. Measured
// on MI355X (ms per call by uniform parts): 65536 tokens x 8 heads 84.7 (1) | 34.3 (4) |
// 20.0 (8) | 17.6 (16); 8192 x 32 heads 11.1 | 9.9 | 8.7 | 7.9 (1, 2, 4, 8). KDA_BWD_PARTS
// overrides P (1..16): then every sequence takes P parts, or with KDA_BWD_PART_TOKENS one
// part per so many tokens (at most P).
struct BwdSplit {
    int P = 1, lstar = 0;   // lstar in blocks of KDA_BWD_BLOCK tokens
};
static BwdSplit bwd_parts(int64_t N, int64_t T, int64_t H, int waves) {
    BwdSplit s;
    const int64_t per_chain = waves == 8 ? 2 : 4;
    int64_t lstar = std::max<int64_t>(1024, (T * H * per_chain + 1023) / 1024);
    if (const char *e = std::getenv("KDA_BWD_PARTS")) {
        const int p = std::atoi(e);
        if (p >= 1 && p <= 16) {
            s.P = p;
            s.lstar = 1;   // every sequence in p parts, or (KDA_BWD_PART_TOKENS) one per so many
            if (const char *f = std::getenv("KDA_BWD_PART_TOKENS")) {
                const int l = std::atoi(f);
                if (l >= KDA_BWD_BLOCK) s.lstar = l / KDA_BWD_BLOCK;
            }
            return s;
        }
    }
    while (s.P < 16 && (int64_t)s.P * 2 * lstar <= T) s.P *= 2;
    s.lstar = (int)((lstar + KDA_BWD_BLOCK - 1) / KDA_BWD_BLOCK);
    (void)N;
    return s;
}

struct BwdLayout {
    size_t ck = 0, psum = 0, parts = 0, total = 0;
    int waves = 8, P = 1, lstar = 0;
};

static bool bwd_layout(int64_t N, int64_t T, int64_t H, BwdLayout *B) {
    if (!shape_ok(N, T, H)) return false;
    if (max_chunks(N, T, KDA_BWD_BLOCK) * H > (int64_t)1 << 31) return false;
    const Layout L = ws_layout(N, T, H, KDA_VARIANT_FUSED, 1, 0);
    B->waves = bwd_waves(N, T, H);
    const BwdSplit sp = bwd_parts(N, T, H, B->waves);
    B->P = sp.P, B->lstar = sp.lstar;
    // the parts' four state arrays stay within 8 GiB
    if (N * B->P * H > (int64_t)1 << 24 || 4 * N * B->P * H * (int64_t)STATE_BYTES > ((int64_t)8 << 30)) B->P = 1;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    B->ck = L.total;
    B->psum = up(B->ck + (size_t)max_chunks(N, T, KDA_BWD_BLOCK) * (size_t)H * STATE_BYTES);
    B->parts = up(B->psum + (size_t)kda::bwd_partial_floats(T, H, B->waves) * sizeof(float));
    size_t parts_bytes = 0;
    if (B->P > 1) {
        const size_t nv = (size_t)N * B->P;
        parts_bytes = up(2 * (nv + 1) * sizeof(int32_t)) + 4 * nv * (size_t)H * STATE_BYTES;
    }
    B->total = B->parts + parts_bytes;
    return true;
}

size_t kda_bwd_workspace_bytes(int32_t num_seqs, int32_t total_tokens, int32_t num_heads) {
    BwdLayout B;
    return bwd_layout(num_seqs, total_tokens, num_heads, &B) ? B.total : 0;
}

int kda_bwd(const void *q, const void *k, const void *v, const float *g, const float *beta, float scale,
            const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
            int32_t head_dim, const float *initial_state, const float *d_out, const float *d_final_state,
            float *dq, float *dk, float *dv, float *dg, float *dbeta, float *d_initial_state, void *stream,
            void *workspace, size_t workspace_bytes) {

    if (head_dim != KDA_HEAD_DIM) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return KDA_ERR_UNSUPPORTED;
    const int N = num_seqs, T = total_tokens, H = num_heads;
    BwdLayout B;
    if (!bwd_layout(N, T, H, &B)) return KDA_ERR_SHAPE;
    const size_t total = B.total;
    if (!cu_seqlens && N != 1) return KDA_ERR_SHAPE;
    if (T > 0 && (!q || !k || !v || !g || !beta || !d_out || !dq || !dk || !dv || !dg || !dbeta))
        return KDA_ERR_NULL;
    if (kda::bwd_block_tokens() != KDA_BWD_BLOCK) return KDA_ERR_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    char *ws = nullptr;
    bool owned = false;
    if (workspace) {
        if (workspace_bytes < total) return KDA_ERR_ALLOC;
        ws = (char *)workspace;
    } else {
        if (hipMallocAsync((void **)&ws, total, st) != hipSuccess) {
            (void)hipGetLastError();
            return KDA_ERR_ALLOC;
        }
        owned = true;
    }
    const Layout L = ws_layout(N, T, H, KDA_VARIANT_FUSED, 1, 0);
    int32_t *chunk_off = (int32_t *)(ws + L.chunk_off), *order = (int32_t *)(ws + L.order);
    int32_t *err = (int32_t *)(ws + L.err), *cus = (int32_t *)(ws + L.cu);
    int rc = KDA_OK;
    kda::BwdParts parts{};
    parts.P = B.P;
    parts.lstar = B.lstar;
    if (B.P > 1) {
        const size_t nv = (size_t)N * B.P;
        char *pw = ws + B.parts;
        parts.vcu = (int32_t *)pw;
        parts.vco = parts.vcu + (nv + 1);
        float *f = (float *)(pw + ((2 * (nv + 1) * sizeof(int32_t) + 255) & ~(size_t)255));
        const size_t st1 = nv * (size_t)H * KDA_HEAD_DIM * KDA_HEAD_DIM;
        parts.rb = f, parts.ri = f + st1, parts.sinf = f + 2 * st1, parts.sinb = f + 3 * st1;
    }
    if (kda::launch_chunk_map(cu_seqlens, N, T, cus, chunk_off, order, err, KDA_BWD_BLOCK, st) != hipSuccess ||
        kda::launch_bwd((const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, g, beta, scale, cus, chunk_off,
                        N, T, H, initial_state, d_out, d_final_state, dq, dk, dv, dg, dbeta, d_initial_state,
                        (float *)(ws + B.ck), (float *)(ws + B.psum), B.waves, parts, st) != hipSuccess)
        rc = KDA_ERR_LAUNCH;
    if (owned && hipFreeAsync(ws, st) != hipSuccess && rc == KDA_OK) rc = KDA_ERR_DEVICE;
    return rc;
}

int kda_device_errors(void *stream, int32_t *bits, int32_t clear) {
    if (!bits) return KDA_ERR_NULL;
    int32_t *w = kda::device_error_word();
    if (!w) return KDA_ERR_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    static const int32_t zero = 0;
    int32_t got = 0;
    if (hipMemcpyAsync(&got, w, sizeof(got), hipMemcpyDeviceToHost, st) != hipSuccess ||
        (clear && hipMemcpyAsync(w, &zero, sizeof(zero), hipMemcpyHostToDevice, st) != hipSuccess) ||
        hipStreamSynchronize(st) != hipSuccess) {
        (void)hipGetLastError();
        return KDA_ERR_DEVICE;
    }
    *bits = got;
    return KDA_OK;
}

int kda_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
            float scale, const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens,
            int32_t num_heads, int32_t head_dim, const float *initial_state, float *out,
            float *final_state, void *stream) {
    return kda_fwd_ex(q, k, v, g, beta, scale, cu_seqlens, num_seqs, total_tokens, num_heads,
                      head_dim, initial_state, out, final_state, stream, nullptr);
}

int kda_fwd_noalloc(const void *q, const void *k, const void *v, const float *g, const float *beta,
                    float scale, const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                    int32_t num_heads, int32_t head_dim, const float *initial_state, float *out,
                    float *final_state, void *stream) {
    if (!shape_ok(num_seqs, total_tokens, num_heads)) return KDA_ERR_SHAPE;
    const int picked = kda_select_variant(num_seqs, total_tokens, num_heads);
    const int variant = picked == KDA_VARIANT_RECURRENT ? KDA_VARIANT_RECURRENT : KDA_VARIANT_FUSED;
    kda_options opt{};
    opt.variant = variant;
    if (variant == KDA_VARIANT_FUSED) {
        if (num_seqs > KDA_NOALLOC_MAX_SEQS) return KDA_ERR_SCRATCH;
        const size_t need = ws_layout(num_seqs, total_tokens, num_heads, KDA_VARIANT_FUSED, 1, 0).total;
        if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
        void *ws = kda::noalloc_scratch();
        if (!ws) return KDA_ERR_DEVICE;
        opt.workspace = ws;
        opt.workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    }
    return kda_fwd_ex(q, k, v, g, beta, scale, cu_seqlens, num_seqs, total_tokens, num_heads, head_dim,
                      initial_state, out, final_state, stream, &opt);
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
