/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * Operation (per sequence n and head h, tokens t of that sequence in order):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp(max(g_t, -5))) S_{t-1} + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 *
 * with S_0 = initial_state[n,h] (zeros when NULL) and final_state[n,h] = S_last.
 * This is the gated delta rule with one decay per key channel that the
 * FlashKDA articles describe (smzdm.com, "KDA 内核到底难在哪": per-channel
 * decay over a fixed-size recurrent state, log-decay bounded below by
 * lower_bound = -5, 16-token chunks); variable-length batches are packed
 * through cu_seqlens (nerdleveltech.com, summary and "FLA" sections); only
 * head dimension K = V = 128 is supported (same article, requirements).
 *
 * All pointers except `opt` are DEVICE pointers on the current HIP device.
 * The caller owns every buffer; the library keeps no pointer after return.
 * Calls are asynchronous: work is enqueued on `stream` (NULL = the default
 * stream) and the call returns without synchronising. Errors found on the
 * host are returned before anything is enqueued; no C++ exception crosses
 * this interface.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128
#define KDA_CHUNK 16
#define KDA_LOWER_BOUND (-5.0f)

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL                              */
    KDA_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, too big  */
    KDA_ERR_UNSUPPORTED = 3, /* head_dim != 128, unknown variant, non-finite scale      */
    KDA_ERR_ALLOC = 4,       /* workspace allocation failed or caller workspace too small */
    KDA_ERR_LAUNCH = 5,      /* a kernel launch failed                                  */
    KDA_ERR_DEVICE = 6,      /* no usable gfx950 device, or a HIP runtime call failed   */
    KDA_ERR_ALIAS = 7,       /* final_state partially overlaps initial_state            */
    KDA_ERR_SCRATCH = 8      /* kda_fwd_noalloc: the call needs more than its fixed scratch */
} kda_status;

typedef enum kda_variant {
    KDA_VARIANT_AUTO = 0,  /* library picks by shape                                   */
    KDA_VARIANT_SPLIT = 1, /* chunk-parallel prep kernel + sequential recurrence kernel */
    KDA_VARIANT_FUSED = 2, /* one kernel: prep produced on chip, feeding the recurrence */
    KDA_VARIANT_RECURRENT = 3 /* token by token, no chunking: for sequences of a few tokens */
} kda_variant;

#define KDA_MAX_STAGE_EVENTS 64

/* Error bits the kernels raise on the device (they cannot be returned by the call that
 * enqueues them). Each call writes its own bits to the error word of its workspace (see
 * kda_workspace_bytes) and ORs them into the device error word that kda_device_errors
 * reads. */
#define KDA_DEVERR_TIMEOUT 1      /* the fused variant's hand-off wait gave up: that
                                     call's outputs and final_state are not valid        */
#define KDA_DEVERR_CU_SEQLENS 2   /* cu_seqlens was not 0 = c_0 <= ... <= c_N = T; the
                                     offsets were sanitised before use (see kda_fwd)     */

/* Kernel kinds reported by kda_launch_plan (profiling). */
#define KDA_KERNEL_CHUNK_MAP 0
#define KDA_KERNEL_PREP 1
#define KDA_KERNEL_RECUR 2
#define KDA_KERNEL_FUSED 3
#define KDA_KERNEL_RECUR_PREP 4   /* recurrence over one chunk range + prep of the next */
#define KDA_KERNEL_RECURRENT 5    /* token-by-token recurrence (no chunk ranges)          */
#define KDA_KERNEL_PARTS 6        /* recurrence over parts of each sequence: setup, two passes, composition */

/* Element types of kda_options.g_dtype / state_dtype (and of kda_decode_ex). */
#define KDA_DTYPE_F32 0
#define KDA_DTYPE_BF16 1

typedef struct kda_options {
    int32_t variant;        /* kda_variant                                              */
    int32_t n_stage_events; /* 0, or the length of stage_events (2..KDA_MAX_STAGE_EVENTS) */
    void *workspace;        /* device scratch, or NULL: then the library allocates it   */
                            /* stream-ordered on `stream`                               */
    size_t workspace_bytes; /* size of `workspace`; see kda_workspace_bytes()           */
    void **stage_events;    /* profiling: hipEvent_t[n_stage_events], caller-created.   */
                            /* [0] is recorded on `stream` before the first kernel      */
                            /* launch and [i] after the i-th (kda_launch_plan lists     */
                            /* them); slots past the last launch are left untouched.   */
                            /* NULL = no events.                                        */
    int32_t g_dtype;        /* KDA_DTYPE_F32 (0) or KDA_DTYPE_BF16: g holds bf16 values */
                            /* [T, H, 128] (the input-byte diet: half of g's bytes)     */
    int32_t state_dtype;    /* KDA_DTYPE_F32 (0) or KDA_DTYPE_BF16: initial_state and   */
                            /* final_state are bf16 [N, H, 128, 128] (stored in bf16,   */
                            /* updated in fp32; final_state rounded to nearest even)    */
    int32_t reserved;       /* must be 0                                                */
} kda_options;
/* bf16 g or states are read by the split variant (its 32-token forms, which it then
 * uses whatever the shape) and by the token loop; with the fused variant the call
 * returns KDA_ERR_UNSUPPORTED. */

/*
 * kda_fwd -- KDA forward (prefill) over a packed batch.
 *
 *   q, k        bf16 [total_tokens, num_heads, 128], contiguous (token-major)
 *   v           bf16 [total_tokens, num_heads, 128]
 *   g           fp32 [total_tokens, num_heads, 128]: natural-log decay per key
 *               channel (expected <= 0); values below -5 act as -5
 *   beta        fp32 [total_tokens, num_heads]: write strength per token and head
 *   scale       output scale (e.g. 1/sqrt(128)); must be finite
 *   cu_seqlens  int32 [num_seqs+1], 0 = c_0 <= c_1 <= ... <= c_N = total_tokens
 *               (sequence n owns tokens [c_n, c_{n+1})); NULL means one
 *               sequence of total_tokens tokens (then num_seqs must be 1).
 *               Monotonicity and c_N = total_tokens are preconditions checked on
 *               the device: malformed offsets are clamped to [0, T] and made
 *               non-decreasing (each raised to the largest offset before it) before
 *               any kernel uses them, by every variant (every access stays in bounds;
 *               rows outside the resulting ranges are not written), and the error bit
 *               KDA_DEVERR_CU_SEQLENS is raised (see kda_device_errors).
 *   num_seqs    N >= 1;  total_tokens T >= 0;  num_heads H >= 1;  head_dim == 128
 *   initial_state  fp32 [N, H, 128(key), 128(value)] or NULL (zeros)
 *   out         fp32 [T, H, 128]: o_t (written for every token)
 *   final_state fp32 [N, H, 128, 128] or NULL (not written). It may be the
 *               same pointer as initial_state (updated in place) but must not
 *               otherwise overlap it.
 *   stream      hipStream_t or NULL
 *
 * Returns KDA_OK or a kda_status code. Inputs are not modified.
 */
int kda_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
            float scale, const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens,
            int32_t num_heads, int32_t head_dim, const float *initial_state, float *out,
            float *final_state, void *stream);

/* kda_fwd with options (variant choice, caller-provided workspace). opt may be NULL. */
int kda_fwd_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
               float scale, const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens,
               int32_t num_heads, int32_t head_dim, const float *initial_state, float *out,
               float *final_state, void *stream, const kda_options *opt);

/* Bytes of device workspace kda_fwd_ex needs for this shape and variant
 * (0 for a variant that needs none). Returns 0 for invalid shapes too.
 * The workspace begins with int32 chunk offsets [N+1] and a sequence order [N],
 * each padded to a multiple of 256 bytes, followed by an int32 error word that a
 * call leaves at 0 or at its KDA_DEVERR_* bits. */
size_t kda_workspace_bytes(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                           int32_t variant);

/*
 * kda_fwd_noalloc -- kda_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments, outputs and errors as kda_fwd, but no allocation of any kind. The scratch
 * its kernels need (chunk offsets, sequence order, sanitised offsets and an error word:
 * about 12 bytes per sequence) lives in a fixed device array of KDA_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends. It runs the
 * token loop where KDA_VARIANT_AUTO would, and otherwise the fused variant (the split
 * variant's chunk records do not fit a fixed buffer).
 *   num_seqs at most KDA_NOALLOC_MAX_SEQS; beyond it the call returns KDA_ERR_SCRATCH
 *   before anything is enqueued.
 * Every call on one device shares that device's scratch and leaves its contents there;
 * each call rewrites what it reads before reading it. Calls that overlap in time on one
 * device (on different streams, or from different threads without ordering) race on the
 * scratch: order them on one stream.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (256 * 1024)
#define KDA_NOALLOC_MAX_SEQS 16384
int kda_fwd_noalloc(const void *q, const void *k, const void *v, const float *g, const float *beta,
                    float scale, const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                    int32_t num_heads, int32_t head_dim, const float *initial_state, float *out,
                    float *final_state, void *stream);

/* The variant KDA_VARIANT_AUTO resolves to for this shape. */
int kda_select_variant(int32_t num_seqs, int32_t total_tokens, int32_t num_heads);

/* One kernel launch of a kda_fwd_ex call: its KDA_KERNEL_* kind and the segments
 * [begin, end) whose records it prepares and whose recurrence it runs. A segment is a
 * fraction of every sequence, in units of 1/KDA_SEGMENT_ONE: of a sequence with c
 * chunks of chunk_len tokens it holds the chunks floor(c*begin/KDA_SEGMENT_ONE) to
 * floor(c*end/KDA_SEGMENT_ONE) - 1, so that every sequence advances in every launch.
 * [0, KDA_SEGMENT_ONE) is the whole batch; an empty range is 0, 0. */
#define KDA_SEGMENT_ONE 65536

typedef struct kda_launch_info {
    int32_t kind;
    int32_t prep_begin, prep_end;
    int32_t recur_begin, recur_end;
    int32_t chunk_len;          /* tokens per chunk of these ranges (16 or 32) */
} kda_launch_info;

/* The kernel launches (in order) a kda_fwd_ex call with this shape and variant makes:
 * writes up to max_launches entries to info (may be NULL) and returns the count
 * (0 for an invalid shape). When the recurrence of a shape leaves CUs idle,
 * the split variant cuts the sequences into segments and prepares the records of
 * segment s+1 inside the launch that runs the recurrence of segment s. For batches of
 * at most 63 sequences on the 32-token chunks, the first prep launch also forms the
 * chunk map (no KDA_KERNEL_CHUNK_MAP entry). The plan is that of fp32 g and states:
 * bf16 ones move a shape that would run 16-token chunks onto the 32-token ones. */
int32_t kda_launch_plan(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                        int32_t variant, kda_launch_info *info, int32_t max_launches);

/*
 * kda_decode -- one recurrence step per sequence: the decode step that continues
 * from a prefill's final_state. Sequence n has exactly one token, at row n of the
 * token-major inputs, so the operation is that of kda_fwd with cu_seqlens =
 * [0, 1, ..., N] (same formula as at the top of this file). A step costs the same
 * at any context length because the state has a fixed size (nerdleveltech.com,
 * section "سياق Kimi Linear", on Kimi Linear's decoding; smzdm.com, "KDA 内核到底难在哪",
 * on the fixed-size state): its cost is one read and one write of the fp32 state,
 * 64 KiB each per (sequence, head).
 *
 *   q, k, v     bf16 [num_seqs, num_heads, 128]
 *   g           fp32 [num_seqs, num_heads, 128] natural-log decay; below -5 acts as -5
 *   beta        fp32 [num_seqs, num_heads]
 *   scale       finite output scale
 *   num_seqs N >= 1;  num_heads H >= 1;  head_dim == 128
 *   state_in    fp32 [N, H, 128(key), 128(value)] or NULL (zeros)
 *   state_out   fp32 [N, H, 128, 128] or NULL (not written); may be the same
 *               pointer as state_in (updated in place) but must not otherwise
 *               overlap it
 *   out         fp32 [N, H, 128]
 *   stream      hipStream_t or NULL
 *
 * Needs no workspace and allocates nothing. Returns KDA_OK or a kda_status code
 * (host-side checks, before anything is enqueued; KDA_ERR_LAUNCH if the launch
 * fails). Inputs are not modified (except state_in when it is state_out).
 */
int kda_decode(const void *q, const void *k, const void *v, const float *g, const float *beta,
               float scale, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
               const float *state_in, float *state_out, float *out, void *stream);

/* State element types of kda_decode_ex. */
#define KDA_STATE_F32 0
#define KDA_STATE_BF16 1

/*
 * kda_decode_ex -- kda_decode with the state held in HBM as fp32 (KDA_STATE_F32, the
 * same as kda_decode) or as bf16 (KDA_STATE_BF16): the BF16-state form, where the state
 * is stored in bf16 and updated in fp32 (smzdm.com, "KDA 内核到底难在哪" and "反转二").
 * state_in and state_out are then bf16 [N, H, 128, 128] (state_out rounded to nearest
 * even), which halves the step's HBM traffic. Other arguments, aliasing rules and
 * errors as kda_decode; an unknown state_dtype returns KDA_ERR_UNSUPPORTED.
 */
int kda_decode_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  float scale, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                  const void *state_in, void *state_out, float *out, void *stream, int32_t state_dtype);

/*
 * kda_bwd -- gradients of kda_fwd (training). The released FlashKDA kernels run the
 * forward only, and training still goes through the Triton implementation (kucoin.com
 * news flash on the FlashKDA release); this is the backward of the operation at the top
 * of this file, derived by the chain rule through its token recurrence. Given the
 * gradient d_out of a loss with respect to out and d_final_state with respect to
 * final_state, it writes the gradients of that loss with respect to every input:
 *
 *   q, k, v, g, beta, scale, cu_seqlens, num_seqs, total_tokens, num_heads, head_dim,
 *   initial_state   as for kda_fwd (g fp32 only; initial_state fp32 or NULL = zeros)
 *   d_out           fp32 [T, H, 128] (required when T > 0)
 *   d_final_state   fp32 [N, H, 128, 128] or NULL (zeros: the loss does not read the
 *                   final state)
 *   dq, dk, dv, dg  fp32 [T, H, 128] (required when T > 0; every row of a sequence is
 *                   written). dg_t is 0 where g_t < -5: there the decay is the constant
 *                   exp(-5); at g_t = -5 it is the derivative from above.
 *   dbeta           fp32 [T, H] (required when T > 0)
 *   d_initial_state fp32 [N, H, 128, 128] or NULL (not written). Written even where
 *                   initial_state is NULL (the gradient with respect to a zero state).
 *   workspace       device scratch of kda_bwd_workspace_bytes() bytes, or NULL: then the
 *                   library allocates it stream-ordered on `stream`. It holds the state
 *                   before every KDA_BWD_BLOCK-th token of each chain (64 KiB each: about
 *                   16 KiB per token-head) and, for batches of fewer than 96 (sequence,
 *                   head) chains, four partial sums of dq, dk, dg and dbeta (6,160 B per
 *                   token-head); for few long sequences, cut into P parts, four states
 *                   of 64 KiB per part and head.
 *
 * The outputs must not overlap the inputs or each other. cu_seqlens is sanitised on the
 * device as in kda_fwd (KDA_DEVERR_CU_SEQLENS). dq, dk, dg and dbeta are sums over parts
 * of the value columns: two halves added onto zero in either order, or (fewer than 96
 * chains) four partial sums added in a fixed order. Either way the results are the same
 * from run to run. Returns KDA_OK or a kda_status code
 * (host-side checks before anything is enqueued). Inputs are not modified.
 */
#define KDA_BWD_BLOCK 4
size_t kda_bwd_workspace_bytes(int32_t num_seqs, int32_t total_tokens, int32_t num_heads);
int kda_bwd(const void *q, const void *k, const void *v, const float *g, const float *beta, float scale,
            const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
            int32_t head_dim, const float *initial_state, const float *d_out, const float *d_final_state,
            float *dq, float *dk, float *dv, float *dg, float *dbeta, float *d_initial_state, void *stream,
            void *workspace, size_t workspace_bytes);

/*
 * kda_device_errors -- the device error word of the current device: the OR of the
 * KDA_DEVERR_* bits that kernels of every call on this device (any variant, with or
 * without a caller workspace, kda_fwd included) have raised since it was last cleared.
 * Synchronises `stream` (hipStream_t or NULL) after reading, so *bits covers every call
 * enqueued on that stream before this one; calls still running on other streams may
 * raise bits later. clear != 0 resets the word to 0 (stream-ordered after the read).
 * Returns KDA_OK, KDA_ERR_NULL (bits is NULL) or KDA_ERR_DEVICE.
 */
int kda_device_errors(void *stream, int32_t *bits, int32_t clear);

/* Static, NUL-terminated description of a status code. */
const char *kda_status_string(int status);

/* Static version string. */
const char *kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
