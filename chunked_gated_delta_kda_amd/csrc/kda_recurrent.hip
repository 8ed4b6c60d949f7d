// kda_recurrent.hip -- token-by-token KDA recurrence on gfx950: the decode step
// (one token per sequence, state in and out) and the recurrent variant of the
// forward pass (any cu_seqlens, one token after another).
//
// One token of the recurrence (smzdm.com, "KDA 内核到底难在哪": per-channel decay
// over a fixed-size state; nerdleveltech.com, section "سياق Kimi Linear": a decode
// step costs the same at any context length because the state does not grow) is, with
// e = exp(max(g, -5)) per key row i and value column j:
//
//   S1[i][j] = e_i S[i][j]                     (decay)
//   u_j      = sum_i k_i S1[i][j]              (what the state predicts for k)
//   d_j      = beta (v_j - u_j)                (delta-rule correction)
//   S'[i][j] = S1[i][j] + k_i d_j              (= (I - beta k k^T) S1 + beta k v^T)
//   o_j      = scale sum_i q_i S'[i][j] = scale (sum_i q_i S1[i][j] + (q.k) d_j)
//
// so a step reads and writes the 64 KiB fp32 state once and needs two reductions
// over the key index (u and sum_i q_i S1) plus q.k. The work per step is a few
// flops per state element: the decode step is bound by HBM traffic of the state.
//
// Block = 256 threads = one (sequence, head, tile of DVT value columns). Thread
// (cg, rg) owns columns [4cg, 4cg+4) of the tile for key rows rg + RG*m: a wave's
// float4 load covers 64/CG consecutive rows of the tile, so state traffic is
// coalesced in whole rows (DVT = 128: 1 KiB per wave instruction). The state tile
// lives in registers for the whole sequence. Per token: q, k and the decay are
// staged in LDS (double-buffered: one barrier), the column reductions go through
// lane shuffles inside a wave and an LDS exchange across the four waves (second
// barrier), then every thread updates its rows. The next token's inputs are
// loaded while the current token computes.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <type_traits>

#include "kda.h"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int D = KDA_HEAD_DIM;
constexpr int NT = 256;
constexpr int NWAVE = NT / 64;
constexpr float LB = KDA_LOWER_BOUND;
constexpr float LOG2E_R = 1.4426950408889634f;
constexpr int32_t ERR_CU_SEQLENS_BIT = KDA_DEVERR_CU_SEQLENS;

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// The state is read once and written once per call: nontemporal accesses keep it
// from evicting reusable lines (measured on MI355X, decode of 256 sequences x 32
// heads: 0.193 ms against 0.215 ms with ordinary loads and stores). In HBM it is fp32,
// or bf16 (the BF16-state form: stored in bf16, updated in fp32 registers; smzdm.com,
// "KDA 内核到底难在哪" and "反转二"), which halves the decode step's traffic.
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Four consecutive value columns of one key row of the fp32 state: one 16-byte access.
__device__ __forceinline__ void load_state(const float *base, int64_t i, float (&x)[4]) {
    const f32x4v y = __builtin_nontemporal_load((const f32x4v *)(base + i));
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = y[j];
}
__device__ __forceinline__ void store_state(float *base, int64_t i, const float (&x)[4]) {
    const f32x4v y = {x[0], x[1], x[2], x[3]};
    __builtin_nontemporal_store(y, (f32x4v *)(base + i));
}
// The same four columns of a bf16 state (the input-byte diet form of the prefill's
// initial and final state): one 8-byte access, widened to fp32 / rounded to nearest even.
__device__ __forceinline__ void load_state(const uint16_t *base, int64_t i, float (&x)[4]) {
    const uint2 y = *(const uint2 *)(base + i);
    x[0] = __uint_as_float(y.x << 16), x[1] = __uint_as_float(y.x & 0xffff0000u);
    x[2] = __uint_as_float(y.y << 16), x[3] = __uint_as_float(y.y & 0xffff0000u);
}
__device__ __forceinline__ void store_state(uint16_t *base, int64_t i, const float (&x)[4]) {
    *(uint2 *)(base + i) = uint2{bf16_rne(x[0]) | (bf16_rne(x[1]) << 16), bf16_rne(x[2]) | (bf16_rne(x[3]) << 16)};
}
// g of one element: fp32, or bf16 bits
__device__ __forceinline__ float g_val(const float *g, int64_t i) { return g[i]; }
__device__ __forceinline__ float g_val(const uint16_t *g, int64_t i) { return __uint_as_float((uint32_t)g[i] << 16); }

template <int DVT, int CPT>
struct Tile {
    static constexpr int CG = DVT / CPT;  // column groups per tile
    static constexpr int RG = NT / CG;    // row groups
    static constexpr int RPT = D / RG;    // key rows per thread
    static constexpr int TILES = D / DVT;
    static_assert(CG <= 64 && 64 % CG == 0, "a wave holds whole row groups");
};

// Inputs of one token for this thread: q, k, g of key row `tid` (threads < 128),
// and v (CPT columns, bf16) and beta for every thread.
template <int CPT>
struct TokIn {
    float q, k, g;
    uint32_t v[CPT / 2];
    float beta;
};

template <int CPT, typename GT>
__device__ __forceinline__ TokIn<CPT> load_token(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                 const uint16_t *__restrict__ v, const GT *__restrict__ g,
                                                 const float *__restrict__ beta, int64_t th, int tid, int col) {
    TokIn<CPT> r;
    const int64_t o = th * D;
    const int row = tid & (D - 1);  // threads >= 128 load a row they do not use: keeps the loads unconditional
    r.q = __uint_as_float((uint32_t)q[o + row] << 16);
    r.k = __uint_as_float((uint32_t)k[o + row] << 16);
    r.g = g_val(g, o + row);
    if constexpr (CPT == 8) {
        const uint4 x = *(const uint4 *)(v + o + col);
        r.v[0] = x.x, r.v[1] = x.y, r.v[2] = x.z, r.v[3] = x.w;
    } else {
        const uint2 x = *(const uint2 *)(v + o + col);
        r.v[0] = x.x, r.v[1] = x.y;
    }
    r.beta = beta[th];
    return r;
}

// GT: g's element type (float, or uint16_t for bf16 bits); ST: the states' element type
// (float, or uint16_t for bf16 states, widened on load and rounded on store).
template <int DVT, typename GT, typename ST>
__global__ __launch_bounds__(NT) void recurrent_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const GT *__restrict__ g, const float *__restrict__ beta, float scale, const int32_t *__restrict__ cu,
    int N, int T, int H, int one_token_per_seq, const ST *s0, float *__restrict__ out, ST *sfin,
    int32_t *dev_err) {
    constexpr int CPT = 4;
    using TL = Tile<DVT, CPT>;
    __shared__ float sq[2][D], sk[2][D], se[2][D];
    __shared__ float sqk[2][2];
    __shared__ float red[NWAVE][2][TL::CG][CPT];
    __shared__ int32_t cmax[NWAVE][2];

    const int tile = blockIdx.x % TL::TILES;
    const int nh = blockIdx.x / TL::TILES;
    const int h = nh % H, n = nh / H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % TL::CG, rg = tid / TL::CG;
    const int col = tile * DVT + cg * CPT;

    // tokens of sequence n. Malformed cu_seqlens are sanitised as the split and fused
    // variants' chunk map does: every offset clamped to [0, T] and raised to the largest
    // offset before it (a running maximum, taken here over cu[0..n+1] by the block), so
    // that the ranges stay ordered, disjoint and inside [0, T]. The blocks of sequence n
    // check its own offsets and raise the device error bit when they are malformed.
    int t0, t1;
    if (one_token_per_seq) {
        t0 = n, t1 = n + 1;
    } else if (cu) {
        int32_t m0 = 0, m1 = 0;
        for (int i = tid; i <= n + 1; i += NT) {
            const int32_t x = min(max(cu[i], 0), T);
            if (i <= n) m0 = max(m0, x);
            m1 = max(m1, x);
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            m0 = max(m0, __shfl_xor(m0, off));
            m1 = max(m1, __shfl_xor(m1, off));
        }
        if (lane == 0) cmax[wave][0] = m0, cmax[wave][1] = m1;
        __syncthreads();
        t0 = cmax[0][0], t1 = cmax[0][1];
#pragma unroll
        for (int x = 1; x < NWAVE; ++x) t0 = max(t0, cmax[x][0]), t1 = max(t1, cmax[x][1]);
        if (tid == 0 && dev_err && blockIdx.x % (H * TL::TILES) == 0) {
            const int32_t a = cu[n], b = cu[n + 1];
            if ((n == 0 && a != 0) || b < a || a < 0 || b > T || (n == N - 1 && b != T))
                atomicOr(dev_err, ERR_CU_SEQLENS_BIT);
        }
    } else {
        t0 = 0, t1 = T;
    }

    const int64_t sbase = ((int64_t)n * H + h) * D * D + col;
    float st[TL::RPT][CPT];
#pragma unroll
    for (int m = 0; m < TL::RPT; ++m) {
        if (s0) {
            load_state(s0, sbase + (int64_t)(rg + TL::RG * m) * D, st[m]);
        } else {
#pragma unroll
            for (int j = 0; j < CPT; ++j) st[m][j] = 0.f;
        }
    }

    TokIn<CPT> cur{};
    if (t0 < t1) cur = load_token<CPT, GT>(q, k, v, g, beta, (int64_t)t0 * H + h, tid, col);
    for (int t = t0; t < t1; ++t) {
        const int buf = (t - t0) & 1;
        const int64_t th = (int64_t)t * H + h;
        // stage q, k and the decay of this token; q.k per wave
        if (tid < D) {
            sq[buf][tid] = cur.q;
            sk[buf][tid] = cur.k;
            se[buf][tid] = __builtin_amdgcn_exp2f(fmaxf(cur.g, LB) * LOG2E_R);
            float p = cur.q * cur.k;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) p += __shfl_xor(p, off);
            if (lane == 0) sqk[buf][wave] = p;
        }
        float vv[CPT];
#pragma unroll
        for (int j = 0; j < CPT / 2; ++j) vv[2 * j] = bf16_lo(cur.v[j]), vv[2 * j + 1] = bf16_hi(cur.v[j]);
        const float bt = cur.beta;
        // next token's inputs (the last token reloads itself: loads stay unconditional)
        const int tn = t + 1 < t1 ? t + 1 : t;
        cur = load_token<CPT, GT>(q, k, v, g, beta, (int64_t)tn * H + h, tid, col);
        __syncthreads();

        // decay, and this thread's part of u = S1^T k and w = S1^T q
        float u[CPT], w[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) u[j] = 0.f, w[j] = 0.f;
#pragma unroll
        for (int m = 0; m < TL::RPT; ++m) {
            const int r = rg + TL::RG * m;
            const float e = se[buf][r], kr = sk[buf][r], qr = sq[buf][r];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                st[m][j] *= e;
                u[j] = fmaf(kr, st[m][j], u[j]);
                w[j] = fmaf(qr, st[m][j], w[j]);
            }
        }
        // sum over the row groups of this wave (lanes that differ in the rg bits)
#pragma unroll
        for (int off = TL::CG; off < 64; off <<= 1) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) u[j] += __shfl_xor(u[j], off), w[j] += __shfl_xor(w[j], off);
        }
        if (lane < TL::CG) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) red[wave][0][lane][j] = u[j], red[wave][1][lane][j] = w[j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPT; ++j) u[j] = red[0][0][cg][j], w[j] = red[0][1][cg][j];
#pragma unroll
        for (int x = 1; x < NWAVE; ++x) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) u[j] += red[x][0][cg][j], w[j] += red[x][1][cg][j];
        }
        const float qk = sqk[buf][0] + sqk[buf][1];
        float dl[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) dl[j] = bt * (vv[j] - u[j]);
#pragma unroll
        for (int m = 0; m < TL::RPT; ++m) {
            const float kr = sk[buf][rg + TL::RG * m];
#pragma unroll
            for (int j = 0; j < CPT; ++j) st[m][j] = fmaf(kr, dl[j], st[m][j]);
        }
        if (rg == 0) {
#pragma unroll
            for (int j = 0; j < CPT; j += 4) {
                float4 o;
                o.x = scale * fmaf(qk, dl[j], w[j]), o.y = scale * fmaf(qk, dl[j + 1], w[j + 1]);
                o.z = scale * fmaf(qk, dl[j + 2], w[j + 2]), o.w = scale * fmaf(qk, dl[j + 3], w[j + 3]);
                *(float4 *)(out + th * D + col + j) = o;
            }
        }
    }
    if (sfin) {
#pragma unroll
        for (int m = 0; m < TL::RPT; ++m) store_state(sfin, sbase + (int64_t)(rg + TL::RG * m) * D, st[m]);
    }
}

// The decode step (one token per sequence), fp32 or bf16 state. The state tile stays in
// registers as it arrives (for the bf16 state: two values per VGPR, half the registers of
// an fp32 copy, so a thread keeps twice the rows and bytes in flight) and is widened
// where it is used; without the token loop of recurrent_kernel (no next-token prefetch)
// fewer registers are live. The arithmetic is that of recurrent_kernel on one token.
// For the bf16 state the sums widen through an opaque instruction and the update widens
// again in plain code, so the compiler cannot keep a widened tile alive across the
// barrier in place of the packed one.
__device__ __forceinline__ float bf16_lo_opaque(uint32_t x) {
    uint32_t r;
    asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(r) : "v"(x));
    return __uint_as_float(r);
}
__device__ __forceinline__ float bf16_hi_opaque(uint32_t x) {
    uint32_t r;
    asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(r) : "v"(x));
    return __uint_as_float(r);
}

template <int DVT, bool BF16S>
__global__ __launch_bounds__(NT) void decode_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float scale, int H,
    const void *s0, float *__restrict__ out, void *sfin) {
    constexpr int CPT = BF16S ? 8 : 4;      // value columns per thread: one 16-byte state access per row
    using SV = std::conditional_t<BF16S, u32x4v, f32x4v>;
    using SE = std::conditional_t<BF16S, uint16_t, float>;
    using TL = Tile<DVT, CPT>;
    __shared__ float sq[D], sk[D], se[D];
    __shared__ float sqk[2];
    __shared__ float red[NWAVE][2][TL::CG][CPT];

    const int tile = blockIdx.x % TL::TILES;
    const int nh = blockIdx.x / TL::TILES;
    const int h = nh % H, n = nh / H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % TL::CG, rg = tid / TL::CG;
    const int col = tile * DVT + cg * CPT;
    const int64_t sbase = ((int64_t)n * H + h) * D * D + col;

    SV sp[TL::RPT];
#pragma unroll
    for (int m = 0; m < TL::RPT; ++m) {
        if (s0)
            sp[m] = __builtin_nontemporal_load((const SV *)((const SE *)s0 + sbase + (int64_t)(rg + TL::RG * m) * D));
        else
            sp[m] = SV{};
    }
    const int64_t th = (int64_t)n * H + h;
    const TokIn<CPT> cur = load_token<CPT, float>(q, k, v, g, beta, th, tid, col);
    if (tid < D) {
        sq[tid] = cur.q;
        sk[tid] = cur.k;
        se[tid] = __builtin_amdgcn_exp2f(fmaxf(cur.g, LB) * LOG2E_R);
        float p = cur.q * cur.k;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) p += __shfl_xor(p, off);
        if (lane == 0) sqk[wave] = p;
    }
    float vv[CPT];
#pragma unroll
    for (int j = 0; j < CPT / 2; ++j) vv[2 * j] = bf16_lo(cur.v[j]), vv[2 * j + 1] = bf16_hi(cur.v[j]);
    __syncthreads();

    float u[CPT], w[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) u[j] = 0.f, w[j] = 0.f;
#pragma unroll
    for (int m = 0; m < TL::RPT; ++m) {
        const int r = rg + TL::RG * m;
        const float e = se[r], kr = sk[r], qr = sq[r];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            float x;
            if constexpr (BF16S)
                x = (j & 1) ? bf16_hi_opaque(sp[m][j >> 1]) : bf16_lo_opaque(sp[m][j >> 1]);
            else
                x = sp[m][j];
            const float s1 = x * e;
            u[j] = fmaf(kr, s1, u[j]);
            w[j] = fmaf(qr, s1, w[j]);
        }
    }
#pragma unroll
    for (int off = TL::CG; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) u[j] += __shfl_xor(u[j], off), w[j] += __shfl_xor(w[j], off);
    }
    if (lane < TL::CG) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) red[wave][0][lane][j] = u[j], red[wave][1][lane][j] = w[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPT; ++j) u[j] = red[0][0][cg][j], w[j] = red[0][1][cg][j];
#pragma unroll
    for (int x = 1; x < NWAVE; ++x) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) u[j] += red[x][0][cg][j], w[j] += red[x][1][cg][j];
    }
    const float qk = sqk[0] + sqk[1];
    float dl[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) dl[j] = cur.beta * (vv[j] - u[j]);
    if (sfin) {
#pragma unroll
        for (int m = 0; m < TL::RPT; ++m) {
            const int r = rg + TL::RG * m;
            const float e = se[r], kr = sk[r];
            SV y;
            if constexpr (BF16S) {
#pragma unroll
                for (int j = 0; j < CPT / 2; ++j) {
                    const float lo = fmaf(kr, dl[2 * j], bf16_lo(sp[m][j]) * e);
                    const float hi = fmaf(kr, dl[2 * j + 1], bf16_hi(sp[m][j]) * e);
                    y[j] = bf16_rne(lo) | (bf16_rne(hi) << 16);
                }
            } else {
#pragma unroll
                for (int j = 0; j < CPT; ++j) y[j] = fmaf(kr, dl[j], sp[m][j] * e);
            }
            __builtin_nontemporal_store(y, (SV *)((SE *)sfin + sbase + (int64_t)(rg + TL::RG * m) * D));
        }
    }
    if (rg == 0) {
#pragma unroll
        for (int j = 0; j < CPT; j += 4) {
            float4 o;
            o.x = scale * fmaf(qk, dl[j], w[j]), o.y = scale * fmaf(qk, dl[j + 1], w[j + 1]);
            o.z = scale * fmaf(qk, dl[j + 2], w[j + 2]), o.w = scale * fmaf(qk, dl[j + 3], w[j + 3]);
            *(float4 *)(out + th * D + col + j) = o;
        }
    }
}

}  // namespace

int recurrent_tile(int64_t chains, int64_t tokens, int64_t seqs, bool bf16_state) {
    // KDA_RECURRENT_TILE (128, 64 or 32) overrides the choice, for tuning
    if (const char *e = std::getenv("KDA_RECURRENT_TILE")) {
        const int t = std::atoi(e);
        if (t == 128 || t == 64 || t == 32) return t;
    }
    // Measured on MI355X, 32 heads (ms per call for 128 | 64 | 32 columns per block).
    // One token per sequence (decode_kernel): fp32 state, 24 sequences 0.022 | 0.026 |
    // 0.027, 256 sequences 0.195 | 0.199 | 0.208, 1024 sequences 0.812 | 0.801 | 0.833;
    // bf16 state, 256 sequences 0.100 | 0.106, 1024 sequences 0.370 | 0.393. Several
    // tokens per sequence (recurrent_kernel): a wider
    // tile shares the per-token work (inputs, barriers, q.k) over more columns, a narrower
    // one gives more blocks: 1 x 16 tokens 0.025 | 0.022 | 0.020; 8 x 8 0.017 | 0.015 |
    // 0.021; 64 x 16 0.096 | 0.124 | 0.222; 256 x 8 0.178 | 0.230 | 0.433.
    if (tokens <= seqs) return (chains >= 16384 && !bf16_state) ? 64 : 128;
    if (chains >= 1024) return 128;
    return chains >= 256 ? 64 : 32;
}

template <int DVT, bool BF16S>
static void launch_tile(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                        float scale, const int32_t *cu, int N, int T, int H, bool one_token_per_seq, const void *s0,
                        float *out, void *sfin, hipStream_t st) {
    const int64_t blocks = (int64_t)N * H * (D / DVT);
    if (one_token_per_seq)
        hipLaunchKernelGGL((decode_kernel<DVT, BF16S>), dim3((unsigned)blocks), dim3(NT), 0, st, q, k, v, g, beta,
                           scale, H, s0, out, sfin);
    else if constexpr (!BF16S)
        hipLaunchKernelGGL((recurrent_kernel<DVT, float, float>), dim3((unsigned)blocks), dim3(NT), 0, st, q, k, v,
                           g, beta, scale, cu, N, T, H, 0, (const float *)s0, out, (float *)sfin, device_error_word());
}

template <int DVT, typename GT, typename ST>
static void launch_fwd_tile(const uint16_t *q, const uint16_t *k, const uint16_t *v, const void *g,
                            const float *beta, float scale, const int32_t *cu, int N, int T, int H, const void *s0,
                            float *out, void *sfin, hipStream_t st) {
    const int64_t blocks = (int64_t)N * H * (D / DVT);
    hipLaunchKernelGGL((recurrent_kernel<DVT, GT, ST>), dim3((unsigned)blocks), dim3(NT), 0, st, q, k, v,
                       (const GT *)g, beta, scale, cu, N, T, H, 0, (const ST *)s0, out, (ST *)sfin,
                       device_error_word());
}

hipError_t launch_recurrent_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const void *g, bool g_bf16,
                                const float *beta, float scale, const int32_t *cu, int N, int T, int H,
                                const void *s0, float *out, void *sfin, bool s_bf16, int dvt, hipStream_t st) {
    if (!g_bf16 && !s_bf16) {
        return launch_recurrent(q, k, v, (const float *)g, beta, scale, cu, N, T, H, false, s0, out, sfin, false, dvt,
                                st);
    }
#define KDA_FWD_TILE(W)                                                                                            \
    case W:                                                                                                        \
        if (g_bf16 && s_bf16)                                                                                      \
            launch_fwd_tile<W, uint16_t, uint16_t>(q, k, v, g, beta, scale, cu, N, T, H, s0, out, sfin, st);       \
        else if (g_bf16)                                                                                           \
            launch_fwd_tile<W, uint16_t, float>(q, k, v, g, beta, scale, cu, N, T, H, s0, out, sfin, st);          \
        else                                                                                                       \
            launch_fwd_tile<W, float, uint16_t>(q, k, v, g, beta, scale, cu, N, T, H, s0, out, sfin, st);          \
        break;
    switch (dvt) {
        KDA_FWD_TILE(128)
        KDA_FWD_TILE(64)
        KDA_FWD_TILE(32)
    default:
        return hipErrorInvalidValue;
    }
#undef KDA_FWD_TILE
    return hipGetLastError();
}

hipError_t launch_recurrent(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                            const float *beta, float scale, const int32_t *cu, int N, int T, int H,
                            bool one_token_per_seq, const void *s0, float *out, void *sfin, bool bf16_state,
                            int dvt, hipStream_t st) {
    if (bf16_state && !one_token_per_seq) return hipErrorInvalidValue;   // the BF16-state form is a decode step
#define KDA_TILE_CASE(W)                                                                                     \
    case W:                                                                                                  \
        if (bf16_state)                                                                                      \
            launch_tile<W, true>(q, k, v, g, beta, scale, cu, N, T, H, one_token_per_seq, s0, out, sfin, st); \
        else                                                                                                 \
            launch_tile<W, false>(q, k, v, g, beta, scale, cu, N, T, H, one_token_per_seq, s0, out, sfin, st); \
        break;
    switch (dvt) {
        KDA_TILE_CASE(128)
        KDA_TILE_CASE(64)
        KDA_TILE_CASE(32)
    default:
        return hipErrorInvalidValue;
    }
#undef KDA_TILE_CASE
    return hipGetLastError();
}

}  // namespace kda
