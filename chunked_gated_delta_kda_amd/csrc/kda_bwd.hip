// kda_bwd.hip -- gradients of the KDA forward on gfx950 (a first backward kernel).
//
// The articles release the forward kernels only and leave training to the Triton
// implementation (kucoin.com news flash); this is the backward pass, derived by the
// chain rule from the per-token recurrence (a = exp(max(g, -5)) per key row):
//
//   S1 = Diag(a) S_{t-1};  u = S1^T k;  r = v - u;  d = beta r;  S_t = S1 + k d^T;
//   o_t = scale S_t^T q
//
// Walking the tokens backwards with dS = dL/dS_t (dL/dS_final to start):
//
//   dS += scale q do^T;         dq = scale (S1 do + k (d . do))
//   dd = dS^T k;   dk = dS d;   dbeta = dd . r;   dv = beta dd;   du = -beta dd
//   dS1 = dS + k du^T;          dk += S1 du;      dg_i = sum_j S1_ij dS1_ij (g_i >= -5)
//   dS = Diag(a) dS1
//
// Every value column j of the state evolves on its own (u_j, d_j, dd_j and du_j read
// column j only); dq, dk, dg and dbeta sum over all columns. So a wave owns CW = 8 value
// columns of one (sequence, head) chain, its state and state gradient in registers (lane
// l: key rows l and l + 64): sums over columns stay inside a lane, sums over rows (u, dd)
// are one reduction across the wave. Eight waves make a block (64 columns), two blocks a
// chain; the waves of a block add their row gradients through LDS, and the two blocks add
// theirs into zeroed outputs with one atomic add each (two addends onto zero: the result
// does not depend on their order). For batches of few chains, four blocks of four waves
// per chain, whose partial sums a last kernel adds in a fixed order (see Geo).
//
// The reverse walk needs the state before every token: a forward pass stores the state
// every BLK tokens in the workspace, then, block by block from the last, the block's
// tokens are recomputed from its checkpoint, keeping S1 and r of each in registers, and
// walked backwards. The inputs of a block of tokens reach the waves through LDS, loaded
// while the previous block computes. Work per token is O(dk dv) on the vector units (no
// MFMA): a token loop, not the chunked form; one chain occupies two CUs for the length of
// its sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "kda.h"
#include "kda_device.hpp"

namespace kda {
namespace {

constexpr int BLK = KDA_BWD_BLOCK;      // tokens per checkpoint
constexpr int CW = 8;                   // value columns per wave
constexpr float LB = KDA_LOWER_BOUND;

// A block of NWV waves owns NCOL = 8 NWV value columns of one chain; PARTS blocks make the
// chain. With 8 waves (two blocks per chain) the blocks add their row gradients straight
// into the zeroed outputs (two addends onto zero: the result does not depend on their
// order); with 4 waves (for batches of few chains, to occupy more CUs) each block writes
// its partial sums and bwd_sum_kernel adds the PARTS of them in a fixed order.
template <int NWV>
struct Geo {
    static constexpr int NCOL = CW * NWV, PARTS = D / NCOL, THREADS = 64 * NWV;
    static constexpr bool ATOMIC = PARTS == 2;
    // pieces of 16 bytes of a staged token, in this order: k, g, v (the block's columns), q,
    // d_out (the block's columns); then beta
    static constexpr int PK = 0, PG = 16, PV = 48, PQ = PV + NCOL * 2 / 16, PO = PQ + 16;
    static constexpr int PIECES = PO + NCOL * 4 / 16;
    static constexpr int PER_THREAD = (PIECES * BLK + THREADS - 1) / THREADS;
};

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_ROW_MIRROR = 0x140, DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_QUAD_2301 = 0x4e, DPP_QUAD_1032 = 0xb1;   // quad_perm [2,3,0,1], [1,0,3,2]

// Sum over the 64 lanes of x[c] for the wave's 8 columns: returns, in every lane l, the
// total of column col_of_lane(l). Three halving steps pair each lane with one that keeps
// the other half of its columns (lanes l and l ^ 32 by a 32-lane swap, rows of 16 lanes
// by a 16-lane swap, lane i of a row with lane 15 - i), then an all-reduce over each half
// row (its mirror image, then within quads). No step goes through LDS.
__device__ __forceinline__ float colsum8(const float (&x)[CW], int lane) {
    float y[4], z[2];
#pragma unroll
    for (int m = 0; m < 4; ++m) {   // lanes < 32 keep columns 0..3, the others 4..7
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[m]), __float_as_uint(x[4 + m]), false, false);
        y[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {   // even rows keep the lower two, odd rows the upper
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[m]), __float_as_uint(y[2 + m]), false, false);
        z[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const bool b3 = lane & 8;
    float s = (b3 ? z[1] : z[0]) + dpp<DPP_ROW_MIRROR>(b3 ? z[0] : z[1]);
    s += dpp<DPP_ROW_HALF_MIRROR>(s);
    s += dpp<DPP_QUAD_2301>(s);
    s += dpp<DPP_QUAD_1032>(s);
    return s;
}
// the column whose total colsum8 leaves in lane l, and a lane that holds column c
__device__ __forceinline__ int col_of_lane(int l) { return ((l >> 5) & 1) * 4 + ((l >> 4) & 1) * 2 + ((l >> 3) & 1); }
__host__ __device__ constexpr int lane_of_col(int c) { return ((c >> 2) & 1) << 5 | ((c >> 1) & 1) << 4 | (c & 1) << 3; }
// the column totals, uniform across the wave
__device__ __forceinline__ void broadcast8(float s, float (&out)[CW]) {
#pragma unroll
    for (int c = 0; c < CW; ++c) out[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), lane_of_col(c)));
}

// One token's inputs as a lane uses them: k, q, g and e = exp(max(g, -5)) of its key rows
// l and l + 64; v of the lane's column in the colsum8 layout (vl); the wave's CW value
// columns of d_out; beta.
//
// Scalars per value column (u, d = beta (v - u), dd, du, and r = v - u) are kept in the
// colsum8 layout, one column per lane, where each costs one operation; only what the
// per-element updates use (d, du) is broadcast to the whole wave.
struct Tok {
    float k[2], q[2], e[2], g[2];
    float vl, dov[CW];
    float beta;
};

// The inputs reach the waves through LDS, a group of BLK tokens at a time: while the block
// computes on one group, each thread has its pieces (16 bytes each) of the next group in
// flight, and stores them at the end of the group, behind the group's barrier. So a load
// is only waited for after a whole group of computation, in either direction of the walk,
// and the waves issue no per-token loads. A staged token is the pieces of Geo, in order.
template <int NCOL>
struct InTok {
    uint16_t k[D];        // bf16 bits
    float g[D];
    uint16_t v[NCOL];     // the block's value columns, bf16 bits
    uint16_t q[D];
    float dout[NCOL];     // the block's value columns
    float beta[4];        // [0]
};

template <int NWV>
struct Stage {
    uint4 x0, x1, x2;   // this thread's pieces (Geo::PER_THREAD of them; kept as scalars, an
                        // array here ended up in scratch memory)
    float beta;         // beta of token (tid mod BLK) of the group
    static_assert(Geo<NWV>::PER_THREAD <= 3, "pieces per thread");
};

// Load this thread's pieces of the group of BLK tokens starting at t0 (tokens past last
// repeat it: their pieces are loaded and stored but never read; so are the repeats of the
// last piece that fill the threads' share).
template <int NWV>
__device__ __forceinline__ void stage_load(Stage<NWV> &st, const uint16_t *__restrict__ q,
                                           const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                           const float *__restrict__ g, const float *__restrict__ beta,
                                           const float *__restrict__ dout, int64_t t0, int64_t last, int part,
                                           int H, int h, int tid) {
    using G = Geo<NWV>;
    auto piece = [&](int m) -> uint4 {
        const int idx = min(tid + G::THREADS * m, G::PIECES * BLK - 1);
        const int j = idx / G::PIECES, p = idx - j * G::PIECES;
        const int64_t t = min(t0 + j, last);
        const int64_t o = (t * H + h) * D;
        const int cb = G::NCOL * part;   // the block's first value column
        const char *src;
        if (p < G::PG)
            src = (const char *)(k + o) + 16 * (p - G::PK);
        else if (p < G::PV)
            src = (const char *)(g + o) + 16 * (p - G::PG);
        else if (p < G::PQ)
            src = (const char *)(v + o + cb) + 16 * (p - G::PV);
        else if (p < G::PO)
            src = (const char *)(q + o) + 16 * (p - G::PQ);
        else
            src = (const char *)(dout + o + cb) + 16 * (p - G::PO);
        return *(const uint4 *)src;
    };
    st.x0 = piece(0);
    if constexpr (G::PER_THREAD > 1) st.x1 = piece(1);
    if constexpr (G::PER_THREAD > 2) st.x2 = piece(2);
    st.beta = beta[min(t0 + (tid & (BLK - 1)), last) * H + h];
}
template <int NWV>
__device__ __forceinline__ void stage_store(InTok<Geo<NWV>::NCOL> *grp, const Stage<NWV> &st, int tid) {
    using G = Geo<NWV>;
    auto put = [&](int m, const uint4 &x) {
        const int idx = tid + G::THREADS * m;
        if (idx < G::PIECES * BLK) {
            const int j = idx / G::PIECES, p = idx - j * G::PIECES;
            *(uint4 *)((char *)&grp[j] + 16 * p) = x;
        }
    };
    put(0, st.x0);
    if constexpr (G::PER_THREAD > 1) put(1, st.x1);
    if constexpr (G::PER_THREAD > 2) put(2, st.x2);
    if (tid < BLK) grp[tid].beta[0] = st.beta;
}

// token inputs from a staged token (q and d_out only for the reverse walk); vz is a zero
// the compiler cannot see through, which keeps d_out in vector registers (it meets the
// broadcast d, held in scalar registers, in one operation)
template <int NCOL>
__device__ __forceinline__ void tok_from(Tok &x, const InTok<NCOL> &in, int wave, int lane, bool reverse, int vz) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        x.k[i] = bf16f(in.k[lane + 64 * i]);
        x.g[i] = in.g[lane + 64 * i];
        x.e[i] = __expf(fmaxf(x.g[i], LB));
        x.q[i] = reverse ? bf16f(in.q[lane + 64 * i]) : 0.f;
    }
    x.vl = bf16f(in.v[CW * wave + col_of_lane(lane)]);
    x.beta = in.beta[0];
    if (reverse) {
#pragma unroll
        for (int j = 0; j < CW / 4; ++j) {
            const float4 f = *(const float4 *)&in.dout[CW * wave + 4 * j + vz];
            x.dov[4 * j] = f.x, x.dov[4 * j + 1] = f.y, x.dov[4 * j + 2] = f.z, x.dov[4 * j + 3] = f.w;
        }
    }
}

// S1 = Diag(e) S in place; returns this lane's part of u = S1^T k (colsum8 layout)
__device__ __forceinline__ float decay_u(float (&S)[2][CW], const Tok &x, int lane) {
    float p[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) {
        S[0][c] *= x.e[0];
        S[1][c] *= x.e[1];
        p[c] = fmaf(S[1][c], x.k[1], S[0][c] * x.k[0]);
    }
    return colsum8(p, lane);
}
// S <- S1 + k d^T, d given in the colsum8 layout
__device__ __forceinline__ void write_d(float (&S)[2][CW], const Tok &x, float dl) {
    float d[CW];
    broadcast8(dl, d);
#pragma unroll
    for (int c = 0; c < CW; ++c) {
        S[0][c] = fmaf(x.k[0], d[c], S[0][c]);
        S[1][c] = fmaf(x.k[1], d[c], S[1][c]);
    }
}
// one token forward: S <- Diag(e) S + k d^T, d = beta (v - S1^T k)
__device__ __forceinline__ void fwd_step(float (&S)[2][CW], const Tok &x, int lane) {
    const float ul = decay_u(S, x, lane);
    write_d(S, x, x.beta * (x.vl - ul));
}

// this lane's rows l, l + 64 of columns [c0, c0 + CW) of a 128 x 128 fp32 state (zeros
// for a NULL source)
__device__ __forceinline__ void load_slice(float (&S)[2][CW], const float *src, int c0, int lane) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (!src) {
#pragma unroll
            for (int c = 0; c < CW; ++c) S[r][c] = 0.f;
            continue;
        }
        const float4 *p = (const float4 *)(src + (int64_t)(lane + 64 * r) * D + c0);
#pragma unroll
        for (int i = 0; i < CW / 4; ++i) {
            const float4 f = p[i];
            S[r][4 * i] = f.x, S[r][4 * i + 1] = f.y, S[r][4 * i + 2] = f.z, S[r][4 * i + 3] = f.w;
        }
    }
}
__device__ __forceinline__ void store_slice(float *dst, const float (&S)[2][CW], int c0, int lane) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        float4 *p = (float4 *)(dst + (int64_t)(lane + 64 * r) * D + c0);
#pragma unroll
        for (int i = 0; i < CW / 4; ++i)
            p[i] = make_float4(S[r][4 * i], S[r][4 * i + 1], S[r][4 * i + 2], S[r][4 * i + 3]);
    }
}

// Per-wave row gradients of the BLK tokens of a block (double-buffered by block): the waves
// add them once per block, behind one barrier. And the staged inputs, two groups.
template <int NWV>
struct BwdLds {
    float part[2][BLK][NWV][3][D];   // dq, dk, dg
    float pb[2][BLK][NWV][CW];       // dbeta, per value column
    float dv[2][BLK][Geo<NWV>::NCOL];
    InTok<Geo<NWV>::NCOL> in[2][BLK];
};
template <int NWV>
constexpr int bwd_lds() {
    static_assert(sizeof(InTok<Geo<NWV>::NCOL>) == 16 * Geo<NWV>::PIECES + 16, "staged token: whole pieces, beta");
    static_assert(sizeof(BwdLds<NWV>) <= 160 * 1024, "LDS");
    return (int)sizeof(BwdLds<NWV>);
}

// sum of a block's NWV partials of one output (stride apart), in a fixed order
template <int NWV>
__device__ __forceinline__ float sum_waves(const float *p, int stride) {
    float s[NWV];
#pragma unroll
    for (int w = 0; w < NWV; ++w) s[w] = p[w * stride];
#pragma unroll
    for (int m = NWV / 2; m > 0; m >>= 1)
#pragma unroll
        for (int w = 0; w < m; ++w) s[w] += s[w + m];
    return s[0];
}

// an atomic add and a store to global memory at an address held as an integer
typedef float f4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) f4v gf4v;
typedef __attribute__((address_space(1))) float gfloat;
__device__ __forceinline__ void gadd(uint64_t a, float v) { __builtin_amdgcn_global_atomic_fadd_f32((gfloat *)a, v); }
__device__ __forceinline__ void gstore(uint64_t a, float v) { *(gfloat *)a = v; }

// sum of n consecutive partials, in a fixed order
template <int N>
__device__ __forceinline__ float sum_fixed(const float *p) {
    float s[N];
#pragma unroll
    for (int w = 0; w < N; ++w) s[w] = p[w];
#pragma unroll
    for (int m = N / 2; m > 0; m >>= 1)
#pragma unroll
        for (int w = 0; w < m; ++w) s[w] += s[w + m];
    return s[0];
}

// grid: PARTS blocks per (sequence, head); chunk_off counts blocks of BLK tokens; ck holds
// a state per block of tokens and head. Without ATOMIC, the row gradients go to psum
// ([PARTS][T H][3][128]: dq, dk, dg) and pbeta ([PARTS][T H]) instead of dq, dk, dg, dbeta.
template <int NWV>
__global__ __launch_bounds__(64 * NWV) void bwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float scale, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int H, const float *__restrict__ s0, const float *__restrict__ dout,
    const float *__restrict__ dsf, float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv,
    float *__restrict__ dg, float *__restrict__ dbeta, float *__restrict__ ds0, float *__restrict__ ck,
    float *__restrict__ psum, float *__restrict__ pbeta, int64_t TH, int rev_parts,
    const float *__restrict__ s0_seq, const float *__restrict__ dsf_seq) {
    using G = Geo<NWV>;
    constexpr int NCOL = G::NCOL;
    extern __shared__ __attribute__((aligned(16))) char bwd_smem[];
    BwdLds<NWV> &L = *(BwdLds<NWV> *)bwd_smem;
    const int bid = xcd_remap(blockIdx.x, gridDim.x, G::PARTS);
    const int part = bid % G::PARTS, chain = bid / G::PARTS;
    const int h = chain % H, n = chain / H;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, tid = threadIdx.x;
    const int c0 = NCOL * part + CW * wave;
    const int64_t bos = cu[n], eos = cu[n + 1];
    // over parts, an empty part after the first of its sequence has nothing to do (the
    // first writes d_initial_state, even for an empty sequence)
    if (rev_parts > 0 && n % rev_parts != 0 && bos >= eos) return;
    const int nblk = (int)((eos - bos + BLK - 1) / BLK);
    const int64_t sbase = ((int64_t)n * H + h) * D * D;
    const int64_t ck_stride = (int64_t)H * D * D;
    float *ckc = ck + (int64_t)chunk_off[n] * ck_stride + (int64_t)h * D * D;   // block b: ckc + b ck_stride
    int vz;   // 0, in a vector register (see tok_from)
    asm volatile("v_mov_b32 %0, 0" : "=v"(vz));
    Stage<NWV> st;
    auto stage = [&](int64_t t0) { stage_load<NWV>(st, q, k, v, g, beta, dout, t0, eos - 1, part, H, h, tid); };
    int buf = 0;   // the staged group in use

    // Over parts (rev_parts > 0): the entry state of a sequence's first part is the
    // sequence's (s0_seq), of the others the composition's (s0); the exit gradient of its
    // last part with tokens is the sequence's (dsf_seq), of the others the composition's
    // (dsf, the part at index rev_parts - 1 - p).
    const int pidx = rev_parts > 0 ? n % rev_parts : 0;
    const int64_t seqbase = rev_parts > 0 ? ((int64_t)(n / rev_parts) * H + h) * D * D : sbase;
    const bool first_part = rev_parts == 0 || pidx == 0;
    const bool last_part = rev_parts == 0 || pidx + 1 == rev_parts || cu[n + 1] >= cu[n + 2];

    // ---- forward: the state before every BLK-th token (the start of every block)
    float S[2][CW];
    {
        const float *src = first_part ? (rev_parts > 0 ? s0_seq : s0) : s0;
        load_slice(S, src ? src + (first_part ? seqbase : sbase) : nullptr, c0, lane);
    }
    if (nblk > 0) {
        stage(bos);
        stage_store<NWV>(L.in[0], st, tid);
        __syncthreads();
    }
    // Nothing in flight as the loops start: a load pending from before a loop would be
    // waited for (with everything issued after it) at its first use in every iteration.
    __builtin_amdgcn_s_waitcnt(0);
    for (int b = 0; b < nblk; ++b) {
        const int64_t tb = bos + (int64_t)b * BLK;
        // the next group: block b + 1, or after the last, the last again for the reverse walk
        stage(b + 1 < nblk ? tb + BLK : tb);
        store_slice(ckc + (int64_t)b * ck_stride, S, c0, lane);
        const InTok<NCOL> *in = L.in[buf];
        const int nin = (int)std::min((int64_t)BLK, eos - tb);
        if (nin == BLK) {
#pragma unroll
            for (int i = 0; i < BLK; ++i) {
                Tok x;
                tok_from(x, in[i], wave, lane, false, vz);
                fwd_step(S, x, lane);
            }
        } else {
#pragma unroll
            for (int i = 0; i < BLK; ++i) {
                if (i < nin) {
                    Tok x;
                    tok_from(x, in[i], wave, lane, false, vz);
                    fwd_step(S, x, lane);
                }
            }
        }
        buf ^= 1;
        stage_store<NWV>(L.in[buf], st, tid);
        __syncthreads();
    }

    // ---- backward, block by block from the last: recompute the block's tokens from its
    // checkpoint (S1 and u of each kept in registers), then walk them backwards
    float dS[2][CW];
    {
        const int nsrc = rev_parts > 0 ? n + rev_parts - 1 - 2 * pidx : n;
        const float *src = last_part ? (rev_parts > 0 ? dsf_seq : dsf) : dsf;
        load_slice(dS, src ? src + (last_part ? seqbase : ((int64_t)nsrc * H + h) * D * D) : nullptr, c0, lane);
    }
    int par = 0;
    float Sck[2][CW];
    if (nblk > 0) load_slice(S, ckc + (int64_t)(nblk - 1) * ck_stride, c0, lane);
    __builtin_amdgcn_s_waitcnt(0);
    auto block = [&](auto full, int64_t tb, int nin, const InTok<NCOL> *in) {
        constexpr bool FULL = decltype(full)::value;
        float S1s[BLK][2][CW], rl[BLK], dl[BLK];   // S1, r = v - u and d of each token
#pragma unroll
        for (int i = 0; i < BLK; ++i) {
            if (FULL || i < nin) {
                Tok x;
                tok_from(x, in[i], wave, lane, false, vz);
                rl[i] = x.vl - decay_u(S, x, lane);
                dl[i] = x.beta * rl[i];
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int c = 0; c < CW; ++c) S1s[i][r][c] = S[r][c];
                if (i + 1 < BLK) write_d(S, x, dl[i]);
            }
        }
#pragma unroll
        for (int i = BLK - 1; i >= 0; --i) {
            if (!FULL && i >= nin) continue;
            Tok x;
            tok_from(x, in[i], wave, lane, true, vz);
            const float(&dov)[CW] = x.dov;
            const float(&S1)[2][CW] = S1s[i];
            float d[CW];
            broadcast8(dl[i], d);
            float d_do = 0.f;
#pragma unroll
            for (int c = 0; c < CW; ++c) d_do = fmaf(d[c], dov[c], d_do);
            // o_t = scale S_t^T q: dq, and the output's term of dS
            float gq[2], gk[2], gg[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                float a = 0.f;
                const float sq = scale * x.q[rr];
#pragma unroll
                for (int c = 0; c < CW; ++c) {
                    a = fmaf(S1[rr][c], dov[c], a);
                    dS[rr][c] = fmaf(sq, dov[c], dS[rr][c]);
                }
                gq[rr] = scale * fmaf(x.k[rr], d_do, a);
            }
            // dd = dS^T k; dv = beta dd; du = -beta dd; dbeta = dd . r
            float p[CW];
#pragma unroll
            for (int c = 0; c < CW; ++c) p[c] = fmaf(dS[1][c], x.k[1], dS[0][c] * x.k[0]);
            const float ddl = colsum8(p, lane);
            if ((lane & 7) == 0) {   // one lane per column
                L.dv[par][i][CW * wave + col_of_lane(lane)] = x.beta * ddl;
                L.pb[par][i][wave][col_of_lane(lane)] = ddl * rl[i];
            }
            float du[CW];
            broadcast8(-x.beta * ddl, du);
            // dk = dS d + S1 du; dS1 = dS + k du^T; dg = rows of S1 . dS1; dS_{t-1} = Diag(e) dS1
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                float a = 0.f, bs = 0.f, gs = 0.f;
#pragma unroll
                for (int c = 0; c < CW; ++c) {
                    a = fmaf(dS[rr][c], d[c], a);
                    dS[rr][c] = fmaf(x.k[rr], du[c], dS[rr][c]);
                    bs = fmaf(S1[rr][c], du[c], bs);
                    gs = fmaf(S1[rr][c], dS[rr][c], gs);
                    dS[rr][c] *= x.e[rr];
                }
                gk[rr] = a + bs;
                gg[rr] = x.g[rr] >= LB ? gs : 0.f;
            }
            // this wave's row gradients of the token, added over the block's waves below
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                L.part[par][i][wave][0][lane + 64 * rr] = gq[rr];
                L.part[par][i][wave][1][lane + 64 * rr] = gk[rr];
                L.part[par][i][wave][2][lane + 64 * rr] = gg[rr];
            }
        }
    };
    constexpr int KINDS = 7;   // combine tasks per token: dq, dk, dg (two 64-row pieces each), dv
    constexpr int TASKS = BLK * KINDS + 1, ROUNDS = (TASKS + NWV - 1) / NWV;
    constexpr int CROUNDS = G::ATOMIC ? ROUNDS : 1, PROUNDS = G::ATOMIC ? 1 : (BLK * 3 * D / 4 + G::THREADS - 1) / G::THREADS;
    float cval[CROUNDS] = {};      // the values of a wave's combine tasks (see there)
    uint64_t cadr[CROUNDS] = {};   // and their addresses
    f4v pval[PROUNDS] = {};        // without ATOMIC, the partial sums stored
    uint64_t padr[PROUNDS] = {};
    // One block of the walk, with the combine of its row gradients. Only the last block of
    // a sequence (the first walked) can be partial; the others run the FULL form, whose
    // combine has a fixed trip count.
    auto step = [&](auto full, int b) {
        constexpr bool FULL = decltype(full)::value;
        const int64_t tb = bos + (int64_t)b * BLK;
        const int nin = FULL ? BLK : (int)std::min((int64_t)BLK, eos - tb);
        // the next block's inputs and checkpoint (block 0: its own again, unused)
        const int bn = b > 0 ? b - 1 : 0;
        stage(bos + (int64_t)bn * BLK);
        load_slice(Sck, ckc + (int64_t)bn * ck_stride, c0, lane);
        block(full, tb, nin, L.in[buf]);
        // Take the next block's loads here, before this block's atomic adds are issued
        // (loads, stores and atomics share one in-order counter: a wait for a load issued
        // before the adds, if taken after them, waits for the adds too). The asm pins the
        // copy here; else the compiler moves it to the loop's back edge.
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                S[r][c] = Sck[r][c];
                asm volatile("" : "+v"(S[r][c]));
            }
        buf ^= 1;
        stage_store<NWV>(L.in[buf], st, tid);
        __syncthreads();
        // The block's waves add through LDS; then per token one atomic add (or, without
        // ATOMIC, one store of the partial sum) per row of dq, dk and dg and one for dbeta,
        // and the block's columns of dv (the reverse walk itself touches no global
        // memory). Each wave takes whole 64-row pieces, so the output it writes is the same
        // in all its lanes.
        if constexpr (G::ATOMIC) {
            // Each store's address and value stay in registers of their own until the next
            // block's combine: a register a store reads is rewritten only once the store is
            // done (the compiler waits for that), and by then it long is.
    #pragma unroll
            for (int it = 0; it < ROUNDS; ++it) {
                asm volatile("" ::"v"(cval[it]), "v"(cadr[it]));
                const int task = wave + NWV * it;
                if (task < BLK * KINDS) {
                    const int i = task / KINDS, kind = task % KINDS;
                    if (!FULL && i >= nin) continue;
                    const int64_t th = (tb + i) * H + h;
                    if (kind < 6) {
                        const int a = kind >> 1, row = 64 * (kind & 1) + lane;
                        cval[it] = sum_waves<NWV>(&L.part[par][i][0][a][row], 3 * D);
                        if (!G::ATOMIC)
                            cadr[it] = (uint64_t)(psum + (((int64_t)part * TH + th) * 3 + a) * D + row);
                        else if (a == 0)
                            cadr[it] = (uint64_t)(dq + th * D + row);
                        else if (a == 1)
                            cadr[it] = (uint64_t)(dk + th * D + row);
                        else
                            cadr[it] = (uint64_t)(dg + th * D + row);
                        asm volatile("" : "+v"(cadr[it]));
                        if (G::ATOMIC)
                            gadd(cadr[it], cval[it]);
                        else
                            gstore(cadr[it], cval[it]);
                    } else if (lane < NCOL) {
                        cval[it] = L.dv[par][i][lane];
                        cadr[it] = (uint64_t)(dv + th * D + NCOL * part + lane);
                        asm volatile("" : "+v"(cadr[it]));
                        gstore(cadr[it], cval[it]);
                    }
                } else if (task == BLK * KINDS && lane < nin) {
                    cval[it] = sum_fixed<NWV * CW>(&L.pb[par][lane][0][0]);
                    const int64_t th = (tb + lane) * H + h;
                    cadr[it] = (uint64_t)(G::ATOMIC ? dbeta + th : pbeta + (int64_t)part * TH + th);
                    asm volatile("" : "+v"(cadr[it]));
                    if (G::ATOMIC)
                        gadd(cadr[it], cval[it]);
                    else
                        gstore(cadr[it], cval[it]);
                }
            }
        } else {
            // The partial sums, a float4 of 4 rows per thread and round (a token's 384 rows
            // of dq, dk, dg are contiguous in psum), then dv and dbeta, one value per thread.
            // As above, each store's value and address stay in registers of their own.
#pragma unroll
            for (int m = 0; m < PROUNDS; ++m) {
                asm volatile("" ::"v"(pval[m]), "v"(padr[m]));
                const int idx = tid + G::THREADS * m;
                const int i = idx / (3 * D / 4), f = idx % (3 * D / 4);
                if (idx < BLK * 3 * D / 4 && (FULL || i < nin)) {
                    const int a = f / (D / 4), r4 = 4 * (f % (D / 4));
                    const f4v *src = (const f4v *)&L.part[par][i][0][a][r4];
                    f4v x[NWV];
#pragma unroll
                    for (int w = 0; w < NWV; ++w) x[w] = src[w * (3 * D / 4)];
#pragma unroll
                    for (int mm = NWV / 2; mm > 0; mm >>= 1)
#pragma unroll
                        for (int w = 0; w < mm; ++w) x[w] += x[w + mm];
                    pval[m] = x[0];
                    const int64_t th = (tb + i) * H + h;
                    padr[m] = (uint64_t)(psum + (((int64_t)part * TH + th) * 3 + a) * D + r4);
                    asm volatile("" : "+v"(padr[m]));
                    *(gf4v *)padr[m] = pval[m];
                }
            }
            asm volatile("" ::"v"(cval[0]), "v"(cadr[0]));
            if (tid < BLK * NCOL) {
                const int i = tid / NCOL, c = tid % NCOL;
                if (FULL || i < nin) {
                    cval[0] = L.dv[par][i][c];
                    cadr[0] = (uint64_t)(dv + ((tb + i) * H + h) * D + NCOL * part + c);
                    asm volatile("" : "+v"(cadr[0]));
                    gstore(cadr[0], cval[0]);
                }
            } else if (tid < BLK * NCOL + BLK) {
                const int i = tid - BLK * NCOL;
                if (FULL || i < nin) {
                    cval[0] = sum_fixed<NWV * CW>(&L.pb[par][i][0][0]);
                    cadr[0] = (uint64_t)(pbeta + (int64_t)part * TH + (tb + i) * H + h);
                    asm volatile("" : "+v"(cadr[0]));
                    gstore(cadr[0], cval[0]);
                }
            }
        }
        par ^= 1;   // the next block writes the other buffer: the barrier above orders its reuse
    };
    if (nblk > 0) {
        if (eos - (bos + (int64_t)(nblk - 1) * BLK) == BLK)
            step(std::true_type{}, nblk - 1);
        else
            step(std::false_type{}, nblk - 1);
        for (int b = nblk - 2; b >= 0; --b) step(std::true_type{}, b);
    }
    if (ds0 && first_part) store_slice(ds0 + seqbase, dS, c0, lane);   // over parts: the first part's
}

// ---- the backward over parts of each sequence (few long chains). Both maps of a part are
// affine: its exit state is M S_in + B in its entry state, and the state gradient at its
// start is Mg dS_out + Bg in the one at its end (Mg the product of the tokens' Diag(e)
// (I - beta k k^T), applied to the key rows). Each is found by running the part twice:
// from a zero entry with the real inputs (B, Bg), and from the identity with v = 0 (or
// d_out = 0) (M, Mg). The composition then walks the parts, and the full backward runs
// every part from its entry state and exit gradient.

// The parts as virtual sequences: sequence n of c blocks takes Pn = min(P, ceil(c / lstar))
// parts of c / Pn blocks (rounded), in slots n P .. n P + Pn - 1; its other slots are empty
// (at its end). vcu, vco: token and block offsets, N P + 1 each.
__global__ __launch_bounds__(256) void bwd_parts_setup_kernel(const int32_t *__restrict__ cu_safe,
                                                              const int32_t *__restrict__ chunk_off, int N, int P,
                                                              int lstar, int32_t *__restrict__ vcu,
                                                              int32_t *__restrict__ vco) {
    const int64_t nv = (int64_t)N * P;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v <= nv; v += (int64_t)gridDim.x * blockDim.x) {
        if (v == nv) {
            vco[v] = chunk_off[N];
            vcu[v] = cu_safe[N];
            continue;
        }
        const int n = (int)(v / P), p = (int)(v % P);
        const int c0 = chunk_off[n], c = chunk_off[n + 1] - c0;
        const int pn = max(1, min(P, (c + lstar - 1) / lstar));
        const int k = p < pn ? (int)(((int64_t)c * p) / pn) : c;
        vco[v] = c0 + k;
        vcu[v] = min(cu_safe[n + 1], cu_safe[n] + BLK * k);
    }
}

// Forward states only: grid 2 x (parts x H x PARTS); the first half from a zero state into
// rb, the second from the identity with v = 0 into ri ([N P][H][128][128] each). The last
// part of a sequence (the last with tokens) needs no map: no part follows it.
template <int NWV>
__global__ __launch_bounds__(64 * NWV) void bwd_fstate_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ dout,
    const int32_t *__restrict__ cu, int H, int parts, float *__restrict__ rb, float *__restrict__ ri) {
    using G = Geo<NWV>;
    constexpr int NCOL = G::NCOL;
    __shared__ InTok<NCOL> stg[2][BLK];
    const int half_grid = gridDim.x / 2;
    const bool ident = (int)blockIdx.x >= half_grid;
    const int bid = xcd_remap((int)blockIdx.x - (ident ? half_grid : 0), half_grid, G::PARTS);
    const int part = bid % G::PARTS, chain = bid / G::PARTS;
    const int h = chain % H, n = chain / H;
    // only a part followed by another of its sequence needs its map
    if (n % parts + 1 >= parts || cu[n + 1] >= cu[n + 2]) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, tid = threadIdx.x;
    const int c0 = NCOL * part + CW * wave;
    const int64_t bos = cu[n], eos = cu[n + 1];
    const int nblk = (int)((eos - bos + BLK - 1) / BLK);
    int vz;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vz));
    float S[2][CW];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < CW; ++c) S[r][c] = ident && lane + 64 * r == c0 + c ? 1.f : 0.f;
    Stage<NWV> st;
    int buf = 0;
    if (nblk > 0) {
        stage_load<NWV>(st, q, k, v, g, beta, dout, bos, eos - 1, part, H, h, tid);
        stage_store<NWV>(stg[0], st, tid);
        __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(0);
    for (int b = 0; b < nblk; ++b) {
        const int64_t tb = bos + (int64_t)b * BLK;
        stage_load<NWV>(st, q, k, v, g, beta, dout, b + 1 < nblk ? tb + BLK : tb, eos - 1, part, H, h, tid);
        const int nin = (int)std::min((int64_t)BLK, eos - tb);
#pragma unroll
        for (int i = 0; i < BLK; ++i) {
            if (i < nin) {
                Tok x;
                tok_from(x, stg[buf][i], wave, lane, false, vz);
                if (ident) x.vl = 0.f;
                fwd_step(S, x, lane);
            }
        }
        buf ^= 1;
        stage_store<NWV>(stg[buf], st, tid);
        __syncthreads();
    }
    store_slice((ident ? ri : rb) + ((int64_t)n * H + h) * D * D, S, c0, lane);
}

// State gradients only, walking each part backwards: grid as above; the first half from a
// zero gradient with the real d_out into rb, the second from the identity with d_out = 0
// into ri, each at part index parts - 1 - p (part p of a sequence). The first part's map
// is not needed: the backward of that part writes d_initial_state itself.
template <int NWV>
__global__ __launch_bounds__(64 * NWV) void bwd_rstate_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ dout, float scale,
    const int32_t *__restrict__ cu, int H, int parts, float *__restrict__ rb, float *__restrict__ ri) {
    using G = Geo<NWV>;
    constexpr int NCOL = G::NCOL;
    __shared__ InTok<NCOL> stg[2][BLK];
    const int half_grid = gridDim.x / 2;
    const bool ident = (int)blockIdx.x >= half_grid;
    const int bid = xcd_remap((int)blockIdx.x - (ident ? half_grid : 0), half_grid, G::PARTS);
    const int part = bid % G::PARTS, chain = bid / G::PARTS;
    const int h = chain % H, n = chain / H;
    // only a part with tokens after the first of its sequence needs its map
    if (n % parts == 0 || cu[n] >= cu[n + 1]) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, tid = threadIdx.x;
    const int c0 = NCOL * part + CW * wave;
    const int64_t bos = cu[n], eos = cu[n + 1];
    const int nblk = (int)((eos - bos + BLK - 1) / BLK);
    int vz;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vz));
    float dS[2][CW];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < CW; ++c) dS[r][c] = ident && lane + 64 * r == c0 + c ? 1.f : 0.f;
    Stage<NWV> st;
    int buf = 0;
    if (nblk > 0) {
        stage_load<NWV>(st, q, k, v, g, beta, dout, bos + (int64_t)(nblk - 1) * BLK, eos - 1, part, H, h, tid);
        stage_store<NWV>(stg[0], st, tid);
        __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(0);
    for (int b = nblk - 1; b >= 0; --b) {
        const int64_t tb = bos + (int64_t)b * BLK;
        stage_load<NWV>(st, q, k, v, g, beta, dout, bos + (int64_t)(b > 0 ? b - 1 : 0) * BLK, eos - 1, part, H, h,
                        tid);
        const int nin = (int)std::min((int64_t)BLK, eos - tb);
#pragma unroll
        for (int i = BLK - 1; i >= 0; --i) {
            if (i < nin) {
                Tok x;
                tok_from(x, stg[buf][i], wave, lane, true, vz);
                // dS += scale q do^T; dd = dS^T k; dS1 = dS - beta k dd^T; dS <- Diag(e) dS1
                if (!ident) {
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const float sq = scale * x.q[rr];
#pragma unroll
                        for (int c = 0; c < CW; ++c) dS[rr][c] = fmaf(sq, x.dov[c], dS[rr][c]);
                    }
                }
                float p[CW];
#pragma unroll
                for (int c = 0; c < CW; ++c) p[c] = fmaf(dS[1][c], x.k[1], dS[0][c] * x.k[0]);
                float du[CW];
                broadcast8(-x.beta * colsum8(p, lane), du);
#pragma unroll
                for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                    for (int c = 0; c < CW; ++c) dS[rr][c] = fmaf(x.k[rr], du[c], dS[rr][c]) * x.e[rr];
            }
        }
        buf ^= 1;
        stage_store<NWV>(stg[buf], st, tid);
        __syncthreads();
    }
    const int nrev = n + parts - 1 - 2 * (n % parts);
    store_slice((ident ? ri : rb) + ((int64_t)nrev * H + h) * D * D, dS, c0, lane);
}

// dq, dk, dg and dbeta as the fixed-order sums of the PARTS blocks' partials (psum
// [PARTS][T H][3][128], pbeta [PARTS][T H]); zeros for tokens outside the sequences
// (before cu[0] or from cu[N] on, possible only for offsets that were sanitised), which
// no block writes
template <int PARTS>
__global__ __launch_bounds__(256) void bwd_sum_kernel(const float4 *__restrict__ psum, const float *__restrict__ pbeta,
                                                      float4 *__restrict__ dq, float4 *__restrict__ dk,
                                                      float4 *__restrict__ dg, float *__restrict__ dbeta, int64_t TH,
                                                      int H, const int32_t *__restrict__ cu, int N) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = TH * 3 * D / 4;
    const int64_t t_lo = cu[0], t_hi = cu[N];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const int64_t th = i / (3 * D / 4), r = i % (3 * D / 4);
        const int64_t t = th / H;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t >= t_lo && t < t_hi) {
            s = psum[i];
#pragma unroll
            for (int p = 1; p < PARTS; ++p) {
                const float4 x = psum[(int64_t)p * n4 + i];
                s.x += x.x, s.y += x.y, s.z += x.z, s.w += x.w;
            }
        }
        const int a = (int)(r / (D / 4));
        float4 *dst = a == 0 ? dq : a == 1 ? dk : dg;
        dst[th * (D / 4) + r % (D / 4)] = s;
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < TH; i += stride) {
        const int64_t t = i / H;
        float s = 0.f;
        if (t >= t_lo && t < t_hi) {
            s = pbeta[i];
#pragma unroll
            for (int p = 1; p < PARTS; ++p) s += pbeta[(int64_t)p * TH + i];
        }
        dbeta[i] = s;
    }
}

// zero dq, dk, dg ([n4] float4 each) and dbeta ([nb] floats): the backward adds into them
__global__ __launch_bounds__(256) void bwd_zero_kernel(float4 *dq, float4 *dk, float4 *dg, int64_t n4, float *db,
                                                       int64_t nb) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        dq[i] = z;
        dk[i] = z;
        dg[i] = z;
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nb; i += stride) db[i] = 0.f;
}

}  // namespace

template <int NWV>
static hipError_t launch_bwd_form(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                                  const float *beta, float scale, const int32_t *cu_safe, const int32_t *chunk_off,
                                  int N, int T, int H, const float *s0, const float *dout,
                                  const float *dsf, float *dq, float *dk, float *dv, float *dg, float *dbeta, float *ds0,
                                  float *ck, float *psum, const BwdParts &parts, hipStream_t st) {
    using G = Geo<NWV>;
    const int64_t th = (int64_t)T * H;
    const int64_t n4 = th * D / 4;
    const unsigned eblocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n4 + 255) / 256, 4096));
    float *pbeta = psum ? psum + (int64_t)G::PARTS * th * 3 * D : nullptr;
    int rev_parts = 0;
    const float *s0_seq = s0, *dsf_seq = dsf;
    if (parts.P > 1) {
        // the parts as sequences; the state maps of every part (forward, then the gradient's),
        // each composed over the parts; then the backward of every part from its entry state
        // and exit gradient (the composition of the gradient maps writes d_initial_state)
        const int P = parts.P, NV = N * P;
        const unsigned sgrid = (unsigned)(2 * (int64_t)NV * H * G::PARTS);
        hipLaunchKernelGGL(bwd_parts_setup_kernel, dim3((unsigned)std::min<int64_t>((NV + 256) / 256, 1024)), dim3(256),
                           0, st, cu_safe, chunk_off, N, P, parts.lstar, parts.vcu, parts.vco);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        const int32_t *vcu = parts.vcu;
        hipLaunchKernelGGL(bwd_fstate_kernel<NWV>, dim3(sgrid), dim3(G::THREADS), 0, st, q, k, v, g, beta, dout, vcu, H,
                           P, parts.rb, parts.ri);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        if (launch_parts_compose(s0, parts.rb, parts.ri, N, P, H, parts.sinf, nullptr, vcu, false, st) != hipSuccess)
            return hipErrorLaunchFailure;
        hipLaunchKernelGGL(bwd_rstate_kernel<NWV>, dim3(sgrid), dim3(G::THREADS), 0, st, q, k, v, g, beta, dout, scale,
                           vcu, H, P, parts.rb, parts.ri);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        if (launch_parts_compose(dsf, parts.rb, parts.ri, N, P, H, parts.sinb, nullptr, vcu, true, st) != hipSuccess)
            return hipErrorLaunchFailure;
        cu_safe = parts.vcu;
        chunk_off = parts.vco;
        N = NV;
        s0 = parts.sinf;
        dsf = parts.sinb;
        rev_parts = P;
    }
    if (G::ATOMIC && th > 0) {
        hipLaunchKernelGGL(bwd_zero_kernel, dim3(eblocks), dim3(256), 0, st, (float4 *)dq, (float4 *)dk, (float4 *)dg,
                           n4, dbeta, th);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)bwd_kernel<NWV>, bwd_lds<NWV>(), lds_set) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_kernel<NWV>, dim3((unsigned)((int64_t)N * H * G::PARTS)), dim3(G::THREADS), bwd_lds<NWV>(),
                       st, q, k, v, g, beta, scale, cu_safe, chunk_off, H, s0, dout, dsf, dq, dk, dv, dg, dbeta, ds0,
                       ck, psum, pbeta, th, rev_parts, s0_seq, dsf_seq);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    if (!G::ATOMIC && th > 0)
        hipLaunchKernelGGL(bwd_sum_kernel<G::PARTS>, dim3(eblocks), dim3(256), 0, st, (const float4 *)psum, pbeta,
                           (float4 *)dq, (float4 *)dk, (float4 *)dg, dbeta, th, H, cu_safe, N);
    return hipGetLastError();
}

hipError_t launch_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                      float scale, const int32_t *cu_safe, const int32_t *chunk_off, int N,
                      int T, int H, const float *s0, const float *dout, const float *dsf, float *dq, float *dk,
                      float *dv, float *dg, float *dbeta, float *ds0, float *ck, float *psum, int waves,
                      const BwdParts &parts, hipStream_t st) {
    switch (waves) {
    case 8:
        return launch_bwd_form<8>(q, k, v, g, beta, scale, cu_safe, chunk_off, N, T, H, s0, dout, dsf, dq, dk,
                                  dv, dg, dbeta, ds0, ck, nullptr, parts, st);
    case 4:
        return launch_bwd_form<4>(q, k, v, g, beta, scale, cu_safe, chunk_off, N, T, H, s0, dout, dsf, dq, dk,
                                  dv, dg, dbeta, ds0, ck, psum, parts, st);
    default:
        return hipErrorInvalidValue;
    }
}

int bwd_block_tokens() { return BLK; }

}  // namespace kda
