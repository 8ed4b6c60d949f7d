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
// does not depend on their order).
//
// The reverse walk needs the state before every token: a forward pass stores the state
// every BLK tokens in the workspace, then, block by block from the last, the block's
// tokens are recomputed from its checkpoint, keeping S1 and u of each in registers, and
// walked backwards. Work per token is O(dk dv) on the vector units (no MFMA): a token
// loop, not the chunked form; one chain occupies two CUs for the length of its sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "kda.h"
#include "kda_device.hpp"

namespace kda {
namespace {

constexpr int BLK = KDA_BWD_BLOCK;      // tokens per checkpoint
constexpr int CW = 8;                   // value columns per wave
constexpr int WAVES = 8;                // waves per block: 64 value columns
constexpr int HALVES = D / (CW * WAVES);
constexpr float LB = KDA_LOWER_BOUND;
static_assert(HALVES == 2, "two blocks per chain: the atomic sums have two addends");

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

// One token's inputs as this lane needs them, as loaded: bf16 bits of k and q and the
// fp32 g of key rows l and l + 64, the wave's value columns of v (bf16 bits) and d_out,
// and beta. A step converts them (ready) only where it uses them, so that the loads
// issued a step ahead are waited for there and not at their issue.
struct Raw {
    uint16_t k[2], q[2];
    float g[2];
    uint4 v;
    float4 dov[CW / 4];
    float beta;
};
struct Tok {
    float k[2], q[2], e[2], g[2];
    float v[CW], dov[CW];
    float beta;
};

__device__ __forceinline__ void load_raw(Raw &x, const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                         const uint16_t *__restrict__ v, const float *__restrict__ g,
                                         const float *__restrict__ beta, const float *__restrict__ dout, int64_t th,
                                         int c0, int lane, int vz) {
    const int64_t o = th * D;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        x.k[r] = k[o + lane + 64 * r];
        x.q[r] = q[o + lane + 64 * r];
        x.g[r] = g[o + lane + 64 * r];
    }
    // v, beta and dout are the same for every lane of the wave; vz (a zero the compiler
    // cannot see through) keeps them vector loads, which complete in order, so that a use
    // waits only for its own load. As scalar loads (out of order) every use would wait for
    // all loads in flight, the prefetched ones included.
    x.v = *(const uint4 *)(v + o + c0 + vz);
    x.beta = beta[th + vz];
    if (dout) {
#pragma unroll
        for (int j = 0; j < CW / 4; ++j) x.dov[j] = ((const float4 *)(dout + o + c0 + vz))[j];
    }
}

// Make the loads of r complete here (see the block combine in bwd_kernel).
__device__ __forceinline__ void settle(const Raw &r) {
    asm volatile("" ::"v"(r.k[0]), "v"(r.k[1]), "v"(r.q[0]), "v"(r.q[1]), "v"(r.g[0]), "v"(r.g[1]), "v"(r.v.x),
                 "v"(r.v.y), "v"(r.v.z), "v"(r.v.w), "v"(r.dov[0].x), "v"(r.dov[0].y), "v"(r.dov[0].z),
                 "v"(r.dov[0].w), "v"(r.dov[1].x), "v"(r.dov[1].y), "v"(r.dov[1].z), "v"(r.dov[1].w), "v"(r.beta));
}

__device__ __forceinline__ void ready(Tok &x, const Raw &r, bool with_dout) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        x.k[i] = bf16f(r.k[i]);
        x.q[i] = bf16f(r.q[i]);
        x.g[i] = r.g[i];
        x.e[i] = __expf(fmaxf(r.g[i], LB));
    }
    const uint32_t u[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x.v[2 * i] = __uint_as_float(u[i] << 16);
        x.v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
    x.beta = r.beta;
    if (with_dout) {
#pragma unroll
        for (int j = 0; j < CW / 4; ++j) {
            x.dov[4 * j] = r.dov[j].x, x.dov[4 * j + 1] = r.dov[j].y;
            x.dov[4 * j + 2] = r.dov[j].z, x.dov[4 * j + 3] = r.dov[j].w;
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
// S <- S1 + k d^T with d = beta (v - u)
__device__ __forceinline__ void write_step(float (&S)[2][CW], const Tok &x, float ul) {
    float u[CW];
    broadcast8(ul, u);
#pragma unroll
    for (int c = 0; c < CW; ++c) {
        const float d = x.beta * (x.v[c] - u[c]);
        S[0][c] = fmaf(x.k[0], d, S[0][c]);
        S[1][c] = fmaf(x.k[1], d, S[1][c]);
    }
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
// add them once per block, behind one barrier.
struct BwdLds {
    float part[2][BLK][WAVES][3][D];   // dq, dk, dg
    float pb[2][BLK][WAVES];           // dbeta
};
constexpr int BWD_LDS = (int)sizeof(BwdLds);
static_assert(BWD_LDS <= 160 * 1024, "LDS");

// sum of the block's WAVES partials of one output (stride apart), in a fixed order
__device__ __forceinline__ float sum_waves(const float *p, int stride) {
    float s[WAVES];
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s[w] = p[w * stride];
#pragma unroll
    for (int m = WAVES / 2; m > 0; m >>= 1)
#pragma unroll
        for (int w = 0; w < m; ++w) s[w] += s[w + m];
    return s[0];
}

// grid: 2 blocks per (sequence, head); chunk_off counts blocks of BLK tokens; ck holds a
// state per block and head
__global__ __launch_bounds__(64 * WAVES) void bwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float scale, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int H, const float *__restrict__ s0, const float *__restrict__ dout,
    const float *__restrict__ dsf, float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv,
    float *__restrict__ dg, float *__restrict__ dbeta, float *__restrict__ ds0, float *__restrict__ ck) {
    extern __shared__ __attribute__((aligned(16))) char bwd_lds[];
    BwdLds &L = *(BwdLds *)bwd_lds;
    const int bid = xcd_remap(blockIdx.x, gridDim.x, HALVES);
    const int half = bid % HALVES, chain = bid / HALVES;
    const int h = chain % H, n = chain / H;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, tid = threadIdx.x;
    const int c0 = 64 * half + CW * wave;
    const int64_t bos = cu[n], eos = cu[n + 1];
    const int nblk = (int)((eos - bos + BLK - 1) / BLK);
    const int64_t sbase = ((int64_t)n * H + h) * D * D;
    const int64_t ck_stride = (int64_t)H * D * D;
    float *ckc = ck + (int64_t)chunk_off[n] * ck_stride + (int64_t)h * D * D;   // block b: ckc + b ck_stride
    int vz;   // 0, in a VGPR (see load_raw)
    asm volatile("v_mov_b32 %0, 0" : "=v"(vz));
    auto raw = [&](Raw &x, int64_t t) { load_raw(x, q, k, v, g, beta, nullptr, t * H + h, c0, lane, vz); };
    auto rawd = [&](Raw &x, int64_t t) { load_raw(x, q, k, v, g, beta, dout, t * H + h, c0, lane, vz); };

    // ---- forward: the state before every BLK-th token. Inputs come through a ring of PF
    // loads in registers, each issued PF tokens before it is used.
    constexpr int PF = BLK;
    float S[2][CW];
    load_slice(S, s0 ? s0 + sbase : nullptr, c0, lane);
    if (bos < eos) {
        Raw ring[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) raw(ring[j], bos + j < eos ? bos + j : eos - 1);
        int64_t t0 = bos;
        for (; t0 + PF <= eos; t0 += PF) {   // whole groups of PF tokens
            store_slice(ckc + ((t0 - bos) / BLK) * ck_stride, S, c0, lane);
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                // Nothing here is conditional, and each slot is read before its refill is
                // issued, so that the refill can take the slot's registers: else the loop's
                // back edge copies the ring and so waits for every load in flight.
                const int64_t t = t0 + j;
                Tok x;
                ready(x, ring[j], false);
                __builtin_amdgcn_sched_barrier(0);
                raw(ring[j], t + PF < eos ? t + PF : eos - 1);
                write_step(S, x, decay_u(S, x, lane));
            }
        }
        if (t0 < eos) {   // the last, partial group (already in the ring)
            store_slice(ckc + ((t0 - bos) / BLK) * ck_stride, S, c0, lane);
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                if (t0 + j < eos) {
                    Tok x;
                    ready(x, ring[j], false);
                    write_step(S, x, decay_u(S, x, lane));
                }
            }
        }
    }

    // ---- backward, block by block from the last. A block's loads take 2 BLK positions:
    // position i < BLK the inputs of token i (recomputing S1 and u), position 2 BLK - 1 - i
    // those of token i again (the reverse walk); positions past the block's tokens load a
    // valid token and are skipped. They come through the same ring, each issued BLK
    // positions before it is used: recompute token i uses slot i, reverse token i slot
    // BLK - 1 - i, and each slot is refilled BLK positions on, in this block or the next.
    float dS[2][CW];
    load_slice(dS, dsf ? dsf + sbase : nullptr, c0, lane);
    int par = 0;
    Raw ring[BLK];
    float Sck[2][CW];  // the next block's checkpoint
    auto tok_pos = [&](int bb, int pos) -> int64_t {
        const int64_t tbb = bos + (int64_t)bb * BLK;
        const int nb = (int)std::min((int64_t)BLK, eos - tbb);
        const int i = pos < BLK ? pos : 2 * BLK - 1 - pos;
        return tbb + (i < nb ? i : nb - 1);
    };
    if (nblk > 0) {
        load_slice(Sck, ckc + (int64_t)(nblk - 1) * ck_stride, c0, lane);
#pragma unroll
        for (int j = 0; j < BLK; ++j) rawd(ring[j], tok_pos(nblk - 1, j));
    }
    for (int b = nblk - 1; b >= 0; --b) {
        const int64_t tb = bos + (int64_t)b * BLK;
        const int nin = (int)std::min((int64_t)BLK, eos - tb);
        float S1s[BLK][2][CW], us[BLK];   // S1 and u of each token of the block
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int c = 0; c < CW; ++c) S[r][c] = Sck[r][c];
#pragma unroll
        for (int i = 0; i < BLK; ++i) {   // positions 0 .. BLK - 1
            Tok x;
            ready(x, ring[i], false);
            __builtin_amdgcn_sched_barrier(0);
            rawd(ring[i], tok_pos(b, BLK + i));   // position BLK + i: reverse token BLK - 1 - i
            if (i < nin) {
                us[i] = decay_u(S, x, lane);
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int c = 0; c < CW; ++c) S1s[i][r][c] = S[r][c];
                if (i + 1 < nin) write_step(S, x, us[i]);
            }
        }
#pragma unroll
        for (int i = BLK - 1; i >= 0; --i) {   // positions BLK .. 2 BLK - 1
            const int slot = BLK - 1 - i;
            Tok x;
            ready(x, ring[slot], true);
            __builtin_amdgcn_sched_barrier(0);
            // the next block's position slot (block 0 reloads its own: unused)
            rawd(ring[slot], tok_pos(b > 0 ? b - 1 : 0, slot));
            if (i == 0) load_slice(Sck, ckc + (int64_t)(b > 0 ? b - 1 : 0) * ck_stride, c0, lane);
            if (i >= nin) continue;
            const float(&dov)[CW] = x.dov;
            const int64_t th = (tb + i) * H + h;

            const float(&S1)[2][CW] = S1s[i];
            float u[CW], r[CW], d[CW];
            broadcast8(us[i], u);
            float d_do = 0.f;
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                r[c] = x.v[c] - u[c];
                d[c] = x.beta * r[c];
                d_do = fmaf(d[c], dov[c], d_do);
            }
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
            float dd[CW];
            broadcast8(ddl, dd);
            dv[th * D + c0 + col_of_lane(lane)] = x.beta * ddl;   // eight lanes per column, one value
            float pbeta = 0.f, du[CW];
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                pbeta = fmaf(dd[c], r[c], pbeta);
                du[c] = -x.beta * dd[c];
            }
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
            if (lane == 0) L.pb[par][i][wave] = pbeta;
        }
        // The next block's loads (issued during this block's reverse walk) land before the
        // atomic adds below are issued, so that waiting for them later does not also wait
        // for the adds (loads, stores and atomics share one in-order counter).
#pragma unroll
        for (int j = 0; j < BLK; ++j) settle(ring[j]);
        asm volatile("" ::"v"(Sck[0][0]), "v"(Sck[0][1]), "v"(Sck[0][2]), "v"(Sck[0][3]), "v"(Sck[0][4]),
                     "v"(Sck[0][5]), "v"(Sck[0][6]), "v"(Sck[0][7]), "v"(Sck[1][0]), "v"(Sck[1][1]), "v"(Sck[1][2]),
                     "v"(Sck[1][3]), "v"(Sck[1][4]), "v"(Sck[1][5]), "v"(Sck[1][6]), "v"(Sck[1][7]));
        __syncthreads();
        // the block's waves add through LDS, then one atomic add per output and token
        for (int o = tid; o < nin * (3 * D + 1); o += 64 * WAVES) {
            const int i = o / (3 * D + 1), rem = o % (3 * D + 1);
            const int64_t th = (tb + i) * H + h;
            if (rem == 3 * D) {
                unsafeAtomicAdd(dbeta + th, sum_waves(&L.pb[par][i][0], 1));
            } else {
                const int a = rem / D, row = rem % D;
                float *dst = a == 0 ? dq : a == 1 ? dk : dg;
                unsafeAtomicAdd(dst + th * D + row, sum_waves(&L.part[par][i][0][a][row], 3 * D));
            }
        }
        par ^= 1;   // the next block writes the other buffer: the barrier above orders its reuse
    }
    if (ds0) store_slice(ds0 + sbase, dS, c0, lane);
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

hipError_t launch_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                      float scale, const int32_t *cu_safe, const int32_t *chunk_off, int N, int T, int H,
                      const float *s0, const float *dout, const float *dsf, float *dq, float *dk, float *dv,
                      float *dg, float *dbeta, float *ds0, float *ck, hipStream_t st) {
    const int64_t th = (int64_t)T * H;
    if (th > 0) {
        const int64_t n4 = th * D / 4;
        const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (float4 *)dq, (float4 *)dk,
                           (float4 *)dg, n4, dbeta, th);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)bwd_kernel, BWD_LDS, lds_set) != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_kernel, dim3((unsigned)((int64_t)N * H * HALVES)), dim3(64 * WAVES), BWD_LDS, st, q, k,
                       v, g, beta, scale, cu_safe, chunk_off, H, s0, dout, dsf, dq, dk, dv, dg, dbeta, ds0, ck);
    return hipGetLastError();
}

int bwd_block_tokens() { return BLK; }

}  // namespace kda
