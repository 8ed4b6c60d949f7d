// kda_device.hpp -- device building blocks of the gfx950 KDA forward.
//
// Chunked form of the recurrence (per sequence and head; chunk of n <= 16
// tokens, G_r = in-chunk cumulative clamped log-decay per key channel,
// K+ = K.e^{G}, K- = K.e^{-G}, Q+ = scale.Q.e^{G}, K~ = K.e^{G_C - G}):
//
//   A   = Diag(beta) . strict_lower(K+ K-^T)          16x16
//   T   = (I + A)^{-1} = (I - A)(I + A^2)(I + A^4)(I + A^8)   (A^16 = 0)
//   W   = T Diag(beta) K+ ,  U = T Diag(beta) V       16x128
//   Vn  = U - W S                                     true per-token writes
//   O   = Q+ S + incl_lower(Q+ K-^T) Vn               outputs of the chunk
//   S  <- Diag(e^{G_C}) S + K~^T Vn                   next chunk's state
//
// The 16-token chunking, the strictly lower 16x16 matrix whose inverse is a
// Neumann series folded by repeated squaring, and the -5 bound that keeps
// every e^{+-G} inside the floating-point range all follow the description of
// FlashKDA's kernels (smzdm.com, "KDA 内核到底难在哪"). The rest is this
// library's own derivation from the per-token recurrence.
//
// Matrix products run on v_mfma_f32_16x16x32_bf16. Operand layouts (verified
// on gfx950): A-operand lane l holds row l%16, k-slots 8*(l/16)+i (i<8);
// B-operand lane l holds column l%16, the same k-slots; the 16x16 fp32
// result ("D layout") has lane l holding rows 4*(l/16)+j (j<4), column l%16.
// A contraction only needs A and B to agree on which logical k each slot
// carries, so every product below relabels slots freely:
//  * "hi/lo folding": slots 8g+j carry (k = 4g+j, hi part) and 8g+4+j carry
//    (k = 4g+j, lo part) of a split-bf16 operand x = hi + lo, so one MFMA
//    over a D-layout operand gives x_hi.y + x_lo.y or y.(x_hi + x_lo). With
//    A = [a_hi | a_lo] and B = [b_hi | b_hi] then [b_lo | 0], two MFMAs give the
//    three-term product a_hi.b_hi + a_lo.b_hi + a_hi.b_lo, and the B operands
//    are built once per chunk for every A that meets them.
//  * "state permutation": for the 128-deep products against the state, slot
//    8g+j of k-block kb is key channel 32kb+4g+j and slot 8g+4+j is
//    32kb+16+4g+j. With that labelling the fp32 state, kept in D layout as
//    eight 16-row blocks, converts in registers to the B operand of W.S and
//    Q+.S without any data exchange between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_launch.hpp"

namespace kda {

constexpr int D = 128;             // head dimension (key and value)
constexpr int C = 16;              // chunk length
constexpr float LOWER_BOUND = -5.0f;
constexpr float LOG2E = 1.4426950408889634f;

// Precision recipe of the state products (compile-time): whether the state's
// bf16 lo part enters W.S and Q+.S (1) or only its hi part (0).
#ifndef KDA_SPLIT_S_WS
#define KDA_SPLIT_S_WS 1
#endif
#ifndef KDA_SPLIT_S_QS
#define KDA_SPLIT_S_QS 1
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- primitives
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// e^x through the hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp_e(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }

// Two floats to packed bf16 (round to nearest even): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// x = hi + lo with hi = bf16(x) (round to nearest even) and lo = bf16(x - hi);
// 3 VALU operations per element (pack-convert, unpack, subtract, pack-convert).
__device__ __forceinline__ void split2(f32x2 x, bf16x2 &hi, bf16x2 &lo) {
    const uint32_t h = pack2(x.x, x.y);
    const float h0 = __uint_as_float(h << 16), h1 = __uint_as_float(h & 0xffff0000u);
    hi = __builtin_bit_cast(bf16x2, h);
    lo = __builtin_bit_cast(bf16x2, pack2(x.x - h0, x.y - h1));
}

__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
    bf16x2 h0, l0, h1, l1;
    split2(f32x2{x[0], x[1]}, h0, l0);
    split2(f32x2{x[2], x[3]}, h1, l1);
    hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3);
    lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3);
}

// Round four floats to bf16.
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
    return __builtin_bit_cast(bf16x4, (uint2{pack2(x[0], x[1]), pack2(x[2], x[3])}));
}

// Blocks are handed to the 8 XCDs round-robin (block b -> XCD b % 8), in increasing
// b. The logical index is chain * parts + part (parts blocks per (sequence, head)
// chain, chains in priority order, longest sequence first). Chains are dealt to the
// XCDs in turn, eight at a time: the first chains spread over the whole chip and start
// first, and the blocks of one chain share an XCD (and its L2, where they all read
// that chain's records). A chain-contiguous range per XCD would instead pile the
// longest chains onto one XCD's CUs.
__device__ __forceinline__ int xcd_remap(int b, int nb, int parts) {
    const int chains = nb / parts;
    const int full = chains >> 3;                // complete groups of eight chains
    const int g = b / (8 * parts);
    if (g < full) {
        const int j = b - g * 8 * parts;
        return ((g << 3) + (j & 7)) * parts + (j >> 3);
    }
    const int r = chains - (full << 3);          // chains of the last group (1..7)
    if (r <= 0 || b >= nb) return b;
    const int j = b - full * 8 * parts;
    return ((full << 3) + j % r) * parts + j / r;
}

// ---------------------------------------------------------------- chunk record
// Everything the recurrence needs from one (chunk, head), in per-lane order so
// that each lane of a wave reads contiguous 8/16-byte pieces. Offsets in bytes.
struct Rec {
    // pieces the state chain reads, first (one contiguous run of whole 1 KiB loads)
    static constexpr int WN = 0;       // bf16 [4 kb][64 lanes][8]: -W, state-permuted A operand
    static constexpr int KT = 4096;    // bf16 [8 blocks][64][8]: K~[4g+j][16b + l%16] hi(4) | lo(4)
    static constexpr int TB = 12288;   // bf16 [64][8]: (T Diag(beta))[l%16][4g+j] hi | lo
    static constexpr int EGP = 13312;  // f32 [128]: e^{G_C}, lane-permuted (egp_index): 8 B per lane
    static constexpr int EG = 13824;   // f32 [128]: e^{G_C} per key channel
    static constexpr int CHAIN = 14336;
    // pieces the output reads
    static constexpr int QH = 14336;   // bf16 [4][64][8]: Q+ hi, state-permuted A operand
    static constexpr int QL = 18432;   // bf16 [4][64][8]: Q+ lo
    static constexpr int PP = 22528;   // bf16 [64][8]: P[l%16][4g+j] hi(4) | lo(4) (causal, diagonal kept)
    static constexpr int BYTES = 23552; // whole 1 KiB wave loads (64 lanes x 16 B)
};
static_assert(Rec::CHAIN % 1024 == 0 && Rec::BYTES % 1024 == 0, "record pieces in whole wave loads");
// Position of key channel r in the lane-permuted decay vector: lane (c, g) of the
// MFMA D layout holds, as two floats, the decays of rows 16*(c/2) + 4g + 2*(c%2) + i
// (i = 0, 1), so that row 16b + 4g + j sits in lane 2b + j/2 of row group g.
__host__ __device__ constexpr int egp_index(int r) {
    return ((((r & 15) >> 2) * 16 + 2 * (r >> 4) + ((r & 3) >> 1)) * 2) + (r & 1);
}

// x broadcast from lane N of each 16-lane row to the whole row
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N,
                                                              0xf, 0xf, true));
}
// state block B (rows 16B + 4g + j) times its decay; e = this lane's pair of the
// lane-permuted decay vector
template <int B>
__device__ __forceinline__ f32x4 decay_block(f32x4 s, f32x2 e) {
    return f32x4{s[0] * row_bcast<2 * B>(e[0]), s[1] * row_bcast<2 * B>(e[1]),
                 s[2] * row_bcast<2 * B + 1>(e[0]), s[3] * row_bcast<2 * B + 1>(e[1])};
}

// decay_block with a block index that is a constant only after unrolling
__device__ __forceinline__ f32x4 decay_any(int b, f32x4 s, f32x2 e) {
    switch (b) {
    case 0: return decay_block<0>(s, e);
    case 1: return decay_block<1>(s, e);
    case 2: return decay_block<2>(s, e);
    case 3: return decay_block<3>(s, e);
    case 4: return decay_block<4>(s, e);
    case 5: return decay_block<5>(s, e);
    case 6: return decay_block<6>(s, e);
    default: return decay_block<7>(s, e);
    }
}

// LDS scratch of one chunk prep (one wave).
// Unpadded tiles with XOR-swizzled placement (25 KiB: six prep waves fit on a CU).
// Token-row tiles [16 tokens][128 channels]: the 16-byte unit u of row r sits at unit
// u ^ r, so the 16 rows read by one MFMA operand load fall in distinct banks. The
// transposed tile [128 channels][16 tokens]: the 8-byte piece e of channel row c sits
// at piece e ^ ((c >> 2) & 3). No access crosses a unit (or a piece).
struct alignas(16) PrepLds {
    __bf16 kp[16 * D];                 // K+ (single bf16)
    __bf16 kmh[16 * D];                // K- hi
    __bf16 kml[16 * D];                // K- lo
    __bf16 qph[16 * D];                // Q+ hi
    __bf16 qpl[16 * D];                // Q+ lo
    __bf16 kpt[D * C];                 // K+ transposed: [channel][token]
    float egs[D];                      // lane-permutation scratch (32-token records)
    // bf16 index of (token row r, channel c) in a token-row tile
    __device__ static constexpr int at(int r, int c) { return r * D + ((((c >> 3) ^ r) & 15) << 3) + (c & 7); }
    // bf16 index of (channel c, token t) in the transposed tile
    __device__ static constexpr int at_t(int c, int t) {
        return c * C + ((((t >> 2) ^ (c >> 2)) & 3) << 2) + (t & 3);
    }
};

// 16x16 product N.M, given N^T and M in D layout, split-bf16 on both sides
// (error ~ |N||M| 2^-16). Result in D layout.
__device__ __forceinline__ f32x4 mm16(f32x4 Nt, f32x4 M) {
    bf16x4 nh, nl, mh, ml;
    split4(Nt, nh, nl);
    split4(M, mh, ml);
    const bf16x4 z = {};
    const bf16x8 b = cat(mh, ml);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma(cat(nh, nh), b, acc);
    acc = mfma(cat(nl, z), b, acc);
    return acc;
}

// Orders one wave's LDS writes before its later LDS reads of other lanes' data.
// A wave's LDS operations execute in issue order, so this only has to stop the
// compiler from moving memory operations across it; it is not a workgroup
// barrier (other waves may be anywhere).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Identity plus/minus a D-layout matrix.
__device__ __forceinline__ f32x4 eye_plus(f32x4 M, int lane, float sign) {
    const int col = lane & 15, r0 = 4 * (lane >> 4);
    f32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = sign * M[j] + ((r0 + j) == col ? 1.f : 0.f);
    return o;
}

// ---------------------------------------------------------------- chunk prep
// One wave turns one (chunk, head) of raw inputs into a chunk record.
//   q, k: bf16 bits [T, H, 128]; g: fp32 [T, H, 128]; beta: fp32 [T, H]
//   t0: first token of the chunk; nc: its length (1..16); rows past nc are
//   treated as k = q = 0, g = 0, beta = 0, which adds nothing.
// `rec` may point to global memory or LDS.
__device__ __forceinline__ void prep_chunk(const uint16_t *__restrict__ q,
                                           const uint16_t *__restrict__ k,
                                           const float *__restrict__ g,
                                           const float *__restrict__ beta, int64_t t0, int nc,
                                           int h, int H, float scale, PrepLds &L, char *rec) {
    const int l = threadIdx.x & 63;
    const int c0 = 2 * l;            // this lane's two key channels (channel-major phase)
    const int r = l & 15, gq = l >> 4;

    // ---- phase 0: gates and scaled operands, lane = channel pair, loop over tokens
    // G is kept in base-2 units (log2 e folded into the running sum)
    float G0[C], G1[C];
    uint32_t qv[C], kv[C];
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int t = 0; t < C; ++t) {
        f32x2 gt = {0.f, 0.f};
        uint32_t qq = 0, kk = 0;
        if (t < nc) {
            const int64_t row = (t0 + t) * (int64_t)H + h;
            gt = *(const f32x2 *)(g + row * D + c0);
            qq = *(const uint32_t *)(q + row * D + c0);
            kk = *(const uint32_t *)(k + row * D + c0);
        }
        acc0 = __builtin_fmaf(fmaxf(gt.x, LOWER_BOUND), LOG2E, acc0);
        acc1 = __builtin_fmaf(fmaxf(gt.y, LOWER_BOUND), LOG2E, acc1);
        G0[t] = acc0;
        G1[t] = acc1;
        qv[t] = qq;
        kv[t] = kk;
    }
    // padded rows carry g = 0, so acc is G at the last real token
    const float eC0 = __builtin_amdgcn_exp2f(acc0), eC1 = __builtin_amdgcn_exp2f(acc1);
    *(f32x2 *)(rec + Rec::EG + c0 * 4) = f32x2{eC0, eC1};
    *(f32x2 *)(rec + Rec::EGP + egp_index(c0) * 4) = f32x2{eC0, eC1};   // c0 even: one pair

    // per-channel token rows of K+ and K~ (hi, lo), packed two tokens per dword,
    // written to the transposed tiles with wide stores after the loop
    uint32_t kpT[2][8], khT[2][8], klT[2][8];
#pragma unroll
    for (int t = 0; t < C; t += 2) {
        float kpv[2][2], ktv[2][2];   // [token of pair][channel]
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tt = t + u;
            const float ep0 = __builtin_amdgcn_exp2f(G0[tt]), ep1 = __builtin_amdgcn_exp2f(G1[tt]);
            const float en0 = __builtin_amdgcn_exp2f(-G0[tt]), en1 = __builtin_amdgcn_exp2f(-G1[tt]);
            const float k0 = bf_lo(kv[tt]), k1 = bf_hi(kv[tt]);
            const float q0 = bf_lo(qv[tt]), q1 = bf_hi(qv[tt]);
            const f32x2 kp = {k0 * ep0, k1 * ep1};
            const f32x2 km = {k0 * en0, k1 * en1};
            const f32x2 qp = {scale * q0 * ep0, scale * q1 * ep1};
            const int rc = PrepLds::at(tt, c0);
            *(uint32_t *)&L.kp[rc] = pack2(kp.x, kp.y);
            bf16x2 hi, lo;
            split2(km, hi, lo);
            *(bf16x2 *)&L.kmh[rc] = hi;
            *(bf16x2 *)&L.kml[rc] = lo;
            split2(qp, hi, lo);
            *(bf16x2 *)&L.qph[rc] = hi;
            *(bf16x2 *)&L.qpl[rc] = lo;
            kpv[u][0] = kp.x;
            kpv[u][1] = kp.y;
            ktv[u][0] = km.x * eC0;      // K~ = K e^{G_C - G}
            ktv[u][1] = km.y * eC1;
        }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            kpT[ch][t / 2] = pack2(kpv[0][ch], kpv[1][ch]);
            bf16x2 hi, lo;
            split2(f32x2{ktv[0][ch], ktv[1][ch]}, hi, lo);
            khT[ch][t / 2] = __builtin_bit_cast(uint32_t, hi);
            klT[ch][t / 2] = __builtin_bit_cast(uint32_t, lo);
        }
    }
    // K+ transposed into LDS (the A operand of W^T); K~ (hi | lo) straight into the
    // record: channel c, tokens 4e..4e+3 is recurrence lane 16e + c % 16 of key block c / 16
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const int c = c0 + ch;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *(uint2 *)&L.kpt[PrepLds::at_t(c, 4 * e)] = uint2{kpT[ch][2 * e], kpT[ch][2 * e + 1]};
            *(uint4 *)(rec + Rec::KT + (c >> 4) * 1024 + (16 * e + (c & 15)) * 16) =
                uint4{khT[ch][2 * e], khT[ch][2 * e + 1], klT[ch][2 * e], klT[ch][2 * e + 1]};
        }
    }
    // beta of token r (this lane's column) and of tokens 4g+j (this lane's rows)
    float br = 0.f;
    f32x4 bj = {0.f, 0.f, 0.f, 0.f};
    if (r < nc) br = beta[(t0 + r) * (int64_t)H + h];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (4 * gq + j < nc) bj[j] = beta[(t0 + 4 * gq + j) * (int64_t)H + h];
    wave_sync();

    // ---- phase 1: K+K-^T (both orientations) and the causal Q+K-^T, 128-deep
    f32x4 akk = {0.f, 0.f, 0.f, 0.f}, akt = akk, pt = akk;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int off = PrepLds::at(r, 32 * kb + 8 * gq);
        const bf16x8 kp = *(const bf16x8 *)&L.kp[off];
        const bf16x8 kmh = *(const bf16x8 *)&L.kmh[off];
        const bf16x8 kml = *(const bf16x8 *)&L.kml[off];
        const bf16x8 qph = *(const bf16x8 *)&L.qph[off];
        const bf16x8 qpl = *(const bf16x8 *)&L.qpl[off];
        akk = mfma(kp, kmh, akk);   // (K+K-^T)[4g+j][r]
        akt = mfma(kmh, kp, akt);   // (K+K-^T)[r][4g+j]
        pt = mfma(kmh, qph, pt);    // (Q+K-^T)[r][4g+j], split 3-term
        pt = mfma(kmh, qpl, pt);
        pt = mfma(kml, qph, pt);
    }
    f32x4 Am, At, Pm;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 4 * gq + j;
        Am[j] = (r < row) ? bj[j] * akk[j] : 0.f;   // A[row][r]
        At[j] = (row < r) ? br * akt[j] : 0.f;       // A^T[row][r] = A[r][row]
        Pm[j] = (row <= r) ? pt[j] : 0.f;            // P[r][row]
    }
    {
        bf16x4 ph, pl;
        split4(Pm, ph, pl);
        *(bf16x8 *)(rec + Rec::PP + l * 16) = cat(ph, pl);
    }

    // ---- phase 2: T^T = (I + A^T)^{-1} = (I - X)(I + X^2)(I + X^4)(I + X^8), X = A^T
    const f32x4 X2 = mm16(Am, At);
    const f32x4 A2 = mm16(At, Am);
    const f32x4 X4 = mm16(A2, X2);
    const f32x4 A4 = mm16(X2, A2);
    const f32x4 X8 = mm16(A4, X4);
    const f32x4 R1 = mm16(eye_plus(A4, l, 1.f), eye_plus(X8, l, 1.f));
    const f32x4 R2 = mm16(eye_plus(A2, l, 1.f), R1);
    const f32x4 Tt = mm16(eye_plus(Am, l, -1.f), R2);   // Tt[j] = T[r][4g+j]
    bf16x8 tb;
    {
        bf16x4 hi, lo;
        split4(Tt * bj, hi, lo);                       // (T Diag(beta))[r][4g+j]
        tb = cat(hi, lo);
        *(bf16x8 *)(rec + Rec::TB + l * 16) = tb;
    }

    // ---- phase 3: W^T = K+^T (T Diag(beta))^T, one 16-row key block at a time
    f32x4 Wt[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bf16x4 a = *(const bf16x4 *)&L.kpt[PrepLds::at_t(16 * b + r, 4 * gq)];
        Wt[b] = mfma(cat(a, a), tb, f32x4{0.f, 0.f, 0.f, 0.f});   // W[r][16b+4g+j]
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const bf16x4 a = to_bf16x4(-Wt[2 * kb]);
        const bf16x4 b = to_bf16x4(-Wt[2 * kb + 1]);
        const bf16x8 wn = cat(a, b);
        *(bf16x8 *)(rec + Rec::WN + kb * 1024 + l * 16) = wn;
        const int o0 = PrepLds::at(r, 32 * kb + 4 * gq), o1 = PrepLds::at(r, 32 * kb + 16 + 4 * gq);
        const bf16x8 qh = cat(*(const bf16x4 *)&L.qph[o0], *(const bf16x4 *)&L.qph[o1]);
        const bf16x8 ql = cat(*(const bf16x4 *)&L.qpl[o0], *(const bf16x4 *)&L.qpl[o1]);
        *(bf16x8 *)(rec + Rec::QH + kb * 1024 + l * 16) = qh;
        *(bf16x8 *)(rec + Rec::QL + kb * 1024 + l * 16) = ql;
    }
}

// ---------------------------------------------------------------- recurrence
// Inputs of one chunk step for one wave (a 16-column slice of the state).
struct StepIn {
    bf16x8 wn[4], qh[4], ql[4];
    bf16x8 kt[8];     // K~ hi | lo, per key block
    bf16x8 pp;        // P hi | lo
    bf16x8 tb;
    f32x4 eg[8];
    bf16x4 v;     // V[4g+j][col], zero past the chunk end
};

// Read one wave's step inputs from a chunk record (LDS or global).
__device__ __forceinline__ void read_rec(StepIn &s, const char *rec) {
    const int l = threadIdx.x & 63, gq = l >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        s.wn[kb] = *(const bf16x8 *)(rec + Rec::WN + kb * 1024 + l * 16);
        s.qh[kb] = *(const bf16x8 *)(rec + Rec::QH + kb * 1024 + l * 16);
        s.ql[kb] = *(const bf16x8 *)(rec + Rec::QL + kb * 1024 + l * 16);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        s.kt[b] = *(const bf16x8 *)(rec + Rec::KT + b * 1024 + l * 16);
        s.eg[b] = *(const f32x4 *)(rec + Rec::EG + (16 * b + 4 * gq) * 4);
    }
    s.pp = *(const bf16x8 *)(rec + Rec::PP + l * 16);
    s.tb = *(const bf16x8 *)(rec + Rec::TB + l * 16);
}

// ... and this lane's V values from a tile laid out [16 tokens][vcols] bf16, the
// wave's columns starting at vcol0.
__device__ __forceinline__ void read_vtile(StepIn &s, const uint16_t *vtile, int vcols, int vcol0) {
    const int l = threadIdx.x & 63, gq = l >> 4, c = l & 15;
    uint16_t vv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = vtile[(4 * gq + j) * vcols + vcol0 + c];
    s.v = __builtin_bit_cast(bf16x4, (ushort4{vv[0], vv[1], vv[2], vv[3]}));
}

// One chunk of the recurrence on a 16-column state slice S (D layout, 8 key
// blocks). Returns the chunk's outputs O[4g+j][col] (scale already folded in).
__device__ __forceinline__ f32x4 recur_step(const StepIn &s, f32x4 (&S)[8]) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bf16x4 z4 = {};
    // state as B operand, permuted key labelling: hi part first (it gates W.S)
    bf16x8 sh[4], sl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        sh[kb] = cat(to_bf16x4(S[2 * kb]), to_bf16x4(S[2 * kb + 1]));
    // U = (T Diag(beta)) V, then Vn = U - W S  (two accumulators to shorten the chain)
    f32x4 va = mfma(s.tb, cat(s.v, s.v), zero);
    f32x4 vb = zero;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        if (kb & 1) vb = mfma(s.wn[kb], sh[kb], vb);
        else va = mfma(s.wn[kb], sh[kb], va);
    }
    if (KDA_SPLIT_S_WS || KDA_SPLIT_S_QS) {
        // lo part: x - float(hi), rounded
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const f32x4 a = S[2 * kb], b = S[2 * kb + 1];
            const uint2 h0 = __builtin_bit_cast(uint2, __builtin_shufflevector(sh[kb], sh[kb], 0, 1, 2, 3));
            const uint2 h1 = __builtin_bit_cast(uint2, __builtin_shufflevector(sh[kb], sh[kb], 4, 5, 6, 7));
            const uint32_t l0 = pack2(a[0] - __uint_as_float(h0.x << 16), a[1] - __uint_as_float(h0.x & 0xffff0000u));
            const uint32_t l1 = pack2(a[2] - __uint_as_float(h0.y << 16), a[3] - __uint_as_float(h0.y & 0xffff0000u));
            const uint32_t l2 = pack2(b[0] - __uint_as_float(h1.x << 16), b[1] - __uint_as_float(h1.x & 0xffff0000u));
            const uint32_t l3 = pack2(b[2] - __uint_as_float(h1.y << 16), b[3] - __uint_as_float(h1.y & 0xffff0000u));
            sl[kb] = __builtin_bit_cast(bf16x8, (uint4{l0, l1, l2, l3}));
        }
    }
    if (KDA_SPLIT_S_WS) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb & 1) vb = mfma(s.wn[kb], sl[kb], vb);
            else va = mfma(s.wn[kb], sl[kb], va);
        }
    }
    const f32x4 vn = va + vb;
    // O = Q+ S (Q+ split hi/lo; two accumulators keep the dependent chains short) ...
    f32x4 oa = zero, ob = zero;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        oa = mfma(s.qh[kb], sh[kb], oa);
        if (KDA_SPLIT_S_QS) ob = mfma(s.qh[kb], sl[kb], ob);
        oa = mfma(s.ql[kb], sh[kb], oa);
    }
    // ... + P Vn  (three-term split through the shared B operands)
    bf16x4 vh, vl;
    split4(vn, vh, vl);
    const bf16x8 vhh = cat(vh, vh), vl0 = cat(vl, z4);
    ob = mfma(s.pp, vhh, ob);
    ob = mfma(s.pp, vl0, ob);
    const f32x4 o = oa + ob;
    // S <- Diag(e^{G_C}) S + K~^T Vn
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        S[b] = mfma(s.kt[b], vhh, S[b] * s.eg[b]);
        S[b] = mfma(s.kt[b], vl0, S[b]);
    }
    return o;
}


// ---------------------------------------------------------------- shared by the recurrences
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]; others left open
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// vmcnt(N) and lgkmcnt(0) together: own global loads up to the N youngest, and
// every own LDS access, complete
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

#define KDA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Wave roles of the paired recurrence blocks (NW 16-column slices per block): per slice a
// chain wave and two output waves, one loader wave. Waves w and w+4 of a block share a
// SIMD (and its matrix unit), so the roles are placed to keep each chain wave's SIMD free
// of output work:
//   NW = 1: chain 0 | output p0 | output p1 | loader
//   NW = 2: chain 0, chain 1 | output (slice 0, p0), (slice 1, p0) | loader | idle |
//           output (slice 0, p1), (slice 1, p1)
// (the idle wave only keeps the barrier count, so that SIMD 1 hosts chain 1 alone).
//   NW = 4: chain 0..3 | loader (states only, no output waves: the recurrence over
//           parts' first pass)
template <int NW>
struct PairLayout {
    static_assert(NW == 1 || NW == 2 || NW == 4, "one, two or four slices per block");
    static constexpr int SNAP = 64 * 32 * 4 + 64 * 16;   // state fp32 [64 lanes][32] + V_new hi|lo
    static constexpr int SNAPS = 3;                      // snapshot buffers per slice
    static constexpr int WAVES = NW == 1 ? 4 : NW == 2 ? 8 : 5;
    static constexpr int LOADER = NW == 1 ? 3 : 4;
    static constexpr int IDLE = NW == 2 ? 5 : -1;
    // output wave of slice s, parity p (none with four slices)
    __device__ static constexpr int out_wave(int s, int p) {
        return NW == 1 ? 1 + p : NW == 2 ? (p ? 6 : 2) + s : -1;
    }
};

// Global index of the idx-th chunk-head (heads fastest, sequences in input order) of the
// segment [fb, fe), or -1 past its end. The whole range is the global chunk order itself;
// for a part of it the sequences are walked in turn (segmented launches serve few).
__device__ __forceinline__ int seg_chunk_of(const int32_t *__restrict__ chunk_off, int N, int H,
                                            int fb, int fe, int64_t idx, int &h) {
    h = (int)(idx % H);
    int64_t c = idx / H;
    if (fb == 0 && fe == SEG_ONE) return c < chunk_off[N] ? (int)c : -1;
    for (int n = 0; n < N; ++n) {
        const int len = chunk_off[n + 1] - chunk_off[n];
        const int b = seg_chunk(len, fb), e = seg_chunk(len, fe);
        if (c < e - b) return chunk_off[n] + b + (int)c;
        c -= e - b;
    }
    return -1;
}

}  // namespace kda
