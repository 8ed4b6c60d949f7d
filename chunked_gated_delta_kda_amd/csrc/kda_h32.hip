// kda_h32.hip -- the KDA forward over 32-token chunks with fp16 recurrence operands.
//
// A 32-token chunk is prepared as two 16-token halves a, b (each with the 16-token
// chunked form of kda_device.hpp: gates, K+K-^T, Neumann inverse, W) and combined into
// one 32-row WY form, so that one serial step of the recurrence covers 32 tokens:
//
//   V_new = U - W S,                 U = (T Diag(beta)) V           (32 x dv)
//   O     = Q+ S + P V_new                                          (32 x dv)
//   S    <- Diag(e^{G_C}) S + K~^T V_new                            (dk x dv)
//
// With D_a = Diag(e^{G_a}) the first half's total decay and every subscripted quantity
// the 16-token one of its half (gates cumulated from the start of that half), T of the
// whole chunk is block lower triangular, which gives
//
//   W rows a = W_a,  W rows b = W_b D_a - M W_a,        M = (W_b D_a) K-_a^T = W_b K~_a^T
//   T Diag(beta) = [[TB_a, 0], [-M TB_a, TB_b]]
//   P = [[P_aa, 0], [P_ba, P_bb]],                      P_ba = (Q+_b D_a) K-_a^T
//   K~ rows a = K~_a e^{G_b},  Q+ rows b = Q+_b D_a,    e^{G_C} = e^{G_a + G_b}
//
// (this library's derivation from the per-token recurrence; every exponential stays
// within the range of a 16-token chunk, so no anchor is needed). Every factor of the
// serial chain (W, T Diag(beta), K~, the state as an operand, V_new) is bounded by the
// key norms or the state, so it is rounded once to fp16 (11 significant bits) and
// multiplied on v_mfma_f32_16x16x32_f16, where the 16-token path needed two bf16
// pieces (hi + lo) and a second product for the same accuracy. The 32 tokens of a chunk
// fill the 32-deep contraction of K~^T V_new and of P V_new exactly: the state update is
// 8 products per 32 tokens instead of 32. The output's Q+ S, off the chain, keeps split
// bf16 on both sides (three products): where the output is a decaying read-out of the
// state (beta ~ 0), a few early tokens carry most of |o| and single fp16 rounding of Q+
// and S there would reach the max-abs gate, which is relative to the RMS of all of o.
//
// fp16 holds magnitudes below 65504: the recurrence's operands are the state, V_new
// (of the size of v) and quantities bounded by |k| and |q|, which the L2-normalised
// keys and queries of KDA keep far inside that range.
//
// 32-deep token slots. The MFMA A operand lane l holds row l%16 and k-slots 8(l/16)+i;
// here slot 8g+i (g = l/16) carries token tau(8g+i) = 4g+i (i < 4, half a) or
// 16+4g+i-4 (i >= 4, half b), so that V_new, produced as two 16x16 D-layout blocks
// (lane: rows 4g..4g+3 of each half), is the B operand of K~^T V_new and P V_new as it
// stands in registers.
#include <type_traits>

#include "kda.h"
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int CH = 32;   // chunk length of this path

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 to_f16x4(f32x4 x) { return __builtin_convertvector(x, f16x4); }
__device__ __forceinline__ f16x8 cat16(f16x4 a, f16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Write-only sink for output rows past a partial chunk's end (see the output waves).
__device__ float h32_sink[64];

// ---------------------------------------------------------------- chunk record
// One (32-token chunk, head), fp16 MFMA operands in per-lane order (16 bytes per lane per
// 1 KiB piece). The chain's pieces come first, one contiguous run of whole wave loads.
struct RecH {
    static constexpr int WN = 0;         // f16 [2 row blocks][4 kb][64][8]: -W, state-permuted A operand
    static constexpr int KT = 8192;      // f16 [8 key blocks][64][8]: K~^T, token slots tau
    static constexpr int TB = 16384;     // f16 [2][64][8]: T Diag(beta), token slots tau
    static constexpr int EGP = 18432;    // f32 [128]: e^{G_C}, lane-permuted (egp_index); 512 B unused after
    static constexpr int CHAIN = 19456;
    static constexpr int QH = 19456;     // bf16 [2][4][64][8]: Q+ hi (scale folded in), state-permuted A operand
    static constexpr int QL = 27648;     // bf16 [2][4][64][8]: Q+ lo
    static constexpr int PP = 35840;     // f16 [2][64][8]: P = incl_lower(Q+ K-^T), token slots tau
    static constexpr int BYTES = 37888;
};
static_assert(RecH::CHAIN % 1024 == 0 && RecH::BYTES % 1024 == 0, "record pieces in whole wave loads");
static_assert(RecH::BYTES == RECH_BYTES, "record size mismatch");

// ---------------------------------------------------------------- prep
// LDS of one prep wave: the 16-token tiles of kda_device.hpp plus a 16x16 fp32 transpose.
struct PrepHLds {
    PrepLds t;
    float tr[16][17];
};

// Transpose of a D-layout 16x16 matrix (lane (g, c) holds X[4g+j][c]): returns the
// lane's values of X^T in D layout, i.e. X[c][4g+j].
__device__ __forceinline__ f32x4 transpose16(f32x4 x, float (*tr)[17]) {
    const int l = threadIdx.x & 63, c = l & 15, g = l >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) tr[4 * g + j][c] = x[j];
    wave_sync();
    f32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = tr[c][4 * g + j];
    wave_sync();
    return y;
}

// Raw inputs of one 16-token half on this lane's channel pair: g, and q, k (bf16 pairs).
// Loaded unconditionally (rows past the half's nc tokens reread row `fb`, a real token)
// so that both halves' loads are issued together at the start of a chunk and one
// memory latency is exposed instead of one per half; prep_half masks rows past nc.
// GT: the element type of g, float or uint16_t (bf16 bits; the input-byte diet form:
// half the bytes of the largest input).
template <typename GT>
struct HalfIn {
    using GV = typename std::conditional<sizeof(GT) == 4, f32x2, uint32_t>::type;
    GV g[C];
    uint32_t q[C], k[C];
    __device__ f32x2 gval(int t) const {
        if constexpr (sizeof(GT) == 4) return g[t];
        else return f32x2{bf_lo(g[t]), bf_hi(g[t])};
    }
};
template <typename GT>
__device__ __forceinline__ void load_half(HalfIn<GT> &x, const uint16_t *__restrict__ q,
                                          const uint16_t *__restrict__ k, const GT *__restrict__ g, int64_t t0,
                                          int nc, int64_t fb, int h, int H, int c0) {
#pragma unroll
    for (int t = 0; t < C; ++t) {
        const int64_t row = ((t < nc ? t0 + t : fb) * (int64_t)H + h) * D + c0;
        x.g[t] = *(const typename HalfIn<GT>::GV *)(g + row);
        x.q[t] = *(const uint32_t *)(q + row);
        x.k[t] = *(const uint32_t *)(k + row);
    }
}

// One 16-token half of a 32-token chunk (HALF 0 = a, 1 = b), one wave. Rows past nc
// carry k = q = 0, g = 0, beta = 0, which adds nothing. Writes the half's K~ token slots
// (fp16) into the record's KT piece and its Q+ rows into QP; HALF 0 also writes its rows
// of -W. Returns, per lane, with "R layout" meaning lane (g, c) holds X[c][4g+j]:
//   Wt[b]  R layout of W[:, key block b] (HALF 1: scaled by D_a, i.e. W_b D_a)
//   Wd[b]  (HALF 0) D layout of W[:, key block b]
//   tbr    R layout of T Diag(beta);  pr  R layout of P (causal, diagonal kept)
//   ec     e^{G_C} of this half on the lane's channel pair
//   qh, ql hi and lo bf16 A operands of this half's Q+ rows (state permutation; HALF 1:
//          Q+_b D_a), also written to the record
// kts (HALF 0): K~ is further scaled per channel by e^{G_b}; ega (HALF 1): lane-permuted
// e^{G_a}.
template <int HALF, typename GT>
__device__ __forceinline__ void prep_half(const HalfIn<GT> &in, const float *__restrict__ beta,
                                          int64_t t0, int nc, int h, int H, float scale, PrepLds &L,
                                          char *rec, f32x2 kts, f32x2 ega, f32x4 (&Wt)[8], f32x4 (&Wd)[8],
                                          f32x4 &tbr, f32x4 &pr, f32x2 &ec, bf16x8 (&qh)[4], bf16x8 (&ql)[4],
                                          uint32_t (&kta)[2][8]) {
    const int l = threadIdx.x & 63;
    const int c0 = 2 * l;
    const int r = l & 15, gq = l >> 4;

    // ---- gates and scaled operands, lane = channel pair, loop over tokens (base-2 sums)
    float G0[C], G1[C];
    uint32_t qv[C], kv[C];
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int t = 0; t < C; ++t) {
        const bool in_range = t < nc;
        const f32x2 gt = in_range ? in.gval(t) : f32x2{0.f, 0.f};
        const uint32_t qq = in_range ? in.q[t] : 0u, kk = in_range ? in.k[t] : 0u;
        acc0 = __builtin_fmaf(fmaxf(gt.x, LOWER_BOUND), LOG2E, acc0);
        acc1 = __builtin_fmaf(fmaxf(gt.y, LOWER_BOUND), LOG2E, acc1);
        G0[t] = acc0;
        G1[t] = acc1;
        qv[t] = qq;
        kv[t] = kk;
    }
    const float eC0 = __builtin_amdgcn_exp2f(acc0), eC1 = __builtin_amdgcn_exp2f(acc1);
    ec = f32x2{eC0, eC1};
    const float kt0 = HALF == 0 ? eC0 * kts.x : eC0, kt1 = HALF == 0 ? eC1 * kts.y : eC1;

    uint32_t kpT[2][8], ktT[2][8];   // per channel, two tokens per dword: K+ (bf16), K~ (fp16)
#pragma unroll
    for (int t = 0; t < C; t += 2) {
        float kpv[2][2], ktv[2][2];
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
            ktv[u][0] = km.x * kt0;      // K~ = K e^{G_C - G} (times e^{G_b} for half a)
            ktv[u][1] = km.y * kt1;
        }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            kpT[ch][t / 2] = pack2(kpv[0][ch], kpv[1][ch]);
            ktT[ch][t / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{ktv[0][ch], ktv[1][ch]}), f16x2));
        }
    }
    // K+ transposed into LDS (operand of W); K~ into the record: channel c, half-local
    // tokens 4e..4e+3 are token slots 8e + 4 HALF .. + 3 of lane 16e + c % 16 of key block
    // c / 16. Half a's K~ waits in kta for half b's, so that each 16-byte slot is stored
    // whole (two 8-byte halves stored apart leave lines partly written in between).
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const int c = c0 + ch;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *(uint2 *)&L.kpt[PrepLds::at_t(c, 4 * e)] = uint2{kpT[ch][2 * e], kpT[ch][2 * e + 1]};
            if (HALF == 0) {
                kta[ch][2 * e] = ktT[ch][2 * e];
                kta[ch][2 * e + 1] = ktT[ch][2 * e + 1];
            } else {
                *(uint4 *)(rec + RecH::KT + (c >> 4) * 1024 + (16 * e + (c & 15)) * 16) =
                    uint4{kta[ch][2 * e], kta[ch][2 * e + 1], ktT[ch][2 * e], ktT[ch][2 * e + 1]};
            }
        }
    }
    float br = 0.f;
    f32x4 bj = {0.f, 0.f, 0.f, 0.f};
    if (r < nc) br = beta[(t0 + r) * (int64_t)H + h];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (4 * gq + j < nc) bj[j] = beta[(t0 + 4 * gq + j) * (int64_t)H + h];
    wave_sync();

    // ---- K+K-^T (both orientations) and the causal Q+K-^T, 128-deep
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
    f32x4 Am, At;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 4 * gq + j;
        Am[j] = (r < row) ? bj[j] * akk[j] : 0.f;   // A[row][r]
        At[j] = (row < r) ? br * akt[j] : 0.f;       // A^T[row][r] = A[r][row]
        pr[j] = (row <= r) ? pt[j] : 0.f;            // P[r][row]
    }

    // ---- T^T = (I + A^T)^{-1} = (I - X)(I + X^2)(I + X^4)(I + X^8), X = A^T
    const f32x4 X2 = mm16(Am, At);
    const f32x4 A2 = mm16(At, Am);
    const f32x4 X4 = mm16(A2, X2);
    const f32x4 A4 = mm16(X2, A2);
    const f32x4 X8 = mm16(A4, X4);
    const f32x4 R1 = mm16(eye_plus(A4, l, 1.f), eye_plus(X8, l, 1.f));
    const f32x4 R2 = mm16(eye_plus(A2, l, 1.f), R1);
    const f32x4 Tt = mm16(eye_plus(Am, l, -1.f), R2);   // Tt[j] = T[r][4g+j]
    tbr = Tt * bj;                                      // (T Diag(beta))[r][4g+j]
    bf16x8 tb;
    {
        bf16x4 hi, lo;
        split4(tbr, hi, lo);
        tb = cat(hi, lo);
    }

    // ---- W = T Diag(beta) K+, one 16-column key block at a time, in both layouts
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bf16x4 a = *(const bf16x4 *)&L.kpt[PrepLds::at_t(16 * b + r, 4 * gq)];
        Wt[b] = mfma(cat(a, a), tb, f32x4{0.f, 0.f, 0.f, 0.f});   // W[r][16b+4g+j]
        if (HALF == 1) Wt[b] = decay_any(b, Wt[b], ega);
        if (HALF == 0) Wd[b] = mfma(tb, cat(a, a), f32x4{0.f, 0.f, 0.f, 0.f});   // W[4g+j][16b+r]
    }
    // ---- Q+ rows of this half (fp16, scaled to the chunk start) and, for half a, -W rows
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int o0 = PrepLds::at(r, 32 * kb + 4 * gq), o1 = PrepLds::at(r, 32 * kb + 16 + 4 * gq);
        const bf16x4 h0 = *(const bf16x4 *)&L.qph[o0], h1 = *(const bf16x4 *)&L.qph[o1];
        const bf16x4 l0 = *(const bf16x4 *)&L.qpl[o0], l1 = *(const bf16x4 *)&L.qpl[o1];
        if (HALF == 1) {
            f32x4 x0, x1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x0[j] = (float)h0[j] + (float)l0[j];
                x1[j] = (float)h1[j] + (float)l1[j];
            }
            x0 = decay_any(2 * kb, x0, ega);
            x1 = decay_any(2 * kb + 1, x1, ega);
            bf16x4 a0, b0, a1, b1;
            split4(x0, a0, b0);
            split4(x1, a1, b1);
            qh[kb] = cat(a0, a1);
            ql[kb] = cat(b0, b1);
        } else {
            qh[kb] = cat(h0, h1);
            ql[kb] = cat(l0, l1);
        }
        *(bf16x8 *)(rec + RecH::QH + (HALF * 4 + kb) * 1024 + l * 16) = qh[kb];
        *(bf16x8 *)(rec + RecH::QL + (HALF * 4 + kb) * 1024 + l * 16) = ql[kb];
        if (HALF == 0)
            *(f16x8 *)(rec + RecH::WN + kb * 1024 + l * 16) = cat16(to_f16x4(-Wt[2 * kb]), to_f16x4(-Wt[2 * kb + 1]));
    }
}

// One wave turns one (32-token chunk, head) into a chunk record. t0: first token; nc:
// its length (1..32).
template <typename GT>
__device__ __forceinline__ void prep_h32(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                         const GT *__restrict__ g, const float *__restrict__ beta, int64_t t0,
                                         int nc, int h, int H, float scale, PrepHLds &LL, char *rec) {
    PrepLds &L = LL.t;
    const int l = threadIdx.x & 63, c0 = 2 * l, r = l & 15, gq = l >> 4;
    const int nca = nc < C ? nc : C, ncb = nc > C ? nc - C : 0;
    // every input load of the chunk issued at once
    HalfIn<GT> ia, ib;
    load_half(ia, q, k, g, t0, nca, t0, h, H, c0);
    load_half(ib, q, k, g, t0 + C, ncb, t0, h, H, c0);
    // gate total of the second half on this lane's channel pair (base 2)
    float gb0 = 0.f, gb1 = 0.f;
#pragma unroll
    for (int t = 0; t < C; ++t) {
        const f32x2 gt = ib.gval(t);
        gb0 = __builtin_fmaf(t < ncb ? fmaxf(gt.x, LOWER_BOUND) : 0.f, LOG2E, gb0);
        gb1 = __builtin_fmaf(t < ncb ? fmaxf(gt.y, LOWER_BOUND) : 0.f, LOG2E, gb1);
    }
    const f32x2 eb = {__builtin_amdgcn_exp2f(gb0), __builtin_amdgcn_exp2f(gb1)};

    // ---- half a
    f32x4 Wt[8], Wd[8], tba, pa, tbb, pb;
    f32x2 ea, ebx;
    bf16x8 qh[4], ql[4];
    uint32_t kta[2][8];
    prep_half<0>(ia, beta, t0, nca, h, H, scale, L, rec, eb, f32x2{1.f, 1.f}, Wt, Wd, tba, pa, ea, qh, ql, kta);
    *(f32x2 *)(rec + RecH::EGP + egp_index(c0) * 4) = f32x2{ea.x * eb.x, ea.y * eb.y};
    // K-_a as an MFMA operand (row = token of a, k-slots = keys in the state permutation)
    bf16x8 kah[4], kal[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int o0 = PrepLds::at(r, 32 * kb + 4 * gq), o1 = PrepLds::at(r, 32 * kb + 16 + 4 * gq);
        kah[kb] = cat(*(const bf16x4 *)&L.kmh[o0], *(const bf16x4 *)&L.kmh[o1]);
        kal[kb] = cat(*(const bf16x4 *)&L.kml[o0], *(const bf16x4 *)&L.kml[o1]);
    }
    // e^{G_a} lane-permuted, through LDS
    *(f32x2 *)&L.egs[egp_index(c0)] = ea;
    wave_sync();
    const f32x2 ega = *(const f32x2 *)&L.egs[2 * l];
    wave_sync();

    // ---- half b (W and Q+ scaled by D_a)
    f32x4 Wb[8], unused[8];
    prep_half<1>(ib, beta, t0 + C, ncb, h, H, scale, L, rec, f32x2{1.f, 1.f}, ega, Wb, unused, tbb, pb, ebx,
                 qh, ql, kta);

    // ---- cross terms, transposed products so that the results land in R layout
    // M = (W_b D_a) K-_a^T and P_ba = (Q+_b D_a) K-_a^T, 3-term split products
    f32x4 mr = {0.f, 0.f, 0.f, 0.f}, pbr = mr;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        bf16x4 h0, l0, h1, l1;
        split4(Wb[2 * kb], h0, l0);
        split4(Wb[2 * kb + 1], h1, l1);
        const bf16x8 wh = cat(h0, h1), wl = cat(l0, l1);
        mr = mfma(kah[kb], wh, mr);
        mr = mfma(kal[kb], wh, mr);
        mr = mfma(kah[kb], wl, mr);
        pbr = mfma(kah[kb], qh[kb], pbr);
        pbr = mfma(kah[kb], ql[kb], pbr);
        pbr = mfma(kal[kb], qh[kb], pbr);
    }
    // rows b of T Diag(beta), columns a: -M TB_a;  rows b of W: W_b D_a - M W_a
    const f32x4 tbx = -mm16(transpose16(tba, LL.tr), mr);
#pragma unroll
    for (int b = 0; b < 8; ++b) Wb[b] -= mm16(Wd[b], mr);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        *(f16x8 *)(rec + RecH::WN + (4 + kb) * 1024 + l * 16) = cat16(to_f16x4(-Wb[2 * kb]), to_f16x4(-Wb[2 * kb + 1]));
    const f16x4 z = {};
    *(f16x8 *)(rec + RecH::TB + l * 16) = cat16(to_f16x4(tba), z);
    *(f16x8 *)(rec + RecH::TB + 1024 + l * 16) = cat16(to_f16x4(tbx), to_f16x4(tbb));
    *(f16x8 *)(rec + RecH::PP + l * 16) = cat16(to_f16x4(pa), z);
    *(f16x8 *)(rec + RecH::PP + 1024 + l * 16) = cat16(to_f16x4(pbr), to_f16x4(pb));
}

// Record of chunk ci (global index, 32-token chunks), head h.
template <typename GT>
__device__ __forceinline__ void prep_h32_one(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                             const GT *__restrict__ g, const float *__restrict__ beta,
                                             const int32_t *__restrict__ cu, int N, int T, int H, float scale,
                                             const int32_t *__restrict__ chunk_off, char *__restrict__ recs, int ci,
                                             int h, PrepHLds &L) {
    int lo = 0, hi = N - 1;   // sequence owning chunk ci: largest n with chunk_off[n] <= ci
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= ci) lo = mid; else hi = mid - 1;
    }
    const int n = lo;
    const int64_t bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
    const int64_t t0 = bos + (int64_t)CH * (ci - chunk_off[n]);
    const int nc = (int)min<int64_t>(CH, eos - t0);
    prep_h32(q, k, g, beta, t0, nc, h, H, scale, L, recs + ((int64_t)ci * H + h) * RecH::BYTES);
}

template <typename GT>
__global__ __launch_bounds__(64) void prep_h32_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                      const GT *__restrict__ g, const float *__restrict__ beta,
                                                      const int32_t *__restrict__ cu, int N, int T, int H, float scale,
                                                      const int32_t *__restrict__ chunk_off, char *__restrict__ recs,
                                                      int fb, int fe) {
    __shared__ PrepHLds L;
    int h;
    const int ci = seg_chunk_of(chunk_off, N, H, fb, fe, blockIdx.x, h);
    if (ci < 0) return;
    prep_h32_one(q, k, g, beta, cu, N, T, H, scale, chunk_off, recs, ci, h, L);
}

// ---------------------------------------------------------------- chunk map in the prep
// For batches of at most MAP_WAVE_MAX sequences the first prep launch forms the chunk map
// itself instead of a launch of its own before it: each wave derives it from the caller's
// offsets in registers (lane n: offset n and the chunks before sequence n), with the
// sanitising of the chunk-map kernel (every offset clamped to [0, T] and raised to the
// largest offset before it; the error bit when the offsets were not 0 = c_0 <= c_1 <= ...
// <= c_N = T), and block 0 stores it (sanitised offsets, chunk offsets, longest-first
// order, error word) for the kernels after it.
constexpr int MAP_WAVE_MAX = 63;   // N + 1 offsets in one wave's lanes
constexpr int MAP_ERR_CU_SEQLENS = KDA_DEVERR_CU_SEQLENS;

struct WaveMap {
    int32_t cs;   // lane n <= N: sanitised offset n
    int32_t co;   // lane n <= N: chunks (of CH tokens) before sequence n
    bool bad;     // the offsets were malformed (the same in every lane)
};

__device__ __forceinline__ WaveMap wave_map(const int32_t *__restrict__ cu, int N, int T) {
    const int l = threadIdx.x & 63;
    int32_t raw = 0;
    if (l <= N) raw = cu ? cu[l] : (l == 0 ? 0 : T);
    const int32_t prev = __shfl_up(raw, 1);
    const bool bad = l <= N && ((l == 0 && raw != 0) || (l > 0 && raw < prev) || (l == N && raw != T));
    int32_t x = l <= N ? min(max(raw, 0), T) : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {       // running maximum (lanes past N: the last offset)
        const int32_t y = __shfl_up(x, d);
        if (l >= d) x = max(x, y);
    }
    const int32_t nxt = __shfl_down(x, 1);
    int32_t c = l < N ? (nxt - x + CH - 1) / CH : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {       // inclusive sum of the chunk counts
        const int32_t y = __shfl_up(c, d);
        if (l >= d) c += y;
    }
    int32_t co = __shfl_up(c, 1);
    if (l == 0) co = 0;
    WaveMap m;
    m.cs = x;
    m.co = co;
    m.bad = __ballot(bad) != 0;
    return m;
}

// value of lane i (i uniform across the wave)
__device__ __forceinline__ int32_t lane_val(int32_t x, int i) {
    return __builtin_amdgcn_readlane(x, i);
}

// The map's outputs for the later kernels (one wave).
__device__ __forceinline__ void wave_map_store(const WaveMap &m, int N, int32_t *__restrict__ cu_safe,
                                               int32_t *__restrict__ chunk_off, int32_t *__restrict__ order,
                                               int32_t *__restrict__ err, int32_t *dev_err) {
    const int l = threadIdx.x & 63;
    if (l <= N) {
        cu_safe[l] = m.cs;
        chunk_off[l] = m.co;
    }
    const int32_t len = __shfl_down(m.cs, 1) - m.cs;   // lane n < N: length of sequence n
    int rank = 0;
    for (int j = 0; j < N; ++j) {
        const int32_t lj = lane_val(len, j);
        rank += (lj > len) || (lj == len && j < l);
    }
    if (l < N) order[rank] = l;
    if (l == 0) {
        *err = m.bad ? MAP_ERR_CU_SEQLENS : 0;
        if (m.bad && dev_err) atomicOr(dev_err, MAP_ERR_CU_SEQLENS);
    }
}

// The prep of the segment [0, fe) with the chunk map formed in the launch (N <= MAP_WAVE_MAX):
// cu is the caller's offsets; block 0 also stores the map.
template <typename GT>
__global__ __launch_bounds__(64) void prep_h32_map_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                          const GT *__restrict__ g, const float *__restrict__ beta,
                                                          const int32_t *__restrict__ cu, int N, int T, int H,
                                                          float scale, char *__restrict__ recs, int fe,
                                                          int32_t *__restrict__ cu_safe, int32_t *__restrict__ chunk_off,
                                                          int32_t *__restrict__ order, int32_t *__restrict__ err,
                                                          int32_t *dev_err) {
    __shared__ PrepHLds L;
    const WaveMap m = wave_map(cu, N, T);
    if (blockIdx.x == 0) wave_map_store(m, N, cu_safe, chunk_off, order, err, dev_err);
    // chunk and head of this wave (as seg_chunk_of over [0, fe))
    const int h = (int)(blockIdx.x % H);
    int c = (int)(blockIdx.x / H), ci = -1;
    if (fe == SEG_ONE) {
        ci = c < lane_val(m.co, N) ? c : -1;
    } else {
        for (int n = 0; n < N; ++n) {
            const int c0 = lane_val(m.co, n), e = seg_chunk(lane_val(m.co, n + 1) - c0, fe);
            if (c < e) {
                ci = c0 + c;
                break;
            }
            c -= e;
        }
    }
    if (ci < 0) return;
    int lo = 0, hi = N - 1;   // sequence owning chunk ci: largest n with co[n] <= ci
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (lane_val(m.co, mid) <= ci) lo = mid; else hi = mid - 1;
    }
    const int n = lo;
    const int64_t bos = lane_val(m.cs, n), eos = lane_val(m.cs, n + 1);
    const int64_t t0 = bos + (int64_t)CH * (ci - lane_val(m.co, n));
    const int nc = (int)min<int64_t>(CH, eos - t0);
    prep_h32(q, k, g, beta, t0, nc, h, H, scale, L, recs + ((int64_t)ci * H + h) * RecH::BYTES);
}

// ---------------------------------------------------------------- recurrence
// Entry and exit states: fp32, or bf16 where the caller's states are (sbf: the input-byte
// diet form, half the state bytes; rounded to nearest even on the way out). The chain
// keeps an fp32 state; only the caller's s0 and sfin are bf16, the carry between
// segments stays fp32.
__device__ __forceinline__ float state_load(const float *p, bool bf, int64_t i) {
    if (bf) return __uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
    return p[i];
}
__device__ __forceinline__ void state_store(float *p, bool bf, int64_t i, float x) {
    if (bf) {
        ((uint16_t *)p)[i] = (uint16_t)(pack2(x, 0.f) & 0xffffu);
        return;
    }
    p[i] = x;
}
// The chain wave's 32 state elements (rows 16 b + 4 gq + j of one column, at p + base):
// the element type is chosen once for all of them, so that the loads issue back to back
// (a choice per element puts each load in a branch of its own, and the compiler then
// waits for every load before the next one issues).
__device__ __forceinline__ void state_tile_load(f32x4 (&S)[8], const float *p, bool bf, int64_t base, int gq) {
    if (bf) {
        const uint16_t *q = (const uint16_t *)p + base;
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[b][j] = __uint_as_float((uint32_t)q[(int64_t)(16 * b + 4 * gq + j) * D] << 16);
    } else {
        const float *q = p + base;
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[b][j] = q[(int64_t)(16 * b + 4 * gq + j) * D];
    }
}
__device__ __forceinline__ void state_tile_store(float *p, bool bf, int64_t base, int gq, const f32x4 (&S)[8]) {
    if (bf) {
        uint16_t *q = (uint16_t *)p + base;
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                q[(int64_t)(16 * b + 4 * gq + j) * D] = (uint16_t)(pack2(S[b][j], 0.f) & 0xffffu);
    } else {
        float *q = p + base;
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) q[(int64_t)(16 * b + 4 * gq + j) * D] = S[b][j];
    }
}

// The paired recurrence over 32-token records: NW 16-column slices per block, per slice a
// chain wave and two output waves (roles and SIMD placement as PairLayout), one loader
// wave. The chain wave runs V_new = U - W S and S <- D S + K~^T V_new and publishes, per
// chunk, the state it started from (fp32) and V_new; output wave parity p forms
// O = Q+ S + P V_new of chunks m = p mod 2 over the two barriers after the chunk. One
// barrier per chunk; snapshots rotate through three buffers; the loader fills an
// NSLOT-deep LDS ring with the chain's pieces and the block's V tile by direct
// global->LDS loads.
template <int NW>
struct PairH {
    static constexpr int VCOLS = 16 * NW;
    static constexpr int V_LPR = VCOLS * 2 / 16;     // lanes per V row (16 B each)
    static constexpr int V_RPL = 64 / V_LPR;         // V rows per wave load
    static constexpr int V_LOADS = CH / V_RPL;
    static constexpr int REC_LOADS = RecH::CHAIN / 1024;
    static constexpr int LOADS = REC_LOADS + V_LOADS;
    static constexpr int SV = RecH::CHAIN;           // slot: V tile [32][VCOLS] bf16 after the chain pieces
    static constexpr int SLOT = SV + V_LOADS * 1024;
    static constexpr int SNAP = 8 * 1024 + 1024;     // fp32 state (8 key blocks of 16 rows) + V_new (fp16)
    static constexpr int SNAPS = 3;
    static_assert(V_RPL * V_LOADS == CH, "V tile geometry");
};
template <int NW>
constexpr int pairh_nslot() { return NW == 1 ? 5 : 4; }
template <int NW, int NSLOT, bool OUT = true>
struct PairHLds {
    static constexpr int BYTES = NSLOT * PairH<NW>::SLOT + (OUT ? PairH<NW>::SNAPS * NW * PairH<NW>::SNAP : 0);
    static_assert(BYTES <= 160 * 1024 && BYTES > 80 * 1024, "one block per CU");
};

// A launch covers the segment [fb, fe) of every sequence (seg_chunk over 32-token chunks).
// The state enters from s0 (or zeros) at a sequence's first chunk and from `carry`
// otherwise, and leaves to sfin after its last chunk and to `carry` otherwise. Sequences
// without chunks copy s0 to sfin in the launch of the first segment. With zero_v the chain
// runs as if every v were 0 (the part of the chain linear in the entry state; outputs then
// not valid). Without OUT only the states are produced: the output waves only keep the
// barriers and the chain publishes no snapshots.
template <int NW, int NSLOT, bool OUT = true>
__device__ __forceinline__ void recur_h32_block(int bid, char *ring, const char *__restrict__ recs,
                                                const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
                                                const int32_t *__restrict__ chunk_off,
                                                const int32_t *__restrict__ order, int N, int T, int H,
                                                const float *s0, float *__restrict__ out, float *sfin, float *carry,
                                                int fb, int fe, bool sbf, bool zero_v = false) {
    using P = PairH<NW>;
    using PL = PairLayout<NW>;
    static_assert(NW <= 2 || !OUT, "the four-slice block has no output waves");
    constexpr int LOADS = P::LOADS;
    constexpr int SLOT = P::SLOT;
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
    const bool loader = w == PL::LOADER;
    const bool idle = w == PL::IDLE;
    const int parity = (w == PL::out_wave(0, 1) || w == PL::out_wave(NW - 1, 1)) ? 1 : 0;
    const int slice = chain ? w : ((loader || idle) ? 0 : (w == PL::out_wave(0, parity) ? 0 : 1));
    const int vcol0 = part * P::VCOLS;
    const int col = vcol0 + slice * 16 + c;
    const int64_t seq_bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
    const int seq_c0 = chunk_off[n], seq_c1 = chunk_off[n + 1];
    const int ci0 = seq_c0 + seg_chunk(seq_c1 - seq_c0, fb);
    const int ci1 = seq_c0 + seg_chunk(seq_c1 - seq_c0, fe);
    const int64_t sbase = ((int64_t)n * H + h) * D * D + col;
    if (ci0 >= ci1) {
        if (seq_c0 == seq_c1 && fb == 0 && chain && sfin) {
#pragma unroll
            for (int b = 0; b < 8; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t o = sbase + (int64_t)(16 * b + 4 * gq + j) * D;
                    state_store(sfin, sbf, o, s0 ? state_load(s0, sbf, o) : 0.f);
                }
        }
        return;
    }
    const int nch = ci1 - ci0;
    const int64_t bos = seq_bos + (int64_t)CH * (ci0 - seq_c0);
    const float *sin = ci0 == seq_c0 ? s0 : carry;
    float *sout = ci1 == seq_c1 ? sfin : carry;
    const bool sin_bf = sbf && ci0 == seq_c0, sout_bf = sbf && ci1 == seq_c1;
    auto snap_of = [&](int it) { return snaps + ((it % P::SNAPS) * NW + slice) * P::SNAP; };
    auto rec_of = [&](int m) { return recs + ((int64_t)(ci0 + m) * H + h) * RecH::BYTES; };
    auto sync = [] {
        __builtin_amdgcn_s_barrier();      // slots it, it+1 ready; slot it-1 released
        __builtin_amdgcn_sched_barrier(0);
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    if (loader) {
        auto fill = [&](int it) {
            const int m = it < nch ? it : nch - 1;
            const int64_t t0 = bos + (int64_t)CH * m;
            const int nc = (int)min<int64_t>(CH, eos - t0);
            char *slot = ring + (it % NSLOT) * SLOT;
            const char *rec = rec_of(m);
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                if (i < P::REC_LOADS) {
                    __builtin_amdgcn_global_load_lds((const void *)(rec + i * 1024 + l * 16),
                                                     KDA_LDS(slot + i * 1024), 16, 0, 0);
                } else {
                    const int j = i - P::REC_LOADS;
                    const int row = j * P::V_RPL + l / P::V_LPR;
                    const int cc = vcol0 + (l % P::V_LPR) * 8;
                    const int64_t t = t0 + (row < nc ? row : nc - 1);   // rows past the end: finite filler
                    __builtin_amdgcn_global_load_lds((const void *)(v + (t * H + h) * D + cc),
                                                     KDA_LDS(slot + P::SV + j * 1024), 16, 0, 0);
                }
            }
        };
#pragma unroll
        for (int it = 0; it < NSLOT - 1; ++it) fill(it);
        for (int it = 0; it < nch; ++it) {
            wait_vmcnt<(NSLOT - 3) * LOADS>();      // chunks it and it+1 have landed
            sync();
            fill(it + NSLOT - 1);
        }
        sync();
        sync();
        wait_vmcnt<0>();     // no ring write still in flight when the wave ends
        return;
    }

    if (idle || (!OUT && !chain)) {
        for (int it = 0; it < nch + 2; ++it) sync();
        return;
    }

    if (chain) {
        f32x4 S[8];
        if (sin) {
            state_tile_load(S, sin, sin_bf, sbase, gq);
        } else {
#pragma unroll
            for (int b = 0; b < 8; ++b) S[b] = zero;
        }
        // The next chunk's pieces are read one step ahead, except with two slices per block
        // the K~^T pieces (read in the step: the slot stays valid until the barrier after
        // it), which keeps the two chain waves' registers within 256 without spills.
        constexpr bool KT_AHEAD = NW == 1;
        struct ChainIn {
            f16x8 wn[8], kt[KT_AHEAD ? 8 : 1], tb[2];
            f32x2 e;              // lane-permuted decay of the whole chunk
            uint16_t vv[8];       // V[tau(8g+i)][col]
        };
        auto chain_read = [&](ChainIn &x, int it) {
            const char *slot = ring + (it % NSLOT) * SLOT;
            x.tb[0] = *(const f16x8 *)(slot + RecH::TB + l * 16);
            x.tb[1] = *(const f16x8 *)(slot + RecH::TB + 1024 + l * 16);
            const uint16_t *vt = (const uint16_t *)(slot + P::SV);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x.vv[j] = zero_v ? (uint16_t)0 : vt[(4 * gq + j) * P::VCOLS + slice * 16 + c];
                x.vv[4 + j] = zero_v ? (uint16_t)0 : vt[(C + 4 * gq + j) * P::VCOLS + slice * 16 + c];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) x.wn[i] = *(const f16x8 *)(slot + RecH::WN + i * 1024 + l * 16);
            if constexpr (KT_AHEAD) {
#pragma unroll
                for (int b = 0; b < 8; ++b) x.kt[b] = *(const f16x8 *)(slot + RecH::KT + b * 1024 + l * 16);
            }
            x.e = *(const f32x2 *)(slot + RecH::EGP + l * 8);
        };
        auto chain_step = [&](const ChainIn &x, int it) {
            char *snap = snap_of(it);
            f16x8 kt[8];
            if constexpr (!KT_AHEAD) {
                const char *slot = ring + (it % NSLOT) * SLOT;
#pragma unroll
                for (int b = 0; b < 8; ++b) kt[b] = *(const f16x8 *)(slot + RecH::KT + b * 1024 + l * 16);
            }
            f16x8 sh[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sh[kb] = cat16(to_f16x4(S[2 * kb]), to_f16x4(S[2 * kb + 1]));
            // V (bf16) as an fp16 B operand; combined here, not where it was read (the
            // compiler would otherwise wait for the read there)
            f32x4 va, vb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t a = x.vv[j], b = x.vv[4 + j];
                asm volatile("" : "+v"(a), "+v"(b));
                va[j] = __uint_as_float(a << 16);
                vb[j] = __uint_as_float(b << 16);
            }
            const f16x8 vin = cat16(to_f16x4(va), to_f16x4(vb));
            // U - W S for both row blocks: six independent accumulators
            f32x4 a0 = mfma16(x.wn[0], sh[0], zero), b0 = mfma16(x.wn[4], sh[0], zero);
            f32x4 a1 = mfma16(x.wn[1], sh[1], zero), b1 = mfma16(x.wn[5], sh[1], zero);
            const f32x4 ua = mfma16(x.tb[0], vin, zero), ub = mfma16(x.tb[1], vin, zero);
            a0 = mfma16(x.wn[2], sh[2], a0);
            b0 = mfma16(x.wn[6], sh[2], b0);
            a1 = mfma16(x.wn[3], sh[3], a1);
            b1 = mfma16(x.wn[7], sh[3], b1);
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
            if (OUT) {
#pragma unroll
                for (int b = 0; b < 8; ++b) *(f32x4 *)(snap + b * 1024 + l * 16) = S[b];
            }
            const f16x8 vn = cat16(to_f16x4((a0 + a1) + ua), to_f16x4((b0 + b1) + ub));
            if (OUT) *(f16x8 *)(snap + 8192 + l * 16) = vn;
#pragma unroll
            for (int b = 0; b < 8; ++b) S[b] = mfma16(KT_AHEAD ? x.kt[KT_AHEAD ? b : 0] : kt[b], vn, Sd[b]);
        };
        // after each barrier every LDS access of the wave issued before it is waited for
        auto sync_chain = [&] {
            sync();
            __builtin_amdgcn_s_waitcnt(0xc07f);
        };
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
        if (sout) state_tile_store(sout, sout_bf, sbase, gq, S);
        return;
    }

    // ---- output wave: chunks m = parity, parity + 2, ...; key blocks 0-1 of chunk m's
    // output after barrier m+1, the rest and P V_new after barrier m+2. Its Q+ and P
    // pieces come straight from global memory into registers, four chunks ahead.
    // One slice per block: the wave forms both 16-row blocks of its slice. Two slices:
    // output wave `slice` of a parity forms row block `slice` of both slices, so that the
    // block reads each chunk's Q+ and P pieces once (each wave the half of its rows), not
    // once per slice.
    constexpr int NR = NW == 1 ? 2 : 1;     // row blocks per output wave
    constexpr int NSL = NW;                  // slices per output wave
    auto row_block = [&](int r) { return NW == 1 ? r : slice; };
    auto slice_of = [&](int s) { return NW == 1 ? slice : s; };
    struct OutIn {
        bf16x8 qh[4 * NR], ql[4 * NR];
        f16x8 pp[NR];
    };
    auto load = [&](OutIn &x, int m) {
        const char *rec = rec_of(m);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int piece = (4 * row_block(r) + kb) * 1024;
                x.qh[4 * r + kb] = *(const bf16x8 *)(rec + RecH::QH + piece + l * 16);
                x.ql[4 * r + kb] = *(const bf16x8 *)(rec + RecH::QL + piece + l * 16);
            }
            x.pp[r] = *(const f16x8 *)(rec + RecH::PP + row_block(r) * 1024 + l * 16);
        }
    };
    auto snap_sl = [&](int m, int s) { return snaps + ((m % P::SNAPS) * NW + slice_of(s)) * P::SNAP; };
    // two accumulators per (row block, slice): Q+hi S_hi and Q+lo S_hi in oa, Q+hi S_lo
    // and P V_new in oc, so that no product waits on the one before it
    f32x4 oa[NR][NSL], oc[NR][NSL];
    auto half_qs = [&](const OutIn &x, int m, int kb0) {
#pragma unroll
        for (int kb = kb0; kb < kb0 + 2; ++kb) {
            bf16x8 sh[NSL], sl[NSL];
#pragma unroll
            for (int s = 0; s < NSL; ++s) {
                const char *snap = snap_sl(m, s);
                const f32x4 s0 = *(const f32x4 *)(snap + (2 * kb) * 1024 + l * 16);
                const f32x4 s1 = *(const f32x4 *)(snap + (2 * kb + 1) * 1024 + l * 16);
                bf16x4 h0, l0, h1, l1;
                split4(s0, h0, l0);
                split4(s1, h1, l1);
                sh[s] = cat(h0, h1);
                sl[s] = cat(l0, l1);
            }
#pragma unroll
            for (int s = 0; s < NSL; ++s)
#pragma unroll
                for (int r = 0; r < NR; ++r) oa[r][s] = mfma(x.qh[4 * r + kb], sh[s], oa[r][s]);
#pragma unroll
            for (int s = 0; s < NSL; ++s)
#pragma unroll
                for (int r = 0; r < NR; ++r) oc[r][s] = mfma(x.qh[4 * r + kb], sl[s], oc[r][s]);
#pragma unroll
            for (int s = 0; s < NSL; ++s)
#pragma unroll
                for (int r = 0; r < NR; ++r) oa[r][s] = mfma(x.ql[4 * r + kb], sh[s], oa[r][s]);
        }
    };
    auto first = [&](const OutIn &x, int m) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int s = 0; s < NSL; ++s) oa[r][s] = zero, oc[r][s] = zero;
        half_qs(x, m, 0);
        __builtin_amdgcn_s_waitcnt(0xc07f);   // snapshot reads done before the next barrier
    };
    auto finish = [&](const OutIn &x, int m) {
        f16x8 vn[NSL];
#pragma unroll
        for (int s = 0; s < NSL; ++s) vn[s] = *(const f16x8 *)(snap_sl(m, s) + 8192 + l * 16);
        half_qs(x, m, 2);
        const int64_t t0 = bos + (int64_t)CH * m;
        const int nc = (int)min<int64_t>(CH, eos - t0);
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int s = 0; s < NSL; ++s) {
                oc[r][s] = mfma16(x.pp[r], vn[s], oc[r][s]);
                oa[r][s] += oc[r][s];
            }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int s = 0; s < NSL; ++s) {
                    const int row = C * row_block(r) + 4 * gq + j;
                    const int cs = vcol0 + slice_of(s) * 16 + c;
                    float *d = row < nc ? out + ((t0 + row) * H + h) * D + cs : h32_sink + l;
                    *d = oa[r][s][j];
                }
        __builtin_amdgcn_s_waitcnt(0xc07f);
    };
    OutIn X, Y;
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
__global__ __launch_bounds__(64 * PairLayout<NW>::WAVES) void recur_h32_kernel(
    const char *__restrict__ recs, const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order, int N, int T, int H,
    const float *s0, float *__restrict__ out, float *sfin, float *carry, int fb, int fe, int sbf) {
    extern __shared__ __attribute__((aligned(16))) char ring[];
    recur_h32_block<NW, NSLOT>(xcd_remap(blockIdx.x, gridDim.x, D / (16 * NW)), ring, recs, v, cu, chunk_off,
                               order, N, T, H, s0, out, sfin, carry, fb, fe, sbf != 0);
}

// One launch: the recurrence over the segment [fb, fe) on blocks [0, RB) and the records
// of the segment [pb, pe) on the blocks after them (PREP_WAVES chunk-heads per block).
// The LDS request admits one block per CU, and workgroups are dispatched in index
// order, so the prep blocks fill the CUs the recurrence leaves idle.
constexpr int H32_PREP_WAVES = 4;

template <int NW, int NSLOT, typename GT>
__global__ __launch_bounds__(64 * PairLayout<NW>::WAVES) void recur_h32_prep_kernel(
    const char *__restrict__ recs_in, const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order, int N, int T, int H,
    const float *s0, float *__restrict__ out, float *sfin, float *carry, int fb, int fe, int RB, int sbf,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const GT *__restrict__ g,
    const float *__restrict__ beta, float scale, char *__restrict__ recs_out, int pb, int pe, int xsplit) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    int prep_block;
    if (xsplit) {
        // Workgroups are dealt to the eight XCDs in turn (block b to XCD b mod 8). XCDs 0-3
        // run the recurrence, each chain whole on one of them (XCD x, k = b / 8: chain
        // 4 (k / P) + x, column block k mod P); XCDs 4-7 prepare the next segment, so that its
        // HBM reads and record writes stay out of the L2s the recurrence reads its records from.
        constexpr int P = D / (16 * NW);
        const int x = (int)blockIdx.x & 7, kk = (int)blockIdx.x >> 3;
        if (x < 4) {
            const int chain = 4 * (kk / P) + x;
            if (chain * P < RB)
                recur_h32_block<NW, NSLOT>(chain * P + kk % P, lds, recs_in, v, cu, chunk_off, order, N, T, H, s0,
                                           out, sfin, carry, fb, fe, sbf != 0);
            return;
        }
        prep_block = 4 * kk + x - 4;
    } else {
        if ((int)blockIdx.x < RB) {
            recur_h32_block<NW, NSLOT>(xcd_remap(blockIdx.x, RB, D / (16 * NW)), lds, recs_in, v, cu, chunk_off,
                                       order, N, T, H, s0, out, sfin, carry, fb, fe, sbf != 0);
            return;
        }
        prep_block = (int)blockIdx.x - RB;
    }
    const int w = threadIdx.x >> 6;
    if (w >= H32_PREP_WAVES) return;
    const int64_t idx = (int64_t)prep_block * H32_PREP_WAVES + w;
    int h;
    const int ci = seg_chunk_of(chunk_off, N, H, pb, pe, idx, h);
    if (ci < 0) return;
    prep_h32_one(q, k, g, beta, cu, N, T, H, scale, chunk_off, recs_out, ci, h,
                 *(PrepHLds *)(lds + w * (int)sizeof(PrepHLds)));
}

// Pass 1 of the recurrence over parts: blocks [0, G/2) run every part from a zero state,
// blocks [G/2, G) from the identity with v taken as 0 (final state: the part's linear map).
// Its states are all fp32 (workspace); it forms no outputs (pass 2 writes them all), so
// its blocks are four chain waves (64 value columns) and the loader.
template <int NW, int NSLOT>
__global__ __launch_bounds__(64 * PairLayout<NW>::WAVES) void recur_h32_parts_kernel(
    const char *__restrict__ recs, const uint16_t *__restrict__ v, const int32_t *__restrict__ vcu,
    const int32_t *__restrict__ vco, const int32_t *__restrict__ vorder, int NV, int T, int H,
    const float *ident, float *out, float *rb, float *ri) {
    extern __shared__ __attribute__((aligned(16))) char ring[];
    const int RB = (int)(gridDim.x / 2);
    const bool id = (int)blockIdx.x >= RB;
    const int b = id ? (int)blockIdx.x - RB : (int)blockIdx.x;
    recur_h32_block<NW, NSLOT, false>(xcd_remap(b, RB, D / (16 * NW)), ring, recs, v, vcu, vco, vorder, NV, T, H,
                                      id ? ident : nullptr, out, id ? ri : rb, id ? ri : rb, 0, SEG_ONE, false, id);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_prep_h32(const uint16_t *q, const uint16_t *k, const void *g, bool g_bf16, const float *beta,
                           const int32_t *cu, int N, int T, int H, float scale, const int32_t *chunk_off,
                           char *recs, int fb, int fe, int64_t M, hipStream_t st) {
    const int64_t blocks = seg_chunks_bound(M, N, fb, fe) * H;
    if (blocks <= 0 || fe <= fb) return hipSuccess;
    if (g_bf16)
        hipLaunchKernelGGL(prep_h32_kernel<uint16_t>, dim3((unsigned)blocks), dim3(64), 0, st, q, k,
                           (const uint16_t *)g, beta, cu, N, T, H, scale, chunk_off, recs, fb, fe);
    else
        hipLaunchKernelGGL(prep_h32_kernel<float>, dim3((unsigned)blocks), dim3(64), 0, st, q, k, (const float *)g,
                           beta, cu, N, T, H, scale, chunk_off, recs, fb, fe);
    return hipGetLastError();
}

bool prep_h32_maps(int N) { return N >= 1 && N <= MAP_WAVE_MAX; }

hipError_t launch_prep_h32_map(const uint16_t *q, const uint16_t *k, const void *g, bool g_bf16, const float *beta,
                               const int32_t *cu, int N, int T, int H, float scale, char *recs, int fe, int64_t M,
                               int32_t *cu_safe, int32_t *chunk_off, int32_t *order, int32_t *err, hipStream_t st) {
    if (!prep_h32_maps(N) || fe <= 0 || fe > SEG_ONE) return hipErrorInvalidValue;
    // at least one block: block 0 stores the map even when there are no chunks
    int64_t blocks = seg_chunks_bound(M, N, 0, fe) * H;
    if (blocks < 1) blocks = 1;
    if (g_bf16)
        hipLaunchKernelGGL(prep_h32_map_kernel<uint16_t>, dim3((unsigned)blocks), dim3(64), 0, st, q, k,
                           (const uint16_t *)g, beta, cu, N, T, H, scale, recs, fe, cu_safe, chunk_off, order, err,
                           device_error_word());
    else
        hipLaunchKernelGGL(prep_h32_map_kernel<float>, dim3((unsigned)blocks), dim3(64), 0, st, q, k,
                           (const float *)g, beta, cu, N, T, H, scale, recs, fe, cu_safe, chunk_off, order, err,
                           device_error_word());
    return hipGetLastError();
}

template <int NW>
static hipError_t launch_recur_h32_t(const char *recs, const uint16_t *v, const int32_t *cu,
                                     const int32_t *chunk_off, const int32_t *order, int N, int T, int H,
                                     const float *s0, float *out, float *sfin, float *carry, int fb, int fe,
                                     bool sbf, hipStream_t st) {
    constexpr int NS = pairh_nslot<NW>();
    constexpr int lds = PairHLds<NW, NS>::BYTES;
    auto kern = recur_h32_kernel<NW, NS>;
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)kern, lds, lds_set) != hipSuccess) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)N * H * (D / (16 * NW));
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * PairLayout<NW>::WAVES), lds, st, recs, v, cu,
                       chunk_off, order, N, T, H, s0, out, sfin, carry, fb, fe, (int)sbf);
    return hipGetLastError();
}

hipError_t launch_recur_h32_range(const char *recs, const uint16_t *v, const int32_t *cu, const int32_t *chunk_off,
                                  const int32_t *order, int N, int T, int H, const float *s0, float *out, float *sfin,
                                  float *carry, int waves, int fb, int fe, bool sbf, hipStream_t st) {
    switch (waves) {
    case 401: return launch_recur_h32_t<1>(recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, carry, fb, fe, sbf, st);
    case 402: return launch_recur_h32_t<2>(recs, v, cu, chunk_off, order, N, T, H, s0, out, sfin, carry, fb, fe, sbf, st);
    default: return hipErrorInvalidValue;
    }
}

template <int NW, typename GT>
static hipError_t launch_recur_h32_prep_t(const RecurPrepArgs &a, hipStream_t st) {
    constexpr int NS = pairh_nslot<NW>();
    constexpr int pair = PairHLds<NW, NS>::BYTES;
    constexpr int prep = H32_PREP_WAVES * (int)sizeof(PrepHLds);
    constexpr int lds = pair > prep ? pair : prep;
    static_assert(lds <= 160 * 1024 && lds > 80 * 1024, "LDS");
    auto kern = recur_h32_prep_kernel<NW, NS, GT>;
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)kern, lds, lds_set) != hipSuccess) return hipErrorInvalidValue;
    constexpr int P = D / (16 * NW);
    const int64_t chains = (int64_t)a.N * a.H;
    const int64_t rb = chains * P;
    const int64_t pblocks =
        a.pe > a.pb ? (seg_chunks_bound(a.M, a.N, a.pb, a.pe) * a.H + H32_PREP_WAVES - 1) / H32_PREP_WAVES : 0;
    // two-slice blocks of at most 32 chains: the recurrence on XCDs 0-3 (eight chains of
    // four blocks fill an XCD's 32 CUs), the prep on XCDs 4-7 (see the kernel)
    const bool xsplit = NW == 2 && chains <= 32;
    int64_t grid = rb + pblocks;
    if (xsplit) {
        const int64_t krec = (chains + 3) / 4 * P, kprep = (pblocks + 3) / 4;
        grid = 8 * (krec > kprep ? krec : kprep);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * PairLayout<NW>::WAVES), lds, st, a.recs, a.v,
                       a.cu, a.chunk_off, a.order, a.N, a.T, a.H, a.s0, a.out, a.sfin, a.carry, a.fb, a.fe, (int)rb,
                       (int)a.state_bf16, a.q, a.k, (const GT *)a.g, a.beta, a.scale, a.recs, a.pb, a.pe, (int)xsplit);
    return hipGetLastError();
}

hipError_t launch_recur_h32_prep(const RecurPrepArgs &a, int waves, hipStream_t st) {
    switch (waves * 2 + (a.g_bf16 ? 1 : 0)) {
    case 802: return launch_recur_h32_prep_t<1, float>(a, st);
    case 803: return launch_recur_h32_prep_t<1, uint16_t>(a, st);
    case 804: return launch_recur_h32_prep_t<2, float>(a, st);
    case 805: return launch_recur_h32_prep_t<2, uint16_t>(a, st);
    default: return hipErrorInvalidValue;
    }
}

// pass 1 of the recurrence over parts on 32-token records (two-slice blocks, 2 x 4 NV H)
hipError_t launch_h32_parts_pass1(const char *recs, const uint16_t *v, const int32_t *vcu, const int32_t *vco,
                                  const int32_t *vorder, int NV, int T, int H, const float *ident, float *out,
                                  float *rb, float *ri, hipStream_t st) {
    constexpr int NW = 4, NS = 4;
    constexpr int lds = PairHLds<NW, NS, false>::BYTES;
    auto kern = recur_h32_parts_kernel<NW, NS>;
    static std::atomic<uint64_t> lds_set{0};
    if (ensure_lds_limit((const void *)kern, lds, lds_set) != hipSuccess) return hipErrorInvalidValue;
    const int64_t rbk = (int64_t)NV * H * (D / (16 * NW));
    hipLaunchKernelGGL(kern, dim3((unsigned)(2 * rbk)), dim3(64 * PairLayout<NW>::WAVES), lds, st, recs, v, vcu, vco,
                       vorder, NV, T, H, ident, out, rb, ri);
    return hipGetLastError();
}

}  // namespace kda
