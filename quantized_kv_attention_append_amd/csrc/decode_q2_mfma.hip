// Split-K decode attention over the 2-bit pool on the gfx950 matrix cores
// (head_dim 128 or 256; four query heads of a KV head's group a launch, so
// groups 1 and 2 leave rows of the products empty and group 8 takes two
// launches).
//
// At group 4 and 256 dims a decode step does 2 x 4 x 256 multiply-adds for
// every 144 bytes of K and V rows it reads, more than the vector ALUs can
// sustain at full HBM bandwidth, so both contractions run on
// v_mfma_scale_f32_16x16x128_f8f6f4.  Its internal sum drops low-order bits
// of products much smaller than the largest product of a group, but sums
// small-integer products exactly, so every operand is made of small integers
// and every power of two goes into the instruction's per-row / per-column
// scale:
//   * 2-bit codes c become fp4 (e2m1) nibbles whose value is c/2: a 32-bit
//     word of 16 codes spreads into two words of nibbles with one shift and
//     two masks (w & 0x33333333, (w >> 2) & 0x33333333);
//   * the bf16 query of each head becomes a 19-bit fixed-point integer
//     round(q * 2^E) (exact unless |q| < max|q| / 2^11), written as four
//     balanced radix-32 digits in -16..16 (exact in e4m3); row 4h + i of the
//     q.k product is digit i of head h, weighted 32^(3-i) 2^-E by its scale;
//   * the softmax weights w_t = p_t * scale_t become 16-bit fixed-point
//     integers relative to each head's largest weight in a block of 32
//     tokens, split into four 4-bit digits.  An e4m3 byte 0..15 is exactly
//     b * 2^-9, so the digits go into the operand with byte shuffles only;
//     column 4h + i of the p.v product is digit i of head h, and its scale
//     for k-block b (32 tokens) weights it 16^i 2^-F(h, b).
// The dequantization is folded algebraically (q.k^_t = mn_t sum(q) + scale_t
// q.c_t; p.v^ = sum p_t mn_t + sum (p_t scale_t) c_t), and the online softmax,
// its rescaling and every running sum are fp32 registers (the two-level
// accumulation "Half the Cache, Twice the Context" asks for in section "The
// cliff is in the accumulator").
//
// One workgroup of four wavefronts per (sequence, KV head, split); wave w
// takes every fourth pair of pages of the split (128 tokens = one k-block of
// the instruction), keeping the next two pairs' loads in flight while it
// computes the current one, and the four waves combine their partial results
// in LDS.  Token t of the pair sits at page t/64, slot t%64.  Operand lane
// layouts of the instruction: fp4 lane group g holds k = 32g..32g+31; fp8
// lane group g holds k = 16g..16g+15 and 64+16g..64+16g+15; the result lane l
// holds column l%16, rows 4(l/16)..+3.
//   q.k (8 per tile): A = query digits (row 4h + i), B = K codes of tokens
//       16m..16m+15 of the pair (column j = token 16m + j, k = dims), so lane
//       l ends with the score of token 16m + l%16 for head l/16: every
//       (token, head) score of the tile is computed once, eight per lane.
//   p.v (D/16 per tile): A = V codes of 16 dims (k = tokens), B = weight
//       digits (column 4h + i).  The V words put token
//       64(g/2) + 16(t%4) + 8(g%2) + 4u + 2x + t/4 at k = 32g + 16u + 8x + t,
//       and a per-wave LDS transpose moves each lane's digit bytes of its
//       eight tokens to the lanes whose k-ranges hold those tokens.
#include <type_traits>

#include "decode_common.h"

namespace kvq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

constexpr int FMT_FP8 = 0;  // e4m3
constexpr int FMT_FP4 = 4;  // e2m1

// q.k: A = query digits (fp8) with per-row scale, B = K codes (fp4)
__device__ __forceinline__ v4f mma_qk(const v8i& a_fp8, const v8i& b_fp4, v4f c, int scale_a) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp8, b_fp4, c, FMT_FP8, FMT_FP4, 0, scale_a, 0, 127);
}
// p.v: A = V codes (fp4), B = weight digits (fp8) with per-column scale
__device__ __forceinline__ v4f mma_pv(const v8i& a_fp4, const v8i& b_fp8, v4f c, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp4, b_fp8, c, FMT_FP4, FMT_FP8, 0, 127, 0, scale_b);
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// 16 two-bit codes -> two words of eight e2m1 nibbles (value = code / 2).
__device__ __forceinline__ uint32_t nib_lo(uint32_t w) { return w & 0x33333333u; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t w) { return (w >> 2) & 0x33333333u; }

__device__ __forceinline__ v8i fp4_operand(uint32_t w0, uint32_t w1) {
    v8i r;
    r[0] = (int)nib_lo(w0);
    r[1] = (int)nib_hi(w0);
    r[2] = (int)nib_lo(w1);
    r[3] = (int)nib_hi(w1);
    r[4] = r[5] = r[6] = r[7] = 0;
    return r;
}

// Balanced radix-32 digits: x (|x| < 2^19 after scaling) is rounded to an
// integer n and n + DIGIT_BIAS is written in base 32 with fields f0 (6 bits,
// 0..32) f1 f2 f3; digit d = f_d - 16 lies in -16..16 and
// n = sum_d digit_d * 32^(3-d).  Adding 2^23 + DIGIT_BIAS to x in one fused
// multiply-add leaves n + DIGIT_BIAS in the low mantissa bits.
constexpr float DIGIT_BIAS = 541200.0f;  // 16 * (1 + 32 + 32^2 + 32^3)
constexpr float DIGIT_MAGIC = 8388608.0f + DIGIT_BIAS;
__device__ __forceinline__ float digit_of(float x, float scale, int d) {
    const uint32_t u = __float_as_uint(fmaf(x, scale, DIGIT_MAGIC));
    const int f = (int)__builtin_amdgcn_ubfe(u, 15 - 5 * d, d == 0 ? 6 : 5);
    return (float)(f - 16);
}
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }
__device__ __forceinline__ int exponent_of(float x) { return (int)((__float_as_uint(x) >> 23) & 0xFF) - 127; }

// Reductions over the 16 lanes of a DPP row (row_ror by 8, 4, 2, 1).
template <int CTRL>
__device__ __forceinline__ float ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, ror<0x128>(x));
    x = fmaxf(x, ror<0x124>(x));
    x = fmaxf(x, ror<0x122>(x));
    return fmaxf(x, ror<0x121>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
    x += ror<0x128>(x);
    x += ror<0x124>(x);
    x += ror<0x122>(x);
    return x + ror<0x121>(x);
}
// Max over the eight lanes of a half row (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror).
__device__ __forceinline__ float half_row_max8(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
}
// Fixed-point exponent F of a block of weights with max wmax: wmax 2^F in
// [2^15, 2^16), so X = round(w 2^F) fits 16 bits (capped at 2^16 - 1).  F is
// clamped to [-105, 126] so that the column scale 137 + 4i - F stays a valid
// power-of-two byte; weights above 2^120 are out of range.
__device__ __forceinline__ int weight_exp(float wmax) {
    return wmax > 0.f ? max(min(15 - exponent_of(wmax), 126), -105) : 0;
}
// Sum over the four lanes of a quad (quad_perm [1,0,3,2] then [2,3,0,1]).
__device__ __forceinline__ float quad_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// k index of byte s of an fp8 operand held by lane group grp.
__device__ __forceinline__ int fp8_k(int grp, int s) { return s < 16 ? 16 * grp + s : 64 + 16 * grp + (s - 16); }

}  // namespace

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// A head's reference max moves only when a tile's max exceeds it by more than
// 2^8 in weight, so the running sums are rescaled rarely (weights stay < 2^8).
constexpr float RESCALE_LOG2 = 8.0f;

template <int D>
struct Tile {
    uint32_t kc[8][D / 64];  // K code words of token 16m + l%16 of the pair, this lane group's D/16 bytes
    uint4 vc[D / 32];        // V words of dims 32c + l%16 and 32c + 16 + l%16 for this lane group's k-range
    uint4 meta[2];           // K and V metadata (scale, min) of tokens 2l and 2l + 1 of the pair
};

template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& t, const uint8_t* base0, const uint8_t* base1, int l) {
    constexpr int NW = D / 64;
    const int j = l & 15, grp = l >> 4;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const uint8_t* src = (m < 4 ? base0 : base1) + (16 * (m & 3) + j) * (D / 4) + 4 * NW * grp;
        if constexpr (NW == 4) {
            const uint4 w = stream_load4(src);
            t.kc[m][0] = w.x; t.kc[m][1] = w.y; t.kc[m][2] = w.z; t.kc[m][3] = w.w;
        } else {
            const uint2 w = stream_load2(src);
            t.kc[m][0] = w.x; t.kc[m][1] = w.y;
        }
    }
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        t.vc[c] = stream_load4((grp < 2 ? base0 : base1) + q2_vcodes_off(D) + q2_vword_off(D, 32 * c + j, 2 * (grp & 1)));
    const uint8_t* mb = (l < 32 ? base0 : base1) + 16 * (l & 31);
    t.meta[0] = stream_load4(mb + q2_kmeta_off(D));
    t.meta[1] = stream_load4(mb + q2_vmeta_off(D));
}

template <int D>
struct WaveState {
    v4f acc[D / 16];  // p.v sums: block b, column 4h + i of lane l%16, dims 16b + 4(l/16) + r
    float m_ref;      // reference max of head l/16, raw q.k^ units
    float cbm;        // cB * m_ref (log2 units)
    float l_run;      // this lane's share of sum p (head l/16)
    float c_run;      // this lane's share of sum p * min_v (head l/16)
};

struct QConst {
    int scale_a;  // q.k row scale of this lane's row (4h + i): 32^(3-i) 2^-E_h * 2 (codes are c/2)
    float qsum;   // sum_d q_d of head l/16
    float cB;     // log2(e) * sm: raw q.k^ -> log2 units
};

// Per-wave LDS: the tile's metadata as {k scale, k min, v scale, v min} per
// token, and the weight-digit transpose: for head h and digit i, 32 words at
// wdig_base(h, i); word c (c < 16) holds the digits of tokens 16m + c for
// m = 0..3, word 16 + c those for m = 4..7.
struct WaveLds {
    float4 meta[2 * PAGE];
    uint32_t wdig[4 * 4 * 32 + 16 * 3];
};
__device__ __forceinline__ int wdig_base(int h, int i) { return (4 * h + i) * 32 + 16 * h; }

template <int D, bool FULL, bool SCORES>
__device__ __forceinline__ void compute_tile(const Tile<D>& t, WaveLds& lds, int l, const v8i* qop,
                                             const QConst& qc, WaveState<D>& st, int tok0, int ctx,
                                             float* __restrict__ srow) {
    constexpr int NC = D / 128, NB = D / 16;
    const int j = l & 15, grp = l >> 4;
    {
        const uint4 k = t.meta[0], v = t.meta[1];
        lds.meta[2 * l] = make_float4(__uint_as_float(k.x), __uint_as_float(k.y), __uint_as_float(v.x),
                                      __uint_as_float(v.y));
        lds.meta[2 * l + 1] = make_float4(__uint_as_float(k.z), __uint_as_float(k.w), __uint_as_float(v.z),
                                          __uint_as_float(v.w));
    }
    // ---- q.k: raw scores q.k^ of tokens 16m + j, head grp ----
    float s[8];
    float4 mt[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        v4f cq = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) cq = mma_qk(qop[c], fp4_operand(t.kc[m][2 * c], t.kc[m][2 * c + 1]), cq, qc.scale_a);
        mt[m] = lds.meta[16 * m + j];
        float x = fmaf(mt[m].x, (cq[0] + cq[1]) + (cq[2] + cq[3]), mt[m].y * qc.qsum);
        if (!FULL && tok0 + 16 * m + j >= ctx) x = -INFINITY;
        s[m] = x;
        tmax = fmaxf(tmax, x);
    }
    tmax = row_max16(tmax);
    const bool need = (tmax - st.m_ref) * qc.cB > RESCALE_LOG2;
    if (__ballot(need)) {
        const float m_new = need ? tmax : st.m_ref;
        const float cbm_new = qc.cB * m_new;
        const float alpha = __builtin_amdgcn_exp2f(st.cbm - cbm_new);
        st.l_run *= alpha;
        st.c_run *= alpha;
        // accumulator columns of lane l belong to head (l%16)/4
        const float a = __shfl(alpha, 16 * (j >> 2));
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) st.acc[b][r] *= a;
        st.m_ref = m_new;
        st.cbm = cbm_new;
    }
    // ---- weights w = p * scale_v ----
    float w[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[m], qc.cB, -st.cbm));
        float x;
        if (FULL) {
            x = p * mt[m].z;
            st.c_run = fmaf(p, mt[m].w, st.c_run);
        } else {
            const bool valid = tok0 + 16 * m + j < ctx;
            x = valid ? p * mt[m].z : 0.f;
            st.c_run += valid ? p * mt[m].w : 0.f;
        }
        st.l_run += p;
        w[m] = x;
    }
    if (SCORES && srow) {  // lanes of a head past the group's end hold no score row
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int tok = tok0 + 16 * m + j;
            if (FULL || tok < ctx) srow[tok] = s[m] * (qc.cB * LN2);
        }
    }
    // ---- weight digits: X = round(w 2^F) < 2^16, four 4-bit digits per weight ----
    // The p.v column scale of lane l covers k-block l/16 (32 tokens): tokens
    // 16m + c with c in [8 (b % 2), 8 (b % 2) + 8) and m in [4 (b / 2), 4 (b / 2) + 4),
    // so each lane takes the max of its first and last four weights over its
    // half row, and F is set per head and 32-token block.
    const float wlo = half_row_max8(fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3])));
    const float whi = half_row_max8(fmaxf(fmaxf(w[4], w[5]), fmaxf(w[6], w[7])));
    const int FWlo = weight_exp(wlo), FWhi = weight_exp(whi);
    const float wscale_lo = pow2f(FWlo), wscale_hi = pow2f(FWhi);
    uint32_t X[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)  // 2^23 + X in the bits of the fused multiply-add, X capped at 2^16 - 1
        X[m] = min(__float_as_uint(fmaf(w[m], m < 4 ? wscale_lo : wscale_hi, 8388608.0f)), 0x4B00FFFFu);
    uint32_t P[4];  // X of tokens m = 2k (bytes 0-1) and 2k + 1 (bytes 2-3)
#pragma unroll
    for (int k = 0; k < 4; ++k) P[k] = __builtin_amdgcn_perm(X[2 * k + 1], X[2 * k], 0x05040100u);
    uint32_t L[4], H[4];  // nibbles 0 and 2 (L), 1 and 3 (H) of each X, one per byte
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        L[k] = P[k] & 0x0F0F0F0Fu;
        H[k] = (P[k] >> 4) & 0x0F0F0F0Fu;
    }
    // digit i of tokens m = 0..3 and m = 4..7, one byte per token
    const uint32_t d0a = __builtin_amdgcn_perm(L[1], L[0], 0x06040200u), d0b = __builtin_amdgcn_perm(L[3], L[2], 0x06040200u);
    const uint32_t d2a = __builtin_amdgcn_perm(L[1], L[0], 0x07050301u), d2b = __builtin_amdgcn_perm(L[3], L[2], 0x07050301u);
    const uint32_t d1a = __builtin_amdgcn_perm(H[1], H[0], 0x06040200u), d1b = __builtin_amdgcn_perm(H[3], H[2], 0x06040200u);
    const uint32_t d3a = __builtin_amdgcn_perm(H[1], H[0], 0x07050301u), d3b = __builtin_amdgcn_perm(H[3], H[2], 0x07050301u);
    {
        uint32_t* wd = lds.wdig;
        wd[wdig_base(grp, 0) + j] = d0a; wd[wdig_base(grp, 0) + 16 + j] = d0b;
        wd[wdig_base(grp, 1) + j] = d1a; wd[wdig_base(grp, 1) + 16 + j] = d1b;
        wd[wdig_base(grp, 2) + j] = d2a; wd[wdig_base(grp, 2) + 16 + j] = d2b;
        wd[wdig_base(grp, 3) + j] = d3a; wd[wdig_base(grp, 3) + 16 + j] = d3b;
    }
    // p.v operand of column j = 4h + i: k = 16 grp + s <- word 4 grp + s/4 byte s%4,
    // k = 64 + 16 grp + s <- word 16 + 4 grp + s/4 byte s%4
    v8i wop;
    {
        const int base = wdig_base(j >> 2, j & 3) + 4 * grp;
        const uint4 lo = *reinterpret_cast<const uint4*>(&lds.wdig[base]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&lds.wdig[base + 16]);
        wop[0] = (int)lo.x; wop[1] = (int)lo.y; wop[2] = (int)lo.z; wop[3] = (int)lo.w;
        wop[4] = (int)hi.x; wop[5] = (int)hi.y; wop[6] = (int)hi.z; wop[7] = (int)hi.w;
    }
    // column scale of (column j = 4h + i, k-block grp): byte b of digit i is
    // worth b 2^-9 and the code nibble is c / 2, so 2^(4i - F + 10)
    const int fw_pair = __shfl((FWlo + 128) | ((FWhi + 128) << 16), 16 * (j >> 2) + 8 * (grp & 1));
    const int scale_b = 137 + 4 * (j & 3) - (((fw_pair >> (16 * (grp >> 1))) & 0xFFFF) - 128);
    // ---- p.v ----
#pragma unroll
    for (int c = 0; c < NB / 2; ++c) {
        st.acc[2 * c] = mma_pv(fp4_operand(t.vc[c].x, t.vc[c].y), wop, st.acc[2 * c], scale_b);
        st.acc[2 * c + 1] = mma_pv(fp4_operand(t.vc[c].z, t.vc[c].w), wop, st.acc[2 * c + 1], scale_b);
    }
}

template <int D, bool SCORES, bool ROT, bool GENERAL, bool FUSE>
__device__ __forceinline__ void decode_q2_mfma_body(const PoolView& pv, int layer, const BatchDesc& bd,
                                                    const uint16_t* __restrict__ q, float sm, int splits,
                                                    float* __restrict__ ws, float* __restrict__ out,
                                                    float* __restrict__ scores, int64_t sstride, int h0, int nh) {
    // The kernel takes four query heads of a KV head's group at a time: heads
    // h0 .. h0 + nh - 1.  Without GENERAL the group is exactly these four
    // (group 4, h0 = 0, nh = 4, all known when compiling); with it the group
    // size is the pool's, and when nh < 4 the rows of the missing heads are
    // zero queries whose results are dropped.
    constexpr int G = 4;
    constexpr int NC = D / 128;  // k-chunks of the q.k product
    constexpr int NB = D / 16;   // 16-dim blocks of the p.v product
    const int Hkv = pv.Hkv, Hq = pv.Hq;
    const int e = blockIdx.x / Hkv, g = blockIdx.x % Hkv, sp = blockIdx.y;
    const int Gq = GENERAL ? Hq / Hkv : G;  // the pool's GQA group
    if constexpr (!GENERAL) {
        h0 = 0;
        nh = G;
    }
    const int64_t head0 = (int64_t)e * Hq + (int64_t)g * Gq + h0;  // first query row of this launch
    const int ctx = bd.pos[e];
    int pg0, pg1;
    split_range(ctx, bd.per, sp, &pg0, &pg1);
    if (pg0 >= pg1) return;

    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int j = l & 15, grp = l >> 4;
    const int hq = j >> 2, iq = j & 3;  // this lane's q.k row: digit iq of head hq

    __shared__ __align__(16) WaveLds lds_s[4];
    __shared__ float o_s[4][G][D];
    __shared__ float ml_s[4][G][3];

    const int32_t* bt = pv.bt + (int64_t)bd.seq[e] * pv.bt_stride;
    const int64_t lhoff = ((int64_t)layer * Hkv + g) * pv.block_bytes;
    const int n_pages = (ctx + PAGE - 1) / PAGE;
    float* srow = scores && (!GENERAL || grp < nh) ? scores + (head0 + grp) * sstride : nullptr;
    WaveLds& lds = lds_s[wave];

    // ---- this wave's tiles: page pairs pg0/2 + wave + 4i, i < T ----
    const int pr_first = pg0 / 2 + wave;
    const int pr_end = (pg1 + 1) / 2;
    const int T = pr_first < pr_end ? (pr_end - pr_first + 3) / 4 : 0;
    // the last tile of the sequence may be partly past ctx; it is done on its own
    const bool last_partial = T > 0 && 2 * (pr_first + 4 * (T - 1)) * PAGE + 2 * PAGE > ctx;
    const int TF = last_partial ? T - 1 : T;  // full tiles
    auto tok0_of = [&](int t) { return 2 * (pr_first + 4 * t) * PAGE; };

    // Tiles go in chunks of 64: lane k of pid0/pid1 holds the physical ids of
    // the two pages of tile c0 + k.  Two tile buffers keep one tile in flight
    // while the other is computed; every load is issued unconditionally
    // (indices clamped to the chunk's last tile, re-read from cache), and the
    // loop runs whole two-tile rounds with fixed buffer roles so that no
    // buffer is ever copied (a copy would wait for its load).
    Tile<D> ta, tb;
    int pid0 = 0, pid1 = 0, Tc = 0;
    auto fetch_ids = [&](int c0) {
        Tc = min(64, TF - c0);
        pid0 = pid1 = 0;
        if (l < Tc) {
            const int pair = pr_first + 4 * (c0 + l);
            pid0 = bt[2 * pair];
            pid1 = bt[2 * pair + 1];
        }
    };
    auto load = [&](Tile<D>& tile, int t) {
        const int tt = min(t, Tc - 1);
        load_tile<D>(tile, pv.pages + (int64_t)__builtin_amdgcn_readlane(pid0, tt) * pv.page_bytes + lhoff,
                     pv.pages + (int64_t)__builtin_amdgcn_readlane(pid1, tt) * pv.page_bytes + lhoff, l);
    };
    // The query rows of the group's G heads (contiguous, G D bf16) are loaded
    // first, in 16-byte pieces, so that preparing the query operand waits for
    // them only while the first tile is still in flight; they pass through
    // this wave's metadata area of LDS, unused until the first tile.
    constexpr int QPIECES = G * D * 2 / 16 / 64;  // 16-byte pieces per lane
    static_assert(G * D * 2 <= sizeof(WaveLds::meta), "query rows fit the metadata area");
    uint4 qraw[QPIECES];
    {
        const uint4* qsrc = reinterpret_cast<const uint4*>(q + head0 * D);
#pragma unroll
        for (int i = 0; i < QPIECES; ++i) {  // piece p holds bf16 8p .. 8p + 7 of the four rows
            const int p = l + 64 * i;
            qraw[i] = !GENERAL || 8 * p < nh * D ? qsrc[p] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    if (TF > 0) {
        fetch_ids(0);
        load(ta, 0);
    }
    // The rotated variant scores H q against the codes of H k (the launcher
    // passes sm / D): the rows are widened to fp32 over this wave's whole LDS
    // area and transformed there, stages h = 1 .. D/2 as on append.
    static_assert(!ROT || sizeof(WaveLds) >= G * D * sizeof(float), "fp32 query rows fit the wave's LDS area");
    if constexpr (ROT) {
        float* qf = reinterpret_cast<float*>(&lds);
#pragma unroll
        for (int i = 0; i < QPIECES; ++i) {
            const uint32_t u[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                qf[8 * (l + 64 * i) + 2 * k] = bf16lo(u[k]);
                qf[8 * (l + 64 * i) + 2 * k + 1] = bf16hi(u[k]);
            }
        }
        __syncthreads();
        for (int h = 1; h < D; h *= 2) {  // additions only: nothing to contract
            float a[G * D / 128], b[G * D / 128];
            int ia[G * D / 128];
#pragma unroll
            for (int k = 0; k < G * D / 128; ++k) {  // pair p = l + 64 k of the G D / 2 pairs
                const int pr = l + 64 * k, row = pr / (D / 2), jj = pr % (D / 2);
                ia[k] = row * D + (jj / h) * 2 * h + jj % h;
                a[k] = qf[ia[k]];
                b[k] = qf[ia[k] + h];
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < G * D / 128; ++k) {
                qf[ia[k]] = a[k] + b[k];
                qf[ia[k] + h] = a[k] - b[k];
            }
            __syncthreads();
        }
    } else {
        uint4* qdst = reinterpret_cast<uint4*>(lds.meta);
#pragma unroll
        for (int i = 0; i < QPIECES; ++i) qdst[l + 64 * i] = qraw[i];
        __syncthreads();
    }

    // ---- query operand: 19-bit fixed point per head, row 4 hq + iq = digit iq of head hq ----
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(lds.meta) + hq * D;
    const float* qrow_f = reinterpret_cast<const float*>(&lds) + hq * D;
    float qv[NC][32];
    float amax = 0.f, qsum = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            // k of byte s; the K operand puts dim(k) at nibble k % 32 of lane group k / 32
            const int k = fp8_k(grp, s), ga = k >> 5, n = k & 31;
            const int dim = 32 * NC * ga + 32 * c + 16 * (n >> 4) + 2 * (n & 7) + ((n >> 3) & 1);
            const float x = ROT ? qrow_f[dim] : bf16_to_f32(qrow[dim]);
            qv[c][s] = x;
            amax = fmaxf(amax, fabsf(x));
            qsum += x;
        }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    qsum += __shfl_xor(qsum, 16);
    qsum += __shfl_xor(qsum, 32);
    const int EQ = 18 - (amax > 0.f ? exponent_of(amax) : 0);  // |q * 2^EQ| < 2^19
    const float qscale = pow2f(EQ);
    QConst qc;
    qc.scale_a = 127 + 5 * (3 - iq) - EQ + 1;
    qc.qsum = __shfl(qsum, 4 * grp);  // q.k result lanes hold head l/16
    qc.cB = LOG2E * sm;
    v8i qop[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int v = 0; v < 8; ++v)
            qop[c][v] = (int)pack4_fp8(digit_of(qv[c][4 * v], qscale, iq), digit_of(qv[c][4 * v + 1], qscale, iq),
                                       digit_of(qv[c][4 * v + 2], qscale, iq), digit_of(qv[c][4 * v + 3], qscale, iq));

    WaveState<D> st;
#pragma unroll
    for (int b = 0; b < NB; ++b) st.acc[b] = v4f{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.cbm = -INFINITY;
    st.l_run = 0.f;
    st.c_run = 0.f;

    for (int c0 = 0; c0 < TF; c0 += 64) {
        if (c0 > 0) {
            fetch_ids(c0);
            load(ta, 0);
        }
        auto run = [&](const Tile<D>& tile, int t) {
            compute_tile<D, true, SCORES>(tile, lds, l, qop, qc, st, tok0_of(c0 + t), ctx, srow);
        };
        int t = 0;
        for (; t + 2 <= Tc; t += 2) {
            load(tb, t + 1);
            __builtin_amdgcn_sched_barrier(0);
            run(ta, t);
            load(ta, t + 2);
            __builtin_amdgcn_sched_barrier(0);
            run(tb, t + 1);
        }
        // at most one tile left, already loaded into ta
        if (t < Tc) run(ta, t);
    }
    if (last_partial) {
        const int pair = pr_first + 4 * (T - 1);
        const int p1 = 2 * pair + 1 < n_pages ? 2 * pair + 1 : 2 * pair;
        load_tile<D>(ta, pv.pages + (int64_t)bt[2 * pair] * pv.page_bytes + lhoff,
                     pv.pages + (int64_t)bt[p1] * pv.page_bytes + lhoff, l);
        compute_tile<D, false, SCORES>(ta, lds, l, qop, qc, st, tok0_of(T - 1), ctx, srow);
    }

    // ---- this wave's partial: sum the digit columns, and each head's lanes ----
    const float l_run = row_sum16(st.l_run), c_run = row_sum16(st.c_run);  // head grp
    if (j == 0) {
        ml_s[wave][grp][0] = st.cbm;  // log2 units
        ml_s[wave][grp][1] = l_run;
        ml_s[wave][grp][2] = c_run;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float4 o;
        o.x = quad_sum(st.acc[b][0]);
        o.y = quad_sum(st.acc[b][1]);
        o.z = quad_sum(st.acc[b][2]);
        o.w = quad_sum(st.acc[b][3]);
        if (iq == 0) *reinterpret_cast<float4*>(&o_s[wave][hq][16 * b + 4 * grp]) = o;
    }
    __syncthreads();

    // ---- combine the four waves, write this split's partial ----
    DecodeWs w(ws, bd.n, Hq, D, splits);
    {
        const int h = threadIdx.x >> 6;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) M = fmaxf(M, ml_s[v][h][0]);
        float f[4], lsum = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            f[v] = __builtin_amdgcn_exp2f(ml_s[v][h][0] - M);
            lsum += f[v] * ml_s[v][h][1];
        }
        const int64_t row = (head0 + h) * splits + sp;
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
            const int d = l + 64 * k;
            float o = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) o += f[v] * (o_s[v][h][d] + ml_s[v][h][2]);
            if (!GENERAL || h < nh) {
                if constexpr (FUSE) store_agent(&w.o[row * D + d], o);
                else w.o[row * D + d] = o;
            }
        }
        if (l == 0 && (!GENERAL || h < nh)) {
            if constexpr (FUSE) {
                store_agent(&w.ml[2 * row], M);
                store_agent(&w.ml[2 * row + 1], lsum);
            } else {
                w.ml[2 * row] = M;
                w.ml[2 * row + 1] = lsum;
            }
        }
    }
    if constexpr (FUSE) {
        // The last of the sequence's live splits to get here merges them all.
        // Partials travel through agent-scope (L2-coherent) stores and loads
        // only, so no cache writeback or invalidation is needed: every
        // thread's partial stores have completed before the workgroup counts
        // itself, and the merging workgroup loads them after the count shows
        // every split done.
        __shared__ int last_s;
        wait_stores();
        __syncthreads();
        const int live = live_splits(ctx, bd.per);
        int32_t* cnt = pv.cnt + ((int64_t)e * Hkv + g) * 2 + (h0 >> 2);
        if (threadIdx.x == 0) {
            const int before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int is_last = before == live - 1;
            if (is_last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
            last_s = is_last;
        }
        __syncthreads();
        if (!last_s) return;
        const int h = threadIdx.x >> 6;
        if (GENERAL && h >= nh) return;
        merge_live_splits<D / 64>(w, (head0 + h) * splits, live, l, out + (head0 + h) * D);
    }
}

// Group 4: the four heads of each KV head's group in one launch.  FUSE: the
// last split of each (sequence, KV head) to finish merges the partials into
// out (at most FUSED_MERGE_MAX_SPLITS splits).
template <int D, bool SCORES, bool ROT, bool FUSE>
__global__ __launch_bounds__(256) void decode_q2_mfma_kernel(PoolView pv, int layer, BatchDesc bd,
                                                             const uint16_t* __restrict__ q, float sm, int splits,
                                                             float* __restrict__ ws, float* __restrict__ out,
                                                             float* __restrict__ scores, int64_t sstride) {
    decode_q2_mfma_body<D, SCORES, ROT, false, FUSE>(pv, layer, bd, q, sm, splits, ws, out, scores, sstride, 0, 4);
}

// Other groups: heads h0 .. h0 + nh - 1 of each KV head's group.
template <int D, bool SCORES, bool ROT, bool FUSE>
__global__ __launch_bounds__(256) void decode_q2_mfma_group_kernel(PoolView pv, int layer, BatchDesc bd,
                                                                   const uint16_t* __restrict__ q, float sm,
                                                                   int splits, float* __restrict__ ws,
                                                                   float* __restrict__ out,
                                                                   float* __restrict__ scores, int64_t sstride,
                                                                   int h0, int nh) {
    decode_q2_mfma_body<D, SCORES, ROT, true, FUSE>(pv, layer, bd, q, sm, splits, ws, out, scores, sstride, h0, nh);
}

// The split kernels of a decode call; fuse: each launch also merges (out).
static hipError_t launch_decode_q2_splits(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q,
                                          float sm, int splits, float* ws, float* out, float* scores,
                                          int64_t sstride, hipStream_t s, bool rot, bool fuse) {
    dim3 grid(bd.n * pv.Hkv, splits);
    const float smk = rot ? sm / (float)pv.D : sm;  // H q . H k = D q . k
    const int Gq = pv.Hq / pv.Hkv;
    using D128 = std::integral_constant<int, 128>;
    using D256 = std::integral_constant<int, 256>;
    using T = std::true_type;
    using F = std::false_type;
    // template flags: head dim, scores, rotated, fused merge
    auto flags = [&](auto&& go) {
        auto f3 = [&](auto d, auto sc, auto r) { fuse ? go(d, sc, r, T{}) : go(d, sc, r, F{}); };
        auto f2 = [&](auto d, auto sc) { rot ? f3(d, sc, T{}) : f3(d, sc, F{}); };
        auto f1 = [&](auto d) { scores ? f2(d, T{}) : f2(d, F{}); };
        pv.D == 256 ? f1(D256{}) : f1(D128{});
    };
    if (Gq == 4) {
        flags([&](auto d, auto sc, auto r, auto fu) {
            hipLaunchKernelGGL((decode_q2_mfma_kernel<decltype(d)::value, decltype(sc)::value, decltype(r)::value,
                                                      decltype(fu)::value>),
                               grid, dim3(256), 0, s, pv, layer, bd, q, smk, splits, ws, out, scores, sstride);
        });
        return hipGetLastError();
    }
    // other groups: up to four query heads per launch (two launches for group 8)
    for (int h0 = 0; h0 < Gq; h0 += 4) {
        const int nh = Gq - h0 < 4 ? Gq - h0 : 4;
        flags([&](auto d, auto sc, auto r, auto fu) {
            hipLaunchKernelGGL((decode_q2_mfma_group_kernel<decltype(d)::value, decltype(sc)::value,
                                                            decltype(r)::value, decltype(fu)::value>),
                               grid, dim3(256), 0, s, pv, layer, bd, q, smk, splits, ws, out, scores, sstride, h0,
                               nh);
        });
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_decode_q2_partials(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                                     int splits, float* ws, float* scores, int64_t sstride, hipStream_t s, bool rot) {
    return launch_decode_q2_splits(pv, layer, bd, q, sm, splits, ws, nullptr, scores, sstride, s, rot, false);
}

hipError_t launch_decode_q2(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm, int splits,
                            float* ws, float* out, float* scores, int64_t sstride, hipStream_t s, bool rot) {
    if (splits <= FUSED_MERGE_MAX_SPLITS && pv.cnt)
        return launch_decode_q2_splits(pv, layer, bd, q, sm, splits, ws, out, scores, sstride, s, rot, true);
    const hipError_t err = launch_decode_q2_partials(pv, layer, bd, q, sm, splits, ws, scores, sstride, s, rot);
    return err != hipSuccess ? err : launch_merge_splits(bd, pv.Hq, pv.D, splits, ws, out, s);
}

}  // namespace kvq
