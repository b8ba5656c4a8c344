// Split-K decode attention over the 2-bit pool on the gfx950 matrix cores
// (GQA group 4, head_dim 128 or 256).
//
// At group 4 and 256 dims a decode step does 2 x 4 x 256 multiply-adds for
// every 144 bytes of K and V rows it reads, more than the vector ALUs can
// sustain at full HBM bandwidth, so both contractions run on
// v_mfma_scale_f32_16x16x128_f8f6f4.  Its internal sum drops low-order bits
// of products much smaller than the largest product of a group, but sums
// small-integer products exactly, so every operand is made of small
// integers:
//   * 2-bit codes c become fp4 (e2m1) nibbles whose value is c/2: a 32-bit
//     word of 16 codes spreads into two words of nibbles with one shift and
//     two masks (w & 0x33333333, (w >> 2) & 0x33333333);
//   * the bf16 query of each head becomes a 19-bit fixed-point integer
//     round(q * 2^E) (exact unless |q| < max|q| / 2^11), written as four
//     balanced radix-32 digits in -16..16 (exact in e4m3); the 16 columns of
//     the q.k product are 4 heads x 4 digits, recombined with two row
//     rotations;
//   * the softmax weights w_t = p_t * scale_t of a 128-token tile become
//     19-bit fixed-point integers relative to each head's largest weight in
//     the tile, also as four balanced digits; the 16 rows of the p.v product
//     are 4 heads x 4 digits, the instruction's per-row power-of-two scale
//     undoes the tile scale, and each digit row is weighted once at the end.
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
// in LDS.  Token t of the pair sits at
// page t/64, slot t%64.  Operand lane layouts of the instruction (fp4: lane
// group g holds k = 32g..32g+31; fp8: k = 16g..16g+15 and 64+16g..64+16g+15;
// result: lane l holds column l%16, rows 4(l/16)..+3) let the q.k product
// deliver each lane exactly the 32 tokens its p.v operand needs:
//   q.k:  A = K codes (rows = tokens), B = query digits (column 4d + h =
//         digit d of head h); row i of token group m is token
//         (m/4)*64 + 16(i/4) + 4(m%4) + i%4.
//   p.v:  A = weight digits (row 4d + h = digit d of head h),
//         B = V codes of 16 dims (dim-major rows, so k runs over tokens).
#include "decode_common.h"

namespace kvq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

constexpr int FMT_FP8 = 0;  // e4m3
constexpr int FMT_FP4 = 4;  // e2m1

__device__ __forceinline__ v4f mma_fp4_fp8(const v8i& a_fp4, const v8i& b_fp8, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp4, b_fp8, c, FMT_FP4, FMT_FP8, 0, 127, 0, 127);
}
__device__ __forceinline__ v4f mma_fp8_fp4(const v8i& a_fp8, const v8i& b_fp4, v4f c, int scale_a) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp8, b_fp4, c, FMT_FP8, FMT_FP4, 0, scale_a, 0, 127);
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}
__device__ __forceinline__ float fp8_byte(uint32_t w, int i) {
    switch (i) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
    }
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

// Sum over the four lanes j, j+4, j+8, j+12 of each 16-lane row.
__device__ __forceinline__ float row_sum4(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
    return x;
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
    uint32_t kc[8][D / 64];  // K code words of this lane's row for the eight q.k token groups
    uint4 vc[D / 32];        // V code words: 32 token slots of dims 32c + l%16 and 32c + 16 + l%16
    uint4 meta[2];           // this lane's two 16-byte chunks of the pair's metadata
};

template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& t, const uint8_t* base0, const uint8_t* base1, int l) {
    constexpr int NW = D / 64;
    const int j = l & 15, grp = l >> 4;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int slot = 16 * (j >> 2) + 4 * (m & 3) + (j & 3);
        const uint8_t* src = (m < 4 ? base0 : base1) + slot * (D / 4) + 4 * NW * grp;
        if constexpr (NW == 4) {
            const uint4 w = *reinterpret_cast<const uint4*>(src);
            t.kc[m][0] = w.x; t.kc[m][1] = w.y; t.kc[m][2] = w.z; t.kc[m][3] = w.w;
        } else {
            const uint2 w = *reinterpret_cast<const uint2*>(src);
            t.kc[m][0] = w.x; t.kc[m][1] = w.y;
        }
    }
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        t.vc[c] = *reinterpret_cast<const uint4*>((grp < 2 ? base0 : base1) + q2_vcodes_off(D) +
                                                  q2_vword_off(D, 32 * c + j, 2 * (grp & 1)));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ch = l + 64 * h, plane = ch >> 5;
        t.meta[h] = *reinterpret_cast<const uint4*>(((plane & 1) ? base1 : base0) +
                                                    (plane < 2 ? q2_kmeta_off(D) : q2_vmeta_off(D)) + (ch & 31) * 16);
    }
}

template <int D>
struct WaveState {
    v4f acc[D / 16];  // p.v sums: block b, register r = head r, lane group = weight digit
    float m_ref;      // reference max of this lane's head, in units of 1/cB
    float cbm;        // cB * m_ref (log2 units)
    float l_run;      // this lane's share of sum p
    float c_run;      // this lane's share of sum p * min_v
};

struct QConst {
    float qdig_w;  // 32^(3 - digit) of this lane's q.k column
    float cAB;     // sum(q) / (2 * 2^-E): min_k's factor in units of the digit sum
    float cB;      // log2(e) * sm * 2 * 2^-E: digit-sum units -> log2 logits
};

template <int D, bool FULL>
__device__ __forceinline__ void compute_tile(const Tile<D>& t, float2 (*meta)[PAGE], int l, const v8i* qop,
                                             const QConst& qc, WaveState<D>& st, int tok0, int ctx,
                                             float* __restrict__ srow) {
    constexpr int NC = D / 128, NB = D / 16;
    const int j = l & 15, grp = l >> 4, piece = j >> 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ch = l + 64 * h;
        *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(&meta[ch >> 5][0]) + (ch & 31) * 16) = t.meta[h];
    }
    // ---- q.k: scores in units of 1/cB ----
    float s2[8][4];
    float mt = -INFINITY;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        v4f cq = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) cq = mma_fp4_fp8(fp4_operand(t.kc[m][2 * c], t.kc[m][2 * c + 1]), qop[c], cq);
        const int pm = m >> 2, slot0 = 16 * grp + 4 * (m & 3);
        const float4 km0 = *reinterpret_cast<const float4*>(&meta[pm][slot0]);
        const float4 km1 = *reinterpret_cast<const float4*>(&meta[pm][slot0 + 2]);
        const float ks[4] = {km0.x, km0.z, km1.x, km1.z};
        const float kn[4] = {km0.y, km0.w, km1.y, km1.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s = fmaf(ks[r], row_sum4(cq[r] * qc.qdig_w), kn[r] * qc.cAB);
            if (!FULL && tok0 + pm * PAGE + slot0 + r >= ctx) s = -INFINITY;
            s2[m][r] = s;
            mt = fmaxf(mt, s);
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool need = (mt - st.m_ref) * qc.cB > RESCALE_LOG2;
    if (__ballot(need)) {
        const float m_new = need ? mt : st.m_ref;
        const float cbm_new = qc.cB * m_new;
        const float alpha = __builtin_amdgcn_exp2f(st.cbm - cbm_new);
        st.l_run *= alpha;
        st.c_run *= alpha;
        float al[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, (l & ~3) | r);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) st.acc[b][r] *= al[r];
        st.m_ref = m_new;
        st.cbm = cbm_new;
    }
    // ---- weights w = p * scale_v ----
    float wv[8][4];
    float wmax = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int pm = m >> 2, slot0 = 16 * grp + 4 * (m & 3);
        const float4 vm0 = *reinterpret_cast<const float4*>(&meta[2 + pm][slot0]);
        const float4 vm1 = *reinterpret_cast<const float4*>(&meta[2 + pm][slot0 + 2]);
        const float vs[4] = {vm0.x, vm0.z, vm1.x, vm1.z};
        const float vn[4] = {vm0.y, vm0.w, vm1.y, vm1.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s2[m][r], qc.cB, -st.cbm));
            float w;
            if (FULL) {
                w = p * vs[r];
                st.c_run = fmaf(p, vn[r], st.c_run);
            } else {
                const bool valid = tok0 + pm * PAGE + slot0 + r < ctx;
                w = valid ? p * vs[r] : 0.f;
                st.c_run += valid ? p * vn[r] : 0.f;
            }
            st.l_run += p;
            wv[m][r] = w;
            wmax = fmaxf(wmax, w);
        }
    }
    if (srow != nullptr && piece == 0) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = tok0 + (m >> 2) * PAGE + 16 * grp + 4 * (m & 3) + r;
                if (FULL || tok < ctx) srow[tok] = s2[m][r] * (qc.cB * LN2);
            }
    }
    // ---- weight digits, per-head tile scale (lane l's scale byte serves row l%16) ----
    wmax = fmaxf(wmax, __shfl_xor(wmax, 16));
    wmax = fmaxf(wmax, __shfl_xor(wmax, 32));
    const int ew = wmax > 0.f ? (int)((__float_as_uint(wmax) >> 23) & 0xFF) - 127 : 0;
    const int FW = 18 - ew;  // w * 2^FW < 2^19
    const float wscale = pow2f(FW);
    v8i wop;
#pragma unroll
    for (int m = 0; m < 8; ++m)
        wop[m] = (int)pack4_fp8(digit_of(wv[m][0], wscale, piece), digit_of(wv[m][1], wscale, piece),
                                digit_of(wv[m][2], wscale, piece), digit_of(wv[m][3], wscale, piece));
    // ---- p.v ----
#pragma unroll
    for (int c = 0; c < NB / 2; ++c) {
        st.acc[2 * c] = mma_fp8_fp4(wop, fp4_operand(t.vc[c].x, t.vc[c].y), st.acc[2 * c], 127 - FW);
        st.acc[2 * c + 1] = mma_fp8_fp4(wop, fp4_operand(t.vc[c].z, t.vc[c].w), st.acc[2 * c + 1], 127 - FW);
    }
}

template <int D>
__global__ __launch_bounds__(256) void decode_q2_mfma_kernel(PoolView pv, int layer, BatchDesc bd,
                                                             const uint16_t* __restrict__ q, float sm, int splits,
                                                             float* __restrict__ ws, float* __restrict__ out,
                                                             float* __restrict__ scores, int64_t sstride) {
    constexpr int G = 4;
    constexpr int NC = D / 128;  // k-chunks of the q.k product
    constexpr int NB = D / 16;   // 16-dim blocks of the p.v product
    const int Hkv = pv.Hkv, Hq = pv.Hq;
    const int e = blockIdx.x / Hkv, g = blockIdx.x % Hkv, sp = blockIdx.y;
    const int ctx = bd.pos[e];
    int pg0, pg1;
    split_range(ctx, splits, sp, &pg0, &pg1);
    if (pg0 >= pg1) return;

    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int j = l & 15, grp = l >> 4;
    const int hh = j & 3;  // head of this lane's q.k column and p.v row

    __shared__ __align__(16) float2 meta_s[4][4][PAGE];  // per wave: K page 0, K page 1, V page 0, V page 1
    __shared__ float o_s[4][G][D];
    __shared__ float ml_s[4][G][2];

    // ---- query operand: 19-bit fixed point per head, digit (j >> 2) of head hh ----
    const uint16_t* qrow = q + ((int64_t)e * Hq + g * G + hh) * D;
    float qv[NC][32];
    float amax = 0.f, qsum = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            const int k = fp8_k(grp, s), ga = k >> 5, n = k & 31;
            const int dim = 32 * NC * ga + 32 * c + 16 * (n >> 4) + 2 * (n & 7) + ((n >> 3) & 1);
            const float x = bf16_to_f32(qrow[dim]);
            qv[c][s] = x;
            amax = fmaxf(amax, fabsf(x));
            qsum += x;
        }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    qsum += __shfl_xor(qsum, 16);
    qsum += __shfl_xor(qsum, 32);
    const int ea = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 : 0;
    const int EQ = 18 - ea;  // |q * 2^EQ| < 2^19
    const float qscale = pow2f(EQ);
    const int qdig = j >> 2;
    QConst qc;
    qc.qdig_w = pow2f(5 * (3 - qdig));
    qc.cB = LOG2E * sm * pow2f(1 - EQ);  // sum_d q_d c_d = 2 * 2^-EQ * (digit sum)
    qc.cAB = qsum * pow2f(EQ - 1);
    v8i qop[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int v = 0; v < 8; ++v)
            qop[c][v] = (int)pack4_fp8(digit_of(qv[c][4 * v], qscale, qdig), digit_of(qv[c][4 * v + 1], qscale, qdig),
                                       digit_of(qv[c][4 * v + 2], qscale, qdig), digit_of(qv[c][4 * v + 3], qscale, qdig));

    WaveState<D> st;
#pragma unroll
    for (int b = 0; b < NB; ++b) st.acc[b] = v4f{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.cbm = -INFINITY;
    st.l_run = 0.f;
    st.c_run = 0.f;

    const int32_t* bt = pv.bt + (int64_t)bd.seq[e] * pv.bt_stride;
    const int64_t lhoff = ((int64_t)layer * Hkv + g) * pv.block_bytes;
    const int n_pages = (ctx + PAGE - 1) / PAGE;
    float* srow = scores ? scores + ((int64_t)e * Hq + g * G + hh) * sstride : nullptr;
    float2(*meta)[PAGE] = meta_s[wave];

    // ---- this wave's tiles: page pairs pg0/2 + wave + 4i, i < T ----
    const int pr_first = pg0 / 2 + wave;
    const int pr_end = (pg1 + 1) / 2;
    const int T = pr_first < pr_end ? (pr_end - pr_first + 3) / 4 : 0;
    // the last tile of the sequence may be partly past ctx; it is done on its own
    const bool last_partial = T > 0 && 2 * (pr_first + 4 * (T - 1)) * PAGE + 2 * PAGE > ctx;
    const int TF = last_partial ? T - 1 : T;  // full tiles
    auto tok0_of = [&](int t) { return 2 * (pr_first + 4 * t) * PAGE; };

    // Tiles go in chunks of 64: lane k of pid0/pid1 holds the physical ids of
    // the two pages of tile c0 + k.  Three tile buffers rotate so that two
    // tiles are in flight while one is computed; every load is issued
    // unconditionally (indices clamped to the chunk's last tile, re-read from
    // cache), so the count of loads in flight is the same on every path.
    Tile<D> ta, tb, tc;
    for (int c0 = 0; c0 < TF; c0 += 64) {
        const int Tc = min(64, TF - c0);
        int pid0 = 0, pid1 = 0;
        if (l < Tc) {
            const int pair = pr_first + 4 * (c0 + l);
            pid0 = bt[2 * pair];
            pid1 = bt[2 * pair + 1];
        }
        auto load = [&](Tile<D>& tile, int t) {
            const int tt = min(t, Tc - 1);
            load_tile<D>(tile, pv.pages + (int64_t)__builtin_amdgcn_readlane(pid0, tt) * pv.page_bytes + lhoff,
                         pv.pages + (int64_t)__builtin_amdgcn_readlane(pid1, tt) * pv.page_bytes + lhoff, l);
        };
        auto run = [&](const Tile<D>& tile, int t) {
            compute_tile<D, true>(tile, meta, l, qop, qc, st, tok0_of(c0 + t), ctx, srow);
        };
        load(ta, 0);
        load(tb, 1);
        for (int t = 0; t < Tc; t += 3) {
            load(tc, t + 2);
            __builtin_amdgcn_sched_barrier(0);
            run(ta, t);
            if (t + 1 >= Tc) break;
            load(ta, t + 3);
            __builtin_amdgcn_sched_barrier(0);
            run(tb, t + 1);
            if (t + 2 >= Tc) break;
            load(tb, t + 4);
            __builtin_amdgcn_sched_barrier(0);
            run(tc, t + 2);
        }
    }
    if (last_partial) {
        const int pair = pr_first + 4 * (T - 1);
        const int p1 = 2 * pair + 1 < n_pages ? 2 * pair + 1 : 2 * pair;
        load_tile<D>(ta, pv.pages + (int64_t)bt[2 * pair] * pv.page_bytes + lhoff,
                     pv.pages + (int64_t)bt[p1] * pv.page_bytes + lhoff, l);
        compute_tile<D, false>(ta, meta, l, qop, qc, st, tok0_of(T - 1), ctx, srow);
    }

    // ---- this wave's partial: sum weight digits (lane groups) and lanes' sums ----
    float l_run = st.l_run, c_run = st.c_run;
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    c_run += __shfl_xor(c_run, 16);
    c_run += __shfl_xor(c_run, 32);
    float cr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) cr[r] = __shfl(c_run, (l & ~3) | r);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float t[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // digit row weight 32^(3 - grp), and 2 for the code/2 fp4 values
            float v = st.acc[b][r] * pow2f(16 - 5 * grp);
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            t[r] = v + cr[r];
        }
        o_s[wave][grp][16 * b + j] = grp == 0 ? t[0] : grp == 1 ? t[1] : grp == 2 ? t[2] : t[3];
    }
    if (l < 4) {
        ml_s[wave][l][0] = st.cbm;  // log2 units
        ml_s[wave][l][1] = l_run;
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
        const int64_t row = ((int64_t)e * Hq + g * G + h) * splits + sp;
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
            const int d = l + 64 * k;
            float o = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) o += f[v] * o_s[v][h][d];
            w.o[row * D + d] = o;
        }
        if (l == 0) {
            w.ml[2 * row] = M;
            w.ml[2 * row + 1] = lsum;
        }
    }
}

hipError_t launch_decode_q2_valu(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                                 int splits, float* ws, float* out, float* scores, int64_t sstride, hipStream_t s);

hipError_t launch_decode_q2(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm, int splits,
                            float* ws, float* out, float* scores, int64_t sstride, hipStream_t s) {
    if (pv.Hq != 4 * pv.Hkv) return launch_decode_q2_valu(pv, layer, bd, q, sm, splits, ws, out, scores, sstride, s);
    dim3 grid(bd.n * pv.Hkv, splits);
    if (pv.D == 256)
        hipLaunchKernelGGL(decode_q2_mfma_kernel<256>, grid, dim3(256), 0, s, pv, layer, bd, q, sm, splits, ws, out,
                           scores, sstride);
    else
        hipLaunchKernelGGL(decode_q2_mfma_kernel<128>, grid, dim3(256), 0, s, pv, layer, bd, q, sm, splits, ws, out,
                           scores, sstride);
    const hipError_t err = hipGetLastError();
    return err != hipSuccess ? err : launch_merge_splits(bd, pv.Hq, pv.D, splits, ws, out, s);
}

}  // namespace kvq
