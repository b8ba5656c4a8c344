// Split-K decode attention over the 8-bit pool (any GQA group G <= 8,
// head_dim 128 or 256).
//
// The 8-bit format reads 268 bytes per (token, KV head) at D = 128 for 2 x G x
// 128 multiply-adds.  The dequantization is folded into the operands: K is
// scaled per channel, so the query is multiplied by the page's channel scales
// once per page (q.k^_t = sum_d (q_d s_d) c_td), and V is scaled per token,
// so the softmax weight absorbs it (sum_t p_t v^_td = sum_t (p_t s_t) c_dt).
// Scores, the online softmax and every running sum are fp32 (the two-level
// accumulation of "Half the Cache, Twice the Context", section "The cliff is
// in the accumulator"), in base-2 units inside the kernels.
//
// Three forms, one workgroup per (sequence, KV head, split) each:
//   decode_q8_mfma_kernel (D = 128, G in {1, 2, 4, 8}): both products on the
//     int8 matrix cores, pages staged in LDS by DMA;
//   decode_q8_wave_kernel (D = 256, G in {1, 2, 4}): the vector ALUs, each
//     wave its own pages and online softmax;
//   decode_q8_kernel (the other groups): the vector ALUs, the workgroup on
//     one page at a time.
// Partial (m, l, o) go to the workspace; merge_splits8_kernel or
// merge_splits_wide_kernel merges them.
#include <type_traits>

#include "decode_common.h"

namespace kvq {

constexpr bool Q8_MATRIX_CORES = true;  // the matrix-core form where it applies (else the wave-parallel VALU form)

namespace {

// four int8 codes of a word -> fp32
__device__ __forceinline__ void i8x4(uint32_t w, float* f) {
    f[0] = (float)(int8_t)(w & 0xFF);
    f[1] = (float)(int8_t)((w >> 8) & 0xFF);
    f[2] = (float)(int8_t)((w >> 16) & 0xFF);
    f[3] = (float)(int8_t)(w >> 24);
}

}  // namespace

template <int D>
struct PageQ8 {
    static constexpr int KW = D / 16;             // K code words of a lane's dim slice (D/4 bytes)
    static constexpr int VW = D == 128 ? 8 : 16;  // V code words of a thread's (dim, token range)
    uint32_t k[KW];
    uint32_t v[VW];
    float kscale;  // channel tid (tid < D)
    float vscale;  // token tid (tid < 64)
};

template <int D>
__device__ __forceinline__ void load_page_q8(PageQ8<D>& pg, const uint8_t* blk, int tid) {
    const int wave = tid >> 6, lane = tid & 63;
    const uint4* kp = reinterpret_cast<const uint4*>(blk + lane * D + wave * (D / 4));
#pragma unroll
    for (int i = 0; i < PageQ8<D>::KW / 4; ++i) {
        const uint4 w = kp[i];
        pg.k[4 * i] = w.x; pg.k[4 * i + 1] = w.y; pg.k[4 * i + 2] = w.z; pg.k[4 * i + 3] = w.w;
    }
    const int d = D == 128 ? (tid & 127) : tid;
    const int t0 = D == 128 ? 32 * (tid >> 7) : 0;
    const uint4* vp = reinterpret_cast<const uint4*>(blk + q8_vcodes_off(D) + d * PAGE + t0);
#pragma unroll
    for (int i = 0; i < PageQ8<D>::VW / 4; ++i) {
        const uint4 w = vp[i];
        pg.v[4 * i] = w.x; pg.v[4 * i + 1] = w.y; pg.v[4 * i + 2] = w.z; pg.v[4 * i + 3] = w.w;
    }
    pg.kscale = tid < D ? reinterpret_cast<const float*>(blk + q8_kscale_off(D))[tid] : 0.f;
    pg.vscale = tid < PAGE ? reinterpret_cast<const float*>(blk + q8_vscale_off(D))[tid] : 0.f;
}

// Workgroup form: 256 threads, one page of 64 tokens per step, the next page's
// bytes prefetched into registers while the current one is computed:
//   scores:  wave w takes dims [wD/4, (w+1)D/4) of token t = lane for every
//            head; the four partial dots meet in LDS;
//   softmax: wave j % 4 takes heads j;
//   p.v:     thread (d, half) takes dim d over tokens [32 half, 32 half + 32)
//            (D = 128) or all 64 tokens (D = 256) for every head.
template <int D>
__global__ __launch_bounds__(256) void decode_q8_kernel(PoolView pv, int layer, BatchDesc bd,
                                                        const uint16_t* __restrict__ q, float sm, int splits,
                                                        float* __restrict__ ws, float* __restrict__ out,
                                                        float* __restrict__ scores, int64_t sstride) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int DW = D / 4;  // dims per wave in the score phase
    const int Hkv = pv.Hkv, Hq = pv.Hq, G = Hq / Hkv;
    const int e = blockIdx.x / Hkv, g = blockIdx.x % Hkv, sp = blockIdx.y;
    const int ctx = bd.pos[e];
    int pg0, pg1;
    split_range(ctx, bd.per, sp, &pg0, &pg1);
    if (pg0 >= pg1) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    __shared__ float q_s[8][D];    // query (fp32)
    __shared__ float qk_s[8][D];   // query x this page's K channel scales
    __shared__ float part_s[4][8][PAGE];
    __shared__ float w_s[8][PAGE];
    __shared__ float vs_s[PAGE];
    __shared__ float m_s[8], l_s[8], a_s[8];

    for (int i = tid; i < G * D; i += 256) q_s[i / D][i % D] = bf16_to_f32(q[((int64_t)e * Hq + g * G) * D + i]);
    if (tid < 8) {
        m_s[tid] = -INFINITY;
        l_s[tid] = 0.f;
    }
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.f;

    const int32_t* bt = pv.bt + (int64_t)bd.seq[e] * pv.bt_stride;
    const int64_t lhoff = ((int64_t)layer * Hkv + g) * pv.block_bytes;
    auto block_of = [&](int pg) { return pv.pages + (int64_t)bt[pg] * pv.page_bytes + lhoff; };
    const float cs = sm * LOG2E;
    const int dv = D == 128 ? (tid & 127) : tid;
    const int tv0 = D == 128 ? 32 * (tid >> 7) : 0;

    PageQ8<D> cur, nxt;
    load_page_q8<D>(cur, block_of(pg0), tid);
    for (int pg = pg0; pg < pg1; ++pg) {
        if (pg + 1 < pg1) load_page_q8<D>(nxt, block_of(pg + 1), tid);
        const int n_tok = min(PAGE, ctx - pg * PAGE);
        __syncthreads();  // previous page's LDS reads are done
        if (tid < D)
            for (int j = 0; j < G; ++j) qk_s[j][tid] = q_s[j][tid] * cur.kscale;
        if (tid < PAGE) vs_s[tid] = cur.vscale;
        __syncthreads();
        // ---- scores: partial dot over this wave's dims, every head ----
        {
            float kf[DW];
#pragma unroll
            for (int i = 0; i < PageQ8<D>::KW; ++i) i8x4(cur.k[i], &kf[4 * i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j >= G) break;
                const float* qr = &qk_s[j][wave * DW];
                float acc = 0.f;
#pragma unroll
                for (int d = 0; d < DW; ++d) acc = fmaf(qr[d], kf[d], acc);
                part_s[wave][j][lane] = acc;
            }
        }
        __syncthreads();
        // ---- online softmax: wave j % 4 takes head j ----
        for (int j = wave; j < G; j += 4) {
            const float raw = part_s[0][j][lane] + part_s[1][j][lane] + part_s[2][j][lane] + part_s[3][j][lane];
            const bool valid = lane < n_tok;
            if (scores && valid) scores[((int64_t)e * Hq + g * G + j) * sstride + pg * PAGE + lane] = sm * raw;
            const float s = valid ? raw * cs : -INFINITY;
            const float m_old = m_s[j];
            const float m_new = fmaxf(m_old, wave_max(s));
            const float p = valid ? exp2f(s - m_new) : 0.f;
            w_s[j][lane] = valid ? p * vs_s[lane] : 0.f;  // slots past ctx may hold any bytes
            const float psum = wave_sum(p);
            if (lane == 0) {
                const float alpha = exp2f(m_old - m_new);
                a_s[j] = alpha;
                m_s[j] = m_new;
                l_s[j] = l_s[j] * alpha + psum;
            }
        }
        __syncthreads();
        // ---- p.v: thread (dim dv, tokens tv0..) ----
        {
            float vf[4 * PageQ8<D>::VW];
#pragma unroll
            for (int i = 0; i < PageQ8<D>::VW; ++i) i8x4(cur.v[i], &vf[4 * i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j >= G) break;
                const float* wr = &w_s[j][tv0];
                float acc = o[j] * a_s[j];
#pragma unroll
                for (int t = 0; t < 4 * PageQ8<D>::VW; ++t) acc = fmaf(wr[t], vf[t], acc);
                o[j] = acc;
            }
        }
        cur = nxt;
    }

    // ---- this split's partial: (m, l) per head, o per (head, dim) ----
    DecodeWs w(ws, bd.n, Hq, D, splits);
    if constexpr (D == 128) {
        // the two token halves of dim dv meet in LDS
        __syncthreads();
        if (tid >= 128)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < G) part_s[j >> 1][(j & 1) * 4 + (dv >> 5)][dv & 31] = o[j];
        __syncthreads();
        if (tid < 128)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j >= G) break;
                const int64_t r = ((int64_t)e * Hq + g * G + j) * splits + sp;
                w.o[r * D + dv] = o[j] + part_s[j >> 1][(j & 1) * 4 + (dv >> 5)][dv & 31];
            }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= G) break;
            const int64_t r = ((int64_t)e * Hq + g * G + j) * splits + sp;
            w.o[r * D + dv] = o[j];
        }
    }
    if (tid < G) {
        const int64_t r = ((int64_t)e * Hq + g * G + tid) * splits + sp;
        w.ml[2 * r] = m_s[tid];
        w.ml[2 * r + 1] = l_s[tid];
    }
}

// Wave-parallel form for G in {1, 2, 4, 8}: the four waves of a workgroup
// take every fourth page of the split and run their own online softmax, with
// no workgroup barrier until the final combine, so that many workgroups per
// compute unit keep loads in flight while others compute.  Per page, lane t
// holds token t's K row (D codes) and dims DL*t .. DL*t + DL-1 of V (64
// tokens each):
//   scores:  s_j(t) = sum_d (q_jd kscale_d) c_td, the scaled query staged in
//            the wave's LDS and read as broadcasts;
//   softmax: wave-wide max and sum per head, weights p_t vscale_t to LDS;
//   p.v:     o_j,d += sum_t w_j(t) c_dt over the page's 64 tokens.
// (the variant that also stores the raw logits takes one workgroup a compute
// unit: it spills at two)
template <int D, int G, bool SCORES>
__global__ __launch_bounds__(256, SCORES ? 1 : 2) void decode_q8_wave_kernel(PoolView pv, int layer, BatchDesc bd,
                                                             const uint16_t* __restrict__ q, float sm, int splits,
                                                             float* __restrict__ ws, float* __restrict__ out,
                                                             float* __restrict__ scores, int64_t sstride) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int DL = D / 64;  // V dims of a lane
    const int Hkv = pv.Hkv, Hq = pv.Hq;
    const int e = blockIdx.x / Hkv, g = blockIdx.x % Hkv, sp = blockIdx.y;
    const int ctx = bd.pos[e];
    int pg0, pg1;
    split_range(ctx, bd.per, sp, &pg0, &pg1);
    if (pg0 >= pg1) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    __shared__ __align__(16) float qk_s[4][G][D];    // per wave: query x the page's channel scales; partial o at the end
    __shared__ __align__(16) float w_s[4][G][PAGE];  // per wave: the page's weights
    __shared__ float ml_s[4][G][2];

    // this lane's query dims (the ones whose channel scales it loads)
    float qv[G][DL];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int i = 0; i < DL; ++i) qv[j][i] = bf16_to_f32(q[((int64_t)e * Hq + g * G + j) * D + DL * lane + i]);
    float m[G], l[G], o[G][DL];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int i = 0; i < DL; ++i) o[j][i] = 0.f;
    }
    const int32_t* bt = pv.bt + (int64_t)bd.seq[e] * pv.bt_stride;
    const int64_t lhoff = ((int64_t)layer * Hkv + g) * pv.block_bytes;
    const float cs = sm * LOG2E;

    for (int pg = pg0 + wave; pg < pg1; pg += 4) {
        const uint8_t* blk = pv.pages + (int64_t)bt[pg] * pv.page_bytes + lhoff;
        uint4 kc[D / 16];  // K codes of token `lane`
#pragma unroll
        for (int i = 0; i < D / 16; ++i) kc[i] = reinterpret_cast<const uint4*>(blk + lane * D)[i];
        uint4 vc[DL][4];  // V codes of dims DL*lane + dd, tokens 0..63
#pragma unroll
        for (int dd = 0; dd < DL; ++dd)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vc[dd][i] = reinterpret_cast<const uint4*>(blk + q8_vcodes_off(D) + (DL * lane + dd) * PAGE)[i];
        float ksc[DL];
#pragma unroll
        for (int dd = 0; dd < DL; ++dd) ksc[dd] = reinterpret_cast<const float*>(blk + q8_kscale_off(D))[DL * lane + dd];
        const float vsc = reinterpret_cast<const float*>(blk + q8_vscale_off(D))[lane];
        const int n_tok = min(PAGE, ctx - pg * PAGE);
        const bool valid = lane < n_tok;

        // ---- scaled query for this page (the wave's LDS is read in order) ----
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int dd = 0; dd < DL; ++dd) qk_s[wave][j][DL * lane + dd] = qv[j][dd] * ksc[dd];

        // ---- scores of token `lane` ----
        float s[G];
#pragma unroll
        for (int j = 0; j < G; ++j) s[j] = 0.f;
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {  // code word c: dims 4c .. 4c + 3
            const uint4 kw = kc[c >> 2];
            const uint32_t wd = (c & 3) == 0 ? kw.x : (c & 3) == 1 ? kw.y : (c & 3) == 2 ? kw.z : kw.w;
            float kf[4];
            i8x4(wd, kf);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float4 qq = *reinterpret_cast<const float4*>(&qk_s[wave][j][4 * c]);
                s[j] = fmaf(qq.x, kf[0], s[j]);
                s[j] = fmaf(qq.y, kf[1], s[j]);
                s[j] = fmaf(qq.z, kf[2], s[j]);
                s[j] = fmaf(qq.w, kf[3], s[j]);
            }
            // bound the scheduling window: the broadcasts of 16 dims at a time
            if ((c & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        // ---- online softmax per head; slots past ctx weigh nothing (their bytes may be anything) ----
        if constexpr (SCORES) {  // a variant of its own: the branch costs the other variant registers
            if (valid) {
                float* srow = scores + ((int64_t)e * Hq + g * G) * sstride + pg * PAGE + lane;
#pragma unroll
                for (int j = 0; j < G; ++j) srow[j * sstride] = sm * s[j];
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float x = valid ? s[j] * cs : -INFINITY;
            const float m_new = fmaxf(m[j], wave_max(x));  // finite: every page of the split holds a token
            const float alpha = __builtin_amdgcn_exp2f(m[j] - m_new);
            const float p = valid ? __builtin_amdgcn_exp2f(x - m_new) : 0.f;
            l[j] = l[j] * alpha + wave_sum(p);
            m[j] = m_new;
            w_s[wave][j][lane] = valid ? p * vsc : 0.f;
#pragma unroll
            for (int dd = 0; dd < DL; ++dd) o[j][dd] *= alpha;
        }
        // ---- p.v over the page's tokens, four at a time ----
#pragma unroll
        for (int t4 = 0; t4 < PAGE / 4; ++t4) {
            float vf[DL][4];
#pragma unroll
            for (int dd = 0; dd < DL; ++dd) {
                const uint4 vw = vc[dd][t4 >> 2];
                const uint32_t wd = (t4 & 3) == 0 ? vw.x : (t4 & 3) == 1 ? vw.y : (t4 & 3) == 2 ? vw.z : vw.w;
                i8x4(wd, vf[dd]);
            }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float4 ww = *reinterpret_cast<const float4*>(&w_s[wave][j][4 * t4]);
#pragma unroll
                for (int dd = 0; dd < DL; ++dd) {
                    o[j][dd] = fmaf(ww.x, vf[dd][0], o[j][dd]);
                    o[j][dd] = fmaf(ww.y, vf[dd][1], o[j][dd]);
                    o[j][dd] = fmaf(ww.z, vf[dd][2], o[j][dd]);
                    o[j][dd] = fmaf(ww.w, vf[dd][3], o[j][dd]);
                }
            }
            if ((t4 & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- combine the four waves (a wave without pages holds m = -inf, l = 0, o = 0) ----
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int dd = 0; dd < DL; ++dd) qk_s[wave][j][DL * lane + dd] = o[j][dd];
        if (lane == 0) {
            ml_s[wave][j][0] = m[j];
            ml_s[wave][j][1] = l[j];
        }
    }
    __syncthreads();
    DecodeWs w(ws, bd.n, Hq, D, splits);
    for (int idx = tid; idx < G * D; idx += 256) {
        const int j = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) M = fmaxf(M, ml_s[v][j][0]);
        float acc = 0.f, L = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float f = __builtin_amdgcn_exp2f(ml_s[v][j][0] - M);  // 0 for a wave without pages
            acc += f * qk_s[v][j][d];
            L += f * ml_s[v][j][1];
        }
        const int64_t r = ((int64_t)e * Hq + g * G + j) * splits + sp;
        w.o[r * D + d] = acc;
        if (d == 0) {
            w.ml[2 * r] = M;
            w.ml[2 * r + 1] = L;
        }
    }
}

// Matrix-core form for G in {1, 2, 4, 8} at 128 dims, on the int8 products
// (v_mfma_i32_16x16x64_i8).  The codes -127..127 enter as they are stored.
// The query times the page's channel scales, and the weights p_t vscale_t,
// enter as three balanced radix-128 digits each: for a row (a head's 128
// scaled query dims, or a head's 64 weights of the page) with largest
// magnitude in [2^k, 2^(k+1)), e = k - 5 and n = rint(x 2^(14 - e)) (|n| <
// 2^20) = 16384 d0 + 128 d1 + d2 with d1, d2 in -64..63 and |d0| <= 64, so x
// is within 2^(e - 15) <= 2^-20 max|x| of 2^(e - 14) n.  One fused
// multiply-add, x 2^(14 - e) + (2^23 + 3,153,984), leaves n + 3,153,984 =
// (d0 + 192) 128^2 + (d1 + 64) 128 + (d2 + 64) in the low mantissa bits
// (rounded to nearest even), so each digit is one bit-field extract and one
// subtraction.  Row 4j + i of an operand is digit i of head j (row 4j + 3
// zero), four heads a 16-row block; the int32 products are exact and are
// combined in fp32 as 2^(e - 14) (16384 A0 + 128 A1 + A2).  The W waves of a
// workgroup take every W-th page, each through its own LDS slot: the page's
// block arrives there by DMA while the wave computes the page before, whose
// operands it has already read from the slot into registers.  Per page, wave
// and block of four heads:
//   S^T = Q~ K^T for each block of 16 tokens: A = the query digit rows, B = K
//         codes (lane l: token 16tb + l%16, 16 consecutive dims, two k-steps
//         of 64), so lane group g ends with the three digit products of head
//         g for the lane's token;
//   softmax per head over the 64 tokens in the 16 lanes of its group;
//   O += W~ V for each block of 16 dims: A = the weight digit rows (through
//         the wave's LDS), B = V codes (lane l: dim 16db + l%16, 16 consecutive
//         tokens, one k-step); lane group g gets head g's three digit products
//         for the lane's dim, the same head as its softmax, so the rescale and
//         the weights' scale are local.
// The sum over dims and over tokens is order-free, so each k-step takes the
// dims (tokens) that one 16-byte read per lane delivers.  Up to group 4 a
// workgroup has four waves and two share a compute unit, so that one streams
// pages while the other combines its waves and ends; the host picks the split
// count that fills those slots in one round.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ i32x4_t mma_i8(const uint4& a, const uint4& b, i32x4_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a), __builtin_bit_cast(i32x4_t, b), c, 0,
                                                  0, 0);
}
// 2^23 + 64 (1 + 128 + 128^2) + 128^3: x 2^s + Q8_DIGIT_BIAS, rounded to an
// integer in [2^23, 2^24), holds rint(x 2^s) + 3,153,984 in its low 23 bits
constexpr float Q8_DIGIT_BIAS = 11542592.0f;
// 2^e for a normal result, and the unbiased exponent field of x
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }
__device__ __forceinline__ int exponent_of(float x) { return (int)((__float_as_uint(x) >> 23) & 0xFF) - 127; }
// the scale exponent e of a row whose largest magnitude is amax (see above),
// kept where 2^(14 - e) and 2^(e - 14) are normal floats
__device__ __forceinline__ int q8_digit_exp(float amax) {
    return amax > 0.f ? max(exponent_of(amax) - 5, -112) : 0;
}
// digit i (0: most significant) of the biased integer in the low bits of y
__device__ __forceinline__ int q8_digit(float y, int i) {
    const uint32_t u = __float_as_uint(y);
    return i == 0 ? (int)((u >> 14) & 511u) - 192 : (int)((u >> (7 * (2 - i))) & 127u) - 64;
}
// four digits -> their two's-complement bytes in one word
__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d) {
    const uint32_t lo = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0c0c0400u);  // a.b0, b.b0
    const uint32_t hi = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x04000c0cu);  // c.b0, d.b0 in bytes 2, 3
    return lo | hi;
}
// the fp32 value of a digit row triple: 16384 A0 + 128 A1 + A2
__device__ __forceinline__ float q8_digits_value(const i32x4_t& a) {
    return fmaf((float)a[0], 16384.0f, fmaf((float)a[1], 128.0f, (float)a[2]));
}
// Max / sum over each 16-lane row with DPP: quad butterflies, then the row
// rotated by 4 and by 8 (every lane ends with the row's result).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1, 0, 3, 2]
    v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2, 3, 0, 1]
    v = fmaxf(v, dpp_f<0x124>(v));  // row_ror 4
    return fmaxf(v, dpp_f<0x128>(v));  // row_ror 8
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x124>(v);
    return v + dpp_f<0x128>(v);
}

}  // namespace

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t q8_lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// One (layer, KV head) block of an 8-bit page at 128 dims (17,152 bytes) copied
// to LDS at `lds` by one wave with DMA loads (global -> LDS, no registers held
// while they are in flight): lane l moves bytes 16 l + 1024 i, sixteen whole
// pieces in groups of four (the instruction's immediate offset applies to both
// addresses and stays below 4,096), then the last 768 bytes by lanes 0 .. 47.
// The loads are issued in inline asm so that the compiler sees no LDS write in
// flight (it would otherwise wait for the DMA before every LDS read); the
// kernel places the waits.  It first waits for every earlier LDS read of the
// wave to return, since the slot may be the one just read.  M0 is saved and
// restored.
constexpr int Q8_BLOCK_128 = (int)q8_block_bytes(128);
static_assert(Q8_BLOCK_128 == 16 * 1024 + 768, "sixteen whole KiB and 768 bytes");
__device__ __forceinline__ void q8_dma_block(const uint8_t* base_any, uint32_t v0, uint32_t lds, int lane) {
    // the base address is wave-uniform; scalar registers say so to the compiler
    const uint64_t b64 = (uint64_t)(uintptr_t)base_any;
    const uint8_t* base = (const uint8_t*)(uintptr_t)(
        ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64));
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
        const uint32_t vv = v0 + 4096 * gq, ll = __builtin_amdgcn_readfirstlane(lds + 4096 * gq);
        uint32_t saved;
        asm volatile(
            "s_waitcnt lgkmcnt(0)\n\t"
            "s_mov_b32 %[sv], m0\n\t"
            "s_mov_b32 m0, %[l0]\n\t"
            "global_load_lds_dwordx4 %[v0], %[b] nt\n\t"
            "global_load_lds_dwordx4 %[v0], %[b] offset:1024 nt\n\t"
            "global_load_lds_dwordx4 %[v0], %[b] offset:2048 nt\n\t"
            "global_load_lds_dwordx4 %[v0], %[b] offset:3072 nt\n\t"
            "s_mov_b32 m0, %[sv]"
            : [sv] "=&s"(saved)
            : [b] "s"(base), [v0] "v"(vv), [l0] "s"(ll)
            : "memory");
    }
    if (lane < 48) {
        const uint32_t vv = v0 + 16384, ll = __builtin_amdgcn_readfirstlane(lds + 16384);
        uint32_t saved;
        asm volatile(
            "s_waitcnt lgkmcnt(0)\n\t"
            "s_mov_b32 %[sv], m0\n\t"
            "s_mov_b32 m0, %[l0]\n\t"
            "global_load_lds_dwordx4 %[v0], %[b] nt\n\t"
            "s_mov_b32 m0, %[sv]"
            : [sv] "=&s"(saved)
            : [b] "s"(base), [v0] "v"(vv), [l0] "s"(ll)
            : "memory");
    }
}

// Waves a workgroup, one page slot of LDS each: four up to group 4, so that
// two workgroups share a compute unit's LDS (one streams while the other
// finishes); eight at group 8, whose query rows and weights take more.
constexpr int Q8_WAVES(int G) { return G <= 4 ? 4 : 8; }


template <int D, int G, bool SCORES>
__global__ __launch_bounds__(64 * Q8_WAVES(G), G <= 4 ? 2 : 1) void decode_q8_mfma_kernel(PoolView pv, int layer, BatchDesc bd,
                                                                const uint16_t* __restrict__ q, float sm, int splits,
                                                                float* __restrict__ ws, float* __restrict__ out,
                                                                float* __restrict__ scores, int64_t sstride) {
    static_assert(D == 128, "the 8-bit matrix-core form runs at 128 dims");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "groups 1, 2, 4, 8");
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int NRB = (G + 3) / 4;  // 16-row blocks of four heads
    constexpr int HPB = G < 4 ? G : 4;  // heads of a block
    constexpr int NM = D / 64;   // 64-dim k-steps of q.k
    constexpr int NDB = D / 16;  // 16-dim blocks of p.v
    constexpr int WROW = PAGE + 16;  // padded weight digit row, bytes
    constexpr int W = Q8_WAVES(G), BLK = Q8_BLOCK_128;
    const int Hkv = pv.Hkv, Hq = pv.Hq;
    const int e = blockIdx.x / Hkv, g = blockIdx.x % Hkv, sp = blockIdx.y;
    const int ctx = bd.pos[e];
    int pg0, pg1;
    split_range(ctx, bd.per, sp, &pg0, &pg1);
    if (pg0 >= pg1) return;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;

    __shared__ __align__(16) uint8_t slots[W][BLK];           // per wave: one page's block, as stored
    __shared__ __align__(16) int8_t w_s[W][NRB][16][WROW];    // per wave: weight digit rows 4j + i over the page's tokens
    __shared__ float ml_s[W][G][2];
    __shared__ __align__(16) float q_s[G][D];  // the group's query rows, fp32
    static_assert(W * BLK + W * NRB * 16 * WROW + W * G * 2 * 4 + G * D * 4 <= (G <= 4 ? 80 : 160) * 1024,
                  "the workgroups of a compute unit fit its LDS");
    static_assert(W * G * D * 4 <= W * BLK, "the waves' partial outputs fit the page slots");

    // every weight digit row starts at zero: rows 4j + 3 and the rows of heads
    // past the group stay so
    for (int i = lane; i < NRB * 16 * WROW / 4; i += 64) reinterpret_cast<uint32_t*>(&w_s[wave][0][0][0])[i] = 0u;

    // this lane's query operand row in block rb: digit ad of head 4 rb + aj
    const int aj = col >> 2, ad = col & 3;
    const bool arow = aj < HPB && ad < 3;
    // its digit as a bit field of the biased integer: offset, width, bias
    const uint32_t a_off = ad == 0 ? 14u : 7u * (2u - (uint32_t)min(ad, 2)), a_wid = ad == 0 ? 9u : 7u;
    const int a_bias = ad == 0 ? 192 : 64;
    for (int i = tid; i < G * D; i += 64 * W) q_s[i / D][i % D] = bf16_to_f32(q[((int64_t)e * Hq + g * G) * D + i]);
    __syncthreads();

    float o[NRB][NDB];  // head 4 rb + grp, dim 16 db + col
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[rb][db] = 0.f;
    float m_run[NRB], l_run[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
    }
    const float cs = sm * LOG2E;
    // page ids through the constant address space (scalar loads): the DMA takes
    // its base address from scalar registers
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(pv.bt + (int64_t)bd.seq[e] * pv.bt_stride);
    const int64_t lhoff = ((int64_t)layer * Hkv + g) * pv.block_bytes;
    const uint32_t slot = __builtin_amdgcn_readfirstlane(q8_lds_addr(slots[wave]));
    auto issue = [&](int pg) { q8_dma_block(pv.pages + (int64_t)bt[pg] * pv.page_bytes + lhoff, 16 * lane, slot, lane); };
    typedef uint32_t lds_u4 __attribute__((ext_vector_type(4)));
    typedef float lds_f4 __attribute__((ext_vector_type(4)));
    auto lds_u4_at = [&](uint32_t a) {
        const lds_u4 w = *reinterpret_cast<const __attribute__((address_space(3))) lds_u4*>((uintptr_t)a);
        return make_uint4(w.x, w.y, w.z, w.w);
    };
    auto lds_f4_at = [&](uint32_t a) {
        const lds_f4 w = *reinterpret_cast<const __attribute__((address_space(3))) lds_f4*>((uintptr_t)a);
        return make_float4(w.x, w.y, w.z, w.w);
    };
    auto lds_f_at = [&](uint32_t a) { return *reinterpret_cast<const __attribute__((address_space(3))) float*>((uintptr_t)a); };

    // wave w takes pages pg0 + w + W k; page k + 1's DMA is in flight while page k is computed
    if (pg0 + wave < pg1) issue(pg0 + wave);
    for (int pg = pg0 + wave; pg < pg1; pg += W) {
        // every outstanding load: the page's DMA (and with scores the score stores)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        uint4 kraw[4][NM];  // token 16tb + col, dims 64m + 16grp .. +15
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int m = 0; m < NM; ++m) kraw[tb][m] = lds_u4_at(slot + (16 * tb + col) * D + 64 * m + 16 * grp);
        uint4 vraw[NDB];  // dim 16db + col, tokens 16grp .. +15
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            vraw[db] = lds_u4_at(slot + (uint32_t)q8_vcodes_off(D) + (16 * db + col) * PAGE + 16 * grp);
        float vsc[4];  // scale of token 16tb + col
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) vsc[tb] = lds_f_at(slot + (uint32_t)q8_vscale_off(D) + 4 * (16 * tb + col));
        float4 ksc[NM][4];  // channel scales of dims 64m + 16grp + 4c4 .. +3
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                ksc[m][c4] = lds_f4_at(slot + (uint32_t)q8_kscale_off(D) + 4 * (64 * m + 16 * grp + 4 * c4));
        if (pg + W < pg1) issue(pg + W);
        const int n_tok = min(PAGE, ctx - pg * PAGE);

#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            // ---- A: digit ad of the query row of head 4 rb + aj times the channel scales ----
            const float* qrow = &q_s[arow ? 4 * rb + aj : 0][0];
            float x[NM][16];
            float amax = 0.f;
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const float4 k4 = ksc[m][c4];
                    const float4 q4 = *reinterpret_cast<const float4*>(qrow + 64 * m + 16 * grp + 4 * c4);
                    x[m][4 * c4] = q4.x * k4.x;
                    x[m][4 * c4 + 1] = q4.y * k4.y;
                    x[m][4 * c4 + 2] = q4.z * k4.z;
                    x[m][4 * c4 + 3] = q4.w * k4.w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(x[m][4 * c4 + i]));
                }
            // the head's 128 dims are spread over the four lane groups
            amax = fmaxf(amax, __shfl_xor(amax, 16));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const int ea = q8_digit_exp(amax);
            const float amul = pow2f(14 - ea);
            uint4 qa[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                uint32_t wv[4];
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                    int d[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float y = fmaf(x[m][4 * w4 + i], amul, Q8_DIGIT_BIAS);
                        d[i] = (int)__builtin_amdgcn_ubfe(__float_as_uint(y), a_off, a_wid) - a_bias;
                    }
                    wv[w4] = arow ? pack_i8x4(d[0], d[1], d[2], d[3]) : 0u;
                }
                qa[m] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
            // the score scale of head 4 rb + grp (the q.k result rows of lane group grp)
            const float qs = pow2f(__shfl(ea, 4 * grp) - 14);

            // ---- S^T: rows 4grp + i = digit i of head 4 rb + grp, column = token 16tb + col ----
            float sv[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                i32x4_t st = {0, 0, 0, 0};
#pragma unroll
                for (int m = 0; m < NM; ++m) st = mma_i8(qa[m], kraw[tb][m], st);
                sv[tb] = qs * q8_digits_value(st);  // the raw logit over sm
            }
            const int j = 4 * rb + grp;
            const bool live = grp < HPB;
            if constexpr (SCORES) {  // raw logits, stored apart from the softmax
                float* srow = scores + ((int64_t)e * Hq + g * G + min(j, G - 1)) * sstride + pg * PAGE + col;
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    if (live && 16 * tb + col < n_tok) srow[16 * tb] = sm * sv[tb];
            }
            // ---- online softmax of head j over the page's tokens, and the weight digits ----
            float mt = -INFINITY;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const bool valid = 16 * tb + col < n_tok;
                sv[tb] = valid && live ? sv[tb] * cs : -INFINITY;
                mt = fmaxf(mt, sv[tb]);
            }
            const float m_new = fmaxf(m_run[rb], row_max16(mt));
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
            float psum = 0.f, wgt[4], wmax = 0.f;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                // slots past ctx weigh nothing (their codes and scales may be any bytes)
                const float p = sv[tb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb] - m_new);
                psum += p;
                wgt[tb] = p != 0.f ? p * vsc[tb] : 0.f;
                wmax = fmaxf(wmax, wgt[tb]);
            }
            l_run[rb] = l_run[rb] * alpha + row_sum16(psum);
            m_run[rb] = m_new;
            const int ew = q8_digit_exp(row_max16(wmax));
            const float wmul = pow2f(14 - ew), wsc = pow2f(ew - 14);
            if (live) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const float y = fmaf(wgt[tb], wmul, Q8_DIGIT_BIAS);
                    w_s[wave][rb][4 * grp][16 * tb + col] = (int8_t)q8_digit(y, 0);
                    w_s[wave][rb][4 * grp + 1][16 * tb + col] = (int8_t)q8_digit(y, 1);
                    w_s[wave][rb][4 * grp + 2][16 * tb + col] = (int8_t)q8_digit(y, 2);
                }
            }
            // ---- O += W~ V: A = weight digit row col, tokens 16grp .. +15 (the wave's LDS is read in order) ----
            const uint4 wa = *reinterpret_cast<const uint4*>(&w_s[wave][rb][col][16 * grp]);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const i32x4_t pv4 = mma_i8(wa, vraw[db], i32x4_t{0, 0, 0, 0});
                o[rb][db] = fmaf(o[rb][db], alpha, wsc * q8_digits_value(pv4));
            }
        }
    }

    // ---- combine the waves (a wave without pages holds m = -inf, l = 0, o = 0) ----
    // the partial outputs reuse the page slots once every wave is past its last page
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    float(*o_s)[G][D] = reinterpret_cast<float(*)[G][D]>(&slots[0][0]);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const int j = 4 * rb + grp;
        if (grp < HPB) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) o_s[wave][j][16 * db + col] = o[rb][db];
            if (col == 0) {
                ml_s[wave][j][0] = m_run[rb];
                ml_s[wave][j][1] = l_run[rb];
            }
        }
    }
    __syncthreads();
    DecodeWs w(ws, bd.n, Hq, D, splits);
    for (int idx = tid; idx < G * D; idx += 64 * W) {
        const int j = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < W; ++v) M = fmaxf(M, ml_s[v][j][0]);
        float accum = 0.f, L = 0.f;
#pragma unroll
        for (int v = 0; v < W; ++v) {
            const float f = ml_s[v][j][0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml_s[v][j][0] - M);
            accum += f * o_s[v][j][d];
            L += f * ml_s[v][j][1];
        }
        const int64_t r = ((int64_t)e * Hq + g * G + j) * splits + sp;
        w.o[r * D + d] = accum;
        if (d == 0) {
            w.ml[2 * r] = M;
            w.ml[2 * r + 1] = L;
        }
    }
}

hipError_t launch_decode_q8(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                            int splits, float* ws, float* out, float* scores, int64_t sstride, hipStream_t s) {
    dim3 grid(bd.n * pv.Hkv, splits);
    const int G = pv.Hq / pv.Hkv;
    auto go = [&](auto kernel, int threads = 256) {
        hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, pv, layer, bd, q, sm, splits, ws, out, scores, sstride);
    };
    auto wave_form = [&](auto d_tag, auto g_tag) {
        constexpr int DD = decltype(d_tag)::value, GG = decltype(g_tag)::value;
        if constexpr (Q8_MATRIX_CORES && DD == 128)  // at 256 dims its registers spill: the VALU form runs
            scores ? go(decode_q8_mfma_kernel<DD, GG, true>, 64 * Q8_WAVES(GG))
                   : go(decode_q8_mfma_kernel<DD, GG, false>, 64 * Q8_WAVES(GG));
        else
            scores ? go(decode_q8_wave_kernel<DD, GG, true>) : go(decode_q8_wave_kernel<DD, GG, false>);
    };
    using D128 = std::integral_constant<int, 128>;
    using D256 = std::integral_constant<int, 256>;
    if (pv.D == 128 && G == 4)
        wave_form(D128{}, std::integral_constant<int, 4>{});
    else if (pv.D == 128 && G == 8)
        wave_form(D128{}, std::integral_constant<int, 8>{});
    else if (pv.D == 128 && G == 2)
        wave_form(D128{}, std::integral_constant<int, 2>{});
    else if (pv.D == 128 && G == 1)
        wave_form(D128{}, std::integral_constant<int, 1>{});
    else if (pv.D == 256 && G == 4)
        wave_form(D256{}, std::integral_constant<int, 4>{});
    else if (pv.D == 256 && G == 2)
        wave_form(D256{}, std::integral_constant<int, 2>{});
    else if (pv.D == 256 && G == 1)
        wave_form(D256{}, std::integral_constant<int, 1>{});
    else if (pv.D == 256)
        go(decode_q8_kernel<256>);
    else
        go(decode_q8_kernel<128>);
    const hipError_t err = hipGetLastError();
    return err != hipSuccess ? err : launch_merge_splits(bd, pv.Hq, pv.D, splits, ws, out, s);
}

}  // namespace kvq
