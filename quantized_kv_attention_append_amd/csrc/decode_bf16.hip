// Split-K decode attention over the bf16 pool: the exact cache that the
// compressed formats are priced against ("KV at 9 KB a token", section "The
// numbers": the decode price of hq against BF16), read through the same block
// tables and merged by the same split merge.
//
// A (layer, KV head) block of a page holds K token-major (row t: D bf16 at
// 2Dt) and V dim-major (row d: 64 bf16 at 128D + 128d).  Both contractions
// run on v_mfma_f32_16x16x32_bf16 with the stored values as exact operands:
//   S^T = Q K^T per block of 16 tokens: A = the query rows (row 2j holds head
//         j, rows 2j + 1 are zero, so that a lane group's rows are the heads
//         of its softmax), B = K (lane l: token 16tb + l%16, 8 dims a k-step);
//   softmax per head over the page's 64 tokens in the 16 lanes of its group;
//   O += W~ V per block of 16 dims: A = the weight rows 2j + h (the weight
//         rounded to bf16, then the rounded residual, through the wave's LDS),
//         B = V (lane l: dim 16db + l%16, 8 tokens a k-step).
// Every sum is fp32 (the two-level accumulation of "Half the Cache, Twice the
// Context", section "The cliff is in the accumulator"), scores and maxima in
// base-2 units.  The four waves of a workgroup take every fourth page of the
// split, each with its own online softmax, and combine in LDS at the end; the
// partials go to the workspace for the split merge kernels.
#include <type_traits>

#include "decode_common.h"

namespace kvq {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}
// one value as its bf16 rounding (low half) and the rounded residual (high half)
__device__ __forceinline__ uint32_t hi_lo(float x) {
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x, 0.f}, bf16x2_t)) & 0xFFFFu;
    const float r = x - __uint_as_float(hi << 16);  // exact
    const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){r, 0.f}, bf16x2_t));
    return hi | (lo << 16);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// max / sum over a 16-lane row: quad butterflies, then rotations by 4 and 8
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x124>(v));
    return fmaxf(v, dpp<0x128>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x124>(v);
    return v + dpp<0x128>(v);
}

}  // namespace

// TB: 16-token blocks a wave takes per step (4: a whole page, loads of
// 64 KB a wave at D = 256; 2: half a page, few enough registers for two
// waves per SIMD).
template <int D, int G, bool SCORES, int TB>
__global__ __launch_bounds__(256, TB == 2 ? 2 : 1) void decode_bf16_kernel(PoolView pv, int layer, BatchDesc bd,
                                                          const uint16_t* __restrict__ q, float sm, int splits,
                                                          float* __restrict__ ws, float* __restrict__ scores,
                                                          int64_t sstride) {
    static_assert(2 * G <= 16, "two rows per head in a 16-row block");
    static_assert(TB == 2 || TB == 4, "half or whole pages");
    constexpr int KS = TB / 2;  // 32-token k-steps of the p.v product per step
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int NM = D / 64;      // 64-dim slices of a K row (two k-steps each)
    constexpr int NDB = D / 16;     // 16-dim blocks of the p.v product
    constexpr int WROW = PAGE + 8;  // padded weight row, bf16 elements
    const int Hkv = pv.Hkv, Hq = pv.Hq;
    const int e = blockIdx.x / Hkv, g = blockIdx.x % Hkv, sp = blockIdx.y;
    const int ctx = bd.pos[e];
    int pg0, pg1;
    split_range(ctx, bd.per, sp, &pg0, &pg1);
    if (pg0 >= pg1) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;

    __shared__ __align__(16) uint16_t w_s[4][16][WROW];  // per wave: weight rows 2j + h over the page's tokens
    __shared__ __align__(16) float o_s[4][G][D];
    __shared__ float ml_s[4][G][2];

    // rows 2G.. of the weight operand stay zero
    for (int i = lane; i < 16 * WROW; i += 64)
        if (i / WROW >= 2 * G) w_s[wave][i / WROW][i % WROW] = 0;

    // A operand of S^T: row col = head col / 2 if col is even and below 2G,
    // else zero; dims 64m + 16grp .. +7 (k-step 2m) and +8 .. +15 (2m + 1)
    uint4 qa[2 * NM];
    {
        const bool arow = (col & 1) == 0 && col < 2 * G;
        const uint16_t* qrow = q + ((int64_t)e * Hq + g * G + (col >> 1)) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                qa[2 * m + h] = arow ? *reinterpret_cast<const uint4*>(qrow + 64 * m + 16 * grp + 8 * h)
                                     : make_uint4(0u, 0u, 0u, 0u);
    }

    f32x4_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};  // heads 2grp, 2grp + 1
    const float cs = sm * LOG2E;
    const int32_t* bt = pv.bt + (int64_t)bd.seq[e] * pv.bt_stride;
    const int64_t lhoff = ((int64_t)layer * Hkv + g) * pv.block_bytes;

    // a wave takes every fourth page of the split; with half pages, both halves of it in turn
    for (int pg = pg0 + wave; pg < pg1; pg += 4) {
      for (int hf = 0; hf < 4 / TB; ++hf) {
        const int t0 = 16 * TB * hf;                        // first token slot of the step
        const int n_tok = min(PAGE, ctx - pg * PAGE) - t0;  // valid tokens from t0 on
        if (n_tok <= 0) break;                              // the second half of a short last page
        const uint8_t* blk = pv.pages + (int64_t)bt[pg] * pv.page_bytes + lhoff;
        uint4 kraw[TB][2 * NM];  // token t0 + 16tb + col, dims 64m + 16grp + 8h .. +7
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    kraw[tb][2 * m + h] =
                        stream_load4(blk + 2 * ((t0 + 16 * tb + col) * D + 64 * m + 16 * grp + 8 * h));
        uint4 vraw[NDB][KS];  // dim 16db + col, tokens t0 + 8 KS grp + 8h .. +7
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < KS; ++h)
                vraw[db][h] =
                    stream_load4(blk + 128 * D + 2 * ((16 * db + col) * PAGE + t0 + 8 * KS * grp + 8 * h));

        // ---- S^T: row 4grp + r (head 2grp + r/2 when r is even), column = token t0 + 16tb + col ----
        f32x4_t st[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            st[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 2 * NM; ++k) st[tb] = mma_bf16(qa[k], kraw[tb][k], st[tb]);
        }
        // ---- online softmax of heads 2grp, 2grp + 1 over the page's tokens ----
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int j = 2 * grp + hh;
            const bool live = j < G;
            float sv[TB], mt = -INFINITY;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const bool valid = 16 * tb + col < n_tok;
                const float raw = st[tb][2 * hh];
                if constexpr (SCORES)
                    if (live && valid)
                        scores[((int64_t)e * Hq + g * G + j) * sstride + pg * PAGE + t0 + 16 * tb + col] = sm * raw;
                sv[tb] = valid && live ? raw * cs : -INFINITY;
                mt = fmaxf(mt, sv[tb]);
            }
            const float m_new = fmaxf(m_run[hh], row16_max(mt));
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[hh] - m_new);
            float psum = 0.f;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                // slots past ctx weigh nothing (their bytes may be anything, NaN included)
                const float p = sv[tb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb] - m_new);
                psum += p;
                const uint32_t hl = hi_lo(p);
                if (live) {
                    w_s[wave][2 * j][16 * tb + col] = (uint16_t)(hl & 0xFFFF);
                    w_s[wave][2 * j + 1][16 * tb + col] = (uint16_t)(hl >> 16);
                }
            }
            l_run[hh] = l_run[hh] * alpha + row16_sum(psum);
            m_run[hh] = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                acc[db][2 * hh] *= alpha;
                acc[db][2 * hh + 1] *= alpha;
            }
        }
        // ---- O += W~ V: A = weight row col, tokens 8 KS grp .. +8 KS - 1 of the step (the wave's LDS is read in order) ----
        uint4 wa[KS];
#pragma unroll
        for (int h = 0; h < KS; ++h) wa[h] = *reinterpret_cast<const uint4*>(&w_s[wave][col][8 * KS * grp + 8 * h]);
        // a slot past ctx has weight 0, but 0 x NaN would still poison the
        // sum: the V bytes of such slots are replaced by zeros
        if (n_tok < 16 * TB) {
#pragma unroll
            for (int h = 0; h < KS; ++h) {
                const int tv = 8 * KS * grp + 8 * h;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    uint32_t* w = reinterpret_cast<uint32_t*>(&vraw[db][h]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t keep = (tv + 2 * i < n_tok ? 0xFFFFu : 0u) | (tv + 2 * i + 1 < n_tok ? 0xFFFF0000u : 0u);
                        w[i] &= keep;
                    }
                }
            }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < KS; ++h) acc[db] = mma_bf16(wa[h], vraw[db][h], acc[db]);
      }
    }

    // ---- combine the four waves (a wave without pages holds m = -inf, l = 0, o = 0) ----
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int j = 2 * grp + hh;
        if (j < G) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) o_s[wave][j][16 * db + col] = acc[db][2 * hh] + acc[db][2 * hh + 1];
            if (col == 0) {
                ml_s[wave][j][0] = m_run[hh];
                ml_s[wave][j][1] = l_run[hh];
            }
        }
    }
    __syncthreads();
    DecodeWs w(ws, bd.n, Hq, D, splits);
    for (int idx = tid; idx < G * D; idx += 256) {
        const int j = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) M = fmaxf(M, ml_s[v][j][0]);
        float accum = 0.f, L = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
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

constexpr int BF16_STEP_BLOCKS = 4;  // whole pages per step (see decode_bf16_kernel)

hipError_t launch_decode_bf16(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                              int splits, float* ws, float* out, float* scores, int64_t sstride, hipStream_t s) {
    dim3 grid(bd.n * pv.Hkv, splits);
    const int G = pv.Hq / pv.Hkv;
    auto go = [&](auto d_tag, auto g_tag) {
        constexpr int DD = decltype(d_tag)::value, GG = decltype(g_tag)::value;
        if (scores)
            hipLaunchKernelGGL((decode_bf16_kernel<DD, GG, true, BF16_STEP_BLOCKS>), grid, dim3(256), 0, s, pv, layer, bd, q, sm, splits,
                               ws, scores, sstride);
        else
            hipLaunchKernelGGL((decode_bf16_kernel<DD, GG, false, BF16_STEP_BLOCKS>), grid, dim3(256), 0, s, pv, layer, bd, q, sm, splits,
                               ws, scores, sstride);
    };
    auto by_group = [&](auto d_tag) {
        if (G == 1) go(d_tag, std::integral_constant<int, 1>{});
        else if (G == 2) go(d_tag, std::integral_constant<int, 2>{});
        else if (G == 4) go(d_tag, std::integral_constant<int, 4>{});
        else go(d_tag, std::integral_constant<int, 8>{});
    };
    if (pv.D == 256)
        by_group(std::integral_constant<int, 256>{});
    else
        by_group(std::integral_constant<int, 128>{});
    const hipError_t err = hipGetLastError();
    return err != hipSuccess ? err : launch_merge_splits(bd, pv.Hq, pv.D, splits, ws, out, s);
}

}  // namespace kvq
