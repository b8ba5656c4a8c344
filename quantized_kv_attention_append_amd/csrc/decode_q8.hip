// Split-K decode attention over the 8-bit pool on the vector ALUs (any GQA
// group G <= 8, head_dim 128 or 256).
//
// The 8-bit format reads 268 bytes per (token, KV head) at D = 128 for 2 x G x
// 128 multiply-adds, few enough that the vector ALUs keep up with HBM.  The
// dequantization is folded into the operands: K is scaled per channel, so the
// query is multiplied by the page's channel scales once per page
// (q.k^_t = sum_d (q_d s_d) c_td), and V is scaled per token, so the
// softmax weight absorbs it (sum_t p_t v^_td = sum_t (p_t s_t) c_dt).  Scores,
// the online softmax and every running sum are fp32 (the two-level
// accumulation of "Half the Cache, Twice the Context", section "The cliff is
// in the accumulator"), in base-2 units inside the kernel.
//
// One workgroup of 256 threads per (sequence, KV head, split), one page of 64
// tokens per step, the next page's bytes prefetched into registers while the
// current one is computed:
//   scores:  wave w takes dims [wD/4, (w+1)D/4) of token t = lane for every
//            head; the four partial dots meet in LDS;
//   softmax: wave j % 4 takes heads j;
//   p.v:     thread (d, half) takes dim d over tokens [32 half, 32 half + 32)
//            (D = 128) or all 64 tokens (D = 256) for every head.
// Partial (m, l, o) go to the workspace; merge_splits_kernel merges them.
#include "decode_common.h"

namespace kvq {

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
    split_range(ctx, splits, sp, &pg0, &pg1);
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

hipError_t launch_decode_q8(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                            int splits, float* ws, float* out, float* scores, int64_t sstride, hipStream_t s) {
    dim3 grid(bd.n * pv.Hkv, splits);
    if (pv.D == 256)
        hipLaunchKernelGGL(decode_q8_kernel<256>, grid, dim3(256), 0, s, pv, layer, bd, q, sm, splits, ws, out, scores,
                           sstride);
    else
        hipLaunchKernelGGL(decode_q8_kernel<128>, grid, dim3(256), 0, s, pv, layer, bd, q, sm, splits, ws, out, scores,
                           sstride);
    const hipError_t err = hipGetLastError();
    return err != hipSuccess ? err : launch_merge_splits(bd, pv.Hq, pv.D, splits, ws, out, s);
}

}  // namespace kvq
