// Split-K decode attention over the 2-bit pool on the vector ALUs, for any
// GQA group G in {1, 2, 4, 8}.  (Group 4 normally takes the matrix-core
// kernel in decode_q2_mfma.hip; this one covers the other groups.)
//
// One workgroup per (sequence, KV head, split): it walks its pages of the
// sequence's block table and keeps, per query head, the running max m, the
// running sum l of exp(s - m) and the unnormalised output o in fp32 (the
// "two-level" accumulation that "Half the Cache, Twice the Context" asks for in
// section "The cliff is in the accumulator": every sum is a real fp32
// register).  The dequantization is folded algebraically instead of
// materialising K^ and V^:
//     q . k^_t = mn_t * sum(q) + scale_t * sum_d q_d c_td
//     sum_t p_t v^_td = sum_t p_t mn_t + sum_t (p_t scale_t) c_td
// Partial (m, l, o) go to the workspace; merge_splits_kernel then merges the
// splits in fp32.
#include "decode_common.h"

namespace kvq {

template <int D>
__global__ __launch_bounds__(256) void decode_q2_valu_kernel(PoolView pv, int layer, BatchDesc bd,
                                                             const uint16_t* __restrict__ q, float sm, int splits,
                                                             float* __restrict__ ws, float* __restrict__ out,
                                                             float* __restrict__ scores, int64_t sstride) {
    const int Hkv = pv.Hkv, Hq = pv.Hq, G = Hq / Hkv;
    const int e = blockIdx.x / Hkv, g = blockIdx.x % Hkv, sp = blockIdx.y;
    const int ctx = bd.pos[e];
    int pg0, pg1;
    split_range(ctx, bd.per, sp, &pg0, &pg1);
    if (pg0 >= pg1) return;
    const float LOG2E = 1.4426950408889634f;

    __shared__ float q_s[8][D];
    __shared__ float s_s[8][PAGE];
    __shared__ float w_s[8][PAGE];
    __shared__ float qsum_s[8], m_s[8], l_s[8], c_s[8], a_s[8];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    for (int i = tid; i < G * D; i += 256)
        q_s[i / D][i % D] = bf16_to_f32(q[((int64_t)e * Hq + g * G + i / D) * D + i % D]);
    __syncthreads();
    for (int j = wave; j < G; j += 4) {
        float a = 0.f;
        for (int d = lane; d < D; d += 64) a += q_s[j][d];
        a = wave_sum(a);
        if (lane == 0) {
            qsum_s[j] = a;
            m_s[j] = -INFINITY;
            l_s[j] = 0.f;
            c_s[j] = 0.f;
        }
    }
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.f;
    __syncthreads();

    const int32_t* bt = pv.bt + (int64_t)bd.seq[e] * pv.bt_stride;
    for (int pg = pg0; pg < pg1; ++pg) {
        const uint8_t* blk = pv.pages + (int64_t)bt[pg] * pv.page_bytes + ((int64_t)layer * Hkv + g) * pv.block_bytes;
        const int n_tok = min(PAGE, ctx - pg * PAGE);
        // scores
        for (int pr = tid; pr < PAGE * G; pr += 256) {
            const int t = pr & 63, j = pr >> 6;
            float s = -INFINITY;
            if (t < n_tok) {
                const uint32_t* row = reinterpret_cast<const uint32_t*>(blk + t * (D / 4));
                float acc = 0.f;
                for (int w = 0; w < D / 16; ++w) {
                    uint32_t bits = row[w];
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc += q_s[j][16 * w + i] * (float)((bits >> (2 * i)) & 3u);
                }
                float2 meta = *reinterpret_cast<const float2*>(blk + q2_kmeta_off(D) + 8 * t);
                s = sm * (meta.y * qsum_s[j] + meta.x * acc);
                if (scores) scores[((int64_t)e * Hq + g * G + j) * sstride + pg * PAGE + t] = s;
                s *= LOG2E;
            }
            s_s[j][t] = s;
        }
        __syncthreads();
        // online softmax, one wave per head
        for (int j = wave; j < G; j += 4) {
            const float s = s_s[j][lane];
            const float m_old = m_s[j];
            const float m_new = fmaxf(m_old, wave_max(s));
            const float alpha = exp2f(m_old - m_new);
            float p = 0.f, wv = 0.f, cv = 0.f;
            if (lane < n_tok) {
                float2 vm = *reinterpret_cast<const float2*>(blk + q2_vmeta_off(D) + 8 * lane);
                p = exp2f(s - m_new);
                wv = p * vm.x;
                cv = p * vm.y;
            }
            w_s[j][lane] = wv;
            const float psum = wave_sum(p), csum = wave_sum(cv);
            if (lane == 0) {
                m_s[j] = m_new;
                l_s[j] = l_s[j] * alpha + psum;
                c_s[j] = c_s[j] * alpha + csum;
                a_s[j] = alpha;
            }
        }
        __syncthreads();
        // p . v over the dim-major V plane, one thread per dim
        if (tid < D) {
            const uint2 v0 = *reinterpret_cast<const uint2*>(blk + q2_vcodes_off(D) + q2_vword_off(D, tid, 0));
            const uint2 v1 = *reinterpret_cast<const uint2*>(blk + q2_vcodes_off(D) + q2_vword_off(D, tid, 2));
            const uint32_t words[4] = {v0.x, v0.y, v1.x, v1.y};
            for (int j = 0; j < G; ++j) o[j] *= a_s[j];
#pragma unroll
            for (int t = 0; t < PAGE; ++t) {
                const float c = (float)((words[q2_vslot_word(t)] >> q2_vslot_bit(t)) & 3u);
                for (int j = 0; j < G; ++j) o[j] += w_s[j][t] * c;
            }
        }
        __syncthreads();
    }
    DecodeWs w(ws, bd.n, Hq, D, splits);
    if (tid < D)
        for (int j = 0; j < G; ++j) {
            const int64_t r = ((int64_t)e * Hq + g * G + j) * splits + sp;
            w.o[r * D + tid] = o[j] + c_s[j];
        }
    if (tid < G) {
        const int64_t r = ((int64_t)e * Hq + g * G + tid) * splits + sp;
        w.ml[2 * r] = m_s[tid];
        w.ml[2 * r + 1] = l_s[tid];
    }
}

hipError_t launch_decode_q2_valu(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                                 int splits, float* ws, float* out, float* scores, int64_t sstride, hipStream_t s) {
    dim3 grid(bd.n * pv.Hkv, splits);
    if (pv.D == 256)
        hipLaunchKernelGGL(decode_q2_valu_kernel<256>, grid, dim3(256), 0, s, pv, layer, bd, q, sm, splits, ws, out, scores, sstride);
    else
        hipLaunchKernelGGL(decode_q2_valu_kernel<128>, grid, dim3(256), 0, s, pv, layer, bd, q, sm, splits, ws, out, scores, sstride);
    return hipGetLastError();
}

}  // namespace kvq
