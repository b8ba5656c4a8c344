// Split-K bookkeeping shared by the decode kernels: partial (m, l, o) layout
// in the workspace and the fp32 merge done by the last workgroup to finish.
//
// Flash-decoding keeps, for each split p of a sequence's pages, the running
// max m_p, the sum l_p of exp(s - m_p) and o_p = sum exp(s - m_p) v^.  The
// merge is out = sum_p e^{m_p - M} o_p / sum_p e^{m_p - M} l_p with M = max m_p,
// all in fp32 registers (the two-level accumulation of "Half the Cache, Twice
// the Context", section "The cliff is in the accumulator").  Scores and maxima
// are kept in base-2 units inside the kernels (s * log2 e), so exp2 is used.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int MAX_SPLITS = 256;

__device__ __forceinline__ int live_splits(int ctx, int splits) {
    int live = 0;
    for (int p = 0; p < splits; ++p) {
        int a, b;
        split_range(ctx, splits, p, &a, &b);
        if (a < b) live = p + 1;
    }
    return live;
}

struct DecodeWs {
    float* o;   // [n][Hq][splits][D]
    float* ml;  // [n][Hq][splits][2]
    __device__ DecodeWs(float* ws, int n, int Hq, int D, int splits)
        : o(ws), ml(ws + (int64_t)n * Hq * splits * D) {}
};

// Called by every thread of the workgroup after its partials for (e, g) are
// stored.  The last workgroup of the live splits of (e, g) merges them into
// out[e][g*G + j][:] for j < G and resets the arrival counter.
__device__ inline void merge_if_last(const PoolView& pv, const BatchDesc& bd, int e, int g, int splits, float* ws,
                                     float* out) {
    __shared__ int last_s;
    __shared__ float wgt_s[8][MAX_SPLITS];
    __shared__ float inv_s[8];
    const int Hq = pv.Hq, D = pv.D, G = pv.Hq / pv.Hkv;
    const int ctx = bd.pos[e];
    const int live = live_splits(ctx, splits);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        int* cnt = pv.sem + e * pv.Hkv + g;
        const int prev = atomicAdd(cnt, 1);
        last_s = (prev == live - 1);
        if (last_s) atomicExch(cnt, 0);
    }
    __syncthreads();
    if (!last_s) return;
    __threadfence();
    DecodeWs w(ws, bd.n, Hq, D, splits);
    for (int j = threadIdx.x; j < G; j += blockDim.x) {
        const float* ml = w.ml + ((int64_t)(e * Hq + g * G + j) * splits) * 2;
        float M = -INFINITY;
        for (int p = 0; p < live; ++p) M = fmaxf(M, __builtin_nontemporal_load(ml + 2 * p));
        float den = 0.f;
        for (int p = 0; p < live; ++p) {
            const float f = exp2f(__builtin_nontemporal_load(ml + 2 * p) - M);
            wgt_s[j][p] = f;
            den += f * __builtin_nontemporal_load(ml + 2 * p + 1);
        }
        inv_s[j] = 1.0f / den;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
        const int j = i / D, d = i - j * D;
        const int64_t row = (int64_t)e * Hq + g * G + j;
        const float* o = w.o + row * splits * D + d;
        float acc = 0.f;
#pragma unroll 8
        for (int p = 0; p < live; ++p) acc += wgt_s[j][p] * __builtin_nontemporal_load(o + (int64_t)p * D);
        out[row * D + d] = acc * inv_s[j];
    }
}

}  // namespace kvq
