// Merge of the split-K decode partials: one workgroup per (sequence, query
// head), one thread per output dim.  Splits are taken in groups with all of
// a group's loads issued before any is used, so a merge costs one round trip
// to memory per group (one group of up to 8, or groups of 64), and the first
// group's loads do not wait for the sequence's length.
#include "decode_common.h"

namespace kvq {

// The (max, sum, output) of one group of U split partials folded into the
// running values, in base-2 units; empty slots hold (-inf, 0) and 0.
template <int U>
__device__ __forceinline__ void merge_group(const float2 (&m)[U], const float (&v)[U], float& M, float& den,
                                            float& acc) {
    float Mg = M;
#pragma unroll
    for (int u = 0; u < U; ++u) Mg = fmaxf(Mg, m[u].x);
    const float r = exp2f(M - Mg);  // M = -inf on the first group: r = 0
    den *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float f = exp2f(m[u].x - Mg);  // empty slots: exp2(-inf) = 0
        den += f * m[u].y;
        acc += f * v[u];
    }
    M = Mg;
}

// Up to 8 splits: one group, whose loads go out before the live split count
// is known (every slot below `splits` lies inside the workspace; the slots
// of empty splits, never written in this call, are then selected away).
__global__ __launch_bounds__(256) void merge_splits8_kernel(BatchDesc bd, int Hq, int D, int splits,
                                                            const float* __restrict__ ws, float* __restrict__ out) {
    constexpr int U = 8;
    const int d = threadIdx.x;
    const int64_t row = blockIdx.x;  // e * Hq + h
    const float2* ml = reinterpret_cast<const float2*>(ws + (int64_t)bd.n * Hq * splits * D) + row * splits;
    const float* o = ws + row * splits * D + d;
    float2 m[U];
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool in = u < splits;
        m[u] = in ? ml[u] : make_float2(-INFINITY, 0.f);
        v[u] = in ? __builtin_nontemporal_load(o + (int64_t)u * D) : 0.f;
    }
    const int live = live_splits(bd.pos[blockIdx.x / Hq], bd.per);
#pragma unroll
    for (int u = 0; u < U; ++u) {  // select, never multiply, so that an unwritten slot cannot leak in
        m[u] = u < live ? m[u] : make_float2(-INFINITY, 0.f);
        v[u] = u < live ? v[u] : 0.f;
    }
    float M = -INFINITY, den = 0.f, acc = 0.f;
    merge_group<U>(m, v, M, den, acc);
    out[row * D + d] = acc / den;
}

// More than 8 splits, in groups of 64, one wave per (sequence, query head,
// 64 dims): lane t holds the (max, sum) of split p0 + t, the wave reduces
// them, and each lane folds its dim's 64 partial outputs with the split
// weights, which go through the wave's row of LDS.  (A row's dims spread over
// D / 64 workgroups, so that a long sequence's few rows still read their
// partials on many compute units.)  Only slots below `splits` (inside the
// workspace) are loaded and results past the live splits are selected away;
// the first group's loads go out before the live split count is known.
template <int D>
__global__ __launch_bounds__(64) void merge_splits_wide_kernel(BatchDesc bd, int Hq, int splits,
                                                               const float* __restrict__ ws,
                                                               float* __restrict__ out) {
    constexpr int U = 64;
    __shared__ __align__(16) float fs[1][U];  // split weights
    const int lane = threadIdx.x, wave = 0, d = 64 * blockIdx.y + lane;
    const int64_t row = blockIdx.x;  // e * Hq + h
    const float2* ml = reinterpret_cast<const float2*>(ws + (int64_t)bd.n * Hq * splits * D) + row * splits;
    const float* o = ws + row * splits * D + d;
    float2 mine;
    float v[U];
    auto load_group = [&](int p0) {
        const int n = splits - p0;  // slots of this group inside the workspace
        mine = lane < n ? ml[p0 + lane] : make_float2(-INFINITY, 0.f);
        const float* base = o + (int64_t)p0 * D;
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = u < n ? __builtin_nontemporal_load(base + u * D) : 0.f;
    };
    load_group(0);
    const int live = live_splits(bd.pos[blockIdx.x / Hq], bd.per);
    float M = -INFINITY, den = 0.f, acc = 0.f;  // running values in base-2 units
    for (int p0 = 0; p0 < live; p0 += U) {      // the same trip count for every thread
        if (p0 > 0) load_group(p0);
        const bool mine_live = p0 + lane < live;
        const float mx = mine_live ? mine.x : -INFINITY;
        const float Mg = fmaxf(M, wave_max(mx));
        const float r = exp2f(M - Mg);   // M = -inf on the first group: r = 0
        const float f = exp2f(mx - Mg);  // 0 past the live splits
        den = den * r + wave_sum(mine_live ? f * mine.y : 0.f);
        acc *= r;
        fs[wave][lane] = f;
        __syncthreads();
        const float4* f4 = reinterpret_cast<const float4*>(fs[wave]);
#pragma unroll
        for (int k = 0; k < U / 4; ++k) {
            const float4 w = f4[k];
            const float fw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int u = 4 * k + i;
                acc = p0 + u < live ? fmaf(fw[i], v[u], acc) : acc;  // select: an unwritten slot may hold NaN
            }
        }
        __syncthreads();  // the next group rewrites fs
        M = Mg;
    }
    out[row * D + d] = acc / den;
}

hipError_t launch_merge_splits(const BatchDesc& bd, int Hq, int D, int splits, float* ws, float* out, hipStream_t s) {
    const dim3 grid(bd.n * Hq), block(D), wide_grid(bd.n * Hq, D / 64);
    if (splits <= 8)
        hipLaunchKernelGGL(merge_splits8_kernel, grid, block, 0, s, bd, Hq, D, splits, ws, out);
    else if (D == 256)
        hipLaunchKernelGGL(merge_splits_wide_kernel<256>, wide_grid, dim3(64), 0, s, bd, Hq, splits, ws, out);
    else
        hipLaunchKernelGGL(merge_splits_wide_kernel<128>, wide_grid, dim3(64), 0, s, bd, Hq, splits, ws, out);
    return hipGetLastError();
}

}  // namespace kvq
