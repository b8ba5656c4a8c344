// Merge of the split-K decode partials: one workgroup per (sequence, query
// head), one thread per output dim.  Splits are taken in groups (one group
// of up to 8, or groups of 32 when there are more than 8) with all of a
// group's loads issued before any is used, so a merge costs one round trip
// to memory per group; with up to 8 splits the loads do not wait for the
// sequence's length either.
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
// is known (every slot below `splits` lies inside the workspace; the slots of
// empty splits, never written in this call, are then selected away).
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

// More splits: groups of 32, each group's loads issued together.
__global__ __launch_bounds__(256) void merge_splits32_kernel(BatchDesc bd, int Hq, int D, int splits,
                                                             const float* __restrict__ ws, float* __restrict__ out) {
    constexpr int U = 32;
    const int e = blockIdx.x / Hq;
    const int d = threadIdx.x;
    const int live = live_splits(bd.pos[e], bd.per);
    const int64_t row = blockIdx.x;  // e * Hq + h
    const float2* ml = reinterpret_cast<const float2*>(ws + (int64_t)bd.n * Hq * splits * D) + row * splits;
    const float* o = ws + row * splits * D + d;
    float M = -INFINITY, den = 0.f, acc = 0.f;
    for (int p0 = 0; p0 < live; p0 += U) {
        float2 m[U];
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = p0 + u < live;
            m[u] = ok ? ml[p0 + u] : make_float2(-INFINITY, 0.f);
            v[u] = ok ? __builtin_nontemporal_load(o + (int64_t)(p0 + u) * D) : 0.f;
        }
        merge_group<U>(m, v, M, den, acc);
    }
    out[row * D + d] = acc / den;
}

hipError_t launch_merge_splits(const BatchDesc& bd, int Hq, int D, int splits, float* ws, float* out, hipStream_t s) {
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(bd.n * Hq), dim3(D), 0, s, bd, Hq, D, splits, ws, out);
    };
    if (splits > 8)
        go(merge_splits32_kernel);
    else
        go(merge_splits8_kernel);
    return hipGetLastError();
}

}  // namespace kvq
