// Merge of the split-K decode partials: one workgroup per (sequence, query
// head), one thread per output dim.  Splits are taken U at a time (8, or 32
// when there are more than 8) with all of a group's loads issued before any
// is used, so a merge costs one round trip to memory per U splits; the first
// group's loads do not wait for the sequence's length.
#include "decode_common.h"

namespace kvq {

template <int U>
__global__ __launch_bounds__(256) void merge_splits_kernel(BatchDesc bd, int Hq, int D, int splits,
                                                           const float* __restrict__ ws, float* __restrict__ out) {
    const int d = threadIdx.x;
    const int64_t row = blockIdx.x;  // e * Hq + h
    const float2* ml = reinterpret_cast<const float2*>(ws + (int64_t)bd.n * Hq * splits * D) + row * splits;
    const float* o = ws + row * splits * D + d;
    // The first group's loads go out before the live split count is known:
    // every slot below `splits` lies inside the workspace, and the slots of
    // empty splits (never written in this call) are selected away below.
    float2 m[U];
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool in = u < splits;
        m[u] = in ? ml[u] : make_float2(-INFINITY, 0.f);
        v[u] = in ? __builtin_nontemporal_load(o + (int64_t)u * D) : 0.f;
    }
    const int live = live_splits(bd.pos[blockIdx.x / Hq], bd.per);
    // running (max, sum, output) over groups of U splits, in base-2 units
    float M = -INFINITY, den = 0.f, acc = 0.f;
    for (int p0 = 0; p0 < live; p0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = p0 + u < live;
            if (p0 == 0) {  // select, never multiply, so that an unwritten slot cannot leak in
                m[u] = ok ? m[u] : make_float2(-INFINITY, 0.f);
                v[u] = ok ? v[u] : 0.f;
            } else {
                m[u] = ok ? ml[p0 + u] : make_float2(-INFINITY, 0.f);
                v[u] = ok ? __builtin_nontemporal_load(o + (int64_t)(p0 + u) * D) : 0.f;
            }
        }
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
    out[row * D + d] = acc / den;
}

hipError_t launch_merge_splits(const BatchDesc& bd, int Hq, int D, int splits, float* ws, float* out, hipStream_t s) {
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(bd.n * Hq), dim3(D), 0, s, bd, Hq, D, splits, ws, out);
    };
    if (splits > 8)
        go(merge_splits_kernel<32>);
    else
        go(merge_splits_kernel<8>);
    return hipGetLastError();
}

}  // namespace kvq
