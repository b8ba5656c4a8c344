// Merge of the split-K decode partials: one workgroup per (sequence, query
// head), one thread per output dim.
#include "decode_common.h"

namespace kvq {

__global__ __launch_bounds__(256) void merge_splits_kernel(BatchDesc bd, int Hq, int D, int splits,
                                                           const float* __restrict__ ws, float* __restrict__ out) {
    const int e = blockIdx.x / Hq;
    const int d = threadIdx.x;
    const int live = live_splits(bd.pos[e], splits);
    const int64_t row = blockIdx.x;  // e * Hq + h
    const float* ml = ws + (int64_t)bd.n * Hq * splits * D + row * splits * 2;
    const float* o = ws + row * splits * D + d;
    float M = -INFINITY;
    for (int p = 0; p < live; ++p) M = fmaxf(M, ml[2 * p]);
    float den = 0.f, acc = 0.f;
#pragma unroll 4
    for (int p = 0; p < live; ++p) {
        const float f = exp2f(ml[2 * p] - M);
        den += f * ml[2 * p + 1];
        acc += f * __builtin_nontemporal_load(o + (int64_t)p * D);
    }
    out[row * D + d] = acc / den;
}

hipError_t launch_merge_splits(const BatchDesc& bd, int Hq, int D, int splits, float* ws, float* out, hipStream_t s) {
    hipLaunchKernelGGL(merge_splits_kernel, dim3(bd.n * Hq), dim3(D), 0, s, bd, Hq, D, splits, ws, out);
    return hipGetLastError();
}

}  // namespace kvq
