// Copy on write for prefix sharing: a fork copies the page its prefix only
// partly fills, and the exact rows the format keeps for it, into the new
// sequence's own memory ("The KV cache and prompt reuse", section "What a
// sequence is made of").  Up to three byte ranges, 16 bytes a thread,
// grid-stride over the largest.
#include "kvq_internal.h"

namespace kvq {

struct CopyRanges {
    CopyRange r[3];
    int n;
};

__global__ __launch_bounds__(256) void copy_ranges_kernel(CopyRanges cr) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int k = 0; k < cr.n; ++k) {
        const uint4* src = reinterpret_cast<const uint4*>(cr.r[k].src);
        uint4* dst = reinterpret_cast<uint4*>(cr.r[k].dst);
        const int64_t n16 = cr.r[k].bytes / 16;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
    }
}

hipError_t launch_copy_ranges(const CopyRange* r, int n, hipStream_t s) {
    if (n < 1 || n > 3) return hipErrorInvalidValue;
    CopyRanges cr;
    cr.n = n;
    int64_t most = 0;
    for (int k = 0; k < n; ++k) {
        if (r[k].bytes % 16 || ((uintptr_t)r[k].src | (uintptr_t)r[k].dst) % 16) return hipErrorInvalidValue;
        cr.r[k] = r[k];
        most = r[k].bytes > most ? r[k].bytes : most;
    }
    const int64_t blocks = (most / 16 + 255) / 256;
    hipLaunchKernelGGL(copy_ranges_kernel, dim3((unsigned)(blocks < 1024 ? (blocks > 0 ? blocks : 1) : 1024)), dim3(256),
                       0, s, cr);
    return hipGetLastError();
}

}  // namespace kvq
