// Split-K bookkeeping shared by the decode kernels: partial (m, l, o) layout
// in the workspace and the fp32 merge of the splits.
//
// Flash-decoding keeps, for each split p of a sequence's pages, the running
// max m_p, the sum l_p of exp(s - m_p) and o_p = sum exp(s - m_p) v^.  The
// merge is out = sum_p e^{m_p - M} o_p / sum_p e^{m_p - M} l_p with M = max m_p,
// all in fp32 registers (the two-level accumulation of "Half the Cache, Twice
// the Context", section "The cliff is in the accumulator").  Scores and maxima
// are kept in base-2 units inside the kernels (s * log2 e), so exp2 is used.
//
// The merge is a kernel of its own, launched after the split kernel on the
// same stream: the kernel boundary makes the partials visible to it.  Merging
// inside the split kernel (last workgroup to arrive) would need a device-scope
// release and acquire in every workgroup, which on this chip write back and
// invalidate the whole L2 of the workgroup's XCD.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int MAX_SPLITS = 256;

// Streaming loads for what a decode call reads once (codes, metadata, bf16
// rows): nontemporal, so that they do not displace what the caches hold.
typedef uint32_t stream_v4u __attribute__((ext_vector_type(4)));
typedef uint32_t stream_v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 stream_load4(const uint8_t* p) {
    const stream_v4u w = __builtin_nontemporal_load(reinterpret_cast<const stream_v4u*>(p));
    return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ uint2 stream_load2(const uint8_t* p) {
    const stream_v2u w = __builtin_nontemporal_load(reinterpret_cast<const stream_v2u*>(p));
    return make_uint2(w.x, w.y);
}

// Splits p < live_splits(...) hold at least one page; the rest are empty and
// leave their partials unwritten (split_range gives every split the same
// whole number of page pairs, so empty splits only trail).
__host__ __device__ inline int live_splits(int ctx, int per) {
    const int n_pages = (ctx + PAGE - 1) / PAGE;
    const int pairs = (n_pages + 1) / 2;
    return per > 0 ? (pairs + per - 1) / per : 0;
}

struct DecodeWs {
    float* o;   // [n][Hq][splits][D]
    float* ml;  // [n][Hq][splits][2]
    __device__ DecodeWs(float* ws, int n, int Hq, int D, int splits)
        : o(ws), ml(ws + (int64_t)n * Hq * splits * D) {}
};

hipError_t launch_merge_splits(const BatchDesc& bd, int Hq, int D, int splits, float* ws, float* out, hipStream_t s);

}  // namespace kvq
