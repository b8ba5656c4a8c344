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
// With up to FUSED_MERGE_MAX_SPLITS splits the 2-bit decode merges inside
// its split kernel: the last workgroup of a (sequence, KV head) to finish
// merges every split's partials.  Partials and the arrival counter go through
// agent-scope relaxed atomics (coherent across the XCDs' L2 caches without
// the whole-cache writeback and invalidation a release / acquire fence would
// issue).  Otherwise the merge is a kernel of its own, launched after the
// split kernel on the same stream: the kernel boundary makes the partials
// visible to it.
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

// Agent-scope (coherent across the chip's L2 caches) relaxed store and load
// of one float: what split partials merged inside the split kernel travel
// through, so that no whole-cache writeback or invalidation is needed.
__device__ __forceinline__ void store_agent(float* p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every store this thread has issued is complete.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Merge of a (sequence, query head)'s live splits (at most
// FUSED_MERGE_MAX_SPLITS) inside the split kernel, by one wave: lane l
// writes dims l + 64k of out.  Loads go out before any is used.
template <int K>
__device__ __forceinline__ void merge_live_splits(const DecodeWs& w, int64_t row0, int live, int l,
                                                  float* __restrict__ out) {
    constexpr int U = FUSED_MERGE_MAX_SPLITS;
    float m[U], den[U], v[U][K];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool in = u < live;
        m[u] = in ? load_agent(&w.ml[2 * (row0 + u)]) : -INFINITY;
        den[u] = in ? load_agent(&w.ml[2 * (row0 + u) + 1]) : 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) v[u][k] = in ? load_agent(&w.o[(row0 + u) * (64 * K) + l + 64 * k]) : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) M = fmaxf(M, m[u]);
    float dsum = 0.f, acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float f = u < live ? exp2f(m[u] - M) : 0.f;  // select: slots past live were not written
        dsum += f * den[u];
#pragma unroll
        for (int k = 0; k < K; ++k) acc[k] = u < live ? fmaf(f, v[u][k], acc[k]) : acc[k];
    }
#pragma unroll
    for (int k = 0; k < K; ++k) out[l + 64 * k] = acc[k] / dsum;
}

}  // namespace kvq
