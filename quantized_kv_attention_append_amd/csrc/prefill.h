// Chunked prefill: launch entry and workspace sizing shared by the host
// runtime and the prefill kernels.  Not part of the public ABI (include/kvq.h).
#pragma once

#include "kvq_internal.h"

namespace kvq {

// Prefill over a 2-bit, bf16, 2-bit window or rotated 2-bit pool (fmt).
// Window pools: keys from w0 = 64 * floor((A - 1) / 64) on come from the
// window block, and the window's partials sit after the splits' in ws (one
// more split's worth).  Rotated pools: the rotated query's two bf16 terms
// sit after the splits' partials.
hipError_t launch_prefill(const PoolView& pv, int fmt, int layer, int seq, int q_start, int n_q, const uint16_t* q,
                          float sm, int splits, float* ws, float* out, int w0, hipStream_t s);
// (query, head) rows a prefill workgroup takes, in every format.
inline int prefill_rows_per_block(int /*fmt*/) { return 128; }
// Split count a prefill of n_q chunk queries takes when the caller passes 0:
// about one workgroup per compute unit (256 on MI355X).
inline int prefill_auto_splits(int n_q, int Hq, int Hkv, int fmt) {
    const int QB = prefill_rows_per_block(fmt) / (Hq / Hkv);
    const int blocks = ((n_q + QB - 1) / QB) * Hkv;
    const int want = (256 + blocks - 1) / blocks;
    return want < 1 ? 1 : want > 64 ? 64 : want;
}
// Floats a prefill workspace holds beyond the splits' partials: the window's
// partials (2-bit window pools) or the rotated query's two bf16 terms
// (rotated pools).
inline int64_t prefill_extra_floats(int fmt, int n_q, int Hq, int D) {
    return fmt == KV_FMT_Q2_WINDOW ? (int64_t)n_q * Hq * (D + 2) : fmt == KV_FMT_Q2_ROT ? (int64_t)n_q * Hq * D : 0;
}
// Prefill workspace: partial outputs [n_q][Hq][splits][D] then (max, sum) [n_q][Hq][splits][2].
inline int64_t prefill_ws_floats(int n_q, int Hq, int D, int splits) {
    return (int64_t)n_q * Hq * splits * (D + 2);
}

}  // namespace kvq
