// kv_attn_decode_static: the decode step with its workspace in a file-scope
// device array instead of a caller's buffer, for callers that cannot
// allocate device memory at call time (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The array is KV_STATIC_SCRATCH_BYTES per device, held by every device the
// library runs on until the process ends.  Its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) on the
// first call there and kept; host code uses that address only, never the
// array's name.  The call then takes the same checks and kernels as
// kv_attn_decode, with this array as the workspace: nothing is allocated.
// Every call on a device shares its array, so calls that overlap on one
// device (different streams, or several pools) race; the decode kernels
// write every workspace byte they read within the call, so nothing needs
// clearing between calls.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __align__(256) uint8_t scratch[KV_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];  // device address of `scratch` on each device, once looked up

// The device address of this device's array, looked up on first use.
kv_status scratch_on(int dev, void** ptr) {
    if (dev < 0 || dev >= MAX_DEVICES) return set_error(KV_ERR_UNSUPPORTED, "device index beyond the static scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            char msg[256];
            snprintf(msg, sizeof msg, "hipGetSymbolAddress(static scratch) on device %d: %s", dev, hipGetErrorString(e));
            return set_error(KV_ERR_DEVICE, msg);
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return KV_OK;
}

}  // namespace
}  // namespace kvq

extern "C" kv_status kv_attn_decode_static(kv_pool* pool, int32_t layer, int32_t n, const int32_t* seqs,
                                           const int64_t* ctx_len, const uint16_t* d_q, float sm_scale,
                                           int32_t n_splits, float* d_out, float* d_scores, int64_t scores_stride,
                                           kv_stream_t stream) {
    using namespace kvq;
    if (!pool) return set_error(KV_ERR_ARG, "pool is NULL");
    if (n <= 0 || n > KV_MAX_BATCH || !ctx_len || n_splits < 0 || n_splits > 256)
        return kv_attn_decode(pool, layer, n, seqs, ctx_len, d_q, sm_scale, n_splits, nullptr, 0, d_out, d_scores,
                              scores_stride, stream);  // the same argument errors as kv_attn_decode
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(KV_ERR_DEVICE, hipGetErrorString(e));
    if (dev != pool_device(pool)) return set_error(KV_ERR_ARG, "the current device is not the pool's device");
    // the workspace this batch needs must fit the array
    int32_t sp = n_splits;
    kv_status s = sp > 0 ? KV_OK : kv_decode_splits(pool, n, ctx_len, &sp);
    if (s != KV_OK) return s;
    int64_t need = 0;
    s = kv_workspace_bytes(pool, KV_OP_DECODE, n, sp, &need);
    if (s != KV_OK) return s;
    if (need > (int64_t)KV_STATIC_SCRATCH_BYTES) {
        char msg[256];
        snprintf(msg, sizeof msg, "decode of %d sequences at %d splits needs %lld workspace bytes; the static scratch holds %lld",
                 n, sp, (long long)need, (long long)KV_STATIC_SCRATCH_BYTES);
        return set_error(KV_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    s = scratch_on(dev, &ws);
    if (s != KV_OK) return s;
    return kv_attn_decode(pool, layer, n, seqs, ctx_len, d_q, sm_scale, sp, ws, (int64_t)KV_STATIC_SCRATCH_BYTES, d_out,
                          d_scores, scores_stride, stream);
}
