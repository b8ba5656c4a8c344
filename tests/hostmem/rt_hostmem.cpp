// Host-memory backend of the library's host runtime, for the CPU test suite
// (tests/test_host_pool_cpu.py): linked with quantized_kv_attention_append_amd/
// csrc/kvq_host.cpp into a library of its own by g++, no GPU needed.
//
// The device-memory calls of kvq_rt.h work on host memory (malloc, memset,
// memcpy), so every pool, reservation, fork, release, block-table and
// argument-check path of the C ABI runs as in the real library.  No kernel
// runs: each launcher records what the library asked to launch (its kind,
// layer, batch, work items and split count) and returns success, except the
// fork's byte copy, which is done.  This is test infrastructure, never loaded
// by the library's Python binding.
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"
#include "prefill.h"
#include "kvq_rt.h"

namespace kvq {
namespace rt {
hipError_t current_device(int* dev) {
    *dev = 0;
    return hipSuccess;
}
hipError_t alloc(void** p, size_t bytes) {
    *p = std::malloc(bytes ? bytes : 1);
    return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t release(void* p) {
    std::free(p);
    return hipSuccess;
}
hipError_t zero(void* p, size_t bytes) {
    std::memset(p, 0, bytes);
    return hipSuccess;
}
hipError_t upload(void* dst, const void* src, size_t bytes) {
    std::memcpy(dst, src, bytes);
    return hipSuccess;
}
const char* error_string(hipError_t e) { return e == hipSuccess ? "no error" : "host-memory backend error"; }
}  // namespace rt

namespace {
struct Launch {
    std::string kind;
    int layer, n, work, splits;
};
std::mutex g_mu;
std::vector<Launch> g_launches;
hipError_t record(const char* kind, int layer, int n, int work, int splits) {
    std::lock_guard<std::mutex> lock(g_mu);
    g_launches.push_back({kind, layer, n, work, splits});
    return hipSuccess;
}
}  // namespace

hipError_t launch_append_q2(const PoolView&, int layer, const BatchDesc& bd, int work_items, const uint16_t*,
                            const uint16_t*, hipStream_t, bool rot) {
    return record(rot ? "append_q2_rot" : "append_q2", layer, bd.n, work_items, 0);
}
hipError_t launch_append_q8(const PoolView&, int layer, const BatchDesc& bd, int work_items, const uint16_t*,
                            const uint16_t*, hipStream_t) {
    return record("append_q8", layer, bd.n, work_items, 0);
}
hipError_t launch_append_bf16(const PoolView&, int layer, const BatchDesc& bd, int work_items, const uint16_t*,
                              const uint16_t*, hipStream_t) {
    return record("append_bf16", layer, bd.n, work_items, 0);
}
hipError_t launch_append_window(const PoolView&, int layer, const BatchDesc& bd, const uint16_t*, const uint16_t*,
                                hipStream_t) {
    return record("append_window", layer, bd.n, bd.n, 0);
}
hipError_t launch_decode_q2(const PoolView&, int layer, const BatchDesc& bd, const uint16_t*, float, int splits,
                            float*, float*, float*, int64_t, hipStream_t, bool rot) {
    return record(rot ? "decode_q2_rot" : "decode_q2", layer, bd.n, bd.per, splits);
}
hipError_t launch_decode_q2_partials(const PoolView&, int layer, const BatchDesc& bd, const uint16_t*, float,
                                     int splits, float*, float*, int64_t, hipStream_t, bool) {
    return record("decode_q2_partials", layer, bd.n, bd.per, splits);
}
hipError_t launch_decode_window_merge(const PoolView&, int layer, const BatchDesc& bd, const uint16_t*, float,
                                      int splits, const float*, float*, float*, int64_t, hipStream_t) {
    return record("decode_window_merge", layer, bd.n, bd.per, splits);
}
hipError_t launch_decode_q8(const PoolView&, int layer, const BatchDesc& bd, const uint16_t*, float, int splits,
                            float*, float*, float*, int64_t, hipStream_t) {
    return record("decode_q8", layer, bd.n, bd.per, splits);
}
hipError_t launch_decode_bf16(const PoolView&, int layer, const BatchDesc& bd, const uint16_t*, float, int splits,
                              float*, float*, float*, int64_t, hipStream_t) {
    return record("decode_bf16", layer, bd.n, bd.per, splits);
}
hipError_t launch_prefill(const PoolView&, int fmt, int layer, int, int, int n_q, const uint16_t*, float, int splits,
                          float*, float*, int, hipStream_t) {
    return record(fmt == KV_FMT_Q2_ROT ? "prefill_rot" : "prefill", layer, n_q, 0, splits);
}
hipError_t launch_copy_ranges(const CopyRange* r, int n, hipStream_t) {
    for (int i = 0; i < n; ++i) std::memcpy(r[i].dst, r[i].src, (size_t)r[i].bytes);
    record("copy_ranges", 0, n, 0, 0);
    return hipSuccess;
}
hipError_t launch_dequant_page(const PoolView&, int, int, int layer, int, int, float*, hipStream_t) {
    return record("dequant_page", layer, 1, 0, 0);
}

}  // namespace kvq

extern "C" {
// The launches recorded so far: count, and entry i's kind and its numbers
// (layer, batch, work items or page pairs per split, splits).
int kvq_hostmem_launches(void) {
    std::lock_guard<std::mutex> lock(kvq::g_mu);
    return (int)kvq::g_launches.size();
}
const char* kvq_hostmem_launch_kind(int i) {
    std::lock_guard<std::mutex> lock(kvq::g_mu);
    return i >= 0 && i < (int)kvq::g_launches.size() ? kvq::g_launches[(size_t)i].kind.c_str() : "";
}
int kvq_hostmem_launch_arg(int i, int which) {
    std::lock_guard<std::mutex> lock(kvq::g_mu);
    if (i < 0 || i >= (int)kvq::g_launches.size()) return -1;
    const auto& l = kvq::g_launches[(size_t)i];
    return which == 0 ? l.layer : which == 1 ? l.n : which == 2 ? l.work : l.splits;
}
void kvq_hostmem_clear(void) {
    std::lock_guard<std::mutex> lock(kvq::g_mu);
    kvq::g_launches.clear();
}
}
