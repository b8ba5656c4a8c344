// Internal interface between the host runtime (kvq_host.cpp) and the HIP
// kernels.  Not part of the public ABI (include/kvq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int PAGE = KV_PAGE_TOKENS;

// Device view of a pool, passed by value to every kernel.
struct PoolView {
    uint8_t* pages;        // page p at pages + p * page_bytes
    int64_t page_bytes;
    int64_t block_bytes;   // one (layer, KV head) block inside a page
    int32_t L, Hkv, D, Hq;
    const int32_t* bt;     // device block tables [max_seqs][bt_stride]
    int32_t bt_stride;
    uint16_t* stage;       // 8-bit pools: exact K window, bf16 [max_seqs][L][Hkv][64][D]
    uint8_t* win;          // 2-bit window pools: one bf16 block (K [64][D], V [D][64]) per (seq, layer, head)
    int32_t* cnt;          // fused decode merge: arrival counters [KV_MAX_BATCH][Hkv][2], zero between calls
};

// Arrival counters a pool keeps for the fused decode merge: one per (batch
// entry, KV head, four query heads; group 8 takes two).
inline int64_t decode_counters(int Hkv) { return (int64_t)KV_MAX_BATCH * Hkv * 2; }
// Largest split count whose merge runs inside the split kernel (the last
// workgroup of a (sequence, KV head) to finish merges them); more splits are
// merged by a kernel of their own.
constexpr int FUSED_MERGE_MAX_SPLITS = 8;

// The window block of (seq, layer, head) in a 2-bit window pool.
__host__ __device__ inline uint8_t* window_block(const PoolView& pv, int seq, int layer, int head) {
    return pv.win + (((int64_t)seq * pv.L + layer) * pv.Hkv + head) * (256 * (int64_t)pv.D);
}

// Per-call batch description, passed by value as a kernel argument (so it is
// captured with the launch and needs no device copy).
struct BatchDesc {
    int32_t n;
    int32_t seq[KV_MAX_BATCH];        // sequence slot -> block-table row
    int32_t pos[KV_MAX_BATCH];        // append: first position; decode: context length
    int32_t cnt[KV_MAX_BATCH];        // append: tokens appended
    int32_t row0[KV_MAX_BATCH];       // append: first input row of the entry
    int32_t work0[KV_MAX_BATCH + 1];  // prefix sum of work items per entry
    int32_t per;                      // decode: page pairs per split, the same for every entry
    // 2-bit window pools, decode: pos = tokens read from the pages, cnt = the
    // window tokens after them (read from the window block, slots 0 .. cnt-1)
};

// Byte offsets inside a 2-bit (layer, head) block of D dims.
__host__ __device__ constexpr int64_t q2_block_bytes(int D) { return 32 * (int64_t)D + 1024; }
__host__ __device__ constexpr int64_t q2_vcodes_off(int D) { return 16 * (int64_t)D; }
__host__ __device__ constexpr int64_t q2_kmeta_off(int D) { return 32 * (int64_t)D; }
__host__ __device__ constexpr int64_t q2_vmeta_off(int D) { return 32 * (int64_t)D + 512; }
// Offset inside the V plane of word w (token slots 16w..16w+15) of dim d: the
// plane holds two halves of 32 slots (words 0-1, then 2-3); inside a half the
// 8 bytes of dims d and d + 16 (d % 32 < 16) are adjacent.
__host__ __device__ constexpr int64_t q2_vword_off(int D, int d, int w) {
    return 8 * (int64_t)D * (w >> 1) + 16 * (16 * (d >> 5) + (d & 15)) + 8 * ((d >> 4) & 1) + 4 * (w & 1);
}
// Word (0..3) and bit of token slot s (0..63) among a dim's four V-code words:
// slot 16b + 4w + r sits in word w at bit 16 (r % 2) + 4b + 2 (r / 2), so the
// 0x33333333 mask of a word yields its eight slots with r < 2, one per nibble.
__host__ __device__ constexpr int q2_vslot_word(int s) { return (s >> 2) & 3; }
__host__ __device__ constexpr int q2_vslot_bit(int s) { return 16 * (s & 1) + 4 * (s >> 4) + 2 * ((s >> 1) & 1); }
// Byte offsets inside an 8-bit (layer, head) block.
__host__ __device__ constexpr int64_t q8_block_bytes(int D) { return 132 * (int64_t)D + 256; }
__host__ __device__ constexpr int64_t q8_vcodes_off(int D) { return 64 * (int64_t)D; }
__host__ __device__ constexpr int64_t q8_kscale_off(int D) { return 128 * (int64_t)D; }
__host__ __device__ constexpr int64_t q8_vscale_off(int D) { return 132 * (int64_t)D; }

// Byte offsets inside a bf16 (layer, head) block: K [64][D] then V [D][64].
__host__ __device__ constexpr int64_t bf16_block_bytes(int D) { return 256 * (int64_t)D; }

// Launchers (defined in the .hip files).  Each returns the launch status.
// rot: the Hadamard-rotated variant (K rows transformed before quantization)
hipError_t launch_append_q2(const PoolView& pv, int layer, const BatchDesc& bd, int work_items,
                            const uint16_t* k, const uint16_t* v, hipStream_t s, bool rot = false);
hipError_t launch_append_q8(const PoolView& pv, int layer, const BatchDesc& bd, int work_items,
                            const uint16_t* k, const uint16_t* v, hipStream_t s);
hipError_t launch_append_bf16(const PoolView& pv, int layer, const BatchDesc& bd, int work_items,
                              const uint16_t* k, const uint16_t* v, hipStream_t s);
// The same copy into the window blocks of a 2-bit window pool: every entry of
// bd covers slots of one page only (one work item per entry).
hipError_t launch_append_window(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* k,
                                const uint16_t* v, hipStream_t s);
// Decode launchers enqueue the split kernel and then the merge of its
// partials, which writes the fp32 output.
// rot: the Hadamard-rotated variant: the split kernel rotates the query and
// scores with sm / D against the rotated K rows.
hipError_t launch_decode_q2(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                            int splits, float* ws, float* out, float* scores, int64_t sstride, hipStream_t s,
                            bool rot = false);
// The 2-bit split kernel alone (partials to ws, no merge).
hipError_t launch_decode_q2_partials(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                                     int splits, float* ws, float* scores, int64_t sstride, hipStream_t s,
                                     bool rot = false);
// 2-bit window pools: merge of the split partials together with the exact
// window tokens of every entry (bd.pos pages-read tokens, bd.cnt window tokens).
hipError_t launch_decode_window_merge(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q,
                                      float sm, int splits, const float* ws, float* out, float* scores,
                                      int64_t sstride, hipStream_t s);
hipError_t launch_decode_q8(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                            int splits, float* ws, float* out, float* scores, int64_t sstride, hipStream_t s);
hipError_t launch_decode_bf16(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                              int splits, float* ws, float* out, float* scores, int64_t sstride, hipStream_t s);
// Device-to-device copies of byte ranges (multiples of 16 bytes, 16-byte aligned).
struct CopyRange {
    const uint8_t* src;
    uint8_t* dst;
    int64_t bytes;
};
hipError_t launch_copy_ranges(const CopyRange* r, int n, hipStream_t s);
hipError_t launch_dequant_page(const PoolView& pv, int fmt, int page, int layer, int head, int kv, float* out,
                               hipStream_t s);

// Sets the calling thread's last-error message and returns s.
kv_status set_error(kv_status s, const char* msg);
// The device a pool was created on (-1 for NULL).
int pool_device(const kv_pool* p);

// Decode workspace: partial outputs [n][Hq][splits][D] then (max, sum) pairs [n][Hq][splits][2].
inline int64_t decode_ws_floats(int n, int Hq, int D, int splits) {
    return (int64_t)n * Hq * splits * (D + 2);
}

// Decode splits: every split of a batch covers `per` whole pairs of pages
// (the decode kernels step two pages at a time), per = ceil(pairs of the
// longest context / splits), so a shorter context fills fewer splits and no
// split holds more work than another.  Pages of a context of `ctx` tokens
// handled by split `p`:
__host__ __device__ inline int split_pairs_per(int max_ctx, int splits) {
    const int pairs = ((max_ctx + PAGE - 1) / PAGE + 1) / 2;
    return (pairs + splits - 1) / splits;
}
__host__ __device__ inline void split_range(int ctx, int per, int p, int* pg0, int* pg1) {
    int n_pages = (ctx + PAGE - 1) / PAGE;
    int a = p * per * 2, b = a + per * 2;
    *pg0 = a < n_pages ? a : n_pages;
    *pg1 = b < n_pages ? b : n_pages;
}

}  // namespace kvq
