// Append for the bf16 pool: the rows are stored as given, into the same
// 64-token pages as the compressed formats ("KV at 9 KB a token", section
// "How it works": pages of 64 tokens in a byte-budgeted pool; the BF16 row of
// its table, 512 B per head per token at D = 256).
//
// A (layer, KV head) block holds K token-major (row t: D bf16 at 2Dt), which
// is a plain copy of each appended row, and V dim-major (row d: the 64 slots
// of dim d at 128D + 128d), which is a transpose: the page's appended V rows
// are staged in LDS as [dim][slot] and written back a dim row at a time, in
// 16-byte pieces where all eight slots of a piece are appended.
//
// One workgroup of 256 threads per (sequence, page touched, KV head); only
// the slots of the appended range are written.  The same kernel fills the
// exact window of a 2-bit window pool: the block of the last page an append
// reaches goes to the (sequence, layer, head) window block instead of the
// page ("The KV cache and prompt reuse", section "What a sequence is made
// of": the most recent keys are held unquantized).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

template <int D, bool WINDOW>
__global__ __launch_bounds__(256) void append_bf16_kernel(PoolView pv, int layer, BatchDesc bd,
                                                          const uint16_t* __restrict__ kin,
                                                          const uint16_t* __restrict__ vin) {
    constexpr int CH = D / 8;        // 16-byte pieces of a row
    constexpr int VS = PAGE + 8;     // padded slot row of the staged V, bf16 elements
    const int x = blockIdx.x, head = blockIdx.y;
    int e = 0;
    while (e + 1 < bd.n && bd.work0[e + 1] <= x) ++e;
    const int start = bd.pos[e], cnt = bd.cnt[e];
    const int lp = start / PAGE + (x - bd.work0[e]);
    const int slot_lo = max(start, lp * PAGE) - lp * PAGE;
    const int slot_hi = min(start + cnt, (lp + 1) * PAGE) - lp * PAGE;
    uint8_t* blk;
    if constexpr (WINDOW) {
        blk = window_block(pv, bd.seq[e], layer, head);
    } else {
        const int phys = pv.bt[(int64_t)bd.seq[e] * pv.bt_stride + lp];
        blk = pv.pages + (int64_t)phys * pv.page_bytes + ((int64_t)layer * pv.Hkv + head) * pv.block_bytes;
    }
    const int64_t row_of_slot0 = (int64_t)bd.row0[e] + (lp * PAGE - start);  // input row of slot 0 (may be < 0)

    __shared__ __align__(16) uint16_t vt[D * VS];

    // K: copy; V: transpose into LDS
    for (int i = threadIdx.x; i < PAGE * CH; i += 256) {
        const int s = i / CH, c = i % CH;
        if (s < slot_lo || s >= slot_hi) continue;
        const int64_t off = ((row_of_slot0 + s) * pv.Hkv + head) * D + 8 * c;
        const uint4 kw = *reinterpret_cast<const uint4*>(kin + off);
        *reinterpret_cast<uint4*>(blk + 2 * ((int64_t)s * D + 8 * c)) = kw;
        const uint4 vw = *reinterpret_cast<const uint4*>(vin + off);
        const uint32_t u[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            vt[(8 * c + 2 * k) * VS + s] = (uint16_t)(u[k] & 0xFFFF);
            vt[(8 * c + 2 * k + 1) * VS + s] = (uint16_t)(u[k] >> 16);
        }
    }
    __syncthreads();
    // V rows: piece (d, p) holds slots 8p .. 8p + 7 of dim d
    uint8_t* vplane = blk + 128 * (int64_t)D;
    for (int i = threadIdx.x; i < D * (PAGE / 8); i += 256) {
        const int d = i >> 3, p = i & 7;
        const int s0 = 8 * p;
        if (s0 + 7 < slot_lo || s0 >= slot_hi) continue;
        uint16_t* dst = reinterpret_cast<uint16_t*>(vplane + 128 * (int64_t)d) + s0;
        const uint16_t* src = &vt[d * VS + s0];
        if (s0 >= slot_lo && s0 + 8 <= slot_hi) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (s0 + k >= slot_lo && s0 + k < slot_hi) dst[k] = src[k];
        }
    }
}

hipError_t launch_append_bf16(const PoolView& pv, int layer, const BatchDesc& bd, int work_items, const uint16_t* k,
                              const uint16_t* v, hipStream_t s) {
    dim3 grid(work_items, pv.Hkv);
    if (pv.D == 256)
        hipLaunchKernelGGL((append_bf16_kernel<256, false>), grid, dim3(256), 0, s, pv, layer, bd, k, v);
    else
        hipLaunchKernelGGL((append_bf16_kernel<128, false>), grid, dim3(256), 0, s, pv, layer, bd, k, v);
    return hipGetLastError();
}

hipError_t launch_append_window(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* k,
                                const uint16_t* v, hipStream_t s) {
    dim3 grid(bd.n, pv.Hkv);
    if (pv.D == 256)
        hipLaunchKernelGGL((append_bf16_kernel<256, true>), grid, dim3(256), 0, s, pv, layer, bd, k, v);
    else
        hipLaunchKernelGGL((append_bf16_kernel<128, true>), grid, dim3(256), 0, s, pv, layer, bd, k, v);
    return hipGetLastError();
}

}  // namespace kvq
