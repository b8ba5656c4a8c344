// Quantize-on-append for the 8-bit variant: V per token, K per channel over
// the tokens present in the open page ("The KV cache and prompt reuse",
// section "What a sequence is made of": the compressed format keeps a window
// of exact recent keys; "Half the Cache, Twice the Context", section on
// per-channel keys and per-token values, symmetric absmax at 127 levels).
//
//   V row x (one token, one KV head): s = max|x| / 127 (correctly rounded
//     fp32), s == 0 -> 1, c_d = clamp(rint(x_d / s), -127, 127).
//   K channel j of a page: s_j = max over the page's present tokens t of
//     |k_tj| / 127, c_tj = clamp(rint(k_tj / s_j), -127, 127).
// The exact bf16 K rows of the open page are kept in a staging page per
// (sequence, layer, KV head); every append re-derives the codes of all the
// page's present tokens and its channel scales from them, so a page that
// reaches 64 tokens holds exactly the per-channel quantization of its 64
// tokens.
//
// Block layout (D dims): K codes int8 token-major [64][D] at 0, V codes int8
// dim-major [D][64] at 64D, K scales fp32 [D] at 128D, V scales fp32 [64] at
// 132D.
//
// One workgroup of 256 threads per (sequence, page touched, KV head); K
// channels take 256 / D threads each (token ranges whose absmax meet in LDS),
// V codes are staged dim-major in LDS and written in 4-byte runs of slots.  The
// host never launches a page that reads staged rows together with a later
// page of the same sequence that rewrites them (it splits such an append in
// two launches), so staging reads and writes never race.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// clamp(rint(RN(x / s)), -127, 127).  Only the rounded integer is kept, so
// the quotient is first taken as x * rcp(s): within 2.7e-5 of the correctly
// rounded quotient (rcp within one ulp, the product within half an ulp, the
// quotient at most 127.0001 in size), so unless it lies within 1e-4 of a
// half-integer both round to the same integer; the rare element that does
// takes the correctly rounded division, and so does every element whose
// scale lies outside [2^-120, 2^120] (where the reciprocal can overflow or be
// subnormal).
__device__ __forceinline__ int8_t q8_code(float x, float s, float inv) {
#pragma clang fp contract(off)
    const float qa = x * inv;
    float r = rintf(qa);
    if (!(s >= 0x1p-120f && s <= 0x1p120f) || fabsf(qa - r) > 0.5f - 1e-4f) r = rintf(x / s);
    return (int8_t)fminf(fmaxf(r, -127.0f), 127.0f);
}

template <int D>
__global__ __launch_bounds__(256) void append_q8_kernel(PoolView pv, int layer, BatchDesc bd,
                                                        const uint16_t* __restrict__ kin,
                                                        const uint16_t* __restrict__ vin) {
#pragma clang fp contract(off)
    constexpr int DPL = D / 64;  // dims per lane in a row-wide wave operation
    const int x = blockIdx.x, head = blockIdx.y;
    int e = 0;
    while (e + 1 < bd.n && bd.work0[e + 1] <= x) ++e;
    const int start = bd.pos[e], cnt = bd.cnt[e];
    const int lp = start / PAGE + (x - bd.work0[e]);
    const int slot_lo = max(start, lp * PAGE) - lp * PAGE;
    const int slot_hi = min(start + cnt, (lp + 1) * PAGE) - lp * PAGE;
    const int phys = pv.bt[(int64_t)bd.seq[e] * pv.bt_stride + lp];
    uint8_t* blk = pv.pages + (int64_t)phys * pv.page_bytes + ((int64_t)layer * pv.Hkv + head) * pv.block_bytes;
    uint16_t* stage = pv.stage + ((((int64_t)bd.seq[e] * pv.L + layer) * pv.Hkv + head) * PAGE) * D;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    auto in_row = [&](int s) { return ((int64_t)bd.row0[e] + (lp * PAGE + s - start)) * pv.Hkv + head; };

    // exact K rows of slots [0, slot_hi) as bf16 bits: earlier slots from the
    // staging page (16-byte pieces: the staging rows are the bulk of a short
    // append), the new ones from the input
    __shared__ __align__(16) uint16_t k_s[PAGE][D];
    constexpr int PR = D / 8;  // 16-byte pieces of a row
    for (int i = tid; i < slot_lo * PR; i += 256) {
        const int s = i / PR, c = i - s * PR;
        *reinterpret_cast<uint4*>(&k_s[s][8 * c]) = *reinterpret_cast<const uint4*>(stage + (int64_t)s * D + 8 * c);
    }
    for (int i = tid; i < (slot_hi - slot_lo) * D; i += 256) {
        const int s = slot_lo + i / D, d = i % D;
        k_s[s][d] = kin[in_row(s) * D + d];
    }
    __syncthreads();
    // the page stays open: keep its new exact rows for the next append
    if (slot_hi < PAGE)
        for (int i = tid; i < (slot_hi - slot_lo) * D; i += 256) {
            const int s = slot_lo + i / D, d = i % D;
            stage[(int64_t)s * D + d] = k_s[s][d];
        }

    // ---- K: per-channel scales and the codes of every present token; TPD
    // threads per channel, each a range of tokens ----
    constexpr int TPD = 256 / D;
    __shared__ float kamax_s[TPD][D];
    __shared__ __align__(16) int8_t vq_s[D][PAGE];  // this append's V codes, dim-major
    int8_t* kc = reinterpret_cast<int8_t*>(blk);
    float* ks = reinterpret_cast<float*>(blk + q8_kscale_off(D));
    {
        const int d = tid % D, part = tid / D;
        const int t0 = part * (PAGE / TPD), t1 = min(t0 + PAGE / TPD, slot_hi);
        float amax = 0.f;
        for (int s = t0; s < t1; ++s) amax = fmaxf(amax, fabsf(bf16_to_f32(k_s[s][d])));
        if constexpr (TPD > 1) {
            kamax_s[part][d] = amax;
            __syncthreads();
#pragma unroll
            for (int p = 0; p < TPD; ++p) amax = fmaxf(amax, kamax_s[p][d]);
        }
        float sc = amax / 127.0f;
        if (sc == 0.0f) sc = 1.0f;
        if (part == 0) ks[d] = sc;
        const float inv = __builtin_amdgcn_rcpf(sc);
        for (int s = t0; s < t1; ++s) kc[s * D + d] = q8_code(bf16_to_f32(k_s[s][d]), sc, inv);
    }

    // ---- V: per-token scale; wave w takes slots slot_lo + w, + 4, ...; codes
    // go to LDS dim-major, then out in 4-byte runs of slots ----
    float* vs = reinterpret_cast<float*>(blk + q8_vscale_off(D));
    for (int s = slot_lo + wave; s < slot_hi; s += 4) {
        float xv[DPL];
        load_bf16<DPL>(vin + in_row(s) * D + lane * DPL, xv);
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) amax = fmaxf(amax, fabsf(xv[k]));
        amax = wave_max(amax);
        float sc = amax / 127.0f;
        if (sc == 0.0f) sc = 1.0f;
        const float inv = __builtin_amdgcn_rcpf(sc);
#pragma unroll
        for (int k = 0; k < DPL; ++k) vq_s[lane * DPL + k][s] = q8_code(xv[k], sc, inv);
        if (lane == 0) vs[s] = sc;
    }
    __syncthreads();
    uint8_t* vc = blk + q8_vcodes_off(D);
    for (int i = tid; i < D * (PAGE / 4); i += 256) {
        const int d = i / (PAGE / 4), s4 = 4 * (i % (PAGE / 4));
        if (s4 + 3 < slot_lo || s4 >= slot_hi) continue;
        if (s4 >= slot_lo && s4 + 3 < slot_hi) {
            *reinterpret_cast<uint32_t*>(vc + d * PAGE + s4) = *reinterpret_cast<const uint32_t*>(&vq_s[d][s4]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (s4 + r >= slot_lo && s4 + r < slot_hi) vc[d * PAGE + s4 + r] = (uint8_t)vq_s[d][s4 + r];
        }
    }
}

hipError_t launch_append_q8(const PoolView& pv, int layer, const BatchDesc& bd, int work_items, const uint16_t* k,
                            const uint16_t* v, hipStream_t s) {
    dim3 grid(work_items, pv.Hkv);
    if (pv.D == 256)
        hipLaunchKernelGGL(append_q8_kernel<256>, grid, dim3(256), 0, s, pv, layer, bd, k, v);
    else
        hipLaunchKernelGGL(append_q8_kernel<128>, grid, dim3(256), 0, s, pv, layer, bd, k, v);
    return hipGetLastError();
}

}  // namespace kvq
