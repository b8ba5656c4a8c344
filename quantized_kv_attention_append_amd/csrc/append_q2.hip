// Quantize-on-append for the 2-bit format, and page dequantization.
//
// The row format follows the byte budget of "KV at 9 KB a token" (section "How
// it works", table): per (token, KV head), D/4 bytes of 2-bit code plus an
// 8-byte metadata row [fp32 scale, fp32 min].  The codebook is uniform over
// the row's range:
//     mn = min x, mx = max x, scale = (mx - mn) / 3 (correctly rounded fp32),
//     scale == 0 -> 1.0, code = clamp(rint((x - mn) / scale), 0, 3)
// and the dequantized value is fmaf(code, scale, mn).  Every step is a single
// IEEE fp32 operation with round-to-nearest-even, so the codes and metadata are
// a pure function of the bf16 inputs (min and max do not depend on reduction
// order).  A zero min or max is canonicalised to +0.
//
// Layout of one (layer, KV head) block of a page: K codes token-major (row t =
// D/4 bytes, dim j at bit 2*(j%4) of byte j/4), V codes dim-major (four 32-bit
// words per dim holding the 64 token slots; slot 16b + 4w + r sits in word w at
// bit 16(r%2) + 4b + 2(r/2); words placed by q2_vword_off), then 64 K metadata
// rows and 64 V metadata rows.  K rows are read by token for the q.k
// contraction over dims; V rows by dim for the p.v contraction over tokens,
// and masking a V word with 0x33333333 (or its shift right by two) yields
// eight slots, one per 4-bit nibble, which is the matrix-core operand format
// the decode kernel feeds from it.
//
// Work split: one workgroup of four waves per (sequence, page touched, KV
// head); wave w owns the token slots of V word w (slots s with (s/4)%4 == w),
// so the V plane is written with one read-modify-write per (dim, word) and no
// two workgroups or waves share a byte.  A row is spread over the 16 lanes of
// a DPP row, so a wave quantizes four rows at once and its min / max
// reductions stay inside DPP rows.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// Extreme of a row held by the 16 lanes of a DPP row: butterflies with quad
// permutes, then rotations by 4 and 8; every lane of the row ends with it.
template <bool MAX>
__device__ __forceinline__ float row16_extreme(float v) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
    auto dpp = [](float x, auto ctrl_tag) {
        constexpr int CTRL = decltype(ctrl_tag)::value;
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
    };
    v = op(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1, 0, 3, 2]
    v = op(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2, 3, 0, 1]
    v = op(v, dpp(v, std::integral_constant<int, 0x124>{}));  // row_ror 4
    v = op(v, dpp(v, std::integral_constant<int, 0x128>{}));  // row_ror 8
    return v;
}

// Quantize one row spread over the 16 lanes of a DPP row, DPL consecutive
// elements per lane.  Returns the lane's codes; scale and mn are the same in
// every lane of the row.
template <int DPL>
__device__ __forceinline__ void q2_quantize_row(const float (&x)[DPL], uint32_t (&c)[DPL], float& scale, float& mn) {
#pragma clang fp contract(off)
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int k = 1; k < DPL; ++k) {
        lo = fminf(lo, x[k]);
        hi = fmaxf(hi, x[k]);
    }
    lo = row16_extreme<false>(lo) + 0.0f;
    hi = row16_extreme<true>(hi) + 0.0f;
    float sc = (hi - lo) / 3.0f;
    if (sc == 0.0f) sc = 1.0f;
    // code = clamp(rint(RN(RN(x - mn) / sc)), 0, 3).  Only the rounded integer
    // is kept, so the quotient is first taken as d * rcp(sc): that is within
    // 6.6e-7 of the correctly rounded quotient (rcp within one ulp, the product
    // within half an ulp, the quotient below 3.000001), so unless it lies
    // within 2e-6 of a half-integer both round to the same code.  The rare
    // element that does takes the correctly rounded division, and so does
    // every element of a row whose scale lies outside [2^-120, 2^120]: there
    // the reciprocal can overflow (a subnormal scale) or lose its bound (a
    // subnormal reciprocal).
    // Here the clamp to 0..3 cannot bind: d = RN(x - mn) >= 0 and the reciprocal
    // is positive, and d <= RN(mx - mn) with sc = RN(RN(mx - mn) / 3), so the
    // quotient is below 3.000001 and rounds to at most 3 (a zero range gives
    // d = 0; scales outside [2^-120, 2^120] take the division below, which
    // clamps).
    const float inv = __builtin_amdgcn_rcpf(sc);
    bool near = !(sc >= 0x1p-120f && sc <= 0x1p120f);
    float d[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        d[k] = x[k] - lo;
        const float ta = d[k] * inv;
        const float ra = rintf(ta);
        near |= fabsf(ta - ra) > 0.5f - 2e-6f;  // within 2e-6 of a half-integer
        c[k] = (uint32_t)ra;
    }
    if (__builtin_amdgcn_ballot_w64(near)) {
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
            const float t = d[k] / sc;
            c[k] = (uint32_t)fminf(fmaxf(rintf(t), 0.0f), 3.0f);
        }
    }
    scale = sc;
    mn = lo;
}

// N (8 or 16) consecutive bf16 values as fp32, in 16-byte loads
template <int N>
__device__ __forceinline__ void load_bf16_rows(const uint16_t* p, float (&x)[N]) {
    static_assert(N % 8 == 0, "whole 16-byte chunks");
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
        const uint4 w = reinterpret_cast<const uint4*>(p)[i];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[8 * i + 2 * k] = __uint_as_float(u[k] << 16);
            x[8 * i + 2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
        }
    }
}

template <int D, bool ROT>
__global__ __launch_bounds__(256) void append_q2_kernel(PoolView pv, int layer, BatchDesc bd,
                                                        const uint16_t* __restrict__ kin,
                                                        const uint16_t* __restrict__ vin) {
    constexpr int DPL = D / 16;  // dims of a lane: a row is spread over 16 lanes
    const int x = blockIdx.x, head = blockIdx.y;
    int e = 0;
    while (e + 1 < bd.n && bd.work0[e + 1] <= x) ++e;
    const int start = bd.pos[e], cnt = bd.cnt[e];
    const int lp = start / PAGE + (x - bd.work0[e]);
    const int slot_lo = max(start, lp * PAGE) - lp * PAGE;
    const int slot_hi = min(start + cnt, (lp + 1) * PAGE) - lp * PAGE;
    const int phys = pv.bt[(int64_t)bd.seq[e] * pv.bt_stride + lp];
    uint8_t* blk = pv.pages + (int64_t)phys * pv.page_bytes + ((int64_t)layer * pv.Hkv + head) * pv.block_bytes;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4, c = lane & 15;

    uint32_t vw[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) vw[k] = 0;
    uint32_t vmask = 0;
    // this wave's slots 16b + 4 * wave + r; step b takes the four r at once,
    // lane group r (16 lanes, DPL dims each) holding slot 16b + 4 * wave + r
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int s0 = 16 * b + 4 * wave;
        if (s0 + 3 < slot_lo || s0 >= slot_hi) continue;  // none of the four appended
        const int s = s0 + grp;
        const bool in = s >= slot_lo && s < slot_hi;
        const int sl = in ? s : max(s0, slot_lo);  // a slot outside the range re-reads one inside it, unused
        const int64_t row = (int64_t)bd.row0[e] + (lp * PAGE + sl - start);
        const int64_t off = (row * pv.Hkv + head) * D + c * DPL;
        float xk[DPL], xv[DPL];
        load_bf16_rows<DPL>(kin + off, xk);
        load_bf16_rows<DPL>(vin + off, xv);
        if constexpr (ROT) hadamard_row16<DPL>(xk, c);  // the rotated variant quantizes H k (V as given)
        uint32_t ck[DPL], cv[DPL];
        float sk, mk, sv, mv;
        q2_quantize_row<DPL>(xk, ck, sk, mk);
        q2_quantize_row<DPL>(xv, cv, sv, mv);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (s0 + r >= slot_lo && s0 + r < slot_hi) vmask |= 3u << q2_vslot_bit(s0 + r);
        if (in) {
            // K row: dim j at bit 2(j % 4) of byte j / 4, so this lane's DPL dims are
            // 2 DPL bits at byte DPL / 4 * c
            uint32_t bits = 0;
#pragma unroll
            for (int k = 0; k < DPL; ++k) bits |= ck[k] << (2 * k);
            uint8_t* krow = blk + (int64_t)s * (D / 4);
            if constexpr (DPL == 16)
                reinterpret_cast<uint32_t*>(krow)[c] = bits;
            else
                reinterpret_cast<uint16_t*>(krow)[c] = (uint16_t)bits;
            const int sh = q2_vslot_bit(s);
#pragma unroll
            for (int k = 0; k < DPL; ++k) vw[k] |= cv[k] << sh;
            if (c == 0) {
                *reinterpret_cast<float2*>(blk + q2_kmeta_off(D) + 8 * s) = make_float2(sk, mk);
                *reinterpret_cast<float2*>(blk + q2_vmeta_off(D) + 8 * s) = make_float2(sv, mv);
            }
        }
    }
    if (vmask == 0) return;
    // the four lane groups hold disjoint slots of the same dims: OR them, then
    // the first group writes word `wave` of each of the lane's dims
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        vw[k] |= __shfl_xor(vw[k], 16);
        vw[k] |= __shfl_xor(vw[k], 32);
    }
    if (grp != 0) return;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        const int d = c * DPL + k;
        uint32_t* p = reinterpret_cast<uint32_t*>(blk + q2_vcodes_off(D) + q2_vword_off(D, d, wave));
        uint32_t old = (vmask == 0xFFFFFFFFu) ? 0u : *p;
        *p = (old & ~vmask) | vw[k];
    }
}

hipError_t launch_append_q2(const PoolView& pv, int layer, const BatchDesc& bd, int work_items, const uint16_t* k,
                            const uint16_t* v, hipStream_t s, bool rot) {
    dim3 grid(work_items, pv.Hkv);
    auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, pv, layer, bd, k, v); };
    if (pv.D == 256)
        rot ? go(append_q2_kernel<256, true>) : go(append_q2_kernel<256, false>);
    else
        rot ? go(append_q2_kernel<128, true>) : go(append_q2_kernel<128, false>);
    return hipGetLastError();
}

// ------------------------------------------------------------ dequant ----

__global__ __launch_bounds__(256) void dequant_page_kernel(PoolView pv, int fmt, int page, int layer, int head, int kv,
                                                           float* __restrict__ out) {
    const int D = pv.D;
    const uint8_t* blk = pv.pages + (int64_t)page * pv.page_bytes + ((int64_t)layer * pv.Hkv + head) * pv.block_bytes;
    for (int i = threadIdx.x; i < PAGE * D; i += blockDim.x) {
        const int t = i / D, d = i % D;
        float r;
        if (fmt == KV_FMT_Q2) {
            uint32_t c;
            float2 meta;
            if (kv == 0) {
                c = (blk[t * (D / 4) + d / 4] >> (2 * (d % 4))) & 3u;
                meta = *reinterpret_cast<const float2*>(blk + q2_kmeta_off(D) + 8 * t);
            } else {
                const uint32_t word = *reinterpret_cast<const uint32_t*>(blk + q2_vcodes_off(D) +
                                                                         q2_vword_off(D, d, q2_vslot_word(t)));
                c = (word >> q2_vslot_bit(t)) & 3u;
                meta = *reinterpret_cast<const float2*>(blk + q2_vmeta_off(D) + 8 * t);
            }
            r = __fmaf_rn((float)c, meta.x, meta.y);
        } else if (fmt == KV_FMT_BF16) {
            const uint16_t* vals = reinterpret_cast<const uint16_t*>(blk);
            r = bf16_to_f32(kv == 0 ? vals[t * D + d] : vals[64 * D + PAGE * d + t]);
        } else {
            if (kv == 0) {
                int8_t c = (int8_t)blk[t * D + d];
                r = (float)c * *reinterpret_cast<const float*>(blk + q8_kscale_off(D) + 4 * d);
            } else {
                int8_t c = (int8_t)blk[q8_vcodes_off(D) + 64 * d + t];
                r = (float)c * *reinterpret_cast<const float*>(blk + q8_vscale_off(D) + 4 * t);
            }
        }
        out[i] = r;
    }
}

hipError_t launch_dequant_page(const PoolView& pv, int fmt, int page, int layer, int head, int kv, float* out,
                               hipStream_t s) {
    hipLaunchKernelGGL(dequant_page_kernel, dim3(1), dim3(256), 0, s, pv, fmt, page, layer, head, kv, out);
    return hipGetLastError();
}

}  // namespace kvq
