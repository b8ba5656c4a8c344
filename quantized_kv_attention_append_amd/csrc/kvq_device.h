// Device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Load n consecutive bf16 values (n = 2 or 4) as fp32.
template <int N>
__device__ __forceinline__ void load_bf16(const uint16_t* p, float (&x)[N]) {
    if constexpr (N == 4) {
        uint2 w = *reinterpret_cast<const uint2*>(p);
        x[0] = bf16lo(w.x); x[1] = bf16hi(w.x); x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
    } else if constexpr (N == 2) {
        uint32_t w = *reinterpret_cast<const uint32_t*>(p);
        x[0] = bf16lo(w); x[1] = bf16hi(w);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = bf16_to_f32(p[i]);
    }
}

// Unnormalised Walsh-Hadamard transform of a row spread over the 16 lanes of a
// DPP row (lane c holds dims c DPL .. c DPL + DPL - 1), for the rotated
// variant: stages h = 1, 2, .., D/2 in that order, each replacing (x_i,
// x_{i+h}) by (x_i + x_{i+h}, x_i - x_{i+h}) with one fp32 rounding; stages
// h < DPL stay inside the lane, the others pair lane c with lane c ^ (h / DPL).
template <int DPL>
__device__ __forceinline__ void hadamard_row16(float (&x)[DPL], int c) {
#pragma clang fp contract(off)
#pragma unroll
    for (int h = 1; h < DPL; h *= 2)
#pragma unroll
        for (int i = 0; i < DPL; ++i)
            if (!(i & h)) {
                const float a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
#pragma unroll
    for (int m = 1; m < 16; m *= 2) {
        const bool upper = (c & m) != 0;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
            const float o = __shfl_xor(x[i], m);
            x[i] = upper ? o - x[i] : x[i] + o;
        }
    }
}

}  // namespace kvq
