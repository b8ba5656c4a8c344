// Measurement probes for bench.py (libkvq_probe.so, not part of the library's
// C ABI): what this chip sustains on the access pattern and the instruction
// the attention kernels use, so that their figures can be read as a
// fraction of a measured ceiling as well as of the published peak.
//
//   kvq_probe_read_stream: a plain read of `bytes` bytes (16-byte
//     nontemporal loads, one in flight per lane, grid-stride over `grid`
//     workgroups of 256 threads): the streaming read rate.
//   kvq_probe_read_blocks: the 2-bit decode's read pattern without its
//     arithmetic: for every (lane, KV head, split) one workgroup of four
//     waves reads its pages' (layer, head) blocks of `block` bytes, two
//     blocks in flight per wave, pages through the block tables;
//     kvq_probe_read_blocks_lds: the same reads staged through LDS by DMA
//     loads, two page pairs in flight a wave (how the decode stages them).
//   kvq_probe_mfma_bf16: back-to-back bf16 matrix-core products (16x16x32
//     or 32x32x16, several independent chains) on register operands in every
//     wave of `grid` workgroups of 256 threads, no memory traffic: the dense
//     bf16 matrix-core rate.
// Each enqueues one kernel on `stream` and returns a hipError_t.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// keeps the loads alive: a store that practically never happens
__device__ __forceinline__ void sink(v4u acc, uint32_t* out) {
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) out[threadIdx.x] = acc.x;
}

__global__ __launch_bounds__(256) void read_stream_kernel(const v4u* __restrict__ src, int64_t n, uint32_t* out) {
    const int64_t step = (int64_t)gridDim.x * 256;
    v4u acc = {0, 0, 0, 0};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += step) acc ^= __builtin_nontemporal_load(src + i);
    sink(acc, out);
}

// blockIdx.x = (lane * heads + head) * splits + split.  Wave w of the four
// reads blocks b0 + w + 8k and, in flight beside each, b0 + w + 4 + 8k: all
// PIECES 16-byte loads of a lane for both blocks are issued before any is
// used (the decode keeps a page pair in flight while it computes another).
template <int PIECES>
__global__ __launch_bounds__(256) void read_blocks_kernel(const uint8_t* __restrict__ pool, const int32_t* __restrict__ bt,
                                                          int pages_per_lane, int heads, int splits, int64_t page_bytes,
                                                          int64_t layer_off, uint32_t* out) {
    constexpr int BLOCK = PIECES * 1024;
    const int sp = blockIdx.x % splits, lh = blockIdx.x / splits, lane = lh / heads, head = lh % heads;
    const int per = (pages_per_lane + splits - 1) / splits;
    const int b0 = sp * per, b1 = min(b0 + per, pages_per_lane);
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t off = layer_off + (int64_t)head * BLOCK;
    v4u acc = {0, 0, 0, 0};
    for (int b = b0 + wave; b < b1; b += 8) {
        const bool two = b + 4 < b1;
        const v4u* s0 = reinterpret_cast<const v4u*>(pool + (int64_t)bt[lane * pages_per_lane + b] * page_bytes + off);
        const v4u* s1 = two ? reinterpret_cast<const v4u*>(pool + (int64_t)bt[lane * pages_per_lane + b + 4] * page_bytes + off)
                            : s0;
        v4u x[PIECES], y[PIECES];
#pragma unroll
        for (int p = 0; p < PIECES; ++p) x[p] = __builtin_nontemporal_load(s0 + l + 64 * p);
        if (two) {
#pragma unroll
            for (int p = 0; p < PIECES; ++p) y[p] = __builtin_nontemporal_load(s1 + l + 64 * p);
#pragma unroll
            for (int p = 0; p < PIECES; ++p) acc ^= y[p];
        }
#pragma unroll
        for (int p = 0; p < PIECES; ++p) acc ^= x[p];
    }
    sink(acc, out);
}

// The same block reads staged the way the 2-bit decode stages them: each
// wave copies a page's 9,216-byte block pair into its own LDS slots with DMA
// loads (global -> LDS, issued in inline asm, no registers held in flight),
// two slots a wave, reads a slot back and issues the DMA of the pair after
// next into it; no arithmetic.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
__device__ __forceinline__ void dma_block9k(const uint8_t* base, uint32_t v0, uint32_t lds) {
    const uint32_t v1 = v0 + 4096, v2 = v0 + 8192, l1 = lds + 4096, l2 = lds + 8192;
    uint32_t saved;
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[l0]\n\t"
        "global_load_lds_dwordx4 %[v0], %[b] nt\n\t"
        "global_load_lds_dwordx4 %[v0], %[b] offset:1024 nt\n\t"
        "global_load_lds_dwordx4 %[v0], %[b] offset:2048 nt\n\t"
        "global_load_lds_dwordx4 %[v0], %[b] offset:3072 nt\n\t"
        "s_mov_b32 m0, %[l1]\n\t"
        "global_load_lds_dwordx4 %[v1], %[b] nt\n\t"
        "global_load_lds_dwordx4 %[v1], %[b] offset:1024 nt\n\t"
        "global_load_lds_dwordx4 %[v1], %[b] offset:2048 nt\n\t"
        "global_load_lds_dwordx4 %[v1], %[b] offset:3072 nt\n\t"
        "s_mov_b32 m0, %[l2]\n\t"
        "global_load_lds_dwordx4 %[v2], %[b] nt\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [b] "s"(base), [v0] "v"(v0), [v1] "v"(v1), [v2] "v"(v2), [l0] "s"(lds), [l1] "s"(l1), [l2] "s"(l2)
        : "memory");
}

// blockIdx.x = (lane * heads + head) * splits + split; pairs of pages.
__global__ __launch_bounds__(256) void read_blocks_lds_kernel(const uint8_t* __restrict__ pool,
                                                              const int32_t* __restrict__ bt, int pages_per_lane,
                                                              int heads, int splits, int64_t page_bytes,
                                                              int64_t layer_off, uint32_t* out) {
    constexpr int BLK = 9216, TB = 2 * BLK;
    __shared__ __align__(16) uint8_t sl[4][2][TB];
    const int sp = blockIdx.x % splits, lh = blockIdx.x / splits, lane = lh / heads, head = lh % heads;
    const int pairs = pages_per_lane / 2, per = (pairs + splits - 1) / splits;
    const int pr0 = sp * per, pr1 = min(pr0 + per, pairs);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int64_t off = layer_off + (int64_t)head * BLK;
    const __attribute__((address_space(4))) int32_t* lbt =
        (const __attribute__((address_space(4))) int32_t*)(bt + lane * pages_per_lane);
    const uint32_t v0 = 16 * l;
    auto issue = [&](int s, int p) {
        const uint32_t la = lds_addr(sl[wave][s]);
        dma_block9k(pool + (int64_t)lbt[2 * p] * page_bytes + off, v0, la);
        dma_block9k(pool + (int64_t)lbt[2 * p + 1] * page_bytes + off, v0, la + BLK);
    };
    v4u acc = {0, 0, 0, 0};
    int p = pr0 + wave;
    if (p < pr1) issue(0, p);
    if (p + 4 < pr1) issue(1, p + 4);
    for (int t = 0; p < pr1; p += 4, ++t) {
        if (p + 4 < pr1) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int s = t & 1;
        v4u x[18];
#pragma unroll
        for (int i = 0; i < 18; ++i) x[i] = *reinterpret_cast<const v4u*>(&sl[wave][s][1024 * i + 16 * l]);
        if (p + 8 < pr1) issue(s, p + 8);
#pragma unroll
        for (int i = 0; i < 18; ++i) acc ^= x[i];
    }
    sink(acc, out);
}

// SHAPE 0: v_mfma_f32_16x16x32_bf16; SHAPE 1: v_mfma_f32_32x32x16_bf16.
// CHAINS independent accumulators a wave, so the matrix core never waits on
// a result.
template <int SHAPE, int CHAINS>
__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, float* out) {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (threadIdx.x + i));
        b[i] = (__bf16)(0.002f * (i + 1));
    }
    float s = 0.f;
    if constexpr (SHAPE == 0) {
        f32x4 c[CHAINS];
#pragma unroll
        for (int k = 0; k < CHAINS; ++k) c[k] = f32x4{0, 0, 0, 0};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int k = 0; k < CHAINS; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
#pragma unroll
        for (int k = 0; k < CHAINS; ++k) s += c[k][k % 4];
    } else {
        typedef float f32x16 __attribute__((ext_vector_type(16)));
        f32x16 c[CHAINS];
#pragma unroll
        for (int k = 0; k < CHAINS; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) c[k][r] = 0.f;
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int k = 0; k < CHAINS; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
#pragma unroll
        for (int k = 0; k < CHAINS; ++k) s += c[k][k % 16];
    }
    if (s == 1234.5f) out[threadIdx.x] = s;
}

}  // namespace

extern "C" {

int kvq_probe_read_stream(const void* src, int64_t bytes, int grid, void* out, void* stream) {
    hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const v4u*>(src), bytes / 16, reinterpret_cast<uint32_t*>(out));
    return (int)hipGetLastError();
}

int kvq_probe_read_blocks(const void* pool, const int32_t* bt, int lanes, int pages_per_lane, int heads, int splits,
                          int64_t page_bytes, int64_t layer_off, int block, void* out, void* stream) {
    const dim3 grid(lanes * heads * splits);
    if (block == 9216)
        hipLaunchKernelGGL(read_blocks_kernel<9>, grid, dim3(256), 0, (hipStream_t)stream,
                           reinterpret_cast<const uint8_t*>(pool), bt, pages_per_lane, heads, splits, page_bytes,
                           layer_off, reinterpret_cast<uint32_t*>(out));
    else if (block == 5120)
        hipLaunchKernelGGL(read_blocks_kernel<5>, grid, dim3(256), 0, (hipStream_t)stream,
                           reinterpret_cast<const uint8_t*>(pool), bt, pages_per_lane, heads, splits, page_bytes,
                           layer_off, reinterpret_cast<uint32_t*>(out));
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

// The pattern through LDS DMA, as the decode stages it (9,216-byte blocks,
// an even page count a lane).
int kvq_probe_read_blocks_lds(const void* pool, const int32_t* bt, int lanes, int pages_per_lane, int heads,
                              int splits, int64_t page_bytes, int64_t layer_off, void* out, void* stream) {
    if (pages_per_lane % 2) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_blocks_lds_kernel, dim3(lanes * heads * splits), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint8_t*>(pool), bt, pages_per_lane, heads, splits, page_bytes, layer_off,
                       reinterpret_cast<uint32_t*>(out));
    return (int)hipGetLastError();
}

// shape 0: 16x16x32 (32,768 flops a product), 1: 32x32x16 (32,768 flops a
// product); flops of one call: grid * 4 waves * iters * chains * 32,768.
int kvq_probe_mfma_bf16(int shape, int chains, int grid, int iters, void* out, void* stream) {
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, reinterpret_cast<float*>(out));
    };
    if (shape == 0 && chains == 4) go(mfma_bf16_kernel<0, 4>);
    else if (shape == 0 && chains == 8) go(mfma_bf16_kernel<0, 8>);
    else if (shape == 1 && chains == 2) go(mfma_bf16_kernel<1, 2>);
    else if (shape == 1 && chains == 4) go(mfma_bf16_kernel<1, 4>);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // extern "C"
