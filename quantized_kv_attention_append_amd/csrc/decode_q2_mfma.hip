// Split-K decode attention over the 2-bit pool on the gfx950 matrix cores
// (head_dim 128 or 256; four query heads of a KV head's group a workgroup, so
// groups 1 and 2 leave rows of the products empty and group 8 takes two
// workgroups a split, launched together so that the second reads the pages
// from L2).
//
// At group 4 and 256 dims a decode step does 2 x 4 x 256 multiply-adds for
// every 144 bytes of K and V rows it reads, more than the vector ALUs can
// sustain at full HBM bandwidth, so both contractions run on
// v_mfma_scale_f32_16x16x128_f8f6f4.  Its internal sum drops low-order bits
// of products much smaller than the largest product of a group, but sums
// small-integer products exactly, so every operand is made of small integers
// and every power of two goes into the instruction's per-row / per-column
// scale:
//   * 2-bit codes c become fp4 (e2m1) nibbles whose value is c/2: a 32-bit
//     word of 16 codes spreads into two words of nibbles with one shift and
//     two masks (w & 0x33333333, (w >> 2) & 0x33333333);
//   * the bf16 query of each head becomes a 19-bit fixed-point integer
//     round(q * 2^E) (exact unless |q| < max|q| / 2^11), written as four
//     balanced radix-32 digits in -16..16 (exact in e4m3); row 4h + i of the
//     q.k product is digit i of head h, weighted 32^(3-i) 2^-E by its scale;
//   * the softmax weights w_t = p_t * scale_t become 16-bit fixed-point
//     integers relative to each head's largest weight in a block of 32
//     tokens, split into four 4-bit digits.  An e4m3 byte 0..15 is exactly
//     b * 2^-9, so the digits go into the operand with byte shuffles only;
//     column 4h + i of the p.v product is digit i of head h, and its scale
//     for k-block b (32 tokens) weights it 16^i 2^-F(h, b).
// The dequantization is folded algebraically (q.k^_t = mn_t sum(q) + scale_t
// q.c_t; p.v^ = sum p_t mn_t + sum (p_t scale_t) c_t), and the online softmax,
// its rescaling and every running sum are fp32 registers (the two-level
// accumulation "Half the Cache, Twice the Context" asks for in section "The
// cliff is in the accumulator").
//
// One workgroup of eight wavefronts per (sequence, KV head, split); wave w
// takes every eighth pair of pages of the split (128 tokens = one k-block of
// the instruction).  A pair's two (layer, KV head) blocks are copied into the
// wave's LDS slot by DMA loads (global -> LDS), read from there into
// registers, and the next pair's DMA goes out while the wave computes; the
// eight waves combine their partial results in LDS.  Token t of the pair
// sits at page t/64, slot t%64.  Operand lane
// layouts of the instruction: fp4 lane group g holds k = 32g..32g+31; fp8
// lane group g holds k = 16g..16g+15 and 64+16g..64+16g+15; the result lane l
// holds column l%16, rows 4(l/16)..+3.
//   q.k (8 per tile): A = query digits (row 4h + i), B = K codes of tokens
//       16m..16m+15 of the pair (column j = token 16m + j, k = dims), so lane
//       l ends with the score of token 16m + l%16 for head l/16: every
//       (token, head) score of the tile is computed once, eight per lane.
//   p.v (D/16 per tile): A = V codes of 16 dims (k = tokens), B = weight
//       digits (column 4h + i).  The V words put token
//       64(g/2) + 16(t%4) + 8(g%2) + 4u + 2x + t/4 at k = 32g + 16u + 8x + t,
//       and a per-wave LDS transpose moves each lane's digit bytes of its
//       eight tokens to the lanes whose k-ranges hold those tokens.
#include <type_traits>

#include "decode_common.h"

namespace kvq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

constexpr int FMT_FP8 = 0;  // e4m3
constexpr int FMT_FP4 = 4;  // e2m1

// q.k: A = query digits (fp8) with per-row scale, B = K codes (fp4)
__device__ __forceinline__ v4f mma_qk(const v8i& a_fp8, const v8i& b_fp4, v4f c, int scale_a) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp8, b_fp4, c, FMT_FP8, FMT_FP4, 0, scale_a, 0, 127);
}
// p.v: A = V codes (fp4), B = weight digits (fp8) with per-column scale
__device__ __forceinline__ v4f mma_pv(const v8i& a_fp4, const v8i& b_fp8, v4f c, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp4, b_fp8, c, FMT_FP4, FMT_FP8, 0, 127, 0, scale_b);
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// 16 two-bit codes -> two words of eight e2m1 nibbles (value = code / 2).
__device__ __forceinline__ uint32_t nib_lo(uint32_t w) { return w & 0x33333333u; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t w) { return (w >> 2) & 0x33333333u; }

__device__ __forceinline__ v8i fp4_operand(uint32_t w0, uint32_t w1) {
    v8i r;
    r[0] = (int)nib_lo(w0);
    r[1] = (int)nib_hi(w0);
    r[2] = (int)nib_lo(w1);
    r[3] = (int)nib_hi(w1);
    r[4] = r[5] = r[6] = r[7] = 0;
    return r;
}

// Balanced radix-32 digits: x (|x| < 2^19 after scaling) is rounded to an
// integer n and n + DIGIT_BIAS is written in base 32 with fields f0 (6 bits,
// 0..32) f1 f2 f3; digit d = f_d - 16 lies in -16..16 and
// n = sum_d digit_d * 32^(3-d).  Adding 2^23 + DIGIT_BIAS to x in one fused
// multiply-add leaves n + DIGIT_BIAS in the low mantissa bits.
constexpr float DIGIT_BIAS = 541200.0f;  // 16 * (1 + 32 + 32^2 + 32^3)
constexpr float DIGIT_MAGIC = 8388608.0f + DIGIT_BIAS;
__device__ __forceinline__ float digit_of(float x, float scale, int d) {
    const uint32_t u = __float_as_uint(fmaf(x, scale, DIGIT_MAGIC));
    const int f = (int)__builtin_amdgcn_ubfe(u, 15 - 5 * d, d == 0 ? 6 : 5);
    return (float)(f - 16);
}
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }
__device__ __forceinline__ int exponent_of(float x) { return (int)((__float_as_uint(x) >> 23) & 0xFF) - 127; }

// Reductions over the 16 lanes of a DPP row (row_ror by 8, 4, 2, 1).
template <int CTRL>
__device__ __forceinline__ float ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, ror<0x128>(x));
    x = fmaxf(x, ror<0x124>(x));
    x = fmaxf(x, ror<0x122>(x));
    return fmaxf(x, ror<0x121>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
    x += ror<0x128>(x);
    x += ror<0x124>(x);
    x += ror<0x122>(x);
    return x + ror<0x121>(x);
}
// Max over the eight lanes of a half row (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror).
__device__ __forceinline__ float half_row_max8(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
}
// Fixed-point exponent F of a block of weights with max wmax: wmax 2^F in
// [2^15, 2^16), so X = round(w 2^F) fits 16 bits (capped at 2^16 - 1).  F is
// clamped to [-105, 126] so that the column scale 137 + 4i - F stays a valid
// power-of-two byte; weights above 2^120 are out of range.
__device__ __forceinline__ int weight_exp(float wmax) {
    return wmax > 0.f ? max(min(15 - exponent_of(wmax), 126), -105) : 0;
}
// Sum over the four lanes of a quad (quad_perm [1,0,3,2] then [2,3,0,1]).
__device__ __forceinline__ float quad_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// k index of byte s of an fp8 operand held by lane group grp.
__device__ __forceinline__ int fp8_k(int grp, int s) { return s < 16 ? 16 * grp + s : 64 + 16 * grp + (s - 16); }

}  // namespace

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// A head's reference max moves only when a tile's max exceeds it by more than
// 2^8 in weight, so the running sums are rescaled rarely (weights stay < 2^8).
constexpr float RESCALE_LOG2 = 8.0f;

// A tile is a pair of pages: the two (layer, KV head) blocks, byte for byte
// as they sit in the pool, copied into an LDS slot of the wave by DMA loads
// (global -> LDS, no registers held while they are in flight).
template <int D>
struct TileShape {
    static constexpr int BLK = (int)q2_block_bytes(D);  // 9,216 at D = 256
    static constexpr int BYTES = 2 * BLK;
    static constexpr int DMA = 2 * BLK / 1024;          // 16-byte DMA loads per lane and tile
};

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// One (layer, KV head) block copied to LDS at `lds` by one wave: lane l moves
// bytes 16 l + 1024 i.  The loads are issued in inline asm so that the
// compiler sees no LDS write in flight (it would otherwise wait for every
// outstanding DMA before any LDS read); the kernel places the waits itself.
// The instruction's immediate offset applies to both addresses (M0 + offset +
// 16 lane in LDS, base + voff + offset in memory) and is below 4,096, so the
// block goes in groups of four loads.  It first waits for every earlier LDS
// read of the wave to return, since the slot may be the one just read.  M0
// is saved and restored.
// NT: streaming (nontemporal) loads; without it the lines stay in L2 for a
// second workgroup that reads the same block soon after.
#define KVQ_DMA_256(NTS)                                                                     \
    "s_waitcnt lgkmcnt(0)\n\t"                                                              \
    "s_mov_b32 %[sv], m0\n\t"                                                               \
    "s_mov_b32 m0, %[l0]\n\t"                                                               \
    "global_load_lds_dwordx4 %[v0], %[b]" NTS "\n\t"                                        \
    "global_load_lds_dwordx4 %[v0], %[b] offset:1024" NTS "\n\t"                            \
    "global_load_lds_dwordx4 %[v0], %[b] offset:2048" NTS "\n\t"                            \
    "global_load_lds_dwordx4 %[v0], %[b] offset:3072" NTS "\n\t"                            \
    "s_mov_b32 m0, %[l1]\n\t"                                                               \
    "global_load_lds_dwordx4 %[v1], %[b]" NTS "\n\t"                                        \
    "global_load_lds_dwordx4 %[v1], %[b] offset:1024" NTS "\n\t"                            \
    "global_load_lds_dwordx4 %[v1], %[b] offset:2048" NTS "\n\t"                            \
    "global_load_lds_dwordx4 %[v1], %[b] offset:3072" NTS "\n\t"                            \
    "s_mov_b32 m0, %[l2]\n\t"                                                               \
    "global_load_lds_dwordx4 %[v2], %[b]" NTS "\n\t"                                        \
    "s_mov_b32 m0, %[sv]"
#define KVQ_DMA_128(NTS)                                                                     \
    "s_waitcnt lgkmcnt(0)\n\t"                                                              \
    "s_mov_b32 %[sv], m0\n\t"                                                               \
    "s_mov_b32 m0, %[l0]\n\t"                                                               \
    "global_load_lds_dwordx4 %[v0], %[b]" NTS "\n\t"                                        \
    "global_load_lds_dwordx4 %[v0], %[b] offset:1024" NTS "\n\t"                            \
    "global_load_lds_dwordx4 %[v0], %[b] offset:2048" NTS "\n\t"                            \
    "global_load_lds_dwordx4 %[v0], %[b] offset:3072" NTS "\n\t"                            \
    "s_mov_b32 m0, %[l1]\n\t"                                                               \
    "global_load_lds_dwordx4 %[v1], %[b]" NTS "\n\t"                                        \
    "s_mov_b32 m0, %[sv]"
template <int D, bool NT = true>
__device__ __forceinline__ void dma_block(const uint8_t* base, uint32_t v0, uint32_t lds) {
    const uint32_t v1 = v0 + 4096, l1 = lds + 4096;
    uint32_t saved;
    if constexpr (D == 256) {
        const uint32_t v2 = v0 + 8192, l2 = lds + 8192;
        if constexpr (NT)
            asm volatile(KVQ_DMA_256(" nt")
                         : [sv] "=&s"(saved)
                         : [b] "s"(base), [v0] "v"(v0), [v1] "v"(v1), [v2] "v"(v2), [l0] "s"(lds), [l1] "s"(l1),
                           [l2] "s"(l2)
                         : "memory");
        else
            asm volatile(KVQ_DMA_256("")
                         : [sv] "=&s"(saved)
                         : [b] "s"(base), [v0] "v"(v0), [v1] "v"(v1), [v2] "v"(v2), [l0] "s"(lds), [l1] "s"(l1),
                           [l2] "s"(l2)
                         : "memory");
    } else {
        if constexpr (NT)
            asm volatile(KVQ_DMA_128(" nt")
                         : [sv] "=&s"(saved)
                         : [b] "s"(base), [v0] "v"(v0), [v1] "v"(v1), [l0] "s"(lds), [l1] "s"(l1)
                         : "memory");
        else
            asm volatile(KVQ_DMA_128("")
                         : [sv] "=&s"(saved)
                         : [b] "s"(base), [v0] "v"(v0), [v1] "v"(v1), [l0] "s"(lds), [l1] "s"(l1)
                         : "memory");
    }
}
#undef KVQ_DMA_256
#undef KVQ_DMA_128
static_assert(q2_block_bytes(256) == 9 * 1024 && q2_block_bytes(128) == 5 * 1024, "blocks are whole KiB");

// Waits until at most N of this wave's vector memory operations are
// outstanding.  Loads complete in issue order, so with the next tile's DMA
// (N loads) issued after this tile's, vmcnt(N) means this tile has landed.
template <int N>
__device__ __forceinline__ void wait_vm() {
    if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Loads and stores at an LDS byte address (plain scalar and vector types:
// HIP's vector structs do not bind to LDS-qualified references).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ T lds_load(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T*>((uintptr_t)addr);
}
template <typename T>
__device__ __forceinline__ void lds_store(uint32_t addr, T v) {
    *reinterpret_cast<__attribute__((address_space(3))) T*>((uintptr_t)addr) = v;
}
__device__ __forceinline__ uint4 lds_load4(uint32_t addr) {
    const u32x4 w = lds_load<u32x4>(addr);
    return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ float2 lds_loadf2(uint32_t addr) {
    const u32x2 w = lds_load<u32x2>(addr);
    return make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
}

// The registers a tile is computed from: lane (j, grp) holds the K code words
// of token 16m + j for this lane group's D/16 bytes (q.k operands), the V
// words of dims 32c + j and 32c + 16 + j for its k-range (p.v operands), and
// the (scale, min) rows of token 16m + j.
template <int D>
struct TileRegs {
    uint32_t kc[8][D / 64];
    uint4 vc[D / 32];
    float2 km[8];
    float2 vm[8];
};

template <int D>
__device__ __forceinline__ void read_tile(TileRegs<D>& t, uint32_t slot, int l) {
    constexpr int NW = D / 64, B = TileShape<D>::BLK;
    const int j = l & 15, grp = l >> 4;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const uint32_t src = slot + (m < 4 ? 0 : B) + (16 * (m & 3) + j) * (D / 4) + 4 * NW * grp;
        if constexpr (NW == 4) {
            const uint4 w = lds_load4(src);
            t.kc[m][0] = w.x; t.kc[m][1] = w.y; t.kc[m][2] = w.z; t.kc[m][3] = w.w;
        } else {
            const u32x2 w = lds_load<u32x2>(src);
            t.kc[m][0] = w.x; t.kc[m][1] = w.y;
        }
    }
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        t.vc[c] = lds_load4(slot + (grp < 2 ? 0 : B) + q2_vcodes_off(D) + q2_vword_off(D, 32 * c + j, 2 * (grp & 1)));
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const uint32_t mb = slot + (m < 4 ? 0 : B) + 8 * (16 * (m & 3) + j);
        t.km[m] = lds_loadf2(mb + q2_kmeta_off(D));
        t.vm[m] = lds_loadf2(mb + q2_vmeta_off(D));
    }
}

template <int D>
struct WaveState {
    v4f acc[D / 16];  // p.v sums: block b, column 4h + i of lane l%16, dims 16b + 4(l/16) + r
    float m_ref;      // reference max of head l/16, raw q.k^ units
    float cbm;        // cB * m_ref (log2 units)
    float l_run;      // this lane's share of sum p (head l/16)
    float c_run;      // this lane's share of sum p * min_v (head l/16)
};

struct QConst {
    int scale_a;  // q.k row scale of this lane's row (4h + i): 32^(3-i) 2^-E_h * 2 (codes are c/2)
    float qsum;   // sum_d q_d of head l/16
    float cB;     // log2(e) * sm: raw q.k^ -> log2 units
};

// The weight-digit transpose of a wave: for head h and digit i, 32 words at
// wdig_base(h, i); word c (c < 16) holds the digits of tokens 16m + c for
// m = 0..3, word 16 + c those for m = 4..7.  With four waves a workgroup the
// rows of the four heads are staggered by 16 words (fewer bank conflicts);
// eight waves take the unpadded 2,048 bytes so that the workgroup fits LDS.
template <bool PAD>
__device__ __forceinline__ int wdig_base(int h, int i) { return (4 * h + i) * 32 + (PAD ? 16 * h : 0); }
template <bool PAD>
constexpr int WDIG_BYTES = 4 * (4 * 4 * 32 + (PAD ? 16 * 3 : 0));

template <int D, bool FULL, bool SCORES, bool PAD>
__device__ __forceinline__ void compute_tile(const TileRegs<D>& t, uint32_t wdig, int l, const v8i* qop,
                                             const QConst& qc, WaveState<D>& st, int tok0, int ctx,
                                             float* __restrict__ srow) {
    constexpr int NC = D / 128, NB = D / 16;
    const int j = l & 15, grp = l >> 4;
    // ---- q.k: raw scores q.k^ of tokens 16m + j, head grp ----
    float s[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        v4f cq = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) cq = mma_qk(qop[c], fp4_operand(t.kc[m][2 * c], t.kc[m][2 * c + 1]), cq, qc.scale_a);
        float x = fmaf(t.km[m].x, (cq[0] + cq[1]) + (cq[2] + cq[3]), t.km[m].y * qc.qsum);
        if (!FULL && tok0 + 16 * m + j >= ctx) x = -INFINITY;
        s[m] = x;
        tmax = fmaxf(tmax, x);
    }
    tmax = row_max16(tmax);
    const bool need = (tmax - st.m_ref) * qc.cB > RESCALE_LOG2;
    if (__ballot(need)) {
        const float m_new = need ? tmax : st.m_ref;
        const float cbm_new = qc.cB * m_new;
        const float alpha = __builtin_amdgcn_exp2f(st.cbm - cbm_new);
        st.l_run *= alpha;
        st.c_run *= alpha;
        // accumulator columns of lane l belong to head (l%16)/4
        const float a = __shfl(alpha, 16 * (j >> 2));
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) st.acc[b][r] *= a;
        st.m_ref = m_new;
        st.cbm = cbm_new;
    }
    // ---- weights w = p * scale_v ----
    float w[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[m], qc.cB, -st.cbm));
        float x;
        if (FULL) {
            x = p * t.vm[m].x;
            st.c_run = fmaf(p, t.vm[m].y, st.c_run);
        } else {
            const bool valid = tok0 + 16 * m + j < ctx;
            x = valid ? p * t.vm[m].x : 0.f;
            st.c_run += valid ? p * t.vm[m].y : 0.f;
        }
        st.l_run += p;
        w[m] = x;
    }
    if (SCORES && srow) {  // lanes of a head past the group's end hold no score row
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int tok = tok0 + 16 * m + j;
            if (FULL || tok < ctx) srow[tok] = s[m] * (qc.cB * LN2);
        }
    }
    // ---- weight digits: X = round(w 2^F) < 2^16, four 4-bit digits per weight ----
    // The p.v column scale of lane l covers k-block l/16 (32 tokens): tokens
    // 16m + c with c in [8 (b % 2), 8 (b % 2) + 8) and m in [4 (b / 2), 4 (b / 2) + 4),
    // so each lane takes the max of its first and last four weights over its
    // half row, and F is set per head and 32-token block.
    const float wlo = half_row_max8(fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3])));
    const float whi = half_row_max8(fmaxf(fmaxf(w[4], w[5]), fmaxf(w[6], w[7])));
    const int FWlo = weight_exp(wlo), FWhi = weight_exp(whi);
    const float wscale_lo = pow2f(FWlo), wscale_hi = pow2f(FWhi);
    uint32_t X[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)  // 2^23 + X in the bits of the fused multiply-add, X capped at 2^16 - 1
        X[m] = min(__float_as_uint(fmaf(w[m], m < 4 ? wscale_lo : wscale_hi, 8388608.0f)), 0x4B00FFFFu);
    uint32_t P[4];  // X of tokens m = 2k (bytes 0-1) and 2k + 1 (bytes 2-3)
#pragma unroll
    for (int k = 0; k < 4; ++k) P[k] = __builtin_amdgcn_perm(X[2 * k + 1], X[2 * k], 0x05040100u);
    uint32_t L[4], H[4];  // nibbles 0 and 2 (L), 1 and 3 (H) of each X, one per byte
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        L[k] = P[k] & 0x0F0F0F0Fu;
        H[k] = (P[k] >> 4) & 0x0F0F0F0Fu;
    }
    // digit i of tokens m = 0..3 and m = 4..7, one byte per token
    const uint32_t d0a = __builtin_amdgcn_perm(L[1], L[0], 0x06040200u), d0b = __builtin_amdgcn_perm(L[3], L[2], 0x06040200u);
    const uint32_t d2a = __builtin_amdgcn_perm(L[1], L[0], 0x07050301u), d2b = __builtin_amdgcn_perm(L[3], L[2], 0x07050301u);
    const uint32_t d1a = __builtin_amdgcn_perm(H[1], H[0], 0x06040200u), d1b = __builtin_amdgcn_perm(H[3], H[2], 0x06040200u);
    const uint32_t d3a = __builtin_amdgcn_perm(H[1], H[0], 0x07050301u), d3b = __builtin_amdgcn_perm(H[3], H[2], 0x07050301u);
    {
        auto put = [&](int i, int half, uint32_t v) { lds_store<uint32_t>(wdig + 4 * (wdig_base<PAD>(grp, i) + 16 * half + j), v); };
        put(0, 0, d0a); put(0, 1, d0b);
        put(1, 0, d1a); put(1, 1, d1b);
        put(2, 0, d2a); put(2, 1, d2b);
        put(3, 0, d3a); put(3, 1, d3b);
    }
    // p.v operand of column j = 4h + i: k = 16 grp + s <- word 4 grp + s/4 byte s%4,
    // k = 64 + 16 grp + s <- word 16 + 4 grp + s/4 byte s%4
    v8i wop;
    {
        const uint32_t base = wdig + 4 * (wdig_base<PAD>(j >> 2, j & 3) + 4 * grp);
        const uint4 lo = lds_load4(base);
        const uint4 hi = lds_load4(base + 64);
        wop[0] = (int)lo.x; wop[1] = (int)lo.y; wop[2] = (int)lo.z; wop[3] = (int)lo.w;
        wop[4] = (int)hi.x; wop[5] = (int)hi.y; wop[6] = (int)hi.z; wop[7] = (int)hi.w;
    }
    // column scale of (column j = 4h + i, k-block grp): byte b of digit i is
    // worth b 2^-9 and the code nibble is c / 2, so 2^(4i - F + 10)
    const int fw_pair = __shfl((FWlo + 128) | ((FWhi + 128) << 16), 16 * (j >> 2) + 8 * (grp & 1));
    const int scale_b = 137 + 4 * (j & 3) - (((fw_pair >> (16 * (grp >> 1))) & 0xFFFF) - 128);
    // ---- p.v ----
#pragma unroll
    for (int c = 0; c < NB / 2; ++c) {
        st.acc[2 * c] = mma_pv(fp4_operand(t.vc[c].x, t.vc[c].y), wop, st.acc[2 * c], scale_b);
        st.acc[2 * c + 1] = mma_pv(fp4_operand(t.vc[c].z, t.vc[c].w), wop, st.acc[2 * c + 1], scale_b);
    }
}

// LDS of a split workgroup of W waves: SLOTS tile slots per wave, then one
// area per wave for its query rows (before the first tile) and its
// weight-digit transpose (after); at the end, the waves' partial results
// reuse the tile slots.
template <int D, int W, int SLOTS>
struct SplitLds {
    static constexpr bool PAD = W == 4;
    static constexpr int AREA = WDIG_BYTES<PAD>;
    static constexpr int SLOTS_BYTES = W * SLOTS * TileShape<D>::BYTES;
    static constexpr int BYTES = SLOTS_BYTES + W * AREA;
    static_assert(4 * D * 2 <= AREA, "the query rows of four heads fit a wave's area");
    static_assert(64 * 8 * 4 <= AREA, "a pass of the rotated rows (eight fp32 a lane) fits a wave's area");
    static_assert(BYTES <= 160 * 1024, "a workgroup's LDS fits the compute unit");
    static_assert((W * 4 * D + W * 4 * 3) * 4 + 4 <= SLOTS_BYTES, "the waves' partials fit the tile slots");
};

template <int D, bool SCORES, bool ROT, bool GENERAL, bool FUSE, int W, int SLOTS, bool PAIRED = false>
__device__ __forceinline__ void decode_q2_mfma_body(const PoolView& pv, int layer, const BatchDesc& bd,
                                                    const uint16_t* __restrict__ q, float sm, int splits,
                                                    float* __restrict__ ws, float* __restrict__ out,
                                                    float* __restrict__ scores, int64_t sstride, int h0, int nh) {
    // The kernel takes four query heads of a KV head's group at a time: heads
    // h0 .. h0 + nh - 1.  Without GENERAL the group is exactly these four
    // (group 4, h0 = 0, nh = 4, all known when compiling); with it the group
    // size is the pool's, and when nh < 4 the rows of the missing heads are
    // zero queries whose results are dropped.
    constexpr int G = 4;
    constexpr int NC = D / 128;  // k-chunks of the q.k product
    constexpr int NB = D / 16;   // 16-dim blocks of the p.v product
    using LdsT = SplitLds<D, W, SLOTS>;
    constexpr bool PAD = LdsT::PAD;
    constexpr int TB = TileShape<D>::BYTES;
    const int Hkv = pv.Hkv, Hq = pv.Hq;
    // PAIRED (group 8 in one launch): a one-dimensional grid of
    // two workgroups per (sequence, KV head, split), the half h taking heads
    // 4h ..  Each run of 16 workgroups holds both halves of 8 such triples, the
    // second half 8 places after the first: workgroups go round the XCDs in
    // dispatch order, so the two land on the same XCD at nearly the same time and
    // the second reads the blocks mostly from that XCD's L2 (the DMA is then not
    // nontemporal).  A last run of fewer than 16 keeps the halves r apart.
    unsigned bx = blockIdx.x, by = blockIdx.y;
    int half = 0;
    if constexpr (PAIRED) {
        const int M = bd.n * Hkv * splits;  // triples; the grid is 2 M
        const int L = blockIdx.x, base = L & ~15, off = L & 15;
        const int r = min(8, M - (base >> 1));
        half = off >= r;
        const int t = (base >> 1) + off - half * r;
        bx = (unsigned)(t % (bd.n * Hkv));
        by = (unsigned)(t / (bd.n * Hkv));
    }
    const int e = bx / Hkv, g = bx % Hkv, sp = (int)by;
    const int Gq = GENERAL ? Hq / Hkv : G;  // the pool's GQA group
    if constexpr (!GENERAL) {
        h0 = 0;
        nh = G;
    }
    if constexpr (PAIRED) {
        h0 = 4 * half;
        nh = min(4, Gq - h0);
    }
    const int64_t head0 = (int64_t)e * Hq + (int64_t)g * Gq + h0;  // first query row of this launch
    const int ctx = bd.pos[e];
    int pg0, pg1;
    split_range(ctx, bd.per, sp, &pg0, &pg1);
    if (pg0 >= pg1) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int j = l & 15, grp = l >> 4;
    const int hq = j >> 2, iq = j & 3;  // this lane's q.k row: digit iq of head hq

    __shared__ __align__(16) uint8_t smem[LdsT::BYTES];
    const uint32_t slot0 = lds_addr(smem) + wave * SLOTS * TB;
    const uint32_t area = lds_addr(smem) + LdsT::SLOTS_BYTES + wave * LdsT::AREA;
    auto slot_of = [&](int t) { return slot0 + (SLOTS == 2 ? (t & 1) * TB : 0); };

    const int64_t lhoff = ((int64_t)layer * Hkv + g) * pv.block_bytes;
    const int n_pages = (ctx + PAGE - 1) / PAGE;
    float* srow = scores && (!GENERAL || grp < nh) ? scores + (head0 + grp) * sstride : nullptr;
    // the block table through the constant address space: page ids are
    // uniform across a wave, so they come in by scalar loads, which do not
    // queue behind the tiles' DMA loads
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(pv.bt + (int64_t)bd.seq[e] * pv.bt_stride);

    // ---- this wave's tiles: page pairs pg0/2 + wave + W i, i < T ----
    const int pr_first = pg0 / 2 + wave;
    const int pr_end = (pg1 + 1) / 2;
    const int T = pr_first < pr_end ? (pr_end - pr_first + W - 1) / W : 0;
    // the last tile of the sequence may be partly past ctx (and its second
    // page past the last page: it then re-reads the first)
    const bool last_partial = T > 0 && 2 * (pr_first + W * (T - 1)) * PAGE + 2 * PAGE > ctx;
    const int TF = last_partial ? T - 1 : T;  // full tiles
    auto tok0_of = [&](int t) { return 2 * (pr_first + W * t) * PAGE; };
    const uint32_t voff = 16 * l;
    auto issue = [&](int t) {  // tile t's DMA into slot t % SLOTS
        const int pair = pr_first + W * t;
        const int id0 = bt[2 * pair], id1 = bt[min(2 * pair + 1, n_pages - 1)];
        const uint32_t slot = slot_of(t);
        dma_block<D, !PAIRED>(pv.pages + (int64_t)id0 * pv.page_bytes + lhoff, voff, slot);
        dma_block<D, !PAIRED>(pv.pages + (int64_t)id1 * pv.page_bytes + lhoff, voff, slot + TileShape<D>::BLK);
    };

    // The query rows of the group's G heads (contiguous, G D bf16) go to the
    // wave's area of LDS before any tile is in flight (the compiler's wait
    // for them must not be taken after a DMA load).  The rotated variant
    // instead widens each lane's pieces to fp32 in registers, issues the first
    // DMA, and then transforms them there: butterfly stages h = 1, 2, 4 inside
    // a lane's eight dims, h = 8m across the lanes l ^ m of one head's row,
    // with the additions of the append's transform in the same order.  The
    // rotated rows then pass through the wave's area (2 KB) a half at a time.
    constexpr int QPIECES = G * D * 2 / 16 / 64;  // 16-byte pieces per lane
    // piece i of lane l: bf16 8p .. 8p + 7 of the four rows, p = l + 64 i, i.e.
    // dims 8 (l % (D/8)) .. of head 8p / D
    float qr[ROT ? QPIECES : 1][8];
    {
        uint4 qraw[QPIECES];
        const uint4* qsrc = reinterpret_cast<const uint4*>(q + head0 * D);
#pragma unroll
        for (int i = 0; i < QPIECES; ++i) {
            const int p = l + 64 * i;
            qraw[i] = !GENERAL || 8 * p < nh * D ? qsrc[p] : make_uint4(0u, 0u, 0u, 0u);
        }
        if constexpr (ROT) {
#pragma unroll
            for (int i = 0; i < QPIECES; ++i) {
                const uint32_t u[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    qr[i][2 * k] = bf16lo(u[k]);
                    qr[i][2 * k + 1] = bf16hi(u[k]);
                }
            }
            // the values are taken (and the loads waited for) before the DMA below
#pragma unroll
            for (int i = 0; i < QPIECES; ++i)
#pragma unroll
                for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(qr[i][k]));
        } else {
#pragma unroll
            for (int i = 0; i < QPIECES; ++i)
                lds_store<u32x4>(area + 16 * (l + 64 * i), u32x4{qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w});
        }
    }
    if (T > 0) issue(0);
    if constexpr (ROT) {
        // stages h = 1 .. D/2 as on append, additions only: nothing to contract
#pragma unroll
        for (int h = 1; h < 8; h *= 2)
#pragma unroll
            for (int i = 0; i < QPIECES; ++i)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if ((k & h) == 0) {
                        const float a = qr[i][k], b = qr[i][k + h];
                        qr[i][k] = a + b;
                        qr[i][k + h] = a - b;
                    }
#pragma unroll
        for (int m = 1; m < D / 8; m *= 2) {  // h = 8m: the partner is lane l ^ m
            const bool upper = (l & m) != 0;   // this lane holds the element i + h of its pairs
#pragma unroll
            for (int i = 0; i < QPIECES; ++i)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float o = __shfl_xor(qr[i][k], m);
                    qr[i][k] = upper ? o - qr[i][k] : qr[i][k] + o;
                }
        }
    }

    // ---- query operand: 19-bit fixed point per head, row 4 hq + iq = digit iq of head hq ----
    float qv[NC][32];
    float amax = 0.f, qsum = 0.f;
    // byte s of chunk c: k of byte s; the K operand puts dim(k) at nibble k % 32 of lane group k / 32
    auto dim_of = [&](int c, int s) {
        const int k = fp8_k(grp, s), ga = k >> 5, n = k & 31;
        return 32 * NC * ga + 32 * c + 16 * (n >> 4) + 2 * (n & 7) + ((n >> 3) & 1);
    };
    if constexpr (!ROT) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int s = 0; s < 32; ++s) {
                const float x = bf16_to_f32(lds_load<uint16_t>(area + 2 * (hq * D + dim_of(c, s))));
                qv[c][s] = x;
                amax = fmaxf(amax, fabsf(x));
                qsum += x;
            }
    } else {
        // piece `pass` of every lane holds heads HPP pass .. HPP pass + HPP - 1, at float 8 l of the area
        constexpr int NPASS = QPIECES, HPP = G / NPASS;
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            lds_store<u32x4>(area + 32 * l, u32x4{__float_as_uint(qr[pass][0]), __float_as_uint(qr[pass][1]),
                                                  __float_as_uint(qr[pass][2]), __float_as_uint(qr[pass][3])});
            lds_store<u32x4>(area + 32 * l + 16, u32x4{__float_as_uint(qr[pass][4]), __float_as_uint(qr[pass][5]),
                                                       __float_as_uint(qr[pass][6]), __float_as_uint(qr[pass][7])});
            const bool mine = hq / HPP == pass;
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int s = 0; s < 32; ++s) {
                    const float x = lds_load<float>(area + 4 * ((hq % HPP) * D + dim_of(c, s)));
                    if (mine) qv[c][s] = x;
                }
        }
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int s = 0; s < 32; ++s) {
                amax = fmaxf(amax, fabsf(qv[c][s]));
                qsum += qv[c][s];
            }
    }
    if (SLOTS == 2 && T > 1) issue(1);
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    qsum += __shfl_xor(qsum, 16);
    qsum += __shfl_xor(qsum, 32);
    const int EQ = 18 - (amax > 0.f ? exponent_of(amax) : 0);  // |q * 2^EQ| < 2^19
    const float qscale = pow2f(EQ);
    QConst qc;
    qc.scale_a = 127 + 5 * (3 - iq) - EQ + 1;
    qc.qsum = __shfl(qsum, 4 * grp);  // q.k result lanes hold head l/16
    qc.cB = LOG2E * sm;
    v8i qop[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int v = 0; v < 8; ++v)
            qop[c][v] = (int)pack4_fp8(digit_of(qv[c][4 * v], qscale, iq), digit_of(qv[c][4 * v + 1], qscale, iq),
                                       digit_of(qv[c][4 * v + 2], qscale, iq), digit_of(qv[c][4 * v + 3], qscale, iq));

    WaveState<D> st;
#pragma unroll
    for (int b = 0; b < NB; ++b) st.acc[b] = v4f{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.cbm = -INFINITY;
    st.l_run = 0.f;
    st.c_run = 0.f;

    // ---- the tiles: DMA of tile t + SLOTS in flight while tile t is computed ----
    // (score stores may complete out of order with loads: with scores every
    // wait is for all outstanding operations)
    constexpr int DMA = TileShape<D>::DMA;
    auto wait_tile = [&](int t) {
        if (!SCORES && SLOTS == 2 && t + 1 < T) wait_vm<DMA>();
        else wait_vm<0>();
    };
    for (int t = 0; t < TF; ++t) {
        wait_tile(t);
        TileRegs<D> tr;
        read_tile<D>(tr, slot_of(t), l);
        if (t + SLOTS < T) issue(t + SLOTS);
        compute_tile<D, true, SCORES, PAD>(tr, area, l, qop, qc, st, tok0_of(t), ctx, srow);
    }
    if (last_partial) {
        wait_tile(T - 1);
        TileRegs<D> tr;
        read_tile<D>(tr, slot_of(T - 1), l);
        compute_tile<D, false, SCORES, PAD>(tr, area, l, qop, qc, st, tok0_of(T - 1), ctx, srow);
    }

    // ---- this wave's partial: sum the digit columns, and each head's lanes ----
    const float l_run = row_sum16(st.l_run), c_run = row_sum16(st.c_run);  // head grp
    float4 o4[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        o4[b].x = quad_sum(st.acc[b][0]);
        o4[b].y = quad_sum(st.acc[b][1]);
        o4[b].z = quad_sum(st.acc[b][2]);
        o4[b].w = quad_sum(st.acc[b][3]);
    }
    __syncthreads();  // every wave is done with its tile slots, which the partials reuse
    float(*o_s)[G][D] = reinterpret_cast<float(*)[G][D]>(smem);
    float(*ml_s)[G][3] = reinterpret_cast<float(*)[G][3]>(smem + W * G * D * 4);
    if (j == 0) {
        ml_s[wave][grp][0] = st.cbm;  // log2 units
        ml_s[wave][grp][1] = l_run;
        ml_s[wave][grp][2] = c_run;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
        if (iq == 0) *reinterpret_cast<float4*>(&o_s[wave][hq][16 * b + 4 * grp]) = o4[b];
    __syncthreads();

    // ---- combine the W waves, write this split's partial ----
    DecodeWs w(ws, bd.n, Hq, D, splits);
    if (threadIdx.x < 64 * G) {
        const int h = threadIdx.x >> 6;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < W; ++v) M = fmaxf(M, ml_s[v][h][0]);
        float f[W], lsum = 0.f;
#pragma unroll
        for (int v = 0; v < W; ++v) {
            f[v] = __builtin_amdgcn_exp2f(ml_s[v][h][0] - M);
            lsum += f[v] * ml_s[v][h][1];
        }
        const int64_t row = (head0 + h) * splits + sp;
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
            const int d = l + 64 * k;
            float o = 0.f;
#pragma unroll
            for (int v = 0; v < W; ++v) o += f[v] * (o_s[v][h][d] + ml_s[v][h][2]);
            if (!GENERAL || h < nh) {
                if constexpr (FUSE) store_agent(&w.o[row * D + d], o);
                else w.o[row * D + d] = o;
            }
        }
        if (l == 0 && (!GENERAL || h < nh)) {
            if constexpr (FUSE) {
                store_agent(&w.ml[2 * row], M);
                store_agent(&w.ml[2 * row + 1], lsum);
            } else {
                w.ml[2 * row] = M;
                w.ml[2 * row + 1] = lsum;
            }
        }
    }
    if constexpr (FUSE) {
        // The last of the sequence's live splits to get here merges them all.
        // Partials travel through agent-scope (L2-coherent) stores and loads
        // only, so no cache writeback or invalidation is needed: every
        // thread's partial stores have completed before the workgroup counts
        // itself, and the merging workgroup loads them after the count shows
        // every split done.
        int* last_s = reinterpret_cast<int*>(smem + W * G * (D + 3) * 4);  // past the partials
        wait_stores();
        __syncthreads();
        const int live = live_splits(ctx, bd.per);
        int32_t* cnt = pv.cnt + ((int64_t)e * Hkv + g) * 2 + (h0 >> 2);
        if (threadIdx.x == 0) {
            const int before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int is_last = before == live - 1;
            if (is_last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
            *last_s = is_last;
        }
        __syncthreads();
        if (!*last_s || threadIdx.x >= 64 * G) return;
        const int h = threadIdx.x >> 6;
        if (GENERAL && h >= nh) return;
        merge_live_splits<D / 64>(w, (head0 + h) * splits, live, l, out + (head0 + h) * D);
    }
}

// Workgroup shape of the split kernel: eight waves (two per SIMD, 244
// registers a wave) with one tile slot each fill the compute unit's 160 KiB
// of LDS; while a wave computes one tile the DMA of its next is in flight,
// and the SIMD's other wave covers the first's stalls.  (Four waves with two
// slots each, one wave per SIMD, measured 41.3 against 38.9 us a 27B-geometry
// decode call: 296 registers a wave, moved through the accumulation
// registers.)
constexpr int SPLIT_WAVES = 8, SPLIT_SLOTS = 1;

// Group 4: the four heads of each KV head's group in one launch.  FUSE: the
// last split of each (sequence, KV head) to finish merges the partials into
// out (at most FUSED_MERGE_MAX_SPLITS splits).
template <int D, bool SCORES, bool ROT, bool FUSE, int W, int SLOTS>
__global__ __launch_bounds__(64 * W) void decode_q2_mfma_kernel(PoolView pv, int layer, BatchDesc bd,
                                                                const uint16_t* __restrict__ q, float sm, int splits,
                                                                float* __restrict__ ws, float* __restrict__ out,
                                                                float* __restrict__ scores, int64_t sstride) {
    decode_q2_mfma_body<D, SCORES, ROT, false, FUSE, W, SLOTS>(pv, layer, bd, q, sm, splits, ws, out, scores, sstride,
                                                               0, 4);
}

// Group 8: both halves of each KV head's group in one launch.
template <int D, bool SCORES, bool ROT, bool FUSE, int W, int SLOTS>
__global__ __launch_bounds__(64 * W) void decode_q2_mfma_pair_kernel(PoolView pv, int layer, BatchDesc bd,
                                                                     const uint16_t* __restrict__ q, float sm,
                                                                     int splits, float* __restrict__ ws,
                                                                     float* __restrict__ out,
                                                                     float* __restrict__ scores, int64_t sstride) {
    decode_q2_mfma_body<D, SCORES, ROT, true, FUSE, W, SLOTS, true>(pv, layer, bd, q, sm, splits, ws, out, scores,
                                                                    sstride, 0, 0);
}

// Other groups: heads h0 .. h0 + nh - 1 of each KV head's group.
template <int D, bool SCORES, bool ROT, bool FUSE, int W, int SLOTS>
__global__ __launch_bounds__(64 * W) void decode_q2_mfma_group_kernel(PoolView pv, int layer, BatchDesc bd,
                                                                      const uint16_t* __restrict__ q, float sm,
                                                                      int splits, float* __restrict__ ws,
                                                                      float* __restrict__ out,
                                                                      float* __restrict__ scores, int64_t sstride,
                                                                      int h0, int nh) {
    decode_q2_mfma_body<D, SCORES, ROT, true, FUSE, W, SLOTS>(pv, layer, bd, q, sm, splits, ws, out, scores, sstride,
                                                              h0, nh);
}

// The split kernels of a decode call; fuse: each launch also merges (out).
static hipError_t launch_decode_q2_splits(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q,
                                          float sm, int splits, float* ws, float* out, float* scores,
                                          int64_t sstride, hipStream_t s, bool rot, bool fuse) {
    dim3 grid(bd.n * pv.Hkv, splits);
    const float smk = rot ? sm / (float)pv.D : sm;  // H q . H k = D q . k
    const int Gq = pv.Hq / pv.Hkv;
    using D128 = std::integral_constant<int, 128>;
    using D256 = std::integral_constant<int, 256>;
    using T = std::true_type;
    using F = std::false_type;
    // template flags: head dim, scores, rotated, fused merge
    auto flags = [&](auto&& go) {
        auto f3 = [&](auto d, auto sc, auto r) { fuse ? go(d, sc, r, T{}) : go(d, sc, r, F{}); };
        auto f2 = [&](auto d, auto sc) { rot ? f3(d, sc, T{}) : f3(d, sc, F{}); };
        auto f1 = [&](auto d) { scores ? f2(d, T{}) : f2(d, F{}); };
        pv.D == 256 ? f1(D256{}) : f1(D128{});
    };
    if (Gq == 4) {
        flags([&](auto d, auto sc, auto r, auto fu) {
            hipLaunchKernelGGL((decode_q2_mfma_kernel<decltype(d)::value, decltype(sc)::value, decltype(r)::value,
                                                      decltype(fu)::value, SPLIT_WAVES, SPLIT_SLOTS>),
                               grid, dim3(64 * SPLIT_WAVES), 0, s, pv, layer, bd, q, smk, splits, ws, out, scores,
                               sstride);
        });
        return hipGetLastError();
    }
    if (Gq == 8) {  // both halves of the group in one launch
        const dim3 grid2(2 * bd.n * pv.Hkv * splits);
        flags([&](auto d, auto sc, auto r, auto fu) {
            hipLaunchKernelGGL((decode_q2_mfma_pair_kernel<decltype(d)::value, decltype(sc)::value, decltype(r)::value,
                                                           decltype(fu)::value, SPLIT_WAVES, SPLIT_SLOTS>),
                               grid2, dim3(64 * SPLIT_WAVES), 0, s, pv, layer, bd, q, smk, splits, ws, out, scores,
                               sstride);
        });
        return hipGetLastError();
    }
    // other groups: up to four query heads per launch
    for (int h0 = 0; h0 < Gq; h0 += 4) {
        const int nh = Gq - h0 < 4 ? Gq - h0 : 4;
        flags([&](auto d, auto sc, auto r, auto fu) {
            hipLaunchKernelGGL((decode_q2_mfma_group_kernel<decltype(d)::value, decltype(sc)::value,
                                                            decltype(r)::value, decltype(fu)::value, SPLIT_WAVES,
                                                            SPLIT_SLOTS>),
                               grid, dim3(64 * SPLIT_WAVES), 0, s, pv, layer, bd, q, smk, splits, ws, out, scores,
                               sstride, h0, nh);
        });
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_decode_q2_partials(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm,
                                     int splits, float* ws, float* scores, int64_t sstride, hipStream_t s, bool rot) {
    return launch_decode_q2_splits(pv, layer, bd, q, sm, splits, ws, nullptr, scores, sstride, s, rot, false);
}

hipError_t launch_decode_q2(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q, float sm, int splits,
                            float* ws, float* out, float* scores, int64_t sstride, hipStream_t s, bool rot) {
    if (splits <= FUSED_MERGE_MAX_SPLITS && pv.cnt)
        return launch_decode_q2_splits(pv, layer, bd, q, sm, splits, ws, out, scores, sstride, s, rot, true);
    const hipError_t err = launch_decode_q2_partials(pv, layer, bd, q, sm, splits, ws, scores, sstride, s, rot);
    return err != hipSuccess ? err : launch_merge_splits(bd, pv.Hq, pv.D, splits, ws, out, s);
}

}  // namespace kvq
