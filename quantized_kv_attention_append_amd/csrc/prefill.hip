// Chunked causal prefill over the 2-bit pool (and, through the same kernel,
// the bf16 pool): the chunk's queries attend to the prior tokens and to the
// chunk itself, every key and value read from the compressed pages ("KV at 9
// KB a token", opening section: prefill attention reads the compressed cache
// directly, and every workspace byte a launch reads it wrote first).
//
// Query i of the chunk sits at position q_start + i and sees keys
// 0 .. q_start + i (inclusive).  Scores are sm q.k^ with the dequantization
// folded algebraically (q.k^_t = min_t sum(q) + scale_t q.c_t); the online
// softmax and every sum are fp32 (the two-level accumulation of "Half the
// Cache, Twice the Context", section "The cliff is in the accumulator").
//
// Both contractions run on v_mfma_f32_16x16x32_bf16:
//   * codes 0..3 and the bf16 query are exact bf16 operands, so q.c is exact
//     up to the fp32 sum;
//   * the softmax weights w = p scale_v are split into two bf16 terms
//     (w rounded to bf16, then the rounded residual), 17 significant bits.
// The score tile is computed transposed, S^T = K~ Q^T (rows = keys, columns =
// 16 (query, head) rows), so that the lane holding keys 4g..4g+3 and
// 16+4g..16+4g+3 of a 32-key step already holds the p.v operand
// O^T = V~ P^T for the k-slots 8g..8g+7: no transpose of P is needed.
//
// One workgroup of four waves per (KV head, block of 128 / G queries, split of
// the keys).  Each wave owns two 16-column blocks of (query, head) rows (128
// rows per workgroup); every page of 64 keys is converted once per workgroup
// from the packed codes into bf16 LDS tiles (double-buffered, the next page
// converted while the current one is multiplied):
//   K~[key][kappa]  kappa = order of dims in which dim pairs (16u + k,
//                   16u + k + 8) are adjacent (one 2-bit word -> eight bf16
//                   pairs with a byte-permute lookup);
//   V~[dim][key]    natural key order.
// Partials (m, l, o) of every row go to the workspace; prefill_merge_kernel
// merges, for each row, the splits whose first key it can see.
//
// A bf16 pool fills the same tiles with the stored values (K dims interleaved
// into kappa order by byte permutes, V copied) and unit metadata (scale 1,
// offset 0), so that the rest of the kernel is the same code.
#include <climits>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "prefill.h"

namespace kvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

namespace {

// A wave owns NCB 16-column blocks of (query, head) rows, a workgroup four
// waves: 4 NCB 16 rows.  Two blocks a wave in general; one when the query
// enters as two bf16 terms (the rotated format), which doubles the q.k
// products and their query registers.
template <bool ROTQ>
constexpr int PREFILL_NCB = ROTQ ? 1 : 2;
template <bool ROTQ>
constexpr int PREFILL_ROWS = 4 * PREFILL_NCB<ROTQ> * 16;
constexpr int KROW = 8;           // padding of a K~ row, bf16 elements (16 B: the 16 rows a read group
                                  // touches start in distinct 16-byte bank slots)
constexpr int VROW = 12;          // padding of a V~ row, bf16 elements (24 B; 0 is 2.5x slower at
                                  // 256 dims, 4, 8 and 16 are 1 to 20 % slower than 12)
constexpr int LDS_AHEAD = 4;      // LDS fragments in flight ahead of the matrix-core step using them

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Two 2-bit codes at bits 0-1 and 16-17 of x -> a dword of two bf16 values
// (code c -> 0, 1, 2, 3 = 0x0000, 0x3F80, 0x4000, 0x4040), by a byte-permute
// lookup whose selector bytes are 2c and 2c + 1.
__device__ __forceinline__ uint32_t codes_to_bf16x2(uint32_t x) {
    return __builtin_amdgcn_perm(0x40404000u, 0x3F800000u, x * 0x202u + 0x01000100u);
}
// kappa index -> dim: kappa = 16u + 2k + e holds dim 16u + k + 8e
__device__ __forceinline__ int kappa_dim(int kappa) { return (kappa & ~15) + ((kappa & 1) << 3) + ((kappa & 15) >> 1); }
// fp32 -> bf16 rounded to nearest, and the rounded residual, packed for two
// values: a = hi + lo to 2^-18 relative, with unbiased errors (truncation
// would bias every weight low, and the bias survives the sum over the keys
// where the code part and the offset part of the output nearly cancel)
__device__ __forceinline__ void split_hi_lo(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
    const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xFFFF0000u);  // exact
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){ra, rb}, bf16x2));
}

// Max over the four 16-lane rows of the wave (the value of lanes l, l^16,
// l^32, l^48), with the row-swapping permutes instead of LDS shuffles.
__device__ __forceinline__ float max_rows(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

}  // namespace

template <int D>
struct PrefillLds {
    static constexpr int KS = D + KROW;
    static constexpr int VS = PAGE + VROW;
    uint16_t k[2][PAGE * KS];  // K~, two buffers
    uint16_t v[2][D * VS];     // V~, two buffers
    float4 meta[2][PAGE];      // {k scale, k min - 4 k scale, v scale, v min} per key
};

// Packed codes of one page held by a thread between its load and its conversion.
template <int D, int FMT>
struct PackedPage {
    static constexpr int NW = D / 64;  // K words and V words per thread
    uint32_t k[NW];
    uint32_t v[NW];
    uint4 meta;  // threads < 64: {k scale, k min, v scale, v min} of key tid
};
// bf16 pool: the page's values as stored, 16-byte pieces
template <int D>
struct PackedPage<D, KV_FMT_BF16> {
    static constexpr int NK = D / 64;  // K items (key, 16 dims: two pieces) per thread
    static constexpr int NV = D / 32;  // V pieces (dim, 8 keys) per thread
    uint4 k[2 * NK];
    uint4 v[NV];
};

template <int D>
__device__ __forceinline__ void load_packed(PackedPage<D, KV_FMT_BF16>& pk, const uint8_t* blk, int tid) {
    constexpr int NK = PackedPage<D, KV_FMT_BF16>::NK, NV = PackedPage<D, KV_FMT_BF16>::NV;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int item = tid + 256 * i, t = item / (D / 16), u = item % (D / 16);
        const uint4* src = reinterpret_cast<const uint4*>(blk + 2 * (t * D + 16 * u));
        pk.k[2 * i] = src[0];
        pk.k[2 * i + 1] = src[1];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int item = tid + 256 * i;  // dim item / 8, keys 8 (item % 8) ..
        pk.v[i] = *reinterpret_cast<const uint4*>(blk + 128 * D + 16 * item);
    }
}

template <int D>
__device__ __forceinline__ void load_packed(PackedPage<D, KV_FMT_Q2>& pk, const uint8_t* blk, int tid) {
    constexpr int NW = PackedPage<D, KV_FMT_Q2>::NW, KW = D / 16;  // code words per K row
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int item = tid + 256 * i;  // K: (key, word)
        pk.k[i] = *reinterpret_cast<const uint32_t*>(blk + (item / KW) * (D / 4) + 4 * (item % KW));
        const int d = item >> 2, w = item & 3;  // V: (dim, word)
        pk.v[i] = *reinterpret_cast<const uint32_t*>(blk + q2_vcodes_off(D) + q2_vword_off(D, d, w));
    }
    if (tid < PAGE) {
        const float2 km = *reinterpret_cast<const float2*>(blk + q2_kmeta_off(D) + 8 * tid);
        const float2 vm = *reinterpret_cast<const float2*>(blk + q2_vmeta_off(D) + 8 * tid);
        pk.meta = make_uint4(__float_as_uint(km.x), __float_as_uint(km.y), __float_as_uint(vm.x), __float_as_uint(vm.y));
    }
}

// Item i (one K word, one V word) of a thread's share of the page conversion.
template <int D>
__device__ __forceinline__ void convert_item(const PackedPage<D, KV_FMT_Q2>& pk, PrefillLds<D>& L, int buf, int tid,
                                             int i) {
    constexpr int KW = D / 16, KS = PrefillLds<D>::KS, VS = PrefillLds<D>::VS;
    {
        const int item = tid + 256 * i;
        // K word u of key t: dims 16u..16u+15 -> kappa 16u + 2k + e = dim 16u + k + 8e;
        // code c is stored as bf16(c + 4) = 0x4080 + 32 c (two bit operations a pair)
        {
            const int t = item / KW, u = item % KW;
            const uint32_t w = pk.k[i];
            uint32_t o[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t x = (5 - 2 * k) >= 0 ? w << (5 - 2 * k) : w >> (2 * k - 5);
                o[k] = (x & 0x00600060u) | 0x40804080u;
            }
            uint4* dst = reinterpret_cast<uint4*>(&L.k[buf][t * KS + 16 * u]);
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
        // V word w of dim d: slot 16b + 4w + r at bit 16(r % 2) + 4b + 2(r / 2)
        {
            const int d = item >> 2, wi = item & 3;
            const uint32_t w = pk.v[i];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t lo = codes_to_bf16x2((w >> (4 * b)) & 0x00030003u);      // slots r = 0, 1
                const uint32_t hi = codes_to_bf16x2((w >> (4 * b + 2)) & 0x00030003u);  // slots r = 2, 3
                *reinterpret_cast<uint2*>(&L.v[buf][d * VS + 16 * b + 4 * wi]) = make_uint2(lo, hi);
            }
        }
    }
}

// The per-key scale and offset of the page.
template <int D>
__device__ __forceinline__ void convert_meta(const PackedPage<D, KV_FMT_Q2>& pk, PrefillLds<D>& L, int buf, int tid) {
    // the K offset absorbs the +4 of the stored codes: k^ = min + scale c = (min - 4 scale) + scale (c + 4)
    if (tid < PAGE) {
        const float ks = __uint_as_float(pk.meta.x);
        L.meta[buf][tid] = make_float4(ks, __uint_as_float(pk.meta.y) - 4.0f * ks, __uint_as_float(pk.meta.z),
                                       __uint_as_float(pk.meta.w));
    }
}

template <int D>
__device__ __forceinline__ void convert_packed(const PackedPage<D, KV_FMT_Q2>& pk, PrefillLds<D>& L, int buf, int tid,
                                               int /*n_valid: codes are finite in any slot*/) {
#pragma unroll
    for (int i = 0; i < PackedPage<D, KV_FMT_Q2>::NW; ++i) convert_item<D>(pk, L, buf, tid, i);
    convert_meta<D>(pk, L, buf, tid);
}

// bf16 pool: K dims 16u + k and 16u + k + 8 made adjacent (kappa order), V
// copied; unit scales and zero offsets.  Slots from n_valid on were never
// written and may hold NaN patterns: they become zeros (a zero weight times a
// NaN value would still poison the p.v sum).
template <int D>
__device__ __forceinline__ void convert_packed(const PackedPage<D, KV_FMT_BF16>& pk, PrefillLds<D>& L, int buf,
                                               int tid, int n_valid) {
    constexpr int NK = PackedPage<D, KV_FMT_BF16>::NK, NV = PackedPage<D, KV_FMT_BF16>::NV;
    constexpr int KS = PrefillLds<D>::KS, VS = PrefillLds<D>::VS;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int item = tid + 256 * i, t = item / (D / 16), u = item % (D / 16);
        const uint4 a = pk.k[2 * i], b = pk.k[2 * i + 1];  // dims 16u .. +7, 16u + 8 .. +15
        const uint32_t keep = t < n_valid ? 0xFFFFFFFFu : 0u;
        const uint32_t aa[4] = {a.x & keep, a.y & keep, a.z & keep, a.w & keep};
        const uint32_t bb[4] = {b.x & keep, b.y & keep, b.z & keep, b.w & keep};
        uint32_t o[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            o[2 * k] = __builtin_amdgcn_perm(bb[k], aa[k], 0x05040100u);      // dims 16u + 2k, 16u + 2k + 8
            o[2 * k + 1] = __builtin_amdgcn_perm(bb[k], aa[k], 0x07060302u);  // dims 16u + 2k + 1, 16u + 2k + 9
        }
        uint4* dst = reinterpret_cast<uint4*>(&L.k[buf][t * KS + 16 * u]);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int item = tid + 256 * i, d = item >> 3, p = item & 7;
        uint32_t w[4] = {pk.v[i].x, pk.v[i].y, pk.v[i].z, pk.v[i].w};
        if (8 * p + 8 > n_valid) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w[k] &= (8 * p + 2 * k < n_valid ? 0xFFFFu : 0u) | (8 * p + 2 * k + 1 < n_valid ? 0xFFFF0000u : 0u);
        }
        uint2* dst = reinterpret_cast<uint2*>(&L.v[buf][d * VS + 8 * p]);
        dst[0] = make_uint2(w[0], w[1]);
        dst[1] = make_uint2(w[2], w[3]);
    }
    if (tid < PAGE) L.meta[buf][tid] = make_float4(1.f, 0.f, 1.f, 0.f);
}

// Pages [pg0, pg1) of split sp for a block whose last query sits at pos_max;
// only pages below kpl are read from the pool (a window pool's window page
// and later are not).
__device__ __forceinline__ void prefill_split_range(int pos_max, int splits, int sp, int kpl, int* pg0, int* pg1) {
    const int n_pages = min(pos_max / PAGE + 1, kpl);
    const int per = (n_pages + splits - 1) / splits;
    *pg0 = min(sp * per, n_pages);
    *pg1 = min(sp * per + per, n_pages);
}

// ROTQ (the rotated 2-bit format): q holds each (query, head) row as two bf16
// terms of its rotated values, [n_q][Hq][2][D] (rounded value, then rounded
// residual), and both enter the q.k product; the scale passed is sm / D.
template <int D, int FMT, bool ROTQ>
__global__ __launch_bounds__(256) void prefill_kernel(PoolView pv, int layer, int seq, int q_start, int n_q,
                                                      const uint16_t* __restrict__ q, float sm, int splits,
                                                      int kpl, float* __restrict__ ws) {
    constexpr int NCB = PREFILL_NCB<ROTQ>, ROWS = PREFILL_ROWS<ROTQ>;
    constexpr int QTERMS = ROTQ ? 2 : 1;
    constexpr int KSTEPS = D / 32, DB = D / 16;
    constexpr int KS = PrefillLds<D>::KS, VS = PrefillLds<D>::VS;
    const int Hkv = pv.Hkv, Hq = pv.Hq, G = Hq / Hkv;
    const int QB = ROWS / G;  // queries per workgroup
    const int g = blockIdx.x % Hkv, qb = blockIdx.x / Hkv, sp = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, j = l & 15, grp = l >> 4;
    const int q_first = qb * QB;
    const int pos_max = q_start + min(q_first + QB, n_q) - 1;
    int pg0, pg1;
    prefill_split_range(pos_max, splits, sp, kpl, &pg0, &pg1);
    if (pg0 >= pg1) return;

    __shared__ __align__(16) PrefillLds<D> L;

    const int32_t* bt = pv.bt + (int64_t)seq * pv.bt_stride;
    const int64_t lhoff = ((int64_t)layer * Hkv + g) * pv.block_bytes;
    auto block_of = [&](int pg) { return pv.pages + (int64_t)bt[pg] * pv.page_bytes + lhoff; };

    PackedPage<D, FMT> pk;
    load_packed<D>(pk, block_of(pg0), tid);

    // ---- this lane's rows: column j of block cb = (query, head) ----
    int qi[NCB], pos[NCB];
    bool live[NCB];
    float qsum[NCB];
    bf16x8 qop[NCB][QTERMS][KSTEPS];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = 16 * (NCB * wave + cb) + j;
        qi[cb] = q_first + col / G;
        live[cb] = qi[cb] < n_q;
        pos[cb] = q_start + min(qi[cb], n_q - 1);
        const uint16_t* qrow = q + ((int64_t)min(qi[cb], n_q - 1) * Hq + g * G + col % G) * QTERMS * D;
        float s = 0.f;
#pragma unroll
        for (int tm = 0; tm < QTERMS; ++tm)
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                // kappa = 32 ks + 8 grp + e; dims of kappa .. kappa + 7: two runs of four
                const int kap = 32 * ks + 8 * grp, d0 = kappa_dim(kap);
                const uint2 a = *reinterpret_cast<const uint2*>(qrow + tm * D + d0);      // dims d0 .. d0+3
                const uint2 b = *reinterpret_cast<const uint2*>(qrow + tm * D + d0 + 8);  // dims d0+8 .. d0+11
                // interleave: kappa order d0, d0+8, d0+1, d0+9, ...
                const uint4 u = make_uint4(__builtin_amdgcn_perm(b.x, a.x, 0x05040100u),
                                           __builtin_amdgcn_perm(b.x, a.x, 0x07060302u),
                                           __builtin_amdgcn_perm(b.y, a.y, 0x05040100u),
                                           __builtin_amdgcn_perm(b.y, a.y, 0x07060302u));
                qop[cb][tm][ks] = as_bf16x8(u);
                s += bf16_to_f32((uint16_t)(a.x & 0xFFFF)) + bf16_to_f32((uint16_t)(a.x >> 16)) +
                     bf16_to_f32((uint16_t)(a.y & 0xFFFF)) + bf16_to_f32((uint16_t)(a.y >> 16)) +
                     bf16_to_f32((uint16_t)(b.x & 0xFFFF)) + bf16_to_f32((uint16_t)(b.x >> 16)) +
                     bf16_to_f32((uint16_t)(b.y & 0xFFFF)) + bf16_to_f32((uint16_t)(b.y >> 16));
            }
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        qsum[cb] = s;
    }

    constexpr float LOG2E = 1.4426950408889634f;
    const float cB = sm * LOG2E;
    f32x4 acc[NCB][DB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref[NCB], l_run[NCB], c_run[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        m_ref[cb] = -INFINITY;
        l_run[cb] = 0.f;
        c_run[cb] = 0.f;
    }

    const int key_end = q_start + n_q;  // keys at and past it were never appended
    convert_packed<D>(pk, L, 0, tid, key_end - pg0 * PAGE);
    __syncthreads();
    // pages [pg0, pg_full) are visible to every row of the block (no mask);
    // the rest reach past the block's first query position
    const int pg_full = max(pg0, min(pg1, (q_start + q_first + 1) / PAGE));
    float alpha[NCB];
    auto page_step = [&](int pg, auto masked_tag) -> bool {
        const int buf = (pg - pg0) & 1;
        if (pg + 1 < pg1) load_packed<D>(pk, block_of(pg + 1), tid);
        const uint16_t* Kt = L.k[buf];
        const uint16_t* Vt = L.v[buf];
        // ---- S^T = K~ Q^T: keys 16 kb + 4 grp + r of the page, column j ----
        f32x4 st[NCB][4];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) st[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // fragments are read LDS_AHEAD steps before their products, so that
        // the LDS latency hides behind the matrix-core work of the steps between
        constexpr int NQK = 4 * KSTEPS;
        auto kfrag = [&](int idx) {
            const int kb = idx / KSTEPS, ks = idx % KSTEPS;
            return as_bf16x8(*reinterpret_cast<const uint4*>(&Kt[(16 * kb + j) * KS + 32 * ks + 8 * grp]));
        };
        bf16x8 fk[LDS_AHEAD + 1];
#pragma unroll
        for (int idx = 0; idx < LDS_AHEAD; ++idx) fk[idx] = kfrag(idx);
#pragma unroll
        for (int idx = 0; idx < NQK; ++idx) {
            if (idx + LDS_AHEAD < NQK) fk[(idx + LDS_AHEAD) % (LDS_AHEAD + 1)] = kfrag(idx + LDS_AHEAD);
            const int kb = idx / KSTEPS, ks = idx % KSTEPS;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int tm = 0; tm < QTERMS; ++tm) st[cb][kb] = mma(fk[idx % (LDS_AHEAD + 1)], qop[cb][tm][ks], st[cb][kb]);
        }
        // ---- scores and the page's maximum per row (column j) ----
        constexpr bool MASKED = decltype(masked_tag)::value;
        bool need = false;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = 16 * kb + 4 * grp + r;
                    const float2 km = *reinterpret_cast<const float2*>(&L.meta[buf][key]);
                    float x = fmaf(km.x, st[cb][kb][r], km.y * qsum[cb]);
                    if (MASKED && pg * PAGE + key > pos[cb]) x = -INFINITY;
                    st[cb][kb][r] = x;
                    mt = fmaxf(mt, x);
                }
            mt = max_rows(mt);
            // lazy rescale: the reference moves only when a weight would pass 2^8
            const bool up = (mt - m_ref[cb]) * cB > 8.0f;
            alpha[cb] = up ? __builtin_amdgcn_exp2f((m_ref[cb] - mt) * cB) : 1.0f;
            m_ref[cb] = up ? mt : m_ref[cb];
            need |= up;
        }
        // a moved reference rescales the running sums before this page's
        // weights: the page is given back and retried after the rescale
        if (__builtin_amdgcn_ballot_w64(need)) return false;
        // ---- online softmax, weights w = p scale_v ----
        uint32_t phi[NCB][2][4], plo[NCB][2][4];
        {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const float cbm = m_ref[cb] * cB;
                float w[4][4], ls = 0.f, cs = 0.f;  // this page's sums, added to the running ones at the end
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = 16 * kb + 4 * grp + r;
                        const float2 vm =
                            *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(&L.meta[buf][key]) + 2);
                        if (MASKED) {  // slots past a row's position (or past the sequence) weigh nothing
                            const bool valid = pg * PAGE + key <= pos[cb];
                            const float p = valid ? __builtin_amdgcn_exp2f(fmaf(st[cb][kb][r], cB, -cbm)) : 0.f;
                            ls += p;
                            cs += valid ? p * vm.y : 0.f;
                            w[kb][r] = valid ? p * vm.x : 0.f;
                        } else {
                            const float p = __builtin_amdgcn_exp2f(fmaf(st[cb][kb][r], cB, -cbm));
                            ls += p;
                            cs = fmaf(p, vm.y, cs);
                            w[kb][r] = p * vm.x;
                        }
                    }
                l_run[cb] += ls;
                c_run[cb] += cs;
                // p.v operand of 32-key step ks: slots 8 grp .. 8 grp + 7 = keys of blocks 2ks (r) and 2ks + 1 (r)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    split_hi_lo(w[2 * ks][0], w[2 * ks][1], phi[cb][ks][0], plo[cb][ks][0]);
                    split_hi_lo(w[2 * ks][2], w[2 * ks][3], phi[cb][ks][1], plo[cb][ks][1]);
                    split_hi_lo(w[2 * ks + 1][0], w[2 * ks + 1][1], phi[cb][ks][2], plo[cb][ks][2]);
                    split_hi_lo(w[2 * ks + 1][2], w[2 * ks + 1][3], phi[cb][ks][3], plo[cb][ks][3]);
                }
            }
        }
        // ---- O^T += V~ P^T ----
        constexpr int NPV = 2 * DB;
        auto vfrag = [&](int idx) {
            const int db = idx >> 1, ks = idx & 1;
            const uint16_t* vr = &Vt[(16 * db + j) * VS + 32 * ks + 4 * grp];
            const uint2 v0 = *reinterpret_cast<const uint2*>(vr);       // keys 32ks + 4grp .. +3
            const uint2 v1 = *reinterpret_cast<const uint2*>(vr + 16);  // keys 32ks + 16 + 4grp .. +3
            return as_bf16x8(make_uint4(v0.x, v0.y, v1.x, v1.y));
        };
        bf16x8 fv[LDS_AHEAD + 1];
#pragma unroll
        for (int idx = 0; idx < LDS_AHEAD; ++idx) fv[idx] = vfrag(idx);
#pragma unroll
        for (int idx = 0; idx < NPV; ++idx) {
            if (idx + LDS_AHEAD < NPV) fv[(idx + LDS_AHEAD) % (LDS_AHEAD + 1)] = vfrag(idx + LDS_AHEAD);
            const int db = idx >> 1, ks = idx & 1;
            const bf16x8 a = fv[idx % (LDS_AHEAD + 1)];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                acc[cb][db] = mma(a, as_bf16x8(make_uint4(phi[cb][ks][0], phi[cb][ks][1], phi[cb][ks][2],
                                                          phi[cb][ks][3])), acc[cb][db]);
                acc[cb][db] = mma(a, as_bf16x8(make_uint4(plo[cb][ks][0], plo[cb][ks][1], plo[cb][ks][2],
                                                          plo[cb][ks][3])), acc[cb][db]);
            }
        }
        // the next page's tiles (the idle buffer was last read before the
        // previous barrier; after the last page this rewrites it with the page
        // already used, and nothing reads it)
        convert_packed<D>(pk, L, buf ^ 1, tid, key_end - (pg + 1) * PAGE);
        __syncthreads();
        return true;
    };
    // A wave that gives a page back rescales and retries it; every wave still
    // passes the one barrier of each page once.  The retry terminates: after
    // the rescale the page's maximum equals the reference.
    int pg = pg0;
    auto run_pages = [&](int pg_end, auto masked_tag) {
        while (pg < pg_end) {
            while (pg < pg_end && page_step(pg, masked_tag)) ++pg;
            if (pg < pg_end) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    l_run[cb] *= alpha[cb];
                    c_run[cb] *= alpha[cb];
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[cb][db] *= alpha[cb];
                }
            }
        }
    };
    run_pages(pg_full, std::false_type{});
    run_pages(pg1, std::true_type{});

    // ---- partials of this split: o^T lanes hold dims 16 db + 4 grp + r of column j ----
    float* wo = ws;
    float* wml = ws + (int64_t)n_q * Hq * splits * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const float lsum = l_run[cb] + __shfl_xor(l_run[cb], 16);
        const float lt = lsum + __shfl_xor(lsum, 32);
        const float csum = c_run[cb] + __shfl_xor(c_run[cb], 16);
        const float ct = csum + __shfl_xor(csum, 32);
        if (!live[cb]) continue;
        const int col = 16 * (NCB * wave + cb) + j;
        const int64_t row = ((int64_t)qi[cb] * Hq + g * G + col % G) * splits + sp;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const float4 o = make_float4(acc[cb][db][0] + ct, acc[cb][db][1] + ct, acc[cb][db][2] + ct,
                                         acc[cb][db][3] + ct);
            *reinterpret_cast<float4*>(&wo[row * D + 16 * db + 4 * grp]) = o;
        }
        if (grp == 0) {
            wml[2 * row] = m_ref[cb] * cB;  // log2 units
            wml[2 * row + 1] = lt;
        }
    }
}

// Merge of the prefill partials: one workgroup per (query, head); split p
// counts for query i when its first page starts at or before i's position and
// holds a page below kpl.  A window pool's window partials (win: outputs
// [n_q][Hq][D], then (max, sum) pairs; the window starts at key 64 kpl) count
// for the rows whose position reaches the window, the only rows written.
__global__ __launch_bounds__(256) void prefill_merge_kernel(int q_start, int n_q, int Hq, int Hkv, int D, int splits,
                                                            int kpl, int rows_per_block, const float* __restrict__ ws,
                                                            const float* __restrict__ win, float* __restrict__ out) {
    const int row = blockIdx.x;  // i * Hq + h
    const int i = row / Hq, G = Hq / Hkv;
    const int d = threadIdx.x;
    const int QB = rows_per_block / G, qb = i / QB;
    const int pos = q_start + i;
    const int pos_max = q_start + min(qb * QB + QB, n_q) - 1;
    const int n_pages = min(pos_max / PAGE + 1, kpl);
    int live = 0;
    if (n_pages > 0) {
        const int per = (n_pages + splits - 1) / splits;
        live = min(min(splits, pos / (per * PAGE) + 1), (n_pages + per - 1) / per);
    }
    const float2* ml = reinterpret_cast<const float2*>(ws + (int64_t)n_q * Hq * splits * D) + (int64_t)row * splits;
    const float* o = ws + (int64_t)row * splits * D + d;
    float M = -INFINITY, wm = -INFINITY, wl = 0.f, wo = 0.f;
    if (win && pos >= kpl * PAGE) {
        const float2 w = reinterpret_cast<const float2*>(win + (int64_t)n_q * Hq * D)[row];
        wm = w.x;
        wl = w.y;
        wo = win[(int64_t)row * D + d];
        M = wm;
    }
    for (int p = 0; p < live; ++p) M = fmaxf(M, ml[p].x);
    float den = 0.f, acc = 0.f;
    if (wl > 0.f) {
        const float f = exp2f(wm - M);
        den = f * wl;
        acc = f * wo;
    }
    for (int p = 0; p < live; ++p) {
        const float f = exp2f(ml[p].x - M);
        den += f * ml[p].y;
        acc += f * o[(int64_t)p * D];
    }
    out[(int64_t)row * D + d] = acc / den;
}

static_assert(PREFILL_ROWS<true> == 64 && PREFILL_ROWS<false> == 128, "prefill_rows_per_block() matches the kernels");

// The rotated format's query rows: H q in fp32 butterflies (the stages of the
// rotated append, H the unnormalised Walsh-Hadamard matrix), each row written
// as two bf16 terms, the rotated value rounded to nearest and the rounded
// residual: [n_q][Hq][2][D].  A row on the 16 lanes of a DPP row, sixteen rows
// a workgroup.
template <int D>
__global__ __launch_bounds__(256) void rotate_query_kernel(const uint16_t* __restrict__ q, int rows,
                                                           uint16_t* __restrict__ qr) {
    constexpr int DPL = D / 16;
    const int row = blockIdx.x * 16 + (threadIdx.x >> 4), c = threadIdx.x & 15;
    const bool in = row < rows;  // every lane takes part in the row shuffles
    float x[DPL];
    const uint16_t* src = q + (int64_t)min(row, rows - 1) * D + c * DPL;
#pragma unroll
    for (int k = 0; k < DPL; ++k) x[k] = bf16_to_f32(src[k]);
    hadamard_row16<DPL>(x, c);
    uint32_t hi[DPL / 2], lo[DPL / 2];
#pragma unroll
    for (int k = 0; k < DPL / 2; ++k) split_hi_lo(x[2 * k], x[2 * k + 1], hi[k], lo[k]);
    if (in) {
        uint32_t* dh = reinterpret_cast<uint32_t*>(qr + (int64_t)row * 2 * D + c * DPL);
        uint32_t* dl = reinterpret_cast<uint32_t*>(qr + (int64_t)row * 2 * D + D + c * DPL);
#pragma unroll
        for (int k = 0; k < DPL / 2; ++k) {
            dh[k] = hi[k];
            dl[k] = lo[k];
        }
    }
}

hipError_t launch_prefill_window(const PoolView& pv, int layer, int seq, int q_start, int n_q, int w0,
                                 const uint16_t* q, float sm, float* wo, float* wml, hipStream_t s);

hipError_t launch_prefill(const PoolView& pv, int fmt, int layer, int seq, int q_start, int n_q, const uint16_t* q,
                          float sm, int splits, float* ws, float* out, int w0, hipStream_t s) {
    const int G = pv.Hq / pv.Hkv, rows = prefill_rows_per_block(fmt), QB = rows / G;
    const bool window = fmt == KV_FMT_Q2_WINDOW;
    const int kpl = window ? w0 / PAGE : INT_MAX;
    dim3 grid(((n_q + QB - 1) / QB) * pv.Hkv, splits);
    if (fmt == KV_FMT_BF16) {
        if (pv.D == 256)
            hipLaunchKernelGGL((prefill_kernel<256, KV_FMT_BF16, false>), grid, dim3(256), 0, s, pv, layer, seq,
                               q_start, n_q, q, sm, splits, kpl, ws);
        else
            hipLaunchKernelGGL((prefill_kernel<128, KV_FMT_BF16, false>), grid, dim3(256), 0, s, pv, layer, seq,
                               q_start, n_q, q, sm, splits, kpl, ws);
    } else if (fmt == KV_FMT_Q2_ROT) {
        // the rotated query terms sit after the splits' partials
        uint16_t* qr = reinterpret_cast<uint16_t*>(ws + prefill_ws_floats(n_q, pv.Hq, pv.D, splits));
        const int qrows = n_q * pv.Hq;
        const float smr = sm / (float)pv.D;  // H q . H k = D q . k
        if (pv.D == 256) {
            hipLaunchKernelGGL(rotate_query_kernel<256>, dim3((qrows + 15) / 16), dim3(256), 0, s, q, qrows, qr);
            hipLaunchKernelGGL((prefill_kernel<256, KV_FMT_Q2, true>), grid, dim3(256), 0, s, pv, layer, seq, q_start,
                               n_q, qr, smr, splits, kpl, ws);
        } else {
            hipLaunchKernelGGL(rotate_query_kernel<128>, dim3((qrows + 15) / 16), dim3(256), 0, s, q, qrows, qr);
            hipLaunchKernelGGL((prefill_kernel<128, KV_FMT_Q2, true>), grid, dim3(256), 0, s, pv, layer, seq, q_start,
                               n_q, qr, smr, splits, kpl, ws);
        }
    } else if (kpl > 0) {
        if (pv.D == 256)
            hipLaunchKernelGGL((prefill_kernel<256, KV_FMT_Q2, false>), grid, dim3(256), 0, s, pv, layer, seq, q_start,
                               n_q, q, sm, splits, kpl, ws);
        else
            hipLaunchKernelGGL((prefill_kernel<128, KV_FMT_Q2, false>), grid, dim3(256), 0, s, pv, layer, seq, q_start,
                               n_q, q, sm, splits, kpl, ws);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    float* win = nullptr;
    if (window) {
        win = ws + prefill_ws_floats(n_q, pv.Hq, pv.D, splits);
        err = launch_prefill_window(pv, layer, seq, q_start, n_q, w0, q, sm, win, win + (int64_t)n_q * pv.Hq * pv.D, s);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(prefill_merge_kernel, dim3(n_q * pv.Hq), dim3(pv.D), 0, s, q_start, n_q, pv.Hq, pv.Hkv, pv.D,
                       splits, kpl, rows, ws, win, out);
    return hipGetLastError();
}

}  // namespace kvq
