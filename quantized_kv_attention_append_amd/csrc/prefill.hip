// Chunked causal prefill: the chunk's queries attend to the prior tokens and
// to the chunk itself, every key and value read from the compressed pages ("KV
// at 9 KB a token", opening section: prefill attention reads the compressed
// cache directly, and every workspace byte a launch reads it wrote first).
//
// Query i of the chunk sits at position q_start + i and sees keys
// 0 .. q_start + i (inclusive).  Scores are sm q.k^ with the dequantization
// folded algebraically (q.k^_t = min_t sum(q) + scale_t q.c_t); the online
// softmax and every sum are fp32 (the two-level accumulation of "Half the
// Cache, Twice the Context", section "The cliff is in the accumulator").
// Both contractions run on the bf16 matrix cores:
//   * codes and the bf16 query are exact bf16 operands, so q.c is exact up to
//     the fp32 sum;
//   * the softmax weights w = p scale_v are split into two bf16 terms (w
//     rounded to bf16, then the rounded residual), 17 significant bits.
// The score tile is computed transposed, S^T = K~ Q^T (rows = keys, columns =
// (query, head) rows), so that the lanes holding a row's keys already hold
// that row's p.v operand O^T = V~ P^T: no transpose of P is needed.
// Every page of 64 keys is converted once per workgroup into bf16 LDS tiles,
// K~[key][kappa] (kappa: the order of dims in which dims 16u + k and
// 16u + k + 8 are adjacent) and V~[dim][key].  Partials (m, l, o) of every
// row go to the workspace; prefill_merge_kernel merges, for each row, the
// splits whose first key it can see.
//
// Two kernels: prefill_ws_kernel (2-bit pools, plain, window and rotated:
// warp-specialised, on v_mfma_f32_32x32x16_bf16) and prefill_bf16_kernel (bf16
// pools: the stored values in the same tiles with unit metadata, four waves
// of two 16-row blocks on v_mfma_f32_16x16x32_bf16).
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

// bf16 pools: a wave owns NCB = 2 16-column blocks of (query, head) rows, a
// workgroup four waves: 128 rows.
constexpr int PREFILL_NCB = 2;
constexpr int PREFILL_ROWS = 4 * PREFILL_NCB * 16;
constexpr int KROW = 8;           // padding of a K~ row, bf16 elements (16 B: the 16 rows a read group
                                  // touches start in distinct 16-byte bank slots)
constexpr int VROW = 12;          // padding of a V~ row, bf16 elements (24 B; 0 is 2.5x slower at
                                  // 256 dims, 4, 8 and 16 are 1 to 20 % slower than 12)
constexpr int LDS_AHEAD = 4;      // LDS fragments in flight ahead of the matrix-core step using them

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

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
    float4 meta[2][PAGE];      // unit scales and zero offsets (the bf16 pool stores values)
};

// The page's values as stored, held by a thread between their load and their
// conversion: 16-byte pieces.
template <int D>
struct PackedPage {
    static constexpr int NK = D / 64;  // K items (key, 16 dims: two pieces) per thread
    static constexpr int NV = D / 32;  // V pieces (dim, 8 keys) per thread
    uint4 k[2 * NK];
    uint4 v[NV];
};

template <int D>
__device__ __forceinline__ void load_packed(PackedPage<D>& pk, const uint8_t* blk, int tid) {
    constexpr int NK = PackedPage<D>::NK, NV = PackedPage<D>::NV;
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

// bf16 pool: K dims 16u + k and 16u + k + 8 made adjacent (kappa order), V
// copied; unit scales and zero offsets.  Slots from n_valid on were never
// written and may hold NaN patterns: they become zeros (a zero weight times a
// NaN value would still poison the p.v sum).
template <int D>
__device__ __forceinline__ void convert_packed(const PackedPage<D>& pk, PrefillLds<D>& L, int buf,
                                               int tid, int n_valid) {
    constexpr int NK = PackedPage<D>::NK, NV = PackedPage<D>::NV;
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

// Prefill over a bf16 pool (the stored values in the tiles, unit metadata).
template <int D>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(PoolView pv, int layer, int seq, int q_start, int n_q,
                                                           const uint16_t* __restrict__ q, float sm, int splits,
                                                           int kpl, float* __restrict__ ws) {
    constexpr int NCB = PREFILL_NCB, ROWS = PREFILL_ROWS;
    constexpr int QTERMS = 1;
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

    PackedPage<D> pk;
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
            __builtin_amdgcn_sched_barrier(0);  // keeps the read ahead (the scheduler would sink it to its use)
            const int kb = idx / KSTEPS, ks = idx % KSTEPS;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int tm = 0; tm < QTERMS; ++tm) st[cb][kb] = mma(fk[idx % (LDS_AHEAD + 1)], qop[cb][tm][ks], st[cb][kb]);
            __builtin_amdgcn_sched_barrier(0);
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
            __builtin_amdgcn_sched_barrier(0);
            const int db = idx >> 1, ks = idx & 1;
            const bf16x8 a = fv[idx % (LDS_AHEAD + 1)];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                acc[cb][db] = mma(a, as_bf16x8(make_uint4(phi[cb][ks][0], phi[cb][ks][1], phi[cb][ks][2],
                                                          phi[cb][ks][3])), acc[cb][db]);
                acc[cb][db] = mma(a, as_bf16x8(make_uint4(plo[cb][ks][0], plo[cb][ks][1], plo[cb][ks][2],
                                                          plo[cb][ks][3])), acc[cb][db]);
            }
            __builtin_amdgcn_sched_barrier(0);
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

// ---------------------------------------------------------------------------
// Warp-specialised prefill over 2-bit pools (plain, window and rotated).
//
// Eight waves, two on each SIMD (waves w and w + 4 share one): waves 0-3
// ("score waves") take q.k and the online softmax of 32 (query, head) rows
// each, waves 4-7 ("output waves") take p.v of the same rows one page behind.
// Page step t has two phases, each closed by a workgroup barrier, so that on
// every SIMD one wave's matrix products run while the other's vector work
// issues:
//   phase 1  score wave: S^T = K~(t) Q^T from the K tile of page t, then the
//            scores (the dequantization folded in), the page maximum and the
//            row references;
//            output wave: takes the weights and rescale factors of page t - 1
//            into registers, expands the packed V words of page t - 1 into
//            the V tile and page t + 1 into the other K tile;
//   phase 2  score wave: running sums and the weights w = p scale_v of page t
//            as two bf16 terms, with each row's rescale factor;
//            output wave: loads the codes of pages t (V) and t + 2 (K), then
//            rescales its accumulators and adds V~(t - 1) P(t - 1)^T.
// Both products run on v_mfma_f32_32x32x16_bf16 (twice the rate of the
// 16x16x32 shape on this chip).  A wave's 32 rows are the 32 columns of every
// product; lane l holds column l % 32 and, for half h = l / 32 of the 16-deep
// step, operand slots 8h .. 8h + 7; result register r of lane l is row
// 8 (r / 4) + 4h + r % 4.  So a score lane holds keys 8m + 4h + (0..3) of each
// 32-key block (m = 0..3), and the same lane's weights form the p.v operand of
// the step over keys 16 s .. 16 s + 15 of the block (s = 0, 1) with no data
// movement; the V operand of that step reads the same keys from the V tile.
// K codes c enter q.k as bf16(c + 4) (two bit operations a pair of codes), V
// codes p.v as bf16(c - 1.5) (a byte-permute lookup); the offsets carry the
// difference.
// ---------------------------------------------------------------------------
constexpr int WS_PAIRS = 4;                 // (score wave, output wave) pairs
constexpr int WS_NT = 128 * WS_PAIRS;       // 512 threads
constexpr int WS_ROWS = 32 * WS_PAIRS;      // (query, head) rows a workgroup
constexpr int WS_OT = 64 * WS_PAIRS;        // threads of the output waves
constexpr int WS_AHEAD_O = 3;               // steps an LDS fragment read runs ahead of its products
template <bool ROTQ>                        // in p.v and in q.k (the rotated query's second term takes
constexpr int WS_AHEAD_S = ROTQ ? 2 : 4;    // the registers of the deeper q.k prefetch)

typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct WsLds {
    static constexpr int KS = D + KROW;
    static constexpr int VS = PAGE + VROW;
    uint16_t k[2][PAGE * KS];          // K~ of pages t (read) and t + 1 (written), kappa order
    uint16_t v[D * VS];                // V~ of one page, [dim][key]
    uint4 p[WS_PAIRS][4][2][64];       // [pair][16-key step][term][lane] weight fragments of one page
    float2 kmeta[2][PAGE];             // {k scale, k min - 4 k scale}
    float2 vmeta[2][PAGE];             // {v scale, v min + 1.5 v scale}
    float alpha[WS_ROWS];              // rescale factor of each row before the page's p.v
    float cfin[WS_ROWS];               // sum p (v min + 1.5 v scale) of each row, at the end
};

// An output-wave thread's share of a page: one 16-byte piece of the K code
// plane (piece o / 64 of key o % 64's row, so that the 64 lanes of a wave write
// 64 different rows of the K tile) and one of the V code plane (pieces o < D),
// and the metadata of key o (o < 64).
struct WsStageK {
    uint4 piece;
    float2 kmeta, vmeta;  // kept as loaded: assembling them at once would wait for the loads
};

template <int D>
__device__ __forceinline__ void ws_load_k(WsStageK& st, const uint8_t* blk, int o) {
    if (o < D) st.piece = *reinterpret_cast<const uint4*>(blk + 16 * ((o % PAGE) * (D / 64) + o / PAGE));
    if (o < PAGE) {
        st.kmeta = *reinterpret_cast<const float2*>(blk + q2_kmeta_off(D) + 8 * o);
        st.vmeta = *reinterpret_cast<const float2*>(blk + q2_vmeta_off(D) + 8 * o);
    }
}
template <int D>
__device__ __forceinline__ void ws_load_v(uint4& st, const uint8_t* blk, int o) {
    if (o < D) st = *reinterpret_cast<const uint4*>(blk + q2_vcodes_off(D) + 16 * o);
}

// (x & m) | c in one instruction: the mask from a scalar register, the other
// constant from a vector register (one scalar operand per vector instruction)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
    return r;
}
// two 2-bit K codes at bits s and 16 + s of w -> a dword of two bf16(c + 4)
template <int S>
__device__ __forceinline__ uint32_t codes_pair(uint32_t w) {
    const uint32_t x = S <= 5 ? w << (5 - S) : w >> (S - 5);
    return and_or(x, 0x00600060u, 0x40804080u);
}

// The K piece of thread o: words 4 u4 .. 4 u4 + 3 of key t (t = o % 64, u4 =
// o / 64); word u holds dims 16u + k (bits 2k) and 16u + k + 8 (bits 16 + 2k)
// -> kappa 16u + 2k, 16u + 2k + 1.
template <int D>
__device__ __forceinline__ void ws_store_k(const WsStageK& st, WsLds<D>& L, int mb, int o) {
    constexpr int KS = WsLds<D>::KS;
    if (o < D) {
        const int t = o % PAGE, u4 = o / PAGE;
        const uint32_t w4[4] = {st.piece.x, st.piece.y, st.piece.z, st.piece.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = w4[e];
            uint4* dst = reinterpret_cast<uint4*>(&L.k[mb][t * KS + 64 * u4 + 16 * e]);
            dst[0] = make_uint4(codes_pair<0>(w), codes_pair<2>(w), codes_pair<4>(w), codes_pair<6>(w));
            dst[1] = make_uint4(codes_pair<8>(w), codes_pair<10>(w), codes_pair<12>(w), codes_pair<14>(w));
        }
    }
    if (o < PAGE) {  // K codes enter as c + 4, V codes as c - 1.5
        L.kmeta[mb][o] = make_float2(st.kmeta.x, st.kmeta.y - 4.0f * st.kmeta.x);
        L.vmeta[mb][o] = make_float2(st.vmeta.x, st.vmeta.y + 1.5f * st.vmeta.x);
    }
}
// Two 2-bit V codes at bits s and 16 + s of w -> a dword of two bf16(c - 1.5),
// by a byte-permute lookup (selector bytes 2c, 2c + 1 into the table of the four
// values).  Centred codes keep the code part of p.v near the size of the output,
// so the weights' rounding is not magnified by a cancelling offset.
template <int S>
__device__ __forceinline__ uint32_t vcodes_pair(uint32_t w) {
    const uint32_t x = (w >> S) & 0x00030003u;
    return __builtin_amdgcn_perm(0x3FC03F00u, 0xBF00BFC0u, x * 0x202u + 0x01000100u);
}
// Piece o of the V plane (bytes 16 o ..): four words of the plane; word w of
// dim d holds slots 16b + 4w + r at bits 16 (r % 2) + 4b + 2 (r / 2), which go
// to V~[d][16b + 4w + r].
template <int D>
__device__ __forceinline__ void ws_store_v(const uint4& st, WsLds<D>& L, int o) {
    constexpr int VS = WsLds<D>::VS;
    if (o < D) {
        const uint32_t w4[4] = {st.x, st.y, st.z, st.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // byte offset 16 o + 4 e of the plane -> (dim, word), inverting q2_vword_off
            const int off = 16 * o + 4 * e;
            const int half = off / (8 * D), rest = off % (8 * D);
            const int pair = rest / 16, in16 = rest % 16;
            const int d = 32 * (pair / 16) + (pair % 16) + 16 * (in16 / 8);
            const int w = 2 * half + (in16 % 8) / 4;
            const uint32_t x = w4[e];
            uint2* dst = reinterpret_cast<uint2*>(&L.v[d * VS + 4 * w]);
            dst[0] = make_uint2(vcodes_pair<0>(x), vcodes_pair<2>(x));      // b = 0: slots 4w .. 4w + 3
            dst[4] = make_uint2(vcodes_pair<4>(x), vcodes_pair<6>(x));      // b = 1: slots 16 + 4w ..
            dst[8] = make_uint2(vcodes_pair<8>(x), vcodes_pair<10>(x));     // b = 2
            dst[12] = make_uint2(vcodes_pair<12>(x), vcodes_pair<14>(x));   // b = 3
        }
    }
}

template <int D, bool ROTQ>
__global__ __launch_bounds__(WS_NT) void prefill_ws_kernel(PoolView pv, int layer, int seq, int q_start, int n_q,
                                                           const uint16_t* __restrict__ q, float sm, int splits,
                                                           int kpl, float* __restrict__ ws) {
    constexpr int QTERMS = ROTQ ? 2 : 1;
    constexpr int KS16 = D / 16;  // 16-dim steps of q.k
    constexpr int DB = D / 32;    // 32-dim blocks of p.v
    constexpr int KS = WsLds<D>::KS, VS = WsLds<D>::VS;
    const int Hkv = pv.Hkv, Hq = pv.Hq, G = Hq / Hkv;
    const int QB = WS_ROWS / G;  // queries per workgroup
    const int g = blockIdx.x % Hkv, qb = blockIdx.x / Hkv, sp = blockIdx.y;
    const int tid = threadIdx.x, l = tid & 63, c = l & 31, h = l >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the role branches below are scalar
    const int pw = wave & (WS_PAIRS - 1);
    const int q_first = qb * QB;
    const int pos_max = q_start + min(q_first + QB, n_q) - 1;
    int pg0, pg1;
    prefill_split_range(pos_max, splits, sp, kpl, &pg0, &pg1);
    if (pg0 >= pg1) return;  // the whole workgroup, before any barrier
    const int n = pg1 - pg0;

    __shared__ __align__(16) WsLds<D> L;

    const int32_t* bt = pv.bt + (int64_t)seq * pv.bt_stride;
    const int64_t lhoff = ((int64_t)layer * Hkv + g) * pv.block_bytes;
    auto block_at = [&](int id) { return pv.pages + (int64_t)id * pv.page_bytes + lhoff; };

    // this lane's row: column c of pair pw
    const int col = 32 * pw + c;
    const int qi = q_first + col / G;
    const bool live = qi < n_q;
    const int pos = q_start + min(qi, n_q - 1);
    const int64_t row = ((int64_t)min(qi, n_q - 1) * Hq + g * G + col % G) * splits + sp;
    constexpr float LOG2E = 1.4426950408889634f;
    const float cB = sm * LOG2E;
    float* wo = ws;
    float* wml = ws + (int64_t)n_q * Hq * splits * D;

    if (wave < WS_PAIRS) {
        // ================= score waves =================
        bf16x8 qop[QTERMS][KS16];
        float qsum;
        {
            const uint16_t* qrow = q + ((int64_t)min(qi, n_q - 1) * Hq + g * G + col % G) * QTERMS * D;
            float s = 0.f;
#pragma unroll
            for (int tm = 0; tm < QTERMS; ++tm)
#pragma unroll
                for (int ks = 0; ks < KS16; ++ks) {
                    // kappa 16 ks + 8 h + e: dims of kappa .. kappa + 7 are two runs of four
                    const int d0 = kappa_dim(16 * ks + 8 * h);
                    const uint2 a = *reinterpret_cast<const uint2*>(qrow + tm * D + d0);
                    const uint2 b = *reinterpret_cast<const uint2*>(qrow + tm * D + d0 + 8);
                    qop[tm][ks] = as_bf16x8(make_uint4(__builtin_amdgcn_perm(b.x, a.x, 0x05040100u),
                                                       __builtin_amdgcn_perm(b.x, a.x, 0x07060302u),
                                                       __builtin_amdgcn_perm(b.y, a.y, 0x05040100u),
                                                       __builtin_amdgcn_perm(b.y, a.y, 0x07060302u)));
                    s += bf16_to_f32((uint16_t)(a.x & 0xFFFF)) + bf16_to_f32((uint16_t)(a.x >> 16)) +
                         bf16_to_f32((uint16_t)(a.y & 0xFFFF)) + bf16_to_f32((uint16_t)(a.y >> 16)) +
                         bf16_to_f32((uint16_t)(b.x & 0xFFFF)) + bf16_to_f32((uint16_t)(b.x >> 16)) +
                         bf16_to_f32((uint16_t)(b.y & 0xFFFF)) + bf16_to_f32((uint16_t)(b.y >> 16));
                }
            qsum = s + __shfl_xor(s, 32);
        }
        float m_ref = -INFINITY, l_run = 0.f, c_run = 0.f, alpha = 1.f, cbm = 0.f;
        // pages below pg_full are visible to every row of the block (no mask)
        const int pg_full = max(pg0, min(pg1, (q_start + q_first + 1) / PAGE));
        // key of result register r of key block kb
        auto key_of = [&](int kb, int r) { return 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3); };

        // scores of page t from S^T (phase 1): logits with the dequantization folded
        // in, the page's maximum and the row reference
        auto score_step = [&](int t, f32x16 (&st)[2], auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const int pg = pg0 + t;
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float2 kk[4][4];  // K metadata of this lane's keys of block kb
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float4* src = reinterpret_cast<const float4*>(&L.kmeta[t & 1][32 * kb + 8 * m + 4 * h]);
                    const float4 x0 = src[0], x1 = src[1];
                    kk[m][0] = make_float2(x0.x, x0.y);
                    kk[m][1] = make_float2(x0.z, x0.w);
                    kk[m][2] = make_float2(x1.x, x1.y);
                    kk[m][3] = make_float2(x1.z, x1.w);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = fmaf(kk[r >> 2][r & 3].x, st[kb][r], kk[r >> 2][r & 3].y * qsum);
                    if (MASKED && pg * PAGE + key_of(kb, r) > pos) x = -INFINITY;
                    st[kb][r] = x;
                    mt = fmaxf(mt, x);
                }
            }
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
            const float m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            // lazy rescale: the reference moves only when a weight would pass 2^8
            const bool up = (m - m_ref) * cB > 8.0f;
            alpha = up ? __builtin_amdgcn_exp2f((m_ref - m) * cB) : 1.0f;
            m_ref = up ? m : m_ref;
            cbm = m_ref * cB;
        };
        // weights w = p scale_v of page t (phase 2), this page's sums, and the p.v
        // operands as two bf16 terms: step s of block kb = registers 8 s .. 8 s + 7
        auto weight_step = [&](int t, const f32x16 (&st)[2], auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const int pg = pg0 + t;
            float ls = 0.f, cs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float2 vv[4][4];  // V metadata of this lane's keys of block kb
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float4* src = reinterpret_cast<const float4*>(&L.vmeta[t & 1][32 * kb + 8 * m + 4 * h]);
                    const float4 x0 = src[0], x1 = src[1];
                    vv[m][0] = make_float2(x0.x, x0.y);
                    vv[m][1] = make_float2(x0.z, x0.w);
                    vv[m][2] = make_float2(x1.x, x1.y);
                    vv[m][3] = make_float2(x1.z, x1.w);
                }
                float w[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float2 v2 = vv[r >> 2][r & 3];
                    if (MASKED) {  // slots past a row's position (or past the sequence) weigh nothing
                        const bool valid = pg * PAGE + key_of(kb, r) <= pos;
                        const float p = valid ? __builtin_amdgcn_exp2f(fmaf(st[kb][r], cB, -cbm)) : 0.f;
                        ls += p;
                        cs += valid ? p * v2.y : 0.f;
                        w[r] = valid ? p * v2.x : 0.f;
                    } else {
                        const float p = __builtin_amdgcn_exp2f(fmaf(st[kb][r], cB, -cbm));
                        ls += p;
                        cs = fmaf(p, v2.y, cs);
                        w[r] = p * v2.x;
                    }
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    uint32_t hi[4], lo[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) split_hi_lo(w[8 * s2 + 2 * e], w[8 * s2 + 2 * e + 1], hi[e], lo[e]);
                    L.p[pw][2 * kb + s2][0][l] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                    L.p[pw][2 * kb + s2][1][l] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                }
            }
            l_run = fmaf(l_run, alpha, ls);
            c_run = fmaf(c_run, alpha, cs);
            if (h == 0) L.alpha[col] = alpha;
        };
        __syncthreads();  // page 0's K tile converted by the output waves
        for (int t = 0; t <= n; ++t) {
            f32x16 st[2];
            const bool masked = pg0 + t >= pg_full;
            if (t < n) {
                // ---- phase 1: S^T = K~ Q^T (key blocks kb of the page x the wave's 32 rows), then
                // the scores and the page maximum ----
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
                // one 16-dim step a step, both key blocks: A = K~ rows 32 kb + c, slots 8 h ..;
                // each read WS_AHEAD_S steps ahead of its products
                auto kfrag = [&](int ks, int kb) {
                    return as_bf16x8(*reinterpret_cast<const uint4*>(
                        &L.k[t & 1][(32 * kb + c) * KS + 16 * ks + 8 * h]));
                };
                constexpr int AS = WS_AHEAD_S<ROTQ>;
                bf16x8 fk[AS + 1][2];
#pragma unroll
                for (int ks = 0; ks < AS; ++ks) {
                    fk[ks][0] = kfrag(ks, 0);
                    fk[ks][1] = kfrag(ks, 1);
                }
#pragma unroll
                for (int ks = 0; ks < KS16; ++ks) {
                    // the fence keeps the reads ahead of their products (the scheduler would
                    // otherwise sink them next to their use and expose the LDS latency)
                    if (ks + AS < KS16) {
                        fk[(ks + AS) % (AS + 1)][0] = kfrag(ks + AS, 0);
                        fk[(ks + AS) % (AS + 1)][1] = kfrag(ks + AS, 1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int tm = 0; tm < QTERMS; ++tm)
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) st[kb] = mma32(fk[ks % (AS + 1)][kb], qop[tm][ks], st[kb]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (masked) score_step(t, st, std::true_type{});
                else score_step(t, st, std::false_type{});
            }
            __syncthreads();  // phase 1 done: the K tile is free, last page's weights are taken
            if (t < n) {
                // ---- phase 2: weights of page t ----
                if (masked) weight_step(t, st, std::true_type{});
                else weight_step(t, st, std::false_type{});
            }
            __syncthreads();
        }
        // ---- this split's (max, sum) per row; the offsets' sum goes to the output waves ----
        const float lt = l_run + __shfl_xor(l_run, 32);
        const float ct = c_run + __shfl_xor(c_run, 32);
        if (h == 0) {
            L.cfin[col] = ct;
            if (live) {
                wml[2 * row] = m_ref * cB;  // log2 units
                wml[2 * row + 1] = lt;
            }
        }
        __syncthreads();
    } else {
        // ================= output waves =================
        const int o = tid - 64 * WS_PAIRS;  // 0 .. WS_OT - 1
        WsStageK sk;
        uint4 sv = make_uint4(0, 0, 0, 0);
        ws_load_k<D>(sk, block_at(bt[pg0]), o);
        ws_store_k<D>(sk, L, 0, o);
        if (n > 1) ws_load_k<D>(sk, block_at(bt[pg0 + 1]), o);
        // page ids of the loads a step issues, read one step ahead (a load that first
        // waits for its block-table entry would stall the step)
        int id_k = n > 2 ? bt[pg0 + 2] : 0;  // page t + 2 (K), for step t = 0
        int id_v = bt[pg0];                  // page t (V), for step t = 0
        f32x16 acc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
        __syncthreads();  // page 0's K tile converted
        for (int t = 0; t <= n; ++t) {
            // ---- phase 1: weights of page t - 1 into registers, its V words into the V tile,
            // page t + 1 into the idle K tile (loaded a step ago) ----
            float a = 1.f;
            uint4 ph[4], pl[4];
            if (t >= 1) {
                a = L.alpha[col];
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    ph[s4] = L.p[pw][s4][0][l];
                    pl[s4] = L.p[pw][s4][1][l];
                }
                ws_store_v<D>(sv, L, o);
            }
            if (t + 1 < n) ws_store_k<D>(sk, L, (t + 1) & 1, o);
            __syncthreads();
            // ---- phase 2: O^T += V~ P^T for page t - 1; the codes of pages t (V) and t + 2 (K)
            // are loaded first, to land under the products ----
            if (t < n) ws_load_v<D>(sv, block_at(id_v), o);
            if (t + 2 < n) ws_load_k<D>(sk, block_at(id_k), o);
            if (t >= 1) {
                if (__builtin_amdgcn_ballot_w64(a != 1.0f)) {
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[db] *= a;
                }
                // steps of two 32-dim blocks (db = 2 dp, 2 dp + 1) and one 16-key step s4: A =
                // V~ rows 32 db + c at keys 32 (s4 / 2) + 16 (s4 % 2) + 4h + (0..3) and + 8 (slots
                // 8h .. 8h + 7, the order of the weights); two accumulators, each taking the
                // rounded weight and then its residual
                constexpr int NPV = 2 * DB;  // (dp, s4) steps: DB / 2 x 4
                auto vfrag = [&](int idx, int hh) {
                    const int db = 2 * (idx >> 2) + hh, s4 = idx & 3;
                    const uint16_t* vr = &L.v[(32 * db + c) * VS + 32 * (s4 >> 1) + 16 * (s4 & 1) + 4 * h];
                    const uint2 v0 = *reinterpret_cast<const uint2*>(vr);
                    const uint2 v1 = *reinterpret_cast<const uint2*>(vr + 8);
                    return as_bf16x8(make_uint4(v0.x, v0.y, v1.x, v1.y));
                };
                bf16x8 fv[WS_AHEAD_O + 1][2];
#pragma unroll
                for (int idx = 0; idx < WS_AHEAD_O; ++idx) {
                    fv[idx][0] = vfrag(idx, 0);
                    fv[idx][1] = vfrag(idx, 1);
                }
#pragma unroll
                for (int idx = 0; idx < NPV; ++idx) {
                    if (idx + WS_AHEAD_O < NPV) {
                        fv[(idx + WS_AHEAD_O) % (WS_AHEAD_O + 1)][0] = vfrag(idx + WS_AHEAD_O, 0);
                        fv[(idx + WS_AHEAD_O) % (WS_AHEAD_O + 1)][1] = vfrag(idx + WS_AHEAD_O, 1);
                    }
                    __builtin_amdgcn_sched_barrier(0);  // reads stay WS_AHEAD_O steps ahead
                    const int dp = idx >> 2, s4 = idx & 3;
                    const bf16x8 f0 = fv[idx % (WS_AHEAD_O + 1)][0], f1 = fv[idx % (WS_AHEAD_O + 1)][1];
                    acc[2 * dp] = mma32(f0, as_bf16x8(ph[s4]), acc[2 * dp]);
                    acc[2 * dp + 1] = mma32(f1, as_bf16x8(ph[s4]), acc[2 * dp + 1]);
                    acc[2 * dp] = mma32(f0, as_bf16x8(pl[s4]), acc[2 * dp]);
                    acc[2 * dp + 1] = mma32(f1, as_bf16x8(pl[s4]), acc[2 * dp + 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            id_k = t + 3 < n ? bt[pg0 + t + 3] : 0;
            id_v = t + 1 < n ? bt[pg0 + t + 1] : 0;
            __syncthreads();
        }
        __syncthreads();  // the score waves' row sums
        if (live) {
            const float ct = L.cfin[col];
            // result register r of block db: dim 32 db + 8 (r / 4) + 4 h + r % 4
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float4 v = make_float4(acc[db][4 * m] + ct, acc[db][4 * m + 1] + ct, acc[db][4 * m + 2] + ct,
                                                 acc[db][4 * m + 3] + ct);
                    *reinterpret_cast<float4*>(&wo[row * D + 32 * db + 8 * m + 4 * h]) = v;
                }
        }
    }
}

// rows a merge workgroup takes, one after another (tiny workgroups, one a row,
// were bound by their launch rate)
constexpr int PREFILL_MERGE_ROWS = 8;

// Merge of the prefill partials: PREFILL_MERGE_ROWS (query, head) rows a
// workgroup, thread d taking dim d of each; split p
// counts for query i when its first page starts at or before i's position and
// holds a page below kpl.  A window pool's window partials (win: outputs
// [n_q][Hq][D], then (max, sum) pairs; the window starts at key 64 kpl) count
// for the rows whose position reaches the window, the only rows written.
__global__ __launch_bounds__(256) void prefill_merge_kernel(int q_start, int n_q, int Hq, int Hkv, int D, int splits,
                                                            int kpl, int rows_per_block, const float* __restrict__ ws,
                                                            const float* __restrict__ win, float* __restrict__ out) {
    const int G = Hq / Hkv, d = threadIdx.x;
    const int QB = rows_per_block / G;
    const float2* mlb = reinterpret_cast<const float2*>(ws + (int64_t)n_q * Hq * splits * D);
#pragma unroll
    for (int rr = 0; rr < PREFILL_MERGE_ROWS; ++rr) {
        const int row = blockIdx.x * PREFILL_MERGE_ROWS + rr;  // i * Hq + h
        if (row >= n_q * Hq) break;
        const int i = row / Hq, qb = i / QB;
        const int pos = q_start + i;
        const int pos_max = q_start + min(qb * QB + QB, n_q) - 1;
        const int n_pages = min(pos_max / PAGE + 1, kpl);
        int live = 0;
        if (n_pages > 0) {
            const int per = (n_pages + splits - 1) / splits;
            live = min(min(splits, pos / (per * PAGE) + 1), (n_pages + per - 1) / per);
        }
        const float2* ml = mlb + (int64_t)row * splits;
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
}

static_assert(PREFILL_ROWS == 128 && WS_ROWS == 128, "prefill_rows_per_block() matches the kernels");

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
            hipLaunchKernelGGL(prefill_bf16_kernel<256>, grid, dim3(256), 0, s, pv, layer, seq, q_start, n_q, q, sm,
                               splits, kpl, ws);
        else
            hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, dim3(256), 0, s, pv, layer, seq, q_start, n_q, q, sm,
                               splits, kpl, ws);
    } else if (fmt == KV_FMT_Q2_ROT) {
        // the rotated query terms sit after the splits' partials
        uint16_t* qr = reinterpret_cast<uint16_t*>(ws + prefill_ws_floats(n_q, pv.Hq, pv.D, splits));
        const int qrows = n_q * pv.Hq;
        const float smr = sm / (float)pv.D;  // H q . H k = D q . k
        if (pv.D == 256) {
            hipLaunchKernelGGL(rotate_query_kernel<256>, dim3((qrows + 15) / 16), dim3(256), 0, s, q, qrows, qr);
            hipLaunchKernelGGL((prefill_ws_kernel<256, true>), grid, dim3(WS_NT), 0, s, pv, layer, seq, q_start, n_q,
                               qr, smr, splits, kpl, ws);
        } else {
            hipLaunchKernelGGL(rotate_query_kernel<128>, dim3((qrows + 15) / 16), dim3(256), 0, s, q, qrows, qr);
            hipLaunchKernelGGL((prefill_ws_kernel<128, true>), grid, dim3(WS_NT), 0, s, pv, layer, seq, q_start, n_q,
                               qr, smr, splits, kpl, ws);
        }
    } else if (kpl > 0) {
        if (pv.D == 256)
            hipLaunchKernelGGL((prefill_ws_kernel<256, false>), grid, dim3(WS_NT), 0, s, pv, layer, seq, q_start, n_q,
                               q, sm, splits, kpl, ws);
        else
            hipLaunchKernelGGL((prefill_ws_kernel<128, false>), grid, dim3(WS_NT), 0, s, pv, layer, seq, q_start, n_q,
                               q, sm, splits, kpl, ws);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    float* win = nullptr;
    if (window) {
        win = ws + prefill_ws_floats(n_q, pv.Hq, pv.D, splits);
        err = launch_prefill_window(pv, layer, seq, q_start, n_q, w0, q, sm, win, win + (int64_t)n_q * pv.Hq * pv.D, s);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(prefill_merge_kernel, dim3((n_q * pv.Hq + PREFILL_MERGE_ROWS - 1) / PREFILL_MERGE_ROWS),
                       dim3(pv.D), 0, s, q_start, n_q, pv.Hq, pv.Hkv, pv.D, splits, kpl, rows, ws, win, out);
    return hipGetLastError();
}

}  // namespace kvq
