// Attention over the exact window of a 2-bit window pool: the bf16 K and V
// rows of the last page a (sequence, layer) has appended to, kept beside the
// 2-bit pages (the most recent keys, which the compressed format of "The KV
// cache and prompt reuse", section "What a sequence is made of", holds
// unquantized).  A window block has the bf16
// page layout: K token-major (slot t at 2Dt), V dim-major (dim d at
// 128D + 128d).  Slots past the appended tokens hold stale rows, so every
// product with them is selected away, never multiplied by a zero weight.
//
// Decode: the 2-bit split kernel covers the tokens before the window; the
// kernel here computes the window's (max, sum, output) for one (sequence,
// query head) and merges it with the split partials in fp32, like
// the split merge kernels.  Prefill: a window partial per (query, head) row of the
// queries that see the window goes after the splits' partials in the
// workspace, and the prefill merge adds it to those rows.
// Scores and maxima are in base-2 units (s * log2 e), as in the split kernels.
#include "decode_common.h"

namespace kvq {

namespace {
constexpr float WIN_LOG2E = 1.4426950408889634f;
}

// The window's partial for one (query, head) row, computed by a workgroup of
// D threads (D / 64 waves); thread d owns dim d.  window_issue starts every
// global load that does not depend on the scores (the query into LDS, this
// dim's V row of the window into registers); the caller may issue more before
// window_reduce, in which wave w takes dims [64w, 64w + 64) of every window key
// (lane t: key t), wave 0 adds the D / 64 parts and forms the weights, and each
// thread sums its dim over the keys with four partial sums.  Returns the
// window's max M (base 2), sum of weights and this dim's output; M = -inf and
// both sums 0 when nw = 0.
template <int D>
struct WindowLds {
    float qs[D];
    float part[D / 64][PAGE];
    float pw[PAGE];
    float ml[2];
};

template <int D>
__device__ __forceinline__ void window_issue(WindowLds<D>& L, const uint8_t* blk, const uint16_t* qrow,
                                             uint4 (&vrow)[PAGE / 8]) {
    const int d = threadIdx.x;
    L.qs[d] = bf16_to_f32(qrow[d]);
    const uint4* vp = reinterpret_cast<const uint4*>(blk + 128 * (int64_t)D + 128 * (int64_t)d);
#pragma unroll
    for (int k = 0; k < PAGE / 8; ++k) vrow[k] = vp[k];
}

template <int D>
__device__ __forceinline__ void window_reduce(WindowLds<D>& L, const uint8_t* blk, const uint4 (&vrow)[PAGE / 8],
                                              int nw, float sm, float* __restrict__ srow, float& M, float& den,
                                              float& acc) {
    constexpr int NWAVE = D / 64;
    const int d = threadIdx.x, wave = d >> 6, lane = d & 63;
    __syncthreads();
    if (lane < nw) {
        const uint4* kp = reinterpret_cast<const uint4*>(blk + 2 * ((int64_t)D * lane + 64 * wave));
        float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint4 w = kp[k];
            const uint32_t uw[4] = {w.x, w.y, w.z, w.w};
            const float* qq = &L.qs[64 * wave + 8 * k];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = fmaf(qq[2 * i], bf16lo(uw[i]), a[i]);
                a[i] = fmaf(qq[2 * i + 1], bf16hi(uw[i]), a[i]);
            }
        }
        L.part[wave][lane] = (a[0] + a[1]) + (a[2] + a[3]);
    }
    __syncthreads();
    if (wave == 0) {
        float s = -INFINITY, p = 0.f;
        if (lane < nw) {
            float dot = 0.f;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) dot += L.part[w][lane];
            if (srow) srow[lane] = dot * sm;
            s = dot * (sm * WIN_LOG2E);
        }
        const float m = wave_max(s);
        if (lane < nw) p = exp2f(s - m);
        const float l = wave_sum(p);
        L.pw[lane] = p;
        if (lane == 0) {
            L.ml[0] = m;
            L.ml[1] = l;
        }
    }
    __syncthreads();
    M = L.ml[0];
    den = L.ml[1];
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < PAGE / 8; ++k) {
        const uint32_t uw[4] = {vrow[k].x, vrow[k].y, vrow[k].z, vrow[k].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = 8 * k + i;
            const float x = (i & 1) ? bf16hi(uw[i >> 1]) : bf16lo(uw[i >> 1]);
            // slots past the window hold stale rows: select, never multiply by a zero weight
            a[i & 3] = t < nw ? fmaf(L.pw[t], x, a[i & 3]) : a[i & 3];
        }
    }
    acc = (a[0] + a[1]) + (a[2] + a[3]);
}

// Decode: one workgroup per (sequence, query head): the window's partial,
// merged in fp32 with the split partials into the output.  Up to 8 splits:
// the split partials are loaded before the window's reduction and folded in
// one group.  More (WIDE): groups of 64 splits, lane t of each wave holding
// split p0 + t's (max, sum), reduced across the wave, and each thread folding
// its dim's 64 partial outputs with weights passed through the wave's row of
// LDS; the first group is loaded before the window's reduction.  Only slots
// below `splits` (inside the workspace) are loaded, and slots of splits that
// hold no page (never written in this call) are selected away.
template <int D, bool WIDE>
__global__ __launch_bounds__(256) void decode_window_merge_kernel(PoolView pv, int layer, BatchDesc bd,
                                                                  const uint16_t* __restrict__ q, float sm, int splits,
                                                                  const float* __restrict__ ws, float* __restrict__ out,
                                                                  float* __restrict__ scores, int64_t sstride) {
    constexpr int U = WIDE ? 64 : 8;
    const int row = blockIdx.x;  // e * Hq + h
    const int Hq = pv.Hq, e = row / Hq, h = row % Hq, g = h / (Hq / pv.Hkv);
    const int d = threadIdx.x;
    const int c = bd.pos[e], nw = bd.cnt[e];  // tokens from the pages, then window slots 0 .. nw-1
    const int live = live_splits(c, bd.per);
    const uint8_t* blk = window_block(pv, bd.seq[e], layer, g);

    __shared__ WindowLds<D> L;
    uint4 vrow[PAGE / 8];
    window_issue<D>(L, blk, q + (int64_t)row * D, vrow);
    const float2* ml = reinterpret_cast<const float2*>(ws + (int64_t)bd.n * Hq * splits * D) + (int64_t)row * splits;
    const float* o = ws + (int64_t)row * splits * D + d;
    float* srow = scores ? scores + (int64_t)row * sstride + c : nullptr;
    float M, den, acc;  // running (max, sum, output) in base-2 units, the window's first

    if constexpr (WIDE) {
        __shared__ __align__(16) float fs[D / 64][U];  // split weights, one row per wave
        const int lane = d & 63, wave = d >> 6;
        float2 mine;
        float v[U];
        auto load_group = [&](int p0) {
            const int n = splits - p0;  // slots of this group inside the workspace
            mine = lane < n ? ml[p0 + lane] : make_float2(-INFINITY, 0.f);
            const float* base = o + (int64_t)p0 * D;
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = u < n ? base[u * D] : 0.f;
        };
        load_group(0);
        window_reduce<D>(L, blk, vrow, nw, sm, srow, M, den, acc);
        for (int p0 = 0; p0 < live; p0 += U) {  // the same trip count for every thread
            if (p0 > 0) load_group(p0);
            const bool mine_live = p0 + lane < live;
            const float mx = mine_live ? mine.x : -INFINITY;
            const float Mg = fmaxf(M, wave_max(mx));
            const float r = exp2f(M - Mg);   // no window tokens (M = -inf): r = 0
            const float f = exp2f(mx - Mg);  // 0 past the live splits
            den = den * r + wave_sum(mine_live ? f * mine.y : 0.f);
            acc *= r;
            fs[wave][lane] = f;
            __syncthreads();
            const float4* f4 = reinterpret_cast<const float4*>(fs[wave]);
#pragma unroll
            for (int k = 0; k < U / 4; ++k) {
                const float4 w = f4[k];
                const float fw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int u = 4 * k + i;
                    acc = p0 + u < live ? fmaf(fw[i], v[u], acc) : acc;  // select: an unwritten slot may hold NaN
                }
            }
            __syncthreads();  // the next group rewrites fs
            M = Mg;
        }
    } else {
        // every slot below `splits` lies inside the workspace, so these loads do
        // not wait for the live split count; unwritten slots are selected away
        float2 m[U];
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = u < splits;
            m[u] = in ? ml[u] : make_float2(-INFINITY, 0.f);
            v[u] = in ? o[(int64_t)u * D] : 0.f;
        }
        window_reduce<D>(L, blk, vrow, nw, sm, srow, M, den, acc);
        if (live > 0) {
            float Mg = M;
#pragma unroll
            for (int u = 0; u < U; ++u) {  // select, never multiply, so that an unwritten slot cannot leak in
                m[u] = u < live ? m[u] : make_float2(-INFINITY, 0.f);
                v[u] = u < live ? v[u] : 0.f;
                Mg = fmaxf(Mg, m[u].x);
            }
            const float r = exp2f(M - Mg);  // no window tokens (M = -inf): r = 0
            den *= r;
            acc *= r;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float f = exp2f(m[u].x - Mg);
                den += f * m[u].y;
                acc += f * v[u];
            }
        }
    }
    out[(int64_t)row * D + d] = acc / den;
}

hipError_t launch_decode_window_merge(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q,
                                      float sm, int splits, const float* ws, float* out, float* scores,
                                      int64_t sstride, hipStream_t s) {
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(bd.n * pv.Hq), dim3(pv.D), 0, s, pv, layer, bd, q, sm, splits, ws, out,
                           scores, sstride);
    };
    if (pv.D == 256)
        splits > 8 ? go(decode_window_merge_kernel<256, true>) : go(decode_window_merge_kernel<256, false>);
    else
        splits > 8 ? go(decode_window_merge_kernel<128, true>) : go(decode_window_merge_kernel<128, false>);
    return hipGetLastError();
}

// Prefill: one workgroup per (query, head) row of the queries that see the
// window, i.e. the queries i >= i0 = w0 - q_start (at most 64 of them): row
// (i, h) sees window keys w0 .. q_start + i.  Its partial (max, sum, output)
// goes to the window area of the workspace; rows of earlier queries are
// neither written nor read.
template <int D>
__global__ __launch_bounds__(256) void prefill_window_kernel(PoolView pv, int layer, int seq, int q_start, int i0,
                                                             int w0, const uint16_t* __restrict__ q, float sm,
                                                             float* __restrict__ wo, float* __restrict__ wml) {
    const int Hq = pv.Hq, G = Hq / pv.Hkv;
    const int64_t row = (int64_t)i0 * Hq + blockIdx.x;  // i * Hq + h
    const int i = (int)(row / Hq), h = (int)(row % Hq);
    const int nw = q_start + i + 1 - w0;  // 1 .. 64
    const uint8_t* blk = window_block(pv, seq, layer, h / G);
    __shared__ WindowLds<D> L;
    uint4 vrow[PAGE / 8];
    window_issue<D>(L, blk, q + row * D, vrow);
    float M, den, acc;
    window_reduce<D>(L, blk, vrow, nw, sm, nullptr, M, den, acc);
    wo[row * D + threadIdx.x] = acc;
    if (threadIdx.x == 0) reinterpret_cast<float2*>(wml)[row] = make_float2(M, den);
}

hipError_t launch_prefill_window(const PoolView& pv, int layer, int seq, int q_start, int n_q, int w0,
                                 const uint16_t* q, float sm, float* wo, float* wml, hipStream_t s) {
    const int i0 = w0 > q_start ? w0 - q_start : 0;  // first query that sees the window
    if (i0 >= n_q) return hipSuccess;
    dim3 grid((n_q - i0) * pv.Hq);
    if (pv.D == 256)
        hipLaunchKernelGGL(prefill_window_kernel<256>, grid, dim3(256), 0, s, pv, layer, seq, q_start, i0, w0, q, sm,
                           wo, wml);
    else
        hipLaunchKernelGGL(prefill_window_kernel<128>, grid, dim3(128), 0, s, pv, layer, seq, q_start, i0, w0, q, sm,
                           wo, wml);
    return hipGetLastError();
}

}  // namespace kvq
