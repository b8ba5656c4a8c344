// Attention over the exact window of a 2-bit window pool: the bf16 K and V
// rows of the last page a (sequence, layer) has appended to, kept beside the
// 2-bit pages (the window of exact recent keys of "The KV cache and prompt
// reuse", section "What a sequence is made of").  A window block has the bf16
// page layout: K token-major (slot t at 2Dt), V dim-major (dim d at
// 128D + 128d).  Slots past the appended tokens hold stale rows, so every
// product with them is selected away, never multiplied by a zero weight.
//
// Decode: the 2-bit split kernel covers the tokens before the window; the
// kernel here computes the window's (max, sum, output) for one (sequence,
// query head) and merges it with the split partials in fp32, like
// merge_splits_kernel.  Prefill: a window partial per (query, head) row goes
// after the splits' partials in the workspace and the prefill merge adds it.
// Scores and maxima are in base-2 units (s * log2 e), as in the split kernels.
#include "decode_common.h"

namespace kvq {

namespace {
constexpr float WIN_LOG2E = 1.4426950408889634f;
}

// One workgroup of D threads (D / 64 waves) per (sequence, query head);
// thread d owns dim d.  Every global load that does not depend on the scores
// (the query, this dim's V row of the window, the first U split partials) is
// issued first; then wave w takes dims [64w, 64w + 64) of every window key
// (lane t: key t), wave 0 adds the D / 64 parts and forms the weights, and
// each thread sums its dim over the keys with four partial sums.
template <int D>
__global__ __launch_bounds__(256) void decode_window_merge_kernel(PoolView pv, int layer, BatchDesc bd,
                                                                  const uint16_t* __restrict__ q, float sm, int splits,
                                                                  const float* __restrict__ ws, float* __restrict__ out,
                                                                  float* __restrict__ scores, int64_t sstride) {
    constexpr int U = 8;
    constexpr int NWAVE = D / 64;
    const int row = blockIdx.x;  // e * Hq + h
    const int Hq = pv.Hq, e = row / Hq, h = row % Hq, g = h / (Hq / pv.Hkv);
    const int d = threadIdx.x, wave = d >> 6, lane = d & 63;
    const int c = bd.pos[e], nw = bd.cnt[e];  // tokens from the pages, then window slots 0 .. nw-1
    const int live = live_splits(c, bd.per);
    const uint8_t* blk = window_block(pv, bd.seq[e], layer, g);

    __shared__ float qs[D];
    __shared__ float part[NWAVE][PAGE];
    __shared__ float pw[PAGE];
    __shared__ float wml[2];

    qs[d] = bf16_to_f32(q[(int64_t)row * D + d]);
    uint4 vrow[PAGE / 8];
    {
        const uint4* vp = reinterpret_cast<const uint4*>(blk + 128 * (int64_t)D + 128 * (int64_t)d);
#pragma unroll
        for (int k = 0; k < PAGE / 8; ++k) vrow[k] = vp[k];
    }
    const float2* ml = reinterpret_cast<const float2*>(ws + (int64_t)bd.n * Hq * splits * D) + (int64_t)row * splits;
    const float* o = ws + (int64_t)row * splits * D + d;
    float2 m0[U];
    float v0[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool ok = u < live;
        m0[u] = ok ? ml[u] : make_float2(-INFINITY, 0.f);
        v0[u] = ok ? o[(int64_t)u * D] : 0.f;
    }
    __syncthreads();

    // ---- partial dot products: wave w, dims 64w .. 64w + 63, lane t = window slot t ----
    if (lane < nw) {
        const uint4* kp = reinterpret_cast<const uint4*>(blk + 2 * ((int64_t)D * lane + 64 * wave));
        float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint4 w = kp[k];
            const uint32_t uw[4] = {w.x, w.y, w.z, w.w};
            const float* qq = &qs[64 * wave + 8 * k];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = fmaf(qq[2 * i], bf16lo(uw[i]), a[i]);
                a[i] = fmaf(qq[2 * i + 1], bf16hi(uw[i]), a[i]);
            }
        }
        part[wave][lane] = (a[0] + a[1]) + (a[2] + a[3]);
    }
    __syncthreads();

    // ---- weights of the window keys (wave 0) ----
    if (wave == 0) {
        float s = -INFINITY, p = 0.f;
        if (lane < nw) {
            float dot = 0.f;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) dot += part[w][lane];
            if (scores) scores[(int64_t)row * sstride + c + lane] = dot * sm;
            s = dot * (sm * WIN_LOG2E);
        }
        const float M = wave_max(s);
        if (lane < nw) p = exp2f(s - M);
        const float l = wave_sum(p);
        pw[lane] = p;
        if (lane == 0) {
            wml[0] = M;
            wml[1] = l;
        }
    }
    __syncthreads();

    // ---- the window's partial for dim d: o_w = sum_t p_t v[d][t] ----
    float M = wml[0], den = wml[1];  // M = -inf and den = 0 when the window is empty
    float acc;
    {
        float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < PAGE / 8; ++k) {
            const uint32_t uw[4] = {vrow[k].x, vrow[k].y, vrow[k].z, vrow[k].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = 8 * k + i;
                const float x = (i & 1) ? bf16hi(uw[i >> 1]) : bf16lo(uw[i >> 1]);
                // slots past the window hold stale rows: select, never multiply by a zero weight
                a[i & 3] = t < nw ? fmaf(pw[t], x, a[i & 3]) : a[i & 3];
            }
        }
        acc = (a[0] + a[1]) + (a[2] + a[3]);
    }

    // ---- merge with the split partials (running max over groups of U splits) ----
    for (int p0 = 0; p0 < live; p0 += U) {
        float2 m[U];
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (p0 == 0) {
                m[u] = m0[u];
                v[u] = v0[u];
            } else {
                const bool ok = p0 + u < live;
                m[u] = ok ? ml[p0 + u] : make_float2(-INFINITY, 0.f);
                v[u] = ok ? o[(int64_t)(p0 + u) * D] : 0.f;
            }
        }
        float Mg = M;
#pragma unroll
        for (int u = 0; u < U; ++u) Mg = fmaxf(Mg, m[u].x);
        const float r = exp2f(M - Mg);  // M = -inf (no window tokens) on the first group: r = 0
        den *= r;
        acc *= r;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float f = exp2f(m[u].x - Mg);
            den += f * m[u].y;
            acc += f * v[u];
        }
        M = Mg;
    }
    out[(int64_t)row * D + d] = acc / den;
}

hipError_t launch_decode_window_merge(const PoolView& pv, int layer, const BatchDesc& bd, const uint16_t* q,
                                      float sm, int splits, const float* ws, float* out, float* scores,
                                      int64_t sstride, hipStream_t s) {
    if (pv.D == 256)
        hipLaunchKernelGGL(decode_window_merge_kernel<256>, dim3(bd.n * pv.Hq), dim3(256), 0, s, pv, layer, bd, q, sm,
                           splits, ws, out, scores, sstride);
    else
        hipLaunchKernelGGL(decode_window_merge_kernel<128>, dim3(bd.n * pv.Hq), dim3(128), 0, s, pv, layer, bd, q, sm,
                           splits, ws, out, scores, sstride);
    return hipGetLastError();
}

// Prefill: window partials of 64 (query, head) rows per workgroup (64 / G
// queries of KV head g).  The window block and the rows' queries are staged
// in LDS (K and V rows padded by one word, so that the 64 lanes reading 64
// different rows hit 64 different banks); each wave takes every fourth row:
// lane t scores window key t, then lane l accumulates dims l + 64k.  Row
// (query i, head h) sees window keys w0 .. q_start + i; rows that see none
// get an empty partial (max -inf, sum 0).
template <int D>
__global__ __launch_bounds__(256) void prefill_window_kernel(PoolView pv, int layer, int seq, int q_start, int n_q,
                                                             int w0, const uint16_t* __restrict__ q, float sm,
                                                             float* __restrict__ wo, float* __restrict__ wml) {
    constexpr int KW = D / 2 + 1;     // padded K row, words (two bf16 a word)
    constexpr int VW = PAGE / 2 + 1;  // padded V row, words
    constexpr int QW = D / 2;
    const int Hq = pv.Hq, G = Hq / pv.Hkv;
    const int QB = 64 / G;
    const int g = blockIdx.y, q_first = blockIdx.x * QB;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;

    __shared__ uint32_t Kl[PAGE * KW];
    __shared__ uint32_t Vl[D * VW];
    __shared__ __align__(16) uint32_t Ql[64 * QW];

    const uint8_t* blk = window_block(pv, seq, layer, g);
    for (int i = tid; i < PAGE * (D / 8); i += 256) {
        const int t = i / (D / 8), c = i % (D / 8);
        const uint4 w = *reinterpret_cast<const uint4*>(blk + 2 * ((int64_t)t * D + 8 * c));
        uint32_t* dst = &Kl[t * KW + 4 * c];
        dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
    }
    for (int i = tid; i < D * (PAGE / 8); i += 256) {
        const int dd = i / (PAGE / 8), c = i % (PAGE / 8);
        const uint4 w = *reinterpret_cast<const uint4*>(blk + 128 * (int64_t)D + 128 * (int64_t)dd + 16 * c);
        uint32_t* dst = &Vl[dd * VW + 4 * c];
        dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
    }
    for (int i = tid; i < 64 * (D / 8); i += 256) {
        const int r = i / (D / 8), c = i % (D / 8);
        const int qi = min(q_first + r / G, n_q - 1);
        const uint4 w = *reinterpret_cast<const uint4*>(q + ((int64_t)qi * Hq + g * G + r % G) * D + 8 * c);
        *reinterpret_cast<uint4*>(&Ql[r * QW + 4 * c]) = w;
    }
    __syncthreads();

    const float cB = sm * WIN_LOG2E;
    for (int r = wave; r < 64; r += 4) {
        const int qi = q_first + r / G;
        if (qi >= n_q) break;  // rows go in query order
        const int64_t orow = (int64_t)qi * Hq + g * G + r % G;
        const int nvis = q_start + qi + 1 - w0;  // window keys this row sees (at most 64)
        float o[D / 64];
#pragma unroll
        for (int k = 0; k < D / 64; ++k) o[k] = 0.f;
        float M = -INFINITY, lsum = 0.f;
        if (nvis > 0) {
            const uint32_t* kr = &Kl[l * KW];
            const uint32_t* qr = &Ql[r * QW];
            float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int i = 0; i < QW; ++i) {
                const uint32_t kk = kr[i], qq = qr[i];
                a[2 * (i & 1)] = fmaf(bf16lo(qq), bf16lo(kk), a[2 * (i & 1)]);
                a[2 * (i & 1) + 1] = fmaf(bf16hi(qq), bf16hi(kk), a[2 * (i & 1) + 1]);
            }
            const float dot = (a[0] + a[1]) + (a[2] + a[3]);
            const float s = l < nvis ? dot * cB : -INFINITY;
            M = wave_max(s);
            const float p = l < nvis ? exp2f(s - M) : 0.f;
            lsum = wave_sum(p);
            for (int t2 = 0; 2 * t2 < nvis; ++t2) {  // key pairs (2 t2, 2 t2 + 1)
                const float p0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 2 * t2));
                const float p1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 2 * t2 + 1));
                const bool two = 2 * t2 + 1 < nvis;
#pragma unroll
                for (int k = 0; k < D / 64; ++k) {
                    const uint32_t w = Vl[(l + 64 * k) * VW + t2];
                    const float a = fmaf(p0, bf16lo(w), o[k]);
                    o[k] = two ? fmaf(p1, bf16hi(w), a) : a;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < D / 64; ++k) wo[orow * D + l + 64 * k] = o[k];
        if (l == 0) {
            wml[2 * orow] = M;
            wml[2 * orow + 1] = lsum;
        }
    }
}

hipError_t launch_prefill_window(const PoolView& pv, int layer, int seq, int q_start, int n_q, int w0,
                                 const uint16_t* q, float sm, float* wo, float* wml, hipStream_t s) {
    const int QB = 64 / (pv.Hq / pv.Hkv);
    dim3 grid((n_q + QB - 1) / QB, pv.Hkv);
    if (pv.D == 256)
        hipLaunchKernelGGL(prefill_window_kernel<256>, grid, dim3(256), 0, s, pv, layer, seq, q_start, n_q, w0, q, sm,
                           wo, wml);
    else
        hipLaunchKernelGGL(prefill_window_kernel<128>, grid, dim3(256), 0, s, pv, layer, seq, q_start, n_q, w0, q, sm,
                           wo, wml);
    return hipGetLastError();
}

}  // namespace kvq
