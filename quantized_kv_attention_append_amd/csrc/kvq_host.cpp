// Host runtime of the paged, quantized KV cache: pool sizing, admission-time
// page reservation, block tables, argument checks and kernel launch planning.
//
// The pool is a byte budget of 64-token pages shared by every sequence, and a
// sequence reserves the pages of its whole bound when it is admitted, so an
// append inside the bound can never run out of pages ("KV at 9 KB a token",
// section "How it works"; "The KV cache and prompt reuse", section "What a
// sequence is made of").  Every check runs before anything is launched, so a
// refused call has copied or written nothing ("The KV cache and prompt reuse",
// section "When reuse misses"); nothing falls back to another path ("Half the
// Cache, Twice the Context", section "How to apply this", item 6).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"
#include "prefill.h"
#include "kvq_rt.h"

using namespace kvq;

namespace {

thread_local std::string g_last_error;

kv_status fail(kv_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = std::string(kv_status_str(s)) + ": " + buf;
    return s;
}

}  // namespace

namespace kvq {
kv_status set_error(kv_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace kvq

namespace {

kv_status hip_fail(hipError_t e, const char* what) {
    return fail(KV_ERR_DEVICE, "%s: %s", what, rt::error_string(e));
}

// Runs an entry point's body so that no C++ exception crosses the C ABI: a
// failed host allocation (page lists, block-table copies) becomes
// KV_ERR_DEVICE with a message, like a failed HIP call.
template <class F>
kv_status guarded(F&& body) {
    try {
        return body();
    } catch (const std::bad_alloc&) {
        return fail(KV_ERR_DEVICE, "host memory allocation failed");
    } catch (...) {
        return fail(KV_ERR_DEVICE, "unexpected host exception");
    }
}

kv_status check_geom(const kv_geom* g, kv_format fmt) {
    if (!g) return fail(KV_ERR_ARG, "geometry is NULL");
    if (fmt != KV_FMT_Q2 && fmt != KV_FMT_Q8 && fmt != KV_FMT_BF16 && fmt != KV_FMT_Q2_WINDOW && fmt != KV_FMT_Q2_ROT)
        return fail(KV_ERR_FORMAT, "unknown format %d", (int)fmt);
    if (g->n_layers <= 0 || g->n_kv_heads <= 0 || g->n_q_heads <= 0 || g->head_dim <= 0)
        return fail(KV_ERR_ARG, "geometry fields must be positive");
    if (g->n_layers > KV_MAX_LAYERS || g->n_kv_heads > KV_MAX_KV_HEADS)
        return fail(KV_ERR_UNSUPPORTED, "n_layers %d / n_kv_heads %d above %d / %d", g->n_layers, g->n_kv_heads,
                    KV_MAX_LAYERS, KV_MAX_KV_HEADS);
    if (g->head_dim != 128 && g->head_dim != 256)
        return fail(KV_ERR_UNSUPPORTED, "head_dim %d (supported: 128, 256)", g->head_dim);
    if (g->n_q_heads % g->n_kv_heads != 0)
        return fail(KV_ERR_UNSUPPORTED, "n_q_heads %d is not a multiple of n_kv_heads %d", g->n_q_heads,
                    g->n_kv_heads);
    int G = g->n_q_heads / g->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return fail(KV_ERR_UNSUPPORTED, "GQA group %d (supported: 1, 2, 4, 8)", G);
    return KV_OK;
}

// The pages of window and rotated pools are 2-bit pages.
kv_format page_format(kv_format fmt) { return fmt == KV_FMT_Q2_WINDOW || fmt == KV_FMT_Q2_ROT ? KV_FMT_Q2 : fmt; }
int64_t block_bytes_of(kv_format fmt, int D) {
    fmt = page_format(fmt);
    return fmt == KV_FMT_Q2 ? q2_block_bytes(D) : fmt == KV_FMT_Q8 ? q8_block_bytes(D) : bf16_block_bytes(D);
}
const char* fmt_name(kv_format fmt) {
    return fmt == KV_FMT_Q2 ? "q2" : fmt == KV_FMT_Q8 ? "q8" : fmt == KV_FMT_BF16 ? "bf16"
         : fmt == KV_FMT_Q2_WINDOW ? "q2-window" : "q2-rotated";
}
// Formats whose appends are sequential per (sequence, layer): the exact rows
// of the open page are kept only for the tokens appended so far.
bool sequential_appends(kv_format fmt) { return fmt == KV_FMT_Q8 || fmt == KV_FMT_Q2_WINDOW; }

int64_t token_bytes_of(const kv_geom* g, kv_format fmt) {
    return (int64_t)g->n_layers * g->n_kv_heads * block_bytes_of(fmt, g->head_dim) / PAGE;
}

}  // namespace

struct kv_pool {
    kv_geom geom;
    kv_format fmt;
    int64_t n_pages = 0;
    int64_t page_bytes = 0, token_bytes = 0, block_bytes = 0;
    uint8_t* d_pages = nullptr;
    bool own_pages = false;
    int32_t max_seqs = 0;
    int32_t bt_stride = 0;       // max pages per sequence
    int32_t* d_bt = nullptr;     // [max_seqs][bt_stride]
    uint16_t* d_stage = nullptr; // 8-bit exact-K window
    uint8_t* d_win = nullptr;    // 2-bit window pools: exact rows of the last page, per (seq, layer, head)
    int32_t* d_cnt = nullptr;    // split arrival counters of the fused decode merge, zero between calls
    int device = 0;
    // host metadata
    std::vector<int32_t> refs;       // page -> sequences holding it (0: free)
    // Free pages on a stack.  A page reserved by explicit id stays on the
    // stack (skipped when popped, since refs > 0); in_stack marks the pages
    // with an entry, so a page is never on the stack twice, a pop loop can
    // never take one page twice, and the stack never outgrows its n_pages
    // capacity (so a push never allocates).
    std::vector<int32_t> free_stack;
    std::vector<char> in_stack;
    int64_t free_count = 0;
    struct Seq {
        bool live = false;
        int64_t bound = 0;     // reserved tokens
        int64_t appended = 0;  // highest position appended + 1, over all layers
        std::vector<int64_t> layer_appended;  // 8-bit and window pools: tokens appended per layer (sequential)
        std::vector<int32_t> pages;
    };
    std::vector<Seq> seqs;

    PoolView view() const {
        PoolView v;
        v.pages = d_pages;
        v.page_bytes = page_bytes;
        v.block_bytes = block_bytes;
        v.L = geom.n_layers;
        v.Hkv = geom.n_kv_heads;
        v.D = geom.head_dim;
        v.Hq = geom.n_q_heads;
        v.bt = d_bt;
        v.bt_stride = bt_stride;
        v.stage = d_stage;
        v.win = d_win;
        v.cnt = d_cnt;
        return v;
    }
};

namespace {
// Puts a page that has just become free back on the stack, unless its old
// entry is still there.
void push_free(kv_pool* p, int32_t pg) {
    if (!p->in_stack[(size_t)pg]) {
        p->free_stack.push_back(pg);
        p->in_stack[(size_t)pg] = 1;
    }
}
}  // namespace

namespace kvq {
int pool_device(const kv_pool* p) { return p ? p->device : -1; }
}  // namespace kvq

extern "C" {

const char* kv_status_str(kv_status s) {
    switch (s) {
        case KV_OK: return "KV_OK";
        case KV_ERR_ARG: return "KV_ERR_ARG";
        case KV_ERR_NO_SPACE: return "KV_ERR_NO_SPACE";
        case KV_ERR_BOUND: return "KV_ERR_BOUND";
        case KV_ERR_FORMAT: return "KV_ERR_FORMAT";
        case KV_ERR_UNSUPPORTED: return "KV_ERR_UNSUPPORTED";
        case KV_ERR_WORKSPACE: return "KV_ERR_WORKSPACE";
        case KV_ERR_DEVICE: return "KV_ERR_DEVICE";
    }
    return "KV_ERR_UNKNOWN";
}

const char* kv_last_error(void) { return g_last_error.c_str(); }

kv_status kv_token_bytes(const kv_geom* geom, kv_format fmt, int64_t* token_bytes, int64_t* page_bytes) {
    return guarded([&]() -> kv_status {
        kv_status s = check_geom(geom, fmt);
        if (s != KV_OK) return s;
        if (!token_bytes || !page_bytes) return fail(KV_ERR_ARG, "output pointer is NULL");
        *token_bytes = token_bytes_of(geom, fmt);
        *page_bytes = *token_bytes * PAGE;
        return KV_OK;
    });
}

kv_status kv_pool_bytes_for_tokens(const kv_geom* geom, kv_format fmt, int64_t tokens, int64_t* bytes) {
    return guarded([&]() -> kv_status {
        kv_status s = check_geom(geom, fmt);
        if (s != KV_OK) return s;
        if (!bytes) return fail(KV_ERR_ARG, "output pointer is NULL");
        if (tokens < 0) return fail(KV_ERR_ARG, "negative token count");
        const int64_t pages = tokens / PAGE + (tokens % PAGE != 0), pb = token_bytes_of(geom, fmt) * PAGE;
        if (pages > INT64_MAX / pb) return fail(KV_ERR_ARG, "%lld tokens overflow a byte count", (long long)tokens);
        *bytes = pages * pb;
        return KV_OK;
    });
}

kv_status kv_pool_create(int64_t bytes, const kv_geom* geom, kv_format fmt, int32_t max_seqs, int64_t max_seq_tokens,
                         void* d_mem, kv_pool** out) {
    return guarded([&]() -> kv_status {
        kv_status s = check_geom(geom, fmt);
        if (s != KV_OK) return s;
        if (!out) return fail(KV_ERR_ARG, "out is NULL");
        if (bytes < 0 || max_seqs <= 0 || max_seq_tokens <= 0)
            return fail(KV_ERR_ARG, "bytes, max_seqs and max_seq_tokens must be positive");
        if (max_seq_tokens >= (int64_t)1 << 31) return fail(KV_ERR_UNSUPPORTED, "max_seq_tokens must be < 2^31");
        int64_t tb = token_bytes_of(geom, fmt), pb = tb * PAGE;
        int64_t n_pages = bytes / pb;
        if (n_pages <= 0) return fail(KV_ERR_NO_SPACE, "budget of %lld B is below one page (%lld B)", (long long)bytes, (long long)pb);
        if (n_pages >= ((int64_t)1 << 31)) return fail(KV_ERR_UNSUPPORTED, "more than 2^31 pages");

        kv_pool* p = new kv_pool();
        p->geom = *geom;
        p->fmt = fmt;
        p->n_pages = n_pages;
        p->page_bytes = pb;
        p->token_bytes = tb;
        p->block_bytes = block_bytes_of(fmt, geom->head_dim);
        p->max_seqs = max_seqs;
        p->bt_stride = (int32_t)((max_seq_tokens + PAGE - 1) / PAGE);
        hipError_t e = rt::current_device(&p->device);
        if (e != hipSuccess) {
            delete p;
            return hip_fail(e, "hipGetDevice");
        }
        if (d_mem) {
            p->d_pages = (uint8_t*)d_mem;
        } else {
            e = rt::alloc((void**)&p->d_pages, (size_t)(n_pages * pb));
            if (e != hipSuccess) {
                delete p;
                return hip_fail(e, "pool page allocation");
            }
            p->own_pages = true;
        }
        e = rt::alloc((void**)&p->d_bt, (size_t)max_seqs * p->bt_stride * sizeof(int32_t));
        if (e == hipSuccess) e = rt::zero(p->d_bt, (size_t)max_seqs * p->bt_stride * sizeof(int32_t));
        if (e == hipSuccess && fmt == KV_FMT_Q8) {
            size_t sb = (size_t)max_seqs * geom->n_layers * geom->n_kv_heads * PAGE * geom->head_dim * sizeof(uint16_t);
            e = rt::alloc((void**)&p->d_stage, sb);
        }
        if (e == hipSuccess && fmt == KV_FMT_Q2_WINDOW) {
            size_t wb = (size_t)max_seqs * geom->n_layers * geom->n_kv_heads * 256 * (size_t)geom->head_dim;
            e = rt::alloc((void**)&p->d_win, wb);
        }
        if (e == hipSuccess) {
            // one counter per (batch entry, KV head, launch of four query heads); each
            // fused decode launch returns every counter it used to zero
            const size_t cb = decode_counters(geom->n_kv_heads) * sizeof(int32_t);
            e = rt::alloc((void**)&p->d_cnt, cb);
            if (e == hipSuccess) e = rt::zero(p->d_cnt, cb);
        }
        if (e != hipSuccess) {
            kv_status r = hip_fail(e, "block table / window / counter allocation");
            kv_pool_destroy(p);
            return r;
        }
        try {
            p->refs.assign((size_t)n_pages, 0);
            p->free_stack.resize((size_t)n_pages);
            p->in_stack.assign((size_t)n_pages, 1);
            p->seqs.resize((size_t)max_seqs);
        } catch (const std::bad_alloc&) {
            kv_pool_destroy(p);
            return fail(KV_ERR_DEVICE, "host memory allocation failed (page lists of %lld pages)", (long long)n_pages);
        }
        for (int64_t i = 0; i < n_pages; ++i) p->free_stack[(size_t)i] = (int32_t)(n_pages - 1 - i);
        p->free_count = n_pages;
        fprintf(stderr, "kvq: pool %s kv_pool_pages=%lld kv_pool_tokens=%lld kv_page_bytes=%lld token_bytes=%lld\n",
                fmt_name(fmt), (long long)n_pages, (long long)(n_pages * PAGE), (long long)pb,
                (long long)tb);
        *out = p;
        return KV_OK;
    });
}

kv_status kv_pool_destroy(kv_pool* p) {
    return guarded([&]() -> kv_status {
        if (!p) return fail(KV_ERR_ARG, "pool is NULL");
        if (p->own_pages && p->d_pages) (void)rt::release(p->d_pages);
        if (p->d_bt) (void)rt::release(p->d_bt);
        if (p->d_stage) (void)rt::release(p->d_stage);
        if (p->d_win) (void)rt::release(p->d_win);
        if (p->d_cnt) (void)rt::release(p->d_cnt);
        delete p;
        return KV_OK;
    });
}

kv_status kv_pool_stats(const kv_pool* p, kv_pool_stats_t* o) {
    return guarded([&]() -> kv_status {
        if (!p || !o) return fail(KV_ERR_ARG, "NULL argument");
        int64_t used = 0, n = 0;
        std::vector<char> seen((size_t)p->n_pages, 0);  // a shared page counts once
        for (const auto& s : p->seqs) {
            if (!s.live) continue;
            ++n;
            const int64_t held = (s.appended + PAGE - 1) / PAGE;
            for (int64_t i = 0; i < held && i < (int64_t)s.pages.size(); ++i)
                if (!seen[(size_t)s.pages[(size_t)i]]++) ++used;
        }
        o->pages = p->n_pages;
        o->free_pages = p->free_count;
        o->reserved_pages = p->n_pages - p->free_count;
        o->used_pages = used;
        o->page_bytes = p->page_bytes;
        o->token_bytes = p->token_bytes;
        o->tokens = p->n_pages * PAGE;
        o->n_seqs = n;
        return KV_OK;
    });
}

kv_status kv_pool_device_ptr(const kv_pool* p, void** d_pages, int64_t* bytes) {
    return guarded([&]() -> kv_status {
        if (!p || !d_pages || !bytes) return fail(KV_ERR_ARG, "NULL argument");
        *d_pages = p->d_pages;
        *bytes = p->n_pages * p->page_bytes;
        return KV_OK;
    });
}

kv_status kv_seq_reserve(kv_pool* p, int64_t max_tokens, const int32_t* pages, int32_t* seq) {
    return guarded([&]() -> kv_status {
        if (!p || !seq) return fail(KV_ERR_ARG, "NULL argument");
        if (max_tokens <= 0) return fail(KV_ERR_ARG, "max_tokens must be positive");
        int64_t need = (max_tokens + PAGE - 1) / PAGE;
        if (need > p->bt_stride)
            return fail(KV_ERR_BOUND, "bound of %lld tokens exceeds the pool's max_seq_tokens (%d pages)", (long long)max_tokens,
                        p->bt_stride);
        int32_t slot = -1;
        for (int32_t i = 0; i < p->max_seqs; ++i)
            if (!p->seqs[(size_t)i].live) {
                slot = i;
                break;
            }
        if (slot < 0) return fail(KV_ERR_NO_SPACE, "all %d sequence slots are live", p->max_seqs);
        if (need > p->free_count)
            return fail(KV_ERR_NO_SPACE, "need %lld pages, %lld free", (long long)need, (long long)p->free_count);
        std::vector<int32_t> got;
        got.reserve((size_t)need);
        std::vector<int64_t> layer_appended(sequential_appends(p->fmt) ? (size_t)p->geom.n_layers : 0, 0);
        if (pages) {
            std::vector<int32_t> sorted(pages, pages + need);
            std::sort(sorted.begin(), sorted.end());
            for (int64_t i = 0; i < need; ++i) {
                int32_t pg = sorted[(size_t)i];
                if (pg < 0 || pg >= p->n_pages) return fail(KV_ERR_ARG, "page id %d out of range", pg);
                if (i > 0 && sorted[(size_t)i - 1] == pg) return fail(KV_ERR_ARG, "page id %d listed twice", pg);
                if (p->refs[(size_t)pg] != 0) return fail(KV_ERR_NO_SPACE, "page %d is already reserved", pg);
            }
            got.assign(pages, pages + need);
        } else {
            while ((int64_t)got.size() < need) {
                int32_t pg = p->free_stack.back();
                p->free_stack.pop_back();
                p->in_stack[(size_t)pg] = 0;
                if (p->refs[(size_t)pg] == 0) got.push_back(pg);
            }
        }
        hipError_t e = rt::upload(p->d_bt + (size_t)slot * p->bt_stride, got.data(), got.size() * sizeof(int32_t));
        if (e != hipSuccess) {
            if (!pages)
                for (int32_t pg : got) push_free(p, pg);
            return hip_fail(e, "block table upload");
        }
        for (int32_t pg : got) p->refs[(size_t)pg] = 1;
        p->free_count -= need;
        auto& s = p->seqs[(size_t)slot];
        s.live = true;
        s.bound = max_tokens;
        s.appended = 0;
        s.layer_appended = std::move(layer_appended);
        s.pages = std::move(got);
        *seq = slot;
        return KV_OK;
    });
}

kv_status kv_seq_fork(kv_pool* p, int32_t parent, int64_t n, int64_t max_tokens, kv_stream_t stream, int32_t* child) {
    return guarded([&]() -> kv_status {
        if (!p || !child) return fail(KV_ERR_ARG, "NULL argument");
        if (parent < 0 || parent >= p->max_seqs || !p->seqs[(size_t)parent].live)
            return fail(KV_ERR_ARG, "fork: sequence %d is not live", parent);
        const auto& ps = p->seqs[(size_t)parent];
        if (n < 1 || n > max_tokens) return fail(KV_ERR_ARG, "fork: need 1 <= n_tokens (%lld) <= max_tokens (%lld)",
                                                 (long long)n, (long long)max_tokens);
        const int64_t need_total = (max_tokens + PAGE - 1) / PAGE;
        if (need_total > p->bt_stride)
            return fail(KV_ERR_BOUND, "fork: bound of %lld tokens exceeds the pool's max_seq_tokens (%d pages)",
                        (long long)max_tokens, p->bt_stride);
        if (n > ps.appended)
            return fail(KV_ERR_ARG, "fork: n_tokens %lld beyond the %lld tokens appended to sequence %d", (long long)n,
                        (long long)ps.appended, parent);
        for (int layer = 0; layer < (int)ps.layer_appended.size(); ++layer) {
            const int64_t A = ps.layer_appended[(size_t)layer];
            if (p->fmt == KV_FMT_Q8 && A != n)
                return fail(KV_ERR_ARG, "fork: an 8-bit fork takes all %lld tokens of layer %d, not %lld", (long long)A,
                            layer, (long long)n);
            if (p->fmt == KV_FMT_Q2_WINDOW && (n > A || (n - 1) / PAGE != (A - 1) / PAGE))
                return fail(KV_ERR_ARG, "fork: a window fork ends in the last page of layer %d (%lld tokens appended)",
                            layer, (long long)A);
        }
        const int64_t full = n / PAGE;            // pages shared
        const bool copy = n % PAGE != 0;          // the partly filled page is copied
        const int64_t fresh = need_total - full;  // pages the child takes
        int32_t slot = -1;
        for (int32_t i = 0; i < p->max_seqs; ++i)
            if (!p->seqs[(size_t)i].live) {
                slot = i;
                break;
            }
        if (slot < 0) return fail(KV_ERR_NO_SPACE, "all %d sequence slots are live", p->max_seqs);
        if (fresh > p->free_count)
            return fail(KV_ERR_NO_SPACE, "fork needs %lld pages, %lld free", (long long)fresh, (long long)p->free_count);
        // every host allocation happens before the free stack is touched
        std::vector<int32_t> pages;
        pages.reserve((size_t)need_total);
        pages.assign(ps.pages.begin(), ps.pages.begin() + full);
        std::vector<int32_t> got;
        got.reserve((size_t)fresh);
        std::vector<int64_t> layer_appended(ps.layer_appended.size(), n);
        while ((int64_t)got.size() < fresh) {
            const int32_t pg = p->free_stack.back();
            p->free_stack.pop_back();
            p->in_stack[(size_t)pg] = 0;
            if (p->refs[(size_t)pg] == 0) got.push_back(pg);
        }
        pages.insert(pages.end(), got.begin(), got.end());
        hipError_t e = rt::upload(p->d_bt + (size_t)slot * p->bt_stride, pages.data(), pages.size() * sizeof(int32_t));
        CopyRange r[3];
        int nr = 0;
        if (copy)
            r[nr++] = {p->d_pages + (int64_t)ps.pages[(size_t)full] * p->page_bytes,
                       p->d_pages + (int64_t)got[0] * p->page_bytes, p->page_bytes};
        const int64_t per_seq_blocks = (int64_t)p->geom.n_layers * p->geom.n_kv_heads;
        if (p->fmt == KV_FMT_Q8 && copy) {
            const int64_t b = per_seq_blocks * PAGE * p->geom.head_dim * (int64_t)sizeof(uint16_t);
            r[nr++] = {(uint8_t*)p->d_stage + parent * b, (uint8_t*)p->d_stage + slot * b, b};
        }
        if (p->fmt == KV_FMT_Q2_WINDOW) {
            const int64_t b = per_seq_blocks * 256 * (int64_t)p->geom.head_dim;
            r[nr++] = {p->d_win + parent * b, p->d_win + slot * b, b};
        }
        if (e == hipSuccess && nr > 0) e = launch_copy_ranges(r, nr, (hipStream_t)stream);
        if (e != hipSuccess) {
            for (int32_t pg : got) push_free(p, pg);
            return hip_fail(e, "fork");
        }
        for (int64_t i = 0; i < full; ++i) ++p->refs[(size_t)pages[(size_t)i]];
        for (int32_t pg : got) p->refs[(size_t)pg] = 1;
        p->free_count -= fresh;
        auto& cs = p->seqs[(size_t)slot];
        cs.live = true;
        cs.bound = max_tokens;
        cs.appended = n;
        cs.layer_appended = std::move(layer_appended);
        cs.pages = std::move(pages);
        *child = slot;
        return KV_OK;
    });
}

kv_status kv_seq_release(kv_pool* p, int32_t seq) {
    return guarded([&]() -> kv_status {
        if (!p) return fail(KV_ERR_ARG, "pool is NULL");
        if (seq < 0 || seq >= p->max_seqs || !p->seqs[(size_t)seq].live) return fail(KV_ERR_ARG, "sequence %d is not live", seq);
        auto& s = p->seqs[(size_t)seq];
        for (int32_t pg : s.pages)
            if (--p->refs[(size_t)pg] == 0) {
                push_free(p, pg);
                ++p->free_count;
            }
        s = kv_pool::Seq();
        return KV_OK;
    });
}

kv_status kv_seq_block_table(const kv_pool* p, int32_t seq, const int32_t** d_bt, int32_t* n_pages) {
    return guarded([&]() -> kv_status {
        if (!p || !d_bt || !n_pages) return fail(KV_ERR_ARG, "NULL argument");
        if (seq < 0 || seq >= p->max_seqs || !p->seqs[(size_t)seq].live) return fail(KV_ERR_ARG, "sequence %d is not live", seq);
        *d_bt = p->d_bt + (size_t)seq * p->bt_stride;
        *n_pages = (int32_t)p->seqs[(size_t)seq].pages.size();
        return KV_OK;
    });
}

kv_status kv_seq_pages(const kv_pool* p, int32_t seq, int32_t* pages, int32_t cap, int32_t* n_pages) {
    return guarded([&]() -> kv_status {
        if (!p || !n_pages) return fail(KV_ERR_ARG, "NULL argument");
        if (seq < 0 || seq >= p->max_seqs || !p->seqs[(size_t)seq].live) return fail(KV_ERR_ARG, "sequence %d is not live", seq);
        const auto& s = p->seqs[(size_t)seq];
        *n_pages = (int32_t)s.pages.size();
        if (pages)
            for (int32_t i = 0; i < cap && i < *n_pages; ++i) pages[i] = s.pages[(size_t)i];
        return KV_OK;
    });
}

}  // extern "C"

namespace {

kv_status check_seq(const kv_pool* p, int32_t seq, int64_t end_pos, const char* what) {
    if (seq < 0 || seq >= p->max_seqs || !p->seqs[(size_t)seq].live)
        return fail(KV_ERR_ARG, "%s: sequence %d is not live", what, seq);
    if (end_pos > p->seqs[(size_t)seq].bound)
        return fail(KV_ERR_BOUND, "%s: position %lld beyond sequence %d's bound of %lld tokens", what,
                    (long long)end_pos, seq, (long long)p->seqs[(size_t)seq].bound);
    return KV_OK;
}

// Default split count for a decode batch.  2-bit and bf16: about one workgroup per
// compute unit (256 on MI355X) over all (sequence, KV head) pairs, with at
// least eight page pairs per split (two per wavefront of a workgroup); the
// 2-bit formats run group 8 as two workgroups a split.  8-bit:
// its decode holds two workgroups on each compute unit (at 128 dims and group
// up to 4, four waves a workgroup, each with one page slot of LDS; at 256 dims
// two of four) or one (at 128 dims and group 8, eight waves), and a workgroup
// whose split holds no page ends at once; the split count is the largest
// whose workgroups with pages all fit in those slots (512 or 256) together,
// going no further once a split is down to one page pair (measured on 24
// lanes of 16..124 pages, us a layer call: group 4, 8 KV heads: 3 splits 51.5
// with 376 such workgroups, 4 46.6 with 472, 5 51.9 with 568, 6 51.6, 8 49.3;
// group 8, 4 KV heads: 2 splits 45.5, 3 36.7, 4 36.9 with 236, 6 44.7, 8 42.7,
// 10 49.1 with 492).
int auto_splits(const kv_pool* p, int n, const int64_t* ctx) {
    int64_t max_pages = 1;
    for (int i = 0; i < n; ++i) max_pages = std::max<int64_t>(max_pages, (ctx[i] + PAGE - 1) / PAGE);
    const int G = p->geom.n_q_heads / p->geom.n_kv_heads;
    // the 2-bit decode runs group 8 as two workgroups a split
    const bool pair = (p->fmt == KV_FMT_Q2 || p->fmt == KV_FMT_Q2_ROT || p->fmt == KV_FMT_Q2_WINDOW) && G == 8;
    const int64_t base = (int64_t)n * p->geom.n_kv_heads * (pair ? 2 : 1);
    const int64_t want = (256 + base - 1) / base;
    if (p->fmt == KV_FMT_Q8) {
        const int64_t SLOTS = (p->geom.head_dim == 128 && G == 8 ? 1 : 2) * 256;
        const int64_t max_pairs = (max_pages + 1) / 2;
        int best = 1;
        for (int s = 1; s <= 256; ++s) {
            const int64_t per = (max_pairs + s - 1) / s;
            int64_t live = 0;  // workgroups with pages
            for (int i = 0; i < n; ++i) {
                const int64_t pairs = ((ctx[i] + PAGE - 1) / PAGE + 1) / 2;
                live += (pairs + per - 1) / per;
            }
            if (s > 1 && live * p->geom.n_kv_heads > SLOTS) break;
            best = s;
            if (per == 1) break;
        }
        return best;
    }
    const int64_t cap = std::max<int64_t>(1, ((max_pages + 1) / 2) / 8);
    return (int)std::max<int64_t>(1, std::min<int64_t>({want, cap, 256}));
}

}  // namespace

extern "C" {

kv_status kv_append_quant(kv_pool* p, int32_t layer, int32_t n, const int32_t* seqs, const int64_t* start_pos,
                          const int32_t* n_new, const uint16_t* d_k, const uint16_t* d_v, kv_stream_t stream) {
    return guarded([&]() -> kv_status {
        if (!p) return fail(KV_ERR_ARG, "pool is NULL");
        if (n < 0) return fail(KV_ERR_ARG, "negative batch size");
        if (n == 0) return KV_OK;
        if (n > KV_MAX_BATCH) return fail(KV_ERR_UNSUPPORTED, "batch of %d exceeds KV_MAX_BATCH (%d)", n, KV_MAX_BATCH);
        if (!seqs || !start_pos || !n_new) return fail(KV_ERR_ARG, "NULL argument");
        if (layer < 0 || layer >= p->geom.n_layers) return fail(KV_ERR_ARG, "layer %d out of range", layer);
        BatchDesc bd;
        memset(&bd, 0, sizeof bd);
        bd.n = n;
        int64_t rows = 0, work = 0;
        for (int i = 0; i < n; ++i) {
            if (n_new[i] < 0 || start_pos[i] < 0) return fail(KV_ERR_ARG, "entry %d: negative position or count", i);
            if (start_pos[i] > INT32_MAX)
                return fail(KV_ERR_BOUND, "entry %d: position %lld is not below 2^31", i, (long long)start_pos[i]);
            kv_status s = check_seq(p, seqs[i], start_pos[i] + n_new[i], "append");
            if (s != KV_OK) return s;
            if (sequential_appends(p->fmt) && start_pos[i] != p->seqs[(size_t)seqs[i]].layer_appended[(size_t)layer])
                return fail(KV_ERR_ARG,
                            "entry %d: %s appends are sequential per layer (sequence %d layer %d holds %lld tokens, "
                            "append starts at %lld)",
                            i, fmt_name(p->fmt), seqs[i], layer,
                            (long long)p->seqs[(size_t)seqs[i]].layer_appended[(size_t)layer],
                            (long long)start_pos[i]);
            for (int j = 0; j < i; ++j)
                if (seqs[j] == seqs[i]) return fail(KV_ERR_ARG, "sequence %d appears twice in one append", seqs[i]);
            if (n_new[i] > 0) {
                const auto& sq = p->seqs[(size_t)seqs[i]];
                for (int64_t lp = start_pos[i] / PAGE; lp <= (start_pos[i] + n_new[i] - 1) / PAGE; ++lp)
                    if (p->refs[(size_t)sq.pages[(size_t)lp]] > 1)
                        return fail(KV_ERR_ARG, "entry %d: logical page %lld of sequence %d is shared with another sequence",
                                    i, (long long)lp, seqs[i]);
            }
            bd.seq[i] = seqs[i];
            bd.pos[i] = (int32_t)start_pos[i];
            bd.cnt[i] = n_new[i];
            bd.row0[i] = (int32_t)rows;
            bd.work0[i] = (int32_t)work;
            if (n_new[i] > 0) work += (start_pos[i] + n_new[i] - 1) / PAGE - start_pos[i] / PAGE + 1;
            rows += n_new[i];
            if (rows >= ((int64_t)1 << 31)) return fail(KV_ERR_UNSUPPORTED, "more than 2^31 rows in one append");
        }
        bd.work0[n] = (int32_t)work;
        if (work == 0) return KV_OK;  // no token to append: the row pointers are not read
        if (!d_k || !d_v) return fail(KV_ERR_ARG, "NULL k or v rows");
        hipError_t e = hipSuccess;
        if (p->fmt == KV_FMT_Q2 || p->fmt == KV_FMT_Q2_ROT) {
            e = launch_append_q2(p->view(), layer, bd, (int)work, d_k, d_v, (hipStream_t)stream, p->fmt == KV_FMT_Q2_ROT);
        } else if (p->fmt == KV_FMT_Q2_WINDOW) {
            // every row to the 2-bit pages, and the rows of the last page each
            // entry reaches to its window block
            e = launch_append_q2(p->view(), layer, bd, (int)work, d_k, d_v, (hipStream_t)stream);
            BatchDesc wd = bd;
            int m = 0;
            for (int i = 0; i < n; ++i) {
                if (bd.cnt[i] == 0) continue;
                const int end = bd.pos[i] + bd.cnt[i];
                const int lo = std::max(bd.pos[i], PAGE * ((end - 1) / PAGE));
                wd.seq[m] = bd.seq[i];
                wd.pos[m] = lo;
                wd.cnt[m] = end - lo;
                wd.row0[m] = bd.row0[i] + (lo - bd.pos[i]);
                wd.work0[m] = m;
                ++m;
            }
            wd.n = m;
            wd.work0[m] = m;
            if (e == hipSuccess && m > 0) e = launch_append_window(p->view(), layer, wd, d_k, d_v, (hipStream_t)stream);
        } else if (p->fmt == KV_FMT_BF16) {
            e = launch_append_bf16(p->view(), layer, bd, (int)work, d_k, d_v, (hipStream_t)stream);
        } else {
            // An 8-bit append that starts inside a page reads that page's staged
            // exact K rows; if it also runs past the page, its last page rewrites
            // the staging rows.  Such appends go in two launches: every entry's
            // first page, then the rest.
            bool split = false;
            for (int i = 0; i < n; ++i)
                if (bd.pos[i] % PAGE != 0 && bd.pos[i] / PAGE != (bd.pos[i] + bd.cnt[i] - 1) / PAGE) split = true;
            if (!split) {
                e = launch_append_q8(p->view(), layer, bd, (int)work, d_k, d_v, (hipStream_t)stream);
            } else {
                BatchDesc b1 = bd, b2 = bd;
                int64_t w1 = 0, w2 = 0;
                for (int i = 0; i < n; ++i) {
                    const int first = bd.cnt[i] > 0 ? std::min(bd.cnt[i], PAGE - bd.pos[i] % PAGE) : 0;
                    b1.cnt[i] = first;
                    b1.work0[i] = (int32_t)w1;
                    w1 += first > 0 ? 1 : 0;
                    b2.pos[i] = bd.pos[i] + first;
                    b2.cnt[i] = bd.cnt[i] - first;
                    b2.row0[i] = bd.row0[i] + first;
                    b2.work0[i] = (int32_t)w2;
                    if (b2.cnt[i] > 0) w2 += (b2.pos[i] + b2.cnt[i] - 1) / PAGE - b2.pos[i] / PAGE + 1;
                }
                b1.work0[n] = (int32_t)w1;
                b2.work0[n] = (int32_t)w2;
                if (w1 > 0) e = launch_append_q8(p->view(), layer, b1, (int)w1, d_k, d_v, (hipStream_t)stream);
                if (e == hipSuccess && w2 > 0)
                    e = launch_append_q8(p->view(), layer, b2, (int)w2, d_k, d_v, (hipStream_t)stream);
            }
        }
        if (e != hipSuccess) return hip_fail(e, "append launch");
        for (int i = 0; i < n; ++i) {
            auto& s = p->seqs[(size_t)seqs[i]];
            s.appended = std::max<int64_t>(s.appended, start_pos[i] + n_new[i]);
            if (sequential_appends(p->fmt)) s.layer_appended[(size_t)layer] = start_pos[i] + n_new[i];
        }
        return KV_OK;
    });
}

kv_status kv_decode_splits(const kv_pool* p, int32_t n, const int64_t* ctx_len, int32_t* n_splits) {
    return guarded([&]() -> kv_status {
        if (!p || !ctx_len || !n_splits || n <= 0) return fail(KV_ERR_ARG, "bad argument");
        *n_splits = auto_splits(p, n, ctx_len);
        return KV_OK;
    });
}

kv_status kv_workspace_bytes(const kv_pool* p, int32_t op, int32_t n_rows, int32_t n_splits, int64_t* bytes) {
    return guarded([&]() -> kv_status {
        if (!p || !bytes) return fail(KV_ERR_ARG, "NULL argument");
        if (n_rows < 0 || n_splits < 0) return fail(KV_ERR_ARG, "negative size");
        if (op == KV_OP_DECODE) {
            int sp = n_splits > 0 ? n_splits : 256;
            *bytes = 4 * decode_ws_floats(n_rows, p->geom.n_q_heads, p->geom.head_dim, sp);
        } else if (op == KV_OP_PREFILL) {
            const int sp = n_splits > 0 ? n_splits
                         : (n_rows > 0 ? prefill_auto_splits(n_rows, p->geom.n_q_heads, p->geom.n_kv_heads, p->fmt) : 1);
            *bytes = 4 * (prefill_ws_floats(n_rows, p->geom.n_q_heads, p->geom.head_dim, sp) +
                          prefill_extra_floats(p->fmt, n_rows, p->geom.n_q_heads, p->geom.head_dim));
        } else {
            return fail(KV_ERR_ARG, "unknown op %d", op);
        }
        return KV_OK;
    });
}

kv_status kv_attn_decode(kv_pool* p, int32_t layer, int32_t n, const int32_t* seqs, const int64_t* ctx_len,
                         const uint16_t* d_q, float sm_scale, int32_t n_splits, void* d_ws, int64_t ws_bytes,
                         float* d_out, float* d_scores, int64_t scores_stride, kv_stream_t stream) {
    return guarded([&]() -> kv_status {
        if (!p) return fail(KV_ERR_ARG, "pool is NULL");
        if (n <= 0) return fail(KV_ERR_ARG, "batch size must be positive");
        if (n > KV_MAX_BATCH) return fail(KV_ERR_UNSUPPORTED, "batch of %d exceeds KV_MAX_BATCH (%d)", n, KV_MAX_BATCH);
        if (!seqs || !ctx_len || !d_q || !d_out) return fail(KV_ERR_ARG, "NULL argument");
        if (layer < 0 || layer >= p->geom.n_layers) return fail(KV_ERR_ARG, "layer %d out of range", layer);
        if (n_splits < 0 || n_splits > 256) return fail(KV_ERR_ARG, "n_splits %d out of range (0..256)", n_splits);
        if (!(sm_scale > 0.f) || !(sm_scale < INFINITY)) return fail(KV_ERR_ARG, "sm_scale must be finite and positive");
        BatchDesc bd;
        memset(&bd, 0, sizeof bd);
        bd.n = n;
        const bool window = p->fmt == KV_FMT_Q2_WINDOW;
        int64_t max_ctx = 0, max_paged = 0;
        int64_t paged[KV_MAX_BATCH];  // tokens read from the pages
        for (int i = 0; i < n; ++i) {
            if (ctx_len[i] <= 0) return fail(KV_ERR_ARG, "entry %d: ctx_len must be >= 1", i);
            kv_status s = check_seq(p, seqs[i], ctx_len[i], "decode");
            if (s != KV_OK) return s;
            bd.seq[i] = seqs[i];
            paged[i] = ctx_len[i];
            if (window) {
                // tokens 64 floor((A - 1) / 64) .. A - 1 are read from the window block
                const int64_t A = p->seqs[(size_t)seqs[i]].layer_appended[(size_t)layer];
                if (ctx_len[i] > A)
                    return fail(KV_ERR_BOUND, "decode: entry %d: ctx_len %lld beyond the %lld tokens appended to layer %d",
                                i, (long long)ctx_len[i], (long long)A, layer);
                paged[i] = std::min<int64_t>(ctx_len[i], PAGE * ((A - 1) / PAGE));
                bd.cnt[i] = (int32_t)(ctx_len[i] - paged[i]);
            }
            bd.pos[i] = (int32_t)paged[i];
            max_ctx = std::max(max_ctx, ctx_len[i]);
            max_paged = std::max(max_paged, paged[i]);
        }
        if (d_scores && scores_stride < max_ctx) return fail(KV_ERR_ARG, "scores_stride %lld < max ctx_len %lld", (long long)scores_stride, (long long)max_ctx);
        int sp = n_splits > 0 ? n_splits : auto_splits(p, n, paged);
        bd.per = split_pairs_per((int)max_paged, sp);
        int64_t need = 4 * decode_ws_floats(n, p->geom.n_q_heads, p->geom.head_dim, sp);
        if (!d_ws || ws_bytes < need)
            return fail(KV_ERR_WORKSPACE, "decode needs %lld workspace bytes, got %lld", (long long)need, (long long)ws_bytes);
        hipStream_t s = (hipStream_t)stream;
        PoolView pv = p->view();
        if (window) {
            hipError_t e = hipSuccess;
            if (max_paged > 0)
                e = launch_decode_q2_partials(pv, layer, bd, d_q, sm_scale, sp, (float*)d_ws, d_scores, scores_stride, s);
            if (e == hipSuccess)
                e = launch_decode_window_merge(pv, layer, bd, d_q, sm_scale, sp, (const float*)d_ws, d_out, d_scores,
                                               scores_stride, s);
            if (e != hipSuccess) return hip_fail(e, "decode launch");
            return KV_OK;
        }
        hipError_t e =
            p->fmt == KV_FMT_Q2 || p->fmt == KV_FMT_Q2_ROT
                ? launch_decode_q2(pv, layer, bd, d_q, sm_scale, sp, (float*)d_ws, d_out, d_scores, scores_stride, s,
                                   p->fmt == KV_FMT_Q2_ROT)
            : p->fmt == KV_FMT_Q8 ? launch_decode_q8(pv, layer, bd, d_q, sm_scale, sp, (float*)d_ws, d_out, d_scores, scores_stride, s)
                                  : launch_decode_bf16(pv, layer, bd, d_q, sm_scale, sp, (float*)d_ws, d_out, d_scores,
                                                       scores_stride, s);
        if (e != hipSuccess) return hip_fail(e, "decode launch");
        return KV_OK;
    });
}

kv_status kv_attn_prefill(kv_pool* p, int32_t layer, int32_t seq, int64_t q_start, int32_t n_q, const uint16_t* d_q,
                          float sm_scale, int32_t n_splits, void* d_ws, int64_t ws_bytes, float* d_out,
                          kv_stream_t stream) {
    return guarded([&]() -> kv_status {
        if (!p) return fail(KV_ERR_ARG, "pool is NULL");
        if (p->fmt == KV_FMT_Q8)
            return fail(KV_ERR_FORMAT, "prefill is implemented for the 2-bit, bf16, 2-bit window and rotated formats only");
        if (n_q <= 0 || q_start < 0) return fail(KV_ERR_ARG, "bad chunk");
        if (q_start > INT32_MAX) return fail(KV_ERR_BOUND, "q_start %lld is not below 2^31", (long long)q_start);
        if (!d_q || !d_out) return fail(KV_ERR_ARG, "NULL argument");
        if (!(sm_scale > 0.f) || !(sm_scale < INFINITY)) return fail(KV_ERR_ARG, "sm_scale must be finite and positive");
        if (layer < 0 || layer >= p->geom.n_layers) return fail(KV_ERR_ARG, "layer %d out of range", layer);
        kv_status st = check_seq(p, seq, q_start + n_q, "prefill");
        if (st != KV_OK) return st;
        if (n_splits < 0 || n_splits > 64) return fail(KV_ERR_ARG, "n_splits %d out of range", n_splits);
        int w0 = 0;
        if (p->fmt == KV_FMT_Q2_WINDOW) {
            const int64_t A = p->seqs[(size_t)seq].layer_appended[(size_t)layer];
            if (q_start + n_q > A)
                return fail(KV_ERR_BOUND, "prefill: chunk ends at %lld, beyond the %lld tokens appended to layer %d",
                            (long long)(q_start + n_q), (long long)A, layer);
            w0 = (int)(PAGE * ((A - 1) / PAGE));
        }
        int sp = n_splits > 0 ? n_splits : prefill_auto_splits(n_q, p->geom.n_q_heads, p->geom.n_kv_heads, p->fmt);
        int64_t need = 4 * (prefill_ws_floats(n_q, p->geom.n_q_heads, p->geom.head_dim, sp) +
                            prefill_extra_floats(p->fmt, n_q, p->geom.n_q_heads, p->geom.head_dim));
        if (!d_ws || ws_bytes < need)
            return fail(KV_ERR_WORKSPACE, "prefill needs %lld workspace bytes, got %lld", (long long)need, (long long)ws_bytes);
        hipError_t e = launch_prefill(p->view(), (int)p->fmt, layer, seq, (int)q_start, n_q, d_q, sm_scale, sp,
                                      (float*)d_ws, d_out, w0, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "prefill launch");
        return KV_OK;
    });
}

kv_status kv_dequant_page(const kv_pool* p, int32_t page, int32_t layer, int32_t head, int32_t kv, float* d_out,
                          kv_stream_t stream) {
    return guarded([&]() -> kv_status {
        if (!p || !d_out) return fail(KV_ERR_ARG, "NULL argument");
        if (page < 0 || page >= p->n_pages) return fail(KV_ERR_ARG, "page %d out of range", page);
        if (layer < 0 || layer >= p->geom.n_layers) return fail(KV_ERR_ARG, "layer %d out of range", layer);
        if (head < 0 || head >= p->geom.n_kv_heads) return fail(KV_ERR_ARG, "head %d out of range", head);
        if (kv != 0 && kv != 1) return fail(KV_ERR_ARG, "kv must be 0 (K) or 1 (V)");
        hipError_t e = launch_dequant_page(p->view(), (int)page_format(p->fmt), page, layer, head, kv, d_out, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "dequant launch");
        return KV_OK;
    });
}

}  // extern "C"
