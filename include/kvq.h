/*
 * kvq.h — C ABI of a paged, quantized KV cache with attention that reads the
 * compressed pages directly, for AMD Instinct MI355X (gfx950).
 *
 * What it implements, by source page:
 *  - "KV at 9 KB a token" (ignis, why-ignis/kv-in-bytes), section "How it
 *    works": a per-token byte cost of 64 B of 2-bit code plus an 8-byte
 *    metadata row per head per token (9,216 B a token at 16 layers x 4 KV
 *    heads x 256 dims); the pool is a byte budget of 64-token pages; a request
 *    reserves pages for its whole bound when admitted; prefill attention reads
 *    the compressed cache; every workspace byte a launch reads it writes first.
 *    Section "See it, control it": pool size in bytes or tokens, and the pool
 *    figures (pages, used pages, page bytes).
 *  - "The KV cache and prompt reuse" (ignis, concepts), section "What a
 *    sequence is made of": one pool shared by all lanes, a lane is charged for
 *    the pages it holds; the most recent keys are held unquantized by the
 *    compressed format.  Section "When reuse misses": a format mismatch is
 *    rejected with nothing copied.
 *  - "Half the Cache, Twice the Context" (ml.co.ke): the symmetric absmax
 *    quantizer with per-channel K and per-token V scaling (section "What the
 *    cache loses when you round it"), accumulation in real FP32 (section "The
 *    cliff is in the accumulator"), and failing loudly rather than falling
 *    back (section "How to apply this", item 6).
 *
 * Conventions for every call:
 *  - Every entry point returns kv_status.  On any status other than KV_OK the
 *    call has launched nothing and written nothing (host checks run first),
 *    and kv_last_error() returns a message for the calling thread.
 *  - There is no fallback path: an unsupported geometry, format or size is an
 *    error, never a slower route.
 *  - Pointers named d_* are device pointers owned by the caller (for example
 *    torch tensors); all other pointers are host pointers read during the
 *    call only.  A kv_stream_t is a hipStream_t (NULL = the null stream).
 *    Kernels run asynchronously on that stream; host-side pool metadata
 *    (reservations, block tables) is updated synchronously.
 *  - A kv_pool is not thread-safe: calls on one pool must not overlap.
 *  - Token positions and lengths are < 2^31; head_dim is 128 or 256; the GQA
 *    group G = n_q_heads / n_kv_heads must be 1, 2, 4 or 8; n_layers is at
 *    most KV_MAX_LAYERS and n_kv_heads at most KV_MAX_KV_HEADS
 *    (KV_ERR_UNSUPPORTED otherwise).
 *  - A batch holds at most KV_MAX_BATCH sequences per call.
 *  - No C++ exception leaves the library: a failed host allocation returns
 *    KV_ERR_DEVICE, like a failed HIP call, with the pool unchanged.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV_PAGE_TOKENS 64
#define KV_MAX_BATCH 128
#define KV_MAX_LAYERS 1024
#define KV_MAX_KV_HEADS 256

typedef void* kv_stream_t; /* hipStream_t */
typedef struct kv_pool kv_pool;

typedef enum {
    /* 2-bit rows sized like hq-e8-2b: per (token, KV head) D/4 bytes of
     * uniform 2-bit codes plus an 8-byte [fp32 scale, fp32 min] row; the
     * dequantized value is fmaf(code, scale, min). */
    KV_FMT_Q2 = 1,
    /* int8 codes: K scaled per channel over the tokens of its 64-token page,
     * V scaled per token (fp32 scales, symmetric, codes in [-127, 127]). */
    KV_FMT_Q8 = 2,
    /* the rows as given, bf16: 512 B per head per token at D = 256, the BF16
     * row of "KV at 9 KB a token" (section "How it works", table).  It is the
     * exact cache that the compressed format is priced against (same page,
     * sections "The numbers": the decode price of hq against BF16, and "See
     * it, control it": the format is hq-e8-2b or bf16), in the same paged
     * pool and through the same calls. */
    KV_FMT_BF16 = 3,
    /* KV_FMT_Q2 pages plus the unquantized recent keys that "The KV cache
     * and prompt reuse" (section "What a sequence is made of") has the
     * compressed format hold, read as one page: for each (sequence, layer, KV
     * head) the bf16 K and V rows of the last page appended to.  With A
     * tokens of a (sequence, layer) appended, decode and prefill read tokens
     * 64 * floor((A - 1) / 64) .. A - 1 exact and every earlier token from
     * the 2-bit pages, which hold exactly what a KV_FMT_Q2 pool holds.  The
     * pages cost what 2-bit pages cost; the exact rows take 256 x D bytes per
     * (sequence slot, layer, KV head) outside the page budget (4 MiB a slot
     * at 16 x 4 x 256).  Appends are sequential per (sequence, layer), and
     * attention reads at most the tokens appended. */
    KV_FMT_Q2_WINDOW = 4,
    /* KV_FMT_Q2 pages holding the 2-bit rows of H k, with H the
     * unnormalised Walsh-Hadamard matrix (Sylvester order, entries +-1,
     * H H = D I), applied in fp32 butterflies, stages h = 1, 2, .., D/2, each
     * replacing (x_i, x_{i+h}) by (x_i + x_{i+h}, x_i - x_{i+h}), and V rows
     * as KV_FMT_Q2 holds them: the rotation choice at 2 bits that "Half the
     * Cache, Twice the Context" names in its closing notes, applied where its
     * outliers are channels (K), which the rotation spreads over the row
     * before the per-token range is taken.  Decode rotates the query the same
     * way and scores with sm_scale / D (H q . H k = D q . k); prefill
     * rotates the chunk's query rows the same way and takes them as two
     * bf16 terms (the rounded value and the rounded residual), which its
     * workspace holds.  kv_dequant_page returns K rows in the rotated
     * basis. */
    KV_FMT_Q2_ROT = 5
} kv_format;

typedef enum {
    KV_OK = 0,
    KV_ERR_ARG = -1,         /* null pointer, negative size, bad index */
    KV_ERR_NO_SPACE = -2,    /* not enough free pages (or sequence slots) */
    KV_ERR_BOUND = -3,       /* position or length beyond a sequence's reserved bound */
    KV_ERR_FORMAT = -4,      /* operation does not match the pool's format */
    KV_ERR_UNSUPPORTED = -5, /* geometry / batch size this library does not implement */
    KV_ERR_WORKSPACE = -6,   /* workspace null or smaller than kv_workspace_bytes() */
    KV_ERR_DEVICE = -7       /* a HIP runtime call (or a host allocation) failed */
} kv_status;

typedef struct {
    int32_t n_layers;   /* attention layers that keep a cache */
    int32_t n_kv_heads; /* Hkv */
    int32_t head_dim;   /* D: 128 or 256 */
    int32_t n_q_heads;  /* Hq, a multiple of Hkv; query head h reads KV head h / (Hq/Hkv) */
} kv_geom;

typedef struct {
    int64_t pages;          /* pages the byte budget bought */
    int64_t free_pages;     /* pages not reserved by any sequence */
    int64_t reserved_pages; /* pages reserved by live sequences (a shared page counts once) */
    int64_t used_pages;     /* reserved pages that hold at least one appended token (shared: once) */
    int64_t page_bytes;     /* 64 x token_bytes */
    int64_t token_bytes;    /* e.g. 9,216 for 2-bit at 16 x 4 x 256 */
    int64_t tokens;         /* pages x 64 */
    int64_t n_seqs;         /* live sequences */
} kv_pool_stats_t;

/* Bytes one token costs in a format, and the bytes of one 64-token page.
 * 2-bit: 2 x L x Hkv x (D/4 + 8).  8-bit: L x Hkv x (2D + 4 + 4D/64).
 * bf16: 4 x L x Hkv x D. */
kv_status kv_token_bytes(const kv_geom* geom, kv_format fmt, int64_t* token_bytes, int64_t* page_bytes);

/* Byte budget that holds `tokens` tokens in whole pages (the pool size can be
 * given in tokens as well as bytes). */
kv_status kv_pool_bytes_for_tokens(const kv_geom* geom, kv_format fmt, int64_t tokens, int64_t* bytes);

/* Create a pool of floor(bytes / page_bytes) pages.  d_mem: NULL to let the
 * library allocate device memory (freed by kv_pool_destroy), or caller-owned
 * device memory of at least pages x page_bytes bytes.  max_seqs and
 * max_seq_tokens size the device block tables (and, for KV_FMT_Q8 and
 * KV_FMT_Q2_WINDOW, the per-sequence exact window of one page per layer and
 * head).  Prints one
 * line with the page and token counts to stderr.  Errors: KV_ERR_ARG,
 * KV_ERR_UNSUPPORTED (geometry), KV_ERR_NO_SPACE (budget below one page),
 * KV_ERR_DEVICE. */
kv_status kv_pool_create(int64_t bytes, const kv_geom* geom, kv_format fmt, int32_t max_seqs,
                         int64_t max_seq_tokens, void* d_mem, kv_pool** out);

/* Destroy a pool; frees only memory the library allocated (with hipFree, so
 * not while a HIP graph capture is active: that would invalidate it). */
kv_status kv_pool_destroy(kv_pool* pool);

kv_status kv_pool_stats(const kv_pool* pool, kv_pool_stats_t* out);

/* Device address and size of the page array (page p starts at p x page_bytes);
 * for inspection and tests. */
kv_status kv_pool_device_ptr(const kv_pool* pool, void** d_pages, int64_t* bytes);

/* Admission: reserve ceil(max_tokens / 64) pages for a new sequence's whole
 * bound and upload its block table once ("KV at 9 KB a token", section "How
 * it works": the pool cannot run dry halfway through a reply; "The KV cache
 * and prompt reuse", section "What a sequence is made of": one pool shared by
 * every lane).  pages: NULL to take free pages, or an explicit list of
 * exactly ceil(max_tokens / 64) distinct free page ids (logical page i ->
 * physical pages[i]); the library reads that many entries.  Errors: KV_ERR_ARG, KV_ERR_BOUND (max_tokens above the
 * pool's max_seq_tokens), KV_ERR_NO_SPACE (not enough free pages or no free
 * sequence slot), KV_ERR_DEVICE. */
kv_status kv_seq_reserve(kv_pool* pool, int64_t max_tokens, const int32_t* pages, int32_t* seq);

/* Prefix sharing ("The KV cache and prompt reuse", section "What a sequence
 * is made of": a lane is charged for the pages it holds, and the full pages of
 * a shared prefix are held once).  Admit a new sequence with a bound of
 * max_tokens whose first n_tokens tokens are those of sequence `parent`:
 *  - the parent's pages that n_tokens fills completely (logical pages below
 *    n_tokens / 64) are shared: both block tables name them, each page counts
 *    its holders, and neither sequence may append into a page held twice;
 *  - the page n_tokens fills only partly is copied whole, on `stream`, into a
 *    fresh page of the child's (copy on write), with the exact rows the
 *    format keeps for it (8-bit pools: the open page's exact K rows; 2-bit
 *    window pools: every layer's window block);
 *  - the rest of the child's bound takes fresh pages.
 * The child starts with n_tokens appended in every layer.  Requirements:
 * 1 <= n_tokens <= max_tokens, n_tokens at most the tokens appended to the
 * parent; 8-bit pools: n_tokens equals the tokens appended to every layer of
 * the parent; 2-bit window pools: n_tokens lies in the last page appended to
 * in every layer.  Errors: KV_ERR_ARG, KV_ERR_BOUND (max_tokens above the
 * pool's max_seq_tokens), KV_ERR_NO_SPACE, KV_ERR_DEVICE. */
kv_status kv_seq_fork(kv_pool* pool, int32_t parent, int64_t n_tokens, int64_t max_tokens, kv_stream_t stream,
                      int32_t* child);

/* Release a sequence: each of its pages loses a holder, and a page with no
 * holder left returns to the free list. */
kv_status kv_seq_release(kv_pool* pool, int32_t seq);

/* The device block table of a live sequence: *d_bt receives the device
 * address of its int32 page ids (logical page i -> physical page d_bt[i]),
 * the array every kernel walks, and *n_pages their count,
 * ceil(bound / 64), all reserved at admission ("KV at 9 KB a token",
 * section "How it works": a request reserves the pages of its whole bound
 * when it is admitted).  The array is owned by the pool and stays valid and
 * unchanged until the sequence is released; the caller must not write it.
 * Errors: KV_ERR_ARG (NULL argument, sequence not live). */
kv_status kv_seq_block_table(const kv_pool* pool, int32_t seq, const int32_t** d_bt, int32_t* n_pages);

/* Host copy of a sequence's block table: writes up to cap page ids. */
kv_status kv_seq_pages(const kv_pool* pool, int32_t seq, int32_t* pages, int32_t cap, int32_t* n_pages);

/* Quantize-on-append for one layer: every new token costs a fixed number of
 * bytes in its page slot ("KV at 9 KB a token", section "How it works": per
 * head per token, 64 B of 2-bit code and an 8-byte metadata row at 256 dims;
 * the 8-bit variant follows "Half the Cache, Twice the Context", section
 * "What the cache loses when you round it": the symmetric absmax quantizer,
 * K scaled per channel, V per token).  For entry i, rows
 * d_k[row_i .. row_i + n_new[i]) (bf16 [rows][Hkv][D], row_i = sum of earlier
 * n_new) go to positions start_pos[i] .. start_pos[i] + n_new[i] - 1 of
 * sequence seqs[i]; same for d_v.  Each token's K and V rows are quantized in
 * fp32 (2-bit: min, scale = (max - min) / 3 correctly rounded, codes
 * rint((x - min) / scale) clamped to 0..3; 8-bit: V per token; K per channel
 * over the exact rows present in the token's page; bf16: stored as given) and
 * written into slot
 * pos % 64 of page block_table[pos / 64].  No other slot of the pool changes,
 * except that an 8-bit append re-derives the K codes and channel scales of the
 * pages it touches.  8-bit appends are sequential per (sequence, layer):
 * start_pos must equal the tokens already appended to that layer, because
 * the exact K rows of the open page are kept only for the tokens appended so
 * far; the same holds for KV_FMT_Q2_WINDOW, whose append also copies the
 * rows of the last page it reaches into the sequence's exact window.  No
 * append may write into a page that two sequences hold (kv_seq_fork).  The
 * sequences of one call must be distinct; d_k and d_v may be NULL when no
 * entry appends a token.  Errors: KV_ERR_ARG (including a
 * non-sequential 8-bit or window append), KV_ERR_BOUND (a position beyond
 * the reserved bound; nothing is written), KV_ERR_UNSUPPORTED (more than
 * KV_MAX_BATCH entries), KV_ERR_DEVICE. */
kv_status kv_append_quant(kv_pool* pool, int32_t layer, int32_t n, const int32_t* seqs,
                          const int64_t* start_pos, const int32_t* n_new, const uint16_t* d_k,
                          const uint16_t* d_v, kv_stream_t stream);

enum { KV_OP_DECODE = 0, KV_OP_PREFILL = 1 };

/* Workspace bytes for an attention call ("KV at 9 KB a token", section "How
 * it works": the workspace needs no zeroing, since every byte a launch reads
 * it has written first): decode with n_rows sequences, or
 * prefill with n_rows chunk queries, and n_splits splits of the context.
 * n_splits = 0 asks for enough bytes for the split count the library picks
 * by itself (decode: any count up to 256; prefill: the count it picks for
 * n_rows queries, about one workgroup per compute unit).  A KV_FMT_Q2_WINDOW
 * prefill needs one more split's worth for the window's partials, a
 * KV_FMT_Q2_ROT prefill 4 x n_rows x Hq x D more bytes for the rotated
 * query's two bf16 terms. */
kv_status kv_workspace_bytes(const kv_pool* pool, int32_t op, int32_t n_rows, int32_t n_splits, int64_t* bytes);

/* Split-count the library picks for a decode batch when n_splits = 0. */
kv_status kv_decode_splits(const kv_pool* pool, int32_t n, const int64_t* ctx_len, int32_t* n_splits);

/* One decode step for n sequences of one layer, reading the compressed pages
 * directly through the block tables ("KV at 9 KB a token", opening section
 * and "How it works": attention reads the compressed cache, priced per token
 * in section "The numbers"), with every long sum in fp32 registers ("Half the
 * Cache, Twice the Context", section "The cliff is in the accumulator, not
 * the storage": a low-precision accumulator loses the mass of long flat
 * contexts).  d_q: bf16 [n][Hq][D], one
 * query per sequence; sequence i attends to its tokens 0 .. ctx_len[i]-1
 * (ctx_len >= 1, within the reserved bound; n, seqs and ctx_len hold n
 * entries).  Scores are sm_scale x q.k^ (sm_scale finite and > 0) over
 * the dequantized keys; softmax and all sums are kept in fp32; the contexts
 * are split into ranges of whole page pairs (flash-decoding), all of one size:
 * ceil(page pairs of the longest context / n_splits), n_splits in 1..256
 * (0 = kv_decode_splits' choice), so a shorter context fills fewer ranges.
 * The ranges' partial results (max, sum, unnormalised output) go to d_ws and
 * are merged in fp32: for KV_FMT_Q2 and KV_FMT_Q2_ROT at n_splits <= 8 by the
 * last workgroup of the split kernel to finish a (sequence, KV head), else by
 * a second kernel on the same stream.
 * KV_FMT_Q2_WINDOW: the ranges cover the tokens before the window; the merge
 * kernel also attends to the window's exact rows (ctx_len at most the tokens
 * appended to the layer, else KV_ERR_BOUND).
 * d_out: fp32 [n][Hq][D].  d_scores: NULL, or fp32 [n][Hq][scores_stride]
 * receiving the raw logits (scores_stride >= max ctx_len).  Every workspace
 * byte read is written first within the call.  Errors: KV_ERR_ARG,
 * KV_ERR_BOUND, KV_ERR_FORMAT, KV_ERR_UNSUPPORTED, KV_ERR_WORKSPACE,
 * KV_ERR_DEVICE. */
kv_status kv_attn_decode(kv_pool* pool, int32_t layer, int32_t n, const int32_t* seqs, const int64_t* ctx_len,
                         const uint16_t* d_q, float sm_scale, int32_t n_splits, void* d_ws, int64_t ws_bytes,
                         float* d_out, float* d_scores, int64_t scores_stride, kv_stream_t stream);

/* Bytes of the static device array kv_attn_decode_static uses as its
 * workspace (one per device). */
#define KV_STATIC_SCRATCH_BYTES (16ll << 20)

/* kv_attn_decode for callers that cannot allocate device memory at call time
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments and results as kv_attn_decode (and the same
 * split count for n_splits = 0), with the workspace a file-scope device array
 * of KV_STATIC_SCRATCH_BYTES per device instead of d_ws.  Nothing is
 * allocated: the array's device address is looked up once per device on the
 * first call there, with the pool's device current.  A batch whose workspace
 * (kv_workspace_bytes) exceeds the array is refused with KV_ERR_WORKSPACE.
 * All calls on one device share the array: calls that overlap on a device
 * (other streams, other pools) race and must be ordered by the caller.
 * Errors: those of kv_attn_decode, KV_ERR_ARG (the current device is not the
 * pool's), KV_ERR_WORKSPACE (batch too large for the array). */
kv_status kv_attn_decode_static(kv_pool* pool, int32_t layer, int32_t n, const int32_t* seqs, const int64_t* ctx_len,
                                const uint16_t* d_q, float sm_scale, int32_t n_splits, float* d_out, float* d_scores,
                                int64_t scores_stride, kv_stream_t stream);

/* Causal prefill of a chunk of n_q queries of one sequence that sit at
 * positions q_start .. q_start + n_q - 1, after the chunk's own K/V have been
 * appended ("KV at 9 KB a token", opening section and "How it works":
 * prefill attention reads the compressed cache directly): query i attends to
 * tokens 0 .. q_start + i, all read from the pool.  2-bit, bf16, 2-bit window
 * pools (the window's keys come exact from its bf16 rows, through a third
 * kernel whose partials the merge adds; the chunk must lie within the tokens
 * appended) and rotated 2-bit pools (the chunk's query rows are rotated first
 * and enter as two bf16 terms).  Scores are sm_scale x q.k^ (sm_scale finite
 * and > 0); softmax and sums in fp32 ("Half the Cache, Twice the Context",
 * section "The cliff is in the accumulator, not the storage"); both
 * contractions run on bf16 matrix cores with exact code operands and 16-bit
 * softmax weights.  The keys of each block of queries are split into
 * n_splits ranges (1..64, 0 = the library's choice) whose partials go to d_ws
 * and are merged by a second kernel.  d_q: bf16 [n_q][Hq][D]; d_out: fp32
 * [n_q][Hq][D].  The workspace (kv_workspace_bytes) needs no clearing: every
 * byte read is written first within the call.  Errors: KV_ERR_ARG,
 * KV_ERR_BOUND, KV_ERR_FORMAT (an 8-bit pool), KV_ERR_WORKSPACE,
 * KV_ERR_DEVICE. */
kv_status kv_attn_prefill(kv_pool* pool, int32_t layer, int32_t seq, int64_t q_start, int32_t n_q,
                          const uint16_t* d_q, float sm_scale, int32_t n_splits, void* d_ws, int64_t ws_bytes,
                          float* d_out, kv_stream_t stream);

/* Dequantize the 64 token slots of one (page, layer, KV head, K or V) plane
 * into d_out fp32 [64][D] (kv: 0 = K, 1 = V): each row's codes through its
 * metadata row ("KV at 9 KB a token", section "How it works": a row is its
 * 2-bit codes plus an 8-byte metadata row; here fmaf(code, scale, min)), or
 * code x scale for 8-bit rows ("Half the Cache, Twice the Context", section
 * "What the cache loses when you round it"), or the stored bf16 values.  Slots never written hold
 * whatever the decoding of their bytes gives. */
kv_status kv_dequant_page(const kv_pool* pool, int32_t page, int32_t layer, int32_t head, int32_t kv, float* d_out,
                          kv_stream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* kv_last_error(void);

/* Name of a status code. */
const char* kv_status_str(kv_status s);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
