"""GPU parity, 2-bit pools with an exact window of the last appended page:
the pages bit-exact against the oracle's pool image, decode and chunked
prefill within tolerance of the fp64 oracle that reads the window's tokens
exact and the rest through the 2-bit codec.  Pages are filled with 0xFF
before use (a slot never written decodes to NaN), workspaces too."""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import WORKLOADS, Workload, kv_rows, page_permutation, queries
from tests.gpu_helpers import assert_close, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny"]
PREFILL = WORKLOADS["prefill"]
# group 2 at 128 dims (the matrix-core split kernel with two empty query rows), 2 layers
G2_128 = Workload(97, "group 2, D=128, window", "q2w", 2, 2, 128, 4, 3, 400)
# group 8: the split kernel's two workgroups a split
G8_128 = Workload(97, "group 8, D=128, window", "q2w", 2, 2, 128, 16, 3, 400)
NAN_FILL = 0xFF


def _fmt():
    import quantized_kv_attention_append_amd as kvq
    return kvq.FMT_Q2_WINDOW


def _append_both(pool, op, layer, seq, oseq, bt, k, v, pieces, start=0):
    for n in pieces:
        pool.append(layer, [seq], [start], [n], k[start:start + n].cuda(), v[start:start + n].cuda())
        op.append(layer, oseq, bt, start, k[start:start + n].float().numpy(), v[start:start + n].float().numpy())
        start += n
    return start


def test_window_append_pages_bit_exact():
    need_gpu()
    n_pages = 6
    pool, mem = make_pool(TINY, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(TINY, n_pages)[:4]
    seq = pool.reserve(256, pages=bt)
    k, v = kv_rows(TINY, 0, 0, 256)
    op = opool.OraclePool("q2w", 1, 4, 256, n_pages, fill=NAN_FILL)
    _append_both(pool, op, 0, seq, 0, bt, k, v, (100, 1, 27, 64, 64))
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"window append: {diff} differing bytes of {got.size}")
    assert diff == 0


def _decode_check(pool, op, w, layer, seq, oseq, bt, ctx, splits_list, tag):
    q = queries(w, layer, 1, stream=ctx)
    K, V = op.gather(layer, bt, ctx, seq=oseq)
    qn = q[0].float().numpy()
    ref = attention.decode(qn, K, V, w.sm_scale)
    ref_s = attention.scores(qn, K, w.sm_scale)
    for sp in splits_list:
        scores = torch.full((1, w.n_q_heads, ctx), float("nan"), device="cuda")
        ws = torch.full((pool.workspace_bytes(0, 1, sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.decode(layer, [seq], [ctx], q.cuda(), w.sm_scale, n_splits=sp, ws=ws, scores=scores)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy()[0], ref, f"{tag} ctx={ctx} splits={sp}")
        s = scores.cpu().numpy()[0].astype(np.float64)
        assert np.all(np.isfinite(s)), f"{tag}: a score was not written"
        rel = np.linalg.norm(s - ref_s) / np.linalg.norm(ref_s)
        assert rel <= 1e-5, f"{tag} ctx={ctx} splits={sp}: scores rel L2 {rel:.2e}"


@pytest.mark.parametrize("pieces", [(1,), (50,), (64,), (64, 1), (100, 1, 27, 72), (500, 300, 200)])
def test_window_decode_ragged(pieces):
    need_gpu()
    total = sum(pieces)
    n_pages = -(-total // 64) + 2
    pool, mem = make_pool(TINY, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(TINY, n_pages, salt=total)[:-2]
    seq = pool.reserve(total, pages=bt)
    k, v = kv_rows(TINY, 0, 0, total)
    op = opool.OraclePool("q2w", 1, 4, 256, n_pages, fill=NAN_FILL)
    _append_both(pool, op, 0, seq, 0, bt, k, v, pieces)
    w0 = op.window_start(0, 0)
    # the whole context, one token short, the window start and a context before it
    ctxs = sorted({c for c in (total, total - 1, w0, w0 - 5) if c >= 1})
    for ctx in ctxs:
        _decode_check(pool, op, TINY, 0, seq, 0, bt, ctx, [1, 3, 0], f"window pieces={pieces}")


@pytest.mark.parametrize("w", [G2_128, G8_128], ids=lambda w: w.name)
def test_window_decode_batched_d128(w):
    need_gpu()
    lens = [400, 64, 30, 129]
    n_pages = sum(-(-L // 64) for L in lens) + 1
    pool, mem = make_pool(w, n_pages, _fmt(), fill=NAN_FILL)
    perm = page_permutation(w, n_pages)
    op = opool.OraclePool("q2w", w.n_layers, w.n_kv_heads, w.head_dim, n_pages, fill=NAN_FILL)
    bts, seqs, off = [], [], 0
    for L in lens:
        npg = -(-L // 64)
        bts.append(perm[off:off + npg]); off += npg
        seqs.append(pool.reserve(L, pages=bts[-1]))
    layer = 1
    for i, L in enumerate(lens):
        k, v = kv_rows(w, layer, i, L)
        _append_both(pool, op, layer, seqs[i], i, bts[i], k, v, (L // 3, L - L // 3) if L > 3 else (L,))
    ctxs = [400, 64, 30, 100]   # the last lane reads only 2-bit tokens (its window starts at 128)
    q = queries(w, layer, len(lens))
    ref = np.stack([attention.decode(q[i].float().numpy(), *op.gather(layer, bts[i], ctxs[i], seq=i), w.sm_scale)
                    for i in range(len(lens))])
    for sp in (1, 2, 0, 12):  # up to 8 splits the split kernel attends to the window too; 12: a merge kernel does
        ws = torch.full((pool.workspace_bytes(0, len(lens), sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.decode(layer, seqs, ctxs, q.cuda(), w.sm_scale, n_splits=sp, ws=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, f"window batched {w.name} splits={sp}")


def _prefill_case(w, layer, prior, n_q, splits_list, salt=0):
    import quantized_kv_attention_append_amd as kvq
    total = prior + n_q
    n_pages = -(-total // 64) + 1
    pool, mem = make_pool(w, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(w, n_pages, salt=salt)[:-1]
    seq = pool.reserve(total, pages=bt)
    k, v = kv_rows(w, layer, 0, total)
    if prior:
        pool.append(layer, [seq], [0], [prior], k[:prior].cuda(), v[:prior].cuda())
    pool.append(layer, [seq], [prior], [n_q], k[prior:].cuda(), v[prior:].cuda())
    q = queries(w, layer, n_q, stream=1)
    K, V = opool.dequantized_rows("q2w", k.float().numpy(), v.float().numpy())
    ref = attention.prefill(q.float().numpy(), K, V, w.sm_scale, q_start=prior)
    for sp in splits_list:
        ws = torch.full((pool.workspace_bytes(kvq.OP_PREFILL, n_q, sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.prefill(layer, seq, prior, q.cuda(), w.sm_scale, n_splits=sp, ws=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, f"window prefill prior={prior} n_q={n_q} splits={sp}")
    return pool, seq


def test_window_prefill_small():
    need_gpu()
    _prefill_case(TINY, 0, 100, 45, [1, 2, 3, 0])


def test_window_prefill_all_in_window():
    need_gpu()
    _prefill_case(TINY, 0, 0, 50, [1, 2])     # every key is a window key: no page is read


def test_window_prefill_chunk_from_zero_two_pages():
    need_gpu()
    _prefill_case(TINY, 0, 0, 130, [1, 2, 0])


def test_window_prefill_group2_d128():
    need_gpu()
    _prefill_case(G2_128, 1, 70, 64, [1, 3])


def test_window_prefill_full_chunk_sampled():
    """The 65,536 + 1,024 chunk over a window pool: the last 64 keys of the
    sequence are exact (the chunk ends on a page boundary), sampled rows
    against the oracle."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    w = PREFILL
    prior, n_q = w.ctx, w.chunk
    total = prior + n_q
    n_pages = total // 64
    pool, mem = make_pool(w, n_pages, _fmt(), fill=NAN_FILL, max_seqs=1)
    bt = page_permutation(w, n_pages)
    seq = pool.reserve(total, pages=bt)
    k, v = kv_rows(w, 0, 0, total, device="cuda")
    pool.append(0, [seq], [0], [prior], k[:prior].contiguous(), v[:prior].contiguous())
    pool.append(0, [seq], [prior], [n_q], k[prior:].contiguous(), v[prior:].contiguous())
    q = queries(w, 0, n_q, device="cuda", stream=1)
    ws = torch.full((pool.workspace_bytes(kvq.OP_PREFILL, n_q, 0),), 0xFF, dtype=torch.uint8, device="cuda")
    out = pool.prefill(0, seq, prior, q, w.sm_scale, ws=ws)
    torch.cuda.synchronize()
    K, V = opool.dequantized_rows("q2w", k.float().cpu().numpy(), v.float().cpu().numpy())
    rows = [0, 1, 500, 959, 960, 1000, n_q - 1]   # 960.. see window keys
    ref = attention.prefill(q.float().cpu().numpy(), K, V, w.sm_scale, q_start=prior, rows=rows)
    assert_close(out.cpu().numpy()[rows], ref, "window prefill 65536+1024 sampled rows")


def test_window_refusals_before_any_byte_moves():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    n_pages = 4
    pool, mem = make_pool(TINY, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(TINY, n_pages)[:3]
    seq = pool.reserve(192, pages=bt)
    k, v = kv_rows(TINY, 0, 0, 192)
    pool.append(0, [seq], [0], [100], k[:100].cuda(), v[:100].cuda())
    torch.cuda.synchronize()
    before = mem.cpu().clone()
    with pytest.raises(kvq.KvError) as ei:      # appends are sequential per layer
        pool.append(0, [seq], [101], [10], k[101:111].cuda(), v[101:111].cuda())
    assert ei.value.name == "KV_ERR_ARG"
    q = queries(TINY, 0, 1)
    with pytest.raises(kvq.KvError) as ei:      # decode past the appended tokens
        pool.decode(0, [seq], [101], q.cuda(), TINY.sm_scale)
    assert ei.value.name == "KV_ERR_BOUND"
    qc = queries(TINY, 0, 10, stream=1)
    with pytest.raises(kvq.KvError) as ei:      # prefill chunk past the appended tokens
        pool.prefill(0, seq, 95, qc.cuda(), TINY.sm_scale)
    assert ei.value.name == "KV_ERR_BOUND"
    ws = torch.empty((pool.workspace_bytes(kvq.OP_PREFILL, 5, 1) - 4,), dtype=torch.uint8, device="cuda")
    with pytest.raises(kvq.KvError) as ei:      # the window's partials need their room
        pool.prefill(0, seq, 95, qc[:5].cuda(), TINY.sm_scale, n_splits=1, ws=ws)
    assert ei.value.name == "KV_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.equal(mem.cpu(), before)


@pytest.mark.parametrize("ctx_off", [0, 1, 70])
def test_window_decode_many_splits(ctx_off):
    """More than 8 live splits (20 and 64): the window merge folds the split
    partials in several groups after the window's own partial; the context
    ends at the last token, one short of it, or before the window."""
    need_gpu()
    total = 5000
    n_pages = -(-total // 64) + 1
    pool, mem = make_pool(TINY, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(TINY, n_pages, salt=7)[:-1]
    seq = pool.reserve(total, pages=bt)
    k, v = kv_rows(TINY, 0, 0, total)
    op = opool.OraclePool("q2w", 1, 4, 256, n_pages, fill=NAN_FILL)
    _append_both(pool, op, 0, seq, 0, bt, k, v, (2000, 1999, 1001))
    _decode_check(pool, op, TINY, 0, seq, 0, bt, total - ctx_off, [20, 64], f"window many splits, ctx={total - ctx_off}")
