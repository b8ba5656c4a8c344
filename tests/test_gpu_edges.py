"""GPU parity at the library's size limits and on empty inputs, 2-bit pools:
a batch of KV_MAX_BATCH (128) sequences of ragged lengths appended in one
call (entries with no tokens among them) and decoded in one call, at the
library's split count and at the maximum of 256 splits; one entry more is
refused; an append of no tokens changes no byte."""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import Workload, kv_rows, queries
from tests.gpu_helpers import assert_close, make_pool, need_gpu, say

PAGE_TOKENS = 64

pytestmark = pytest.mark.gpu

# 1 layer x 2 KV heads x 128 dims, 8 query heads (group 4)
W = Workload(95, "edges, D=128", "q2", 1, 2, 128, 8, 128, 300)


def test_max_batch_ragged_and_max_splits():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    B = 128
    rng = np.random.default_rng(11)
    lens = [int(x) for x in rng.integers(1, 300, size=B)]
    n_pages = sum(-(-n // 64) for n in lens)
    pool, mem = make_pool(W, n_pages, kvq.FMT_Q2, fill=0xFF, max_seqs=B)
    seqs = [pool.reserve(n) for n in lens]
    rows = [kv_rows(W, 0, i, n) for i, n in enumerate(lens)]
    # first call: every entry, some with no tokens (their first part is empty)
    first = [0 if i % 7 == 0 else min(n, 40) for i, n in enumerate(lens)]
    pool.append(0, seqs, [0] * B, first, torch.cat([rows[i][0][:first[i]] for i in range(B)]).cuda(),
                torch.cat([rows[i][1][:first[i]] for i in range(B)]).cuda())
    rest = [n - f for n, f in zip(lens, first)]
    pool.append(0, seqs, first, rest, torch.cat([rows[i][0][first[i]:] for i in range(B)]).cuda(),
                torch.cat([rows[i][1][first[i]:] for i in range(B)]).cuda())
    q = queries(W, 0, B)
    refs = []
    for i in range(B):
        K, V = opool.dequantized_rows("q2", rows[i][0].float().numpy(), rows[i][1].float().numpy())
        refs.append(attention.decode(q[i].float().numpy(), K, V, W.sm_scale))
    refs = np.stack(refs)
    for sp in (0, 256):
        ws = torch.full((pool.workspace_bytes(kvq.OP_DECODE, B, sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.decode(0, seqs, lens, q.cuda(), W.sm_scale, n_splits=sp, ws=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), refs, f"128 ragged lanes, splits={sp or pool.decode_splits(lens)}")
    with pytest.raises(kvq.KvError) as ei:
        pool.decode(0, seqs + [seqs[0]], lens + [lens[0]], torch.cat([q, q[:1]]).cuda(), W.sm_scale)
    assert ei.value.name == "KV_ERR_UNSUPPORTED"


def test_empty_append_changes_nothing():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    pool, mem = make_pool(W, 4, kvq.FMT_Q2, fill=0x5A)
    seq = pool.reserve(200)
    k, v = kv_rows(W, 0, 0, 100)
    pool.append(0, [seq], [0], [100], k.cuda(), v.cuda())
    torch.cuda.synchronize()
    before = mem.cpu().clone()
    empty = torch.empty((0, W.n_kv_heads, W.head_dim), dtype=torch.bfloat16, device="cuda")
    pool.append(0, [seq], [100], [0], empty, empty)
    pool.append(0, [seq], [37], [0], empty, empty)
    torch.cuda.synchronize()
    assert torch.equal(mem.cpu(), before)
    say("empty appends: no byte changed")


def test_free_list_after_explicit_reservations():
    """Pages reserved by explicit id, released, then taken from the free list
    (also through a fork) come back once each: a sequence that takes the whole
    pool holds every page exactly once, and its tokens decode as the oracle's
    over the same block table (two logical pages on one physical page would
    overwrite each other)."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    n_pages = 8
    pool, mem = make_pool(W, n_pages, kvq.FMT_Q2, fill=0xFF)
    for _ in range(3):   # explicit reservations and releases, the last page of the stack included
        a = pool.reserve(128, pages=[0, 3])
        b = pool.reserve(64, pages=[7])
        pool.release(a)
        pool.release(b)
    k, v = kv_rows(W, 0, 0, 150)
    parent = pool.reserve(150, pages=[0, 1, 2])
    pool.append(0, [parent], [0], [150], k.cuda(), v.cuda())
    child = pool.fork(parent, 150, 300)          # shares pages 0, 1; copies page 2 into a free-list page
    assert len(set(pool.pages(child))) == 5
    pool.release(parent)
    pool.release(child)
    assert pool.stats()["free_pages"] == n_pages
    total = 64 * n_pages
    seq = pool.reserve(total)
    bt = np.array(pool.pages(seq), np.int32)
    say(f"whole-pool reservation after explicit ones: pages {list(bt)}")
    assert sorted(bt.tolist()) == list(range(n_pages)), "every page exactly once"
    assert pool.stats()["free_pages"] == 0
    with pytest.raises(kvq.KvError) as ei:
        pool.reserve(1)
    assert ei.value.name == "KV_ERR_NO_SPACE"
    k, v = kv_rows(W, 0, 1, total)
    pool.append(0, [seq], [0], [total], k.cuda(), v.cuda())
    op = opool.OraclePool("q2", 1, W.n_kv_heads, W.head_dim, n_pages, fill=0xFF)
    op.append(0, 0, bt, 0, k.float().numpy(), v.float().numpy())
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    assert np.count_nonzero(got != op.data) == 0
    q = queries(W, 0, 1)
    K, V = op.gather(0, bt, total)
    ref = attention.decode(q[0].float().numpy(), K, V, W.sm_scale)
    out = pool.decode(0, [seq], [total], q.cuda(), W.sm_scale)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy()[0], ref, "whole pool after explicit reservations")


def test_positions_beyond_2_31_refused():
    """Positions whose end would overflow are refused as out of bound before
    any byte moves."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    pool, mem = make_pool(W, 2, kvq.FMT_Q2, fill=0x5A)
    seq = pool.reserve(100)
    k, v = kv_rows(W, 0, 0, 4)
    torch.cuda.synchronize()
    before = mem.cpu().clone()
    for pos in (2 ** 31, 2 ** 63 - 2):
        with pytest.raises(kvq.KvError) as ei:
            pool.append(0, [seq], [pos], [4], k.cuda(), v.cuda())
        assert ei.value.name == "KV_ERR_BOUND"
        with pytest.raises(kvq.KvError) as ei:
            pool.prefill(0, seq, pos, queries(W, 0, 4).cuda(), W.sm_scale)
        assert ei.value.name == "KV_ERR_BOUND"
    torch.cuda.synchronize()
    assert torch.equal(mem.cpu(), before)


def test_binding_refuses_mismatched_buffers():
    """The binding checks what the C ABI takes no size for (out, scores) and
    where every buffer lives before anything is launched."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    pool, mem = make_pool(W, 4, kvq.FMT_Q2, fill=0x5A)
    seq = pool.reserve(200)
    k, v = kv_rows(W, 0, 0, 100)
    pool.append(0, [seq], [0], [100], k.cuda(), v.cuda())
    torch.cuda.synchronize()
    before = mem.cpu().clone()
    q = queries(W, 0, 1).cuda()
    ws = torch.empty(pool.workspace_bytes(kvq.OP_DECODE, 1, 2), dtype=torch.uint8, device="cuda")
    bad = [
        dict(ws=ws.cpu()),                                                   # host workspace
        dict(ws=ws, out=torch.empty((1, W.n_q_heads, W.head_dim - 1), device="cuda")),  # short out
        dict(ws=ws, out=torch.empty((1, W.n_q_heads, W.head_dim), device="cuda")[:, ::2]),  # strided
        dict(ws=ws, scores=torch.empty((1, W.n_q_heads - 1, 100), device="cuda")),    # too few score rows
        dict(ws=ws, scores=torch.empty((W.n_q_heads, 100), device="cuda")),           # not [n][Hq][stride]
    ]
    for kw in bad:
        with pytest.raises((TypeError, ValueError)):
            pool.decode(0, [seq], [100], q, W.sm_scale, n_splits=2, **kw)
    with pytest.raises(TypeError):
        pool.decode(0, [seq], [100], q.cpu(), W.sm_scale)                    # host query
    with pytest.raises(TypeError):
        pool.append(0, [seq], [100], [4], k[:4], v[:4])                      # host rows
    with pytest.raises(ValueError):
        pool.prefill(0, seq, 96, queries(W, 0, 4, stream=1).cuda(), W.sm_scale,
                     out=torch.empty((3, W.n_q_heads, W.head_dim), device="cuda"))
    with pytest.raises(ValueError):
        pool.dequant_page(0, 0, 0, 0, out=torch.empty((PAGE_TOKENS, W.head_dim + 1), device="cuda"))
    # per-sequence arrays shorter than the batch (the library takes no length
    # for them and would read past their end)
    kd, vd = k[:4].cuda(), v[:4].cuda()
    with pytest.raises(ValueError):
        pool.append(0, [seq], [100, 104], [4], kd, vd)
    with pytest.raises(ValueError):
        pool.append(0, [seq], [100], [], kd, vd)
    with pytest.raises(ValueError):
        pool.decode(0, [seq, seq], [100], torch.cat([q, q]), W.sm_scale, n_splits=2)
    with pytest.raises(ValueError):
        pool.reserve(200, pages=[0, 1])          # 200 tokens need 4 page ids
    # a scale that is not finite and positive is refused by the library
    for sm in (0.0, -W.sm_scale, float("nan"), float("inf")):
        with pytest.raises(kvq.KvError) as ei:
            pool.decode(0, [seq], [100], q, sm, n_splits=2, ws=ws)
        assert ei.value.name == "KV_ERR_ARG"
        with pytest.raises(kvq.KvError) as ei:
            pool.prefill(0, seq, 96, queries(W, 0, 4, stream=1).cuda(), sm)
        assert ei.value.name == "KV_ERR_ARG"
    torch.cuda.synchronize()
    assert torch.equal(mem.cpu(), before)
    say("binding refusals: no byte changed")


def test_block_table_is_the_reserved_pages():
    """kv_seq_block_table hands out the device array the kernels walk: read
    back from the device it lists the reserved pages in logical order."""
    need_gpu()
    import ctypes as C
    import quantized_kv_attention_append_amd as kvq
    hip = C.CDLL("libamdhip64.so")
    pool, mem = make_pool(W, 12, kvq.FMT_Q2, fill=0x5A, max_seqs=3)
    a = pool.reserve(200, pages=[7, 2, 9, 4])
    b = pool.reserve(130)
    for seq, want in ((a, [7, 2, 9, 4]), (b, pool.pages(b))):
        ptr, n = pool.block_table(seq)
        assert n == len(want) and ptr
        host = (C.c_int32 * n)()
        assert hip.hipMemcpy(host, C.c_void_p(ptr), C.c_size_t(4 * n), 2) == 0  # device to host
        assert list(host) == list(want)
    assert len(set(pool.pages(b)) & {7, 2, 9, 4}) == 0
    pool.release(a)
    with pytest.raises(kvq.KvError) as ei:
        pool.block_table(a)
    assert ei.value.name == "KV_ERR_ARG"


def test_pool_dropped_inside_a_graph_capture():
    """A pool dropped while a HIP graph is captured on the current stream (as
    the garbage collector may do at any allocation) neither breaks the capture
    nor leaks: its destruction waits for the next pool creation outside it."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    pool, mem = make_pool(W, 4, kvq.FMT_Q2)
    seq = pool.reserve(128)
    k, v = kv_rows(W, 0, 0, 100)
    pool.append(0, [seq], [0], [100], k.cuda(), v.cuda())
    q = queries(W, 0, 1).cuda()
    ws = torch.empty(pool.workspace_bytes(kvq.OP_DECODE, 1, 2), dtype=torch.uint8, device="cuda")
    out = torch.empty((1, W.n_q_heads, W.head_dim), dtype=torch.float32, device="cuda")
    pool.decode(0, [seq], [100], q, W.sm_scale, n_splits=2, ws=ws, out=out)
    torch.cuda.synchronize()
    eager = out.clone()
    doomed, _ = make_pool(W, 2, kvq.FMT_Q2)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pool.decode(0, [seq], [100], q, W.sm_scale, n_splits=2, ws=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        pool.decode(0, [seq], [100], q, W.sm_scale, n_splits=2, ws=ws, out=out)
        del doomed                                   # destroyed here: deferred
    assert len(kvq._deferred) == 1
    for _ in range(2):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    fresh, _ = make_pool(W, 2, kvq.FMT_Q2)          # outside the capture: the deferred pool goes
    assert not kvq._deferred
    fresh.close()
    say("pool dropped inside a capture: capture intact, destroyed afterwards")
