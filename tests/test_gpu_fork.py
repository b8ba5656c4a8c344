"""GPU parity, prefix sharing (kv_seq_fork): a child sequence shares the
parent's whole pages and gets a copy of the page its prefix only partly fills.
After the child and the parent each append their own continuation, the whole
pool image equals the oracle's bit for bit (shared pages untouched, the copied
page carried on by the child), both decode within tolerance of the oracle,
page accounting counts shared pages once, and appends into shared pages are
refused with the pool unchanged."""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import Workload, kv_rows, queries
from tests.gpu_helpers import assert_close, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

NAN_FILL = 0xFF
FMTS = {"q2": 1, "q8": 2, "bf16": 3, "q2w": 4, "q2r": 5}


def _w(fmt):
    # 2 layers x 4 KV heads x 128 dims, 16 query heads: every format, multi-layer copies
    return Workload(99, f"fork, {fmt}", fmt, 2, 4, 128, 16, 2, 260)


def _append(pool, op, w, seq, oseq, bt, k, v, start, end):
    for layer in range(w.n_layers):
        pool.append(layer, [seq], [start], [end - start], k[layer][start:end].cuda(), v[layer][start:end].cuda())
        op.append(layer, oseq, bt, start, k[layer][start:end].float().numpy(), v[layer][start:end].float().numpy())


@pytest.mark.parametrize("fmt", ["q2", "q8", "bf16", "q2w", "q2r"])
@pytest.mark.parametrize("n", [150, 128])
def test_fork_then_both_continue(fmt, n):
    need_gpu()
    w = _w(fmt)
    n_pages = 12
    pool, mem = make_pool(w, n_pages, FMTS[fmt], fill=NAN_FILL)
    op = opool.OraclePool(fmt, w.n_layers, w.n_kv_heads, w.head_dim, n_pages, fill=NAN_FILL)
    kp = [kv_rows(w, layer, 0, 260)[0] for layer in range(2)]
    vp = [kv_rows(w, layer, 0, 260)[1] for layer in range(2)]
    kc = [torch.cat([kp[layer][:n], kv_rows(w, layer, 1, 260)[0][n:]]) for layer in range(2)]
    vc = [torch.cat([vp[layer][:n], kv_rows(w, layer, 1, 260)[1][n:]]) for layer in range(2)]
    parent = pool.reserve(260)
    pbt = np.array(pool.pages(parent), np.int32)
    _append(pool, op, w, parent, 0, pbt, kp, vp, 0, 100)
    _append(pool, op, w, parent, 0, pbt, kp, vp, 100, n)
    free0 = pool.stats()["free_pages"]
    child = pool.fork(parent, n, 240)
    cbt = np.array(pool.pages(child), np.int32)
    assert list(cbt[:n // 64]) == list(pbt[:n // 64]), "whole pages are shared"
    assert len(set(cbt[n // 64:]) & set(pbt)) == 0, "the rest of the child's pages are its own"
    assert pool.stats()["free_pages"] == free0 - (len(cbt) - n // 64)
    op.fork(0, pbt, 1, cbt, n)
    q = queries(w, 0, 2)
    # the child reads the parent's prefix right after the fork
    for layer in range(2):
        K, V = op.gather(layer, cbt, n, seq=1)
        ref = attention.decode(q[0].float().numpy(), K, V, w.sm_scale)
        out = pool.decode(layer, [child], [n], q[:1].cuda(), w.sm_scale)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy()[0], ref, f"{fmt} n={n} layer={layer}: child at the fork")
    _append(pool, op, w, child, 1, cbt, kc, vc, n, 230)
    _append(pool, op, w, parent, 0, pbt, kp, vp, n, 260)
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"{fmt} fork n={n}: {diff} differing pool bytes of {got.size}")
    assert diff == 0
    for layer in range(2):
        refs = []
        for oseq, bt, ctx, qi in ((1, cbt, 230, 0), (0, pbt, 260, 1)):
            K, V = op.gather(layer, bt, ctx, seq=oseq)
            refs.append(attention.decode(q[qi].float().numpy(), K, V, w.sm_scale))
        out = pool.decode(layer, [child, parent], [230, 260], q.cuda(), w.sm_scale)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), np.stack(refs), f"{fmt} n={n} layer={layer}: child and parent")
    # accounting: a shared page is reserved once and freed by its last holder
    st = pool.stats()
    assert st["reserved_pages"] == len(set(cbt) | set(pbt))
    pool.release(parent)
    assert pool.stats()["reserved_pages"] == len(cbt)
    pool.release(child)
    assert pool.stats()["free_pages"] == n_pages


def test_fork_refusals_before_any_byte_moves():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    w = _w("q2")
    pool, mem = make_pool(w, 10, FMTS["q2"], fill=NAN_FILL)
    k, v = kv_rows(w, 0, 0, 200)
    parent = pool.reserve(200)
    for layer in range(2):
        pool.append(layer, [parent], [0], [150], k[:150].cuda(), v[:150].cuda())
    with pytest.raises(kvq.KvError) as ei:   # beyond the tokens appended
        pool.fork(parent, 151, 200)
    assert ei.value.name == "KV_ERR_ARG"
    child = pool.fork(parent, 150, 200)
    torch.cuda.synchronize()
    before = mem.cpu().clone()
    with pytest.raises(kvq.KvError) as ei:   # the child may not write into a shared page
        pool.append(0, [child], [60], [10], k[60:70].cuda(), v[60:70].cuda())
    assert ei.value.name == "KV_ERR_ARG"
    with pytest.raises(kvq.KvError) as ei:   # nor may the parent
        pool.append(1, [parent], [120], [10], k[120:130].cuda(), v[120:130].cuda())
    assert ei.value.name == "KV_ERR_ARG"
    with pytest.raises(kvq.KvError) as ei:   # not enough free pages for a third sequence's bound
        pool.fork(child, 150, 64 * 9)
    assert ei.value.name == "KV_ERR_NO_SPACE"
    torch.cuda.synchronize()
    assert torch.equal(mem.cpu(), before)
    # 8-bit: a fork takes every token appended so far
    w8 = _w("q8")
    p8, _ = make_pool(w8, 6, FMTS["q8"])
    s8 = p8.reserve(200)
    for layer in range(2):
        p8.append(layer, [s8], [0], [100], k[:100].cuda(), v[:100].cuda())
    with pytest.raises(kvq.KvError) as ei:
        p8.fork(s8, 90, 200)
    assert ei.value.name == "KV_ERR_ARG"
