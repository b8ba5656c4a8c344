"""GPU parity, compressed-read chunked prefill (2-bit): the chunk is
quantize-appended after the prior tokens, then each chunk query attends
causally to every token up to its own position, all read from the pool.
Compared with the fp64 oracle; the workspace is pre-filled with 0xFF (NaN as
fp32), so any read of an unwritten byte would show."""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import WORKLOADS, Workload, kv_rows, page_permutation, queries
from tests.gpu_helpers import assert_close, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny"]
PREFILL = WORKLOADS["prefill"]
SMALL128 = Workload(90, "small D=128 geometry", "q2", 2, 2, 128, 8, 3, 300)


def _prefill_case(w, layer, prior, n_q, splits_list, salt=0, qscale=1.0):
    import quantized_kv_attention_append_amd as kvq
    total = prior + n_q
    n_pages = -(-total // 64) + 1
    pool, mem = make_pool(w, n_pages, kvq.FMT_Q2)
    bt = page_permutation(w, n_pages, salt=salt)[:-1]
    seq = pool.reserve(total, pages=bt)
    k, v = kv_rows(w, layer, 0, total)
    if prior:
        pool.append(layer, [seq], [0], [prior], k[:prior].cuda(), v[:prior].cuda())
    pool.append(layer, [seq], [prior], [n_q], k[prior:].cuda(), v[prior:].cuda())
    q = queries(w, layer, n_q, stream=1)
    if qscale != 1.0:
        q = (q.float() * qscale).to(torch.bfloat16)
    K, V = opool.dequantized_rows("q2", k.float().numpy(), v.float().numpy())
    ref = attention.prefill(q.float().numpy(), K, V, w.sm_scale, q_start=prior)
    outs = []
    for sp in splits_list:
        ws = torch.full((pool.workspace_bytes(kvq.OP_PREFILL, n_q, sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.prefill(layer, seq, prior, q.cuda(), w.sm_scale, n_splits=sp, ws=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, f"prefill prior={prior} n_q={n_q} splits={sp} q x {qscale:g}")
        outs.append(out.cpu())
    return pool, seq, q, outs


def test_prefill_small_d256_splits():
    need_gpu()
    _prefill_case(TINY, 0, 100, 45, [1, 2, 3, 0])


def test_prefill_small_d256_chunk_from_zero():
    need_gpu()
    _prefill_case(TINY, 0, 0, 77, [1, 2])


def test_prefill_d128_group4():
    need_gpu()
    _prefill_case(SMALL128, 1, 130, 64, [1, 4])


@pytest.mark.parametrize("qscale", [64.0, 1.0 / 64.0])
def test_prefill_peaked_and_flat(qscale):
    """Queries scaled by 64 (a sharply peaked softmax, the lazily rescaled
    reference moving often) and by 1/64 (nearly flat weights), at 256 and 128
    dims, against the oracle's fp64 causal attention."""
    need_gpu()
    _prefill_case(TINY, 0, 300, 70, [1, 2, 0], salt=5, qscale=qscale)
    _prefill_case(SMALL128, 1, 200, 100, [1, 0], salt=6, qscale=qscale)


def test_prefill_last_row_equals_decode():
    need_gpu()
    pool, seq, q, outs = _prefill_case(TINY, 0, 192, 33, [2], salt=4)
    dec = pool.decode(0, [seq], [192 + 33], q[-1:].cuda(), TINY.sm_scale, n_splits=1).cpu()
    # two independent GPU paths, each within ~1e-4 of the oracle: compared at the same bar
    assert_close(outs[0][-1].numpy(), dec[0].numpy().astype(np.float64), "last prefill row vs decode")


def test_prefill_refuses_bad_calls():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    pool, mem = make_pool(TINY, 4, kvq.FMT_Q2)
    seq = pool.reserve(128)
    q = queries(TINY, 0, 10).cuda()
    with pytest.raises(kvq.KvError) as ei:
        pool.prefill(0, seq, 0, q, TINY.sm_scale, n_splits=2, ws=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert ei.value.name == "KV_ERR_WORKSPACE"
    with pytest.raises(kvq.KvError) as ei:
        pool.prefill(0, seq, 120, q, TINY.sm_scale)   # 130 > bound of 128
    assert ei.value.name == "KV_ERR_BOUND"
    w8 = Workload(93, "8-bit", "q8", 1, 4, 128, 16, 1, 64)
    p8, _ = make_pool(w8, 2, kvq.FMT_Q8)
    s8 = p8.reserve(64)
    with pytest.raises(kvq.KvError) as ei:
        p8.prefill(0, s8, 0, torch.zeros((4, 16, 128), dtype=torch.bfloat16, device="cuda"), 0.1)
    assert ei.value.name == "KV_ERR_FORMAT"


@pytest.mark.timeout(900)
def test_c3_chunked_prefill_full_size():
    """65,536 prior tokens + a 1,024-token chunk (1 layer, 4 KV heads x 256, 16
    query heads): the whole 38.3 MB pool byte for byte against the oracle's
    image, and every one of the 1,024 x 16 output rows against the oracle's
    causal prefill (one fp64 product per head)."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    w = PREFILL
    prior, n_q = w.ctx, w.chunk
    total = prior + n_q
    n_pages = total // 64
    pool, mem = make_pool(w, n_pages, kvq.FMT_Q2, max_seqs=1, max_seq_tokens=total)
    perm = page_permutation(w, n_pages)
    seq = pool.reserve(total, pages=perm)
    k, v = kv_rows(w, 0, 0, total, device="cuda")
    pool.append(0, [seq], [0], [prior], k[:prior], v[:prior])
    pool.append(0, [seq], [prior], [n_q], k[prior:], v[prior:])
    q = queries(w, 0, n_q, device="cuda", stream=1)
    ws = torch.full((pool.workspace_bytes(kvq.OP_PREFILL, n_q, 0),), 0xFF, dtype=torch.uint8, device="cuda")
    out = pool.prefill(0, seq, prior, q, w.sm_scale, ws=ws).cpu().numpy()
    assert np.all(np.isfinite(out))
    kf, vf = k.float().cpu().numpy(), v.float().cpu().numpy()
    blocks = opool.sequence_blocks("q2", kf, vf)
    got = mem.view(n_pages, -1)[torch.as_tensor(perm.astype(np.int64), device="cuda")].cpu().numpy()
    bad = int(np.count_nonzero(got != blocks.reshape(n_pages, -1)))
    assert bad == 0, f"65536 + 1024: {bad} pool bytes differ from the oracle"
    K, V = opool.dequantized_rows("q2", kf, vf)
    ref = attention.prefill_dense(q.float().cpu().numpy(), K, V, w.sm_scale, prior)
    assert_close(out, ref, "65536 + 1024 chunk, all 1024 rows x 16 heads")
    say("PREFILL prefill: the whole pool bit-exact, every chunk row within tolerance")


@pytest.mark.timeout(900)
def test_c3_chunked_prefill_full_size_rotated():
    """The 65,536 + 1,024 chunk over a rotated 2-bit pool: the whole pool byte
    for byte against the oracle's image (the 2-bit pages of the rotated K rows
    and of the V rows), and every chunk row against the oracle's causal
    prefill over the pool read back in the original basis."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    from oracle import codec
    w = PREFILL
    prior, n_q = w.ctx, w.chunk
    total = prior + n_q
    n_pages = total // 64
    pool, mem = make_pool(w, n_pages, kvq.FMT_Q2_ROT, max_seqs=1, max_seq_tokens=total)
    perm = page_permutation(w, n_pages)
    seq = pool.reserve(total, pages=perm)
    k, v = kv_rows(w, 0, 0, total, device="cuda")
    pool.append(0, [seq], [0], [prior], k[:prior], v[:prior])
    pool.append(0, [seq], [prior], [n_q], k[prior:], v[prior:])
    q = queries(w, 0, n_q, device="cuda", stream=1)
    ws = torch.full((pool.workspace_bytes(kvq.OP_PREFILL, n_q, 0),), 0xFF, dtype=torch.uint8, device="cuda")
    out = pool.prefill(0, seq, prior, q, w.sm_scale, ws=ws).cpu().numpy()
    assert np.all(np.isfinite(out))
    kf, vf = k.float().cpu().numpy(), v.float().cpu().numpy()
    blocks = opool.sequence_blocks("q2", codec.hadamard_rows(kf), vf)
    got = mem.view(n_pages, -1)[torch.as_tensor(perm.astype(np.int64), device="cuda")].cpu().numpy()
    bad = int(np.count_nonzero(got != blocks.reshape(n_pages, -1)))
    assert bad == 0, f"rotated 65536 + 1024: {bad} pool bytes differ from the oracle"
    K, V = opool.dequantized_rows("q2r", kf, vf)
    ref = attention.prefill_dense(q.float().cpu().numpy(), K, V, w.sm_scale, prior)
    assert_close(out, ref, "rotated 65536 + 1024 chunk, all 1024 rows x 16 heads")
