"""GPU parity, the Hadamard-rotated 2-bit variant: pages bit-exact against
the oracle's image (K rows are rotated in fp32 butterflies before the 2-bit
codec, so the codes are a pure function of the bf16 inputs; V rows are the
2-bit format's), decode within tolerance of the fp64 oracle that reads K back
in the original basis, raw scores against the oracle's, and the refusals the
format documents."""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import WORKLOADS, Workload, kv_rows, page_permutation, queries
from tests.gpu_helpers import assert_close, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny"]
# 2 layers x 2 KV heads x 128 dims, 8 query heads (group 4)
SMALL128 = Workload(91, "rotated, D=128", "q2r", 2, 2, 128, 8, 3, 300)
NAN_FILL = 0xFF


def _fmt():
    import quantized_kv_attention_append_amd as kvq
    return kvq.FMT_Q2_ROT


def test_rotated_append_bit_exact_d256():
    need_gpu()
    n_pages = 6
    pool, mem = make_pool(TINY, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(TINY, n_pages)[:4]
    seq = pool.reserve(256, pages=bt)
    k, v = kv_rows(TINY, 0, 0, 256)
    op = opool.OraclePool("q2r", 1, 4, 256, n_pages, fill=NAN_FILL)
    start = 0
    for n in (100, 1, 27, 64, 64):
        pool.append(0, [seq], [start], [n], k[start:start + n].cuda(), v[start:start + n].cuda())
        op.append(0, 0, bt, start, k[start:start + n].float().numpy(), v[start:start + n].float().numpy())
        start += n
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"rotated append D=256: {diff} differing bytes of {got.size}")
    assert diff == 0


def test_rotated_append_batched_d128_bit_exact():
    need_gpu()
    w = SMALL128
    n_pages = 20
    pool, mem = make_pool(w, n_pages, _fmt(), fill=NAN_FILL)
    perm = page_permutation(w, n_pages)
    lens = [300, 65, 130]
    bts, seqs, off = [], [], 0
    for L in lens:
        npg = -(-L // 64)
        bts.append(perm[off:off + npg]); off += npg
        seqs.append(pool.reserve(L, pages=bts[-1]))
    op = opool.OraclePool("q2r", 2, 2, 128, n_pages, fill=NAN_FILL)
    for layer in range(2):
        rows = [kv_rows(w, layer, i, lens[i]) for i in range(3)]
        ks = torch.cat([r[0] for r in rows])
        vs = torch.cat([r[1] for r in rows])
        pool.append(layer, seqs, [0, 0, 0], lens, ks.cuda(), vs.cuda())
        for i in range(3):
            op.append(layer, i, bts[i], 0, rows[i][0].float().numpy(), rows[i][1].float().numpy())
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"rotated batched append D=128: {diff} differing bytes of {got.size}")
    assert diff == 0


@pytest.mark.parametrize("ctx", [1, 63, 65, 200, 1000])
def test_rotated_decode_ragged(ctx):
    need_gpu()
    n_pages = -(-ctx // 64) + 2
    pool, mem = make_pool(TINY, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(TINY, n_pages, salt=ctx)[:-2]
    seq = pool.reserve(ctx, pages=bt)
    k, v = kv_rows(TINY, 0, 0, ctx)
    pool.append(0, [seq], [0], [ctx], k.cuda(), v.cuda())
    q = queries(TINY, 0, 1, stream=ctx)
    K, V = opool.dequantized_rows("q2r", k.float().numpy(), v.float().numpy())
    qn = q[0].float().numpy()
    ref = attention.decode(qn, K, V, TINY.sm_scale)
    ref_s = attention.scores(qn, K, TINY.sm_scale)
    for sp in (1, 3, 0):
        scores = torch.full((1, TINY.n_q_heads, ctx), float("nan"), device="cuda")
        ws = torch.full((pool.workspace_bytes(0, 1, sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.decode(0, [seq], [ctx], q.cuda(), TINY.sm_scale, n_splits=sp, ws=ws, scores=scores)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy()[0], ref, f"rotated decode ctx={ctx} splits={sp}")
        # raw scores: a check of the library's own, beside the output tolerance.
        # The rotated score is sm / D (H q) . x^_r: the query passes through
        # eight fp32 butterfly stages and its fixed-point digits are taken at
        # the rotated row's larger magnitude, so the bar is 5e-5 here against
        # 1e-5 for the plain 2-bit scores (1.8e-5 measured at ctx = 200).
        s = scores.cpu().numpy()[0].astype(np.float64)
        rel = np.linalg.norm(s - ref_s) / np.linalg.norm(ref_s)
        assert rel <= 5e-5, f"rotated scores ctx={ctx} splits={sp}: rel L2 {rel:.2e}"


@pytest.mark.parametrize("qscale", [64.0, 1.0 / 64.0])
def test_rotated_decode_peaked_and_flat(qscale):
    """The rotated decode with queries scaled by 64 (a sharply peaked softmax)
    and by 1/64 (nearly flat weights): the query's fp32 butterflies and its
    fixed-point digits against the oracle's fp64 attention over the rotated
    rows."""
    need_gpu()
    ctx = 700
    n_pages = -(-ctx // 64) + 1
    pool, mem = make_pool(TINY, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(TINY, n_pages, salt=31)[:-1]
    seq = pool.reserve(ctx, pages=bt)
    k, v = kv_rows(TINY, 0, 0, ctx)
    pool.append(0, [seq], [0], [ctx], k.cuda(), v.cuda())
    q = (queries(TINY, 0, 1, stream=3).float() * qscale).to(torch.bfloat16)
    K, V = opool.dequantized_rows("q2r", k.float().numpy(), v.float().numpy())
    ref = attention.decode(q[0].float().numpy(), K, V, TINY.sm_scale)
    for sp in (1, 3, 0):
        out = pool.decode(0, [seq], [ctx], q.cuda(), TINY.sm_scale, n_splits=sp)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy()[0], ref, f"rotated decode q x {qscale:g} splits={sp}")


def test_rotated_decode_batch_d128():
    need_gpu()
    w = SMALL128
    lens = [300, 65, 130]
    n_pages = sum(-(-L // 64) for L in lens)
    pool, mem = make_pool(w, n_pages, _fmt(), fill=NAN_FILL)
    perm = page_permutation(w, n_pages)
    seqs, off, refs = [], 0, []
    q = queries(w, 1, len(lens))
    for i, L in enumerate(lens):
        npg = -(-L // 64)
        seqs.append(pool.reserve(L, pages=perm[off:off + npg])); off += npg
        k, v = kv_rows(w, 1, i, L)
        pool.append(1, [seqs[-1]], [0], [L], k.cuda(), v.cuda())
        K, V = opool.dequantized_rows("q2r", k.float().numpy(), v.float().numpy())
        refs.append(attention.decode(q[i].float().numpy(), K, V, w.sm_scale))
    for sp in (1, 2, 0):
        out = pool.decode(1, seqs, lens, q.cuda(), w.sm_scale, n_splits=sp)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), np.stack(refs), f"rotated batch D=128 splits={sp}")


def test_rotated_lowers_the_decode_error_against_the_exact_rows():
    """Against attention over the exact bf16 rows, the rotated pool's decode
    error on the outlier-bearing synthetic rows is below the plain 2-bit
    pool's (the quality reason for the variant), measured on the GPU output."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    ctx = 1024
    errs = {}
    k, v = kv_rows(TINY, 0, 0, ctx)
    q = queries(TINY, 0, 1, stream=5)
    exact = attention.decode(q[0].float().numpy(), k.float().numpy(), v.float().numpy(), TINY.sm_scale)
    for name, fmt in (("q2", kvq.FMT_Q2), ("q2r", kvq.FMT_Q2_ROT)):
        pool, _ = make_pool(TINY, ctx // 64, fmt)
        seq = pool.reserve(ctx)
        pool.append(0, [seq], [0], [ctx], k.cuda(), v.cuda())
        out = pool.decode(0, [seq], [ctx], q.cuda(), TINY.sm_scale)
        torch.cuda.synchronize()
        o = out.cpu().numpy()[0].astype(np.float64)
        errs[name] = np.linalg.norm(o - exact) / np.linalg.norm(exact)
    say(f"decode rel L2 against exact rows: 2-bit {errs['q2']:.3e}, rotated {errs['q2r']:.3e}")
    assert errs["q2r"] < errs["q2"]


def _rotated_prefill_case(w, layer, prior, n_q, splits_list, salt=0):
    """Prefill over a rotated pool against the oracle's attention over the
    rotated pool read back in the original basis (rows are the pages of a
    seeded permutation; the workspace is filled with 0xFF)."""
    import quantized_kv_attention_append_amd as kvq
    total = prior + n_q
    n_pages = -(-total // 64) + 1
    pool, mem = make_pool(w, n_pages, _fmt())
    bt = page_permutation(w, n_pages, salt=salt)[:-1]
    seq = pool.reserve(total, pages=bt)
    k, v = kv_rows(w, layer, 0, total)
    if prior:
        pool.append(layer, [seq], [0], [prior], k[:prior].cuda(), v[:prior].cuda())
    pool.append(layer, [seq], [prior], [n_q], k[prior:].cuda(), v[prior:].cuda())
    q = queries(w, layer, n_q, stream=1)
    K, V = opool.dequantized_rows("q2r", k.float().numpy(), v.float().numpy())
    ref = attention.prefill(q.float().numpy(), K, V, w.sm_scale, q_start=prior)
    for sp in splits_list:
        ws = torch.full((pool.workspace_bytes(kvq.OP_PREFILL, n_q, sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.prefill(layer, seq, prior, q.cuda(), w.sm_scale, n_splits=sp, ws=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, f"rotated prefill {w.name} prior={prior} n_q={n_q} splits={sp}")


def test_rotated_prefill_small():
    need_gpu()
    _rotated_prefill_case(TINY, 0, 100, 45, [1, 2, 3, 0])
    _rotated_prefill_case(TINY, 0, 0, 77, [1, 2])


@pytest.mark.parametrize("w", [Workload(96, "rotated prefill, D=128 group 4", "q2r", 2, 2, 128, 8, 1, 300),
                               Workload(96, "rotated prefill, D=256 group 2", "q2r", 1, 4, 256, 8, 1, 300),
                               Workload(96, "rotated prefill, D=128 group 8", "q2r", 1, 2, 128, 16, 1, 300)],
                         ids=lambda w: w.name)
def test_rotated_prefill_geometries(w):
    need_gpu()
    _rotated_prefill_case(w, w.n_layers - 1, 130, 64, [1, 4, 0], salt=3)


def test_rotated_prefill_last_row_equals_decode():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    prior, n_q = 200, 40
    pool, mem = make_pool(TINY, 5, _fmt())
    seq = pool.reserve(prior + n_q)
    k, v = kv_rows(TINY, 0, 0, prior + n_q)
    pool.append(0, [seq], [0], [prior + n_q], k.cuda(), v.cuda())
    q = queries(TINY, 0, n_q, stream=1).cuda()
    out = pool.prefill(0, seq, prior, q, TINY.sm_scale)
    dec = pool.decode(0, [seq], [prior + n_q], q[-1:].contiguous(), TINY.sm_scale)
    torch.cuda.synchronize()
    K, V = opool.dequantized_rows("q2r", k.float().numpy(), v.float().numpy())
    ref = attention.decode(q[-1].float().cpu().numpy(), K, V, TINY.sm_scale)
    assert_close(out[-1].cpu().numpy(), ref, "rotated prefill last row against the oracle's decode")
    assert_close(dec[0].cpu().numpy(), ref, "rotated decode at the same length against the oracle")
    assert_close(out[-1].cpu().numpy(), dec[0].cpu().numpy().astype(np.float64), "rotated prefill last row vs decode")


@pytest.mark.parametrize("w", [Workload(94, "rotated, group 8, D=128", "q2r", 1, 2, 128, 16, 2, 300),
                               Workload(94, "rotated, group 1, D=256", "q2r", 1, 4, 256, 4, 2, 300)],
                         ids=lambda w: w.name)
def test_rotated_decode_other_groups(w):
    need_gpu()
    lens = [300, 97]
    n_pages = sum(-(-n // 64) for n in lens)
    pool, mem = make_pool(w, n_pages, _fmt())
    seqs, refs = [], []
    q = queries(w, 0, len(lens))
    for i, n in enumerate(lens):
        seqs.append(pool.reserve(n))
        k, v = kv_rows(w, 0, i, n)
        pool.append(0, [seqs[-1]], [0], [n], k.cuda(), v.cuda())
        K, V = opool.dequantized_rows("q2r", k.float().numpy(), v.float().numpy())
        refs.append(attention.decode(q[i].float().numpy(), K, V, w.sm_scale))
    out = pool.decode(0, seqs, lens, q.cuda(), w.sm_scale, n_splits=2)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), np.stack(refs), w.name)
