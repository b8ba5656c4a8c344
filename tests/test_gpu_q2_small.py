"""GPU parity, 2-bit format, small shapes: append bit-exact against the oracle's
pool image, page dequantization bit-exact, decode within tolerance of the fp64
oracle (tiny decode workload: 1 layer, 4 KV heads x 256, 16 query heads,
256 tokens on a seeded permutation of 4 pages)."""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import WORKLOADS, Workload, kv_rows, page_permutation, queries
from tests.gpu_helpers import assert_close, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny"]
# a second geometry: 2 layers x 2 KV heads x 128 dims, 8 query heads
SMALL128 = Workload(90, "small D=128 geometry", "q2", 2, 2, 128, 8, 3, 300)


def _append_both(pool, op, layer, seq_ids, bts, chunks, k_all, v_all):
    """Append the same ragged chunks through the library and the oracle."""
    starts = {s: 0 for s in seq_ids}
    for chunk in chunks:  # chunk: list of (seq index, n)
        seqs, st, nn, ks, vs = [], [], [], [], []
        for i, n in chunk:
            s0 = starts[seq_ids[i]]
            seqs.append(seq_ids[i]); st.append(s0); nn.append(n)
            ks.append(k_all[i][s0:s0 + n]); vs.append(v_all[i][s0:s0 + n])
            op.append(layer, i, bts[i], s0, k_all[i][s0:s0 + n].float().numpy(), v_all[i][s0:s0 + n].float().numpy())
            starts[seq_ids[i]] += n
        pool.append(layer, seqs, st, nn, torch.cat(ks).cuda(), torch.cat(vs).cuda())


def test_append_q2_tiny_bit_exact():
    need_gpu()
    n_pages = 6
    pool, mem = make_pool(TINY, n_pages, 1)
    bt = page_permutation(TINY, n_pages)[:4]
    seq = pool.reserve(256, pages=bt)
    assert pool.pages(seq) == list(bt)
    k, v = kv_rows(TINY, 0, 0, 256)
    op = opool.OraclePool("q2", 1, 4, 256, n_pages)
    _append_both(pool, op, 0, [seq], [bt], [[(0, 100)], [(0, 1)], [(0, 27)], [(0, 64)], [(0, 64)]], [k], [v])
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"tiny append: {diff} differing bytes of {got.size}")
    assert diff == 0
    st = pool.stats()
    assert st["used_pages"] == 4 and st["reserved_pages"] == 4 and st["free_pages"] == 2


def test_append_q2_half_step_rows_bit_exact():
    """Rows whose values sit on half steps of the code grid, x = lo + (k/2) s
    with s a power of two: every odd k is a tie of the rounding to a code
    (round half to even), the case where the quotient must be the correctly
    rounded one."""
    need_gpu()
    w = TINY
    n_pages = 3
    pool, mem = make_pool(w, n_pages, 1)
    bt = page_permutation(w, n_pages, salt=5)[:2]
    seq = pool.reserve(128, pages=bt)
    rng = np.random.default_rng(1234)
    rows = []
    for _ in range(2 * 128 * w.n_kv_heads):
        s = 2.0 ** int(rng.integers(-4, 3))
        m = int(rng.integers(-40, 40))
        k = rng.integers(0, 7, size=w.head_dim)
        k[int(rng.integers(0, w.head_dim))] = 0
        k[int(rng.integers(0, w.head_dim))] = 6
        rows.append((m + k) * s / 2)
    x = torch.tensor(np.array(rows, np.float32)).to(torch.bfloat16)   # exact: |m + k| < 256
    assert torch.equal(x.float(), torch.tensor(np.array(rows, np.float32)))
    x = x.view(2, 128, w.n_kv_heads, w.head_dim)
    k_all, v_all = x[0], x[1]
    op = opool.OraclePool("q2", 1, w.n_kv_heads, w.head_dim, n_pages)
    _append_both(pool, op, 0, [seq], [bt], [[(0, 70)], [(0, 58)]], [k_all], [v_all])
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"half-step rows: {diff} differing bytes of {got.size}")
    assert diff == 0


def test_append_q2_batched_ragged_d128_bit_exact():
    need_gpu()
    w = SMALL128
    n_pages = 20
    pool, mem = make_pool(w, n_pages, 1)
    perm = page_permutation(w, n_pages)
    lens = [300, 65, 130]
    bts, seq_ids, ks, vs = [], [], [], []
    off = 0
    for i, L in enumerate(lens):
        npg = -(-L // 64)
        bts.append(perm[off:off + npg]); off += npg
        seq_ids.append(pool.reserve(L, pages=bts[-1]))
    op = opool.OraclePool("q2", 2, 2, 128, n_pages)
    for layer in range(2):
        ks = [kv_rows(w, layer, i, lens[i])[0] for i in range(3)]
        vs = [kv_rows(w, layer, i, lens[i])[1] for i in range(3)]
        chunks = [[(0, 37), (1, 1), (2, 64)], [(0, 200), (2, 66)], [(0, 63), (1, 64)]]
        _append_both(pool, op, layer, seq_ids, bts, chunks, ks, vs)
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"batched append: {diff} differing bytes of {got.size}")
    assert diff == 0


def test_dequant_page_bit_exact():
    need_gpu()
    n_pages = 6
    pool, mem = make_pool(TINY, n_pages, 1, fill=0)
    bt = page_permutation(TINY, n_pages)[:4]
    seq = pool.reserve(256, pages=bt)
    k, v = kv_rows(TINY, 0, 0, 256)
    pool.append(0, [seq], [0], [256], k.cuda(), v.cuda())
    K, V = opool.dequantized_rows("q2", k.float().numpy(), v.float().numpy())
    for lp in range(4):
        for h in (0, 3):
            gk = pool.dequant_page(int(bt[lp]), 0, h, 0).cpu().numpy()
            gv = pool.dequant_page(int(bt[lp]), 0, h, 1).cpu().numpy()
            assert np.array_equal(gk.view(np.uint32), K[64 * lp:64 * lp + 64, h].view(np.uint32))
            assert np.array_equal(gv.view(np.uint32), V[64 * lp:64 * lp + 64, h].view(np.uint32))


def _decode_case(w, ctx, splits_list, layer=0):
    n_pages = -(-ctx // 64) + 2
    pool, mem = make_pool(w, n_pages, 1)
    bt = page_permutation(w, n_pages, salt=ctx)[:-(2)]
    seq = pool.reserve(ctx, pages=bt)
    k, v = kv_rows(w, layer, 0, ctx)
    pool.append(layer, [seq], [0], [ctx], k.cuda(), v.cuda())
    q = queries(w, layer, 1)
    K, V = opool.dequantized_rows("q2", k.float().numpy(), v.float().numpy())
    ref = attention.decode(q[0].float().numpy(), K, V, w.sm_scale)
    ref_s = attention.scores(q[0].float().numpy(), K, w.sm_scale)
    outs = []
    for sp in splits_list:
        scores = torch.full((1, w.n_q_heads, ctx), float("nan"), device="cuda")
        ws = torch.full((pool.workspace_bytes(0, 1, sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.decode(layer, [seq], [ctx], q.cuda(), w.sm_scale, n_splits=sp, ws=ws, scores=scores)
        torch.cuda.synchronize()
        assert_close(out[0].cpu().numpy(), ref, f"decode ctx={ctx} splits={sp}")
        assert_close(scores[0].cpu().numpy(), ref_s, f"scores ctx={ctx} splits={sp}", max_abs=2e-3, rel_l2=1e-5)
        outs.append(out.cpu())
    return outs


def test_decode_q2_tiny():
    need_gpu()
    _decode_case(TINY, 256, [1, 2, 3, 0])


@pytest.mark.parametrize("ctx", [1, 63, 65, 200, 1000])
def test_decode_q2_ragged_lengths(ctx):
    need_gpu()
    _decode_case(TINY, ctx, [1, 4])


@pytest.mark.parametrize("qscale", [64.0, 1.0 / 64.0])
def test_decode_q2_peaked_and_flat(qscale):
    """Queries scaled by 64 (a softmax concentrated on a few tokens, most
    weights far below their block's largest) and by 1/64 (nearly flat
    weights), at 256 and 128 dims: the fixed-point query digits and the 16-bit
    weight digits of the decode kernel against the oracle's fp64 attention."""
    need_gpu()
    for w, ctx in ((TINY, 700), (SMALL128, 450)):
        n_pages = -(-ctx // 64) + 1
        pool, mem = make_pool(w, n_pages, 1)
        bt = page_permutation(w, n_pages, salt=29)[:-1]
        seq = pool.reserve(ctx, pages=bt)
        k, v = kv_rows(w, 0, 0, ctx)
        pool.append(0, [seq], [0], [ctx], k.cuda(), v.cuda())
        q = (queries(w, 0, 1).float() * qscale).to(torch.bfloat16)
        K, V = opool.dequantized_rows("q2", k.float().numpy(), v.float().numpy())
        ref = attention.decode(q[0].float().numpy(), K, V, w.sm_scale)
        for sp in (1, 3, 0):
            out = pool.decode(0, [seq], [ctx], q.cuda(), w.sm_scale, n_splits=sp)
            torch.cuda.synchronize()
            assert_close(out[0].cpu().numpy(), ref, f"2-bit {w.name} q x {qscale:g} ctx={ctx} splits={sp}")


def test_decode_q2_block_table_permutation_invariance():
    need_gpu()
    w, ctx = TINY, 256
    k, v = kv_rows(w, 0, 0, ctx)
    q = queries(w, 0, 1).cuda()
    outs = []
    for salt in (1, 2):
        pool, mem = make_pool(w, 8, 1)
        bt = page_permutation(w, 8, salt=salt)[:4]
        seq = pool.reserve(ctx, pages=bt)
        pool.append(0, [seq], [0], [ctx], k.cuda(), v.cuda())
        outs.append(pool.decode(0, [seq], [ctx], q, w.sm_scale, n_splits=2).cpu())
    assert torch.equal(outs[0], outs[1])


def test_decode_q2_batch_of_lanes_d128():
    need_gpu()
    w = SMALL128
    lens = [300, 65, 130]
    n_pages = 20
    pool, mem = make_pool(w, n_pages, 1)
    perm = page_permutation(w, n_pages, salt=5)
    off, seqs, bts = 0, [], []
    for L in lens:
        npg = -(-L // 64)
        bts.append(perm[off:off + npg]); off += npg
        seqs.append(pool.reserve(L, pages=bts[-1]))
    layer = 1
    ks = [kv_rows(w, layer, i, lens[i]) for i in range(3)]
    pool.append(layer, seqs, [0, 0, 0], lens, torch.cat([a for a, _ in ks]).cuda(), torch.cat([b for _, b in ks]).cuda())
    q = queries(w, layer, 3)
    out = pool.decode(layer, seqs, lens, q.cuda(), w.sm_scale, n_splits=2).cpu().numpy()
    for i in range(3):
        K, V = opool.dequantized_rows("q2", ks[i][0].float().numpy(), ks[i][1].float().numpy())
        ref = attention.decode(q[i].float().numpy(), K, V, w.sm_scale)
        assert_close(out[i], ref, f"lane {i} ctx={lens[i]}")


def test_errors_refused_before_any_write():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    pool, mem = make_pool(TINY, 4, 1)
    seq = pool.reserve(100)
    k, v = kv_rows(TINY, 0, 0, 101)
    before = mem.clone()
    with pytest.raises(kvq.KvError) as ei:
        pool.append(0, [seq], [0], [101], k.cuda(), v.cuda())   # beyond the 100-token bound
    assert ei.value.name == "KV_ERR_BOUND"
    with pytest.raises(kvq.KvError) as ei:
        pool.reserve(64 * 3)                                     # only 2 pages left
    assert ei.value.name == "KV_ERR_NO_SPACE"
    q = queries(TINY, 0, 1).cuda()
    with pytest.raises(kvq.KvError) as ei:
        pool.decode(0, [seq], [50], q, 0.0625, n_splits=1, ws=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.name == "KV_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.equal(mem, before)


# GQA groups other than 4 run the same matrix-core kernel four query heads at
# a time (group 8 as two workgroups a split in one launch; groups 1 and 2 with
# empty rows)
GROUPS = [
    Workload(93, "group 1, D=128", "q2", 1, 4, 128, 4, 2, 300),
    Workload(93, "group 2, D=256", "q2", 1, 2, 256, 4, 2, 300),
    Workload(93, "group 8, D=128", "q2", 1, 2, 128, 16, 2, 300),
    Workload(93, "group 8, D=256", "q2", 1, 1, 256, 8, 2, 300),
]


@pytest.mark.parametrize("w", GROUPS, ids=lambda w: w.name)
def test_decode_q2_other_groups(w):
    need_gpu()
    lens = [300, 97]
    n_pages = sum(-(-n // 64) for n in lens)
    pool, mem = make_pool(w, n_pages, 1)
    seqs, refs, refs_s = [], [], []
    q = queries(w, 0, len(lens))
    for i, n in enumerate(lens):
        seqs.append(pool.reserve(n))
        k, v = kv_rows(w, 0, i, n)
        pool.append(0, [seqs[-1]], [0], [n], k.cuda(), v.cuda())
        K, V = opool.dequantized_rows("q2", k.float().numpy(), v.float().numpy())
        refs.append(attention.decode(q[i].float().numpy(), K, V, w.sm_scale))
        refs_s.append(attention.scores(q[i].float().numpy(), K, w.sm_scale))
    for sp in (1, 3, 12):  # 12: more splits than the fused merge takes, most of them empty
        scores = torch.full((len(lens), w.n_q_heads, max(lens)), float("nan"), device="cuda")
        ws = torch.full((pool.workspace_bytes(0, len(lens), sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.decode(0, seqs, lens, q.cuda(), w.sm_scale, n_splits=sp, ws=ws, scores=scores)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), np.stack(refs), f"{w.name} splits={sp}")
        sc = scores.cpu().numpy().astype(np.float64)
        for i, n in enumerate(lens):
            rel = np.linalg.norm(sc[i, :, :n] - refs_s[i]) / np.linalg.norm(refs_s[i])
            assert rel <= 1e-5, f"{w.name} lane {i}: scores rel L2 {rel:.2e}"
