"""GPU parity, bf16 pool format (the exact cache the compressed formats are
priced against): append bit-exact against the oracle's pool image, page
reads bit-exact, decode and chunked prefill within tolerance of the fp64
oracle over the same rows.  The pools are filled with 0xFF before use, so
every slot never written holds a bf16 NaN pattern: a kernel that lets an
unwritten slot into a sum fails these tests."""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import WORKLOADS, Workload, kv_rows, page_permutation, queries
from tests.gpu_helpers import assert_close, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny"]
GEOM27B = WORKLOADS["27b"]
# 2 layers x 2 KV heads x 128 dims, 8 query heads (group 4)
SMALL128 = Workload(90, "small D=128 geometry", "bf16", 2, 2, 128, 8, 3, 300)
# group 8 and group 1 at 128 dims, group 2 at 256
G8_128 = Workload(94, "group 8, D=128", "bf16", 1, 2, 128, 16, 1, 300)
G1_128 = Workload(95, "group 1, D=128", "bf16", 1, 4, 128, 4, 1, 300)
G2_256 = Workload(96, "group 2, D=256", "bf16", 1, 2, 256, 4, 1, 300)

NAN_FILL = 0xFF


def _fmt():
    import quantized_kv_attention_append_amd as kvq
    return kvq.FMT_BF16


def test_append_bf16_ragged_chunks_bit_exact():
    need_gpu()
    n_pages = 6
    pool, mem = make_pool(TINY, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(TINY, n_pages)[:4]
    seq = pool.reserve(256, pages=bt)
    k, v = kv_rows(TINY, 0, 0, 256)
    op = opool.OraclePool("bf16", 1, 4, 256, n_pages, fill=NAN_FILL)
    start = 0
    for n in (100, 1, 27, 64, 64):   # ragged chunks, some crossing page ends
        pool.append(0, [seq], [start], [n], k[start:start + n].cuda(), v[start:start + n].cuda())
        op.append(0, 0, bt, start, k[start:start + n].float().numpy(), v[start:start + n].float().numpy())
        start += n
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"bf16 append: {diff} differing bytes of {got.size}")
    assert diff == 0


def test_append_bf16_batched_d128_bit_exact():
    need_gpu()
    w = SMALL128
    n_pages = 20
    pool, mem = make_pool(w, n_pages, _fmt(), fill=NAN_FILL)
    perm = page_permutation(w, n_pages)
    lens = [300, 65, 130]
    bts, seqs = [], []
    off = 0
    for L in lens:
        npg = -(-L // 64)
        bts.append(perm[off:off + npg]); off += npg
        seqs.append(pool.reserve(L, pages=bts[-1]))
    op = opool.OraclePool("bf16", 2, 2, 128, n_pages, fill=NAN_FILL)
    for layer in range(2):
        rows = [kv_rows(w, layer, i, lens[i]) for i in range(3)]
        starts = [0, 0, 0]
        for chunk in ([(0, 37), (1, 1), (2, 64)], [(0, 200), (2, 66)], [(0, 63), (1, 64)]):
            ks, vs, ss, st, nn = [], [], [], [], []
            for i, n in chunk:
                s0 = starts[i]
                ks.append(rows[i][0][s0:s0 + n]); vs.append(rows[i][1][s0:s0 + n])
                ss.append(seqs[i]); st.append(s0); nn.append(n)
                op.append(layer, i, bts[i], s0, rows[i][0][s0:s0 + n].float().numpy(),
                          rows[i][1][s0:s0 + n].float().numpy())
                starts[i] += n
            pool.append(layer, ss, st, nn, torch.cat(ks).cuda(), torch.cat(vs).cuda())
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(n_pages, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"bf16 batched append: {diff} differing bytes of {got.size}")
    assert diff == 0


def test_dequant_page_bf16_returns_rows():
    need_gpu()
    n_pages = 6
    pool, mem = make_pool(TINY, n_pages, _fmt(), fill=0)
    bt = page_permutation(TINY, n_pages)[:4]
    seq = pool.reserve(256, pages=bt)
    k, v = kv_rows(TINY, 0, 0, 256)
    pool.append(0, [seq], [0], [256], k.cuda(), v.cuda())
    K, V = k.float().numpy(), v.float().numpy()
    for lp in range(4):
        for h in (0, 3):
            gk = pool.dequant_page(int(bt[lp]), 0, h, 0).cpu().numpy()
            gv = pool.dequant_page(int(bt[lp]), 0, h, 1).cpu().numpy()
            assert np.array_equal(gk.view(np.uint32), K[64 * lp:64 * lp + 64, h].view(np.uint32))
            assert np.array_equal(gv.view(np.uint32), V[64 * lp:64 * lp + 64, h].view(np.uint32))


def _decode_case(w, ctx, splits_list, layer=0, qscale=1.0):
    n_pages = -(-ctx // 64) + 2
    pool, mem = make_pool(w, n_pages, _fmt(), fill=NAN_FILL)
    bt = page_permutation(w, n_pages, salt=ctx)[:-2]
    seq = pool.reserve(ctx, pages=bt)
    k, v = kv_rows(w, layer, 0, ctx)
    pool.append(layer, [seq], [0], [ctx], k.cuda(), v.cuda())
    q = queries(w, layer, 1)
    if qscale != 1.0:
        q = (q.float() * qscale).to(torch.bfloat16)
    K, V = k.float().numpy(), v.float().numpy()
    ref = attention.decode(q[0].float().numpy(), K, V, w.sm_scale)
    ref_s = attention.scores(q[0].float().numpy(), K, w.sm_scale)
    for sp in splits_list:
        scores = torch.full((1, w.n_q_heads, ctx), float("nan"), device="cuda")
        ws = torch.full((pool.workspace_bytes(0, 1, sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.decode(layer, [seq], [ctx], q.cuda(), w.sm_scale, n_splits=sp, ws=ws, scores=scores)
        torch.cuda.synchronize()
        assert_close(out[0].cpu().numpy(), ref, f"bf16 decode {w.name} ctx={ctx} splits={sp} q x {qscale:g}")
        assert_close(scores[0].cpu().numpy(), ref_s, f"bf16 scores ctx={ctx} splits={sp}", max_abs=2e-3, rel_l2=1e-5)


@pytest.mark.parametrize("qscale", [64.0, 1.0 / 64.0])
def test_decode_bf16_peaked_and_flat(qscale):
    """bf16 pools with queries scaled by 64 and by 1/64: the weights' two bf16
    terms under a sharply peaked and a nearly flat softmax."""
    need_gpu()
    _decode_case(TINY, 700, [1, 3, 0], qscale=qscale)
    _decode_case(SMALL128, 450, [1, 0], layer=1, qscale=qscale)


@pytest.mark.parametrize("ctx", [1, 63, 65, 256, 1000])
def test_decode_bf16_ragged_lengths(ctx):
    need_gpu()
    _decode_case(TINY, ctx, [1, 3, 0])


@pytest.mark.parametrize("w", [G8_128, G1_128, G2_256], ids=lambda w: w.name)
def test_decode_bf16_groups(w):
    need_gpu()
    _decode_case(w, 300, [1, 2])


def test_decode_bf16_batch_of_lanes_d128():
    need_gpu()
    w = SMALL128
    lens = [300, 65, 130]
    n_pages = 20
    pool, mem = make_pool(w, n_pages, _fmt(), fill=NAN_FILL)
    perm = page_permutation(w, n_pages, salt=5)
    off, seqs = 0, []
    for L in lens:
        npg = -(-L // 64)
        seqs.append(pool.reserve(L, pages=perm[off:off + npg])); off += npg
    layer = 1
    rows = [kv_rows(w, layer, i, lens[i]) for i in range(3)]
    pool.append(layer, seqs, [0, 0, 0], lens, torch.cat([a for a, _ in rows]).cuda(),
                torch.cat([b for _, b in rows]).cuda())
    q = queries(w, layer, 3)
    out = pool.decode(layer, seqs, lens, q.cuda(), w.sm_scale, n_splits=2).cpu().numpy()
    for i in range(3):
        ref = attention.decode(q[i].float().numpy(), rows[i][0].float().numpy(), rows[i][1].float().numpy(), w.sm_scale)
        assert_close(out[i], ref, f"bf16 lane {i} ctx={lens[i]}")


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
    ref = attention.prefill(q.float().numpy(), k.float().numpy(), v.float().numpy(), w.sm_scale, q_start=prior)
    for sp in splits_list:
        ws = torch.full((pool.workspace_bytes(kvq.OP_PREFILL, n_q, sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.prefill(layer, seq, prior, q.cuda(), w.sm_scale, n_splits=sp, ws=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, f"bf16 prefill prior={prior} n_q={n_q} splits={sp}")


def test_prefill_bf16_d256():
    need_gpu()
    _prefill_case(TINY, 0, 100, 45, [1, 2, 0])


def test_prefill_bf16_chunk_from_zero_d256():
    need_gpu()
    _prefill_case(TINY, 0, 0, 77, [1, 2])


def test_prefill_bf16_d128_group4():
    need_gpu()
    _prefill_case(SMALL128, 1, 130, 64, [1, 4])


@pytest.mark.timeout(600)
def test_decode_bf16_27b_geometry_layer_sampled_lanes():
    """One layer of the 27B-geometry batch in bf16 (8 lanes x 40,960 tokens,
    4 KV heads x 256 dims, 16 query heads; 1.34 GB of K and V), decoded at the
    split count the library picks; lanes 0 and 7 against the oracle."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    w = Workload(GEOM27B.cfg, GEOM27B.name, "bf16", 1, GEOM27B.n_kv_heads, GEOM27B.head_dim, GEOM27B.n_q_heads, GEOM27B.lanes, GEOM27B.ctx)
    B, ctx = w.lanes, w.ctx
    ppl = ctx // 64
    n_pages = B * ppl
    pool, mem = make_pool(w, n_pages, kvq.FMT_BF16, fill=NAN_FILL, max_seqs=B, max_seq_tokens=ctx)
    perm = page_permutation(GEOM27B, n_pages)
    seqs = [pool.reserve(ctx, pages=perm[i * ppl:(i + 1) * ppl]) for i in range(B)]
    rows = []
    for lane in range(B):
        k, v = kv_rows(GEOM27B, 3, lane, ctx, device="cuda")   # the rows of layer 3 of the 27B batch
        pool.append(0, [seqs[lane]], [0], [ctx], k, v)
        if lane in (0, B - 1):
            rows.append((lane, k.float().cpu().numpy(), v.float().cpu().numpy()))
        del k, v
    q = queries(GEOM27B, 3, B, device="cuda")
    out = pool.decode(0, seqs, [ctx] * B, q, w.sm_scale).cpu().numpy()
    assert np.all(np.isfinite(out))
    qn = q.float().cpu().numpy()
    for lane, K, V in rows:
        ref = attention.decode(qn[lane], K, V, w.sm_scale)
        assert_close(out[lane], ref, f"bf16 27B-geometry lane {lane}")
