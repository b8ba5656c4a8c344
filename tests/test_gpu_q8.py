"""GPU parity, 8-bit format: append bit-exact against the oracle's pool image
(per-token V, per-channel K over the exact rows of the open page), decode
within tolerance of the fp64 oracle, and the 24-lane, 32-layer workload
(8 KV heads x 128 dims, 32 query heads, lengths 64 * U[16, 128]) with one more
token appended per lane after the first decode."""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import WORKLOADS, Workload, q8_batch_lengths, kv_rows, page_permutation, queries
from tests.gpu_helpers import assert_close, geom_of, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

Q8B = WORKLOADS["q8"]
# 2 layers of the 8-bit geometry, 3 lanes
SMALL8 = Workload(91, "small 8-bit geometry", "q8", 2, 8, 128, 32, 3, 300)
# a D = 256, group-2 geometry on the 8-bit format
SMALL8_256 = Workload(92, "small 8-bit D=256 geometry", "q8", 1, 4, 256, 8, 2, 200)
# the other group sizes of the wave-parallel decode (1, 8; 4 at D = 256) and the
# one that takes the workgroup-per-page form (8 at D = 256)
G1 = Workload(94, "8-bit group 1", "q8", 1, 4, 128, 4, 2, 300)
G2 = Workload(96, "8-bit group 2", "q8", 1, 4, 128, 8, 2, 300)
G8 = Workload(95, "8-bit group 8", "q8", 1, 2, 128, 16, 2, 300)
G4_256 = Workload(97, "8-bit D=256 group 4", "q8", 1, 2, 256, 8, 2, 200)
G8_256 = Workload(98, "8-bit D=256 group 8", "q8", 1, 1, 256, 8, 2, 200)


def _setup(w, lens, n_pages, salt=0, fill=0xA5):
    import quantized_kv_attention_append_amd as kvq
    pool, mem = make_pool(w, n_pages, kvq.FMT_Q8, fill=fill)
    perm = page_permutation(w, n_pages, salt=salt)
    bts, seqs, off = [], [], 0
    for L in lens:
        npg = -(-L // 64)
        bts.append(perm[off:off + npg])
        off += npg
        seqs.append(pool.reserve(L, pages=bts[-1]))
    op = opool.OraclePool("q8", w.n_layers, w.n_kv_heads, w.head_dim, n_pages, fill=fill)
    return pool, mem, op, bts, seqs


def _append_chunks(pool, op, layer, seqs, bts, chunks, ks, vs, starts):
    """chunks: list of [(seq index, n), ...]; each inner list is one batched append."""
    for chunk in chunks:
        sq, st, nn, kk, vv = [], [], [], [], []
        for i, n in chunk:
            s0 = starts[i]
            sq.append(seqs[i]); st.append(s0); nn.append(n)
            kk.append(ks[i][s0:s0 + n]); vv.append(vs[i][s0:s0 + n])
            op.append(layer, i, bts[i], s0, ks[i][s0:s0 + n].float().numpy(), vs[i][s0:s0 + n].float().numpy())
            starts[i] += n
        pool.append(layer, sq, st, nn, torch.cat(kk).cuda(), torch.cat(vv).cuda())


def test_append_q8_bit_exact_ragged():
    need_gpu()
    w = SMALL8
    lens = [300, 130, 64]
    pool, mem, op, bts, seqs = _setup(w, lens, 12)
    for layer in range(w.n_layers):
        ks = [kv_rows(w, layer, i, lens[i])[0] for i in range(3)]
        vs = [kv_rows(w, layer, i, lens[i])[1] for i in range(3)]
        starts = [0, 0, 0]
        chunks = [[(0, 37), (1, 1), (2, 64)],   # mid-page end, single token, one full page
                  [(0, 1)], [(0, 1)],             # decode-style single tokens into the open page
                  [(0, 150), (1, 70)],            # from mid-page across pages: two launches
                  [(0, 111), (1, 59)]]            # lane 0 crosses again, lane 1 fills to 130
        _append_chunks(pool, op, layer, seqs, bts, chunks, ks, vs, starts)
        assert starts == lens
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(12, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"8-bit ragged append: {diff} differing bytes of {got.size}")
    assert diff == 0


def test_append_q8_half_step_rows_bit_exact():
    """Codes on ties: every K channel and every V row holds 127 * 2^e (so the
    scale is exactly 2^e) and values (k + 1/2) 2^e elsewhere, each a tie of the
    rounding to an integer code (round half to even)."""
    need_gpu()
    w = SMALL8
    L = 128
    pool, mem, op, bts, seqs = _setup(w, [L], 3)
    rng = np.random.default_rng(4321)
    H, D = w.n_kv_heads, w.head_dim
    ek = rng.integers(-6, 3, size=(1, H, D)).astype(np.float64)
    kq = rng.integers(-127, 127, size=(L, H, D)) + 0.5
    kq[0] = 127.0                                   # token 0: the absmax of every channel
    ev = rng.integers(-6, 3, size=(L, 1, 1)).astype(np.float64)
    vq = rng.integers(-127, 127, size=(L, H, D)) + 0.5
    vq[:, :, 0] = -127.0                            # dim 0: the absmax of every row
    kf, vf = (kq * 2.0 ** ek).astype(np.float32), (vq * 2.0 ** ev).astype(np.float32)
    k, v = torch.tensor(kf).to(torch.bfloat16), torch.tensor(vf).to(torch.bfloat16)
    assert torch.equal(k.float(), torch.tensor(kf)) and torch.equal(v.float(), torch.tensor(vf))
    starts = [0]
    _append_chunks(pool, op, 0, seqs, bts, [[(0, 37)], [(0, 1)], [(0, 90)]], [k], [v], starts)
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(3, -1)
    diff = np.count_nonzero(got != op.data)
    say(f"8-bit half-step rows: {diff} differing bytes of {got.size}")
    assert diff == 0


def test_append_q8_d256_and_dequant():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    w = SMALL8_256
    lens = [200, 65]
    pool, mem, op, bts, seqs = _setup(w, lens, 6, salt=3)
    ks = [kv_rows(w, 0, i, lens[i])[0] for i in range(2)]
    vs = [kv_rows(w, 0, i, lens[i])[1] for i in range(2)]
    starts = [0, 0]
    _append_chunks(pool, op, 0, seqs, bts, [[(0, 5), (1, 64)], [(0, 195), (1, 1)]], ks, vs, starts)
    torch.cuda.synchronize()
    got = mem.cpu().numpy().reshape(6, -1)
    assert np.count_nonzero(got != op.data) == 0
    # page dequantization equals the oracle's single-product dequantization
    K, V = op.gather(0, bts[0], 200)
    for lp in (0, 3):
        n = min(64, 200 - 64 * lp)
        for h in (0, 3):
            gk = pool.dequant_page(int(bts[0][lp]), 0, h, 0).cpu().numpy()[:n]
            gv = pool.dequant_page(int(bts[0][lp]), 0, h, 1).cpu().numpy()[:n]
            assert np.array_equal(gk.view(np.uint32), K[64 * lp:64 * lp + n, h].view(np.uint32))
            assert np.array_equal(gv.view(np.uint32), V[64 * lp:64 * lp + n, h].view(np.uint32))
    assert kvq.FMT_Q8 == 2


def test_append_q8_must_be_sequential():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    w = SMALL8
    pool, mem, op, bts, seqs = _setup(w, [128], 4)
    k, v = kv_rows(w, 0, 0, 128)
    pool.append(0, [seqs[0]], [0], [10], k[:10].cuda(), v[:10].cuda())
    before = mem.clone()
    with pytest.raises(kvq.KvError) as ei:
        pool.append(0, [seqs[0]], [20], [5], k[20:25].cuda(), v[20:25].cuda())   # gap
    assert ei.value.name == "KV_ERR_ARG"
    with pytest.raises(kvq.KvError) as ei:
        pool.append(1, [seqs[0]], [10], [5], k[10:15].cuda(), v[10:15].cuda())   # layer 1 holds 0 tokens
    assert ei.value.name == "KV_ERR_ARG"
    torch.cuda.synchronize()
    assert torch.equal(mem, before)


# lanes of 1,100 and 1,300 tokens give each wave of the matrix-core form several
# pages, one in LDS while the next arrives (four waves up to group 4, eight at 8)
@pytest.mark.parametrize("w,lens", [(SMALL8, [300, 130, 64]), (SMALL8_256, [200, 65]), (G1, [300, 70]),
                                    (G1, [1100, 300]), (G2, [300, 70]), (G8, [300, 129]), (G8, [1300, 129]),
                                    (G4_256, [200, 65]), (G8_256, [130, 200])])
def test_decode_q8_small(w, lens):
    need_gpu()
    n_pages = sum(-(-L // 64) for L in lens) + 2
    pool, mem, op, bts, seqs = _setup(w, lens, n_pages, salt=11)
    layer = w.n_layers - 1
    ks = [kv_rows(w, layer, i, L)[0] for i, L in enumerate(lens)]
    vs = [kv_rows(w, layer, i, L)[1] for i, L in enumerate(lens)]
    starts = [0] * len(lens)
    _append_chunks(pool, op, layer, seqs, bts, [[(i, L) for i, L in enumerate(lens)]], ks, vs, starts)
    q = queries(w, layer, len(lens))
    ctxs = [L - 3 for L in lens]   # ragged: the last page is read partly
    for sp in (1, 2, 0):
        scores = torch.full((len(lens), w.n_q_heads, max(ctxs)), float("nan"), device="cuda")
        ws = torch.full((pool.workspace_bytes(0, len(lens), sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.decode(layer, seqs, ctxs, q.cuda(), w.sm_scale, n_splits=sp, ws=ws, scores=scores)
        plain = pool.decode(layer, seqs, ctxs, q.cuda(), w.sm_scale, n_splits=sp, ws=ws)  # the variant without scores
        torch.cuda.synchronize()
        for i, c in enumerate(ctxs):
            K, V = op.gather(layer, bts[i], c)
            qi = q[i].float().numpy()
            ref = attention.decode(qi, K, V, w.sm_scale)
            assert_close(out[i].cpu().numpy(), ref, f"8-bit lane {i} ctx={c} splits={sp}")
            assert_close(plain[i].cpu().numpy(), ref, f"8-bit lane {i} ctx={c} splits={sp}, no scores")
            assert_close(scores[i, :, :c].cpu().numpy(), attention.scores(qi, K, w.sm_scale),
                         f"8-bit scores lane {i}", rel_l2=1e-5)


@pytest.mark.parametrize("w,qscale", [(SMALL8, 64.0), (SMALL8, 1.0 / 64.0), (G8, 64.0), (G1, 1.0 / 64.0)])
def test_decode_q8_peaked_and_flat(w, qscale):
    """Queries scaled by 64 (a softmax concentrated on a few tokens, most weights
    far below each page's largest) and by 1/64 (nearly flat weights): the
    matrix-core form keeps the scaled query and the weights to 2^-20 of each
    row's largest value, which the oracle's fp64 attention must confirm."""
    need_gpu()
    lens = [300, 190]
    n_pages = sum(-(-L // 64) for L in lens) + 1
    pool, mem, op, bts, seqs = _setup(w, lens, n_pages, salt=17)
    layer = 0
    ks = [kv_rows(w, layer, i, L)[0] for i, L in enumerate(lens)]
    vs = [kv_rows(w, layer, i, L)[1] for i, L in enumerate(lens)]
    _append_chunks(pool, op, layer, seqs, bts, [[(i, L) for i, L in enumerate(lens)]], ks, vs, [0] * len(lens))
    q = (queries(w, layer, len(lens)).float() * qscale).to(torch.bfloat16)
    for sp in (1, 0):
        out = pool.decode(layer, seqs, lens, q.cuda(), w.sm_scale, n_splits=sp)
        torch.cuda.synchronize()
        for i, c in enumerate(lens):
            K, V = op.gather(layer, bts[i], c)
            ref = attention.decode(q[i].float().numpy(), K, V, w.sm_scale)
            assert_close(out[i].cpu().numpy(), ref, f"8-bit q x {qscale:g}, lane {i} ctx={c} splits={sp}")


def test_decode_q8_long_lanes_many_splits():
    """Two lanes of 9,000 and 2,500 tokens at 12 and 40 splits (the merge of more
    than 8 splits, one split a lane of a wave) and at the library's count, with
    the workspace pre-filled with 0xFF so that an unwritten partial would show."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    w = SMALL8
    lens = [9000, 2500]
    n_pages = sum(-(-L // 64) for L in lens) + 1
    pool, mem, op, bts, seqs = _setup(w, lens, n_pages, salt=23)
    layer = 1
    ks = [kv_rows(w, layer, i, L)[0] for i, L in enumerate(lens)]
    vs = [kv_rows(w, layer, i, L)[1] for i, L in enumerate(lens)]
    _append_chunks(pool, op, layer, seqs, bts, [[(i, L) for i, L in enumerate(lens)]], ks, vs, [0] * len(lens))
    q = queries(w, layer, len(lens))
    refs = []
    for i, c in enumerate(lens):
        K, V = op.gather(layer, bts[i], c)
        refs.append(attention.decode(q[i].float().numpy(), K, V, w.sm_scale))
    for sp in (12, 40, 0):
        ws = torch.full((pool.workspace_bytes(kvq.OP_DECODE, len(lens), sp),), 0xFF, dtype=torch.uint8, device="cuda")
        out = pool.decode(layer, seqs, lens, q.cuda(), w.sm_scale, n_splits=sp, ws=ws)
        torch.cuda.synchronize()
        for i, c in enumerate(lens):
            assert_close(out[i].cpu().numpy(), refs[i], f"8-bit long lane {i} ctx={c} splits={sp or pool.decode_splits(lens)}")


@pytest.mark.timeout(900)
def test_q8_batch_decode_then_append():
    """Full 8-bit workload: populate 32 layers x 24 lanes, decode every layer,
    append one token per lane, decode again.  For layers 0, 13 and 31: every
    lane's full pages byte for byte against the oracle's image, the page the
    appended token opens against the oracle pool's image of it, and the whole
    decode output of all 24 lanes (before and after the append) against the
    oracle."""
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    w = Q8B
    lens = [int(x) for x in q8_batch_lengths(w)]
    geom = geom_of(w)
    _, pb = kvq.token_bytes(geom, kvq.FMT_Q8)
    n_pages = int(sum(-(-(L + 1) // 64) for L in lens))
    mem = torch.full((n_pages * pb,), 0xA5, dtype=torch.uint8, device="cuda")
    pool = kvq.Pool(n_pages * pb, geom, kvq.FMT_Q8, max_seqs=w.lanes, max_seq_tokens=max(lens) + 64, memory=mem)
    perm = page_permutation(w, n_pages)
    seqs, bts, off = [], [], 0
    for L in lens:
        npg = -(-(L + 1) // 64)
        bts.append(perm[off:off + npg])
        seqs.append(pool.reserve(L + 1, pages=bts[-1]))
        off += npg
    say(f"8-bit workload: {n_pages} pages, {n_pages * pb / 1e9:.2f} GB, lengths {min(lens)}..{max(lens)}")
    B, H, D = w.lanes, w.n_kv_heads, w.head_dim
    block = 132 * D + 256
    ws = torch.empty(pool.workspace_bytes(0, B, 0), dtype=torch.uint8, device="cuda")
    pages_of = lambda lane, lp: torch.as_tensor(np.asarray(bts[lane][lp], np.int64), device="cuda")
    for layer in range(w.n_layers):
        kv = [kv_rows(w, layer, i, lens[i] + 1, device="cuda") for i in range(B)]
        pool.append(layer, seqs, [0] * B, lens,
                    torch.cat([k[:L] for (k, _), L in zip(kv, lens)]), torch.cat([v[:L] for (_, v), L in zip(kv, lens)]))
        q = queries(w, layer, B, device="cuda")
        out1 = pool.decode(layer, seqs, lens, q, w.sm_scale, ws=ws).cpu().numpy()
        check = layer in (0, 13, 31)
        if check:   # the full pages before the next token opens a page
            full = [mem.view(-1, pb).index_select(0, pages_of(i, slice(0, lens[i] // 64)))[
                :, layer * H * block:(layer + 1) * H * block].cpu().numpy() for i in range(B)]
        pool.append(layer, seqs, lens, [1] * B,
                    torch.cat([k[L:L + 1] for (k, _), L in zip(kv, lens)]),
                    torch.cat([v[L:L + 1] for (_, v), L in zip(kv, lens)]))
        out2 = pool.decode(layer, seqs, [L + 1 for L in lens], q, w.sm_scale, ws=ws).cpu().numpy()
        if check:
            qh = q.float().cpu().numpy()
            ref1, ref2 = [], []
            for i, L in enumerate(lens):
                k, v = (t.cpu().float().numpy() for t in kv[i])
                blocks = opool.sequence_blocks("q8", k[:L], v[:L])
                bad = int(np.count_nonzero(full[i] != blocks.reshape(L // 64, H * block)))
                assert bad == 0, f"8-bit layer {layer} lane {i}: {bad} bytes of the full pages differ"
                one = opool.OraclePool("q8", w.n_layers, H, D, 1, fill=0xA5)
                one.append(layer, 0, [0], 0, k[L:L + 1], v[L:L + 1])
                got = mem.view(-1, pb)[int(bts[i][L // 64])][layer * H * block:(layer + 1) * H * block].cpu().numpy()
                assert np.array_equal(got, one.data[0, layer * H * block:(layer + 1) * H * block]), \
                    f"8-bit layer {layer} lane {i}: the page of token {L} differs"
                K, V = opool.dequantized_rows("q8", k[:L], v[:L])
                ref1.append(attention.decode(qh[i], K, V, w.sm_scale))
                K, V = opool.dequantized_rows("q8", k, v)
                ref2.append(attention.decode(qh[i], K, V, w.sm_scale))
            assert_close(out1, np.stack(ref1), f"8-bit layer {layer}, all 24 lanes")
            assert_close(out2, np.stack(ref2), f"8-bit layer {layer}, all 24 lanes after one more token")
            say(f"8-bit layer {layer}: pages bit-exact, whole outputs within tolerance")
        del kv
